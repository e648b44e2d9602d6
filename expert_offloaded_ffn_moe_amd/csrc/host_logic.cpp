#include "host_logic.h"

#include <algorithm>
#include <cstring>
#include <numeric>

namespace moe {

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

Layout make_layout(int64_t H, int64_t I, int64_t G, int64_t bits) {
  Layout L;
  L.H = H;
  L.I = I;
  L.G = G;
  L.bits = bits;
  L.kc = bits == 4 ? 32 : 64;
  L.gu_tiles = I / 32;
  L.gu_chunks = H / L.kc;
  L.gu_groups = H / G;
  L.dn_tiles = H / 64;
  L.dn_chunks = I / L.kc;
  L.dn_groups = I / G;
  const int64_t hi_block = bits == 3 ? 512 : 0;
  int64_t off = 0;
  L.off_gu_codes = off;
  off = round_up(off + L.gu_tiles * L.gu_chunks * 1024, 256);
  L.off_gu_hi = off;
  off = round_up(off + L.gu_tiles * L.gu_chunks * hi_block, 256);
  L.off_gu_scales = off;
  off = round_up(off + L.gu_tiles * L.gu_groups * 128, 256);
  L.off_dn_codes = off;
  off = round_up(off + L.dn_tiles * L.dn_chunks * 1024, 256);
  L.off_dn_hi = off;
  off = round_up(off + L.dn_tiles * L.dn_chunks * hi_block, 256);
  L.off_dn_scales = off;
  off = round_up(off + L.dn_tiles * L.dn_groups * 128, 256);
  L.bytes = off;
  L.canonical_bytes = 3 * H * I * bits / 8 + 6 * H * I / G;
  return L;
}

std::string check_config(const moe_config& c) {
  if (c.hidden <= 0 || c.inter <= 0) return "hidden and inter must be positive";
  if (c.group_size != 32 && c.group_size != 64 && c.group_size != 128 && c.group_size != 256)
    return "group_size must be 32, 64, 128 or 256";
  if (c.hidden % 64) return "hidden must be a multiple of 64";
  if (c.inter % 32) return "inter must be a multiple of 32";
  if (c.hidden % c.group_size) return "hidden must be a multiple of group_size";
  if (c.inter % c.group_size) return "inter must be a multiple of group_size";
  if (c.num_experts < 1 || c.num_experts > 1024) return "num_experts must be in 1..1024";
  if (c.top_k < 1 || c.top_k > c.num_experts || c.top_k > 32) return "top_k must be in 1..min(num_experts, 32)";
  if (c.num_layers < 1) return "num_layers must be >= 1";
  if (c.act_dtype != MOE_ACT_F32 && c.act_dtype != MOE_ACT_BF16) return "act_dtype must be MOE_ACT_F32 or MOE_ACT_BF16";
  if (c.max_tokens < 1 || c.max_tokens > (1 << 20)) return "max_tokens must be in 1..2^20";
  if ((int64_t)c.max_tokens * c.top_k > (1 << 22)) return "max_tokens * top_k must be <= 2^22";
  if (c.hbm_slots < 0 || c.hbm_slots > c.num_experts) return "hbm_slots must be in 0..num_experts";
  if (c.prefill_stage_slots < 0 || c.prefill_stage_slots > c.num_experts)
    return "prefill_stage_slots must be in 0..num_experts";
  if (c.prefetch_slots < 0 || c.prefetch_slots > c.num_experts || c.prefetch_slots > 64)
    return "prefetch_slots must be in 0..min(num_experts, 64)";
  if (c.hidden > 65536 || c.inter > 65536) return "hidden and inter must be <= 65536";
  const int bits = c.weight_bits == 0 ? 4 : c.weight_bits;
  if (bits != 2 && bits != 3 && bits != 4) return "weight_bits must be 0 (4), 2, 3 or 4";
  if (bits < 4) {
    if (c.act_dtype != MOE_ACT_BF16) return "2- and 3-bit weights need bf16 activations";
    if (c.group_size < 64) return "2- and 3-bit weights need group_size 64, 128 or 256";
    if (c.inter % 64) return "2- and 3-bit weights need inter to be a multiple of 64";
  }
  return "";
}

// One internal dword from 4 canonical bytes (8 consecutive K values): canonical
// byte j holds offsets 2j (low nibble) and 2j+1 (high nibble); the internal
// dword wants offset 2j at bits [4j, 4j+4) and 2j+1 at bits [16+4j, 20+4j),
// each as n = q + 8, which for a two's complement nibble is the nibble XOR 8.
static inline uint32_t internal_dword(uint32_t w) {
  uint32_t lo = w & 0x0F0F0F0Fu;
  lo = (lo | (lo >> 4)) & 0x00FF00FFu;
  lo = (lo | (lo >> 8)) & 0x0000FFFFu;
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  hi = (hi | (hi >> 4)) & 0x00FF00FFu;
  hi = (hi | (hi >> 8)) & 0x0000FFFFu;
  return (lo | (hi << 16)) ^ 0x88888888u;
}

// 16 internal bytes from the 16 canonical bytes of one row's K chunk.
static inline void chunk16(const uint8_t* src, uint8_t* dst) {
  for (int d = 0; d < 4; ++d) {
    uint32_t w;
    std::memcpy(&w, src + 4 * d, 4);
    w = internal_dword(w);
    std::memcpy(dst + 4 * d, &w, 4);
  }
}

static void repack_expert4(const Layout& L, const uint8_t* canon, uint8_t* out) {
  const int64_t H = L.H, I = L.I, G = L.G;
  const uint8_t* q_gate = canon;
  const uint8_t* q_up = q_gate + I * H / 2;
  const uint8_t* q_down = q_up + I * H / 2;
  const uint16_t* s_gate = reinterpret_cast<const uint16_t*>(q_down + H * I / 2);
  const uint16_t* s_up = s_gate + I * (H / G);
  const uint16_t* s_down = s_up + I * (H / G);
  std::memset(out, 0, (size_t)L.bytes);

  // gate/up codes and scales
  for (int64_t t = 0; t < L.gu_tiles; ++t) {
    for (int lane = 0; lane < 64; ++lane) {
      const bool up = lane >= 32;
      const int64_t row = 32 * t + (lane & 31);
      const uint8_t* src = (up ? q_up : q_gate) + row * (H / 2);
      for (int64_t c = 0; c < L.gu_chunks; ++c)
        chunk16(src + 16 * c, out + L.off_gu_codes + ((t * L.gu_chunks + c) * 64 + lane) * 16);
      const uint16_t* srow = (up ? s_up : s_gate) + row * (H / G);
      for (int64_t g = 0; g < H / G; ++g) {
        uint8_t* dst = out + L.off_gu_scales + ((t * L.gu_groups + g) * 64 + lane) * 2;
        std::memcpy(dst, srow + g, 2);
      }
    }
  }
  // down codes and scales
  for (int64_t t = 0; t < L.dn_tiles; ++t) {
    for (int lane = 0; lane < 64; ++lane) {
      const int64_t row = 64 * t + lane;
      const uint8_t* src = q_down + row * (I / 2);
      for (int64_t c = 0; c < L.dn_chunks; ++c)
        chunk16(src + 16 * c, out + L.off_dn_codes + ((t * L.dn_chunks + c) * 64 + lane) * 16);
      const uint16_t* srow = s_down + row * (I / G);
      for (int64_t g = 0; g < I / G; ++g) {
        uint8_t* dst = out + L.off_dn_scales + ((t * L.dn_groups + g) * 64 + lane) * 2;
        std::memcpy(dst, srow + g, 2);
      }
    }
  }
}

// Code i of a canonical row of b-bit codes: bits [b*i, b*i+b) of the row's
// little-endian bit string (bit j = bit j % 8 of byte j / 8).
static inline uint32_t code_at(const uint8_t* row, int64_t i, int64_t b) {
  const int64_t bit = i * b;
  uint32_t w = row[bit >> 3];
  if ((bit & 7) + b > 8) w |= (uint32_t)row[(bit >> 3) + 1] << 8;
  return (w >> (bit & 7)) & ((1u << b) - 1u);
}

// The 16-byte low-plane word and (3-bit codes) the 8-byte high-plane word of one
// lane for the 64 codes of `row` starting at K offset k0.
static void lane_words_lowbit(const uint8_t* row, int64_t k0, int64_t b, uint8_t* lo16, uint8_t* hi8) {
  uint32_t lo[4] = {0, 0, 0, 0}, hi[2] = {0, 0};
  for (int d = 0; d < 4; ++d)
    for (int j = 0; j < 8; ++j) {
      const uint32_t n0 = code_at(row, k0 + 16 * d + 2 * j, b), n1 = code_at(row, k0 + 16 * d + 2 * j + 1, b);
      lo[d] |= ((n0 & 3u) << (2 * j)) | ((n1 & 3u) << (16 + 2 * j));
    }
  std::memcpy(lo16, lo, 16);
  if (!hi8) return;
  for (int e = 0; e < 2; ++e)
    for (int i = 0; i < 16; ++i) {
      const uint32_t n0 = code_at(row, k0 + 32 * e + 2 * i, b), n1 = code_at(row, k0 + 32 * e + 2 * i + 1, b);
      hi[e] |= ((n0 >> 2) << i) | ((n1 >> 2) << (16 + i));
    }
  std::memcpy(hi8, hi, 8);
}

static void repack_expert_lowbit(const Layout& L, const uint8_t* canon, uint8_t* out) {
  const int64_t H = L.H, I = L.I, G = L.G, b = L.bits, kc = L.kc;
  const int64_t rb_h = H * b / 8, rb_i = I * b / 8;  // canonical bytes per row, K = H / K = I
  const uint8_t* q_gate = canon;
  const uint8_t* q_up = q_gate + I * rb_h;
  const uint8_t* q_down = q_up + I * rb_h;
  const uint16_t* s_gate = reinterpret_cast<const uint16_t*>(q_down + H * rb_i);
  const uint16_t* s_up = s_gate + I * (H / G);
  const uint16_t* s_down = s_up + I * (H / G);
  std::memset(out, 0, (size_t)L.bytes);
  const bool three = b == 3;
  for (int64_t t = 0; t < L.gu_tiles; ++t)
    for (int lane = 0; lane < 64; ++lane) {
      const bool up = lane >= 32;
      const int64_t row = 32 * t + (lane & 31);
      const uint8_t* src = (up ? q_up : q_gate) + row * rb_h;
      for (int64_t c = 0; c < L.gu_chunks; ++c) {
        const int64_t blk = (t * L.gu_chunks + c) * 64 + lane;
        lane_words_lowbit(src, c * kc, b, out + L.off_gu_codes + blk * 16, three ? out + L.off_gu_hi + blk * 8 : nullptr);
      }
      const uint16_t* srow = (up ? s_up : s_gate) + row * (H / G);
      for (int64_t g = 0; g < H / G; ++g)
        std::memcpy(out + L.off_gu_scales + ((t * L.gu_groups + g) * 64 + lane) * 2, srow + g, 2);
    }
  for (int64_t t = 0; t < L.dn_tiles; ++t)
    for (int lane = 0; lane < 64; ++lane) {
      const int64_t row = 64 * t + lane;
      const uint8_t* src = q_down + row * rb_i;
      for (int64_t c = 0; c < L.dn_chunks; ++c) {
        const int64_t blk = (t * L.dn_chunks + c) * 64 + lane;
        lane_words_lowbit(src, c * kc, b, out + L.off_dn_codes + blk * 16, three ? out + L.off_dn_hi + blk * 8 : nullptr);
      }
      const uint16_t* srow = s_down + row * (I / G);
      for (int64_t g = 0; g < I / G; ++g)
        std::memcpy(out + L.off_dn_scales + ((t * L.dn_groups + g) * 64 + lane) * 2, srow + g, 2);
    }
}

void repack_expert(const Layout& L, const uint8_t* canon, uint8_t* out) {
  if (L.bits == 4)
    repack_expert4(L, canon, out);
  else
    repack_expert_lowbit(L, canon, out);
}

void cache_policy_step(int32_t E, int32_t n_slots, double decay, int32_t max_promotions,
                       const int64_t* counts, double* score, int32_t* slot_of,
                       std::vector<Promotion>* promoted, std::vector<int32_t>* evicted) {
  promoted->clear();
  evicted->clear();
  for (int32_t e = 0; e < E; ++e) score[e] = decay * score[e] + (double)counts[e];

  std::vector<int32_t> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (score[a] != score[b]) return score[a] > score[b];
    bool ra = slot_of[a] >= 0, rb = slot_of[b] >= 0;
    if (ra != rb) return ra;
    return a < b;
  });
  std::vector<char> wanted(E, 0);
  for (int32_t i = 0; i < n_slots && i < E; ++i) wanted[order[i]] = 1;

  std::vector<int32_t> promos, victims;
  for (int32_t e = 0; e < E; ++e) {
    if (wanted[e] && slot_of[e] < 0) promos.push_back(e);
    if (!wanted[e] && slot_of[e] >= 0) victims.push_back(e);
  }
  std::sort(promos.begin(), promos.end(), [&](int32_t a, int32_t b) {
    if (score[a] != score[b]) return score[a] > score[b];
    return a < b;
  });
  std::sort(victims.begin(), victims.end(), [&](int32_t a, int32_t b) {
    if (score[a] != score[b]) return score[a] < score[b];
    return a > b;
  });
  std::vector<char> used(n_slots > 0 ? n_slots : 0, 0);
  for (int32_t e = 0; e < E; ++e)
    if (slot_of[e] >= 0 && slot_of[e] < n_slots) used[slot_of[e]] = 1;
  int32_t next_free = 0;
  size_t vi = 0;
  int32_t n = 0;
  for (int32_t p : promos) {
    if (n >= max_promotions) break;
    while (next_free < n_slots && used[next_free]) ++next_free;
    int32_t slot;
    if (next_free < n_slots) {
      slot = next_free;
      used[slot] = 1;
    } else if (vi < victims.size()) {
      int32_t v = victims[vi++];
      slot = slot_of[v];
      slot_of[v] = -1;
      evicted->push_back(v);
    } else {
      break;
    }
    slot_of[p] = slot;
    promoted->push_back({p, slot});
    ++n;
  }
}

bool cache_set_resident(int32_t E, int32_t n_slots, double decay, const int64_t* counts, const int32_t* want,
                        double* score, int32_t* slot_of, std::vector<Promotion>* promoted,
                        std::vector<int32_t>* evicted) {
  promoted->clear();
  evicted->clear();
  int32_t n_want = 0;
  for (int32_t e = 0; e < E; ++e) n_want += want[e] != 0;
  if (n_want > n_slots) return false;
  for (int32_t e = 0; e < E; ++e) score[e] = decay * score[e] + (double)counts[e];
  std::vector<char> used(n_slots > 0 ? n_slots : 0, 0);
  for (int32_t e = 0; e < E; ++e) {
    if (slot_of[e] < 0) continue;
    if (want[e]) {
      used[slot_of[e]] = 1;
    } else {
      slot_of[e] = -1;
      evicted->push_back(e);
    }
  }
  int32_t next_free = 0;
  for (int32_t e = 0; e < E; ++e) {
    if (!want[e] || slot_of[e] >= 0) continue;
    while (used[next_free]) ++next_free;  // a free slot exists: n_want <= n_slots
    used[next_free] = 1;
    slot_of[e] = next_free;
    promoted->push_back({e, next_free});
  }
  return true;
}

}  // namespace moe
