// Command-line driver of the library's host-side logic (host_logic.cpp), built on its
// own with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_logic_native.py. One command per input line; every answer is one
// line. Floats travel as C99 hex literals, so values cross the pipe exactly.
//
//   layout H I G B                    -> the Layout fields (B bits per code)
//   repack H I G B in_path out_path   -> internal blob of the canonical blob in in_path
//   policy E S decay maxp             -> then lines: counts, score, slot_of
//                                        answers: score, slot_of, promoted pairs, evicted
//   setres E S decay                  -> then lines: counts, score, slot_of, want
//   check H I E k G L act T S gmin stage bits -> "OK" or the reason
//   ffn H I G M threads hbf16 blob_path x_path o_path -> the host expert FFN (host_ffn.cpp) of
//                                     the canonical 4-bit blob on M fp32 token rows (h rounded to
//                                     bf16 when hbf16 is 1), o rows written
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>
#include <type_traits>
#include <vector>

#include "host_ffn.h"
#include "host_logic.h"

using namespace moe;

template <typename T>
static std::vector<T> read_line(size_t n) {
  std::string line;
  std::getline(std::cin, line);
  std::istringstream in(line);
  std::vector<T> v(n);
  for (size_t i = 0; i < n; ++i) {
    std::string tok;
    in >> tok;
    if constexpr (std::is_floating_point<T>::value)
      v[i] = std::strtod(tok.c_str(), nullptr);
    else
      v[i] = (T)std::strtoll(tok.c_str(), nullptr, 10);
  }
  return v;
}

static void print_scores(const std::vector<double>& s) {
  for (size_t i = 0; i < s.size(); ++i) std::printf("%s%a", i ? " " : "", s[i]);
  std::printf("\n");
}

static void print_ints(const int32_t* v, size_t n) {
  for (size_t i = 0; i < n; ++i) std::printf("%s%d", i ? " " : "", v[i]);
  std::printf("\n");
}

static void print_moves(const std::vector<Promotion>& p, const std::vector<int32_t>& ev) {
  for (size_t i = 0; i < p.size(); ++i) std::printf("%s%d:%d", i ? " " : "", p[i].expert, p[i].slot);
  std::printf("\n");
  print_ints(ev.data(), ev.size());
}

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    if (cmd == "layout") {
      int64_t H, I, G, B;
      in >> H >> I >> G >> B;
      const Layout L = make_layout(H, I, G, B);
      std::printf("%lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld %lld\n", (long long)L.kc,
                  (long long)L.gu_tiles, (long long)L.gu_chunks, (long long)L.gu_groups, (long long)L.dn_tiles,
                  (long long)L.dn_chunks, (long long)L.dn_groups, (long long)L.off_gu_codes, (long long)L.off_gu_hi,
                  (long long)L.off_gu_scales, (long long)L.off_dn_codes, (long long)L.off_dn_hi,
                  (long long)L.off_dn_scales, (long long)L.bytes, (long long)L.canonical_bytes);
    } else if (cmd == "repack") {
      int64_t H, I, G, B;
      std::string ip, op;
      in >> H >> I >> G >> B >> ip >> op;
      const Layout L = make_layout(H, I, G, B);
      std::vector<uint8_t> src((size_t)L.canonical_bytes), dst((size_t)L.bytes);
      FILE* f = std::fopen(ip.c_str(), "rb");
      if (!f || std::fread(src.data(), 1, src.size(), f) != src.size()) return 2;
      std::fclose(f);
      repack_expert(L, src.data(), dst.data());
      f = std::fopen(op.c_str(), "wb");
      if (!f || std::fwrite(dst.data(), 1, dst.size(), f) != dst.size()) return 3;
      std::fclose(f);
      std::printf("done\n");
    } else if (cmd == "policy" || cmd == "setres") {
      int E, S, maxp = 0;
      std::string dtok;
      in >> E >> S >> dtok;
      if (cmd == "policy") in >> maxp;
      const double decay = std::strtod(dtok.c_str(), nullptr);
      std::vector<int64_t> counts = read_line<int64_t>(E);
      std::vector<double> score = read_line<double>(E);
      std::vector<int32_t> slot_of = read_line<int32_t>(E);
      std::vector<Promotion> prom;
      std::vector<int32_t> ev;
      if (cmd == "policy") {
        cache_policy_step(E, S, decay, maxp, counts.data(), score.data(), slot_of.data(), &prom, &ev);
      } else {
        std::vector<int32_t> want = read_line<int32_t>(E);
        if (!cache_set_resident(E, S, decay, counts.data(), want.data(), score.data(), slot_of.data(), &prom, &ev)) {
          std::printf("refused\n\n\n\n");
          std::fflush(stdout);
          continue;
        }
      }
      print_scores(score);
      print_ints(slot_of.data(), slot_of.size());
      print_moves(prom, ev);
    } else if (cmd == "check") {
      moe_config c{};
      in >> c.hidden >> c.inter >> c.num_experts >> c.top_k >> c.group_size >> c.num_layers >> c.act_dtype >>
          c.max_tokens >> c.hbm_slots >> c.gemm_min_tokens >> c.prefill_stage_slots >> c.weight_bits;
      const std::string why = check_config(c);
      std::printf("%s\n", why.empty() ? "OK" : why.c_str());
    } else if (cmd == "ffn") {
      int64_t H, I, G;
      int M, threads, hbf16;
      std::string bp, xp, op;
      in >> H >> I >> G >> M >> threads >> hbf16 >> bp >> xp >> op;
      const Layout L = make_layout(H, I, G, 4);
      std::vector<uint8_t> canon((size_t)L.canonical_bytes), blob((size_t)L.bytes);
      std::vector<float> x((size_t)M * H), h((size_t)M * I), o((size_t)M * H);
      FILE* f = std::fopen(bp.c_str(), "rb");
      if (!f || std::fread(canon.data(), 1, canon.size(), f) != canon.size()) return 4;
      std::fclose(f);
      f = std::fopen(xp.c_str(), "rb");
      if (!f || std::fread(x.data(), sizeof(float), x.size(), f) != x.size()) return 5;
      std::fclose(f);
      repack_expert(L, canon.data(), blob.data());
      HostPool pool(threads);
      host_expert_ffn(L, blob.data(), x.data(), M, h.data(), o.data(), hbf16 != 0, pool);
      f = std::fopen(op.c_str(), "wb");
      if (!f || std::fwrite(o.data(), sizeof(float), o.size(), f) != o.size()) return 6;
      std::fclose(f);
      std::printf("done\n");
    } else if (cmd.empty()) {
      continue;
    } else {
      std::printf("unknown\n");
    }
    std::fflush(stdout);
  }
  return 0;
}
