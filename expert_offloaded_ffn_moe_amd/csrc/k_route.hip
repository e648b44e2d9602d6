// Routing kernels for gfx950: router logits, per-group activation sums, top-k
// gate choice, grouping of assignments by expert (counts, offsets, stable
// permutation, active-expert list, link counters) and the gate-weighted combine.
//
// The routed choice follows page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存",
// section "显存缺口从哪里来" (a few experts per token per layer, picked at run
// time); softmax scores, ties to the lower expert id and renormalisation over
// the k chosen are the plain reading of it.
//
// Decode (T <= 64, T*k <= 256) runs as one launch: router blocks compute the
// logits, and the last block to finish (an atomic arrival counter, no waiting)
// does the top-k and the grouping. Larger T: top-k with per-block counts, then a
// block-parallel scatter (two launches).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>

#include "copy_dev.h"
#include "kernels.h"
#include "route_dev.h"
#include "wave.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ----------------------------------------------------------------------------- router

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;

__device__ __forceinline__ float dot16(const u32x4& w, const u32x4& x, float s, bool bf16) {
  if (bf16) {
    s = dot2_bf16(w.x, x.x, s);
    s = dot2_bf16(w.y, x.y, s);
    s = dot2_bf16(w.z, x.z, s);
    s = dot2_bf16(w.w, x.w, s);
  } else {
    s = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), s);
    s = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), s);
    s = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), s);
    s = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), s);
  }
  return s;
}

// Router rows, split over RW waves each (RW = 1, 2, 4 or 8, so that a wave holds at
// most NCH 16-byte chunks of its part of the row in registers and a launch spreads
// over enough CUs: kRouterWaves waves per workgroup take kRouterWaves / RW rows).
// Lane l of a part owns chunks c0 + l, c0 + l + 64, ... of it. Per token, in
// passes of up to kRouterTok tokens whose x chunks are all loaded before the dot
// products: fp32 sums in chunk order per lane, a fixed DPP tree across the lanes,
// then the RW parts added in order by the row's first wave.
// NCH == 0: parts longer than 8 * 64 chunks, a plain strided loop.
constexpr int kRouterTok = 4;

template <int BF16, int NCH>
__device__ __forceinline__ void router_rows(const RouterArgs& a, int bid, float (*part)[kRouterTok]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int RW = a.rw;
  const int e = bid * (kRouterWaves / RW) + wave / RW, pt = wave % RW;
  const bool row_ok = e < a.E;
  const int esz = BF16 ? 2 : 4;
  const int nchunk = a.H * esz / 16;
  const int per = (nchunk + RW - 1) / RW;
  const int c0 = pt * per, c1 = min(nchunk, c0 + per);
  gu32x4* wrow = (gu32x4*)(static_cast<const char*>(a.w) + (size_t)min(e, a.E - 1) * a.H * esz);
  const float bias = (row_ok && a.b) ? a.b[e] : 0.f;
  constexpr int NW = NCH > 0 ? NCH : 1;
  u32x4 wv[NW];
  if (NCH > 0) {
#pragma unroll
    for (int i = 0; i < NW; ++i) wv[i] = wrow[min(c0 + lane + 64 * i, nchunk - 1)];
  }
  for (int t0 = 0; t0 < a.T; t0 += kRouterTok) {
    const int nt = min(kRouterTok, a.T - t0);
    float sum[kRouterTok];
    if (NCH > 0) {
      u32x4 xv[kRouterTok][NW];
#pragma unroll
      for (int tt = 0; tt < kRouterTok; ++tt) {
        if (tt < nt) {
          gu32x4* xrow = (gu32x4*)(static_cast<const char*>(a.x) + (size_t)(t0 + tt) * a.H * esz);
#pragma unroll
          for (int i = 0; i < NW; ++i) xv[tt][i] = xrow[min(c0 + lane + 64 * i, nchunk - 1)];
        }
      }
#pragma unroll
      for (int tt = 0; tt < kRouterTok; ++tt) {
        float v = 0.f;
        if (tt < nt) {
#pragma unroll
          for (int i = 0; i < NW; ++i) {
            const float d = dot16(wv[i], xv[tt][i], 0.f, BF16);
            v += (c0 + lane + 64 * i < c1) ? d : 0.f;
          }
        }
        sum[tt] = wave_sum(v);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < kRouterTok; ++tt) {
        float v = 0.f;
        if (tt < nt) {
          gu32x4* xrow = (gu32x4*)(static_cast<const char*>(a.x) + (size_t)(t0 + tt) * a.H * esz);
          for (int c = c0 + lane; c < c1; c += 64) {
            const u32x4 wc = wrow[c], xc = xrow[c];
            v = dot16(wc, xc, v, BF16);
          }
        }
        sum[tt] = wave_sum(v);
      }
    }
    if (RW == 1) {
      if (lane < nt && row_ok) {
        float v = sum[0];
#pragma unroll
        for (int tt = 1; tt < kRouterTok; ++tt) v = lane == tt ? sum[tt] : v;
        st_shared_dev(a.logits + (size_t)(t0 + lane) * a.E + e, v + bias);
      }
    } else {
      if (lane < kRouterTok) {
        float v = sum[0];
#pragma unroll
        for (int tt = 1; tt < kRouterTok; ++tt) v = lane == tt ? sum[tt] : v;
        part[wave][lane] = v;
      }
      __syncthreads();
      if (pt == 0 && lane < nt && row_ok) {
        float v = 0.f;
        for (int q = 0; q < RW; ++q) v += part[wave + q][lane];
        st_shared_dev(a.logits + (size_t)(t0 + lane) * a.E + e, v + bias);
      }
      __syncthreads();
    }
  }
}

// Chunks per lane of the router's row parts (0: the strided loop).
inline int router_nch(const RouterArgs& a, int act_bf16) {
  const int nchunk = a.H * (act_bf16 ? 2 : 4) / 16;
  const int per = (nchunk + a.rw - 1) / a.rw;
  const int n = (per + 63) / 64;
  return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 0;
}

// sum of x[t][g*G .. (g+1)*G) for flat index gid = t * (H/G) + g (bf16 x)
__device__ __forceinline__ void xsum_one(const RouterArgs& a, int gid) {
  const int ng = a.H / a.G;
  const int t = gid / ng, g = gid % ng;
  const uint4* src =
      reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * a.H + (size_t)g * a.G);
  float s = 0.f;
  for (int c = 0; c < a.G / 8; ++c) {
    const uint4 v = src[c];
    s += bf16_lo(v.x);
    s += bf16_hi(v.x);
    s += bf16_lo(v.y);
    s += bf16_hi(v.y);
    s += bf16_lo(v.z);
    s += bf16_hi(v.z);
    s += bf16_lo(v.w);
    s += bf16_hi(v.w);
  }
  a.xsum[gid] = s;
}

// Any T: blocks [0, router_blocks) take router rows, the rest the group sums.
template <int BF16, int NCH>
__global__ __launch_bounds__(512) void k_router(RouterArgs a) {
  __shared__ float part[kRouterWaves][kRouterTok];
  if ((int)blockIdx.x < a.router_blocks) {
    router_rows<BF16, NCH>(a, blockIdx.x, part);
  } else if (BF16) {
    const int gid = (blockIdx.x - a.router_blocks) * 512 + threadIdx.x;
    if (gid < a.T * (a.H / a.G)) xsum_one(a, gid);
  }
}

void launch_router(const RouterArgs& a, int act_bf16, const Timing& tm, hipStream_t s) {
  const int xs_blocks = (act_bf16 && a.xsum) ? (a.T * (a.H / a.G) + 511) / 512 : 0;
  const int grid = a.router_blocks + xs_blocks;
  if (grid == 0) return;
  const int nch = router_nch(a, act_bf16);
#define ROUTER(B, N) launch_timed(k_router<B, N>, dim3(grid), dim3(512), 0, s, tm, a)
#define ROUTER_NCH(B) \
  if (nch == 1)       \
    ROUTER(B, 1);     \
  else if (nch == 2)  \
    ROUTER(B, 2);     \
  else if (nch == 4)  \
    ROUTER(B, 4);     \
  else if (nch == 8) \
    ROUTER(B, 8); \
  else                \
    ROUTER(B, 0);
  if (act_bf16) {
    ROUTER_NCH(1)
  } else {
    ROUTER_NCH(0)
  }
#undef ROUTER_NCH
#undef ROUTER
}

// ----------------------------------------------------------------------------- align / permute


// Exclusive scan of one int per thread over a 1024-thread block; *total = sum.
__device__ __forceinline__ int block_exscan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int tw = tmp[w];
    base += (w < wave) ? tw : 0;
    tot += tw;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// LDS of the fused decode routing kernel's tail (the last block to arrive).
struct DecodeShared {
  int is_host[1024];
  const uint8_t* wptr[1024];
  int ids_small[kRouteSmallMaxAssign];
  float part[kRouterWaves][kRouterTok];  // router row parts
  int a_cnt[kRouteSmallMaxAssign], a_off[kRouteSmallMaxAssign];  // per assignment: its expert's count, offset
  uint64_t m[kRouteSmallMaxAssign / 64][10], vmask[kRouteSmallMaxAssign / 64];
  uint64_t lead[kRouteSmallMaxAssign / 64], hostm[kRouteSmallMaxAssign / 64];
  int last;
};

// The grouping for n = T*k <= 64 assignments, lane i of a wave holding assignment
// i: the id-bit masks stay in scalar registers and every result (positions, expert
// counts and offsets, active list, descriptors) comes from count_below on them.
// Every wave takes the same masks; wave 0 places the assignments and writes the
// active list and descriptors while the other waves write the per-expert counts
// and offsets, 64 experts each (one wave doing all of it spent 1.9 us on those for
// a 384-expert layer). The shortest code path, for the common decode batches.
__device__ __forceinline__ void align_one(const RouteArgs& a, DecodeShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int n = a.T * a.k, E = a.E, NB = (E + 63) >> 6;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool valid = lane < n;
  const int e = valid ? sh.ids_small[lane] : 0;
  const uint64_t vm = __ballot(valid);
  uint64_t m[kIdBits];
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) m[b] = __ballot(valid && ((e >> b) & 1));
  if (wave > 0) {
    // the other waves (each with the same masks) write the expert counts and
    // offsets, 64 experts each, beside wave 0's placement and descriptors
    for (int b = wave - 1; b < NB; b += nw - 1) {
      const int ee = 64 * b + lane;
      uint64_t q;
      const int lt = count_below(ee, m, vm, nbits, &q);
      if (ee < E) {
        a.offsets[ee] = lt;
        a.counts[ee] = __popcll(q);
      }
    }
    return;
  }
  uint64_t eq;
  const int off = count_below(e, m, vm, nbits, &eq);
  const int rank = __popcll(eq & lt_mask), cnt = __popcll(eq);
  if (valid) {
    a.sorted[off + rank] = lane;
    a.inv[lane] = off + rank;
    if (a.aptr) a.aptr[lane] = sh.wptr[e];
  }
  const bool host = valid && sh.is_host[e] != 0;
  const uint64_t lead = __ballot(valid && rank == 0), hm = __ballot(host);
  const int n_host = __popcll(lead & hm), n_act = __popcll(lead), misses = __popcll(hm);
  if (lane == 0) a.offsets[E] = n;
  if (valid && rank == 0) {
    uint64_t q;
    const int ap = (host ? 0 : n_host) + count_below(e, m, lead & (host ? hm : ~hm), nbits, &q);
    a.active[ap] = e;
    atomicAdd(reinterpret_cast<unsigned long long*>(a.counts_acc + e), (unsigned long long)cnt);
    WorkDesc* d = a.work + ap;
    d->w = sh.wptr[e];
    d->p0 = off;
    d->M = skipped(a, host) ? 0 : cnt;
    const float inv_k = 1.f / (float)a.k;
    uint64_t mm = eq;
    for (int j = 0; mm && j < kDescTok; ++j) {
      d->tok[j] = (int)(((float)__builtin_ctzll(mm) + 0.5f) * inv_k);  // i / k: margin to the next integer >= 1/(2k)
      mm &= mm - 1;
    }
  }
  for (int sl = n_act + lane; sl < min(E, n); sl += 64) a.work[sl].M = 0;
  if (lane == 0) {
    a.n_active[0] = n_act;
    a.n_active[1] = n_host;
    unsigned long long* st = reinterpret_cast<unsigned long long*>(a.stats);
    atomicAdd(st + ST_FORWARDS, 1ull);
    atomicAdd(st + ST_TOKENS, (unsigned long long)a.T);
    atomicAdd(st + ST_HITS, (unsigned long long)(n - misses));
    atomicAdd(st + ST_MISSES, (unsigned long long)misses);
    atomicAdd(st + ST_BYTES_HBM, (unsigned long long)((int64_t)(n_act - n_host) * a.expert_bytes));
    atomicAdd(st + ST_BYTES_HOST, (unsigned long long)((int64_t)n_host * a.expert_bytes));
  }
}

// The grouping of n = T*k <= kRouteSmallMaxAssign assignments (ids in
// sh.ids_small, sh.is_host / sh.wptr loaded) by all threads of the block.
// Assignment i = 64c + lane sits in chunk c, handled by wave c. Each chunk's
// wave takes one ballot per id bit; from those masks any thread finds, for an
// id v, how many assignments have a lower id (v's offset) and which ones have
// id v (ranks and counts). The work is split over the waves so that the short
// one-off code paths run side by side: chunk waves place the assignments, then
// every thread writes expert counts/offsets or, for the first assignment of an
// expert, its active-list entry (host-read experts first, ascending ids in each
// part) and GEMV work descriptor.
__device__ __forceinline__ void align_small(const RouteArgs& a, DecodeShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T * a.k, E = a.E, NC = (n + 63) >> 6;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (wave < NC) {
    const int i = 64 * wave + lane;
    const bool valid = i < n;
    const int e = valid ? sh.ids_small[i] : 0;
    const uint64_t vm = __ballot(valid);
    uint64_t mb[kIdBits];
#pragma unroll
    for (int b = 0; b < kIdBits; ++b) mb[b] = __ballot(valid && ((e >> b) & 1));
    if (lane == 0) {
      sh.vmask[wave] = vm;
#pragma unroll
      for (int b = 0; b < kIdBits; ++b) sh.m[wave][b] = mb[b];
    }
  }
  __syncthreads();
  if (wave < NC) {  // positions in the permutation, leaders, host flags
    const int i = 64 * wave + lane;
    const bool valid = i < n;
    const int e = valid ? sh.ids_small[i] : 0;
    int lt = 0, rank = 0, cnt = 0;
    for (int c = 0; c < NC; ++c) {
      uint64_t eq;
      lt += count_below(e, sh.m[c], sh.vmask[c], nbits, &eq);
      cnt += __popcll(eq);
      rank += c < wave ? __popcll(eq) : (c == wave ? __popcll(eq & lt_mask) : 0);
    }
    if (valid) {
      a.sorted[lt + rank] = i;
      a.inv[i] = lt + rank;
      sh.a_cnt[i] = cnt;
      sh.a_off[i] = lt;
      if (a.aptr) a.aptr[i] = sh.wptr[e];
    }
    const uint64_t ld = __ballot(valid && rank == 0), hm = __ballot(valid && sh.is_host[e] != 0);
    if (lane == 0) {
      sh.lead[wave] = ld;
      sh.hostm[wave] = hm;
    }
  }
  __syncthreads();
  int n_host = 0, n_act = 0, misses = 0;
  for (int c = 0; c < NC; ++c) {
    n_host += __popcll(sh.lead[c] & sh.hostm[c]);
    n_act += __popcll(sh.lead[c]);
    misses += __popcll(sh.hostm[c]);
  }
  // counts and offsets of every expert
  for (int e = tid; e < E; e += blockDim.x) {
    int lt = 0, cnt = 0;
    for (int c = 0; c < NC; ++c) {
      uint64_t eq;
      lt += count_below(e, sh.m[c], sh.vmask[c], nbits, &eq);
      cnt += __popcll(eq);
    }
    a.offsets[e] = lt;
    a.counts[e] = cnt;
  }
  if (tid == 0) a.offsets[E] = n;
  // active list and work descriptors, one thread per expert (its first assignment)
  if (tid < n && ((sh.lead[tid >> 6] >> lane) & 1)) {
    const int c0 = tid >> 6;
    const int e = sh.ids_small[tid];
    const bool host = (sh.hostm[c0] >> lane) & 1;
    int ap = host ? 0 : n_host;
    for (int c = 0; c < NC; ++c) {
      uint64_t eq;
      ap += count_below(e, sh.m[c], sh.lead[c] & (host ? sh.hostm[c] : ~sh.hostm[c]), nbits, &eq);
    }
    const int cnt = sh.a_cnt[tid];
    a.active[ap] = e;
    atomicAdd(reinterpret_cast<unsigned long long*>(a.counts_acc + e), (unsigned long long)cnt);
    WorkDesc* d = a.work + ap;
    d->w = sh.wptr[e];
    d->p0 = sh.a_off[tid];
    d->M = skipped(a, host) ? 0 : cnt;
    const float inv_k = 1.f / (float)a.k;
    int j = 0;
    for (int c = 0; c < NC && j < kDescTok; ++c) {
      uint64_t mm;
      count_below(e, sh.m[c], sh.vmask[c], nbits, &mm);
      while (mm && j < kDescTok) {
        const int i = 64 * c + __builtin_ctzll(mm);
        d->tok[j++] = (int)(((float)i + 0.5f) * inv_k);  // i / k: the margin to the next integer is >= 1/(2k)
        mm &= mm - 1;
      }
    }
  }
  // unused GEMV slots up to min(E, T*k) (the GEMV grid) have no rows
  for (int sl = n_act + tid; sl < min(E, n); sl += blockDim.x) a.work[sl].M = 0;
  if (tid == 0) {
    a.n_active[0] = n_act;
    a.n_active[1] = n_host;
    unsigned long long* st = reinterpret_cast<unsigned long long*>(a.stats);
    atomicAdd(st + ST_FORWARDS, 1ull);
    atomicAdd(st + ST_TOKENS, (unsigned long long)a.T);
    atomicAdd(st + ST_HITS, (unsigned long long)(n - misses));
    atomicAdd(st + ST_MISSES, (unsigned long long)misses);
    atomicAdd(st + ST_BYTES_HBM, (unsigned long long)((int64_t)(n_act - n_host) * a.expert_bytes));
    atomicAdd(st + ST_BYTES_HOST, (unsigned long long)((int64_t)n_host * a.expert_bytes));
  }
}


// Decode routing in one launch. Blocks [0, router_blocks): kRouterWaves / rw expert
// rows each (rw waves per row); then xsum blocks; every block then arrives on the
// counter, and the last one (which reads every other block's logits with loads that
// miss its L2, after their write-through stores: no fences) picks the top-k of
// every token (one wave per token) and groups the assignments with its waves.
// NCH: 16-byte chunks per lane of a wave's part of a router row (1, 2, 4, 8; 0 =
// longer parts).
// One instance per row length, so the kernel's registers are those of its own
// router path (the longest rows' path needs more of them than the tail).
template <int BF16, int NCH>
__global__ __launch_bounds__(512) void k_route_decode(RouteArgs a, RouterArgs r, unsigned* counter) {
  __shared__ DecodeShared sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bid = blockIdx.x;
  // residency and blob tables for the grouping step, loaded while the router
  // runs (only the last block to arrive uses them)
  for (int e = threadIdx.x; e < a.E; e += 512) {
    sh.is_host[e] = a.is_host[e];
    sh.wptr[e] = a.wptr[e];
  }
  if (bid < r.router_blocks) {
    router_rows<BF16, NCH>(r, bid, sh.part);
  } else if (BF16 && r.xsum) {
    const int gid = (bid - r.router_blocks) * 512 + threadIdx.x;
    if (gid < r.T * (r.H / r.G)) xsum_one(r, gid);
  }
  if (!arrive_last(counter, gridDim.x, &sh.last)) return;
  for (int t = wave; t < a.T; t += 8)
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.k, lane, a.ids + (size_t)t * a.k, a.wts + (size_t)t * a.k,
              sh.ids_small + t * a.k);
  __syncthreads();
  if (a.T * a.k <= 64) {
    align_one(a, sh);
  } else {
    align_small(a, sh);
  }
}

void launch_route_decode(const RouteArgs& a, const RouterArgs& r, int act_bf16, unsigned* counter,
                         const Timing& tm, hipStream_t s) {
  const int xs_blocks = (act_bf16 && r.xsum) ? (r.T * (r.H / r.G) + 511) / 512 : 0;
  const int grid = std::max(1, r.router_blocks + xs_blocks);
  const int nch = router_nch(r, act_bf16);
#define ROUTE_DECODE(B, N) launch_timed(k_route_decode<B, N>, dim3(grid), dim3(512), 0, s, tm, a, r, counter)
#define ROUTE_DECODE_NCH(B)   \
  if (nch == 1)               \
    ROUTE_DECODE(B, 1);       \
  else if (nch == 2)          \
    ROUTE_DECODE(B, 2);       \
  else if (nch == 4)          \
    ROUTE_DECODE(B, 4);       \
  else if (nch == 8) \
    ROUTE_DECODE(B, 8); \
  else                        \
    ROUTE_DECODE(B, 0);
  if (act_bf16) {
    ROUTE_DECODE_NCH(1)
  } else {
    ROUTE_DECODE_NCH(0)
  }
#undef ROUTE_DECODE_NCH
#undef ROUTE_DECODE
}


// ----------------------------------------------------------------------------- predictive prefetch

// Prediction of a prefetch. Blocks [0, router_blocks): router rows, 8 per block, into
// a.logits (none when the logits are given); every block arrives on the counter,
// and the last one picks each token's kp best experts (the routing's order: logit
// descending, id ascending). The predicted set is the first P distinct candidates,
// in token order then candidate order, whose weights are read from host memory
// without the prefetch (their host copy, or a prefetch slot of this layer). A slot
// whose expert is predicted again keeps it; every other slot gives its expert back
// to its host copy (where the table still points at the slot: a cache update may
// have rewritten the entry) and is free; each predicted expert not yet in a slot
// takes the lowest free slot and goes on the copy list.
template <int BF16, int NCH>
__global__ __launch_bounds__(512) void k_predict(PrefetchArgs a, RouterArgs r, unsigned* counter) {
  __shared__ int32_t ids[kPrefetchMaxCand];
  __shared__ float wts[kPrefetchMaxCand];
  __shared__ int16_t in_slot[kPrefetchMaxE];  // slot + 1 of an expert the table reads from a slot, else 0
  __shared__ uint8_t chosen[kPrefetchMaxE];
  __shared__ float part[kRouterWaves][kRouterTok];
  __shared__ int last;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < r.router_blocks) router_rows<BF16, NCH>(r, blockIdx.x, part);
  if (!arrive_last(counter, gridDim.x, &last)) return;
  for (int e = threadIdx.x; e < a.E; e += 512) {
    in_slot[e] = 0;
    chosen[e] = 0;
  }
  for (int t = wave; t < a.T; t += 8)
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.kp, lane, ids + t * a.kp, wts + t * a.kp, nullptr);
  __syncthreads();
  if (threadIdx.x != 0) return;
  for (int i = 0; i < a.P; ++i) {
    const int e = a.occ[i];
    if (e >= 0 && a.wptr[e] == a.slots + (size_t)i * a.bytes) in_slot[e] = (int16_t)(i + 1);
  }
  int n = 0;
  for (int c = 0; c < a.T * a.kp && n < a.P; ++c) {
    const int e = ids[c];
    if (chosen[e] || !(a.is_host[e] != 0 || in_slot[e] != 0)) continue;
    chosen[e] = 1;
    if (a.predicted_out) a.predicted_out[n] = e;
    ++n;
  }
  if (a.predicted_out)
    for (int i = n; i < a.P; ++i) a.predicted_out[i] = -1;
  for (int i = 0; i < a.P; ++i) {  // slots kept, and slots given back
    const int e = a.occ[i];
    if (e < 0) continue;
    if (in_slot[e] == i + 1) {
      if (chosen[e]) {
        chosen[e] = 2;  // stays in slot i
        continue;
      }
      a.wptr[e] = a.host_pool + (size_t)e * a.bytes;
      a.is_host[e] = 1;
    }
    a.occ[i] = -1;
  }
  int m = 0, free_slot = 0;
  for (int c = 0; c < a.T * a.kp; ++c) {  // the new ones, in prediction order
    const int e = ids[c];
    if (chosen[e] != 1) continue;
    chosen[e] = 2;
    while (a.occ[free_slot] >= 0) ++free_slot;  // a free slot exists: at most P are chosen
    a.occ[free_slot] = e;
    a.list[m++] = free_slot;
  }
  a.list[a.P] = m;
  atomicAdd(reinterpret_cast<unsigned long long*>(a.stats + ST_PREFETCHED), (unsigned long long)m);
}

// The copies: block (j, part) copies part `part` of the expert going into slot
// list[j] from its host copy; block 0 points the table at the new slots. Forwards
// of the layer start only after this kernel has finished, so the order of the two
// inside it does not matter.
__global__ __launch_bounds__(kCopyThreads) void k_prefetch_copy(PrefetchArgs a) {
  const int m = a.list[a.P];
  if (blockIdx.x == 0 && (int)threadIdx.x < m) {
    const int slot = a.list[threadIdx.x];
    const int e = a.occ[slot];
    a.wptr[e] = a.slots + (size_t)slot * a.bytes;
    a.is_host[e] = 0;
  }
  const int j = blockIdx.x / a.blocks_per_expert, part = blockIdx.x % a.blocks_per_expert;
  if (j >= m) return;
  const int slot = a.list[j];
  const int e = a.occ[slot];
  const int64_t n16 = a.bytes / 16;
  const int64_t u0 = (int64_t)part * kCopyUnits, u1 = u0 + kCopyUnits < n16 ? u0 + kCopyUnits : n16;
  copy_units(a.host_pool + (size_t)e * a.bytes, a.slots + (size_t)slot * a.bytes, u0, u1);
}

void launch_prefetch(PrefetchArgs a, const RouterArgs& r, int act_bf16, unsigned* counter, hipStream_t s) {
  a.blocks_per_expert = (int)((a.bytes / 16 + kCopyUnits - 1) / kCopyUnits);
  const int grid = std::max(1, r.router_blocks);
  const int nch = router_nch(r, act_bf16);
#define PREDICT(B, N) hipLaunchKernelGGL((k_predict<B, N>), dim3(grid), dim3(512), 0, s, a, r, counter)
#define PREDICT_NCH(B)  \
  if (nch == 1)         \
    PREDICT(B, 1);      \
  else if (nch == 2)    \
    PREDICT(B, 2);      \
  else if (nch == 4)    \
    PREDICT(B, 4);      \
  else if (nch == 8) \
    PREDICT(B, 8); \
  else                  \
    PREDICT(B, 0);
  if (act_bf16) {
    PREDICT_NCH(1)
  } else {
    PREDICT_NCH(0)
  }
#undef PREDICT_NCH
#undef PREDICT
  hipLaunchKernelGGL(k_prefetch_copy, dim3(a.P * a.blocks_per_expert), dim3(kCopyThreads), 0, s, a);
}

// ----------------------------------------------------------------------------- multi-block grouping

// Top-k and grouping for any number of assignments, over blocks of kGroupTokens
// tokens. k_topk_count: each block picks its tokens' experts (one wave per
// token) and counts them per expert; the last block to arrive turns the block
// counts into expert counts, offsets and per-block bases (expert e's rows from
// block b start at offsets[e] + the counts of e in blocks before b), and writes
// the active list (host-read experts first), GEMV descriptors, GEMM row tiles,
// counters and stats. k_scatter: each block places its assignments at its bases
// plus their rank among the block's earlier assignments to the same expert, so
// the permutation is the stable one; it also fills the descriptors' first tokens.
struct CountShared {
  int cnt[1024];
  int off[1024];
  int is_host[1024];
  int ids[kGroupTokens * 32];
  int scan_tmp[16];
  int stat[4];
  int last;
};

__global__ __launch_bounds__(1024) void k_topk_count(RouteArgs a, unsigned* counter) {
  __shared__ CountShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = a.E, k = a.k, nb = gridDim.x;
  const int t0 = blockIdx.x * kGroupTokens, nt = min(kGroupTokens, a.T - t0);
  sh.cnt[tid] = 0;
  sh.is_host[tid] = tid < E ? a.is_host[tid] : 0;
  if (tid < 4) sh.stat[tid] = 0;
  if (wave < nt) {
    const int t = t0 + wave;
    topk_wave(a.logits + (size_t)t * E, E, k, lane, a.ids + (size_t)t * k, a.wts + (size_t)t * k, sh.ids + wave * k);
  }
  __syncthreads();
  if (tid < nt * k) atomicAdd(&sh.cnt[sh.ids[tid]], 1);
  __syncthreads();
  if (tid < E) st_shared_dev(a.hist + (size_t)blockIdx.x * E + tid, sh.cnt[tid]);
  // arrive; the last block sees every block's counts
  if (!arrive_last(counter, (unsigned)nb, &sh.last)) return;
  const int n = a.T * k;
  // expert totals, offsets and per-block bases (written over the counts): J threads
  // per expert, thread (e = tid % E, j = tid / E) summing blocks [j nb / J, (j+1) nb / J)
  const int J = max(1, (int)blockDim.x / E);
  const int ej = tid % E, jj = tid / E;
  const bool sum_thread = jj < J;
  const int b0 = (nb * jj) / J, b1 = (nb * (jj + 1)) / J;
  int part = 0;
  if (sum_thread) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {  // eight loads in flight
      int h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = ld_shared_dev(a.hist + (size_t)(b + i) * E + ej);
      part += ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
    }
    for (; b < b1; ++b) part += ld_shared_dev(a.hist + (size_t)b * E + ej);
  }
  int* jpart = sh.off;  // [J][E] partial sums (J * E <= 1024)
  if (sum_thread) jpart[jj * E + ej] = part;
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int j = 0; j < J; ++j) c += jpart[j * E + tid];
  int jbefore = 0;
  if (sum_thread)
    for (int j = 0; j < jj; ++j) jbefore += jpart[j * E + ej];
  int total;
  const int off = block_exscan(c, sh.scan_tmp, &total);  // (barriers inside: jpart reads are done)
  if (tid < E) {
    a.counts[tid] = c;
    a.offsets[tid] = off;
    sh.cnt[tid] = off;  // offsets for the base pass
  }
  if (tid == 0) a.offsets[E] = n;
  __syncthreads();
  if (sum_thread) {  // counts of 8 blocks loaded together, then their bases written
    int run = sh.cnt[ej] + jbefore;
    for (int b = b0; b < b1; b += 8) {
      int hb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) hb[i] = (b + i < b1) ? ld_shared_dev(a.hist + (size_t)(b + i) * E + ej) : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (b + i < b1) a.hist[(size_t)(b + i) * E + ej] = run;
        run += hb[i];
      }
    }
  }
  __syncthreads();
  // active experts, host-read ones first: scan over 2E flags, two per thread
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  sh.cnt[tid] = c;
  sh.off[tid] = off;
  __syncthreads();
  auto flag = [&](int it) -> int {
    if (it >= 2 * E) return 0;
    const int e = it < E ? it : it - E;
    const bool host = sh.is_host[e] != 0;
    return (sh.cnt[e] > 0 && (it < E ? host : !host)) ? 1 : 0;
  };
  const int f0 = flag(i0), f1 = flag(i1);
  int n_act;
  const int pos = block_exscan(f0 + f1, sh.scan_tmp, &n_act);
  if (f0) {
    const int e = i0 < E ? i0 : i0 - E;
    a.active[pos] = e;
    a.act_pos[e] = pos;
    if (a.work) {
      a.work[pos].w = a.wptr[e];
      a.work[pos].p0 = sh.off[e];
      a.work[pos].M = skipped(a, i0 < E) ? 0 : sh.cnt[e];
    }
  }
  if (f1) {
    const int e = i1 < E ? i1 : i1 - E;
    a.active[pos + f0] = e;
    a.act_pos[e] = pos + f0;
    if (a.work) {
      a.work[pos + f0].w = a.wptr[e];
      a.work[pos + f0].p0 = sh.off[e];
      a.work[pos + f0].M = skipped(a, i1 < E) ? 0 : sh.cnt[e];
    }
  }
  if (a.work)  // unused GEMV slots up to min(E, T*k) (the GEMV grid) have no rows
    for (int sl = n_act + tid; sl < min(E, n); sl += blockDim.x) a.work[sl].M = 0;
  if (tid == 0) a.n_active[0] = n_act;
  if (a.tiles) {  // prefill GEMM tiles of kGemmRows rows, expert by expert
    const int ntile = (tid < E) ? (c + kGemmRows - 1) / kGemmRows : 0;
    int n_all;
    const int q0 = block_exscan(ntile, sh.scan_tmp, &n_all);
    for (int i = 0; i < ntile; ++i) a.tiles[q0 + i] = make_int2(tid, i * kGemmRows);
    if (tid == 0) *a.n_tiles = n_all;
  }
  if (tid < E && c > 0) {
    const bool host = sh.is_host[tid] != 0;
    atomicAdd(&sh.stat[host ? 1 : 0], c);
    atomicAdd(&sh.stat[host ? 3 : 2], 1);
    atomicAdd(reinterpret_cast<unsigned long long*>(a.counts_acc + tid), (unsigned long long)c);
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long* st = reinterpret_cast<unsigned long long*>(a.stats);
    atomicAdd(st + ST_FORWARDS, 1ull);
    atomicAdd(st + ST_TOKENS, (unsigned long long)a.T);
    atomicAdd(st + ST_HITS, (unsigned long long)sh.stat[0]);
    atomicAdd(st + ST_MISSES, (unsigned long long)sh.stat[1]);
    atomicAdd(st + ST_BYTES_HBM, (unsigned long long)((int64_t)sh.stat[2] * a.expert_bytes));
    atomicAdd(st + ST_BYTES_HOST, (unsigned long long)((int64_t)sh.stat[3] * a.expert_bytes));
    a.n_active[1] = sh.stat[3];  // host-read experts, the first entries of the active list
  }
}

// One block per kGroupTokens tokens, one thread per assignment (ascending order).
// A thread's rank among the block's earlier assignments to its expert: within its
// wave from the ballot of equal ids, over earlier waves from their id-bit masks.
__global__ __launch_bounds__(kGroupTokens * 32) void k_scatter(RouteArgs a) {
  constexpr int kW = kGroupTokens * 32 / 64;
  __shared__ uint64_t masks[kW][kIdBits + 1];  // per wave: id-bit ballots, then the valid mask
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int E = a.E, k = a.k;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int base = blockIdx.x * kGroupTokens * k;
  const int n_blk = min(kGroupTokens * k, a.T * k - base);
  const int i = base + tid;
  const bool valid = tid < n_blk;
  const int e = valid ? a.ids[i] : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t m[kIdBits];
#pragma unroll
  for (int b = 0; b < kIdBits; ++b) m[b] = __ballot(valid && ((e >> b) & 1));
  const uint64_t vm = __ballot(valid);
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < kIdBits; ++b) masks[wave][b] = m[b];
    masks[wave][kIdBits] = vm;
  }
  __syncthreads();
  uint64_t eq;
  count_below(e, m, vm, nbits, &eq);
  int rank = __popcll(eq & lt_mask);
  for (int w = 0; w < wave; ++w) {
    uint64_t q;
    count_below(e, masks[w], masks[w][kIdBits], nbits, &q);
    rank += __popcll(q);
  }
  if (valid) {
    const int pos = a.hist[(size_t)blockIdx.x * E + e] + rank;
    a.sorted[pos] = i;
    a.inv[i] = pos;
    if (a.work) {
      const int j = pos - a.offsets[e];
      if (j < kDescTok) a.work[a.act_pos[e]].tok[j] = i / k;
    }
  }
}

void launch_topk_group(const RouteArgs& a, unsigned* counter, const Timing& tm, hipStream_t s) {
  Timing t1 = tm, t2 = tm;
  t1.stop = nullptr;
  t2.start = nullptr;
  const int nb = (a.T + kGroupTokens - 1) / kGroupTokens;
  launch_timed(k_topk_count, dim3(nb), dim3(1024), 0, s, t1, a, counter);
  const int threads = ((kGroupTokens * a.k + 63) / 64) * 64;
  launch_timed(k_scatter, dim3(nb), dim3(threads), 0, s, t2, a);
}

// ----------------------------------------------------------------------------- combine

// y[t][n] = sum over slots j = 0..k-1, in order, of w[t][j] * o[inv[t*k+j]][n] (fp32).
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * 256 + threadIdx.x;  // float4 index
  if (n4 * 4 >= a.H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < a.k; ++j) {
    const int slot = t * a.k + j;
    const float w = a.wts[slot];
    const float4 v = reinterpret_cast<const float4*>(a.o + (size_t)a.inv[slot] * a.H)[n4];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  reinterpret_cast<float4*>(a.y + (size_t)t * a.H)[n4] = acc;
  if (a.xout) {
    const size_t i4 = (size_t)t * a.H / 4 + n4;
    if (a.act_bf16) {
      const ushort4 xv = static_cast<const ushort4*>(a.xres)[i4];
      ushort4 r;
      r.x = residual_bf16(xv.x, acc.x);
      r.y = residual_bf16(xv.y, acc.y);
      r.z = residual_bf16(xv.z, acc.z);
      r.w = residual_bf16(xv.w, acc.w);
      static_cast<ushort4*>(a.xout)[i4] = r;
    } else {
      const float4 xv = static_cast<const float4*>(a.xres)[i4];
      static_cast<float4*>(a.xout)[i4] = make_float4(xv.x + acc.x, xv.y + acc.y, xv.z + acc.z, xv.w + acc.w);
    }
  }
}

void launch_combine(const CombineArgs& a, const Timing& tm, hipStream_t s) {
  launch_timed(k_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, s, tm, a);
}

}  // namespace moe
