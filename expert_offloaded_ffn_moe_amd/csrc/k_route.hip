// Routing kernels for gfx950: router logits, per-group activation sums, top-k
// gate choice, grouping of assignments by expert (counts, offsets, stable
// permutation, active-expert list, link counters) and the gate-weighted combine.
//
// The routed choice follows page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存",
// section "显存缺口从哪里来" (a few experts per token per layer, picked at run
// time); softmax scores, ties to the lower expert id and renormalisation over
// the k chosen are the plain reading of it.
//
// Decode (T <= 64, T*k <= 1024) runs as one launch: router blocks compute the
// logits, and the last block to finish (an atomic arrival counter, no waiting)
// does the top-k and the grouping. Larger T uses separate launches.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>

#include "kernels.h"
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

// One wave: logits of expert row e for every token. Lane l owns the 16-byte
// chunks l, l+64, ... of the row (at most NCH of them, held in registers); for
// each token the matching x chunks are all loaded before the dot products.
// fp32 sums in chunk order, then a fixed DPP tree across lanes.
template <int BF16, int NCH>
__device__ void router_row(const RouterArgs& a, int e, int lane) {
  const int esz = BF16 ? 2 : 4;
  const int nchunk = a.H * esz / 16;
  gu32x4* wrow = (gu32x4*)(static_cast<const char*>(a.w) + (size_t)e * a.H * esz);
  const float bias = a.b ? a.b[e] : 0.f;
  u32x4 wv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) wv[i] = wrow[min(lane + 64 * i, nchunk - 1)];
  for (int t = 0; t < a.T; ++t) {
    gu32x4* xrow = (gu32x4*)(static_cast<const char*>(a.x) + (size_t)t * a.H * esz);
    u32x4 xv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) xv[i] = xrow[min(lane + 64 * i, nchunk - 1)];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float d = dot16(wv[i], xv[i], 0.f, BF16);
      s += (lane + 64 * i < nchunk) ? d : 0.f;
    }
    const float v = wave_sum(s);
    if (lane == 0) a.logits[(size_t)t * a.E + e] = v + bias;
  }
}

// Rows longer than 64 * 16 chunks: plain strided loop.
template <int BF16>
__device__ void router_row_long(const RouterArgs& a, int e, int lane) {
  const int esz = BF16 ? 2 : 4;
  const int nchunk = a.H * esz / 16;
  gu32x4* wrow = (gu32x4*)(static_cast<const char*>(a.w) + (size_t)e * a.H * esz);
  const float bias = a.b ? a.b[e] : 0.f;
  for (int t = 0; t < a.T; ++t) {
    gu32x4* xrow = (gu32x4*)(static_cast<const char*>(a.x) + (size_t)t * a.H * esz);
    float s = 0.f;
    for (int c = lane; c < nchunk; c += 64) {
      const u32x4 wv = wrow[c], xv = xrow[c];
      s = dot16(wv, xv, s, BF16);
    }
    const float v = wave_sum(s);
    if (lane == 0) a.logits[(size_t)t * a.E + e] = v + bias;
  }
}

template <int BF16>
__device__ void router_row_any(const RouterArgs& a, int e, int lane) {
  const int nch = (a.H * (BF16 ? 2 : 4) / 16 + 63) / 64;
  if (nch <= 1)
    router_row<BF16, 1>(a, e, lane);
  else if (nch <= 2)
    router_row<BF16, 2>(a, e, lane);
  else if (nch <= 4)
    router_row<BF16, 4>(a, e, lane);
  else if (nch <= 8)
    router_row<BF16, 8>(a, e, lane);
  else if (nch <= 16)
    router_row<BF16, 16>(a, e, lane);
  else
    router_row_long<BF16>(a, e, lane);
}

// sum of x[t][g*G .. (g+1)*G) for flat index gid = t * (H/G) + g (bf16 x)
__device__ void xsum_one(const RouterArgs& a, int gid) {
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

// Any T: blocks [0, router_blocks) do 4 expert rows each, the rest the group sums.
template <int BF16>
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < a.router_blocks) {
    const int e = blockIdx.x * 4 + wave;
    if (e < a.E) router_row_any<BF16>(a, e, lane);
  } else if (BF16) {
    const int gid = (blockIdx.x - a.router_blocks) * 256 + threadIdx.x;
    if (gid < a.T * (a.H / a.G)) xsum_one(a, gid);
  }
}

void launch_router(const RouterArgs& a, int act_bf16, const Timing& tm, hipStream_t s) {
  const int xs_blocks = (act_bf16 && a.xsum) ? (a.T * (a.H / a.G) + 255) / 256 : 0;
  const int grid = a.router_blocks + xs_blocks;
  if (grid == 0) return;
  if (act_bf16)
    launch_timed(k_router<1>, dim3(grid), dim3(256), 0, s, tm, a);
  else
    launch_timed(k_router<0>, dim3(grid), dim3(256), 0, s, tm, a);
}

// ----------------------------------------------------------------------------- top-k

// One wave chooses the k experts of one token, in k rounds. Lane l holds the
// logits of experts l, l+64, ... (NV of them; missing ones are -inf). A round
// takes the wave maximum m (DPP), then the lowest expert id whose logit equals m
// (ballots, lowest set bit), so ties go to the lower id and -0.0 ties +0.0;
// that logit is then set to -inf, which never wins while a real candidate is
// left (k <= E). Lane j keeps slot j. Weights: the softmax of the chosen logits,
// exp(l_j - l_0) / sum over the chosen.
template <int NV>
__device__ void topk_wave_nv(const float* __restrict__ lrow, int E, int k, int lane, int32_t* __restrict__ ids_out,
                             float* __restrict__ w_out, int32_t* lds_ids) {
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? lrow[min(e, E - 1)] : -INFINITY;
  }
  float my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float m = v[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) m = fmaxf(m, v[i]);
    m = wave_max(m);
    int win = -1;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const unsigned long long b = __ballot(v[i] == m);
      if (win < 0 && b != 0ull) win = 64 * i + (int)__builtin_ctzll(b);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = (lane + 64 * i == win) ? -INFINITY : v[i];
    my_v = (lane == j) ? m : my_v;
    my_e = (lane == j) ? win : my_e;
  }
  const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
  const float ex = (lane < k) ? __expf(my_v - m0) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / sum;
    if (lds_ids) lds_ids[lane] = my_e;
  }
}

__device__ void topk_wave(const float* __restrict__ lrow, int E, int k, int lane, int32_t* __restrict__ ids_out,
                          float* __restrict__ w_out, int32_t* lds_ids) {
  switch ((E + 63) >> 6) {
    case 1: return topk_wave_nv<1>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    case 2: return topk_wave_nv<2>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    case 3: return topk_wave_nv<3>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    case 4: return topk_wave_nv<4>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    case 5:
    case 6: return topk_wave_nv<6>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    case 7:
    case 8: return topk_wave_nv<8>(lrow, E, k, lane, ids_out, w_out, lds_ids);
    default: return topk_wave_nv<16>(lrow, E, k, lane, ids_out, w_out, lds_ids);
  }
}

__global__ __launch_bounds__(1024) void k_topk(RouteArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 16 + wave;
  if (t >= a.T) return;
  topk_wave(a.logits + (size_t)t * a.E, a.E, a.k, lane, a.ids + (size_t)t * a.k, a.wts + (size_t)t * a.k, nullptr);
}

// ----------------------------------------------------------------------------- align / permute

struct AlignShared {
  int cnt[1024];
  int off[1025];
  int running[1024];
  int is_host[1024];
  int wave_cnt[16][1024];
  int scan_tmp[16];
  int stat[4];  // hits, misses, unique hbm, unique host
  int last;
};

// Exclusive scan of one int per thread over a 1024-thread block; *total = sum.
__device__ int block_exscan(int v, int* tmp, int* total) {
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

__device__ __forceinline__ void load_is_host(const RouteArgs& a, AlignShared& sh) {
  const int tid = threadIdx.x;
  sh.is_host[tid] = tid < a.E ? a.is_host[tid] : 0;
}

// Counts, offsets, stable permutation, active list and counters for the n = T*k
// assignments of a.ids.
// Called by all 1024 threads; sh.is_host must be loaded and visible.
__device__ void align_block(const RouteArgs& a, AlignShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T * a.k, E = a.E;
  sh.cnt[tid] = 0;
  sh.running[tid] = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) sh.wave_cnt[w][tid] = 0;
  if (tid < 4) sh.stat[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int e = a.ids[i];
    atomicAdd(&sh.cnt[e], 1);
  }
  __syncthreads();
  int total;
  const int c = (tid < E) ? sh.cnt[tid] : 0;
  const int ex = block_exscan(c, sh.scan_tmp, &total);
  if (tid < E) {
    sh.off[tid] = ex;
    a.counts[tid] = c;
    a.offsets[tid] = ex;
  }
  if (tid == 0) {
    sh.off[E] = total;
    a.offsets[E] = total;
  }
  __syncthreads();

  // stable scatter, 1024 assignments per round in ascending order
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const bool valid = i < n;
    const int e = valid ? (a.ids[i]) : 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const unsigned long long bm = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bm : ~bm;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && (peers & lt_mask) == 0) sh.wave_cnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += sh.wave_cnt[w][e];
      const int pos = sh.off[e] + sh.running[e] + before + rank;
      a.sorted[pos] = i;
      a.inv[i] = pos;
    }
    __syncthreads();
    if (tid < E) {
      int s = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        s += sh.wave_cnt[w][tid];
        sh.wave_cnt[w][tid] = 0;
      }
      sh.running[tid] += s;
    }
    __syncthreads();
  }

  // active experts, host-read ones first: scan over 2E flags, two per thread
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  auto flag = [&](int it) -> int {
    if (it >= 2 * E) return 0;
    const int e = it < E ? it : it - E;
    const bool host = sh.is_host[e] != 0;
    return (sh.cnt[e] > 0 && (it < E ? host : !host)) ? 1 : 0;
  };
  const int f0 = flag(i0), f1 = flag(i1);
  int n_act;
  const int pos = block_exscan(f0 + f1, sh.scan_tmp, &n_act);
  if (f0) a.active[pos] = i0 < E ? i0 : i0 - E;
  if (f1) a.active[pos + f0] = i1 < E ? i1 : i1 - E;
  if (tid == 0) *a.n_active = n_act;

  if (a.tiles) {  // prefill GEMM tiles of kGemmRows rows, expert by expert
    const int nt = (tid < E) ? (c + kGemmRows - 1) / kGemmRows : 0;
    int n_all;
    const int t0 = block_exscan(nt, sh.scan_tmp, &n_all);
    for (int i = 0; i < nt; ++i) a.tiles[t0 + i] = make_int2(tid, i * kGemmRows);
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
  }
}

struct DecodeShared {
  int cnt[1024];
  int off[1025];
  int running[1024];
  int is_host[1024];
  int ids_small[kRouteSmallMaxAssign];
  int last;
};

// The same grouping done by one wave, for n = T*k <= kRouteSmallMaxAssign
// assignments with ids in sh.ids_small and sh.is_host loaded: no block
// barriers, only wave-level scans and ballots. Experts are taken 64 at a time,
// expert e = 64b + lane, so every step is one coalesced access per wave.
__device__ void align_wave(const RouteArgs& a, DecodeShared& sh) {
  const int lane = threadIdx.x & 63;
  const int n = a.T * a.k, E = a.E, NB = (E + 63) >> 6;
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b = 0; b < NB; ++b) {
    const int e = 64 * b + lane;
    if (e < E) {
      sh.cnt[e] = 0;
      sh.running[e] = 0;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int i = lane; i < n; i += 64) atomicAdd(&sh.cnt[sh.ids_small[i]], 1);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  int carry = 0;
  for (int b = 0; b < NB; ++b) {
    const int e = 64 * b + lane;
    const int c = (e < E) ? sh.cnt[e] : 0;
    const int incl = wave_incl_scan(c);
    if (e < E) {
      sh.off[e] = carry + incl - c;
      a.offsets[e] = carry + incl - c;
      a.counts[e] = c;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) {
    sh.off[E] = carry;
    a.offsets[E] = carry;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // stable positions, 64 assignments per round in ascending order
  for (int base = 0; base < n; base += 64) {
    const int i = base + lane;
    const bool valid = i < n;
    const int e = valid ? sh.ids_small[i] : 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const unsigned long long bm = __ballot(valid && ((e >> bit) & 1));
      peers &= ((e >> bit) & 1) ? bm : ~bm;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid) {
      const int pos = sh.off[e] + sh.running[e] + rank;
      a.sorted[pos] = i;
      a.inv[i] = pos;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (valid && (peers & lt_mask) == 0) sh.running[e] += __popcll(peers);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }

  // active experts: host-read ones first, then the HBM ones, ascending id in each
  int pos = 0, n_host = 0, hits = 0, misses = 0;
  for (int pass = 0; pass < 2; ++pass) {
    for (int b = 0; b < NB; ++b) {
      const int e = 64 * b + lane;
      const int c = (e < E) ? sh.cnt[e] : 0;
      const bool host = (e < E) && sh.is_host[e] != 0;
      const bool flag = c > 0 && (pass == 0 ? host : !host);
      const unsigned long long m = __ballot(flag);
      if (flag) {
        a.active[pos + __popcll(m & lt_mask)] = e;
        atomicAdd(reinterpret_cast<unsigned long long*>(a.counts_acc + e), (unsigned long long)c);
      }
      pos += __popcll(m);
      if (pass == 0)
        misses += flag ? c : 0;
      else
        hits += flag ? c : 0;
    }
    if (pass == 0) n_host = pos;
  }
  hits = wave_sum_i(hits);
  misses = wave_sum_i(misses);
  if (lane == 0) {
    *a.n_active = pos;
    unsigned long long* st = reinterpret_cast<unsigned long long*>(a.stats);
    atomicAdd(st + ST_FORWARDS, 1ull);
    atomicAdd(st + ST_TOKENS, (unsigned long long)a.T);
    atomicAdd(st + ST_HITS, (unsigned long long)hits);
    atomicAdd(st + ST_MISSES, (unsigned long long)misses);
    atomicAdd(st + ST_BYTES_HBM, (unsigned long long)((int64_t)(pos - n_host) * a.expert_bytes));
    atomicAdd(st + ST_BYTES_HOST, (unsigned long long)((int64_t)n_host * a.expert_bytes));
  }
}

__global__ __launch_bounds__(1024) void k_align(RouteArgs a) {
  __shared__ AlignShared sh;
  load_is_host(a, sh);
  __syncthreads();
  align_block(a, sh);
}

// Decode routing in one launch. Blocks [0, router_blocks): 8 expert rows each
// (one per wave); then xsum blocks; every block then arrives on the counter,
// and the last one (which sees every other block's logits after the
// device-scope fences) picks the top-k of every token (one wave per token) and
// groups the assignments in one wave.
template <int BF16>
__global__ __launch_bounds__(512) void k_route_decode(RouteArgs a, RouterArgs r, unsigned* counter) {
  __shared__ DecodeShared sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bid = blockIdx.x;
  if (bid < r.router_blocks) {
    const int e = bid * 8 + wave;
    if (e < r.E) router_row_any<BF16>(r, e, lane);
  } else if (BF16 && r.xsum) {
    const int gid = (bid - r.router_blocks) * 512 + threadIdx.x;
    if (gid < r.T * (r.H / r.G)) xsum_one(r, gid);
  }
  // every wave drains its stores; one thread publishes the block's writes with a
  // device-scope release and arrives; the last arrival acquires
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(counter, 1u);
    sh.last = (prev == gridDim.x - 1) ? 1 : 0;
    if (sh.last) __threadfence();
  }
  __syncthreads();
  if (!sh.last) return;
  for (int e = threadIdx.x; e < a.E; e += 512) sh.is_host[e] = a.is_host[e];
  if (threadIdx.x == 0) *counter = 0u;  // ready for the next launch on this stream
  for (int t = wave; t < a.T; t += 8)
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.k, lane, a.ids + (size_t)t * a.k, a.wts + (size_t)t * a.k,
              sh.ids_small + t * a.k);
  __syncthreads();
  if (threadIdx.x < 64) align_wave(a, sh);
}

void launch_route_decode(const RouteArgs& a, const RouterArgs& r, int act_bf16, unsigned* counter,
                         const Timing& tm, hipStream_t s) {
  const int xs_blocks = (act_bf16 && r.xsum) ? (r.T * (r.H / r.G) + 511) / 512 : 0;
  const int grid = std::max(1, r.router_blocks + xs_blocks);
  if (act_bf16)
    launch_timed(k_route_decode<1>, dim3(grid), dim3(512), 0, s, tm, a, r, counter);
  else
    launch_timed(k_route_decode<0>, dim3(grid), dim3(512), 0, s, tm, a, r, counter);
}

void launch_topk_align(const RouteArgs& a, const Timing& tm, hipStream_t s) {
  Timing t1 = tm, t2 = tm;
  t1.stop = nullptr;
  t2.start = nullptr;
  launch_timed(k_topk, dim3((a.T + 15) / 16), dim3(1024), 0, s, t1, a);
  launch_timed(k_align, dim3(1), dim3(1024), 0, s, t2, a);
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
}

void launch_combine(const CombineArgs& a, const Timing& tm, hipStream_t s) {
  launch_timed(k_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, s, tm, a);
}

}  // namespace moe
