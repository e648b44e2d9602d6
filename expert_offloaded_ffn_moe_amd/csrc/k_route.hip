// Routing kernels for gfx950: router logits, per-group activation sums, top-k
// gate choice, grouping of assignments by expert (counts, offsets, stable
// permutation, active-expert list, link counters) and the gate-weighted combine.
//
// The routed choice itself follows page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进
// 主机内存", section "显存缺口从哪里来" (a few experts per token per layer, picked
// at run time); softmax scores, ties to the lower id and renormalisation over
// the k chosen are the plain reading of it.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>

#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ----------------------------------------------------------------------------- router

// Blocks [0, router_blocks): one wave per expert row, lanes stride over 16-byte
// chunks of H, tokens in passes of 16; fp32 sums, then a fixed wave tree.
// Blocks past router_blocks: one thread per (token, group) sums x over the group.
template <int BF16>
__global__ __launch_bounds__(256) void k_router(RouterArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < a.router_blocks) {
    const int e = blockIdx.x * 4 + wave;
    if (e >= a.E) return;
    const int esz = BF16 ? 2 : 4;
    const int nchunk = a.H * esz / 16;
    const uint4* wrow = reinterpret_cast<const uint4*>(static_cast<const char*>(a.w) + (size_t)e * a.H * esz);
    const float bias = a.b ? a.b[e] : 0.f;
    for (int t0 = 0; t0 < a.T; t0 += 16) {
      const int nt = min(16, a.T - t0);
      float acc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
      for (int c = lane; c < nchunk; c += 64) {
        const uint4 wv = wrow[c];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i < nt) {
            const uint4 xv = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) +
                                                            (size_t)(t0 + i) * a.H * esz)[c];
            if (BF16) {
              float s = acc[i];
              s = dot2_bf16(wv.x, xv.x, s);
              s = dot2_bf16(wv.y, xv.y, s);
              s = dot2_bf16(wv.z, xv.z, s);
              s = dot2_bf16(wv.w, xv.w, s);
              acc[i] = s;
            } else {
              float s = acc[i];
              s = fmaf(__uint_as_float(wv.x), __uint_as_float(xv.x), s);
              s = fmaf(__uint_as_float(wv.y), __uint_as_float(xv.y), s);
              s = fmaf(__uint_as_float(wv.z), __uint_as_float(xv.z), s);
              s = fmaf(__uint_as_float(wv.w), __uint_as_float(xv.w), s);
              acc[i] = s;
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < nt) {
          const float v = wave_sum(acc[i]);
          if (lane == 0) a.logits[(size_t)(t0 + i) * a.E + e] = v + bias;
        }
      }
    }
  } else if (BF16) {
    const int ng = a.H / a.G;
    const int gid = (blockIdx.x - a.router_blocks) * 256 + threadIdx.x;
    if (gid >= a.T * ng) return;
    const int t = gid / ng, g = gid % ng;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + (size_t)t * a.H +
                                                      (size_t)g * a.G);
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
}

void launch_router(const RouterArgs& a0, int act_bf16, hipStream_t s) {
  RouterArgs a = a0;
  const int xs_blocks = (act_bf16 && a.xsum) ? (a.T * (a.H / a.G) + 255) / 256 : 0;
  const int grid = a.router_blocks + xs_blocks;
  if (grid == 0) return;
  if (act_bf16)
    hipLaunchKernelGGL(k_router<1>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_router<0>, dim3(grid), dim3(256), 0, s, a);
}

// ----------------------------------------------------------------------------- top-k

// One wave chooses the k experts of one token: k rounds of a wave-wide arg-max
// under the order (logit descending, id ascending); lane j keeps slot j. The
// weights are the softmax of the chosen logits: exp(l_j - l_0) / sum.
__device__ void topk_wave(const float* __restrict__ lrow, int E, int k, int lane, int32_t* __restrict__ ids_out,
                          float* __restrict__ w_out, int32_t* lds_ids) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? lrow[e] : -FLT_MAX;
  }
  uint32_t taken = 0;
  float my_v = 0.f;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u)) {
        if (v[i] > bv || (v[i] == bv && e < be)) {
          bv = v[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  const float m = __shfl(my_v, 0, 64);
  const float ex = (lane < k) ? __expf(my_v - m) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / sum;
    if (lds_ids) lds_ids[lane] = my_e;
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
  int wave_cnt[16][1024];
  int wave_tot[16];
  int scan_tmp[16];
  int stat[4];  // hits, misses, unique hbm, unique host
  int ids_small[kRouteSmallMaxAssign];
};

// Exclusive scan of one int per thread over a 1024-thread block; returns the
// exclusive prefix, *total gets the sum.
__device__ int block_exscan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int tw = tmp[w];
    if (w < wave) base += tw;
    tot += tw;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Counts, offsets, stable permutation, active list and counters for the n = T*k
// assignments of ids (global memory, or sh.ids_small when from_lds).
// Must be called by all 1024 threads of the block.
__device__ void align_block(const RouteArgs& a, AlignShared& sh, bool from_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.T * a.k, E = a.E;
  sh.cnt[tid] = 0;
  sh.running[tid] = 0;
  for (int w = 0; w < 16; ++w) sh.wave_cnt[w][tid] = 0;
  if (tid < 4) sh.stat[tid] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int e = from_lds ? sh.ids_small[i] : a.ids[i];
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
    const int e = valid ? (from_lds ? sh.ids_small[i] : a.ids[i]) : 0;
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const unsigned long long bm = __ballot(valid && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? bm : ~bm;
    }
    const int rank = __popcll(peers & lt_mask);
    const bool leader = valid && ((peers & lt_mask) == 0);
    if (leader) sh.wave_cnt[wave][e] = __popcll(peers);
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
    const bool host = a.is_host[e] != 0;
    return (sh.cnt[e] > 0 && (it < E ? host : !host)) ? 1 : 0;
  };
  const int f0 = flag(i0), f1 = flag(i1);
  int n_act;
  const int pos = block_exscan(f0 + f1, sh.scan_tmp, &n_act);
  if (f0) a.active[pos] = i0 < E ? i0 : i0 - E;
  if (f1) a.active[pos + f0] = i1 < E ? i1 : i1 - E;
  if (tid == 0) *a.n_active = n_act;

  if (tid < E && c > 0) {
    const bool host = a.is_host[tid] != 0;
    atomicAdd(&sh.stat[host ? 1 : 0], c);
    atomicAdd(&sh.stat[host ? 3 : 2], 1);
    a.counts_acc[tid] += c;
  }
  __syncthreads();
  if (tid == 0) {
    a.stats[ST_FORWARDS] += 1;
    a.stats[ST_TOKENS] += a.T;
    a.stats[ST_HITS] += sh.stat[0];
    a.stats[ST_MISSES] += sh.stat[1];
    a.stats[ST_BYTES_HBM] += (int64_t)sh.stat[2] * a.expert_bytes;
    a.stats[ST_BYTES_HOST] += (int64_t)sh.stat[3] * a.expert_bytes;
  }
}

__global__ __launch_bounds__(1024) void k_align(RouteArgs a) {
  __shared__ AlignShared sh;
  align_block(a, sh, false);
}

// Decode-sized routing in one workgroup: top-k of every token (one wave per
// token), then the grouping by expert.
__global__ __launch_bounds__(1024) void k_route_small(RouteArgs a) {
  __shared__ AlignShared sh;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < a.T; t += 16)
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.k, lane, a.ids + (size_t)t * a.k, a.wts + (size_t)t * a.k,
              sh.ids_small + t * a.k);
  __syncthreads();
  align_block(a, sh, true);
}

void launch_route_small(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_route_small, dim3(1), dim3(1024), 0, s, a);
}

void launch_topk(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((a.T + 15) / 16), dim3(1024), 0, s, a);
}

void launch_align(const RouteArgs& a, hipStream_t s) { hipLaunchKernelGGL(k_align, dim3(1), dim3(1024), 0, s, a); }

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

void launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3((a.H / 4 + 255) / 256, a.T), dim3(256), 0, s, a);
}

}  // namespace moe
