// Device helpers of the routing step: per-token top-k with softmax gate
// weights, and counting by expert id from per-bit ballot masks.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>

#include "kernels.h"
#include "wave.h"

namespace moe {

// Whether the GEMVs skip an active expert's rows (its FFN computed by the host
// cores): skip_host 1 = the experts read from host memory, 2 = every expert.
__device__ __forceinline__ bool skipped(const RouteArgs& a, bool host) {
  return a.skip_host == 2 || (a.skip_host == 1 && host);
}

// ----------------------------------------------------------------------------- cross-block hand-off

// Data that one workgroup of a launch writes and the last workgroup to arrive reads
// (router logits, per-block counts) is stored and loaded as agent-scope relaxed
// atomics: on gfx950 these are write-through stores and loads that miss the XCD's
// own L2 (the sc1 forms), coherent across the XCDs without the whole-L2 writeback
// and invalidate that a release or acquire fence costs. Each workgroup waits for
// its stores to complete (vmcnt 0) before it increments the arrival counter, so
// they are performed before the increment; the last arrival reads them afterwards.
template <typename T>
__device__ __forceinline__ void st_shared_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_shared_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by every thread of a workgroup after its hand-off stores: true in the last
// workgroup of `n` to arrive. The counter is reset for the next launch on the stream.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned n, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores performed
  __syncthreads();                // every wave's
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = prev == n - 1 ? 1 : 0;
  }
  __syncthreads();
  const bool last = *flag != 0;
  if (last && threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
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
__device__ __forceinline__ void topk_wave_nv(const float* __restrict__ lrow, int E, int k, int lane, int32_t* __restrict__ ids_out,
                             float* __restrict__ w_out, int32_t* lds_ids) {
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? ld_shared_dev(lrow + min(e, E - 1)) : -INFINITY;
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
    win = max(win, 0);  // only NaN logits (outside the contract) leave no winner; keep ids in range
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

__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, int E, int k, int lane, int32_t* __restrict__ ids_out,
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


// Counting by expert id over one 64-assignment chunk, from the chunk's bit
// masks m[b] = ballot(bit b of the id) and the set `in` of assignments counted:
// returns how many of them have an id below v; *eq = which of them have id v.
// Every thread evaluates its own v with register operations on uniform masks.
constexpr int kIdBits = 10;  // E <= 1024
__device__ __forceinline__ int count_below(int v, const uint64_t* m, uint64_t in, int nbits, uint64_t* eq) {
  uint64_t q = in;
  int lt = 0;
#pragma unroll
  for (int b = kIdBits - 1; b >= 0; --b) {
    if (b < nbits) {
      const uint64_t mb = m[b];
      const bool one = (v >> b) & 1;
      lt += one ? __popcll(q & ~mb) : 0;
      q &= one ? mb : ~mb;
    }
  }
  *eq = q;
  return lt;
}

}  // namespace moe
