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
