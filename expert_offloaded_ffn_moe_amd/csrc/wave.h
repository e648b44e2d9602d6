// Wave64 reductions and scans on gfx950 through DPP row operations (no LDS
// round trips). Every helper must be called with all 64 lanes active; the
// reduced value is taken from lane 63 and broadcast with readlane.
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

enum : int {
  kDppXor1 = 0xB1,         // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,         // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,  // row_half_mirror
  kDppMirror = 0x140,      // row_mirror
  kDppBcast15 = 0x142,     // row_bcast:15
  kDppBcast31 = 0x143,     // row_bcast:31
  kDppShr1 = 0x111,
  kDppShr2 = 0x112,
  kDppShr4 = 0x114,
  kDppShr8 = 0x118,
};

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int old, int src) {
  return __builtin_amdgcn_update_dpp(old, src, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float dppf(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROWS, 0xF, false));
}

// Sum over the wave, broadcast to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<kDppXor1, 0xF>(0.f, v);
  v += dppf<kDppXor2, 0xF>(0.f, v);
  v += dppf<kDppHalfMirror, 0xF>(0.f, v);
  v += dppf<kDppMirror, 0xF>(0.f, v);
  v += dppf<kDppBcast15, 0xA>(0.f, v);
  v += dppf<kDppBcast31, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp<kDppXor1, 0xF>(0, v);
  v += dpp<kDppXor2, 0xF>(0, v);
  v += dpp<kDppHalfMirror, 0xF>(0, v);
  v += dpp<kDppMirror, 0xF>(0, v);
  v += dpp<kDppBcast15, 0xA>(0, v);
  v += dpp<kDppBcast31, 0xC>(0, v);
  return __builtin_amdgcn_readlane(v, 63);
}

// Maximum over the wave, broadcast to every lane (rows left out keep their value).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dppf<kDppXor1, 0xF>(v, v));
  v = fmaxf(v, dppf<kDppXor2, 0xF>(v, v));
  v = fmaxf(v, dppf<kDppHalfMirror, 0xF>(v, v));
  v = fmaxf(v, dppf<kDppMirror, 0xF>(v, v));
  v = fmaxf(v, dppf<kDppBcast15, 0xA>(v, v));
  v = fmaxf(v, dppf<kDppBcast31, 0xC>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One step of the arg-max: take (ov, oid) when it comes first in the order
// (value descending, id ascending).
__device__ __forceinline__ void better(float& v, int& id, float ov, int oid) {
  const bool take = (ov > v) | ((ov == v) & (oid < id));
  v = take ? ov : v;
  id = take ? oid : id;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(float& v, int& id) {
  const float ov = dppf<CTRL, ROWS>(v, v);  // rows left out keep their own value
  const int oid = dpp<CTRL, ROWS>(id, id);
  better(v, id, ov, oid);
}

// Arg-max over the wave under (value descending, id ascending), broadcast.
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
  argmax_step<kDppXor1, 0xF>(v, id);
  argmax_step<kDppXor2, 0xF>(v, id);
  argmax_step<kDppHalfMirror, 0xF>(v, id);
  argmax_step<kDppMirror, 0xF>(v, id);
  argmax_step<kDppBcast15, 0xA>(v, id);
  argmax_step<kDppBcast31, 0xC>(v, id);
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  id = __builtin_amdgcn_readlane(id, 63);
}

// Inclusive prefix sum over the lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp<kDppShr1, 0xF>(0, x);
  x += dpp<kDppShr2, 0xF>(0, x);
  x += dpp<kDppShr4, 0xF>(0, x);
  x += dpp<kDppShr8, 0xF>(0, x);
  x += dpp<kDppBcast15, 0xA>(0, x);
  x += dpp<kDppBcast31, 0xC>(0, x);
  return x;
}

}  // namespace moe
