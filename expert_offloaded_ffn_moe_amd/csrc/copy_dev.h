// Device-side bulk copy of expert blobs (prefill staging, predictive prefetch):
// one workgroup copies a range of 16-byte units with eight loads in flight per
// thread before their stores, consecutive threads on consecutive units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopyUnits = (int64_t)kCopyThreads * kCopyUnroll * 2;  // 16-byte units per workgroup (64 KiB)

typedef uint32_t cp_u32x4 __attribute__((ext_vector_type(4)));

// Units [u0, u1) of src to dst; every thread of the workgroup calls it.
__device__ __forceinline__ void copy_units(const void* src_, void* dst_, int64_t u0, int64_t u1) {
  const cp_u32x4* src = static_cast<const cp_u32x4*>(src_);
  cp_u32x4* dst = static_cast<cp_u32x4*>(dst_);
  for (int64_t u = u0 + threadIdx.x; u < u1; u += (int64_t)kCopyThreads * kCopyUnroll) {
    if (u + (int64_t)(kCopyUnroll - 1) * kCopyThreads < u1) {
      cp_u32x4 v[kCopyUnroll];
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) v[i] = src[u + (int64_t)i * kCopyThreads];
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) dst[u + (int64_t)i * kCopyThreads] = v[i];
    } else {
      for (int64_t q = u; q < u1; q += kCopyThreads) dst[q] = src[q];
    }
  }
}

}  // namespace moe
