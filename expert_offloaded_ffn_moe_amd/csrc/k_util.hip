// Small utility kernels: a 32-bit fill (the workspace poison of the debug mode)
// and the streaming-read probe behind moe_measure_link_ceilings.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void k_fill32(uint32_t* __restrict__ p, uint32_t v, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

void launch_fill32(void* p, uint32_t v, size_t n_words, hipStream_t s) {
  if (n_words == 0) return;
  const size_t blocks = std::min<size_t>((n_words + 255) / 256, 4096);
  hipLaunchKernelGGL(k_fill32, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), v, n_words);
}

// Reads n16 16-byte units once each: a thread takes units i, i + S, i + 2S, ...
// (S = all threads of the grid), four loads in flight, and folds them with XOR so
// that none is dead; a thread stores its fold only if it is all ones (never for
// the zero-filled probe buffers), which keeps the loads live at no store cost.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  gu32x4* p = (gu32x4*)src;
  const size_t S = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * S < n16; i += 4 * S) {
    const u32x4 a = p[i], b = p[i + S], c = p[i + 2 * S], d = p[i + 3 * S];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += S) acc ^= p[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0xFFFFFFFFu) sink[blockIdx.x] = v;
}

int stream_read_blocks() { return 2048; }

// The routing results and x of a forward into the pinned staging of its host part,
// with plain stores through the staging's device address (one launch instead of a
// DMA copy per buffer): dst = n_active[2] | active[E] | offsets[E+1] | sorted[A], x to
// xdst (xwords 32-bit words).
__global__ __launch_bounds__(256) void k_export_route(const int32_t* __restrict__ n_active,
                                                      const int32_t* __restrict__ active,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ sorted, const uint32_t* __restrict__ x,
                                                      int32_t* __restrict__ dst, uint32_t* __restrict__ xdst, int E, int A,
                                                      int xwords) {
  const int n_route = 3 + 2 * E + A;
  const int stride = gridDim.x * blockDim.x;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_route + xwords; i += stride) {
    if (i >= n_route) {
      xdst[i - n_route] = x[i - n_route];
    } else if (i < 2) {
      dst[i] = n_active[i];
    } else if (i < 2 + E) {
      dst[i] = active[i - 2];
    } else if (i < 3 + 2 * E) {
      dst[i] = offsets[i - 2 - E];
    } else {
      dst[i] = sorted[i - 3 - 2 * E];
    }
  }
}

void launch_export_route(const int32_t* n_active, const int32_t* active, const int32_t* offsets,
                         const int32_t* sorted, const void* x, size_t x_bytes, int32_t* dst, void* xdst, int E, int A,
                         hipStream_t s) {
  const int xwords = (int)(x_bytes / 4);
  const int n = 3 + 2 * E + A + xwords;
  const int blocks = std::min(64, (n + 255) / 256);
  hipLaunchKernelGGL(k_export_route, dim3(blocks), dim3(256), 0, s, n_active, active, offsets, sorted,
                     static_cast<const uint32_t*>(x), dst, static_cast<uint32_t*>(xdst), E, A, xwords);
}

void launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(k_stream_read, dim3(stream_read_blocks()), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     bytes / 16, sink);
}

}  // namespace moe
