// Grouped int4 dequant-GEMV for decode on gfx950: the per-expert SwiGLU FFN
// of the routed MoE layer, reading each touched expert's weights once, from
// its HBM slot or in place from its pinned host copy over the host link.
//
// Offloaded experts are dereferenced by the kernels directly, without staging
// copies (page "763B MoE 塞进两张 96GB 显卡：闲置专家丢进主机内存", section
// "显存缺口从哪里来"); which pointer an expert has is the per-expert plan of
// section "同一个思路，vLLM 原生方案反而跑不通". The kernels do not know or care
// which memory a pointer refers to, so results do not depend on residency.
//
// Work decomposition: a workgroup owns (active expert, row tile) and its W
// waves split K by quantisation groups. Lane l owns one weight row and reads
// 16 bytes (32 int4 values) per K chunk, so each wave load is one contiguous
// KiB. The activations of the tokens routed to the expert are wave-uniform and
// come in through scalar loads. Partial sums of the W waves are added in LDS in
// wave order, so the summation order is fixed.
//
// bf16 activations: a nibble n = q + 8 placed in the top mantissa bits of a
// bf16 1.0 gives v = 1 + n/16 = 1.5 + q/16 exactly; v_dot2_f32_bf16 multiplies
// two such values by two activations per instruction. Over a group,
// sum q x = 16 * (sum v x - 1.5 * sum x), with sum x precomputed per group, so
// the int4 weight is exact and only fp32 accumulation rounds.
// fp32 activations: q is converted exactly to fp32 and used in fmaf.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// bf16 pair (1 + n_lo/16, 1 + n_hi/16) of pair j of a code dword
__device__ __forceinline__ uint32_t pair0(uint32_t d) { return ((d << 3) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair1(uint32_t d) { return ((d >> 1) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair2(uint32_t d) { return ((d >> 5) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair3(uint32_t d) { return ((d >> 9) & 0x00780078u) | 0x3F803F80u; }

__device__ __forceinline__ float scale_of(const uint4& sv, int g) {
  const int w = (g & 7) >> 1;
  const uint32_t d = w == 0 ? sv.x : w == 1 ? sv.y : w == 2 ? sv.z : sv.w;
  const uint16_t bits = (g & 1) ? (uint16_t)(d >> 16) : (uint16_t)(d & 0xFFFFu);
  return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// sum over one 32-wide chunk of (code row) x (activation row), bf16 path:
// returns acc + sum_i v_i x_i with v = 1 + n/16.
__device__ __forceinline__ float chunk_dot_bf16(const uint4& wv, const uint32_t* __restrict__ xr, float acc) {
  acc = dot2(pair0(wv.x), xr[0], acc);
  acc = dot2(pair1(wv.x), xr[1], acc);
  acc = dot2(pair2(wv.x), xr[2], acc);
  acc = dot2(pair3(wv.x), xr[3], acc);
  acc = dot2(pair0(wv.y), xr[4], acc);
  acc = dot2(pair1(wv.y), xr[5], acc);
  acc = dot2(pair2(wv.y), xr[6], acc);
  acc = dot2(pair3(wv.y), xr[7], acc);
  acc = dot2(pair0(wv.z), xr[8], acc);
  acc = dot2(pair1(wv.z), xr[9], acc);
  acc = dot2(pair2(wv.z), xr[10], acc);
  acc = dot2(pair3(wv.z), xr[11], acc);
  acc = dot2(pair0(wv.w), xr[12], acc);
  acc = dot2(pair1(wv.w), xr[13], acc);
  acc = dot2(pair2(wv.w), xr[14], acc);
  acc = dot2(pair3(wv.w), xr[15], acc);
  return acc;
}

// fp32 path: acc + sum_i q_i x_i, q = n - 8 exact in fp32.
__device__ __forceinline__ float dword_dot_f32(uint32_t d, const float* __restrict__ xr, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float qlo = (float)(int)((d >> (4 * j)) & 0xFu) - 8.f;
    const float qhi = (float)(int)((d >> (16 + 4 * j)) & 0xFu) - 8.f;
    acc = fmaf(qlo, xr[2 * j], acc);
    acc = fmaf(qhi, xr[2 * j + 1], acc);
  }
  return acc;
}

__device__ __forceinline__ float chunk_dot_f32(const uint4& wv, const float* __restrict__ xr, float acc) {
  acc = dword_dot_f32(wv.x, xr, acc);
  acc = dword_dot_f32(wv.y, xr + 8, acc);
  acc = dword_dot_f32(wv.z, xr + 16, acc);
  acc = dword_dot_f32(wv.w, xr + 24, acc);
  return acc;
}

// K loop of one wave over groups [g0, g1) for MT token rows.
// rows[m]: element offset of token m's activation row in `in`; insum_rows[m]:
// offset of its per-chunk or per-group sums (bf16 path).
template <int BF16, int MT>
__device__ __forceinline__ void k_loop(const uint4* __restrict__ codes, const uint4* __restrict__ scales,
                                       const void* __restrict__ in, const float* __restrict__ insum,
                                       const int64_t* rows, const int64_t* sum_rows, int mc, int g0, int g1,
                                       int cpg, bool sums_per_chunk, float* acc) {
  for (int g = g0; g < g1; ++g) {
    const uint4 sv = scales[(size_t)(g >> 3) * 64];
    const float s = scale_of(sv, g);
    float accg[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) accg[m] = 0.f;
#pragma unroll 4
    for (int cc = 0; cc < cpg; ++cc) {
      const int c = g * cpg + cc;
      const uint4 wv = codes[(size_t)c * 64];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mc) {
          if (BF16) {
            const uint32_t* xr = static_cast<const uint32_t*>(in) + rows[m] / 2 + c * 16;
            accg[m] = chunk_dot_bf16(wv, xr, accg[m]);
          } else {
            const float* xr = static_cast<const float*>(in) + rows[m] + c * 32;
            accg[m] = chunk_dot_f32(wv, xr, accg[m]);
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < mc) {
        if (BF16) {
          float xs;
          if (sums_per_chunk) {
            xs = 0.f;
            for (int cc = 0; cc < cpg; ++cc) xs += insum[sum_rows[m] + g * cpg + cc];
          } else {
            xs = insum[sum_rows[m] + g];
          }
          acc[m] = fmaf(16.f * s, accg[m] - 1.5f * xs, acc[m]);
        } else {
          acc[m] = fmaf(s, accg[m], acc[m]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------- gate/up + SwiGLU

template <int BF16, int MT, int W>
__global__ __launch_bounds__(64 * W) void k_gateup(const uint8_t* const* __restrict__ wptr,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ n_active,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted,
                                                   const void* __restrict__ x, const float* __restrict__ xsum,
                                                   void* __restrict__ h, float* __restrict__ hpart,
                                                   int64_t off_codes, int64_t off_scales, int chunks, int gblocks,
                                                   int tiles, int H, int I, int G, int k) {
  __shared__ float red[W][MT][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int p0 = offsets[e], M = offsets[e + 1] - p0;
  const uint8_t* base = wptr[e];
  const uint4* codes = reinterpret_cast<const uint4*>(base + off_codes) + (size_t)tile * chunks * 64 + lane;
  const uint4* scales = reinterpret_cast<const uint4*>(base + off_scales) + (size_t)tile * gblocks * 64 + lane;
  const int ng = H / G, cpg = G / 32;
  const int g0 = (ng * wave) / W, g1 = (ng * (wave + 1)) / W;

  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mc = min(MT, M - m0);
    int64_t rows[MT], sum_rows[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int t = sorted[p0 + m0 + min(m, mc - 1)] / k;
      rows[m] = (int64_t)t * H;
      sum_rows[m] = (int64_t)t * ng;
    }
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    k_loop<BF16, MT>(codes, scales, x, xsum, rows, sum_rows, mc, g0, g1, cpg, false, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    if (threadIdx.x < MT * 32) {
      const int m = threadIdx.x >> 5, j = threadIdx.x & 31;
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        gs += red[w][m][j];
        us += red[w][m][32 + j];
      }
      const float hv = gs / (1.f + __expf(-gs)) * us;
      const int64_t p = p0 + m0 + m;
      const int col = tile * 32 + j;
      if (BF16) {
        const uint16_t hb = f32_to_bf16_rne(hv);
        if (m < mc) static_cast<uint16_t*>(h)[p * I + col] = hb;
        float hr = __uint_as_float((uint32_t)hb << 16);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) hr += __shfl_xor(hr, off, 64);
        if (j == 0 && m < mc) hpart[p * (I / 32) + tile] = hr;
      } else {
        if (m < mc) static_cast<float*>(h)[p * I + col] = hv;
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- down projection

template <int BF16, int MT, int W>
__global__ __launch_bounds__(64 * W) void k_down(const uint8_t* const* __restrict__ wptr,
                                                 const int32_t* __restrict__ active,
                                                 const int32_t* __restrict__ n_active,
                                                 const int32_t* __restrict__ offsets, const void* __restrict__ h,
                                                 const float* __restrict__ hpart, float* __restrict__ o,
                                                 int64_t off_codes, int64_t off_scales, int chunks, int gblocks,
                                                 int tiles, int H, int I, int G) {
  __shared__ float red[W][MT][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int p0 = offsets[e], M = offsets[e + 1] - p0;
  const uint8_t* base = wptr[e];
  const uint4* codes = reinterpret_cast<const uint4*>(base + off_codes) + (size_t)tile * chunks * 64 + lane;
  const uint4* scales = reinterpret_cast<const uint4*>(base + off_scales) + (size_t)tile * gblocks * 64 + lane;
  const int ng = I / G, cpg = G / 32;
  const int g0 = (ng * wave) / W, g1 = (ng * (wave + 1)) / W;

  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mc = min(MT, M - m0);
    int64_t rows[MT], sum_rows[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int64_t p = p0 + m0 + min(m, mc - 1);
      rows[m] = p * I;
      sum_rows[m] = p * (I / 32);
    }
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    k_loop<BF16, MT>(codes, scales, h, hpart, rows, sum_rows, mc, g0, g1, cpg, true, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    for (int i = threadIdx.x; i < MT * 64; i += 64 * W) {
      const int m = i >> 6, r = i & 63;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) s += red[w][m][r];
      if (m < mc) o[(int64_t)(p0 + m0 + m) * H + tile * 64 + r] = s;
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------- launchers

template <int BF16, int MT>
static void gateup_w(const GemvArgs& a, int W, int grid, hipStream_t s) {
  if (W == 8)
    hipLaunchKernelGGL((k_gateup<BF16, MT, 8>), dim3(grid), dim3(512), 0, s, a.wptr, a.active, a.n_active,
                       a.offsets, a.sorted, a.in, a.insum, a.out, a.outpart, a.off_codes, a.off_scales, a.chunks,
                       a.gblocks, a.tiles, a.H, a.I, a.G, a.k);
  else
    hipLaunchKernelGGL((k_gateup<BF16, MT, 4>), dim3(grid), dim3(256), 0, s, a.wptr, a.active, a.n_active,
                       a.offsets, a.sorted, a.in, a.insum, a.out, a.outpart, a.off_codes, a.off_scales, a.chunks,
                       a.gblocks, a.tiles, a.H, a.I, a.G, a.k);
}

template <int BF16, int MT>
static void down_w(const GemvArgs& a, int W, int grid, hipStream_t s) {
  if (W == 8)
    hipLaunchKernelGGL((k_down<BF16, MT, 8>), dim3(grid), dim3(512), 0, s, a.wptr, a.active, a.n_active,
                       a.offsets, a.in, a.insum, static_cast<float*>(a.out), a.off_codes, a.off_scales, a.chunks,
                       a.gblocks, a.tiles, a.H, a.I, a.G);
  else
    hipLaunchKernelGGL((k_down<BF16, MT, 4>), dim3(grid), dim3(256), 0, s, a.wptr, a.active, a.n_active,
                       a.offsets, a.in, a.insum, static_cast<float*>(a.out), a.off_codes, a.off_scales, a.chunks,
                       a.gblocks, a.tiles, a.H, a.I, a.G);
}

static int pick_mt(int max_tok) { return max_tok <= 1 ? 1 : max_tok <= 2 ? 2 : max_tok <= 4 ? 4 : 8; }

void launch_gateup(const GemvArgs& a, int act_bf16, int max_tok, int grid, hipStream_t s) {
  const int W = (a.H / a.G) >= 16 ? 8 : 4;
  const int mt = pick_mt(max_tok);
#define GU(B, M) \
  if (act_bf16 == B && mt == M) return gateup_w<B, M>(a, W, grid, s);
  GU(1, 1) GU(1, 2) GU(1, 4) GU(1, 8) GU(0, 1) GU(0, 2) GU(0, 4) GU(0, 8)
#undef GU
}

void launch_down(const GemvArgs& a, int act_bf16, int max_tok, int grid, hipStream_t s) {
  const int W = (a.I / a.G) >= 16 ? 8 : 4;
  const int mt = pick_mt(max_tok);
#define DN(B, M) \
  if (act_bf16 == B && mt == M) return down_w<B, M>(a, W, grid, s);
  DN(1, 1) DN(1, 2) DN(1, 4) DN(1, 8) DN(0, 1) DN(0, 2) DN(0, 4) DN(0, 8)
#undef DN
}

}  // namespace moe
