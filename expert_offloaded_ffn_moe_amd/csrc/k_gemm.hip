// Prefill path on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16): the router as a
// dense GEMM, and the per-expert SwiGLU FFN as grouped GEMMs over the tokens
// routed to each expert. With many tokens per expert (a prefill micro-batch,
// page "125B 稀疏模型塞进一张 32GB 消费卡", section "真正卡死容量的是一块计算缓冲",
// sets it at 2048 or 1024 tokens) the expert FFN is a real dense contraction.
//
// MFMA 32x32x16 lane layout (checked on the hardware): lane l supplies A[i][k]
// for i = l % 32, k = 8 * (l / 32) + e (e = 0..7), B[k][j] for j = l % 32 and
// the same k; it receives C[i][j] for j = l % 32, i = 8 * (v / 4) + 4 * (l / 32)
// + v % 4 (v = 0..15).
//
// int4 weights stay exact: a code n = q + 8 in the top mantissa bits of a bf16
// 1.0 is v = 1.5 + q / 16; per quantisation group the MFMA sums x * v in fp32
// and sum x q = 16 * (that - 1.5 * sum x), with the row sums of x taken while
// the activation tile is staged in LDS. The group scale multiplies that fp32
// partial sum, so no rounded q * s ever enters the MFMA.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const uint16_t gu16;

__device__ __forceinline__ uint32_t pair0(uint32_t d) { return ((d << 3) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair1(uint32_t d) { return ((d >> 1) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair2(uint32_t d) { return ((d >> 5) & 0x00780078u) | 0x3F803F80u; }
__device__ __forceinline__ uint32_t pair3(uint32_t d) { return ((d >> 9) & 0x00780078u) | 0x3F803F80u; }

// 8 codes of one dword (K offsets 8d .. 8d+7 in order) -> bf16x8 of 1 + n/16
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t d) {
  u32x4 p;
  p.x = pair0(d);
  p.y = pair1(d);
  p.z = pair2(d);
  p.w = pair3(d);
  return __builtin_bit_cast(bf16x8_t, p);
}

__device__ __forceinline__ float half_bits(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ----------------------------------------------------------------------------- router

// logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]: one wave per 32 x 32 output
// tile, operands read straight from global memory (x and Wr rows are K-contiguous).
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                     const float* __restrict__ b, float* __restrict__ logits, int T,
                                                     int H, int E) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nte = (E + 31) / 32;
  const int mt = wave / nte, et = wave % nte;
  if (mt * 32 >= T) return;
  const int i = lane & 31, half = lane >> 5;
  const int row = min(mt * 32 + i, T - 1), col = min(et * 32 + i, E - 1);
  gu32x4* xa = (gu32x4*)(x + (size_t)row * H) + half;
  gu32x4* wb = (gu32x4*)(w + (size_t)col * H) + half;
  f32x16 acc = {};
  int k0 = 0;
  for (; k0 + 128 <= H; k0 += 128) {  // 8 k-steps: all 16 loads before the MFMAs
    u32x4 av[8], bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      av[q] = xa[(k0 + 16 * q) / 8];
      bv[q] = wb[(k0 + 16 * q) / 8];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = mfma(__builtin_bit_cast(bf16x8_t, av[q]), __builtin_bit_cast(bf16x8_t, bv[q]), acc);
  }
  for (; k0 < H; k0 += 16) {
    const u32x4 av = xa[k0 / 8], bv = wb[k0 / 8];
    acc = mfma(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv), acc);
  }
  const int j = et * 32 + i;
  if (j < E) {
    const float bias = b ? b[j] : 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = mt * 32 + 8 * (v / 4) + 4 * half + (v % 4);
      if (r < T) logits[(size_t)r * E + j] = acc[v] + bias;
    }
  }
}

void launch_router_mfma(const RouterArgs& a, const Timing& tm, hipStream_t s) {
  const int waves = ((a.T + 31) / 32) * ((a.E + 31) / 32);
  launch_timed(k_router_mfma, dim3((waves + 3) / 4), dim3(256), 0, s, tm, static_cast<const uint16_t*>(a.x),
               static_cast<const uint16_t*>(a.w), a.b, a.logits, a.T, a.H, a.E);
}

// ----------------------------------------------------------------------------- grouped GEMM

constexpr int kBM = 64;          // token rows per tile
constexpr int kWaves = 4;        // waves per workgroup, one 64-row weight n-tile each

// A tile of one quantisation group in LDS: kBM rows x G bf16, row stride padded by 16 bytes.
template <int G>
struct GemmShared {
  static constexpr int kStride = G * 2 + 16;  // bytes
  uint8_t a[kBM * kStride];
  float rowsum[kBM];
};

// One workgroup: tile (expert e, rows [m0, m0 + 64) of its tokens) x 4 weight
// n-tiles of 64 rows. GATEUP: A = gathered x rows (K = H), n-tile = 32 gate + 32
// up rows, epilogue SwiGLU -> h (bf16, by sorted position). Otherwise: A = h rows
// (K = I), n-tile = 64 down rows, epilogue -> o (fp32, by sorted position).
template <int G, bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* const* __restrict__ wptr,
                                              const int2* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
                                              const int32_t* __restrict__ offsets,
                                              const int32_t* __restrict__ sorted, const uint16_t* __restrict__ a_src,
                                              void* __restrict__ out, int64_t off_codes, int64_t off_scales,
                                              int chunks, int groups, int ntiles_n, int K, int out_ld, int k) {
  constexpr int CPG = G / 32;
  __shared__ GemmShared<G> sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ngroup_wg = (ntiles_n + kWaves - 1) / kWaves;
  const int tile_idx = blockIdx.x / ngroup_wg;
  if (tile_idx >= *n_tiles) return;
  const int nt = (blockIdx.x % ngroup_wg) * kWaves + wave;
  const bool active_wave = nt < ntiles_n;
  const int2 tl = tiles[tile_idx];
  const int e = tl.x, m0 = tl.y;
  const int p0 = offsets[e], M = offsets[e + 1] - p0;
  const int mrows = min(kBM, M - m0);

  // staging assignment: 4 threads per row, G/32 16-byte pieces each
  const int srow = threadIdx.x >> 2, spart = threadIdx.x & 3;
  const int src_r = min(srow, mrows - 1);
  const int64_t src_row = GATEUP ? (int64_t)(sorted[p0 + m0 + src_r] / k) : (int64_t)(p0 + m0 + src_r);
  const uint16_t* src = a_src + src_row * K;

  const uint8_t* base = wptr[e];
  gu32x4* codes = (gu32x4*)(base + off_codes) + (size_t)(active_wave ? nt : 0) * chunks * 64 + lane;
  gu16* scales = (gu16*)(base + off_scales) + (size_t)(active_wave ? nt : 0) * groups * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int o = 0; o < 2; ++o) acc[s][o] = f32x16{};

  const int i32 = lane & 31, half = lane >> 5;
  for (int g = 0; g < groups; ++g) {
    // stage A[64][G] of this group, with per-row sums
    __syncthreads();
    {
      float rs = 0.f;
#pragma unroll
      for (int q = 0; q < CPG; ++q) {
        const int piece = spart * CPG + q;  // 16-byte piece (8 values) of the row
        const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)g * G + piece * 8);
        *reinterpret_cast<uint4*>(sh.a + srow * GemmShared<G>::kStride + piece * 16) = v;
        rs += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) + bf16_hi(v.z) +
              bf16_lo(v.w) + bf16_hi(v.w);
      }
      rs += __shfl_xor(rs, 1, 64);
      rs += __shfl_xor(rs, 2, 64);
      if (spart == 0) sh.rowsum[srow] = rs;
    }
    __syncthreads();
    if (!active_wave) continue;
    const float sc0 = half_bits(scales[(size_t)g * 64 + i32]);
    const float sc1 = half_bits(scales[(size_t)g * 64 + 32 + i32]);
    f32x16 ag[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int o = 0; o < 2; ++o) ag[s][o] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = g * CPG + cc;
      u32x4 wv = codes[(size_t)c * 64];
      // lanes 0-31 hold n-tile rows 0-31 (gate), lanes 32-63 rows 32-63 (up / second
      // half), 32 K values each; the swaps give each half's K 0-15 and 16-31 operands
      const auto s01 = __builtin_amdgcn_permlane32_swap(wv.x, wv.y, false, false);
      const auto s23 = __builtin_amdgcn_permlane32_swap(wv.z, wv.w, false, false);
      const bf16x8_t b00 = codes_to_bf16(s01[0]), b10 = codes_to_bf16(s01[1]);  // k-step 0: half 0, half 1
      const bf16x8_t b01 = codes_to_bf16(s23[0]), b11 = codes_to_bf16(s23[1]);  // k-step 1
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* arow = sh.a + (32 * s + i32) * GemmShared<G>::kStride + cc * 64 + half * 16;
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow));
        const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow + 32));
        ag[s][0] = mfma(a0, b00, ag[s][0]);
        ag[s][1] = mfma(a0, b10, ag[s][1]);
        ag[s][0] = mfma(a1, b01, ag[s][0]);
        ag[s][1] = mfma(a1, b11, ag[s][1]);
      }
    }
    // acc += 16 * s * (sum x v - 1.5 * sum x), per output element
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float r15 = 1.5f * sh.rowsum[32 * s + 8 * (v / 4) + 4 * half + (v % 4)];
        acc[s][0][v] = fmaf(16.f * sc0, ag[s][0][v] - r15, acc[s][0][v]);
        acc[s][1][v] = fmaf(16.f * sc1, ag[s][1][v] - r15, acc[s][1][v]);
      }
    }
  }
  if (!active_wave) return;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * s + 8 * (v / 4) + 4 * half + (v % 4);
      if (r < mrows) {
        const int64_t p = p0 + m0 + r;
        if (GATEUP) {
          const float gv = acc[s][0][v], uv = acc[s][1][v];
          const float hv = gv / (1.f + __expf(-gv)) * uv;
          static_cast<uint16_t*>(out)[p * out_ld + nt * 32 + i32] = f32_to_bf16_rne(hv);
        } else {
          float* o = static_cast<float*>(out) + p * out_ld + nt * 64;
          o[i32] = acc[s][0][v];
          o[32 + i32] = acc[s][1][v];
        }
      }
    }
  }
}

template <bool GATEUP>
static void gemm_g(const GemmArgs& a, const Timing& tm, hipStream_t s) {
  const int ngroup_wg = (a.ntiles_n + kWaves - 1) / kWaves;
  const dim3 grid(a.max_tiles * ngroup_wg), block(64 * kWaves);
#define GEMM_LAUNCH(GG)                                                                                          \
  launch_timed(k_gemm<GG, GATEUP>, grid, block, 0, s, tm, a.wptr, a.tiles, a.n_tiles, a.offsets, a.sorted, a.a_src, \
               a.out, a.off_codes, a.off_scales, a.chunks, a.groups, a.ntiles_n, a.K, a.out_ld, a.k)
  switch (a.G) {
    case 32: GEMM_LAUNCH(32); break;
    case 64: GEMM_LAUNCH(64); break;
    case 128: GEMM_LAUNCH(128); break;
    default: GEMM_LAUNCH(256); break;
  }
#undef GEMM_LAUNCH
}

void launch_gemm_gateup(const GemmArgs& a, const Timing& tm, hipStream_t s) { gemm_g<true>(a, tm, s); }
void launch_gemm_down(const GemmArgs& a, const Timing& tm, hipStream_t s) { gemm_g<false>(a, tm, s); }

}  // namespace moe
