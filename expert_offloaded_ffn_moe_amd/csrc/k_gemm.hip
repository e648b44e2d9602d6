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

#include <type_traits>

#include "kernels.h"
#include "wave.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const uint16_t gu16;

// (a & m) | c in one instruction. A gfx9 VOP3 instruction reads at most one
// literal or scalar operand, so the two constants are held in vector registers
// and passed in; the compiler would otherwise emit a separate AND and OR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// The nibble mask 0x00780078 and the bf16 pair 1.0, 1.0 = 0x3F803F80, in vector registers.
struct GemmCodeConsts {
  uint32_t m, c;
  __device__ __forceinline__ GemmCodeConsts() {
    asm volatile("v_mov_b32 %0, 0x00780078" : "=v"(m));
    asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(c));
  }
};

// 8 codes of one dword (K offsets 8d .. 8d+7 in order) -> bf16x8 of 1 + n/16:
// pair j of the dword moved to mantissa bits 3..6 of both halves, then masked
// and or-ed into 1.0
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t d, const GemmCodeConsts& k) {
  u32x4 p;
  p.x = and_or(d << 3, k.m, k.c);
  p.y = and_or(d >> 1, k.m, k.c);
  p.z = and_or(d >> 5, k.m, k.c);
  p.w = and_or(d >> 9, k.m, k.c);
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

// fp32 32x32x2: lane l gives A[l % 32][l / 32] and B[l / 32][l % 32]; C/D in the
// same lane layout as the bf16 32x32 MFMA.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// sum over each aligned group of N lanes (N <= 32), in every lane: DPP steps inside a
// row of 16 (quad xor 1, xor 2, half-row mirror, row mirror), one shuffle across rows
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  if (N >= 2) v += dppf<kDppXor1, 0xF>(0.f, v);
  if (N >= 4) v += dppf<kDppXor2, 0xF>(0.f, v);
  if (N >= 8) v += dppf<kDppHalfMirror, 0xF>(0.f, v);
  if (N >= 16) v += dppf<kDppMirror, 0xF>(0.f, v);
  if (N >= 32) v += __shfl_xor(v, 16, 64);
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// ----------------------------------------------------------------------------- router

// logits[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]: one workgroup per 32 x 32
// output tile, its 8 waves splitting K (operands straight from global memory,
// x and Wr rows are K-contiguous); the partial tiles are added in LDS in wave order.
// When xsum is given, workgroups past the logits tiles (all of them when
// tile_blocks is 0) write xsum[t][g] = sum of x[t][gG .. gG+G) for the GEMVs, in
// element order.
__global__ __launch_bounds__(64 * kRouterWaves) void k_router_mfma(const uint16_t* __restrict__ x,
                                                                   const uint16_t* __restrict__ w,
                                                                   const float* __restrict__ b,
                                                                   float* __restrict__ logits, float* __restrict__ xsum,
                                                                   int tile_blocks, int T, int H, int E, int G) {
  __shared__ float part[kRouterWaves][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if ((int)blockIdx.x >= tile_blocks) {
    const int ng = H / G;
    const int gid = (blockIdx.x - tile_blocks) * (64 * kRouterWaves) + threadIdx.x;
    if (gid >= T * ng) return;
    const int t = gid / ng, g = gid % ng;
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * H + (size_t)g * G);
    float sum = 0.f;
    for (int c = 0; c < G / 8; ++c) {
      const uint4 v = src[c];
      sum += bf16_lo(v.x);
      sum += bf16_hi(v.x);
      sum += bf16_lo(v.y);
      sum += bf16_hi(v.y);
      sum += bf16_lo(v.z);
      sum += bf16_hi(v.z);
      sum += bf16_lo(v.w);
      sum += bf16_hi(v.w);
    }
    xsum[gid] = sum;
    return;
  }
  const int nte = (E + 31) / 32;
  const int mt = blockIdx.x / nte, et = blockIdx.x % nte;
  const int i = lane & 31, half = lane >> 5;
  const int row = min(mt * 32 + i, T - 1), col = min(et * 32 + i, E - 1);
  gu32x4* xa = (gu32x4*)(x + (size_t)row * H) + half;
  gu32x4* wb = (gu32x4*)(w + (size_t)col * H) + half;
  const int ks_all = H / 16;  // k-steps of 16
  const int k0 = (ks_all * wave) / kRouterWaves, k1 = (ks_all * (wave + 1)) / kRouterWaves;
  f32x16 acc = {};
  for (int ks = k0; ks < k1; ks += 8) {  // 8 k-steps: all 16 loads before the MFMAs
    u32x4 av[8], bv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kq = min(ks + q, k1 - 1);
      av[q] = xa[2 * kq];
      bv[q] = wb[2 * kq];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (ks + q < k1) acc = mfma(__builtin_bit_cast(bf16x8_t, av[q]), __builtin_bit_cast(bf16x8_t, bv[q]), acc);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) part[wave][v][lane] = acc[v];
  __syncthreads();
  if (wave != 0) return;
  const int j = et * 32 + i;
  if (j >= E) return;
  const float bias = b ? b[j] : 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kRouterWaves; ++ww) sum += part[ww][v][lane];
    const int r = mt * 32 + 8 * (v / 4) + 4 * half + (v % 4);
    if (r < T) logits[(size_t)r * E + j] = sum + bias;
  }
}

void launch_router_mfma(const RouterArgs& a, const Timing& tm, hipStream_t s) {
  const int tiles = a.router_blocks > 0 ? ((a.T + 31) / 32) * ((a.E + 31) / 32) : 0;
  const int xs = a.xsum ? (a.T * (a.H / a.G) + 64 * kRouterWaves - 1) / (64 * kRouterWaves) : 0;
  if (tiles + xs == 0) return;
  launch_timed(k_router_mfma, dim3(tiles + xs), dim3(64 * kRouterWaves), 0, s, tm, static_cast<const uint16_t*>(a.x),
               static_cast<const uint16_t*>(a.w), a.b, a.logits, a.xsum, tiles, a.T, a.H, a.E, a.G);
}

// ----------------------------------------------------------------------------- grouped GEMM

constexpr int kBM = 64;          // token rows per tile
constexpr int kWaves = 4;        // waves per workgroup, one 64-row weight n-tile each

// A tile of one quantisation group in LDS: kBM rows x G bf16, row stride padded
// by 16 bytes; two of them, so staging group g + 1 overlaps the MFMAs of group g.
template <int G>
struct GemmShared {
  static constexpr int kStride = G * 2 + 16;  // bytes
  alignas(16) uint8_t a[2][kBM * kStride];
  float rowsum[2][kBM];
};

// sum of the 8 bf16 of a 16-byte piece, by dot products with (1, 1)
__device__ __forceinline__ float piece_sum(const uint4& v) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.x), one, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.y), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.z), one, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w), one, s, false);
}

// Workgroups are dealt to the 8 XCDs round-robin (block b on XCD b % 8), each XCD
// with its own L2. Logical block ids are laid out so that each XCD runs one
// contiguous range of them: the workgroups of one row tile (same gathered
// activation rows) and of neighbouring row tiles (same expert's weights) then
// share an L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
  constexpr int kXcd = 8;
  const int per = nb / kXcd, rem = nb % kXcd;
  const int x = b % kXcd, i = b / kXcd;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

// One workgroup: tile (expert e, rows [m0, m0 + 64) of its tokens) x 4 weight
// n-tiles of 64 rows. GATEUP: A = gathered x rows (K = H), n-tile = 32 gate + 32
// up rows, epilogue SwiGLU -> h (bf16, by sorted position). Otherwise: A = h rows
// (K = I), n-tile = 64 down rows, epilogue -> o (fp32, by sorted position).
// Per quantisation group: the A rows and the wave's codes and scales of group
// g + 1 are loaded into registers while group g runs on the MFMAs.
template <int G, bool GATEUP>
__global__ __launch_bounds__(256, 2) void k_gemm(const uint8_t* const* __restrict__ wptr,
                                                 const int2* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ sorted, const uint16_t* __restrict__ a_src,
                                                 void* __restrict__ out, int64_t off_codes, int64_t off_scales,
                                                 int chunks, int groups, int ntiles_n, int K, int out_ld, int k) {
  // The loop runs over sub-groups of SG <= 128 K values (G = 256 takes two per
  // quantisation group, sharing its scale), so that two register sets of a
  // sub-group's operands fit beside the accumulators at two waves per SIMD.
  constexpr int SG = G > 128 ? 128 : G, SPG = G / SG;
  constexpr int CPG = SG / 32;
  __shared__ GemmShared<SG> sh;
  const int nsub = groups * SPG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ngroup_wg = (ntiles_n + kWaves - 1) / kWaves;
  // the grid is sized for the most tiles a batch can have; the order is laid out
  // over the tiles this batch has, so every XCD gets its share of the real work
  const int nb = *n_tiles * ngroup_wg;
  if ((int)blockIdx.x >= nb) return;
  const int lb = xcd_logical_block(blockIdx.x, nb);
  const int tile_idx = lb / ngroup_wg;
  const int nt = (lb % ngroup_wg) * kWaves + wave;
  const bool active_wave = nt < ntiles_n;
  const int2 tl = tiles[tile_idx];
  const int e = tl.x, m0 = tl.y;
  const int p0 = offsets[e], M = offsets[e + 1] - p0;
  const int mrows = min(kBM, M - m0);
  const bool two = mrows > 32;  // second 32-row block has rows

  // staging assignment: a group's A tile is 64 rows of PPR = G/8 16-byte pieces;
  // thread t stages pieces t + 256 q (q < CPG): row (t + 256 q) / PPR, piece t % PPR,
  // so PPR consecutive lanes cover one row's contiguous bytes (no LDS bank conflicts)
  constexpr int PPR = SG / 8;
  const int spiece = threadIdx.x % PPR;
  const uint4* src[CPG];
#pragma unroll
  for (int q = 0; q < CPG; ++q) {
    const int r = min((int)(threadIdx.x + 256 * q) / PPR, mrows - 1);
    const int64_t row = GATEUP ? (int64_t)(sorted[p0 + m0 + r] / k) : (int64_t)(p0 + m0 + r);
    src[q] = reinterpret_cast<const uint4*>(a_src + row * K) + spiece;
  }
  const GemmCodeConsts kc;

  const uint8_t* base = wptr[e];
  gu32x4* codes = (gu32x4*)(base + off_codes) + (size_t)(active_wave ? nt : 0) * chunks * 64 + lane;
  gu16* scales = (gu16*)(base + off_scales) + (size_t)(active_wave ? nt : 0) * groups * 64;
  const int i32 = lane & 31, half = lane >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int o = 0; o < 2; ++o) acc[s][o] = f32x16{};
  // the previous group's column factors and row sums (rows 32 s + lane % 32), kept
  // in registers: its LDS buffer is rewritten by waves already on the next group
  float fp0 = 0.f, fp1 = 0.f, rp[2] = {0.f, 0.f};

  // a group's operands in registers: this thread's staging pieces of the A rows,
  // the wave's codes (CPG dwords x 4 per lane) and the two column scales
  struct Regs {
    uint4 a[CPG];
    u32x4 b[CPG];
    uint16_t s0, s1;
  };
  auto load = [&](Regs& r, int gl) {
#pragma unroll
    for (int q = 0; q < CPG; ++q) r.a[q] = src[q][(size_t)gl * PPR];
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) r.b[cc] = codes[(size_t)(gl * CPG + cc) * 64];
    r.s0 = scales[(size_t)(gl / SPG) * 64 + i32];
    r.s1 = scales[(size_t)(gl / SPG) * 64 + 32 + i32];
  };

  // Group g: its A rows (in `cur`) -> LDS buffer g & 1 with their row sums, group
  // g + 1 (clamped to the last group) loaded into `nxt` while g runs on the MFMAs.
  // The two register sets alternate between even and odd groups, so the loads
  // in flight are only waited for where the next group first uses them.
  auto step = [&](auto two_c, auto odd_c, int g, Regs& cur, Regs& nxt) {
    constexpr bool TWO = decltype(two_c)::value;  // second 32-row block has rows
    constexpr bool ODD = decltype(odd_c)::value;  // g is odd
    constexpr int buf = ODD ? 1 : 0;
    {
      float rs[CPG];
#pragma unroll
      for (int q = 0; q < CPG; ++q) {
        const int P = threadIdx.x + 256 * q;
        *reinterpret_cast<uint4*>(sh.a[buf] + (P / PPR) * GemmShared<SG>::kStride + spiece * 16) = cur.a[q];
        rs[q] = piece_sum(cur.a[q]);
      }
#pragma unroll
      for (int q = 0; q < CPG; ++q) rs[q] = lane_group_sum<PPR>(rs[q]);
      if (spiece == 0) {
#pragma unroll
        for (int q = 0; q < CPG; ++q) sh.rowsum[buf][(threadIdx.x + 256 * q) / PPR] = rs[q];
      }
    }
    load(nxt, min(g + 1, nsub - 1));
    __syncthreads();  // buffer `buf` complete; the other one is no longer read
    if (!active_wave) return;
    f32x16 ag[2][2];
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      // lanes 0-31 hold n-tile rows 0-31 (gate), lanes 32-63 rows 32-63 (up / second
      // half), 32 K values each; the swaps give each half's K 0-15 and 16-31 operands
      const auto s01 = __builtin_amdgcn_permlane32_swap(cur.b[cc].x, cur.b[cc].y, false, false);
      const auto s23 = __builtin_amdgcn_permlane32_swap(cur.b[cc].z, cur.b[cc].w, false, false);
      const bf16x8_t b00 = codes_to_bf16(s01[0], kc), b10 = codes_to_bf16(s01[1], kc);  // k-step 0: half 0, half 1
      const bf16x8_t b01 = codes_to_bf16(s23[0], kc), b11 = codes_to_bf16(s23[1], kc);  // k-step 1
#pragma unroll
      for (int s = 0; s < (TWO ? 2 : 1); ++s) {
        const uint8_t* arow = sh.a[buf] + (32 * s + i32) * GemmShared<SG>::kStride + cc * 64 + half * 16;
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow));
        const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(arow + 32));
        ag[s][0] = mfma(a0, b00, cc == 0 ? f32x16{} : ag[s][0]);
        ag[s][1] = mfma(a0, b10, cc == 0 ? f32x16{} : ag[s][1]);
        ag[s][0] = mfma(a1, b01, ag[s][0]);
        ag[s][1] = mfma(a1, b11, ag[s][1]);
      }
    }
    // acc += 16 s * sum x v per output element; the -16 s * 1.5 * sum x part goes in
    // below as a rank-2 fp32 MFMA per two groups (rows' sums x columns' factors)
    const float f0 = 16.f * half_bits(cur.s0), f1 = 16.f * half_bits(cur.s1);
#pragma unroll
    for (int s = 0; s < (TWO ? 2 : 1); ++s) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[s][0][v] = fmaf(f0, ag[s][0][v], acc[s][0][v]);
        acc[s][1][v] = fmaf(f1, ag[s][1][v], acc[s][1][v]);
      }
    }
    // groups (g - 1, g) when g is odd, or the last group alone: A = -1.5 * row sums
    // (k = 0: group g - 1, k = 1: group g), B = the columns' 16 s of those groups
    float rc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) rc[s] = sh.rowsum[buf][32 * s + i32];
    if (ODD || g == nsub - 1) {
      const int kg = half;  // this lane's k: 0 -> previous group, 1 -> this one
      const float fb0 = ODD ? (kg ? f0 : fp0) : (kg ? 0.f : f0);
      const float fb1 = ODD ? (kg ? f1 : fp1) : (kg ? 0.f : f1);
#pragma unroll
      for (int s = 0; s < (TWO ? 2 : 1); ++s) {
        const float ra = -1.5f * ((ODD && !kg) ? rp[s] : rc[s]);
        acc[s][0] = mfma_f32(ra, fb0, acc[s][0]);
        acc[s][1] = mfma_f32(ra, fb1, acc[s][1]);
      }
    }
    if (!ODD) {
      fp0 = f0;
      fp1 = f1;
      rp[0] = rc[0];
      rp[1] = rc[1];
    }
  };

  Regs r0, r1;
  load(r0, 0);
  auto run = [&](auto two_c) {
    for (int g = 0; g < nsub; g += 2) {
      step(two_c, std::false_type{}, g, r0, r1);
      if (g + 1 < nsub) step(two_c, std::true_type{}, g + 1, r1, r0);
    }
  };
  if (two)
    run(std::true_type{});
  else
    run(std::false_type{});
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
