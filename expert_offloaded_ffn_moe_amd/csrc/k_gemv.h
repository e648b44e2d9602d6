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
// KiB. A wave issues the loads of up to 16 chunks (and their group scales)
// before any arithmetic. The activations of the tokens routed to the expert are
// wave-uniform and come in through scalar loads. Partial sums of the W waves
// are added in LDS in wave order, so the summation order is fixed.
//
// bf16 activations: a nibble n = q + 8 placed in the top mantissa bits of a
// bf16 1.0 gives v = 1 + n/16 = 1.5 + q/16 exactly; v_dot2_f32_bf16 multiplies
// two such values by two activations per instruction. Over a group,
// sum q x = 16 * (sum v x - 1.5 * sum x), with sum x precomputed per group, so
// the int4 weight is exact and only fp32 accumulation rounds.
// fp32 activations: q is converted exactly to fp32 and used in fmaf.
//
// 2- and 3-bit codes (the lower-bit formats: odd levels q = 2n - (2^b - 1)): a lane
// word holds 64 values of K, their low two bits at mantissa bits 5..6 (2-bit,
// v = 1 + n/4) or 4..5 (3-bit, v = 1 + n/8, the third bit from the high-plane word
// at mantissa bit 6), one shift and mask per pair of values as for 4-bit codes.
// Over a group, sum q x = A (sum v x - C sum x) with (A, C) = (16, 1.5) for 4-bit
// codes, (8, 1.375) for 2-bit and (16, 1.4375) for 3-bit, all exact in fp32.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// The nibble mask 0x00780078 and the bf16 pair (1.0, 1.0), placed in vector registers
// by asm that the compiler cannot see through. A gfx9 VOP3 instruction reads at most
// one literal or scalar operand, so with the constants folded in as literals the
// compiler emits an AND and an OR per pair; with both in vector registers it forms one
// v_and_or_b32 (a quarter fewer VALU instructions per chunk; 7168-wide layer: gate/up
// 21.0 -> 20.0 us at batch 1, fused down + combine 33.0 -> 29.3 us at batch 4). A
// kernel builds them once, before its K loop, and passes them down: the compiler does
// not merge separate constructions, and then would not share one pair's conversion
// among the token rows that use it.
// The 2- and 3-bit codes use the same form with their own masks: m selects the low two
// bits of both halves' codes at their mantissa places, mh the third bit of 3-bit codes.
template <int BITS>
struct CodeConsts {
  uint32_t m, c, mh;
  __device__ __forceinline__ CodeConsts() {
    if (BITS == 4)
      asm("v_mov_b32 %0, 0x00780078" : "=v"(m));
    else if (BITS == 3)
      asm("v_mov_b32 %0, 0x00300030" : "=v"(m));
    else
      asm("v_mov_b32 %0, 0x00600060" : "=v"(m));
    asm("v_mov_b32 %0, 0x3f803f80" : "=v"(c));
    asm("v_mov_b32 %0, 0x00400040" : "=v"(mh));
  }
};
typedef CodeConsts<4> PairConsts;

// bf16 pair (1 + n_lo/16, 1 + n_hi/16) of pair j of a code dword
static __device__ __forceinline__ uint32_t pair0(uint32_t d, const PairConsts& k) { return ((d << 3) & k.m) | k.c; }
static __device__ __forceinline__ uint32_t pair1(uint32_t d, const PairConsts& k) { return ((d >> 1) & k.m) | k.c; }
static __device__ __forceinline__ uint32_t pair2(uint32_t d, const PairConsts& k) { return ((d >> 5) & k.m) | k.c; }
static __device__ __forceinline__ uint32_t pair3(uint32_t d, const PairConsts& k) { return ((d >> 9) & k.m) | k.c; }

static __device__ __forceinline__ float half_bits(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

static __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// acc + sum_i v_i x_i over one 32-wide chunk, v = 1 + n/16 (bf16 path)
template <typename P>
static __device__ __forceinline__ float chunk_dot_bf16(const u32x4& wv, const P& xr, float acc, const PairConsts& k) {
  acc = dot2(pair0(wv.x, k), xr[0], acc);
  acc = dot2(pair1(wv.x, k), xr[1], acc);
  acc = dot2(pair2(wv.x, k), xr[2], acc);
  acc = dot2(pair3(wv.x, k), xr[3], acc);
  acc = dot2(pair0(wv.y, k), xr[4], acc);
  acc = dot2(pair1(wv.y, k), xr[5], acc);
  acc = dot2(pair2(wv.y, k), xr[6], acc);
  acc = dot2(pair3(wv.y, k), xr[7], acc);
  acc = dot2(pair0(wv.z, k), xr[8], acc);
  acc = dot2(pair1(wv.z, k), xr[9], acc);
  acc = dot2(pair2(wv.z, k), xr[10], acc);
  acc = dot2(pair3(wv.z, k), xr[11], acc);
  acc = dot2(pair0(wv.w, k), xr[12], acc);
  acc = dot2(pair1(wv.w, k), xr[13], acc);
  acc = dot2(pair2(wv.w, k), xr[14], acc);
  acc = dot2(pair3(wv.w, k), xr[15], acc);
  return acc;
}

// acc + sum_i q_i x_i, q = n - 8 exact in fp32 (fp32 path)
template <typename P>
static __device__ __forceinline__ float dword_dot_f32(uint32_t d, const P& xr, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float qlo = (float)(int)((d >> (4 * j)) & 0xFu) - 8.f;
    const float qhi = (float)(int)((d >> (16 + 4 * j)) & 0xFu) - 8.f;
    acc = fmaf(qlo, xr[2 * j], acc);
    acc = fmaf(qhi, xr[2 * j + 1], acc);
  }
  return acc;
}

template <typename P>
static __device__ __forceinline__ float chunk_dot_f32(const u32x4& wv, const P& xr, float acc) {
  acc = dword_dot_f32(wv.x, &xr[0], acc);
  acc = dword_dot_f32(wv.y, &xr[8], acc);
  acc = dword_dot_f32(wv.z, &xr[16], acc);
  acc = dword_dot_f32(wv.w, &xr[24], acc);
  return acc;
}

typedef __attribute__((address_space(1))) const u32x4 guint4;    // global-memory views, so
typedef __attribute__((address_space(1))) const uint16_t gushort;  // loads are global_load, not flat
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 guint2;

// K values per 16-byte lane word, and the group-sum constants of the bf16 path.
template <int BITS> constexpr int kChunkK = BITS == 4 ? 32 : 64;
template <int BITS> constexpr float kFixA = BITS == 2 ? 8.f : 16.f;
template <int BITS> constexpr float kFixC = BITS == 4 ? 1.5f : BITS == 3 ? 1.4375f : 1.375f;

// x << sh for sh >= 0, x >> -sh otherwise (sh a constant after unrolling)
static __device__ __forceinline__ uint32_t shift_by(uint32_t x, int sh) { return sh >= 0 ? x << sh : x >> -sh; }

// acc + sum_i v_i x_i over the 64 values of a 2- or 3-bit lane word: dword d pair j
// (values 16d+2j, 16d+2j+1) against x pair 8d+j; for 3-bit codes the third bit of
// that pair is bit i = 8 (d & 1) + j (and 16 + i) of high-plane dword d >> 1.
template <int BITS, typename P>
static __device__ __forceinline__ float chunk_dot_bf16_low(const u32x4& wv, const u32x2& hv, const P& xr, float acc,
                                                           const CodeConsts<BITS>& k) {
  const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
  const uint32_t h[2] = {hv.x, hv.y};
  constexpr int kDst = BITS == 2 ? 5 : 4;  // mantissa bit of the code's lowest bit
#pragma unroll
  for (int d = 0; d < 4; ++d) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t v = (shift_by(w[d], kDst - 2 * j) & k.m) | k.c;  // k.m = (3 << kDst) | (3 << (16 + kDst))
      if (BITS == 3) v |= shift_by(h[d >> 1], 6 - (8 * (d & 1) + j)) & k.mh;
      acc = dot2(v, xr[8 * d + j], acc);
    }
  }
  return acc;
}

constexpr int kBatch = 8;   // chunks whose loads are issued together
constexpr int kMaxW = 16;   // waves per workgroup at most
// Multi-token variants keep twice the accumulators and activation registers;
// they run at most 8 waves per workgroup so that 256 VGPRs fit without spills.
template <int MT>
constexpr int kMaxThreads = MT == 1 ? 1024 : 512;

// K loop of one wave over groups [g0, g1) (CPG chunks each) for MT token rows.
// rows[m]: element offset of token m's activation row in `in`; sum_rows[m]: offset
// of its per-group (gate/up) or per-chunk (down) sums in insum (bf16 path).
// Each batch issues kBatch code loads and their scale loads unconditionally,
// indices clamped to the wave's last chunk/group (repeats hit in cache), then
// computes on the groups that exist.
typedef __attribute__((address_space(3))) const uint32_t lds_u32;
typedef __attribute__((address_space(3))) const float lds_f32;

// Activation chunk c of row `row` (element offset): XS == 0 reads it from global
// memory (wave-uniform address, scalar loads), XS == 1 from the LDS copy.
template <int XS, int BITS = 4>
static __device__ __forceinline__ float chunk_dot_bf16_src(const u32x4& wv, const u32x2& hv, const void* in,
                                                           int64_t row, int c, float acc, const CodeConsts<BITS>& k) {
  constexpr int NX = kChunkK<BITS> / 2;  // x pairs per lane word
  if (XS) {
    lds_u32* xr = (lds_u32*)in + row / 2 + c * NX;
    uint32_t v[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) v[i] = xr[i];
    if constexpr (BITS == 4) return chunk_dot_bf16(wv, v, acc, k);
    else return chunk_dot_bf16_low<BITS>(wv, hv, v, acc, k);
  }
  const uint32_t* xg = static_cast<const uint32_t*>(in) + row / 2 + c * NX;
  if constexpr (BITS == 4) return chunk_dot_bf16(wv, xg, acc, k);
  else return chunk_dot_bf16_low<BITS>(wv, hv, xg, acc, k);
}

template <int XS>
static __device__ __forceinline__ float chunk_dot_f32_src(const u32x4& wv, const void* in, int64_t row, int c,
                                                          float acc) {
  if (XS) {
    lds_f32* xr = (lds_f32*)in + row + c * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = xr[i];
    return chunk_dot_f32(wv, v, acc);
  }
  return chunk_dot_f32(wv, static_cast<const float*>(in) + row + c * 32, acc);
}

// One batch: kBatch code chunks (GB groups) and their scales (and, for 3-bit codes,
// the chunks' high-plane words), loaded unconditionally with indices clamped to the
// wave's last chunk/group (repeats hit in cache).
template <int CPG, int BITS = 4, int NBATCH = kBatch>
struct Batch {
  static constexpr int NB = CPG > NBATCH ? CPG : NBATCH;
  static constexpr int GB = NB / CPG;
  u32x4 wv[NB];
  u32x2 hv[BITS == 3 ? NB : 1];
  uint16_t sb[GB];
  __device__ __forceinline__ void load(guint4* codes, guint2* his, gushort* scales, int gb, int g1) {
    const int c_last = g1 * CPG - 1;
#pragma unroll
    for (int q = 0; q < GB; ++q) sb[q] = scales[(size_t)min(gb + q, g1 - 1) * 64];
#pragma unroll
    for (int i = 0; i < NB; ++i) wv[i] = codes[(size_t)min(gb * CPG + i, c_last) * 64];
    if (BITS == 3) {
#pragma unroll
      for (int i = 0; i < NB; ++i) hv[i] = his[(size_t)min(gb * CPG + i, c_last) * 64];
    } else {
      hv[0] = u32x2{0u, 0u};
    }
  }
  __device__ __forceinline__ const u32x2& high(int i) const { return hv[BITS == 3 ? i : 0]; }
};

// Arithmetic of one batch starting at group gb: groups past g1 repeat the last
// group and count with weight 0 (no branch, so loads issued earlier stay ahead).
template <int BF16, int MT, int CPG, bool SUMS_PER_CHUNK, int XS, int BITS = 4, int NBATCH = kBatch>
static __device__ __forceinline__ void batch_math(const Batch<CPG, BITS, NBATCH>& bt, const void* __restrict__ in,
                                                  const float* __restrict__ insum, const int64_t* rows,
                                                  const int64_t* sum_rows, int mc, int gb, int g1, float* acc,
                                                  const CodeConsts<BITS>& k) {
  constexpr int SPG = CPG * kChunkK<BITS> / 32;  // 32-value sums (down: h chunk sums) per group
#pragma unroll
  for (int q = 0; q < Batch<CPG, BITS, NBATCH>::GB; ++q) {
    const int g = min(gb + q, g1 - 1);
    const float keep = (gb + q < g1) ? 1.f : 0.f;
    float accg[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) accg[m] = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPG; ++cc) {
      const int c = g * CPG + cc;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mc) {
          if (BF16)
            accg[m] = chunk_dot_bf16_src<XS, BITS>(bt.wv[q * CPG + cc], bt.high(q * CPG + cc), in, rows[m], c,
                                                   accg[m], k);
          else
            accg[m] = chunk_dot_f32_src<XS>(bt.wv[q * CPG + cc], in, rows[m], c, accg[m]);
        }
      }
    }
    const float s = keep * half_bits(bt.sb[q]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < mc) {
        if (BF16) {
          float xs;
          if (SUMS_PER_CHUNK) {
            xs = 0.f;
#pragma unroll
            for (int cc = 0; cc < SPG; ++cc) xs += insum[sum_rows[m] + g * SPG + cc];
          } else {
            xs = insum[sum_rows[m] + g];
          }
          acc[m] = fmaf(kFixA<BITS> * s, accg[m] - kFixC<BITS> * xs, acc[m]);
        } else {
          acc[m] = fmaf(s, accg[m], acc[m]);
        }
      }
    }
  }
}

// K loop of wave `part` of the `parts` waves that split a row tile's K, over the
// load batches part, part + parts, ... (GB groups of CPG chunks each) of `groups`
// groups, for MT token rows. rows[m]: element offset of token m's activation row in
// `in`; sum_rows[m]: offset of its per-group (gate/up) or per-chunk (down) sums in
// insum (bf16 path). Interleaving the batches makes the waves of a workgroup read
// neighbouring kilobytes at the same time instead of one distant range each, which
// the memory serves faster (7168-wide layer, batch 1: gate/up 23.7 -> 21.1 us).
// Each batch issues all of its loads before its arithmetic. (Issuing the next
// batch's loads ahead of the current batch's arithmetic measured slower here:
// the second register set costs more occupancy than the overlap gains; 7168-wide
// layer, batch 1, gate/up: 23.3 -> 26.8 us. Batches of 16 chunks for one token
// also lost: 23.9 -> 24.8 us there, and 6.7 -> 9.0 us on a 2048-wide layer.)
template <int BF16, int MT, int CPG, bool SUMS_PER_CHUNK, int XS, int BITS = 4, int NBATCH = kBatch>
static __device__ __forceinline__ void k_loop(guint4* codes, guint2* his, gushort* scales, const void* __restrict__ in,
                                              const float* __restrict__ insum, const int64_t* rows,
                                              const int64_t* sum_rows, int mc, int part, int parts, int groups,
                                              float* acc) {
  constexpr int GB = Batch<CPG, BITS, NBATCH>::GB;
  const int g1 = groups;
  const CodeConsts<BITS> k;
  for (int gb = part * GB; gb < g1; gb += GB * parts) {
    Batch<CPG, BITS, NBATCH> A;
    A.load(codes, his, scales, gb, g1);
    batch_math<BF16, MT, CPG, SUMS_PER_CHUNK, XS, BITS, NBATCH>(A, in, insum, rows, sum_rows, mc, gb, g1, acc, k);
  }
}

// ----------------------------------------------------------------------------- gate/up + SwiGLU

// Activation rows of the current token pass staged in dynamic LDS (XS == 1).
extern __shared__ uint4 moe_dyn_lds[];

// Copy MT rows of `len16` 16-byte units (rows[m] / elements given by idx) to LDS.
static __device__ __forceinline__ void stage_rows(const void* __restrict__ src, const int64_t* src_rows16,
                                                  int mc, int len16) {
  const uint4* s4 = static_cast<const uint4*>(src);
  for (int m = 0; m < mc; ++m)
    for (int i = threadIdx.x; i < len16; i += blockDim.x) moe_dyn_lds[m * len16 + i] = s4[src_rows16[m] + i];
}

// The rows of one active expert and one output tile, MT token rows per pass
// (red: the workgroup's [W][MT][64] partial sums in LDS).
template <int BF16, int MT, int CPG, int XS, int BITS>
static __device__ __forceinline__ void gateup_expert(float* __restrict__ red, int W, int wave, int lane, int tile,
                                                     const WorkDesc* d, int M, int p0, guint4* codes, guint2* his,
                                                     gushort* scales, const int32_t* __restrict__ sorted,
                                                     const void* __restrict__ x, const float* __restrict__ xsum,
                                                     void* __restrict__ h, float* __restrict__ hpart, int groups,
                                                     int H, int I, int k) {
  for (int m0 = 0; m0 < M; m0 += MT) {
    const int mc = min(MT, M - m0);
    int64_t rows[MT], sum_rows[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = m0 + min(m, mc - 1);
      const int t = (MT <= kDescTok && m0 == 0) ? d->tok[min(m, mc - 1)] : sorted[p0 + r] / k;
      rows[m] = (int64_t)t * H;
      sum_rows[m] = (int64_t)t * groups;
    }
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.f;
    if (XS) {
      const int len16 = H * (BF16 ? 2 : 4) / 16;
      int64_t src16[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        src16[m] = rows[m] * (BF16 ? 2 : 4) / 16;
        rows[m] = (int64_t)m * H;
      }
      stage_rows(x, src16, mc, len16);
      __syncthreads();
      k_loop<BF16, MT, CPG, false, XS, BITS>(codes, his, scales, moe_dyn_lds, xsum, rows, sum_rows, mc, wave, W, groups,
                                             acc);
    } else {
      k_loop<BF16, MT, CPG, false, XS, BITS>(codes, his, scales, x, xsum, rows, sum_rows, mc, wave, W, groups, acc);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) red[(wave * MT + m) * 64 + lane] = acc[m];
    __syncthreads();
    for (int i = threadIdx.x; i < MT * 32; i += blockDim.x) {  // whole 32-lane groups per m
      const int m = i >> 5, j = i & 31;
      float gs = 0.f, us = 0.f;
      for (int w = 0; w < W; ++w) {
        gs += red[(w * MT + m) * 64 + j];
        us += red[(w * MT + m) * 64 + 32 + j];
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

// A workgroup: (active-expert slot, output tile). Multi-token variants (MT > 1)
// give an expert that holds a single token the one-token path, whose activation
// row comes in through scalar loads with no LDS staging or barrier before the
// weights: in a batch of a few tokens most experts hold one.
template <int BF16, int MT, int CPG, int XS, int BITS>
__global__ __launch_bounds__(kMaxThreads<MT>) void k_gateup(const WorkDesc* __restrict__ work,
                                                   const int32_t* __restrict__ sorted,
                                                   const void* __restrict__ x, const float* __restrict__ xsum,
                                                   void* __restrict__ h, float* __restrict__ hpart,
                                                   int64_t off_codes, int64_t off_hi, int64_t off_scales, int chunks,
                                                   int groups, int tiles, int H, int I, int k) {
  __shared__ float red[kMaxW * MT * 64];
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  // slots past the active count carry M = 0 (written by the grouping step), so
  // the descriptor is the only dependent load before the weights
  const WorkDesc* d = work + slot;
  const uint8_t* base = d->w;
  int M = d->M;
  asm volatile("" : "+v"(M) : "v"(base));  // fetch the blob pointer with the row count, not after it
  M = __builtin_amdgcn_readfirstlane(M);    // wave-uniform again for the compiler
  const int p0 = d->p0;
  guint4* codes = (guint4*)(base + off_codes) + (size_t)tile * chunks * 64 + lane;
  guint2* his = (guint2*)(base + off_hi) + (size_t)tile * chunks * 64 + lane;
  gushort* scales = (gushort*)(base + off_scales) + (size_t)tile * groups * 64 + lane;
  if (MT > 1 && M == 1)
    gateup_expert<BF16, 1, CPG, 0, BITS>(red, W, wave, lane, tile, d, M, p0, codes, his, scales, sorted, x, xsum, h,
                                         hpart, groups, H, I, k);
  else
    gateup_expert<BF16, MT, CPG, XS, BITS>(red, W, wave, lane, tile, d, M, p0, codes, his, scales, sorted, x, xsum, h,
                                           hpart, groups, H, I, k);
}

// ----------------------------------------------------------------------------- down projection

template <int BF16, int MT, int CPG, int XS, int BITS>
__global__ __launch_bounds__(kMaxThreads<MT>) void k_down(const WorkDesc* __restrict__ work, const void* __restrict__ h,
                                                 const float* __restrict__ hpart, float* __restrict__ o,
                                                 int64_t off_codes, int64_t off_hi, int64_t off_scales, int chunks,
                                                 int groups, int tiles, int H, int I) {
  __shared__ float red[kMaxW][MT][64];
  const int W = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  // slots past the active count carry M = 0 (written by the grouping step), so
  // the descriptor is the only dependent load before the weights
  const WorkDesc* d = work + slot;
  const uint8_t* base = d->w;
  int M = d->M;
  asm volatile("" : "+v"(M) : "v"(base));  // fetch the blob pointer with the row count, not after it
  M = __builtin_amdgcn_readfirstlane(M);    // wave-uniform again for the compiler
  const int p0 = d->p0;
  guint4* codes = (guint4*)(base + off_codes) + (size_t)tile * chunks * 64 + lane;
  guint2* his = (guint2*)(base + off_hi) + (size_t)tile * chunks * 64 + lane;
  gushort* scales = (gushort*)(base + off_scales) + (size_t)tile * groups * 64 + lane;

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
    if (XS) {
      const int len16 = I * (BF16 ? 2 : 4) / 16;
      int64_t src16[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        src16[m] = rows[m] * (BF16 ? 2 : 4) / 16;
        rows[m] = (int64_t)m * I;
      }
      stage_rows(h, src16, mc, len16);
      __syncthreads();
      k_loop<BF16, MT, CPG, true, XS, BITS>(codes, his, scales, moe_dyn_lds, hpart, rows, sum_rows, mc, wave, W, groups,
                                            acc);
    } else {
      k_loop<BF16, MT, CPG, true, XS, BITS>(codes, his, scales, h, hpart, rows, sum_rows, mc, wave, W, groups, acc);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    for (int i = threadIdx.x; i < MT * 64; i += 64 * W) {
      const int m = i >> 6, r = i & 63;
      float s = 0.f;
      for (int w = 0; w < W; ++w) s += red[w][m][r];
      if (m < mc) o[(int64_t)(p0 + m0 + m) * H + tile * 64 + r] = s;
    }
    __syncthreads();
  }
}


// ----------------------------------------------------------------------------- launch

// Launch shape of one dequant-GEMV launch, chosen by the policy in k_gemv.hip:
// tokens per pass (mt), waves per workgroup, activations staged in LDS or not.
struct GemvShape {
  int mt, waves;
  bool lds;
};

template <int BF16, int MT, int CPG, int BITS>
static void gateup_launch3(const GemvArgs& a, const GemvShape& sh, int grid, const Timing& tm, hipStream_t s) {
  const size_t lds = (size_t)MT * a.H * (BF16 ? 2 : 4);
  if (sh.lds)
    launch_timed(k_gateup<BF16, MT, CPG, 1, BITS>, dim3(grid), dim3(64 * sh.waves), lds, s, tm, a.work, a.sorted, a.in,
                 a.insum, a.out, a.outpart, a.off_codes, a.off_hi, a.off_scales, a.chunks, a.groups, a.tiles, a.H,
                 a.I, a.k);
  else
    launch_timed(k_gateup<BF16, MT, CPG, 0, BITS>, dim3(grid), dim3(64 * sh.waves), 0, s, tm, a.work, a.sorted, a.in,
                 a.insum, a.out, a.outpart, a.off_codes, a.off_hi, a.off_scales, a.chunks, a.groups, a.tiles, a.H,
                 a.I, a.k);
}

template <int BF16, int MT, int CPG, int BITS>
static void down_launch3(const GemvArgs& a, const GemvShape& sh, int grid, const Timing& tm, hipStream_t s) {
  float* o = static_cast<float*>(a.out);
  const size_t lds = (size_t)MT * a.I * (BF16 ? 2 : 4);
  if (sh.lds)
    launch_timed(k_down<BF16, MT, CPG, 1, BITS>, dim3(grid), dim3(64 * sh.waves), lds, s, tm, a.work, a.in, a.insum,
                 o, a.off_codes, a.off_hi, a.off_scales, a.chunks, a.groups, a.tiles, a.H, a.I);
  else
    launch_timed(k_down<BF16, MT, CPG, 0, BITS>, dim3(grid), dim3(64 * sh.waves), 0, s, tm, a.work, a.in, a.insum, o,
                 a.off_codes, a.off_hi, a.off_scales, a.chunks, a.groups, a.tiles, a.H, a.I);
}

// Chunks of a quantisation group: G / 32 (4-bit codes: 1, 2, 4, 8) or G / 64 (2-, 3-bit: 1, 2, 4).
template <int BF16, int MT, int BITS, bool DOWN>
static void gemv_cpg(const GemvArgs& a, const GemvShape& sh, int grid, const Timing& tm, hipStream_t s) {
  auto go = [&](auto cpg_c) {
    constexpr int C = decltype(cpg_c)::value;
    if constexpr (DOWN)
      down_launch3<BF16, MT, C, BITS>(a, sh, grid, tm, s);
    else
      gateup_launch3<BF16, MT, C, BITS>(a, sh, grid, tm, s);
  };
  const int cpg = a.G / kChunkK<BITS>;
  if (cpg <= 1) return go(std::integral_constant<int, 1>{});
  if (cpg == 2) return go(std::integral_constant<int, 2>{});
  if constexpr (BITS == 4) {
    if (cpg == 4) return go(std::integral_constant<int, 4>{});
    // G = 256 with two tokens: the 4-token kernel (the 2-token one spills)
    if constexpr (MT == 2)
      return gemv_cpg<BF16, 4, BITS, DOWN>(a, sh, grid, tm, s);
    else
      return go(std::integral_constant<int, 8>{});
  } else {
    return go(std::integral_constant<int, 4>{});
  }
}

// Every (tokens per pass, chunks per group, staging) instance of one kernel family;
// instantiated once per (activation dtype, code width) in its own source file. The
// 8-token down GEMV of 3-bit codes spills, so 3-bit down passes take 4 tokens.
template <int BF16, int BITS, bool DOWN>
void run_gemv(const GemvArgs& a, const GemvShape& sh, int grid, const Timing& tm, hipStream_t s) {
  constexpr int MT8 = (BITS == 3 && DOWN) ? 4 : 8;
  switch (sh.mt) {
    case 1: return gemv_cpg<BF16, 1, BITS, DOWN>(a, sh, grid, tm, s);
    case 2:
      if constexpr (BF16 && DOWN && BITS == 4) return gemv_cpg<BF16, 2, BITS, DOWN>(a, sh, grid, tm, s);
      return gemv_cpg<BF16, 4, BITS, DOWN>(a, sh, grid, tm, s);
    case 4: return gemv_cpg<BF16, 4, BITS, DOWN>(a, sh, grid, tm, s);
    default: return gemv_cpg<BF16, MT8, BITS, DOWN>(a, sh, grid, tm, s);
  }
}

}  // namespace moe
