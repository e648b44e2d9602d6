// Decode down projection, bf16 activations, 4-bit codes: the instances of the grouped
// dequant-GEMV, and the down projection fused with the combine for small batches.
#include "k_gemv.h"

namespace moe {

template void run_gemv<1, 4, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);

// Down projection fused with the gate-weighted combine, for batches of a few
// tokens: a workgroup owns (64-row tile of H, token t) and its k * S waves the
// token's k slots, S waves per slot splitting K. Each wave streams its slot's
// expert tile once (the same 1 KiB blocks and group scales as k_down) against
// the slot's h row; the partial sums meet in LDS and one wave forms
//   y[t][r] = sum over j = 0..k-1, in order, of w_j * (sum over s of part[j][s][r]).
// No o round trip and no separate combine launch; the order of every sum is fixed.
// Load batches of four chunks instead of the GEMVs' eight (7168-wide layer, batch
// 4: 33.8 -> 33.0 us; the gate/up GEMV lost with four: 54.6 -> 55.3 us).
constexpr int kDownCombBatch = 4;
template <int CPG>
__global__ __launch_bounds__(1024) void k_down_comb(const uint8_t* const* __restrict__ aptr,
                                                    const int32_t* __restrict__ inv, const float* __restrict__ wts,
                                                    const void* __restrict__ h, const float* __restrict__ hpart,
                                                    float* __restrict__ y, const uint16_t* __restrict__ xres,
                                                    uint16_t* __restrict__ xout, int64_t off_codes, int64_t off_scales,
                                                    int chunks, int groups, int H, int I, int k, int splits) {
  __shared__ float part[kMaxW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x, t = blockIdx.y;
  const int j = wave / splits, sp = wave % splits;
  const int slot = t * k + j;
  const uint8_t* base = aptr[slot];
  int p = inv[slot];
  asm volatile("" : "+v"(p) : "v"(base));  // both loads in flight together
  p = __builtin_amdgcn_readfirstlane(p);    // and the row stays wave-uniform (scalar loads of h)
  guint4* codes = (guint4*)(base + off_codes) + (size_t)tile * chunks * 64 + lane;
  gushort* scales = (gushort*)(base + off_scales) + (size_t)tile * groups * 64 + lane;
  int64_t rows[1] = {(int64_t)p * I}, sum_rows[1] = {(int64_t)p * (I / 32)};
  float acc[1] = {0.f};
  k_loop<1, 1, CPG, true, 0, 4, kDownCombBatch>(codes, nullptr, scales, h, hpart, rows, sum_rows, 1, sp, splits, groups,
                                                acc);
  part[wave][lane] = acc[0];
  __syncthreads();
  if (wave == 0) {
    float yv = 0.f;
    for (int jj = 0; jj < k; ++jj) {
      float o = 0.f;
      for (int s2 = 0; s2 < splits; ++s2) o += part[jj * splits + s2][lane];
      yv = fmaf(wts[t * k + jj], o, yv);
    }
    const size_t i = (size_t)t * H + tile * 64 + lane;
    y[i] = yv;
    if (xout) xout[i] = residual_bf16(xres[i], yv);
  }
}

// The same fusion on 16-row tiles of H, for batches too small to give the
// 64-row form enough workgroups (a batch-1 layer with H = 2048 has only 32 of
// those). A workgroup owns (16-row tile of H, token t); lane l of a wave takes
// row l % 16 of the tile and every fourth K chunk starting at l / 16, so each
// code load reads a quarter (256 contiguous bytes) of four of the 1 KiB blocks
// that the wide form reads whole. A lane's h chunk is not wave-uniform: with
// long rows (STAGE, I > 1024) the token's k rows of h and their chunk sums are
// staged once per workgroup in LDS (their global loads issued together with the
// first code loads); shorter rows are read straight from global memory, where
// they stay in cache (measured: I = 768, batch 1: 8.4 -> 7.5 us without the
// staging; I = 2048: 16.9 -> 15.3 us with it; reading the k sorted positions once
// and issuing the chunk-sum loads with the h loads: 15.6 -> 14.5 us on the
// 7168-wide layer, batch 1). Each lane keeps IT chunk loads in flight besides the
// IT it computes on: IT = 2, or 1 where a lane has at most four chunk iterations.
// More measured slower (7168-wide layer, batch 1, 8 iterations: 14.5 us at four,
// 13.2 us at two, 17.3 us with all eight issued before the staging; 2048-wide,
// batch 4, 6 iterations: 10.6 us at four, 9.1 at two, 9.5 at one; batch 1, 3
// iterations: 7.2 us at two, 6.6 at one). Per chunk:
//   part += 16 s (sum v h - 1.5 sum h),  v = 1 + n/16,
// then the four chunk lanes of a row are added (lanes r, r+16, r+32, r+48, in
// a fixed tree), the S waves of a slot and the k slots meet in LDS, and
//   y[t][r] = sum over j = 0..k-1, in order, of w_j * (sum over s of part[j][s][r]).
constexpr int kNarrowStage = 2;  // h units (16 bytes) per thread and pass staged from registers

// IT: chunks per lane whose code loads are issued together
template <int CPG, int IT>
struct NarrowBatch {
  u32x4 wv[IT];
  uint16_t sc[IT];
  __device__ __forceinline__ void load(guint4* codes, gushort* scales, int cfirst, int c1) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = min(cfirst + 4 * i, c1 - 1);
      wv[i] = codes[(size_t)c * 64];
      sc[i] = scales[(size_t)(c / CPG) * 64];
    }
  }
};

// Workgroups are dealt to the 8 XCDs round-robin by block id, and each XCD has its
// own L2. The four 16-row tiles of a 64-row block share its 128-byte group-scale
// lines, so they are given to four blocks of one XCD (ids b, b + 8, b + 16, b + 24)
// rather than to four neighbouring ids on four XCDs, each of which would fetch
// every shared line from memory. Needs a multiple of 32 tiles, else identity.
__device__ __forceinline__ int comb16_tile(int b, int n) {
  if (n & 31) return b;
  const int x = b & 7, i = b >> 3;
  return (((i >> 2) << 3) + x) * 4 + (i & 3);
}

template <int CPG, bool STAGE, int IT>
__global__ __launch_bounds__(1024) void k_down_comb16(const uint8_t* const* __restrict__ aptr,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ wts, const void* __restrict__ h,
                                                      const float* __restrict__ hpart, float* __restrict__ y,
                                                      const uint16_t* __restrict__ xres, uint16_t* __restrict__ xout,
                                                      int64_t off_codes, int64_t off_scales, int chunks, int groups,
                                                      int H, int I, int k, int splits) {
  __shared__ float part[kMaxW][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, cl = lane >> 4;
  const int tile = comb16_tile(blockIdx.x, gridDim.x), t = blockIdx.y;
  const int j = wave / splits, sp = wave % splits;
  const uint8_t* base = aptr[t * k + j];
  const int lane_off = (tile & 3) * 16 + r;  // place of row r in its 64-row block
  guint4* codes = (guint4*)(base + off_codes) + (size_t)(tile >> 2) * chunks * 64 + lane_off;
  gushort* scales = (gushort*)(base + off_scales) + (size_t)(tile >> 2) * groups * 64 + lane_off;
  const int c0 = (chunks * sp) / splits, c1 = (chunks * (sp + 1)) / splits;
  const int n_it = (c1 - c0 + 3) >> 2;  // chunk iterations of the wave (lanes past c1 count 0)

  // the first load batch goes out before the h staging, each next one while the
  // previous one computes
  NarrowBatch<CPG, IT> cur;
  if (n_it > 0) cur.load(codes, scales, c0 + cl, c1);

  const uint4* hrow;
  const float* hs_row;
  if (STAGE) {
    // stage h rows [k][I] (bf16, 16-byte units) and chunk sums [k][I/32] of token t:
    // the k sorted positions are read once (one lane each) and shared by shuffles,
    // then the h and chunk-sum loads of the first pass go out together
    const int units = I / 8, n_units = k * units, nsum = I / 32, n_sums = k * nsum;
    uint4* hl = moe_dyn_lds;
    float* hsl = reinterpret_cast<float*>(moe_dyn_lds + n_units);
    const uint4* h4 = static_cast<const uint4*>(h);
    const int nthr = blockDim.x;
    const int pos = inv[t * k + min(lane, k - 1)];
    const int si = min((int)threadIdx.x, n_sums - 1);
    const float hs0 = hpart[(size_t)__shfl(pos, si / nsum, 64) * nsum + si % nsum];
    for (int u0 = 0; u0 < n_units; u0 += kNarrowStage * nthr) {
      uint4 hv[kNarrowStage];
#pragma unroll
      for (int i = 0; i < kNarrowStage; ++i) {
        const int u = min(u0 + (int)threadIdx.x + i * nthr, n_units - 1);
        hv[i] = h4[(size_t)__shfl(pos, u / units, 64) * units + u % units];
      }
#pragma unroll
      for (int i = 0; i < kNarrowStage; ++i) {
        const int u = u0 + (int)threadIdx.x + i * nthr;
        if (u < n_units) hl[u] = hv[i];
      }
    }
    if ((int)threadIdx.x < n_sums) hsl[threadIdx.x] = hs0;
    for (int i = threadIdx.x + nthr; i < n_sums; i += nthr)
      hsl[i] = hpart[(size_t)__shfl(pos, i / nsum, 64) * nsum + i % nsum];
    __syncthreads();
    hrow = hl + j * units;
    hs_row = hsl + j * nsum;
  } else {
    const int p = __builtin_amdgcn_readfirstlane(inv[t * k + j]);
    hrow = static_cast<const uint4*>(h) + (size_t)p * (I / 8);
    hs_row = hpart + (size_t)p * (I / 32);
  }
  float acc = 0.f;
  const PairConsts pk;
  // chunk iterations ib .. ib + IT - 1 of batch bt
  auto math = [&](const NarrowBatch<CPG, IT>& bt, int ib) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int c = c0 + cl + 4 * (ib + i);
      const int cc = min(c, c1 - 1);
      uint32_t xw[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = hrow[cc * 4 + q];
        xw[4 * q] = v.x;
        xw[4 * q + 1] = v.y;
        xw[4 * q + 2] = v.z;
        xw[4 * q + 3] = v.w;
      }
      const float d = chunk_dot_bf16(bt.wv[i], xw, 0.f, pk);
      const float sc = (c < c1) ? 16.f * half_bits(bt.sc[i]) : 0.f;
      acc = fmaf(sc, d - 1.5f * hs_row[cc], acc);
    }
  };
  for (int ib = 0; ib < n_it; ib += IT) {
    NarrowBatch<CPG, IT> nxt;
    if (ib + IT < n_it) nxt.load(codes, scales, c0 + cl + 4 * (ib + IT), c1);
    math(cur, ib);
    cur = nxt;
  }
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane < 16) part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float yv = 0.f;
    for (int jj = 0; jj < k; ++jj) {
      float o = 0.f;
      for (int s2 = 0; s2 < splits; ++s2) o += part[jj * splits + s2][lane];
      yv = fmaf(wts[t * k + jj], o, yv);
    }
    const size_t i = (size_t)t * H + tile * 16 + lane;
    y[i] = yv;
    if (xout) xout[i] = residual_bf16(xres[i], yv);
  }
}

size_t down_combine16_lds(int k, int I) { return (size_t)k * I * 2 + (size_t)k * (I / 32) * 4; }

void launch_down_combine16(const DownCombArgs& a, const Timing& tm, hipStream_t s) {
  const dim3 grid(a.H / 16, a.T), block(64 * a.k * a.splits);
  const bool stage = a.I > 1024;
  const size_t lds = stage ? down_combine16_lds(a.k, a.I) : 0;
  // one chunk load per lane in flight when a lane has at most four chunk iterations,
  // else two
  const int per_wave = (a.chunks + a.splits - 1) / a.splits;
  const bool one = (per_wave + 3) / 4 <= 4;
#define DOWN_COMB16_K(C, ST, IT)                                                                                  \
  launch_timed(k_down_comb16<C, ST, IT>, grid, block, lds, s, tm, a.aptr, a.inv, a.wts, a.h, a.hpart, a.y, a.xres, \
               a.xout, a.off_codes, a.off_scales, a.chunks, a.groups, a.H, a.I, a.k, a.splits)
#define DOWN_COMB16(C)                                         \
  if (stage)                                                   \
    one ? DOWN_COMB16_K(C, true, 1) : DOWN_COMB16_K(C, true, 2);  \
  else                                                         \
    one ? DOWN_COMB16_K(C, false, 1) : DOWN_COMB16_K(C, false, 2);
  switch (a.G / 32) {
    case 1: DOWN_COMB16(1); break;
    case 2: DOWN_COMB16(2); break;
    case 4: DOWN_COMB16(4); break;
    default: DOWN_COMB16(8); break;
  }
#undef DOWN_COMB16
#undef DOWN_COMB16_K
}

void launch_down_combine(const DownCombArgs& a, const Timing& tm, hipStream_t s) {
  const dim3 grid(a.H / 64, a.T), block(64 * a.k * a.splits);
#define DOWN_COMB(C)                                                                                           \
  launch_timed(k_down_comb<C>, grid, block, 0, s, tm, a.aptr, a.inv, a.wts, a.h, a.hpart, a.y, a.xres, a.xout, a.off_codes, \
               a.off_scales, a.chunks, a.groups, a.H, a.I, a.k, a.splits)
  switch (a.G / 32) {
    case 1: DOWN_COMB(1); break;
    case 2: DOWN_COMB(2); break;
    case 4: DOWN_COMB(4); break;
    default: DOWN_COMB(8); break;
  }
#undef DOWN_COMB
}

}  // namespace moe
