// Instantiations of the decode dequant-GEMV kernels: gate/up + SwiGLU, bf16 activations.
#include "k_gemv.h"

namespace moe {

// waves per workgroup: about kBatch chunks of K per wave, at most 8 waves. With
// 16 waves (1024 threads) only one workgroup fits a CU, and a 384-workgroup
// batch-1 launch of a 7168-wide layer then runs in two rounds: 26.6 us against
// 23.2 us at 8 waves, where two fit and all are resident at once.
static int waves_for(const GemvArgs& a, int mt) {
  (void)mt;
  const int chunks = a.groups * (a.G / 32);
  const int wmax = 8;
  return std::max(1, std::min(std::min(wmax, a.groups), (chunks + kBatch - 1) / kBatch));
}

// Activations from an LDS copy when an expert carries several tokens and the
// rows fit in 64 KiB; else scalar loads. (One token on 7168-wide rows: 23.9 us
// through LDS, 23.1 us with scalar loads, which need no barrier before the weights.)
static bool use_lds(size_t bytes, int mt) { return bytes <= 65536 && mt >= 2; }

// Experts of a two- to four-token batch take the 4-token kernel: the 2-token
// variant needs 202 VGPRs against 96 and ran slower (2048-wide layer, batch 2:
// gate/up 12.3 -> 11.0 us; 7168-wide: 38.0 -> 37.7 us).
static int pick_mt(int max_tok) { return max_tok <= 1 ? 1 : max_tok <= 4 ? 4 : 8; }

template <int MT, int CPG>
static void gateup_w(const GemvArgs& a, int W, int grid, const Timing& tm, hipStream_t s) {
  const size_t lds = (size_t)MT * a.H * 2;
  if (use_lds(lds, MT))
    launch_timed(k_gateup<1, MT, CPG, 1>, dim3(grid), dim3(64 * W), lds, s, tm, a.work,
                 a.sorted, a.in, a.insum, a.out, a.outpart, a.off_codes, a.off_scales, a.chunks,
                 a.groups, a.tiles, a.H, a.I, a.k);
  else
    launch_timed(k_gateup<1, MT, CPG, 0>, dim3(grid), dim3(64 * W), 0, s, tm, a.work,
                 a.sorted, a.in, a.insum, a.out, a.outpart, a.off_codes, a.off_scales, a.chunks,
                 a.groups, a.tiles, a.H, a.I, a.k);
}

template <int MT>
static void gateup_cpg(const GemvArgs& a, int W, int grid, const Timing& tm, hipStream_t s) {
  switch (a.G / 32) {
    case 1: return gateup_w<MT, 1>(a, W, grid, tm, s);
    case 2: return gateup_w<MT, 2>(a, W, grid, tm, s);
    case 4: return gateup_w<MT, 4>(a, W, grid, tm, s);
    default: return gateup_w<MT, 8>(a, W, grid, tm, s);
  }
}

void launch_gateup_bf16(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  const int W = waves_for(a, pick_mt(max_tok));
  switch (pick_mt(max_tok)) {
    case 1: return gateup_cpg<1>(a, W, grid, tm, s);
    case 4: return gateup_cpg<4>(a, W, grid, tm, s);
    default: return gateup_cpg<8>(a, W, grid, tm, s);
  }
}

}  // namespace moe
