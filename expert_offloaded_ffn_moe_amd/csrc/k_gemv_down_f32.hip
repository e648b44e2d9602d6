// Instantiations of the decode dequant-GEMV kernels: down projection (+ fused combine), f32 activations.
#include "k_gemv.h"

namespace moe {

// waves per workgroup: about kBatch chunks of K per wave, at most kMaxW waves
static int waves_for(const GemvArgs& a, int mt) {
  const int chunks = a.groups * (a.G / 32);
  const int wmax = kMaxThreads<1> / 64 >> (mt > 1 ? 1 : 0);  // within the variant's launch bound
  return std::max(1, std::min(std::min(wmax, a.groups), (chunks + kBatch - 1) / kBatch));
}

// Activations from an LDS copy when an expert carries several tokens or K is
// long (measured faster there), and the rows fit in 64 KiB; else scalar loads.
static bool use_lds(size_t bytes, int mt, int K) { return bytes <= 65536 && (mt >= 2 || K >= 4096); }

// No two-token variant for fp32 rows: it needs more than 256 VGPRs and spills, so
// experts with 2 tokens take the 4-token kernel (rows past the count are skipped).
static int pick_mt(int max_tok) { return max_tok <= 1 ? 1 : max_tok <= 4 ? 4 : 8; }

template <int MT, int CPG>
static void down_w(const GemvArgs& a, int W, int grid, const Timing& tm, hipStream_t s) {
  float* o = static_cast<float*>(a.out);
  const size_t lds = (size_t)MT * a.I * 4;
  if (use_lds(lds, MT, a.I))
    launch_timed(k_down<0, MT, CPG, 1>, dim3(grid), dim3(64 * W), lds, s, tm, a.work,
                 a.in, a.insum, o, a.off_codes, a.off_scales, a.chunks, a.groups, a.tiles, a.H, a.I);
  else
    launch_timed(k_down<0, MT, CPG, 0>, dim3(grid), dim3(64 * W), 0, s, tm, a.work,
                 a.in, a.insum, o, a.off_codes, a.off_scales, a.chunks, a.groups, a.tiles, a.H, a.I);
}

template <int MT>
static void down_cpg(const GemvArgs& a, int W, int grid, const Timing& tm, hipStream_t s) {
  switch (a.G / 32) {
    case 1: return down_w<MT, 1>(a, W, grid, tm, s);
    case 2: return down_w<MT, 2>(a, W, grid, tm, s);
    case 4: return down_w<MT, 4>(a, W, grid, tm, s);
    default: return down_w<MT, 8>(a, W, grid, tm, s);
  }
}

static void down_mt(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  const int W = waves_for(a, pick_mt(max_tok));
  switch (pick_mt(max_tok)) {
    case 1: return down_cpg<1>(a, W, grid, tm, s);
    case 4: return down_cpg<4>(a, W, grid, tm, s);
    default: return down_cpg<8>(a, W, grid, tm, s);
  }
}

void launch_down_f32(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  down_mt(a, max_tok, grid, tm, s);
}

}  // namespace moe
