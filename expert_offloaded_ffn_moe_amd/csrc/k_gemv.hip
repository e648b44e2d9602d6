// Launch policy of the decode dequant-GEMVs (kernels in k_gemv.h; their instances
// are compiled in k_gemv_{gateup,down}_{bf16,f32}.hip and k_gemv_lowbit_*.hip). Every
// rule that shapes a GEMV launch lives here: tokens per pass, waves per workgroup,
// and whether the activation rows are staged in LDS.
#include "k_gemv.h"

namespace moe {

template <int BF16, int BITS, bool DOWN>
void run_gemv(const GemvArgs& a, const GemvShape& sh, int grid, const Timing& tm, hipStream_t s);
extern template void run_gemv<1, 4, false>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<0, 4, false>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<1, 4, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<0, 4, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<1, 2, false>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<1, 3, false>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<1, 2, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
extern template void run_gemv<1, 3, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);

// Tokens per pass for the largest number of tokens an expert holds. Experts of a two-
// to four-token batch take the 4-token kernels: a 2-token gate/up variant needed 202
// VGPRs against 96 and ran slower (2048-wide layer, batch 2: 12.3 -> 11.0 us), and the
// 2-token fp32 variants spill. Only the bf16 down GEMV of 4-bit codes keeps a 2-token
// kernel, except for G = 256, where it spills too.
static int pick_mt(int max_tok, bool bf16, bool down, int bits, int G) {
  if (max_tok <= 1) return 1;
  if (max_tok <= 2 && bf16 && down && bits == 4 && G != 256) return 2;
  if (down && bits == 3) return 4;  // the 8-token 3-bit down GEMV spills
  return max_tok <= 4 ? 4 : 8;
}

// Waves per workgroup: about kBatch lane words of K per wave. Gate/up with bf16
// activations stops at 8 waves: at 16 (1024 threads) only one workgroup fits a CU, and
// a 384-workgroup batch-1 launch of a 7168-wide layer then runs in two rounds (26.6 us
// against 23.2 us at 8 waves, where two fit and all are resident at once). The other
// families run up to the launch bound of their variant (1024 threads for one token,
// 512 for several).
static int pick_waves(const GemvArgs& a, int mt, bool bf16, bool down, int bits) {
  const int words = a.groups * (a.G / (bits == 4 ? 32 : 64));
  const int wmax = (bf16 && !down) ? 8 : (mt > 1 ? 8 : 16);
  return std::max(1, std::min(std::min(wmax, a.groups), (words + kBatch - 1) / kBatch));
}

// Activations from an LDS copy when an expert carries several tokens (or, except for
// bf16 gate/up, when K >= 4096, measured faster there) and the rows fit in 64 KiB;
// else through scalar loads (one token on 7168-wide rows: 23.9 us through LDS,
// 23.1 us with scalar loads, which need no barrier before the weights).
static bool pick_lds(int mt, int K, bool bf16, bool down) {
  const size_t bytes = (size_t)mt * K * (bf16 ? 2 : 4);
  const bool long_rows = !(bf16 && !down) && K >= 4096;
  return bytes <= 65536 && (mt >= 2 || long_rows);
}

static GemvShape shape_of(const GemvArgs& a, int bf16, int max_tok, bool down, int bits) {
  GemvShape sh;
  sh.mt = pick_mt(max_tok, bf16, down, bits, a.G);
  sh.waves = pick_waves(a, sh.mt, bf16, down, bits);
  sh.lds = pick_lds(sh.mt, down ? a.I : a.H, bf16, down);
  return sh;
}

void launch_gateup(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  const GemvShape sh = shape_of(a, act_bf16, max_tok, false, a.bits);
  if (!act_bf16) return run_gemv<0, 4, false>(a, sh, grid, tm, s);  // fp32 activations: 4-bit codes only
  switch (a.bits) {
    case 2: return run_gemv<1, 2, false>(a, sh, grid, tm, s);
    case 3: return run_gemv<1, 3, false>(a, sh, grid, tm, s);
    default: return run_gemv<1, 4, false>(a, sh, grid, tm, s);
  }
}

void launch_down(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  const GemvShape sh = shape_of(a, act_bf16, max_tok, true, a.bits);
  if (!act_bf16) return run_gemv<0, 4, true>(a, sh, grid, tm, s);
  switch (a.bits) {
    case 2: return run_gemv<1, 2, true>(a, sh, grid, tm, s);
    case 3: return run_gemv<1, 3, true>(a, sh, grid, tm, s);
    default: return run_gemv<1, 4, true>(a, sh, grid, tm, s);
  }
}

}  // namespace moe
