// Dispatch of the decode dequant-GEMV kernels by activation dtype; the kernels
// are in k_gemv.h, instantiated in k_gemv_{gateup,down}_{bf16,f32}.hip.
#include "kernels.h"

namespace moe {

void launch_gateup_bf16(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s);
void launch_gateup_f32(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s);
void launch_down_bf16(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s);
void launch_down_f32(const GemvArgs& a, int max_tok, int grid, const Timing& tm, hipStream_t s);

void launch_gateup(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  if (act_bf16)
    launch_gateup_bf16(a, max_tok, grid, tm, s);
  else
    launch_gateup_f32(a, max_tok, grid, tm, s);
}

void launch_down(const GemvArgs& a, int act_bf16, int max_tok, int grid, const Timing& tm, hipStream_t s) {
  if (act_bf16)
    launch_down_bf16(a, max_tok, grid, tm, s);
  else
    launch_down_f32(a, max_tok, grid, tm, s);
}

}  // namespace moe
