// Instances of the decode dequant-GEMV: gate/up + SwiGLU, fp32 activations, 4-bit codes.
#include "k_gemv.h"

namespace moe {
template void run_gemv<0, 4, false>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
}  // namespace moe
