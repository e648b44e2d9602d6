// Instances of the decode dequant-GEMV: down projection, bf16 activations, 2- and 3-bit codes.
#include "k_gemv.h"

namespace moe {
template void run_gemv<1, 2, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
template void run_gemv<1, 3, true>(const GemvArgs&, const GemvShape&, int, const Timing&, hipStream_t);
}  // namespace moe
