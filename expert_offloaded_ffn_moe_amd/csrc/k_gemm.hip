// Grouped int4 GEMM for prefill on bf16 MFMA (gfx950). Filled in by the prefill path.
#include <hip/hip_runtime.h>

#include "kernels.h"
