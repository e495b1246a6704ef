// Instantiates the single-pass prefill kernels for one (dtype, state size).
#include "m3_fused_kernel.h"
M3_FUSED_INSTANTIATE(m3::bf16, bf16, 128)
