// m3_fused.hip -- host-side dispatch of the single-pass prefill (kernels in
// m3_fused_kernel.h, instantiated per (dtype, state size) in m3_fused_*_n*.hip;
// N = 16..128: a 256-state chunk does not fit the register budget without
// spilling, and the prefill rejects that size).
#include "m3_fused_kernel.h"

namespace m3 {

hipError_t launch_fused_bf16_16(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_bf16_32(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_bf16_64(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_bf16_128(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_f32_16(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_f32_32(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_f32_64(const FusedParams&, size_t, hipStream_t);
hipError_t launch_fused_f32_128(const FusedParams&, size_t, hipStream_t);

size_t fused_lds_bytes(int Q, int R, int N, int P, int esize, int pro) {
  return fused::lds_layout(Q, R, N, P, esize, pro).total;
}

hipError_t launch_fused_prefill(const FusedParams& p, size_t lds, int dtype, hipStream_t s) {
  const bool bf = dtype == M3_BF16;
  switch (p.N) {
    case 16: return bf ? launch_fused_bf16_16(p, lds, s) : launch_fused_f32_16(p, lds, s);
    case 32: return bf ? launch_fused_bf16_32(p, lds, s) : launch_fused_f32_32(p, lds, s);
    case 64: return bf ? launch_fused_bf16_64(p, lds, s) : launch_fused_f32_64(p, lds, s);
    case 128: return bf ? launch_fused_bf16_128(p, lds, s) : launch_fused_f32_128(p, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m3
