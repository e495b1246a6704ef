// m3_prologue.h -- the prologue as a stage of its own (m3_prologue.hip), for
// the prologue prefill's staged form.
#pragma once

#include "m3_internal.h"

namespace m3 {

// The prologue as a stage of its own (m3_prologue.hip): B, C and B_prev
// normalized with their biases added, and the angles dt x theta, written to
// Bn, Cn, Bpn and phi (the inputs' layouts and dtype; phi fp32).  tokens =
// b x L x H, pairs = b x H.
struct PrologueStage {
  int dtype, N, H, R;
  size_t tokens, pairs;
  float eps;
  const void* B; const void* C; const void* Bp;
  const float* dt; const float* theta;
  const float* biasB; const float* biasC;
  void* Bn; void* Cn; void* Bpn; float* phi;
};
hipError_t launch_prologue_stage(const PrologueStage& p, hipStream_t stream);

// Dynamic LDS of the streaming prefill with the prologue fused (its bias
// tables beside the chunk's tiles; m3_stream.hip).
size_t stream_lds_bytes_pro(int Q, int R, int N, int P);

}  // namespace m3
