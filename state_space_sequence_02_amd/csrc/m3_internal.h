// m3_internal.h -- internal declarations of the gfx950 Mamba-3 recurrence library.
// Not installed; the public surface is include/m3.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/m3.h"

namespace m3 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Supported geometry.  Everything the kernels index is a power of two.
constexpr int kMaxRank = 8;
constexpr int kLdsBudget = 160 * 1024;   // LDS per compute unit on gfx950

inline bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int v) { int r = 0; while ((1 << r) < v) ++r; return r; }

inline bool supported_state(int N) { return N == 16 || N == 32 || N == 64 || N == 128 || N == 256; }
inline bool supported_head(int P) { return P == 16 || P == 32 || P == 64 || P == 128; }
inline bool supported_rank(int R) { return R == 1 || R == 2 || R == 4 || R == 8; }

// ---------------------------------------------------------------------------
// Prefill: one launch per call, one workgroup per (sequence, chunk); chunk
// states are handed from chunk to chunk with decoupled look-back.
// Workspace (each region 256-byte aligned): control word | flags [b*H*nc] u64 |
// recs [b*H*nc][N+2] fp32 (a_c, pad, cos/sin Psi_c per pair) |
// maps [b*H*nc][fused_slot_floats] fp32 | states [b*H*nc][same] fp32.
// The control word holds the call's ticket count (low kTicketBits bits) and an
// epoch (the rest).  The workgroup that takes a call's last ticket sets the
// count back to 0 and advances the epoch, and every flag carries the epoch of
// the call that wrote it ((epoch + 1) << 2 | state), so a zero-filled
// workspace stays ready for the next call with no reset between calls: flags
// left by earlier calls never match.
constexpr int kTicketBits = 26;
constexpr unsigned long long kTicketMask = (1ull << kTicketBits) - 1;
constexpr size_t kMaxChunks = (size_t)kTicketMask;   // chunks per call, at most
struct PrefillPlan {
  int Q;              // tokens per chunk
  int nc;             // chunks per sequence
  size_t off_flags, off_recs, off_maps, off_states, bytes;
  size_t lds;         // dynamic LDS per workgroup
};

// Fills `plan` for a validated shape; returns false if no chunk size fits.
bool plan_prefill(const m3_shape& s, PrefillPlan* plan);

struct FusedParams {
  const void* x; const void* B; const void* C;
  const float* dt; const float* A; const float* lam; const float* theta;
  const float* h0; const void* Bp; const void* xp;
  void* y; float* h_out;   // y is NULL when `out` is given
  void* out;               // gated readout out [b,L,H,P], or NULL
  const void* z; const float* wy; const float* wz;   // gate input and weights (each may be NULL)
  unsigned long long* ctl; unsigned long long* flags; float* recs; float* maps; float* states;
  int batch, L, H, N, P, R, logR, Q, nc;
  int use_maps;          // publish chunk maps when the predecessor's state is late
  int pro; float eps;    // prologue: B/C/B_prev column RMS norm (+ eps), angle = dt x theta
  const float* biasB; const float* biasC;             // prologue biases [H][R][N] (each may be NULL)
};
// Threads per prefill workgroup: 1024 for N >= 128 (one workgroup fills a CU
// there, and twice the waves share each chunk's work), 512 below.
__host__ __device__ constexpr int fused_threads(int N) { return N >= 128 ? 1024 : 512; }
// Floats one chunk's map or state occupies in the workspace: each thread
// stores its state tiles (n-tile x p-tile of 16 x 16 shared out over the
// waves as NPW x PTW tiles per wave, 4 floats per lane) contiguously.
__host__ __device__ constexpr int fused_slot_floats(int N, int P) {
  return ((N / 16) / ((N / 16) < fused_threads(N) / 64 ? (N / 16) : fused_threads(N) / 64)) *
         (((P / 16) + (fused_threads(N) / 64) / ((N / 16) < fused_threads(N) / 64 ? (N / 16) : fused_threads(N) / 64) - 1) /
          ((fused_threads(N) / 64) / ((N / 16) < fused_threads(N) / 64 ? (N / 16) : fused_threads(N) / 64))) *
         fused_threads(N) * 4;
}
// Chunk limits of the single-pass prefill: (token, rank) rows per chunk and
// angles (tokens x N/2) per chunk; they bound the per-thread prefetch registers.
inline int fused_max_rows(int N) { return N <= 32 ? 512 : N <= 128 ? 256 : 128; }
constexpr int kFusedAngleCap = 8192;
size_t fused_lds_bytes(int Q, int R, int N, int P, int esize, int pro = 0);
hipError_t launch_fused_prefill(const FusedParams& p, size_t lds, int dtype, hipStream_t stream);

// ---------------------------------------------------------------------------
// Decode: one workgroup per (sequence, head).
struct DecodeParams {
  void* h;               // fp32 or (state_bf16) bf16 state
  int state_bf16;
  const void* Bp; const void* xp;
  const void* x; const void* B; const void* C;
  const float* dt; const float* A; const float* lam; const float* theta;
  void* y;               // y [b,H,R,P], or NULL when `out` is given
  void* out;             // gated readout out [b,H,P], or NULL
  const void* z; const float* wy; const float* wz;   // gate input and weights (each may be NULL)
  int pro; float eps;    // prologue: B/C/B_prev column RMS norm (+ eps), angle = dt x theta
  const float* biasB; const float* biasC;             // prologue biases [H][R][N] (each may be NULL)
  int batch, H, N, P, R;
};

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream);

// Copies (or zero-fills when src is NULL) `n` floats on the stream with a kernel
// (no memset/memcpy nodes, so the call stays safe under graph capture).
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream);

}  // namespace m3
