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
// Bits of the workspace's error word (offset 8), set by the prefill kernel and
// read back (and cleared) by m3_prefill_status.
constexpr unsigned kErrLookback = 1u;   // a look-back wait gave up (outputs of that chunk are NaN)
constexpr unsigned kErrControl = 2u;    // the control word was out of range (workspace not zero-filled)
constexpr unsigned kDefaultSpinLimit = 1u << 20;
struct PrefillPlan {
  int Q;              // tokens per chunk
  int nc;             // chunks per sequence
  size_t off_flags, off_recs, off_maps, off_states, bytes;
  size_t lds;         // dynamic LDS per workgroup
  int kernel;         // M3_KERNEL_PER_CHUNK or M3_KERNEL_STREAM
};

// Fills `plan` for a validated shape and entry point (gated readout,
// prologue); returns false if no chunk size fits.
bool plan_prefill(const m3_shape& s, PrefillPlan* plan, int gated, int pro);

struct FusedParams {
  const void* x; const void* B; const void* C;
  const float* dt; const float* A; const float* lam; const float* theta;
  const float* h0; const void* Bp; const void* xp;
  void* y; float* h_out;   // y is NULL when `out` is given
  void* out;               // gated readout out [b,L,H,P], or NULL
  const void* z; const float* wy; const float* wz;   // gate input and weights (each may be NULL)
  unsigned long long* ctl; unsigned long long* flags; float* recs; float* maps; float* states;
  unsigned long long* err;   // sticky error word (kErr* bits), read back by m3_prefill_status
  unsigned spin_limit;       // polls a look-back wait makes before it gives up
  int batch, L, H, N, P, R, logR, Q, nc;
  int use_maps;          // publish chunk maps when the predecessor's state is late
  int late_flag;         // streaming kernel: raise the state flag after the readout, not before
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
__host__ __device__ constexpr int fused_rows_cap(int N) { return N <= 32 ? 512 : N <= 128 ? 256 : 128; }
inline int fused_max_rows(int N) { return fused_rows_cap(N); }
// Output row tiles per wave -- the kernel variant's RT -- for a chunk of Q
// tokens x R ranks at state size N: the rows rounded up to 32, in 16-row tiles
// shared out over the waves, rounded up to 1, 2 or 4.
inline int fused_row_tiles(int Q, int R, int N) {
  const int rows = (Q * R + 31) / 32 * 32, waves = fused_threads(N) / 64;
  const int rt = (rows / 16 + waves - 1) / waves;
  return rt <= 1 ? 1 : rt <= 2 ? 2 : rt <= 4 ? 4 : 0;
}
// A prefill kernel variant: the template arguments the launch picks.
struct PrefillVariant { int dtype, N, P, R, RT, gated, pro; };
// Whether the build's compiler report gave this variant any scratch (private
// memory) per lane.  The library launches no such kernel: every GPU memory
// fault and the one wrong result met in this kernel's development came from
// variants that spilled to scratch, and their cause was not established.
bool prefill_variant_spills(const PrefillVariant& v);
constexpr int kFusedAngleCap = 8192;
size_t fused_lds_bytes(int Q, int R, int N, int P, int esize, int pro = 0);
hipError_t launch_fused_prefill(const FusedParams& p, size_t lds, int dtype, hipStream_t stream);
// The persistent streaming prefill (m3_stream.hip): the shapes it takes, its
// LDS per workgroup, and its launch (one workgroup per compute unit; same
// workspace layout and slot size as the per-chunk kernel, plus an exit
// counter in the workspace's third 8-byte word).
bool stream_supported(int dtype, int N, int P, int R, int Q, int gated, int pro);
size_t stream_lds_bytes(int Q, int R, int N, int P);
hipError_t launch_stream_prefill(const FusedParams& p, hipStream_t stream);

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

// Backward (m3_backward.hip): inputs of the forward call, the cotangents dy
// [b,L,H,R,P] (input dtype) and dh [b,H,N,P] (fp32 or NULL), the fp32
// gradients (dtheta / dh0 / dBp / dxp may be NULL: not computed; dA must be
// zero on entry: workgroups add into it), and the workspace: the per-segment
// hand-off of the segment-parallel passes.
struct BackwardParams {
  const void* x; const void* B; const void* C;
  const float* dt; const float* A; const float* lam; const float* theta;
  const float* h0; const void* Bp; const void* xp;
  const void* dy; const float* dh;
  float* dx; float* dB; float* dC; float* ddt; float* dA; float* dlam; float* dtheta;
  float* dh0; float* dBp; float* dxp;
  float* sega;                  // [b*H][nseg][N][P]: forward local end states, then backward local G
  float* segb;                  // [b*H][nseg][N][P]: the state entering each segment
  float* segc;                  // [b*H][nseg][N][P]: the G entering each segment from the right
  float* zf;                    // [b*H][nseg][N/2] (re, im): forward propagator of each segment
  float* zb;                    // [b*H][nseg][N/2] (re, im): backward propagator of each segment
  int batch, L, H;
  int S, nseg;                  // tokens per segment, segments per sequence
};
// LDS of the backward's segment kernel (floats, each array 16-byte aligned;
// N and P strides padded to 32, the rows to MK = a multiple of 32 >= S*R):
// B~, C~ [MK][N]; X, dY [MK][P]; S0', D' [N][P]; four [MK]^2 pairwise arrays;
// [S]^2; cos/sin [S][N/2] and [N/2]; per-token fields [S][16]; five [S][N/2]
// partial sums; per-row e^{l}; the previous write [R][N], [R][P]; reduction
// scratch.
struct BwdLds {
  size_t MK, B, C, X, Y, S, D, G1, G1T, G2T, PR, OM, CS, CN, TK, PA, PC, PB, PK, PI, EL, BM, XM, RD, total;
};
__host__ __device__ constexpr size_t bwd_r4(size_t n) { return (n + 3) & ~(size_t)3; }
__host__ __device__ constexpr BwdLds bwd_lds(int Q, int R, int N, int P) {
  const size_t NS = N < 32 ? 32 : N, PS = P < 32 ? 32 : P, NH = (size_t)N / 2;
  const size_t MK = ((size_t)Q * R + 31) / 32 * 32;
  BwdLds o{};
  size_t at = 0;
  o.MK = MK;
  o.B = at; at += bwd_r4(MK * NS);
  o.C = at; at += bwd_r4(MK * NS);
  o.X = at; at += bwd_r4(MK * PS);
  o.Y = at; at += bwd_r4(MK * PS);
  o.S = at; at += bwd_r4(NS * PS);
  o.D = at; at += bwd_r4(NS * PS);
  o.G1 = at; at += bwd_r4(MK * MK);
  o.G1T = at; at += bwd_r4(MK * MK);
  o.G2T = at; at += bwd_r4(MK * MK);
  o.PR = at; at += bwd_r4(MK * MK);
  o.OM = at; at += bwd_r4((size_t)Q * Q);
  o.CS = at; at += bwd_r4((size_t)Q * NH * 2);
  o.CN = at; at += bwd_r4(NH * 2);
  o.TK = at; at += bwd_r4((size_t)Q * 16);
  o.PA = at; at += bwd_r4((size_t)Q * NH);
  o.PC = at; at += bwd_r4((size_t)Q * NH);
  o.PB = at; at += bwd_r4((size_t)Q * NH);
  o.PK = at; at += bwd_r4((size_t)Q * NH);
  o.PI = at; at += bwd_r4((size_t)Q * NH);
  o.EL = at; at += bwd_r4(MK);
  o.BM = at; at += bwd_r4((size_t)R * N);
  o.XM = at; at += bwd_r4((size_t)R * P);
  o.RD = at; at += bwd_r4(336);
  o.total = at;
  return o;
}
// Tokens per backward segment: the largest of 32, 16, ..., 1 whose segment
// kernel fits a compute unit's LDS.
__host__ __device__ constexpr int backward_segment(int R, int N, int P) {
  for (int S = 32; S >= 1; S /= 2)
    if (bwd_lds(S, R, N, P).total * sizeof(float) <= (size_t)kLdsBudget) return S;
  return 0;
}
hipError_t launch_backward(const BackwardParams& p, int dtype, int N, int P, int R, hipStream_t stream);

// The device-resident prefill scratch of m3_scan_prefill_noalloc: its size
// (M3_NOALLOC_SCRATCH_BYTES in m3.h) and its device address on the current
// device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** out);

// Copies (or zero-fills when src is NULL) `n` floats on the stream with a kernel
// (no memset/memcpy nodes, so the call stays safe under graph capture).
hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream);

}  // namespace m3
