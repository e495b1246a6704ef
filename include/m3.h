/*
 * m3.h -- C ABI of the MI355X (gfx950) Mamba-3 SSM recurrence library (libm3.so).
 *
 * The library computes the per-head Mamba-3 state-space recurrence described on
 * the Mamba-3 pages ("Mamba-3: Improved Sequence Modeling using State Space
 * Principles", explainer page sections 3.1-3.3 and panels 1-4; paper page
 * Table 1 caption):
 *
 *   alpha_t = exp(dt_t A), beta_t = (1 - lam_t) dt_t alpha_t, gamma_t = lam_t dt_t
 *   H_t = alpha_t R(phi_t) H_{t-1} + beta_t R(phi_t) B_{t-1} X_{t-1}^T + gamma_t B_t X_t^T
 *   Y_t = H_t^T C_t
 *
 * per (batch, head), with H an N x P fp32 state whose adjacent row pairs
 * (2k, 2k+1) rotate by the per-step angle phi_t[k] (the real form of the complex
 * state, Prop. 2), B_t, C_t N x R and X_t P x R (rank-R MIMO, Eqs. 12-14).
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers into memory the caller owns; the
 *    library allocates nothing and keeps no data between calls (it caches only
 *    per-device launch properties).  The prefill's workspace carries a call
 *    epoch from one call to the next (see m3_prefill_workspace_bytes).
 *  - Tensors are dense and row-major in the layouts given below.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the
 *    call returns without waiting.  Shape, pointer and dtype checks run on the
 *    host before anything is enqueued; on failure nothing is launched and a
 *    nonzero status is returned.  A launch failure returns M3_ERR_DEVICE.  No C++
 *    exception crosses this boundary.
 *  - Value preconditions are NOT checked on the device (as the pages' helper
 *    states them: finite values, dt >= 0, A <= 0, lam in [0, 1]); violating them
 *    gives unspecified (but memory-safe) results.
 *  - The state is exported in the physical frame, so no absolute phase crosses
 *    the boundary between calls.
 *  - Calls on different streams touching disjoint buffers may run concurrently.
 */
#ifndef M3_H
#define M3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_OK = 0,
    M3_ERR_NULL = 1,        /* a required pointer is NULL */
    M3_ERR_SHAPE = 2,       /* a size is negative, inconsistent or not supported */
    M3_ERR_DTYPE = 3,       /* unknown dtype code */
    M3_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than m3_prefill_workspace_bytes */
    M3_ERR_DEVICE = 5,      /* a HIP call or kernel launch failed */
    M3_ERR_ALIAS = 6        /* an output aliases an input it must not alias */
} m3_status;

/* Element type of x, B, C, B_prev, x_prev and y.  dt, A, lam, theta and the state
 * are always fp32. */
typedef enum { M3_FP32 = 0, M3_BF16 = 1 } m3_dtype;

/* Problem geometry.
 *   batch   b  >= 0   independent sequences
 *   seqlen  L  >= 0   tokens per sequence (ignored by m3_decode_step)
 *   nheads  H  >= 0   heads; A and all per-token tensors carry a head axis
 *   headdim P         columns of the state, rows of X_t: one of 16, 32, 64, 128
 *   dstate  N         rows of the state, rows of B_t / C_t: one of 16, 32, 64, 128, 256
 *                     (always even: it holds N/2 rotation pairs)
 *   rank    R         MIMO rank: 1, 2, 4 or 8
 *   chunk             prefill tokens per chunk; 0 picks the library default.  The
 *                     result does not depend on it (the chunked form is an exact
 *                     rearrangement); m3_prefill_chunk_used reports the value used.
 *   dtype             an m3_dtype code */
typedef struct {
    int32_t batch, seqlen, nheads, headdim, dstate, rank, chunk;
    int32_t dtype;
} m3_shape;

/* Bytes of device workspace m3_scan_prefill needs for this shape (0 on an
 * invalid or unsupported shape, including one of more than 2^26 - 1 chunks).
 * The buffer holds a control word (ticket count and call epoch), per-chunk
 * flags and per-chunk states.  Zero-fill it once before its first use (e.g.
 * hipMemset); every call leaves it ready for the next one, whatever shape that
 * has, so it may be reused across calls on the same stream with nothing done in
 * between.  Calls that may run at the same time (other streams) need workspaces
 * of their own.  A workspace that was not zero-filled before its first use
 * gives wrong results (never an access outside the buffers) until it is. */
size_t m3_prefill_workspace_bytes(const m3_shape* s);

/* Tokens per chunk m3_scan_prefill will actually use for this shape (the
 * requested value rounded to a supported power of two and capped so that one
 * chunk's tiles fit on a compute unit), or 0 on an invalid shape.  The prefill
 * takes N = 16..128 (N = 256 is decode-only) and every P and R with them
 * except fp32 N=128 P=128 R=8, whose tiles do not fit a compute unit's LDS even
 * at 16 tokens per chunk; those get 0 here and M3_ERR_SHAPE from
 * m3_scan_prefill. */
int32_t m3_prefill_chunk_used(const m3_shape* s);

/* Chunked prefill over a whole sequence (the recurrence above for t = 0..L-1).
 * Defined by: explainer panels 1 (coefficients, Eq. 6), 2 (causal operator as a
 * decay x two-band product, Eq. 7), 3 (rotations as data-dependent RoPE,
 * Prop. 3/4, Eq. 11) and 4 (MIMO write/readout, Eqs. 12-14); the chunked
 * evaluation follows the explainer's section 3.3 remark on the chunked
 * algorithm (an exact rearrangement).
 *
 *   x      [b, L, H, R, P]   dtype   X_t stored rank-major: x[b,t,h,r,p] = X_t[p, r]
 *   B, C   [b, L, H, R, N]   dtype   B[b,t,h,r,n] = B_t[n, r]
 *   dt     [b, L, H]         fp32    step size dt_t (>= 0)
 *   A      [H]               fp32    per-head decay generator (<= 0)
 *   lam    [b, L, H]         fp32    current-endpoint weight in [0, 1]
 *   theta  [b, L, H, N/2]    fp32    per-step angle phi_t[k] of pair k (already
 *                                    scaled by dt), or NULL = no rotation
 *   h0     [b, H, N, P]      fp32    incoming state, or NULL = zeros
 *   B_prev [b, H, R, N]      dtype   B and x of the token before t = 0 (the
 *   x_prev [b, H, R, P]      dtype   delayed endpoint of the first step), both
 *                                    NULL = zero previous write.  Give both or none.
 *   y      [b, L, H, R, P]   dtype   out: y[b,t,h,r,p] = Y_t[p, r]
 *   h_out  [b, H, N, P]      fp32    out: H_{L-1} (physical frame), or NULL
 *   workspace, workspace_bytes       device scratch of at least
 *                                    m3_prefill_workspace_bytes(s), zero-filled
 *                                    before its first use (see above)
 * Aliasing: h_out may equal h0.  y must not alias any input (M3_ERR_ALIAS).
 * With L = 0 nothing is computed and h_out (if given) receives h0 (or zeros). */
m3_status m3_scan_prefill(const m3_shape* s,
                          const void* x, const void* B, const void* C,
                          const float* dt, const float* A, const float* lam,
                          const float* theta,
                          const float* h0, const void* B_prev, const void* x_prev,
                          void* y, float* h_out,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* One single-token decode step for b sequences x H heads, updating the state in
 * place: h <- R(phi)[alpha h + beta B_prev x_prev^T] + gamma B x^T, y = h^T C.
 * Defined by the same passages as the prefill, one token at a time (explainer
 * panel 3's physical-frame loop; the decode arithmetic-intensity discussion of
 * section 3.3 and Table 2 is why the state is streamed exactly once).
 *
 *   h      [b, H, N, P]      fp32    state, read and written in place
 *   B_prev [b, H, R, N]      dtype   previous token's B and x (the caller passes
 *   x_prev [b, H, R, P]      dtype   the previous step's B and x pointers), both
 *                                    NULL = zero previous write
 *   x      [b, H, R, P]      dtype   this token's X (rank-major as in the prefill)
 *   B, C   [b, H, R, N]      dtype
 *   dt     [b, H]            fp32
 *   A      [H]               fp32
 *   lam    [b, H]            fp32
 *   theta  [b, H, N/2]       fp32 or NULL
 *   y      [b, H, R, P]      dtype   out
 * s->seqlen and s->chunk are ignored.  y must not alias any input; B_prev/x_prev
 * must not alias B/x of the same step (M3_ERR_ALIAS). */
m3_status m3_decode_step(const m3_shape* s,
                         float* h,
                         const void* B_prev, const void* x_prev,
                         const void* x, const void* B, const void* C,
                         const float* dt, const float* A, const float* lam,
                         const float* theta,
                         void* y, void* stream);

/* m3_decode_step with the state held in bf16 between steps: the pages' decode
 * kernels are benchmarked with an FP32 or a BF16 state (paper page, Table 6).
 * Each step reads the bf16 state, does the update in fp32, reads y from the
 * updated fp32 values and stores the state rounded to nearest even bf16.
 *
 *   h      [b, H, N, P]      bf16    state, read and written in place
 *
 * Every other argument is as for m3_decode_step; s->dtype must be M3_BF16
 * (M3_ERR_DTYPE otherwise).  The same aliasing rules apply (M3_ERR_ALIAS). */
m3_status m3_decode_step_bf16_state(const m3_shape* s,
                                    void* h,
                                    const void* B_prev, const void* x_prev,
                                    const void* x, const void* B, const void* C,
                                    const float* dt, const float* A, const float* lam,
                                    const float* theta,
                                    void* y, void* stream);

/* The two calls above with the gated readout fused into their output stage:
 * instead of y [.., H, R, P] they write
 *   out[.., h, p] = sum_r w_y[h, r, p] * Y[p, r] * silu(w_z[h, r, p] * z[.., h, p]),
 *   silu(v) = v / (1 + exp(-v)),
 * from the fp32 outputs before any rounding (one value per head column: the
 * ranks are contracted).  Defined by: the explainer's note that the
 * architecture uses learned elementwise rank expansion for x, y and the gate
 * instead of dense rank projections (no formula printed; this is the reading
 * adopted: the gate is expanded per rank, applied to that rank's output, and
 * the ranks are summed with weights w_y), and the paper page's Tables 11 and 12,
 * which fuse the gate into the SSM kernel for prefill and decode.
 *   z     [b, L, H, P] (prefill) / [b, H, P] (decode)  dtype  gate input, or
 *                                         NULL = no gate (factor 1)
 *   w_y   [H, R, P]  fp32   rank contraction weights, or NULL = all ones
 *   w_z   [H, R, P]  fp32   rank expansion of the gate, or NULL = all ones
 *                           (unused without z)
 *   out   [b, L, H, P] (prefill) / [b, H, P] (decode)  dtype  out
 * Every other argument, the workspace and the error codes as in
 * m3_scan_prefill / m3_decode_step (fp32 state).  out must not alias any input,
 * the state or the workspace (M3_ERR_ALIAS). */
m3_status m3_scan_prefill_gated(const m3_shape* s,
                                const void* x, const void* B, const void* C,
                                const float* dt, const float* A, const float* lam,
                                const float* theta,
                                const float* h0, const void* B_prev, const void* x_prev,
                                const void* z, const float* w_y, const float* w_z,
                                void* out, float* h_out,
                                void* workspace, size_t workspace_bytes,
                                void* stream);
m3_status m3_decode_step_gated(const m3_shape* s,
                               float* h,
                               const void* B_prev, const void* x_prev,
                               const void* x, const void* B, const void* C,
                               const float* dt, const float* A, const float* lam,
                               const float* theta,
                               const void* z, const float* w_y, const float* w_z,
                               void* out, void* stream);

/* The fused prologue: the pre-processing of B, C and the angles done inside
 * the kernels' load stage.  Defined by: the explainer's note that Mamba-3's B
 * and C receive RMS normalization followed by learned head-specific channel
 * biases (its sec. 3.4 and Table 5(a) remark), and its complex transition
 * generator (Prop. 2: each complex entry a decayed rotation of a pair), whose
 * discretization over a step dt turns the generator's angle theta into the
 * rotation dt * theta as it turns A into the decay exp(dt A).  Reading adopted: every
 * (token, head, rank) column of B, of C and of B_prev (N values) is divided by
 * sqrt(mean of its squares + eps) and then gets bias[h, r, :] added (B_prev
 * takes B's bias; a NULL B_prev stays a zero previous write); `theta` holds raw
 * angles and the step's angle of pair k is dt_t * theta[.., k]. */
typedef struct {
    float eps;              /* added to the mean square before the square root (>= 0;
                               a zero column with eps = 0 gives NaN) */
    const float* bias_B;    /* [H, R, N] fp32 added to B and B_prev after the norm, or NULL */
    const float* bias_C;    /* [H, R, N] fp32 added to C after the norm, or NULL */
} m3_prologue;

/* m3_scan_prefill with the fused prologue applied to B, C, B_prev and theta
 * inside the kernel's load stage.  pro must not be NULL (M3_ERR_NULL).  The
 * bias tables take R x (2N + 4) x 4 bytes of LDS per workgroup beside the chunk's
 * tiles; a shape whose tiles leave too little room gets M3_ERR_SHAPE, and so
 * does a chunk of more than 128 (token, rank) rows for N <= 64 or 256 for
 * N = 128 (the default chunks never are).  fp32 inputs take N <= 64 only
 * (M3_ERR_SHAPE at N = 128); bf16 inputs every N the prefill takes.  The workspace is the one
 * m3_prefill_workspace_bytes gives for the shape.  Everything else as
 * m3_scan_prefill. */
m3_status m3_scan_prefill_prologue(const m3_shape* s, const m3_prologue* pro,
                                   const void* x, const void* B, const void* C,
                                   const float* dt, const float* A, const float* lam,
                                   const float* theta,
                                   const float* h0, const void* B_prev, const void* x_prev,
                                   void* y, float* h_out,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* m3_decode_step (fp32 state) with the fused prologue applied to B, C, B_prev
 * and theta.  pro must not be NULL (M3_ERR_NULL); the bias tables are inputs
 * (they must not overlap y or h, M3_ERR_ALIAS).  Everything else as
 * m3_decode_step. */
m3_status m3_decode_step_prologue(const m3_shape* s, const m3_prologue* pro,
                                  float* h,
                                  const void* B_prev, const void* x_prev,
                                  const void* x, const void* B, const void* C,
                                  const float* dt, const float* A, const float* lam,
                                  const float* theta,
                                  void* y, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* m3_status_str(m3_status st);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int32_t m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3_H */
