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
    M3_ERR_ALIAS = 6,       /* an output aliases an input it must not alias */
    M3_ERR_TIMEOUT = 7      /* (m3_prefill_status) a prefill's look-back wait gave up */
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

/* Bytes of device workspace m3_scan_prefill, m3_scan_prefill_gated and the
 * fused form of m3_scan_prefill_prologue need for this shape (the largest of
 * the three; the staged prologue needs more: m3_prefill_prologue_workspace_bytes; 0 on an
 * invalid or unsupported shape, including one of more than 2^26 - 1
 * chunks).  The buffer holds a control word (ticket count and call epoch) at
 * offset 0, a sticky error word at offset 8 (see m3_prefill_status), per-chunk
 * flags and per-chunk states.  Zero-fill it once before its first use (e.g.
 * hipMemset); every call leaves it ready for the next one, whatever shape that
 * has, so it may be reused across calls on the same stream with nothing done in
 * between.  Calls that may run at the same time (other streams) need workspaces
 * of their own.  A workspace that was not zero-filled before its first use is
 * detected when its control word is out of range (the call then computes
 * nothing and m3_prefill_status reports M3_ERR_WORKSPACE); if garbage happens
 * to look valid, the look-back waits give up and m3_prefill_status reports
 * M3_ERR_TIMEOUT.  No access ever leaves the buffers. */
size_t m3_prefill_workspace_bytes(const m3_shape* s);

/* Tokens per chunk m3_scan_prefill will use for this shape, or 0 when it
 * takes none (M3_ERR_SHAPE from m3_scan_prefill).  A requested chunk (s->chunk
 * > 0) is used exactly as given: it must be a power of two in [16, 256] whose
 * (token, rank) rows, angles and LDS tiles fit one compute unit and whose
 * kernel variant uses no scratch memory, otherwise the shape is refused
 * (m3_prefill_max_chunk gives the largest that is taken).  With s->chunk = 0
 * the library picks 128 (token, rank) rows for N <= 64 and 256 above, halved
 * until taken.  The prefill takes N = 16..128 (N = 256 is decode-only).  The
 * library never launches a kernel variant that the build's compiler report
 * gives any scratch (private memory) per lane: every GPU memory fault and the
 * one wrong result met in this kernel's development came from such variants,
 * and their cause was not established.  Those shapes (fp32 at N = 128, bf16 at
 * N = 128 with P = 128, fp32 N <= 32 P = 128 at chunks of four output tiles
 * per wave, some prologue variants) get 0 here and M3_ERR_SHAPE from the call. */
int32_t m3_prefill_chunk_used(const m3_shape* s);

/* The largest chunk (tokens) m3_scan_prefill takes for this shape, ignoring
 * s->chunk, or 0 when it takes none. */
int32_t m3_prefill_max_chunk(const m3_shape* s);

/* m3_prefill_chunk_used for m3_scan_prefill_gated (which has kernel variants
 * of its own) and for m3_scan_prefill_prologue (its fused variant's chunk, or
 * in the staged form m3_scan_prefill's): the chunk each will use, or 0 when it
 * refuses the shape. */
int32_t m3_prefill_gated_chunk_used(const m3_shape* s);
int32_t m3_prefill_prologue_chunk_used(const m3_shape* s);

/* Waits for `stream`, then reads and clears the workspace's error word, which
 * the prefill kernels set instead of hanging or faulting:
 *   M3_OK           no error since the last query
 *   M3_ERR_TIMEOUT  a chunk's look-back wait for its predecessors gave up (a
 *                   bounded spin); that chunk's outputs and final state are NaN
 *   M3_ERR_WORKSPACE the control word was out of range (the workspace was not
 *                   zero-filled before its first use); nothing was computed
 *   M3_ERR_NULL / M3_ERR_DEVICE on a NULL workspace or a failed HIP call.
 * The error word accumulates over calls on the workspace until it is queried.
 * The workspace is as passed to the prefill calls (at least 16 bytes). */
m3_status m3_prefill_status(void* workspace, size_t workspace_bytes, void* stream);

/* For tests of the error path only: the number of polls a prefill look-back
 * wait makes before it gives up (0 restores the default, 2^20).  Process-wide;
 * not for use while prefill calls run on other threads. */
void m3_debug_set_spin_limit(uint32_t polls);

/* The two implementations of m3_scan_prefill.  Both compute the same chunked
 * rearrangement of the recurrence (explainer sec. 3.3) with the same
 * workspace:
 *   M3_KERNEL_PER_CHUNK  one workgroup per (sequence, chunk), every variant
 *                        (dtype, N = 16..128, P, R, gate, prologue);
 *   M3_KERNEL_STREAM     one persistent workgroup per compute unit streaming
 *                        its chunks' B and X through LDS in 32-row blocks while
 *                        the next blocks' loads are in flight; bf16 inputs,
 *                        P = 64, no gate or prologue, N = 64 at R = 1, 2 or 4
 *                        with chunks of 128 or 256 (token, rank) rows, N = 128
 *                        with 128 rows (R = 1, 2, 4) or 256 rows (R = 4). */
enum { M3_KERNEL_PER_CHUNK = 1, M3_KERNEL_STREAM = 2 };

/* The kernel m3_scan_prefill runs for this shape (s->chunk as in
 * m3_prefill_chunk_used): M3_KERNEL_STREAM where that kernel takes the shape
 * at N = 128 (at N = 64 the per-chunk kernel is the faster one), else
 * M3_KERNEL_PER_CHUNK; 0 when the call refuses the shape. */
int32_t m3_prefill_kernel_used(const m3_shape* s);

/* For tests and measurement: restricts m3_scan_prefill (and the queries) to one
 * kernel.  0 restores the library's choice, M3_KERNEL_PER_CHUNK uses only the
 * per-chunk kernel, M3_KERNEL_STREAM the streaming kernel wherever it takes
 * the shape.  Any other value: M3_ERR_SHAPE, nothing changed.  Process-wide;
 * not for use while prefill calls run on other threads. */
m3_status m3_debug_set_prefill_kernel(int32_t which);

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

/* Size of the scratch buffer m3_scan_prefill_noalloc uses on each device. */
#define M3_NOALLOC_SCRATCH_BYTES (64u << 20)

/* m3_scan_prefill for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same computation and arguments without the workspace.  The chunk hand-off
 * lives in a buffer of M3_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds
 * on each device it runs on until the process ends; the call allocates nothing
 * and calls no allocating routine.  Shapes whose workspace
 * (m3_prefill_workspace_bytes) is larger get M3_ERR_WORKSPACE (e.g. a few
 * thousand chunks of a 128 x 64 state); nothing is launched then.  Every call
 * on a device shares that device's buffer and clears its control words first
 * (with a kernel on `stream`): calls that overlap on one device race, so a
 * caller serialises them (one stream, or events).  Errors of the look-back
 * show as NaN outputs (there is no status query for this buffer).  Everything
 * else as m3_scan_prefill. */
m3_status m3_scan_prefill_noalloc(const m3_shape* s,
                                  const void* x, const void* B, const void* C,
                                  const float* dt, const float* A, const float* lam,
                                  const float* theta,
                                  const float* h0, const void* B_prev, const void* x_prev,
                                  void* y, float* h_out, void* stream);

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

/* m3_scan_prefill with the prologue applied to B, C, B_prev and theta.  It
 * takes every shape m3_scan_prefill takes, in one of two forms
 * (m3_prefill_prologue_mode):
 *   M3_PROLOGUE_FUSED   the prologue runs inside the prefill kernel's load
 *                       stage (one launch; its bias tables take about
 *                       R x 2N x 4 bytes of LDS beside the chunk's tiles).
 *                       Used where such a kernel variant exists and uses no
 *                       scratch memory: in the streaming kernel wherever the
 *                       plain prefill streams (bf16, P = 64, R = 2 or 4 at
 *                       N = 128, among them the MIMO and long shapes), else in
 *                       the per-chunk kernel: bf16 or fp32 inputs at N <= 64 and
 *                       bf16 at N = 128 with P <= 32, at chunks of one 16-row
 *                       output tile per wave (m3_prefill_prologue_kernel_used
 *                       says which kernel);
 *   M3_PROLOGUE_STAGED  elsewhere: a prologue kernel writes the normalized B,
 *                       C, B_prev and the angles dt x theta into the workspace
 *                       (the inputs' layouts and dtype, bf16 rounded to nearest
 *                       even; angles fp32), then the plain prefill runs on them
 *                       with the chunk m3_scan_prefill takes.  The results equal
 *                       the fused form's up to that rounding.
 * pro must not be NULL (M3_ERR_NULL).  The workspace must hold
 * m3_prefill_prologue_workspace_bytes(s) bytes (M3_ERR_WORKSPACE), zero-filled
 * before its first use as for m3_scan_prefill, and in the staged form it must
 * not overlap any input, y or h_out (M3_ERR_ALIAS).  Everything else as
 * m3_scan_prefill. */
enum { M3_PROLOGUE_FUSED = 1, M3_PROLOGUE_STAGED = 2 };
int32_t m3_prefill_prologue_mode(const m3_shape* s);   /* 0 when the shape is refused */
/* The prefill kernel a m3_scan_prefill_prologue call runs (M3_KERNEL_STREAM or
 * M3_KERNEL_PER_CHUNK, as m3_prefill_kernel_used; in the staged form the plain
 * prefill's), or 0 when the shape is refused. */
int32_t m3_prefill_prologue_kernel_used(const m3_shape* s);
/* Likewise for m3_scan_prefill_gated: the streaming kernel, with the gated
 * readout in its output stage, wherever the plain prefill streams and that
 * variant uses no scratch; else the per-chunk kernel's gated variant. */
int32_t m3_prefill_gated_kernel_used(const m3_shape* s);
/* Bytes of workspace m3_scan_prefill_prologue needs for this shape (never less
 * than m3_prefill_workspace_bytes, so one buffer serves every prefill entry
 * point; 0 when the shape is refused).  In the staged form it adds, behind the
 * plain prefill's part, b x L x H x R x N elements each for B and C,
 * b x H x R x N for B_prev and b x L x H x N/2 fp32 angles. */
size_t m3_prefill_prologue_workspace_bytes(const m3_shape* s);
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

/* Bytes of device workspace m3_scan_backward needs for this shape (0 when it
 * takes none): per segment of the sequence (1..32 tokens, the most whose rows
 * fit one compute unit's 160 KB LDS for this N, P, R; 32 at R = 1, 8 at R = 4)
 * three N x P fp32 hand-off arrays (the segment's state from a zero start,
 * its true entering state, the state gradient entering from its right) and
 * two N/2 complex propagators.  No per-token state is stored.
 * The backward takes N = 16..128, P = 16..64, every R, fp32 or bf16 inputs,
 * except variants whose compiled kernels use scratch memory (none in the
 * current build); the call refuses those with M3_ERR_SHAPE. */
size_t m3_scan_backward_workspace_bytes(const m3_shape* s);

/* Gradients of the prefill (the recurrence of m3_scan_prefill): given the
 * forward call's inputs and the cotangents dy of y and dh_out of h_out, the
 * gradients of <dy, y> + <dh_out, h_out> with respect to every input.
 * Defined by the recurrence itself (explainer panels 1, 3, 4; paper page,
 * Table 1 caption), differentiated backwards through time as the explainer's
 * training remark describes (a recurrence of the same form):
 *   G_t = C_t dY_t^T + alpha_{t+1} R(phi_{t+1})^T G_{t+1},  Q_t = R(phi_t)^T G_t,
 *   dV_t = gamma_t G_t + beta_{t+1} Q_{t+1},  dC_t = H_t dY_t,  dB_t = dV_t X_t,
 *   dX_t = dV_t^T B_t,  dalpha_t = <Q_t, H_{t-1}>,  dbeta_t = <Q_t, V_{t-1}>,
 *   dgamma_t = <G_t, V_t>, dphi_t[k] = sum_p (G_t[2k+1] K_t[2k] - G_t[2k] K_t[2k+1])
 *   with K_t = H_t - gamma_t V_t, and the chain rule of alpha, beta, gamma into
 * dt, lam and A.
 *
 *   inputs       as m3_scan_prefill (theta, h0, B_prev/x_prev may be NULL)
 *   dy           [b, L, H, R, P]  dtype   cotangent of y
 *   dh_out       [b, H, N, P]     fp32    cotangent of h_out, or NULL (zeros)
 *   outputs, all fp32, written whole (not accumulated):
 *   dx [b,L,H,R,P], dB, dC [b,L,H,R,N], ddt, dlam [b,L,H], dA [H],
 *   dtheta [b,L,H,N/2]   (NULL exactly when theta is NULL)
 *   dh0 [b,H,N,P]        or NULL (not computed; given h0 NULL it is the
 *                        gradient with respect to a zero initial state)
 *   dB_prev [b,H,R,N], dx_prev [b,H,R,P]  or NULL; must be NULL when B_prev is
 *   workspace            at least m3_scan_backward_workspace_bytes(s); no
 *                        contents required
 * Errors: M3_ERR_NULL (a required pointer, or dtheta not matching theta),
 * M3_ERR_SHAPE, M3_ERR_WORKSPACE, M3_ERR_ALIAS (an output overlapping an input,
 * the workspace or another output).  Work runs on `stream` in five launches:
 * each segment of each (sequence, head) runs forward from a zero state and
 * forms its propagator, a short pass per (sequence, head) composes them into
 * every segment's entering state, the same two steps run backwards through
 * time for the state gradient entering each segment from its right, and a
 * last launch forms every gradient of a segment from those two in closed
 * matrix form (pairwise products of the segment's rows), without a stored
 * per-token state. */
m3_status m3_scan_backward(const m3_shape* s,
                           const void* x, const void* B, const void* C,
                           const float* dt, const float* A, const float* lam, const float* theta,
                           const float* h0, const void* B_prev, const void* x_prev,
                           const void* dy, const float* dh_out,
                           float* dx, float* dB, float* dC, float* ddt, float* dA, float* dlam,
                           float* dtheta, float* dh0, float* dB_prev, float* dx_prev,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* m3_status_str(m3_status st);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int32_t m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3_H */
