// m3_api.cpp -- the extern "C" boundary of libm3.so (declared in include/m3.h).
//
// Host-side only: validates shapes, pointers, dtype, workspace size and
// aliasing before anything is enqueued, plans the chunking and workspace, and
// hands off to the launchers.  No allocation, no synchronisation, no exceptions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>

#include "m3_internal.h"
#include "m3_prologue.h"

namespace m3 {
namespace {

size_t esize(int dtype) { return dtype == M3_BF16 ? 2 : 4; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

m3_status check_common(const m3_shape* s, bool need_seq) {
  if (!s) return M3_ERR_NULL;
  if (s->dtype != M3_FP32 && s->dtype != M3_BF16) return M3_ERR_DTYPE;
  if (s->batch < 0 || s->nheads < 0 || (need_seq && s->seqlen < 0) || s->chunk < 0) return M3_ERR_SHAPE;
  if (!supported_head(s->headdim) || !supported_state(s->dstate) || !supported_rank(s->rank))
    return M3_ERR_SHAPE;
  return M3_OK;
}

// Tokens per chunk.  A chunk of q tokens fits when q is a power of two in
// [16, 256], its q x R rows and q x N/2 angles fit the kernel's register
// budget and its LDS tiles fit on a compute unit.  A requested chunk must fit
// as given (no silent change: anything else is M3_ERR_SHAPE); chunk 0 takes the
// default, 128 (token, rank) rows for N <= 64 and 256 rows above (the state
// hand-off per chunk grows with N; so does the work that amortises it),
// halved until it fits.
size_t lds_need(int q, const m3_shape& s) {
  return fused_lds_bytes(q, s.rank, s.dstate, s.headdim, (int)esize(s.dtype));
}

// The prologue prefill's own limits on top of the plain one's: bf16 inputs
// at every N, fp32 at N <= 64, and one 16-row output tile per wave (its
// variants with more made a GPU memory fault whose cause is not established,
// as did an fp32 N = 128 one), plus its bias tables' LDS.
bool prologue_ok(const m3_shape& s, int q) {
  if (s.dtype == M3_FP32 && s.dstate >= 128) return false;
  if (fused_row_tiles(q, s.rank, s.dstate) != 1) return false;
  return fused_lds_bytes(q, s.rank, s.dstate, s.headdim, (int)esize(s.dtype), 1) <= (size_t)kLdsBudget;
}

bool chunk_fits(int q, const m3_shape& s, int gated, int pro) {
  if (q < 16 || q > 256 || !is_pow2(q)) return false;
  if (q * s.rank > fused_max_rows(s.dstate) || q * (s.dstate / 2) > kFusedAngleCap) return false;
  if (lds_need(q, s) > (size_t)kLdsBudget) return false;
  if (pro && !prologue_ok(s, q)) return false;
  const PrefillVariant v{s.dtype, s.dstate, s.headdim, s.rank, fused_row_tiles(q, s.rank, s.dstate), gated, pro};
  return v.RT != 0 && !prefill_variant_spills(v);
}

int max_chunk(const m3_shape& s, int gated, int pro) {
  for (int q = 256; q >= 16; q /= 2)
    if (chunk_fits(q, s, gated, pro)) return q;
  return 0;
}

int choose_chunk(const m3_shape& s, int gated, int pro) {
  if (s.chunk > 0) return chunk_fits(s.chunk, s, gated, pro) ? s.chunk : 0;
  const int rows = s.dstate <= 64 ? 128 : 256;
  for (int q = std::max(16, rows / s.rank); q >= 16; q /= 2)
    if (chunk_fits(q, s, gated, pro)) return q;
  return 0;
}

// The streaming prefill variants {N, P, R, 32-row blocks, prologue, gated}
// that use scratch (build report): those shapes take the per-chunk kernel.
const int kStreamScratch[][6] = {
#include "m3_scratch_table_stream.inc"
    {-1, 0, 0, 0, 0, 0}};

bool stream_spills(int N, int P, int R, int Q, int pro, int gated) {
  for (const auto& k : kStreamScratch)
    if (k[0] == N && k[1] == P && k[2] == R && k[3] * 32 == Q * R && k[4] == (pro ? 1 : 0) &&
        k[5] == (gated ? 1 : 0))
      return true;
  return false;
}

// The backward variants {dtype, N, P, R} that use scratch (build report).
const int kBackwardScratch[][4] = {
#include "m3_scratch_table_bwd.inc"
    {-1, 0, 0, 0}};

// The prefill variants that use scratch, from the build's compiler report:
// {dtype, N, P, R, RT, gated, prologue} per line.
const PrefillVariant kScratchVariants[] = {
#include "m3_scratch_table.inc"
    {-1, 0, 0, 0, 0, 0, 0}};

// Look-back polls before a wait gives up (tests lower it to force the
// error path; see m3_debug_set_spin_limit).
std::atomic<unsigned> g_spin_limit{kDefaultSpinLimit};

// Which prefill kernel plain calls may use (m3_debug_set_prefill_kernel):
// 0 the library's choice, M3_KERNEL_PER_CHUNK only that one, M3_KERNEL_STREAM
// the streaming kernel wherever it takes the shape.
std::atomic<int> g_prefill_kernel{0};

}  // namespace

bool prefill_variant_spills(const PrefillVariant& v) {
  for (const PrefillVariant& k : kScratchVariants)
    if (k.dtype == v.dtype && k.N == v.N && k.P == v.P && k.R == v.R && k.RT == v.RT && k.gated == v.gated &&
        k.pro == v.pro)
      return true;
  return false;
}

bool plan_prefill(const m3_shape& s, PrefillPlan* plan, int gated, int pro) {
  // N = 256 is decode-only: its prefill kernels spill 76-708 bytes per lane to
  // scratch, and a memory fault was seen in one of them whose cause is not
  // established, so that path is not built.
  if (s.dstate > 128) return false;
  const int mode = g_prefill_kernel.load(std::memory_order_relaxed);
  // whether the streaming kernel runs a shape at chunk q (the library's choice
  // at N = 128; at N = 64 only when asked for)
  auto streams = [&](int q, int with_pro) {
    return q > 0 && mode != M3_KERNEL_PER_CHUNK && (mode == M3_KERNEL_STREAM || s.dstate == 128) &&
           stream_supported(s.dtype, s.dstate, s.headdim, s.rank, q, gated, with_pro) &&
           !stream_spills(s.dstate, s.headdim, s.rank, q, with_pro, gated);
  };
  int q = 0;
  bool stream_pro = false;
  if (pro && !gated) {
    // the prologue fused into the streaming kernel, at the plain prefill's
    // chunk, wherever the plain prefill would stream
    const int qs = choose_chunk(s, 0, 0);
    if (streams(qs, 0) && streams(qs, 1)) {
      q = qs;
      stream_pro = true;
    }
  }
  if (!stream_pro) q = choose_chunk(s, gated, pro);
  if (q == 0) return false;
  plan->Q = q;
  plan->nc = s.seqlen > 0 ? (s.seqlen + q - 1) / q : 0;
  const size_t bhc = (size_t)s.batch * s.nheads * plan->nc;
  if (bhc > kMaxChunks) return false;
  const size_t map = (size_t)fused_slot_floats(s.dstate, s.headdim) * sizeof(float);
  plan->off_flags = 256;
  plan->off_recs = align256(plan->off_flags + bhc * sizeof(unsigned long long));
  plan->off_maps = align256(plan->off_recs + bhc * (s.dstate + 2) * sizeof(float));
  plan->off_states = align256(plan->off_maps + bhc * map);
  plan->bytes = align256(plan->off_states + bhc * map);
  plan->lds = pro ? fused_lds_bytes(q, s.rank, s.dstate, s.headdim, (int)esize(s.dtype), 1) : lds_need(q, s);
  plan->kernel = M3_KERNEL_PER_CHUNK;
  // The streaming kernel takes the shapes it supports at N = 128, where a
  // chunk of the per-chunk kernel fills a compute unit's LDS on its own, so
  // nothing overlaps its loads with its arithmetic.  At N = 64 the per-chunk
  // kernel runs two workgroups per compute unit and measured faster (SISO,
  // 4 x 4096 tokens x 32 heads, chunk 128: 134 us against 196 us); the
  // streaming kernel runs there only when asked for (m3_debug_set_prefill_kernel).
  if (stream_pro || (!pro && streams(q, 0))) {
    plan->kernel = M3_KERNEL_STREAM;
    plan->lds = pro ? stream_lds_bytes_pro(q, s.rank, s.dstate, s.headdim) : stream_lds_bytes(q, s.rank, s.dstate, s.headdim);
  }
  return true;
}

// The prologue prefill in one of two forms: fused into the prefill's load
// stage (the shape's prologue kernel variant), or, where the library does not
// launch that variant, staged: a prologue kernel writes the normalized B, C,
// B_prev and the angles dt x theta into the workspace behind the plain
// prefill's part, and the plain prefill runs on them.  The staged form takes
// every shape the plain prefill takes.
struct StagedLayout { size_t off_B, off_C, off_Bp, off_phi, bytes; };

StagedLayout staged_layout(const m3_shape& s, const PrefillPlan& plain) {
  const size_t es = esize(s.dtype), tok = (size_t)s.batch * s.seqlen * s.nheads, bh = (size_t)s.batch * s.nheads;
  const size_t rowsz = (size_t)s.rank * s.dstate * es;
  StagedLayout o;
  o.off_B = align256(plain.bytes);
  o.off_C = align256(o.off_B + tok * rowsz);
  o.off_Bp = align256(o.off_C + tok * rowsz);
  o.off_phi = align256(o.off_Bp + bh * rowsz);
  o.bytes = align256(o.off_phi + tok * (s.dstate / 2) * sizeof(float));
  return o;
}

// M3_PROLOGUE_FUSED or M3_PROLOGUE_STAGED with that form's plan, or 0 when
// the shape is refused.
int prologue_mode(const m3_shape& s, PrefillPlan* plan) {
  if (plan_prefill(s, plan, 0, 1)) return M3_PROLOGUE_FUSED;
  if (plan_prefill(s, plan, 0, 0)) return M3_PROLOGUE_STAGED;
  return 0;
}

}  // namespace m3

using namespace m3;

extern "C" {

size_t m3_prefill_workspace_bytes(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  // the largest of the three entry points' needs for this shape (they share
  // the layout; they differ only in which chunks they take)
  size_t bytes = 0;
  for (int v = 0; v < 3; ++v) {
    PrefillPlan plan;
    if (plan_prefill(*s, &plan, v == 1, v == 2)) bytes = std::max(bytes, plan.bytes);
  }
  return bytes;
}

int32_t m3_prefill_chunk_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, 0, 0)) return 0;
  return plan.Q;
}

int32_t m3_prefill_gated_chunk_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, 1, 0)) return 0;
  return plan.Q;
}

int32_t m3_prefill_prologue_chunk_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!prologue_mode(*s, &plan)) return 0;
  return plan.Q;
}

int32_t m3_prefill_gated_kernel_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, 1, 0)) return 0;
  return plan.kernel;
}

int32_t m3_prefill_prologue_kernel_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!prologue_mode(*s, &plan)) return 0;
  return plan.kernel;
}

int32_t m3_prefill_prologue_mode(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  return prologue_mode(*s, &plan);
}

size_t m3_prefill_prologue_workspace_bytes(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  const int mode = prologue_mode(*s, &plan);
  if (!mode) return 0;
  const size_t own = mode == M3_PROLOGUE_STAGED ? staged_layout(*s, plan).bytes : plan.bytes;
  return std::max(own, m3_prefill_workspace_bytes(s));
}

int32_t m3_prefill_max_chunk(const m3_shape* s) {
  if (check_common(s, true) != M3_OK || s->dstate > 128) return 0;
  return max_chunk(*s, 0, 0);
}

m3_status m3_prefill_status(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return M3_ERR_NULL;
  if (workspace_bytes < 16) return M3_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  unsigned long long word = 0;
  unsigned long long* dev = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + 8);
  if (hipMemcpyAsync(&word, dev, sizeof(word), hipMemcpyDeviceToHost, hs) != hipSuccess) return M3_ERR_DEVICE;
  if (hipStreamSynchronize(hs) != hipSuccess) return M3_ERR_DEVICE;
  if (word == 0) return M3_OK;
  if (launch_copy_or_zero(reinterpret_cast<float*>(dev), nullptr, 2, hs) != hipSuccess) return M3_ERR_DEVICE;
  if (hipStreamSynchronize(hs) != hipSuccess) return M3_ERR_DEVICE;
  return (word & kErrControl) ? M3_ERR_WORKSPACE : M3_ERR_TIMEOUT;
}

void m3_debug_set_spin_limit(uint32_t polls) { g_spin_limit.store(polls ? polls : kDefaultSpinLimit); }

int32_t m3_prefill_kernel_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, 0, 0)) return 0;
  return plan.kernel;
}

m3_status m3_debug_set_prefill_kernel(int32_t which) {
  if (which != 0 && which != M3_KERNEL_PER_CHUNK && which != M3_KERNEL_STREAM) return M3_ERR_SHAPE;
  g_prefill_kernel.store(which, std::memory_order_relaxed);
  return M3_OK;
}

}  // extern "C"

namespace {

// The gated readout's operands (gated = false: plain y output).
struct Gate {
  bool gated;
  const void* z; const float* w_y; const float* w_z;
};

// The prologue's options (on = false: inputs used as given).
struct Pro {
  bool on;
  float eps; const float* bias_B; const float* bias_C;
};
constexpr Pro kNoPro{false, 0.f, nullptr, nullptr};

// Shared by both prefill entry points: `y` is y [b,L,H,R,P], or with a gate
// out [b,L,H,P].
m3_status prefill_common(const m3_shape* s,
                         const void* x, const void* B, const void* C,
                         const float* dt, const float* A, const float* lam,
                         const float* theta,
                         const float* h0, const void* B_prev, const void* x_prev,
                         const Gate& g, const Pro& pro, void* y, float* h_out,
                         void* workspace, size_t workspace_bytes,
                         void* stream) {
  m3_status st = check_common(s, true);
  if (st != M3_OK) return st;
  const int b = s->batch, L = s->seqlen, H = s->nheads, P = s->headdim, N = s->dstate, R = s->rank;
  const size_t es = esize(s->dtype);
  const size_t tok = (size_t)b * L * H;
  const size_t bh = (size_t)b * H;
  if ((B_prev == nullptr) != (x_prev == nullptr)) return M3_ERR_NULL;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (bh == 0) return M3_OK;
  if (L == 0) {
    if (h_out && launch_copy_or_zero(h_out, h0, bh * N * P, hs) != hipSuccess) return M3_ERR_DEVICE;
    return M3_OK;
  }
  if (!x || !B || !C || !dt || !A || !lam || !y) return M3_ERR_NULL;

  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, g.gated ? 1 : 0, pro.on ? 1 : 0)) return M3_ERR_SHAPE;
  if (!workspace || workspace_bytes < plan.bytes) return M3_ERR_WORKSPACE;

  // y (or out) must not alias any input, the final state or the workspace;
  // h_out may be exactly h0 but must not overlap anything else.
  const size_t ybytes = tok * (g.gated ? 1 : R) * P * es;
  const size_t sbytes = bh * N * P * sizeof(float);
  const size_t wbytes = (size_t)H * R * P * sizeof(float);
  struct { const void* p; size_t n; } ins[] = {
      {x, tok * R * P * es}, {B, tok * R * N * es}, {C, tok * R * N * es},
      {dt, tok * sizeof(float)}, {A, (size_t)H * sizeof(float)}, {lam, tok * sizeof(float)},
      {theta, theta ? tok * (N / 2) * sizeof(float) : 0}, {h0, h0 ? sbytes : 0},
      {B_prev, bh * R * N * es}, {x_prev, bh * R * P * es}, {workspace, plan.bytes},
      {g.z, g.z ? tok * P * es : 0}, {g.w_y, g.w_y ? wbytes : 0}, {g.w_z, g.w_z ? wbytes : 0},
      {pro.bias_B, pro.bias_B ? (size_t)H * R * N * sizeof(float) : 0},
      {pro.bias_C, pro.bias_C ? (size_t)H * R * N * sizeof(float) : 0}};
  for (const auto& in : ins) {
    if (overlaps(y, ybytes, in.p, in.n)) return M3_ERR_ALIAS;
    if (h_out && in.p != h0 && overlaps(h_out, sbytes, in.p, in.n)) return M3_ERR_ALIAS;
  }
  const size_t lds = plan.lds;   // (the prologue's plan includes its bias tables)
  if (h_out && overlaps(h_out, sbytes, y, ybytes)) return M3_ERR_ALIAS;
  if (h_out && h0 && h_out != h0 && overlaps(h_out, sbytes, h0, sbytes)) return M3_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  FusedParams f;
  f.x = x; f.B = B; f.C = C; f.dt = dt; f.A = A; f.lam = lam; f.theta = theta;
  f.h0 = h0; f.Bp = B_prev; f.xp = x_prev; f.h_out = h_out;
  f.y = g.gated ? nullptr : y;
  f.out = g.gated ? y : nullptr;
  f.z = g.z; f.wy = g.w_y; f.wz = g.z ? g.w_z : nullptr;
  f.pro = pro.on ? 1 : 0; f.eps = pro.eps; f.biasB = pro.bias_B; f.biasC = pro.bias_C;
  f.ctl = reinterpret_cast<unsigned long long*>(ws);
  f.err = reinterpret_cast<unsigned long long*>(ws + 8);
  f.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
  f.flags = reinterpret_cast<unsigned long long*>(ws + plan.off_flags);
  f.recs = reinterpret_cast<float*>(ws + plan.off_recs);
  f.maps = reinterpret_cast<float*>(ws + plan.off_maps);
  f.states = reinterpret_cast<float*>(ws + plan.off_states);
  f.batch = b; f.L = L; f.H = H; f.N = N; f.P = P; f.R = R; f.logR = ilog2(R);
  f.Q = plan.Q; f.nc = plan.nc;
  f.use_maps = 1;   // (the launch decides from the device's resident workgroups)
  f.late_flag = 0;  // (likewise, for the streaming kernel)
  const hipError_t e = plan.kernel == M3_KERNEL_STREAM ? launch_stream_prefill(f, hs)
                                                       : launch_fused_prefill(f, lds, s->dtype, hs);
  if (e == hipErrorNotSupported) return M3_ERR_SHAPE;   // the loaded kernel uses scratch
  if (e != hipSuccess) return M3_ERR_DEVICE;
  return M3_OK;
}

// Shared by both decode entry points: the state is fp32 or (state_bf16) bf16.
// `y` is y [b,H,R,P], or with a gate out [b,H,P].
m3_status decode_common(const m3_shape* s, void* h, int state_bf16,
                        const void* B_prev, const void* x_prev,
                        const void* x, const void* B, const void* C,
                        const float* dt, const float* A, const float* lam,
                        const float* theta, const Gate& g, const Pro& pro, void* y, void* stream) {
  m3_status st = check_common(s, false);
  if (st != M3_OK) return st;
  if (state_bf16 && s->dtype != M3_BF16) return M3_ERR_DTYPE;
  const int b = s->batch, H = s->nheads, P = s->headdim, N = s->dstate, R = s->rank;
  const size_t es = esize(s->dtype);
  const size_t bh = (size_t)b * H;
  if ((B_prev == nullptr) != (x_prev == nullptr)) return M3_ERR_NULL;
  if (bh == 0) return M3_OK;
  if (!h || !x || !B || !C || !dt || !A || !lam || !y) return M3_ERR_NULL;

  const size_t ybytes = bh * (g.gated ? 1 : R) * P * es;
  const size_t hbytes = bh * N * P * (state_bf16 ? 2 : sizeof(float));
  const size_t wbytes = (size_t)H * R * P * sizeof(float);
  struct { const void* p; size_t n; } ins[] = {
      {x, bh * R * P * es}, {B, bh * R * N * es}, {C, bh * R * N * es},
      {dt, bh * sizeof(float)}, {A, (size_t)H * sizeof(float)}, {lam, bh * sizeof(float)},
      {theta, theta ? bh * (N / 2) * sizeof(float) : 0},
      {B_prev, bh * R * N * es}, {x_prev, bh * R * P * es},
      {g.z, g.z ? bh * P * es : 0}, {g.w_y, g.w_y ? wbytes : 0}, {g.w_z, g.w_z ? wbytes : 0},
      {pro.bias_B, pro.bias_B ? (size_t)H * R * N * sizeof(float) : 0},
      {pro.bias_C, pro.bias_C ? (size_t)H * R * N * sizeof(float) : 0}};
  for (const auto& in : ins) {
    if (overlaps(y, ybytes, in.p, in.n)) return M3_ERR_ALIAS;
    if (overlaps(h, hbytes, in.p, in.n)) return M3_ERR_ALIAS;
  }
  if (overlaps(y, ybytes, h, hbytes)) return M3_ERR_ALIAS;
  if (overlaps(B_prev, bh * R * N * es, B, bh * R * N * es) ||
      overlaps(x_prev, bh * R * P * es, x, bh * R * P * es))
    return M3_ERR_ALIAS;

  DecodeParams p;
  p.h = h; p.state_bf16 = state_bf16; p.Bp = B_prev; p.xp = x_prev; p.x = x; p.B = B; p.C = C;
  p.dt = dt; p.A = A; p.lam = lam; p.theta = theta;
  p.y = g.gated ? nullptr : y;
  p.out = g.gated ? y : nullptr;
  p.z = g.z; p.wy = g.w_y; p.wz = g.z ? g.w_z : nullptr;
  p.pro = pro.on ? 1 : 0; p.eps = pro.eps; p.biasB = pro.bias_B; p.biasC = pro.bias_C;
  p.batch = b; p.H = H; p.N = N; p.P = P; p.R = R;
  if (launch_decode(p, s->dtype, static_cast<hipStream_t>(stream)) != hipSuccess) return M3_ERR_DEVICE;
  return M3_OK;
}

}  // namespace

extern "C" {

m3_status m3_decode_step(const m3_shape* s,
                         float* h,
                         const void* B_prev, const void* x_prev,
                         const void* x, const void* B, const void* C,
                         const float* dt, const float* A, const float* lam,
                         const float* theta,
                         void* y, void* stream) {
  return decode_common(s, h, 0, B_prev, x_prev, x, B, C, dt, A, lam, theta, Gate{false, nullptr, nullptr, nullptr},
                       kNoPro, y, stream);
}

m3_status m3_decode_step_gated(const m3_shape* s,
                               float* h,
                               const void* B_prev, const void* x_prev,
                               const void* x, const void* B, const void* C,
                               const float* dt, const float* A, const float* lam,
                               const float* theta,
                               const void* z, const float* w_y, const float* w_z,
                               void* out, void* stream) {
  return decode_common(s, h, 0, B_prev, x_prev, x, B, C, dt, A, lam, theta, Gate{true, z, w_y, w_z}, kNoPro, out, stream);
}

m3_status m3_decode_step_bf16_state(const m3_shape* s,
                                    void* h,
                                    const void* B_prev, const void* x_prev,
                                    const void* x, const void* B, const void* C,
                                    const float* dt, const float* A, const float* lam,
                                    const float* theta,
                                    void* y, void* stream) {
  return decode_common(s, h, 1, B_prev, x_prev, x, B, C, dt, A, lam, theta, Gate{false, nullptr, nullptr, nullptr},
                       kNoPro, y, stream);
}

m3_status m3_decode_step_prologue(const m3_shape* s, const m3_prologue* pro,
                                  float* h,
                                  const void* B_prev, const void* x_prev,
                                  const void* x, const void* B, const void* C,
                                  const float* dt, const float* A, const float* lam,
                                  const float* theta,
                                  void* y, void* stream) {
  if (!pro) return M3_ERR_NULL;
  return decode_common(s, h, 0, B_prev, x_prev, x, B, C, dt, A, lam, theta, Gate{false, nullptr, nullptr, nullptr},
                       Pro{true, pro->eps, pro->bias_B, pro->bias_C}, y, stream);
}

m3_status m3_scan_prefill(const m3_shape* s,
                          const void* x, const void* B, const void* C,
                          const float* dt, const float* A, const float* lam,
                          const float* theta,
                          const float* h0, const void* B_prev, const void* x_prev,
                          void* y, float* h_out,
                          void* workspace, size_t workspace_bytes,
                          void* stream) {
  return prefill_common(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, Gate{false, nullptr, nullptr, nullptr},
                        kNoPro, y, h_out, workspace, workspace_bytes, stream);
}

namespace {
// Backward workspace: three segment hand-off arrays [b*H][nseg][N][P] (local
// states then local G; the state entering each segment; the G entering each
// segment) | the forward and backward propagators [b*H][nseg][N/2] (re, im),
// each region 256-byte aligned.
struct BackwardLayout {
  int S, nseg;
  size_t off_sega, off_segb, off_segc, off_zf, off_zb, bytes;
};
BackwardLayout backward_layout(const m3_shape& s) {
  BackwardLayout o;
  const size_t nbh = (size_t)s.batch * s.nheads, NP = (size_t)s.dstate * s.headdim;
  o.S = backward_segment(s.rank, s.dstate, s.headdim);
  o.nseg = s.seqlen > 0 && o.S > 0 ? (s.seqlen + o.S - 1) / o.S : 0;
  const size_t seg = align256(nbh * o.nseg * NP * sizeof(float));
  const size_t z = align256(nbh * o.nseg * (s.dstate / 2) * 2 * sizeof(float));
  o.off_sega = 0;
  o.off_segb = seg;
  o.off_segc = 2 * seg;
  o.off_zf = 3 * seg;
  o.off_zb = 3 * seg + z;
  o.bytes = 3 * seg + 2 * z;
  return o;
}
}  // namespace

size_t m3_scan_backward_workspace_bytes(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  if (s->dstate > 128 || s->headdim > 64) return 0;
  for (const auto& k : kBackwardScratch)
    if (k[0] == s->dtype && k[1] == s->dstate && k[2] == s->headdim && k[3] == s->rank) return 0;
  if (backward_segment(s->rank, s->dstate, s->headdim) == 0) return 0;
  return std::max<size_t>(256, backward_layout(*s).bytes);
}

m3_status m3_scan_backward(const m3_shape* s,
                           const void* x, const void* B, const void* C,
                           const float* dt, const float* A, const float* lam, const float* theta,
                           const float* h0, const void* B_prev, const void* x_prev,
                           const void* dy, const float* dh_out,
                           float* dx, float* dB, float* dC, float* ddt, float* dA, float* dlam,
                           float* dtheta, float* dh0, float* dB_prev, float* dx_prev,
                           void* workspace, size_t workspace_bytes, void* stream) {
  m3_status st = check_common(s, true);
  if (st != M3_OK) return st;
  const int b = s->batch, L = s->seqlen, H = s->nheads, P = s->headdim, N = s->dstate, R = s->rank;
  if ((B_prev == nullptr) != (x_prev == nullptr)) return M3_ERR_NULL;
  if (!B_prev && (dB_prev || dx_prev)) return M3_ERR_NULL;     // no previous write, no gradient of it
  if ((theta == nullptr) != (dtheta == nullptr)) return M3_ERR_NULL;
  const size_t need = m3_scan_backward_workspace_bytes(s);
  if (need == 0) return M3_ERR_SHAPE;
  const size_t bh = (size_t)b * H, tok = bh * L;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (bh == 0) return M3_OK;
  if (!A || !dA) return M3_ERR_NULL;
  if (L > 0 && (!x || !B || !C || !dt || !lam || !dy || !dx || !dB || !dC || !ddt || !dlam))
    return M3_ERR_NULL;
  if (L > 0 && (!workspace || workspace_bytes < need)) return M3_ERR_WORKSPACE;
  const size_t es = esize(s->dtype);
  const size_t sbytes = bh * N * P * sizeof(float);
  struct Buf { const void* p; size_t n; };
  const Buf ins[] = {{x, tok * R * P * es}, {B, tok * R * N * es}, {C, tok * R * N * es},
                     {dt, tok * 4}, {A, (size_t)H * 4}, {lam, tok * 4}, {theta, theta ? tok * (N / 2) * 4 : 0},
                     {h0, h0 ? sbytes : 0}, {B_prev, B_prev ? bh * R * N * es : 0},
                     {x_prev, x_prev ? bh * R * P * es : 0}, {dy, tok * R * P * es}, {dh_out, dh_out ? sbytes : 0},
                     {workspace, L > 0 ? need : 0}};
  const Buf outs[] = {{dx, tok * R * P * 4}, {dB, tok * R * N * 4}, {dC, tok * R * N * 4}, {ddt, tok * 4},
                      {dA, (size_t)H * 4}, {dlam, tok * 4}, {dtheta, dtheta ? tok * (N / 2) * 4 : 0},
                      {dh0, dh0 ? sbytes : 0}, {dB_prev, dB_prev ? bh * R * N * 4 : 0},
                      {dx_prev, dx_prev ? bh * R * P * 4 : 0}};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Buf& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return M3_ERR_ALIAS;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return M3_ERR_ALIAS;
  }
  // dA is a sum over the batch and the tokens: start it at zero (a kernel)
  if (launch_copy_or_zero(dA, nullptr, (size_t)H, hs) != hipSuccess) return M3_ERR_DEVICE;
  if (L == 0) {   // nothing between the incoming state and h_out: dh0 = dh_out
    if (dh0 && launch_copy_or_zero(dh0, dh_out, bh * N * P, hs) != hipSuccess) return M3_ERR_DEVICE;
    if (dB_prev && launch_copy_or_zero(dB_prev, nullptr, bh * R * N, hs) != hipSuccess) return M3_ERR_DEVICE;
    if (dx_prev && launch_copy_or_zero(dx_prev, nullptr, bh * R * P, hs) != hipSuccess) return M3_ERR_DEVICE;
    return M3_OK;
  }
  BackwardParams p;
  p.x = x; p.B = B; p.C = C; p.dt = dt; p.A = A; p.lam = lam; p.theta = theta;
  p.h0 = h0; p.Bp = B_prev; p.xp = x_prev; p.dy = dy; p.dh = dh_out;
  p.dx = dx; p.dB = dB; p.dC = dC; p.ddt = ddt; p.dA = dA; p.dlam = dlam; p.dtheta = dtheta;
  p.dh0 = dh0; p.dBp = dB_prev; p.dxp = dx_prev;
  const BackwardLayout lay = backward_layout(*s);
  char* ws = static_cast<char*>(workspace);
  p.sega = reinterpret_cast<float*>(ws + lay.off_sega);
  p.segb = reinterpret_cast<float*>(ws + lay.off_segb);
  p.segc = reinterpret_cast<float*>(ws + lay.off_segc);
  p.zf = reinterpret_cast<float*>(ws + lay.off_zf);
  p.zb = reinterpret_cast<float*>(ws + lay.off_zb);
  p.batch = b; p.L = L; p.H = H;
  p.S = lay.S; p.nseg = lay.nseg;
  if (launch_backward(p, s->dtype, N, P, R, hs) != hipSuccess) return M3_ERR_DEVICE;
  return M3_OK;
}

m3_status m3_scan_prefill_noalloc(const m3_shape* s,
                                  const void* x, const void* B, const void* C,
                                  const float* dt, const float* A, const float* lam,
                                  const float* theta,
                                  const float* h0, const void* B_prev, const void* x_prev,
                                  void* y, float* h_out, void* stream) {
  static_assert(kNoAllocScratchBytes == (size_t)M3_NOALLOC_SCRATCH_BYTES, "scratch size");
  m3_status st = check_common(s, true);
  if (st != M3_OK) return st;
  if ((size_t)s->batch * s->nheads == 0 || s->seqlen == 0)   // nothing to hand off between chunks
    return m3_scan_prefill(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, y, h_out, nullptr, 0, stream);
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan, 0, 0)) return M3_ERR_SHAPE;
  if (plan.bytes > kNoAllocScratchBytes) return M3_ERR_WORKSPACE;   // larger than the built-in scratch
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return M3_ERR_DEVICE;
  // The buffer keeps the last call's contents: its control word, error word
  // and flags must start at zero, so this call clears them (with a kernel, so
  // that a captured call records no memset node).
  if (launch_copy_or_zero(static_cast<float*>(ws), nullptr, plan.off_recs / sizeof(float),
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return M3_ERR_DEVICE;
  return m3_scan_prefill(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, y, h_out, ws, kNoAllocScratchBytes,
                         stream);
}

m3_status m3_scan_prefill_gated(const m3_shape* s,
                                const void* x, const void* B, const void* C,
                                const float* dt, const float* A, const float* lam,
                                const float* theta,
                                const float* h0, const void* B_prev, const void* x_prev,
                                const void* z, const float* w_y, const float* w_z,
                                void* out, float* h_out,
                                void* workspace, size_t workspace_bytes,
                                void* stream) {
  return prefill_common(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, Gate{true, z, w_y, w_z},
                        kNoPro, out, h_out, workspace, workspace_bytes, stream);
}

m3_status m3_scan_prefill_prologue(const m3_shape* s, const m3_prologue* pro,
                                   const void* x, const void* B, const void* C,
                                   const float* dt, const float* A, const float* lam,
                                   const float* theta,
                                   const float* h0, const void* B_prev, const void* x_prev,
                                   void* y, float* h_out,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!pro) return M3_ERR_NULL;
  const Gate nog{false, nullptr, nullptr, nullptr};
  m3_status st = check_common(s, true);
  if (st != M3_OK) return st;
  PrefillPlan plan;
  const int mode = prologue_mode(*s, &plan);
  const size_t bh = (size_t)s->batch * s->nheads;
  if (mode != M3_PROLOGUE_STAGED || bh == 0 || s->seqlen == 0)   // (no rows to stage: nothing differs)
    return prefill_common(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, nog,
                          Pro{true, pro->eps, pro->bias_B, pro->bias_C}, y, h_out, workspace, workspace_bytes, stream);
  // staged: the prologue kernel, then the plain prefill on its results
  if (!x || !B || !C || !dt || !A || !lam || !y) return M3_ERR_NULL;
  if ((B_prev == nullptr) != (x_prev == nullptr)) return M3_ERR_NULL;
  const StagedLayout lay = staged_layout(*s, plan);
  if (!workspace || workspace_bytes < lay.bytes) return M3_ERR_WORKSPACE;
  const int L = s->seqlen, H = s->nheads, P = s->headdim, N = s->dstate, R = s->rank;
  const size_t es = esize(s->dtype), tok = (size_t)s->batch * L * H;
  const size_t ybytes = tok * R * P * es, sbytes = bh * N * P * sizeof(float);
  // the workspace is written before the prefill reads it: it must not overlap
  // any input, nor y or h_out (which the prefill checks against the inputs it
  // is given, the staged ones; the original B, C, B_prev, angles and bias
  // tables are checked here)
  struct { const void* p; size_t n; } ins[] = {
      {x, tok * R * P * es}, {B, tok * R * N * es}, {C, tok * R * N * es},
      {dt, tok * sizeof(float)}, {A, (size_t)H * sizeof(float)}, {lam, tok * sizeof(float)},
      {theta, theta ? tok * (N / 2) * sizeof(float) : 0}, {h0, h0 ? sbytes : 0},
      {B_prev, bh * R * N * es}, {x_prev, bh * R * P * es},
      {pro->bias_B, pro->bias_B ? (size_t)H * R * N * sizeof(float) : 0},
      {pro->bias_C, pro->bias_C ? (size_t)H * R * N * sizeof(float) : 0}};
  for (const auto& in : ins) {
    if (overlaps(workspace, lay.bytes, in.p, in.n)) return M3_ERR_ALIAS;
    if (overlaps(y, ybytes, in.p, in.n)) return M3_ERR_ALIAS;
    if (h_out && in.p != h0 && overlaps(h_out, sbytes, in.p, in.n)) return M3_ERR_ALIAS;
  }
  if (overlaps(workspace, lay.bytes, y, ybytes) || (h_out && overlaps(workspace, lay.bytes, h_out, sbytes)))
    return M3_ERR_ALIAS;
  char* ws = static_cast<char*>(workspace);
  PrologueStage ps;
  ps.dtype = s->dtype; ps.N = N; ps.H = H; ps.R = R;
  ps.tokens = tok; ps.pairs = bh; ps.eps = pro->eps;
  ps.B = B; ps.C = C; ps.Bp = B_prev; ps.dt = dt; ps.theta = theta;
  ps.biasB = pro->bias_B; ps.biasC = pro->bias_C;
  ps.Bn = ws + lay.off_B; ps.Cn = ws + lay.off_C;
  ps.Bpn = B_prev ? ws + lay.off_Bp : nullptr;
  ps.phi = theta ? reinterpret_cast<float*>(ws + lay.off_phi) : nullptr;
  if (launch_prologue_stage(ps, static_cast<hipStream_t>(stream)) != hipSuccess) return M3_ERR_DEVICE;
  return prefill_common(s, x, ps.Bn, ps.Cn, dt, A, lam, ps.phi, h0, ps.Bpn, x_prev, nog, kNoPro, y, h_out,
                        workspace, plan.bytes, stream);
}

const char* m3_status_str(m3_status st) {
  // read as an integer: a C caller may pass any int, which would not be a
  // valid value of the enum type in this C++ translation unit
  static_assert(sizeof(m3_status) == sizeof(int32_t), "status width");
  int32_t v;
  std::memcpy(&v, &st, sizeof v);
  switch (v) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "a required pointer is NULL";
    case M3_ERR_SHAPE: return "invalid or unsupported shape";
    case M3_ERR_DTYPE: return "unknown dtype";
    case M3_ERR_WORKSPACE: return "workspace missing or too small";
    case M3_ERR_DEVICE: return "HIP launch failed";
    case M3_ERR_ALIAS: return "an output aliases an input";
    case M3_ERR_TIMEOUT: return "a prefill look-back wait gave up (outputs of the affected chunks are NaN)";
  }
  return "unknown status";
}

int32_t m3_version(void) { return 100; }

}  // extern "C"
