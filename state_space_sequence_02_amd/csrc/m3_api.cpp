// m3_api.cpp -- the extern "C" boundary of libm3.so (declared in include/m3.h).
//
// Host-side only: validates shapes, pointers, dtype, workspace size and
// aliasing before anything is enqueued, plans the chunking and workspace, and
// hands off to the launchers.  No allocation, no synchronisation, no exceptions.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "m3_internal.h"

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

// Tokens per chunk: the requested value (or a default of 128 (token, rank)
// rows for N <= 64 and 256 rows above),
// rounded down to a power of two in [16, 256], then halved until the chunk's
// rows and angles fit the kernel's register budget and its LDS tiles fit on a
// compute unit.
size_t lds_need(int q, const m3_shape& s) {
  return fused_lds_bytes(q, s.rank, s.dstate, s.headdim, (int)esize(s.dtype));
}

int choose_chunk(const m3_shape& s) {
  // default: 128 (token, rank) rows per chunk for N <= 64, 256 above (the
  // state hand-off per chunk grows with N; so does the work that amortises it)
  const int rows = s.dstate <= 64 ? 128 : 256;
  int q = s.chunk > 0 ? s.chunk : std::max(16, rows / s.rank);
  int p2 = 16;
  while (p2 * 2 <= q && p2 < 256) p2 *= 2;
  q = std::max(16, std::min(p2, 256));
  while (q > 16 && (q * s.rank > fused_max_rows(s.dstate) || q * (s.dstate / 2) > kFusedAngleCap))
    q /= 2;
  while (q > 16 && lds_need(q, s) > (size_t)kLdsBudget) q /= 2;
  if (lds_need(q, s) > (size_t)kLdsBudget) return 0;
  return q;
}

}  // namespace

bool plan_prefill(const m3_shape& s, PrefillPlan* plan) {
  // N = 256 is decode-only: its prefill kernels spill 76-708 bytes per lane to
  // scratch, and a memory fault was seen in one of them whose cause is not
  // established, so that path is not built.
  if (s.dstate > 128) return false;
  const int q = choose_chunk(s);
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
  plan->lds = lds_need(q, s);
  return true;
}

}  // namespace m3

using namespace m3;

extern "C" {

size_t m3_prefill_workspace_bytes(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan)) return 0;
  return plan.bytes;
}

int32_t m3_prefill_chunk_used(const m3_shape* s) {
  if (check_common(s, true) != M3_OK) return 0;
  PrefillPlan plan;
  if (!plan_prefill(*s, &plan)) return 0;
  return plan.Q;
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
  if (!plan_prefill(*s, &plan)) return M3_ERR_SHAPE;
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
  // the prologue's bias tables take LDS of their own; the prologue runs with
  // one 16-row output tile per wave only (its variants with two or more
  // spilled 40-96 bytes per lane to scratch, and one of them made a memory
  // fault whose cause is not established), and not for fp32 inputs at
  // N = 128 (those kernels spill 60-324 bytes per lane; one of them made a
  // memory fault whose cause is not established either)
  size_t lds = plan.lds;
  if (pro.on) {
    if (s->dtype == M3_FP32 && N >= 128) return M3_ERR_SHAPE;
    const int waves = fused_threads(N) / 64;
    const int tiles = (plan.Q * R + 31) / 32 * 2;
    if ((tiles + waves - 1) / waves > 1) return M3_ERR_SHAPE;
    lds = fused_lds_bytes(plan.Q, R, N, P, (int)es, 1);
    if (lds > (size_t)kLdsBudget) return M3_ERR_SHAPE;
  }
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
  f.flags = reinterpret_cast<unsigned long long*>(ws + plan.off_flags);
  f.recs = reinterpret_cast<float*>(ws + plan.off_recs);
  f.maps = reinterpret_cast<float*>(ws + plan.off_maps);
  f.states = reinterpret_cast<float*>(ws + plan.off_states);
  f.batch = b; f.L = L; f.H = H; f.N = N; f.P = P; f.R = R; f.logR = ilog2(R);
  f.Q = plan.Q; f.nc = plan.nc;
  f.use_maps = 1;   // (the launch decides from the device's resident workgroups)
  if (launch_fused_prefill(f, lds, s->dtype, hs) != hipSuccess) return M3_ERR_DEVICE;
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
  return prefill_common(s, x, B, C, dt, A, lam, theta, h0, B_prev, x_prev, Gate{false, nullptr, nullptr, nullptr},
                        Pro{true, pro->eps, pro->bias_B, pro->bias_C}, y, h_out, workspace, workspace_bytes, stream);
}

const char* m3_status_str(m3_status st) {
  switch (st) {
    case M3_OK: return "ok";
    case M3_ERR_NULL: return "a required pointer is NULL";
    case M3_ERR_SHAPE: return "invalid or unsupported shape";
    case M3_ERR_DTYPE: return "unknown dtype";
    case M3_ERR_WORKSPACE: return "workspace missing or too small";
    case M3_ERR_DEVICE: return "HIP launch failed";
    case M3_ERR_ALIAS: return "an output aliases an input";
  }
  return "unknown status";
}

int32_t m3_version(void) { return 100; }

}  // extern "C"
