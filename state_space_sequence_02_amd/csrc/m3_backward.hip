// m3_backward.hip -- gradients of the Mamba-3 recurrence (m3_scan_backward).
//
// The forward map is the prefill's, per (sequence, head), t = 0..L-1 (Mamba-3
// explainer panels 1, 3, 4; paper page Table 1 caption):
//   H_t = R(phi_t) [alpha_t H_{t-1} + beta_t V_{t-1}] + gamma_t V_t,  V_t = B_t X_t^T,  Y_t = H_t^T C_t.
// Its vector-Jacobian product runs the recurrence backwards (the explainer's
// training remark: the same recurrence, differentiated):
//   G_t  = C_t dY_t^T + alpha_{t+1} R(phi_{t+1})^T G_{t+1}   (+ dH at t = L-1)
//   Q_t  = R(phi_t)^T G_t,   dV_t = gamma_t G_t + beta_{t+1} Q_{t+1}
//   dC_t = H_t dY_t,  dB_t = dV_t X_t,  dX_t = dV_t^T B_t
//   d alpha_t = <Q_t, H_{t-1}>,  d beta_t = <Q_t, V_{t-1}>,  d gamma_t = <G_t, V_t>
//   d phi_t[k] = sum_p (G_t[2k+1,p] K_t[2k,p] - G_t[2k,p] K_t[2k+1,p]),  K_t = H_t - gamma_t V_t
//   d h0 = alpha_0 Q_0,  dV_{-1} = beta_0 Q_0 (-> d B_prev, d x_prev)
// and the coefficients' chain rule into dt, lam and A.
//
// Segment-parallel.  The transition alpha_t R(phi_t) is one complex scalar per
// row pair, so over a segment of S tokens each direction is a local result
// plus a per-pair propagator times what enters from outside:
//   forward:  H_{s1} = U_j + [prod_{t=s0..s1} alpha_t R(phi_t)] H_{s0-1}
//   backward: G_{s0} = G~_j + [prod_{t=s0+1..s1+1} alpha_t R(phi_t)^T] G_{s1+1}
// (U_j, G~_j: the segment's own result with zero entering).  Six launches:
//  1. fwd_maps_kernel   per (segment, sequence, head): U_j and its propagator;
//  2. fwd_combine_kernel per (sequence, head), over the segments in order: the
//     state entering each segment;
//  3. states_kernel     per segment: the recurrence from its entering state,
//     storing every H_t (fp32) in the workspace [b, H, L, N, P];
//  4. bwd_maps_kernel   per segment: G~_j and its propagator;
//  5. bwd_combine_kernel per (sequence, head), over the segments in reverse: the
//     G entering each segment from the right;
//  6. grads_kernel      per segment: t = s1..s0 with G carried in registers from
//     the entering G, reading H_t back from the workspace, writing every
//     gradient of the segment's tokens (the first segment also d h0, d B_prev,
//     d x_prev; every segment adds its part of dA with one atomic).
// The propagators are accumulated step by step as complex products (unit
// rotations times decays), not from summed angles.
#include "m3_device.h"

namespace m3 {
namespace {

constexpr int bwd_units(int N, int P) { return (N / 2) * (P / 4); }
constexpr int bwd_threads(int N, int P) {
  return bwd_units(N, P) >= 512 ? 512 : (bwd_units(N, P) + 63) / 64 * 64;
}

template <typename T> __device__ __forceinline__ float ld1(const T* p) { return to_f(*p); }

// Two consecutive elements (a row pair's entries of one rank) / four (a quad).
__device__ __forceinline__ float2 ld2(const float* p) { return *reinterpret_cast<const float2*>(p); }
__device__ __forceinline__ float2 ld2(const bf16* p) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

__device__ __forceinline__ float4 f4(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float4 fma4(float a, float4 x, float4 y) {
  return make_float4(fmaf(a, x.x, y.x), fmaf(a, x.y, y.y), fmaf(a, x.z, y.z), fmaf(a, x.w, y.w));
}
__device__ __forceinline__ float4 mul4(float a, float4 x) { return make_float4(a * x.x, a * x.y, a * x.z, a * x.w); }
__device__ __forceinline__ float4 addv(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 subv(float4 a, float4 b) { return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w); }
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

// The row pair (r0, r1) turned by (c, s): R = [[c, -s], [s, c]].
__device__ __forceinline__ void rot(float c, float s, float4& r0, float4& r1) {
  const float4 a = r0, b = r1;
  r0 = make_float4(c * a.x - s * b.x, c * a.y - s * b.y, c * a.z - s * b.z, c * a.w - s * b.w);
  r1 = make_float4(s * a.x + c * b.x, s * a.y + c * b.y, s * a.z + c * b.z, s * a.w + c * b.w);
}

// Write V = sum_r B[r, (2k, 2k+1)] X[r, quad] of one unit (the two rows).
template <int R>
__device__ __forceinline__ void vwrite(const float2 (&b)[R], const float4 (&xq)[R], float4& v0, float4& v1) {
  v0 = f4(0.f);
  v1 = f4(0.f);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    v0 = fma4(b[r].x, xq[r], v0);
    v1 = fma4(b[r].y, xq[r], v1);
  }
}

// Segment j of work item blockIdx.x = j * (b*H) + (sequence, head).
struct Seg {
  int j, bh, b, h, s0, s1;
};
__device__ __forceinline__ Seg segment_of(const BackwardParams& p) {
  Seg g;
  const int nbh = p.batch * p.H;
  g.j = blockIdx.x / nbh;
  g.bh = blockIdx.x - g.j * nbh;
  g.b = g.bh / p.H;
  g.h = g.bh - g.b * p.H;
  g.s0 = g.j * p.S;
  g.s1 = min(p.L, g.s0 + p.S) - 1;
  return g;
}

// The write of the token before s0 (B_prev / x_prev, or zeros, before token 0)
// for the unit's pair k and quad q.
template <typename T, int N, int P, int R>
__device__ __forceinline__ void prev_write(const BackwardParams& p, const Seg& g, size_t tok0, int k, int q,
                                           float4& v0, float4& v1) {
  const T* Bm = g.s0 > 0 ? static_cast<const T*>(p.B) + (tok0 + (size_t)(g.s0 - 1) * p.H) * R * N
                         : (p.Bp ? static_cast<const T*>(p.Bp) + (size_t)g.bh * R * N : nullptr);
  const T* Xm = g.s0 > 0 ? static_cast<const T*>(p.x) + (tok0 + (size_t)(g.s0 - 1) * p.H) * R * P
                         : (p.xp ? static_cast<const T*>(p.xp) + (size_t)g.bh * R * P : nullptr);
  float4 xq[R];
  float2 bq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    xq[r] = Xm ? ld4(Xm + r * P + 4 * q) : f4(0.f);
    bq[r] = Bm ? ld2(Bm + r * N + 2 * k) : make_float2(0.f, 0.f);
  }
  vwrite<R>(bq, xq, v0, v1);
}

// One forward step of a unit: H <- R(phi)[alpha H + beta V_prev] + gamma V_t.
template <typename T, int N, int P, int R>
__device__ __forceinline__ void fwd_step(const T* Bt, const float4 (&xq)[R], int k, float al, float be, float ga,
                                         float c, float s, float4& H0, float4& H1, float4& V0, float4& V1) {
  float2 bq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) bq[r] = ld2(Bt + r * N + 2 * k);
  float4 w0, w1;
  vwrite<R>(bq, xq, w0, w1);
  float4 m0 = fma4(be, V0, mul4(al, H0)), m1 = fma4(be, V1, mul4(al, H1));
  rot(c, s, m0, m1);
  H0 = fma4(ga, w0, m0);
  H1 = fma4(ga, w1, m1);
  V0 = w0;
  V1 = w1;
}

// 1. The segment's end state from a zero entering state (its previous write
// included) and the product of its alpha_t R(phi_t) per pair.
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(bwd_threads(N, P)) void fwd_maps_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT;
  const Seg g = segment_of(p);
  const int tid = threadIdx.x, q = tid % QP;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h;
  const float Ah = p.A[g.h];
  float4 H0[UPT], H1[UPT], V0[UPT], V1[UPT];
  float zr[UPT], zi[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT, k = (u < UNITS ? u : 0) / QP;
    H0[i] = H1[i] = f4(0.f);
    prev_write<T, N, P, R>(p, g, tok0, k, q, V0[i], V1[i]);
    zr[i] = 1.f;
    zi[i] = 0.f;
  }
  for (int t = g.s0; t <= g.s1; ++t) {
    const size_t tok = tok0 + (size_t)t * p.H;
    const float d = p.dt[tok], lm = p.lam[tok];
    const float al = __expf(d * Ah), be = (1.f - lm) * d * al, ga = lm * d;
    const T* Bt = static_cast<const T*>(p.B) + tok * R * N;
    const T* Xt = static_cast<const T*>(p.x) + tok * R * P;
    float4 xq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xq[r] = ld4(Xt + r * P + 4 * q);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= UNITS) continue;
      const int k = u / QP;
      float c = 1.f, sn = 0.f;
      if (p.theta) __sincosf(p.theta[tok * (N / 2) + k], &sn, &c);
      fwd_step<T, N, P, R>(Bt, xq, k, al, be, ga, c, sn, H0[i], H1[i], V0[i], V1[i]);
      const float r0 = zr[i];
      zr[i] = al * (r0 * c - zi[i] * sn);
      zi[i] = al * (r0 * sn + zi[i] * c);
    }
  }
  const size_t slot = (size_t)g.bh * p.nseg + g.j;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u >= UNITS) continue;
    const int k = u / QP;
    float* row = p.sega + (slot * N + 2 * k) * P + 4 * q;
    *reinterpret_cast<float4*>(row) = H0[i];
    *reinterpret_cast<float4*>(row + P) = H1[i];
    if (q == 0) *reinterpret_cast<float2*>(p.zf + (slot * (N / 2) + k) * 2) = make_float2(zr[i], zi[i]);
  }
}

// 2. The state entering each segment, segment by segment:
//   S_{-1} = h0 (or 0),  entering_j = S_{j-1},  S_j = z_j S_{j-1} + U_j.
template <int N, int P>
__global__ __launch_bounds__(bwd_threads(N, P)) void fwd_combine_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT;
  const int bh = blockIdx.x, tid = threadIdx.x, q = tid % QP;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u >= UNITS) continue;
    const int k = u / QP;
    const size_t r0 = (size_t)(2 * k) * P + 4 * q;
    float4 S0 = p.h0 ? ld4(p.h0 + (size_t)bh * N * P + r0) : f4(0.f);
    float4 S1 = p.h0 ? ld4(p.h0 + (size_t)bh * N * P + r0 + P) : f4(0.f);
    for (int j = 0; j < p.nseg; ++j) {
      const size_t slot = (size_t)bh * p.nseg + j;
      float* e = p.segb + slot * N * P + r0;
      *reinterpret_cast<float4*>(e) = S0;
      *reinterpret_cast<float4*>(e + P) = S1;
      if (j + 1 < p.nseg) {
        const float2 z = *reinterpret_cast<const float2*>(p.zf + (slot * (N / 2) + k) * 2);
        const float* U = p.sega + slot * N * P + r0;
        rot(z.x, z.y, S0, S1);
        S0 = addv(S0, ld4(U));
        S1 = addv(S1, ld4(U + P));
      }
    }
  }
}

// 3. The recurrence over the segment from its entering state, every H_t stored.
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(bwd_threads(N, P)) void states_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT;
  const Seg g = segment_of(p);
  const int tid = threadIdx.x, q = tid % QP;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h;
  const float Ah = p.A[g.h];
  const size_t slot = (size_t)g.bh * p.nseg + g.j;
  float4 H0[UPT], H1[UPT], V0[UPT], V1[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT, k = (u < UNITS ? u : 0) / QP;
    const float* e = p.segb + (slot * N + 2 * k) * P + 4 * q;
    H0[i] = ld4(e);
    H1[i] = ld4(e + P);
    prev_write<T, N, P, R>(p, g, tok0, k, q, V0[i], V1[i]);
  }
  float* hs = p.hs + (size_t)g.bh * p.L * N * P;
  for (int t = g.s0; t <= g.s1; ++t) {
    const size_t tok = tok0 + (size_t)t * p.H;
    const float d = p.dt[tok], lm = p.lam[tok];
    const float al = __expf(d * Ah), be = (1.f - lm) * d * al, ga = lm * d;
    const T* Bt = static_cast<const T*>(p.B) + tok * R * N;
    const T* Xt = static_cast<const T*>(p.x) + tok * R * P;
    float4 xq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xq[r] = ld4(Xt + r * P + 4 * q);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= UNITS) continue;
      const int k = u / QP;
      float c = 1.f, sn = 0.f;
      if (p.theta) __sincosf(p.theta[tok * (N / 2) + k], &sn, &c);
      fwd_step<T, N, P, R>(Bt, xq, k, al, be, ga, c, sn, H0[i], H1[i], V0[i], V1[i]);
      float* row = hs + ((size_t)t * N + 2 * k) * P + 4 * q;
      *reinterpret_cast<float4*>(row) = H0[i];
      *reinterpret_cast<float4*>(row + P) = H1[i];
    }
  }
}

// 4. The segment's G at its first token from a zero G entering at its end (the
// last segment starts from dh_out), and the product of alpha_u R(phi_u)^T,
// u = s0+1 .. s1+1, per pair.
template <typename T, int N, int P, int R>
__global__ __launch_bounds__(bwd_threads(N, P)) void bwd_maps_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT;
  const Seg g = segment_of(p);
  const int tid = threadIdx.x, q = tid % QP;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h;
  const float Ah = p.A[g.h];
  const bool last = g.j == p.nseg - 1;
  float4 G0[UPT], G1[UPT];
  float wr[UPT], wi[UPT];
  // coefficients of the token after the segment (none after the last token)
  float a_n = 1.f;
  const bool next = g.s1 + 1 < p.L;
  const size_t tokn = tok0 + (size_t)(next ? g.s1 + 1 : g.s1) * p.H;
  if (next) a_n = __expf(p.dt[tokn] * Ah);
  float cn[UPT], sn[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT, k = (u < UNITS ? u : 0) / QP;
    G0[i] = G1[i] = f4(0.f);
    if (last && p.dh) {
      G0[i] = ld4(p.dh + ((size_t)g.bh * N + 2 * k) * P + 4 * q);
      G1[i] = ld4(p.dh + ((size_t)g.bh * N + 2 * k + 1) * P + 4 * q);
    }
    cn[i] = 1.f;
    sn[i] = 0.f;
    if (next && p.theta) __sincosf(p.theta[tokn * (N / 2) + k], &sn[i], &cn[i]);
    wr[i] = 1.f;
    wi[i] = 0.f;
  }
  for (int t = g.s1; t >= g.s0; --t) {
    const size_t tok = tok0 + (size_t)t * p.H;
    const T* Ct = static_cast<const T*>(p.C) + tok * R * N;
    const T* dYt = static_cast<const T*>(p.dy) + tok * R * P;
    float4 dyq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dyq[r] = ld4(dYt + r * P + 4 * q);
    const float al = __expf(p.dt[tok] * Ah);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= UNITS) continue;
      const int k = u / QP;
      // G_t = C_t dY_t^T + alpha_{t+1} R(phi_{t+1})^T G_{t+1}
      rot(cn[i], -sn[i], G0[i], G1[i]);
      G0[i] = mul4(a_n, G0[i]);
      G1[i] = mul4(a_n, G1[i]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float2 cq = ld2(Ct + r * N + 2 * k);
        G0[i] = fma4(cq.x, dyq[r], G0[i]);
        G1[i] = fma4(cq.y, dyq[r], G1[i]);
      }
      const float r0 = wr[i];
      wr[i] = a_n * (r0 * cn[i] + wi[i] * sn[i]);
      wi[i] = a_n * (wi[i] * cn[i] - r0 * sn[i]);
      float c = 1.f, s = 0.f;
      if (p.theta) __sincosf(p.theta[tok * (N / 2) + k], &s, &c);
      cn[i] = c;
      sn[i] = s;
    }
    a_n = al;
  }
  const size_t slot = (size_t)g.bh * p.nseg + g.j;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u >= UNITS) continue;
    const int k = u / QP;
    float* row = p.sega + (slot * N + 2 * k) * P + 4 * q;
    *reinterpret_cast<float4*>(row) = G0[i];
    *reinterpret_cast<float4*>(row + P) = G1[i];
    if (q == 0) *reinterpret_cast<float2*>(p.zb + (slot * (N / 2) + k) * 2) = make_float2(wr[i], wi[i]);
  }
}

// 5. The G entering each segment from the right, last segment first:
//   E_last = 0,  E_{j-1} = G~_j + w_j E_j.
template <int N, int P>
__global__ __launch_bounds__(bwd_threads(N, P)) void bwd_combine_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT;
  const int bh = blockIdx.x, tid = threadIdx.x, q = tid % QP;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u >= UNITS) continue;
    const int k = u / QP;
    const size_t r0 = (size_t)(2 * k) * P + 4 * q;
    float4 E0 = f4(0.f), E1 = f4(0.f);
    for (int j = p.nseg - 1; j >= 0; --j) {
      const size_t slot = (size_t)bh * p.nseg + j;
      float* e = p.segb + slot * N * P + r0;
      *reinterpret_cast<float4*>(e) = E0;
      *reinterpret_cast<float4*>(e + P) = E1;
      if (j > 0) {
        const float2 w = *reinterpret_cast<const float2*>(p.zb + (slot * (N / 2) + k) * 2);
        const float* Gl = p.sega + slot * N * P + r0;
        rot(w.x, w.y, E0, E1);
        E0 = addv(E0, ld4(Gl));
        E1 = addv(E1, ld4(Gl + P));
      }
    }
  }
}

template <typename T, int N, int P, int R>
__global__ __launch_bounds__(bwd_threads(N, P)) void grads_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P);
  constexpr int UPT = (UNITS + NT - 1) / NT, NW = NT / 64;
  const Seg g = segment_of(p);
  const int bh = g.bh, h = g.h;
  const int tid = threadIdx.x, q = tid % QP, lane = tid & 63, wave = tid >> 6;
  const int L = p.L;
  const size_t tstep = (size_t)p.H;
  const size_t tok0 = (size_t)g.b * L * p.H + h;
  const float Ah = p.A[h];
  const bool last = g.j == p.nseg - 1;
  __shared__ float s_dx[2][NW][R * P];   // dX partial sums per wave (by step parity)
  __shared__ float s_sc[2][NW][4];       // d alpha, d beta, d gamma partials per wave
  const float* hs = p.hs + (size_t)bh * L * N * P;
  const T* Bp = p.Bp ? static_cast<const T*>(p.Bp) + (size_t)bh * R * N : nullptr;
  const T* Xp = p.xp ? static_cast<const T*>(p.xp) + (size_t)bh * R * P : nullptr;

  // carried from step t + 1: G, Q, alpha, beta, phi; and of step t: H_t, V_t, B_t, X_t
  float4 G0[UPT], G1[UPT], Q0[UPT], Q1[UPT], H0[UPT], H1[UPT], V0[UPT], V1[UPT];
  float2 Bc[UPT][R];
  float4 Xc[R];
  float cn[UPT], sn[UPT];   // cos / sin of phi_{t+1} of each unit's pair
  // Entering the segment's last token s1: for the sequence's last token, G_L =
  // dH with a unit coefficient and no turn; otherwise G_{s1+1} (from the
  // combine) with token s1+1's alpha, beta and phi, and Q_{s1+1} = R(phi)^T G.
  float a_n = 1.f, b_n = 0.f, dA_acc = 0.f;
  if (!last) {
    const size_t tokn = tok0 + (size_t)(g.s1 + 1) * tstep;
    const float dn = p.dt[tokn], ln = p.lam[tokn];
    a_n = __expf(dn * Ah);
    b_n = (1.f - ln) * dn * a_n;
  }
  {
    const size_t tok = tok0 + (size_t)g.s1 * tstep;
    const T* Bt = static_cast<const T*>(p.B) + tok * R * N;
    const T* Xt = static_cast<const T*>(p.x) + tok * R * P;
    const size_t slot = (size_t)bh * p.nseg + g.j;
#pragma unroll
    for (int r = 0; r < R; ++r) Xc[r] = ld4(Xt + r * P + 4 * q);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT, k = (u < UNITS ? u : 0) / QP;
#pragma unroll
      for (int r = 0; r < R; ++r) Bc[i][r] = ld2(Bt + r * N + 2 * k);
      vwrite<R>(Bc[i], Xc, V0[i], V1[i]);
      const float* row = hs + ((size_t)g.s1 * N + 2 * k) * P + 4 * q;
      H0[i] = ld4(row);
      H1[i] = ld4(row + P);
      G0[i] = G1[i] = Q0[i] = Q1[i] = f4(0.f);
      cn[i] = 1.f;
      sn[i] = 0.f;
      if (last) {
        if (p.dh) {   // dH enters G_{L-1}
          G0[i] = ld4(p.dh + ((size_t)bh * N + 2 * k) * P + 4 * q);
          G1[i] = ld4(p.dh + ((size_t)bh * N + 2 * k + 1) * P + 4 * q);
        }
      } else {
        const float* e = p.segb + (slot * N + 2 * k) * P + 4 * q;
        G0[i] = ld4(e);
        G1[i] = ld4(e + P);
        if (p.theta) __sincosf(p.theta[(tok + tstep) * (N / 2) + k], &sn[i], &cn[i]);
        Q0[i] = G0[i];
        Q1[i] = G1[i];
        rot(cn[i], -sn[i], Q0[i], Q1[i]);
      }
    }
  }
  for (int t = g.s1; t >= g.s0; --t) {
    const size_t tok = tok0 + (size_t)t * tstep;
    const float d = p.dt[tok], lm = p.lam[tok];
    const float al = __expf(d * Ah), be = (1.f - lm) * d * al, ga = lm * d;
    const T* Ct = static_cast<const T*>(p.C) + tok * R * N;
    const T* dYt = static_cast<const T*>(p.dy) + tok * R * P;
    // the previous token's B, X (B_prev, x_prev or zeros at t = 0) and H_{t-1}
    const T* Bm = t > 0 ? static_cast<const T*>(p.B) + (tok - tstep) * R * N : Bp;
    const T* Xm = t > 0 ? static_cast<const T*>(p.x) + (tok - tstep) * R * P : Xp;
    float4 dyq[R], xm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dyq[r] = ld4(dYt + r * P + 4 * q);
      xm[r] = Xm ? ld4(Xm + r * P + 4 * q) : f4(0.f);
    }
    float4 dxq[R];   // this thread's sum over its units of dV^T B (columns of its quad)
#pragma unroll
    for (int r = 0; r < R; ++r) dxq[r] = f4(0.f);
    float sa = 0.f, sb = 0.f, sg = 0.f;
    float2 Bm_u[UPT][R];
    float4 Hm0[UPT], Hm1[UPT], Vm0[UPT], Vm1[UPT];
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      const bool live = u < UNITS;
      const int k = (live ? u : 0) / QP;
      float c = 1.f, s = 0.f;
      if (p.theta) __sincosf(p.theta[tok * (N / 2) + k], &s, &c);
      // G_t = C_t dY_t^T + alpha_{t+1} R(phi_{t+1})^T G_{t+1}
      float4 g0 = G0[i], g1 = G1[i];
      rot(cn[i], -sn[i], g0, g1);
      g0 = mul4(a_n, g0);
      g1 = mul4(a_n, g1);
      float2 cq[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        cq[r] = ld2(Ct + r * N + 2 * k);
        g0 = fma4(cq[r].x, dyq[r], g0);
        g1 = fma4(cq[r].y, dyq[r], g1);
      }
      float4 qq0 = g0, qq1 = g1;
      rot(c, -s, qq0, qq1);
      // dV_t = gamma_t G_t + beta_{t+1} Q_{t+1}
      const float4 dv0 = fma4(b_n, Q0[i], mul4(ga, g0)), dv1 = fma4(b_n, Q1[i], mul4(ga, g1));
      // H_{t-1}, V_{t-1}
      if (t > 0) {
        const float* row = hs + ((size_t)(t - 1) * N + 2 * k) * P + 4 * q;
        Hm0[i] = ld4(row);
        Hm1[i] = ld4(row + P);
      } else {
        Hm0[i] = p.h0 ? ld4(p.h0 + ((size_t)bh * N + 2 * k) * P + 4 * q) : f4(0.f);
        Hm1[i] = p.h0 ? ld4(p.h0 + ((size_t)bh * N + 2 * k + 1) * P + 4 * q) : f4(0.f);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) Bm_u[i][r] = Bm ? ld2(Bm + r * N + 2 * k) : make_float2(0.f, 0.f);
      vwrite<R>(Bm_u[i], xm, Vm0[i], Vm1[i]);
      // column sums of this unit: dC (rows 2k, 2k+1 per rank), dB, d phi
      float pc[2 * R], pb[2 * R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        pc[2 * r] = dot4(H0[i], dyq[r]);
        pc[2 * r + 1] = dot4(H1[i], dyq[r]);
        pb[2 * r] = dot4(dv0, Xc[r]);
        pb[2 * r + 1] = dot4(dv1, Xc[r]);
        if (live) {
          dxq[r] = fma4(Bc[i][r].x, dv0, dxq[r]);
          dxq[r] = fma4(Bc[i][r].y, dv1, dxq[r]);
        }
      }
      const float4 k0 = subv(H0[i], mul4(ga, V0[i])), k1 = subv(H1[i], mul4(ga, V1[i]));
      float pphi = dot4(g1, k0) - dot4(g0, k1);
      if (live) {
        sa += dot4(qq0, Hm0[i]) + dot4(qq1, Hm1[i]);
        sb += dot4(qq0, Vm0[i]) + dot4(qq1, Vm1[i]);
        sg += dot4(g0, V0[i]) + dot4(g1, V1[i]);
      } else {
        pphi = 0.f;
#pragma unroll
        for (int e = 0; e < 2 * R; ++e) pc[e] = pb[e] = 0.f;
      }
      // sums over the pair's QP quads (consecutive lanes)
#pragma unroll
      for (int off = 1; off < QP; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 2 * R; ++e) {
          pc[e] += __shfl_xor(pc[e], off);
          pb[e] += __shfl_xor(pb[e], off);
        }
        pphi += __shfl_xor(pphi, off);
      }
      if (live && q == 0) {
        float* dCt = p.dC + tok * R * N;
        float* dBt = p.dB + tok * R * N;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          *reinterpret_cast<float2*>(dCt + r * N + 2 * k) = make_float2(pc[2 * r], pc[2 * r + 1]);
          *reinterpret_cast<float2*>(dBt + r * N + 2 * k) = make_float2(pb[2 * r], pb[2 * r + 1]);
        }
        if (p.dtheta) p.dtheta[tok * (N / 2) + k] = pphi;
      }
      // carry to step t - 1
      G0[i] = g0;
      G1[i] = g1;
      Q0[i] = qq0;
      Q1[i] = qq1;
      cn[i] = c;
      sn[i] = s;
    }
    // sums over the state rows: lanes holding the same quad, then the waves
#pragma unroll
    for (int off = QP; off < 64; off <<= 1) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        dxq[r].x += __shfl_xor(dxq[r].x, off);
        dxq[r].y += __shfl_xor(dxq[r].y, off);
        dxq[r].z += __shfl_xor(dxq[r].z, off);
        dxq[r].w += __shfl_xor(dxq[r].w, off);
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      sa += __shfl_xor(sa, off);
      sb += __shfl_xor(sb, off);
      sg += __shfl_xor(sg, off);
    }
    const int par = t & 1;
    if (lane < QP) {
#pragma unroll
      for (int r = 0; r < R; ++r) *reinterpret_cast<float4*>(&s_dx[par][wave][r * P + 4 * lane]) = dxq[r];
    }
    if (lane == 0) {
      s_sc[par][wave][0] = sa;
      s_sc[par][wave][1] = sb;
      s_sc[par][wave][2] = sg;
    }
    __syncthreads();
    float* dXt = p.dx + tok * R * P;
    for (int j = tid; j < R * P; j += NT) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_dx[par][w][j];
      dXt[j] = v;
    }
    if (tid == 0) {
      float da = 0.f, db = 0.f, dg = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        da += s_sc[par][w][0];
        db += s_sc[par][w][1];
        dg += s_sc[par][w][2];
      }
      p.ddt[tok] = da * Ah * al + db * (1.f - lm) * al * (1.f + d * Ah) + dg * lm;
      p.dlam[tok] = -db * d * al + dg * d;
      dA_acc += da * d * al + db * (1.f - lm) * d * d * al;
    }
    // step t - 1 sees: alpha_t, beta_t, and H_{t-1}, V_{t-1}, B_{t-1}, X_{t-1} as its own
    a_n = al;
    b_n = be;
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      H0[i] = Hm0[i];
      H1[i] = Hm1[i];
      V0[i] = Vm0[i];
      V1[i] = Vm1[i];
#pragma unroll
      for (int r = 0; r < R; ++r) Bc[i][r] = Bm_u[i][r];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) Xc[r] = xm[r];
  }
  if (g.j != 0) {   // the token before s0 belongs to the previous segment
    if (tid == 0) atomicAdd(p.dA + h, dA_acc);
    return;
  }
  // d h0 = alpha_0 Q_0;  dV_{-1} = beta_0 Q_0 -> d B_prev, d x_prev
  float4 dxq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) dxq[r] = f4(0.f);
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    const bool live = u < UNITS;
    const int k = (live ? u : 0) / QP;
    if (live && p.dh0) {
      *reinterpret_cast<float4*>(p.dh0 + ((size_t)bh * N + 2 * k) * P + 4 * q) = mul4(a_n, Q0[i]);
      *reinterpret_cast<float4*>(p.dh0 + ((size_t)bh * N + 2 * k + 1) * P + 4 * q) = mul4(a_n, Q1[i]);
    }
    const float4 dv0 = mul4(b_n, Q0[i]), dv1 = mul4(b_n, Q1[i]);
    float pb[2 * R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      pb[2 * r] = live ? dot4(dv0, Xc[r]) : 0.f;
      pb[2 * r + 1] = live ? dot4(dv1, Xc[r]) : 0.f;
      if (live) {
        dxq[r] = fma4(Bc[i][r].x, dv0, dxq[r]);
        dxq[r] = fma4(Bc[i][r].y, dv1, dxq[r]);
      }
    }
#pragma unroll
    for (int off = 1; off < QP; off <<= 1)
#pragma unroll
      for (int e = 0; e < 2 * R; ++e) pb[e] += __shfl_xor(pb[e], off);
    if (live && q == 0 && p.dBp) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        *reinterpret_cast<float2*>(p.dBp + ((size_t)bh * R + r) * N + 2 * k) = make_float2(pb[2 * r], pb[2 * r + 1]);
    }
  }
#pragma unroll
  for (int off = QP; off < 64; off <<= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      dxq[r].x += __shfl_xor(dxq[r].x, off);
      dxq[r].y += __shfl_xor(dxq[r].y, off);
      dxq[r].z += __shfl_xor(dxq[r].z, off);
      dxq[r].w += __shfl_xor(dxq[r].w, off);
    }
  }
  __syncthreads();
  if (lane < QP) {
#pragma unroll
    for (int r = 0; r < R; ++r) *reinterpret_cast<float4*>(&s_dx[0][wave][r * P + 4 * lane]) = dxq[r];
  }
  __syncthreads();
  if (p.dxp) {
    for (int j = tid; j < R * P; j += NT) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += s_dx[0][w][j];
      p.dxp[(size_t)bh * R * P + j] = v;
    }
  }
  if (tid == 0) atomicAdd(p.dA + h, dA_acc);
}

}  // namespace
}  // namespace m3

namespace m3 {
namespace {

template <typename T, int N, int P, int R>
hipError_t run_backward(const BackwardParams& p, hipStream_t s) {
  const unsigned nbh = (unsigned)(p.batch * p.H), nsg = nbh * (unsigned)p.nseg;
  const dim3 blk(bwd_threads(N, P));
  hipLaunchKernelGGL((fwd_maps_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  hipLaunchKernelGGL((fwd_combine_kernel<N, P>), dim3(nbh), blk, 0, s, p);
  hipLaunchKernelGGL((states_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  hipLaunchKernelGGL((bwd_maps_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  hipLaunchKernelGGL((bwd_combine_kernel<N, P>), dim3(nbh), blk, 0, s, p);
  hipLaunchKernelGGL((grads_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  return hipGetLastError();
}

template <typename T, int N, int P>
hipError_t bwd_r(const BackwardParams& p, int R, hipStream_t s) {
  switch (R) {
    case 1: return run_backward<T, N, P, 1>(p, s);
    case 2: return run_backward<T, N, P, 2>(p, s);
    case 4: return run_backward<T, N, P, 4>(p, s);
    case 8: return run_backward<T, N, P, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int N>
hipError_t bwd_p(const BackwardParams& p, int P, int R, hipStream_t s) {
  switch (P) {
    case 16: return bwd_r<T, N, 16>(p, R, s);
    case 32: return bwd_r<T, N, 32>(p, R, s);
    case 64: return bwd_r<T, N, 64>(p, R, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t bwd_n(const BackwardParams& p, int N, int P, int R, hipStream_t s) {
  switch (N) {
    case 16: return bwd_p<T, 16>(p, P, R, s);
    case 32: return bwd_p<T, 32>(p, P, R, s);
    case 64: return bwd_p<T, 64>(p, P, R, s);
    case 128: return bwd_p<T, 128>(p, P, R, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_backward(const BackwardParams& p, int dtype, int N, int P, int R, hipStream_t s) {
  if (p.batch == 0 || p.H == 0 || p.L == 0) return hipSuccess;
  return dtype == M3_BF16 ? bwd_n<bf16>(p, N, P, R, s) : bwd_n<float>(p, N, P, R, s);
}

}  // namespace m3
