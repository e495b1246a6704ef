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
// Segment-parallel, in the segments' matrix form.  The transition
// alpha_t R(phi_t) is one complex scalar per row pair, so over a segment of S
// tokens each direction is a local result plus a per-pair propagator times what
// enters from outside:
//   forward:  H_{s1} = U_j + [prod_{t=s0..s1} alpha_t R(phi_t)] H_{s0-1}
//   backward: G_{s0} = G~_j + [prod_{t=s0+1..s1+1} alpha_t R(phi_t)^T] G_{s1+1}
// (U_j, G~_j: the segment's own result with zero entering).  Five launches:
//  1. fwd_maps_kernel   per (segment, sequence, head): U_j and its propagator;
//  2. fwd_combine_kernel per (sequence, head), over the segments in order: the
//     state entering each segment;
//  3. bwd_maps_kernel   per segment: G~_j and its propagator;
//  4. bwd_combine_kernel per (sequence, head), over the segments in reverse: the
//     G entering each segment from the right;
//  5. chunk_grads_kernel per segment: every gradient of the segment's tokens
//     from its entering state and entering G, in the chunked (matrix) form of
//     the recurrence -- pairwise products of the segment's rows in LDS -- so no
//     per-token state is stored anywhere (the first segment also writes d h0,
//     d B_prev, d x_prev; every segment adds its part of dA with one atomic).
// The propagators are accumulated step by step as complex products (unit
// rotations times decays), not from summed angles.
#include <atomic>

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

// Copies the rows of tokens s0..s1 of one (sequence, head) -- `width`
// elements of T per token, at global token index tok0 + t * H -- into LDS
// [s1 - s0 + 1][width], in 16-byte pieces spread over the block's NT threads.
// Every load is issued before any is used, so a segment's token loop pays one
// memory latency instead of one per token.
template <typename T, int NT>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, size_t tok0, int H, int s0, int s1, int width) {
  const int cpr = width * (int)sizeof(T) / 16;   // pieces per row
  const int n = (s1 - s0 + 1) * cpr;
  for (int i = threadIdx.x; i < n; i += NT) {
    const int t = i / cpr, c = i - t * cpr;
    reinterpret_cast<uint4*>(dst + (size_t)t * width)[c] =
        reinterpret_cast<const uint4*>(src + (tok0 + (size_t)(s0 + t) * H) * width)[c];
  }
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
  constexpr int SM = backward_segment(R, N, P);   // tokens per segment (p.S)
  __shared__ __align__(16) T sB[SM * R * N];
  __shared__ __align__(16) T sX[SM * R * P];
  __shared__ __align__(16) float sTh[SM * (N / 2)];
  __shared__ float sD[SM], sL[SM];
  const Seg g = segment_of(p);
  const int tid = threadIdx.x, q = tid % QP;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h;
  const float Ah = p.A[g.h];
  // the segment's operands, all loads in flight at once
  stage_rows<T, NT>(sB, static_cast<const T*>(p.B), tok0, p.H, g.s0, g.s1, R * N);
  stage_rows<T, NT>(sX, static_cast<const T*>(p.x), tok0, p.H, g.s0, g.s1, R * P);
  if (p.theta) stage_rows<float, NT>(sTh, p.theta, tok0, p.H, g.s0, g.s1, N / 2);
  if (tid <= g.s1 - g.s0) {
    sD[tid] = p.dt[tok0 + (size_t)(g.s0 + tid) * p.H];
    sL[tid] = p.lam[tok0 + (size_t)(g.s0 + tid) * p.H];
  }
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
  __syncthreads();
  for (int t = g.s0; t <= g.s1; ++t) {
    const int lt = t - g.s0;
    const float d = sD[lt], lm = sL[lt];
    const float al = __expf(d * Ah), be = (1.f - lm) * d * al, ga = lm * d;
    const T* Bt = sB + lt * R * N;
    const T* Xt = sX + lt * R * P;
    float4 xq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xq[r] = ld4(Xt + r * P + 4 * q);
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + i * NT;
      if (u >= UNITS) continue;
      const int k = u / QP;
      float c = 1.f, sn = 0.f;
      if (p.theta) __sincosf(sTh[lt * (N / 2) + k], &sn, &c);
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
// One thread per unit (a (b, h)'s units spread over kCombSlices(N, P)
// workgroups), the next kCombAhead segments' z and U in flight in registers:
// the chain's only wait is on the arithmetic, not on a load per segment.
constexpr int kCombAhead = 4;
template <int N, int P>
constexpr int comb_slices() { return (bwd_units(N, P) + bwd_threads(N, P) - 1) / bwd_threads(N, P); }

template <int N, int P>
__global__ __launch_bounds__(bwd_threads(N, P)) void fwd_combine_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P), SL = comb_slices<N, P>();
  constexpr int D = kCombAhead;
  const int bh = blockIdx.x / SL, u = (blockIdx.x % SL) * NT + threadIdx.x, q = threadIdx.x % QP;
  if (u >= UNITS) return;
  const int k = u / QP;
  const size_t r0 = (size_t)(2 * k) * P + 4 * q;
  const int ns = p.nseg;
  auto zof = [&](int j) { return *reinterpret_cast<const float2*>(p.zf + (((size_t)bh * ns + j) * (N / 2) + k) * 2); };
  auto uof = [&](int j) { return p.sega + ((size_t)bh * ns + j) * N * P + r0; };
  float2 zq[D];
  float4 u0[D], u1[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < ns - 1) {
      zq[d] = zof(d);
      u0[d] = ld4(uof(d));
      u1[d] = ld4(uof(d) + P);
    }
  float4 S0 = p.h0 ? ld4(p.h0 + (size_t)bh * N * P + r0) : f4(0.f);
  float4 S1 = p.h0 ? ld4(p.h0 + (size_t)bh * N * P + r0 + P) : f4(0.f);
  for (int j0 = 0; j0 < ns; j0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 + d;
      if (j >= ns) break;
      float* e = p.segb + ((size_t)bh * ns + j) * N * P + r0;
      *reinterpret_cast<float4*>(e) = S0;
      *reinterpret_cast<float4*>(e + P) = S1;
      if (j + 1 < ns) {   // segment j's map (in slot d), then slot d takes segment j + D
        rot(zq[d].x, zq[d].y, S0, S1);
        S0 = addv(S0, u0[d]);
        S1 = addv(S1, u1[d]);
        if (j + D < ns - 1) {
          zq[d] = zof(j + D);
          u0[d] = ld4(uof(j + D));
          u1[d] = ld4(uof(j + D) + P);
        }
      }
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
  constexpr int SM = backward_segment(R, N, P);   // tokens per segment (p.S)
  __shared__ __align__(16) T sC[SM * R * N];
  __shared__ __align__(16) T sY[SM * R * P];
  __shared__ __align__(16) float sTh[SM * (N / 2)];
  __shared__ float sD[SM];
  const Seg g = segment_of(p);
  const int tid = threadIdx.x, q = tid % QP;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h;
  const float Ah = p.A[g.h];
  const bool last = g.j == p.nseg - 1;
  // the segment's operands, all loads in flight at once
  stage_rows<T, NT>(sC, static_cast<const T*>(p.C), tok0, p.H, g.s0, g.s1, R * N);
  stage_rows<T, NT>(sY, static_cast<const T*>(p.dy), tok0, p.H, g.s0, g.s1, R * P);
  if (p.theta) stage_rows<float, NT>(sTh, p.theta, tok0, p.H, g.s0, g.s1, N / 2);
  if (tid <= g.s1 - g.s0) sD[tid] = p.dt[tok0 + (size_t)(g.s0 + tid) * p.H];
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
  __syncthreads();
  for (int t = g.s1; t >= g.s0; --t) {
    const int lt = t - g.s0;
    const T* Ct = sC + lt * R * N;
    const T* dYt = sY + lt * R * P;
    float4 dyq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dyq[r] = ld4(dYt + r * P + 4 * q);
    const float al = __expf(sD[lt] * Ah);
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
      if (p.theta) __sincosf(sTh[lt * (N / 2) + k], &s, &c);
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
//   E_last = 0,  E_{j-1} = G~_j + w_j E_j.  (Spread and prefetched as step 2.)
template <int N, int P>
__global__ __launch_bounds__(bwd_threads(N, P)) void bwd_combine_kernel(BackwardParams p) {
  constexpr int NT = bwd_threads(N, P), QP = P / 4, UNITS = bwd_units(N, P), SL = comb_slices<N, P>();
  constexpr int D = kCombAhead;
  const int bh = blockIdx.x / SL, u = (blockIdx.x % SL) * NT + threadIdx.x, q = threadIdx.x % QP;
  if (u >= UNITS) return;
  const int k = u / QP;
  const size_t r0 = (size_t)(2 * k) * P + 4 * q;
  const int ns = p.nseg;
  auto wof = [&](int j) { return *reinterpret_cast<const float2*>(p.zb + (((size_t)bh * ns + j) * (N / 2) + k) * 2); };
  auto gof = [&](int j) { return p.sega + ((size_t)bh * ns + j) * N * P + r0; };
  float2 wq[D];
  float4 g0[D], g1[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (ns - 1 - d > 0) {   // segments ns - 1, ns - 2, ... (segment 0's map is not used)
      wq[d] = wof(ns - 1 - d);
      g0[d] = ld4(gof(ns - 1 - d));
      g1[d] = ld4(gof(ns - 1 - d) + P);
    }
  float4 E0 = f4(0.f), E1 = f4(0.f);
  for (int i0 = 0; i0 < ns; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = ns - 1 - (i0 + d);
      if (j < 0) break;
      float* e = p.segc + ((size_t)bh * ns + j) * N * P + r0;
      *reinterpret_cast<float4*>(e) = E0;
      *reinterpret_cast<float4*>(e + P) = E1;
      if (j > 0) {   // segment j's map (in slot d), then slot d takes segment j - D
        rot(wq[d].x, wq[d].y, E0, E1);
        E0 = addv(E0, g0[d]);
        E1 = addv(E1, g1[d]);
        if (j - D > 0) {
          wq[d] = wof(j - D);
          g0[d] = ld4(gof(j - D));
          g1[d] = ld4(gof(j - D) + P);
        }
      }
    }
  }
}

// 6. Every gradient of one segment's tokens, in the segment's matrix form (no
// per-token state).  In the segment's frame (t, s index its n tokens; l_t =
// sum_{u<=t} dt_u A and Phi_t = sum_{u<=t} phi_u from its first token; B~ =
// R(-Phi) B, C~ = R(-Phi) C; delta = (1 - lam) dt, gamma = lam dt;
// w_ts = gamma_s + [s < t] delta_{s+1}):
//   H_t = e^{l_t} R(Phi_t) K_t,   K_t = S0' + sum_{s<=t} e^{-l_s} w_ts B~_s X_s^T,
//   S0' = H_{s0-1} + delta_0 V_{s0-1},   Y_t = e^{l_t} K_t^T C~_t.
// The gradient of the segment's last state from the right is dH_end
// (alpha_n R(phi_n)^T G_{s1+1}, or dh_out for the last segment) and of its last
// write (beta_n / alpha_n) R(Phi_end) D'; with D' = R(-Phi_end) dH_end,
// f_ts = e^{l_t - l_s} w_ts and om_s = e^{l_end - l_s} w_{end,s}:
//   dB~_s = sum_{t>=s} f_ts (dY_t . X_s) C~_t + om_s D' X_s
//   dX_s  = sum_{t>=s} f_ts (C~_t . B~_s) dY_t + om_s D'^T B~_s
//   dC~_t = e^{l_t} S0' dY_t + sum_{s<=t} f_ts (X_s . dY_t) B~_s
//   dB = R(Phi) dB~, dC = R(Phi) dC~,  dS0' = sum_t e^{l_t} C~_t dY_t^T + e^{l_end} D'
// (every exponent a difference l_t - l_s <= 0), and the scalars through l, w
// and Phi: with Om_ts = e^{l_t - l_s} sum (C~_t . B~_s)(dY_t . X_s) (all rank
// pairs), Omend_s = e^{l_end - l_s} <D', B~_s X_s^T>, I_t = e^{l_t} <C~_t dY_t^T, S0'>,
// Iend = e^{l_end} <D', S0'>:
//   dl_t = I_t + sum_{s<=t} w_ts Om_ts - sum_{t'>=t} w_t't Om_t't - w_end,t Omend_t
//          + [t = end] (Iend + sum_s w_end,s Omend_s)
//   d gamma_s = sum_{t>=s} Om_ts + Omend_s,  d delta_{s+1} = sum_{t>s} Om_ts + Omend_s,
//   d delta_0 = <dS0', V_{s0-1}>,
//   dPhi_t[k] = J(dB~_t, B~_t) + J(dC~_t, C~_t) + [t = end] <K_end, J D>,
// J(u, v) = u_{2k} v_{2k+1} - u_{2k+1} v_{2k} per pair; then dt, lam, A and the
// angles by their definitions (suffix sums over the segment for l and Phi).
// One workgroup per (segment, sequence, head), everything in LDS as fp32; the
// row-by-row products (C~ B~^T, dY X^T, and the five products of the gradient
// formulas above) run as 16x16 fp32 MFMA tiles (v_mfma_f32_16x16x4_f32).
// Threads of the segment kernel: 512 (two waves per SIMD beside the one
// workgroup the LDS allows per CU, so one wave's LDS and MFMA waits overlap
// another's: 12% faster than 256 at the SISO and MIMO shapes), except at
// N = 128 with R = 1, 2 or 8, whose variants would then exceed the 256
// registers a lane gets and spill; those keep 256.
constexpr int grads_threads(int N, int R) { return (N <= 64 || R == 4) ? 512 : 256; }
constexpr int kTok = 16;   // per-token LDS fields

// 16x16 output tile of A B^T over a contraction of K (a multiple of 32):
// A rows m0.., B rows n0.., both with the contraction contiguous.  Lane holds
// C[m0 + 4 (lane/16) + i][n0 + lane % 16], i = 0..3.
__device__ __forceinline__ f32x4 mm_rr(const float* A, int lda, int m0, const float* B, int ldb, int n0, int K,
                                       f32x4 acc) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 32) {
    Frag<float> a, b;
    frag_lds8(a, A + (m0 + r) * lda + k0 + 8 * g);
    frag_lds8(b, B + (n0 + r) * ldb + k0 + 8 * g);
    acc = mma(a, b, acc);
  }
  return acc;
}
// The same with B stored the other way round: B operand (n, k) = Bt[k][n].
__device__ __forceinline__ f32x4 mm_rc(const float* A, int lda, int m0, const float* Bt, int ldbt, int n0, int K,
                                       f32x4 acc) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 32) {
    Frag<float> a, b;
    frag_lds8(a, A + (m0 + r) * lda + k0 + 8 * g);
#pragma unroll
    for (int j = 0; j < 8; ++j) b.v[j] = Bt[(k0 + 8 * g + j) * ldbt + n0 + r];
    acc = mma(a, b, acc);
  }
  return acc;
}
// Both stored the other way round, B scaled per contraction index by sc[k]:
// A operand (m, k) = At[k][m], B operand (n, k) = sc[k] Bt[k][n].
__device__ __forceinline__ f32x4 mm_cc(const float* At, int ldat, int m0, const float* Bt, int ldbt, int n0,
                                       const float* sc, int scs, int K, f32x4 acc) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  for (int k0 = 0; k0 < K; k0 += 32) {
    Frag<float> a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + 8 * g + j;
      a.v[j] = At[k * ldat + m0 + r];
      b.v[j] = sc[k * scs] * Bt[k * ldbt + n0 + r];
    }
    acc = mma(a, b, acc);
  }
  return acc;
}

// Per-(token, pair) sums over the rows a lane holds in a 16-row output tile:
// rows m0 + 4 (lane/16) + i are (token, rank) = (row / R, row % R).  Returns
// through `add(t, v)` one call per token the lane's 4 rows touch, after
// combining with the lane group that holds the token's other ranks (R = 8).
template <int R, typename F>
__device__ __forceinline__ void per_token(int m0, const float (&v)[4], F add) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  if constexpr (R <= 4) {
#pragma unroll
    for (int i0 = 0; i0 < 4; i0 += R) {
      float s = 0.f;
#pragma unroll
      for (int i = i0; i < i0 + R; ++i) s += v[i];
      add((m0 + 4 * g + i0) / R, s);
    }
  } else {
    float s = v[0] + v[1] + v[2] + v[3];
    s += __shfl_xor(s, 16);
    if ((g & 1) == 0) add((m0 + 4 * g) / R, s);
  }
}

template <typename T, int N, int P, int R>
__global__ __launch_bounds__(grads_threads(N, R)) void chunk_grads_kernel(BackwardParams p) {
  constexpr int NT = grads_threads(N, R), NH = N / 2;
  constexpr int NS = N < 32 ? 32 : N, PS = P < 32 ? 32 : P;   // LDS row strides (contractions padded to 32)
  extern __shared__ __align__(16) float sm[];
  const Seg g = segment_of(p);
  const int n = g.s1 - g.s0 + 1, M = n * R;
  constexpr int Q = backward_segment(R, N, P);   // tokens per segment (the host sets p.S to it)
  static_assert(Q >= 1 && Q <= 32 && (Q & (Q - 1)) == 0, "segment length");
  constexpr BwdLds o = bwd_lds(Q, R, N, P);
  constexpr int MK = (int)o.MK;   // rows of the row arrays, and the contraction over rows (multiple of 32)
  float* sB = sm + o.B;   // B~ [MK][NS]
  float* sC = sm + o.C;   // C~ [MK][NS]
  float* sX = sm + o.X;   // X [MK][PS]
  float* sY = sm + o.Y;   // dY [MK][PS]
  float* sS = sm + o.S;   // S0' [N][PS], later dS0'
  float* sD = sm + o.D;   // D' [N][PS]
  float* sG1 = sm + o.G1;   // f_ts (dY . X)   [(t r')][(s r)]
  float* sG1T = sm + o.G1T; // its transpose
  float* sG2T = sm + o.G2T; // f_ts (C~ . B~)  transposed: [(s r)][(t r')]
  float* sPR = sm + o.PR;   // e^{l_t - l_s} (C~ . B~)(dY . X)
  float* sOm = sm + o.OM;   // Om_ts [Q][Q]
  float2* sCS = reinterpret_cast<float2*>(sm + o.CS);   // cos/sin Phi_t [Q][N/2]
  float2* sCN = reinterpret_cast<float2*>(sm + o.CN);   // cos/sin (Phi_end + phi_n) [N/2]
  float* sTK = sm + o.TK;   // per-token fields [Q][kTok]
  float* sPA = sm + o.PA;   // J(dB~, B~) summed over ranks [Q][N/2]
  float* sPC = sm + o.PC;   // J(dC~, C~) summed over ranks
  float* sPB = sm + o.PB;   // <B~, D' X> summed over ranks and the pair's rows
  float* sPK = sm + o.PK;   // om J(B~, D' X) (the K_end . J D source part)
  float* sPI = sm + o.PI;   // C~ . (S0' dY) (I_t parts)
  float* sBm = sm + o.BM;   // previous write's B [R][N]
  float* sXm = sm + o.XM;   // previous write's X [R][P]
  float* sRD = sm + o.RD;   // block reduction scratch and scalars
  float* sEL = sm + o.EL;   // e^{l_t} of each row (t = row / R; 0 past the segment's rows)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 15, lg = lane >> 4;
  constexpr int NW = NT / 64;
  static_assert(N % 8 == 0 && P % 8 == 0, "row widths");
  const size_t tstep = (size_t)p.H;
  const size_t tok0 = (size_t)g.b * p.L * p.H + g.h + (size_t)g.s0 * tstep;   // the segment's first token
  const float Ah = p.A[g.h];
  const bool last = g.j == p.nseg - 1;
  const size_t slot = (size_t)g.bh * p.nseg + g.j;
  enum { kL = 0, kEl, kGam, kDlt, kDt, kLam, kWend, kOmw, kRowT, kColT, kColOm, kColOmS, kDl, kDg, kDd, kTend };

  // (a) every global read of the segment is issued before any of them is used:
  // token scalars, angles, the rows of B, C, X and dY, the previous write, the
  // entering state and the gradient entering from the right.  Lanes past the
  // segment read a valid address and drop the value.
  constexpr int NB8 = N / 8, NP8 = P / 8, P4 = P / 4;
  constexpr int U_BC = MK * NB8, I_BC = (U_BC + NT - 1) / NT;
  constexpr int U_XY = MK * NP8, I_XY = (U_XY + NT - 1) / NT;
  constexpr int U_S = N * P4, I_S = (U_S + NT - 1) / NT;      // float4 units of S0'
  constexpr int U_D = NH * P4, I_D = (U_D + NT - 1) / NT;     // pair-row float4 units of D'
  constexpr int U_TH = NH * Q, I_TH = (U_TH + NT - 1) / NT;   // (pair, token), token fastest
  constexpr int I_BM = (R * N + NT - 1) / NT, I_XM = (R * P + NT - 1) / NT;
  const T* gB = static_cast<const T*>(p.B);
  const T* gC = static_cast<const T*>(p.C);
  const T* gX = static_cast<const T*>(p.x);
  const T* gY = static_cast<const T*>(p.dy);
  const float* gTh = p.theta ? p.theta : p.dt;
  const bool has_th = p.theta != nullptr;
  float dtv = 0.f, lmv = 0.f, dtn = 0.f, lmn = 0.f;
  {
    const int t = tid < n ? tid : 0;
    dtv = p.dt[tok0 + (size_t)t * tstep];
    lmv = p.lam[tok0 + (size_t)t * tstep];
    if (!last) {
      dtn = p.dt[tok0 + (size_t)n * tstep];
      lmn = p.lam[tok0 + (size_t)n * tstep];
    }
    if (tid >= n) dtv = lmv = 0.f;
  }
  float thv[I_TH];
#pragma unroll
  for (int i = 0; i < I_TH; ++i) {
    const int e = tid + i * NT, k = e / Q, t = e - k * Q;
    const bool ok = has_th && e < U_TH && t < n;
    const float v = gTh[ok ? (tok0 + (size_t)t * tstep) * NH + k : 0];
    thv[i] = ok ? v : 0.f;
  }
  float rb[I_BC][8], rc[I_BC][8], rx[I_XY][8], ry[I_XY][8];
#pragma unroll
  for (int i = 0; i < I_BC; ++i) {
    const int u = tid + i * NT, row = u / NB8, j = u - row * NB8;
    const bool ok = u < U_BC && row < M;
    const int rr = ok ? row : 0, jj = ok ? j : 0, t = rr / R;
    const size_t off = (tok0 + (size_t)t * tstep) * R * N + (size_t)(rr - t * R) * N + 8 * jj;
    load8(gB + off, rb[i]);
    load8(gC + off, rc[i]);
  }
#pragma unroll
  for (int i = 0; i < I_XY; ++i) {
    const int u = tid + i * NT, row = u / NP8, j = u - row * NP8;
    const bool ok = u < U_XY && row < M;
    const int rr = ok ? row : 0, jj = ok ? j : 0, t = rr / R;
    const size_t off = (tok0 + (size_t)t * tstep) * R * P + (size_t)(rr - t * R) * P + 8 * jj;
    load8(gX + off, rx[i]);
    load8(gY + off, ry[i]);
  }
  const T* Bm = g.s0 > 0 ? gB + (tok0 - tstep) * R * N
                         : (p.Bp ? static_cast<const T*>(p.Bp) + (size_t)g.bh * R * N : nullptr);
  const T* Xm = g.s0 > 0 ? gX + (tok0 - tstep) * R * P
                         : (p.xp ? static_cast<const T*>(p.xp) + (size_t)g.bh * R * P : nullptr);
  float bm[I_BM], xm[I_XM];
#pragma unroll
  for (int i = 0; i < I_BM; ++i) {
    const int e = tid + i * NT;
    bm[i] = Bm ? to_f(Bm[e < R * N ? e : 0]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < I_XM; ++i) {
    const int e = tid + i * NT;
    xm[i] = Xm ? to_f(Xm[e < R * P ? e : 0]) : 0.f;
  }
  const float* Hin = p.segb + slot * N * P;
  float4 hv[I_S];
#pragma unroll
  for (int i = 0; i < I_S; ++i) {
    const int u = tid + i * NT;
    hv[i] = *reinterpret_cast<const float4*>(Hin + 4 * (u < U_S ? u : 0));
  }
  // D' source: dh at the sequence's end, else the gradient E that the backward
  // combine left for this segment (times alpha of the next token)
  const float* Dsrc = last ? (p.dh ? p.dh + (size_t)g.bh * N * P : nullptr) : p.segc + slot * N * P;
  float4 dv0[I_D], dv1[I_D];
  float thn[I_D];
#pragma unroll
  for (int i = 0; i < I_D; ++i) {
    const int u = tid + i * NT, uu = u < U_D ? u : 0, k = uu / P4, c4 = uu - k * P4;
    if (Dsrc) {
      dv0[i] = *reinterpret_cast<const float4*>(Dsrc + (2 * k) * P + 4 * c4);
      dv1[i] = *reinterpret_cast<const float4*>(Dsrc + (2 * k + 1) * P + 4 * c4);
    } else {
      dv0[i] = dv1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const bool okn = has_th && !last;
    const float v = gTh[okn ? (tok0 + (size_t)n * tstep) * NH + k : 0];
    thn[i] = okn ? v : 0.f;
  }

  // token scalars: inclusive prefix of l = sum dt A over the segment on wave 0
  // (Q <= 64 tokens); tokens past the segment get zeros
  if (wave == 0) {
    float l = dtv * Ah;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(l, d);
      if (lane >= d) l += y;
    }
    if (lane < Q) {
      float* k = sTK + lane * kTok;
      const bool in = lane < n;
      k[kL] = in ? l : 0.f;
      k[kEl] = in ? __expf(l) : 0.f;
      k[kGam] = lmv * dtv;
      k[kDlt] = (1.f - lmv) * dtv;
      k[kDt] = dtv;
      k[kLam] = lmv;
    }
    if (lane == 0) {
      sRD[256] = last ? 1.f : __expf(dtn * Ah);   // alpha of the next token
      sRD[257] = last ? 0.f : (1.f - lmn) * dtn;  // its beta / alpha
    }
  }
  // angles: Phi_t[k] = sum_{u<=t} phi_u[k], a prefix over each group of Q lanes
#pragma unroll
  for (int i = 0; i < I_TH; ++i) {
    const int e = tid + i * NT, k = e / Q, t = e - k * Q;
    float v = thv[i];
#pragma unroll
    for (int d = 1; d < Q; d <<= 1) {
      const float y = __shfl_up(v, d, Q);
      if (t >= d) v += y;
    }
    if (e < U_TH && t < n) {
      float sn, cs;
      sincosf(v, &sn, &cs);
      sCS[t * NH + k] = make_float2(cs, sn);
      if (t == n - 1) sCN[k] = make_float2(v, 0.f);   // Phi_end, turned into cos/sin below
    }
  }
#pragma unroll
  for (int i = 0; i < I_BM; ++i)
    if (tid + i * NT < R * N) sBm[tid + i * NT] = bm[i];
#pragma unroll
  for (int i = 0; i < I_XM; ++i)
    if (tid + i * NT < R * P) sXm[tid + i * NT] = xm[i];
  __syncthreads();

  // (b) LDS images, zero past the segment's rows and the real columns:
  // B~, C~ turned by -Phi_t, X, dY, S0' = H_{s0-1} + delta_0 V_{s0-1}, D' = R(-Phi_end) dH_end
#pragma unroll
  for (int i = 0; i < I_BC; ++i) {
    const int u = tid + i * NT, row = u / NB8, j = u - row * NB8;
    if (u < U_BC) {
      const bool ok = row < M;
      const int t = ok ? row / R : 0;
      float ob[8], oc[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float2 cs = sCS[t * NH + 4 * j + q];
        const float b0 = rb[i][2 * q], b1 = rb[i][2 * q + 1], c0 = rc[i][2 * q], c1 = rc[i][2 * q + 1];
        ob[2 * q] = ok ? cs.x * b0 + cs.y * b1 : 0.f;
        ob[2 * q + 1] = ok ? -cs.y * b0 + cs.x * b1 : 0.f;
        oc[2 * q] = ok ? cs.x * c0 + cs.y * c1 : 0.f;
        oc[2 * q + 1] = ok ? -cs.y * c0 + cs.x * c1 : 0.f;
      }
      float4* db = reinterpret_cast<float4*>(sB + row * NS + 8 * j);
      float4* dc = reinterpret_cast<float4*>(sC + row * NS + 8 * j);
      db[0] = make_float4(ob[0], ob[1], ob[2], ob[3]);
      db[1] = make_float4(ob[4], ob[5], ob[6], ob[7]);
      dc[0] = make_float4(oc[0], oc[1], oc[2], oc[3]);
      dc[1] = make_float4(oc[4], oc[5], oc[6], oc[7]);
    }
  }
#pragma unroll
  for (int i = 0; i < I_XY; ++i) {
    const int u = tid + i * NT, row = u / NP8, j = u - row * NP8;
    if (u < U_XY) {
      const bool ok = row < M;
      float4* dx = reinterpret_cast<float4*>(sX + row * PS + 8 * j);
      float4* dy = reinterpret_cast<float4*>(sY + row * PS + 8 * j);
      dx[0] = ok ? make_float4(rx[i][0], rx[i][1], rx[i][2], rx[i][3]) : make_float4(0.f, 0.f, 0.f, 0.f);
      dx[1] = ok ? make_float4(rx[i][4], rx[i][5], rx[i][6], rx[i][7]) : make_float4(0.f, 0.f, 0.f, 0.f);
      dy[0] = ok ? make_float4(ry[i][0], ry[i][1], ry[i][2], ry[i][3]) : make_float4(0.f, 0.f, 0.f, 0.f);
      dy[1] = ok ? make_float4(ry[i][4], ry[i][5], ry[i][6], ry[i][7]) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  {
    const float dlt0 = sTK[kDlt];
#pragma unroll
    for (int i = 0; i < I_S; ++i) {
      const int u = tid + i * NT, nn = u / P4, c = 4 * (u - nn * P4);
      if (u < U_S) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float b = sBm[r * N + nn];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] += b * sXm[r * P + c + q];
        }
        *reinterpret_cast<float4*>(sS + nn * PS + c) =
            make_float4(hv[i].x + dlt0 * v[0], hv[i].y + dlt0 * v[1], hv[i].z + dlt0 * v[2], hv[i].w + dlt0 * v[3]);
      }
    }
    const float an = sRD[256];
#pragma unroll
    for (int i = 0; i < I_D; ++i) {
      const int u = tid + i * NT, k = u / P4, c = 4 * (u - k * P4);
      if (u < U_D) {
        float2 cs;
        if (last) {
          cs = sCS[(n - 1) * NH + k];
        } else {
          float sn, cn_;
          sincosf(sCN[k].x + thn[i], &sn, &cn_);
          cs = make_float2(cn_, sn);
        }
        const float a0[4] = {an * dv0[i].x, an * dv0[i].y, an * dv0[i].z, an * dv0[i].w};
        const float a1[4] = {an * dv1[i].x, an * dv1[i].y, an * dv1[i].z, an * dv1[i].w};
        float d0[4], d1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          d0[q] = cs.x * a0[q] + cs.y * a1[q];
          d1[q] = -cs.y * a0[q] + cs.x * a1[q];
        }
        *reinterpret_cast<float4*>(sD + (2 * k) * PS + c) = make_float4(d0[0], d0[1], d0[2], d0[3]);
        *reinterpret_cast<float4*>(sD + (2 * k + 1) * PS + c) = make_float4(d1[0], d1[1], d1[2], d1[3]);
      }
    }
    // padding: columns of B~ / C~ past N, of X / dY / S0' / D' past P, rows of S0' / D' past N
    if constexpr (NS != N) {
      for (int e = tid; e < MK * (NS - N); e += NT) {
        const int row = e / (NS - N), c = N + e - row * (NS - N);
        sB[row * NS + c] = 0.f;
        sC[row * NS + c] = 0.f;
      }
    }
    if constexpr (PS != P) {
      for (int e = tid; e < MK * (PS - P); e += NT) {
        const int row = e / (PS - P), c = P + e - row * (PS - P);
        sX[row * PS + c] = 0.f;
        sY[row * PS + c] = 0.f;
      }
    }
    for (int e = tid; e < NS * PS; e += NT) {
      const int nn = e / PS, c = e - nn * PS;
      if (nn >= N || c >= P) {
        sS[e] = 0.f;
        sD[e] = 0.f;
      }
    }
    for (int e = tid; e < MK; e += NT) sEL[e] = e < M ? sTK[(e / R) * kTok + kEl] : 0.f;
  }
  __syncthreads();
  const float l_end = sTK[(n - 1) * kTok + kL];
  const float eend = __expf(l_end);
  const float cn = sRD[257];
  for (int t = tid; t < n; t += NT) {
    float* k = sTK + t * kTok;
    const float w = k[kGam] + (t < n - 1 ? sTK[(t + 1) * kTok + kDlt] : 0.f);
    k[kWend] = w;
    k[kOmw] = __expf(l_end - k[kL]) * w;
  }
  // (c) pairwise row products on MFMA: C~ B~^T and dY X^T, 16x16 blocks (t-block >= s-block)
  const int nb = MK / 16;
  for (int job = wave; job < nb * nb; job += NW) {
    const int tb = job / nb, sb = job - tb * nb;
    f32x4 cb = zero4(), dx = zero4();
    if (sb <= tb) {
      cb = mm_rr(sC, NS, tb * 16, sB, NS, sb * 16, NS, cb);
      dx = mm_rr(sY, PS, tb * 16, sX, PS, sb * 16, PS, dx);
    }
    const int sr = sb * 16 + lr, s = sr / R;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = tb * 16 + 4 * lg + i, t = tr / R;
      float g1 = 0.f, g2 = 0.f, pr = 0.f;
      if (tr < M && sr < M && s <= t) {
        const float el = __expf(sTK[t * kTok + kL] - sTK[s * kTok + kL]);
        const float w = sTK[s * kTok + kGam] + (s < t ? sTK[(s + 1) * kTok + kDlt] : 0.f);
        g1 = el * w * dx[i];
        g2 = el * w * cb[i];
        pr = el * cb[i] * dx[i];
      }
      sG1[tr * MK + sr] = g1;
      sG1T[sr * MK + tr] = g1;
      sG2T[sr * MK + tr] = g2;
      sPR[tr * MK + sr] = pr;
    }
  }
  __syncthreads();
  for (int e = tid; e < Q * Q; e += NT) {
    const int t = e / Q, s = e - t * Q;
    float om = 0.f;
    if (s <= t && t < n) {
#pragma unroll
      for (int a = 0; a < R; ++a)
#pragma unroll
        for (int c = 0; c < R; ++c) om += sPR[(t * R + a) * MK + s * R + c];
    }
    sOm[e] = om;
  }
  __syncthreads();
  // row and column sums of Om (zero past the segment's tokens):
  //   rowT_u = sum_s w_us Om_us,  colOm_u = sum_t Om_tu,  colOmS_u = sum_{t>u} Om_tu,
  //   colT_u = sum_t w_tu Om_tu = gamma_u colOm_u + delta_{u+1} colOmS_u
  for (int u = tid; u < n; u += NT) {
    float rowT = 0.f, colOm = 0.f, colOmS = 0.f;
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      const float dn = s + 1 < Q ? sTK[(s + 1) * kTok + kDlt] : 0.f;
      const float w = sTK[s * kTok + kGam] + (s < u ? dn : 0.f);
      rowT += w * sOm[u * Q + s];
      const float om = sOm[s * Q + u];
      colOm += om;
      colOmS += s > u ? om : 0.f;
    }
    float* k = sTK + u * kTok;
    const float dnu = u + 1 < Q ? sTK[(u + 1) * kTok + kDlt] : 0.f;
    k[kRowT] = rowT;
    k[kColT] = k[kGam] * colOm + dnu * colOmS;
    k[kColOm] = colOm;
    k[kColOmS] = colOmS;
  }
  // (d) dC~ = e^{l_t} S0' dY + G1 B~ and dB~ = om D' X + G1^T C~, tiles of 16 rows x 16 columns;
  // the pair (2k, 2k+1) of a row sits in lanes (2k - n0, 2k + 1 - n0) of one lane group
  const int ntn = N / 16 > 0 ? N / 16 : 1;
  for (int job = wave; job < 2 * nb * ntn; job += NW) {
    const bool isC = job < nb * ntn;
    const int jj = isC ? job : job - nb * ntn;
    const int rb = jj / ntn, cb_ = jj - rb * ntn;
    const int n0 = cb_ * 16, col = n0 + lr, k = col >> 1;
    const bool even = (lr & 1) == 0;
    f32x4 acc = zero4();
    float pa[4], pb[4], pk[4], pi[4];
    if (isC) {
      f32x4 inter = mm_rr(sY, PS, rb * 16, sS, PS, n0, PS, zero4());   // (S0' dY)[tr][n]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tr = rb * 16 + 4 * lg + i;
        inter[i] *= tr < M ? sTK[(tr / R) * kTok + kEl] : 0.f;
      }
      acc = mm_rc(sG1, MK, rb * 16, sB, NS, n0, MK, inter);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tr = rb * 16 + 4 * lg + i;
        const float cself = sC[tr * NS + col];
        const float iv = inter[i], iw = __shfl_xor(iv, 1);
        const float cw = __shfl_xor(cself, 1);
        const float d = acc[i], dw = __shfl_xor(d, 1);
        // pair quantities, on the even lane: (d, dw) = dC~ (2k, 2k+1), (cself, cw) = C~
        pi[i] = even ? cself * iv + cw * iw : 0.f;
        pa[i] = even ? d * cw - dw * cself : 0.f;
        if (tr < M) {
          const int t = tr / R;
          const float2 cs = sCS[t * NH + k];
          const float outv = even ? cs.x * d - cs.y * dw : cs.y * dw + cs.x * d;
          p.dC[(tok0 + (size_t)t * tstep) * R * N + (size_t)(tr - t * R) * N + col] = outv;
        }
      }
      per_token<R>(rb * 16, pa, [&](int t, float x) { if (even && t < n) sPC[t * NH + k] = x; });
      per_token<R>(rb * 16, pi, [&](int t, float x) { if (even && t < n) sPI[t * NH + k] = x; });
    } else {
      const f32x4 dxv = mm_rr(sX, PS, rb * 16, sD, PS, n0, PS, zero4());   // (D' X)[sr][n]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sr = rb * 16 + 4 * lg + i;
        acc[i] = (sr < M ? sTK[(sr / R) * kTok + kOmw] : 0.f) * dxv[i];
      }
      acc = mm_rc(sG1T, MK, rb * 16, sC, NS, n0, MK, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sr = rb * 16 + 4 * lg + i;
        const float bself = sB[sr * NS + col], bw = __shfl_xor(bself, 1);
        const float d = acc[i], dw = __shfl_xor(d, 1);
        const float x = dxv[i], xw = __shfl_xor(x, 1);
        const float om = sr < M ? sTK[(sr / R) * kTok + kOmw] : 0.f;
        pa[i] = even ? d * bw - dw * bself : 0.f;
        pb[i] = even ? bself * x + bw * xw : 0.f;
        pk[i] = even ? om * (bself * xw - bw * x) : 0.f;
        if (sr < M) {
          const int s = sr / R;
          // the last write's gradient from the right, (beta_n / alpha_n) D' X, joins dB~ after the angle parts
          const float e0 = d + (s == n - 1 ? cn * x : 0.f), e1 = dw + (s == n - 1 ? cn * xw : 0.f);
          const float2 cs = sCS[s * NH + k];
          const float outv = even ? cs.x * e0 - cs.y * e1 : cs.y * e1 + cs.x * e0;
          p.dB[(tok0 + (size_t)s * tstep) * R * N + (size_t)(sr - s * R) * N + col] = outv;
        }
      }
      per_token<R>(rb * 16, pa, [&](int t, float x) { if (even && t < n) sPA[t * NH + k] = x; });
      per_token<R>(rb * 16, pb, [&](int t, float x) { if (even && t < n) sPB[t * NH + k] = x; });
      per_token<R>(rb * 16, pk, [&](int t, float x) { if (even && t < n) sPK[t * NH + k] = x; });
    }
  }
  // (e) dX = G2^T dY + (om_s + [s = end] beta_n / alpha_n) B~ D'
  const int ntp = P / 16 > 0 ? P / 16 : 1;
  for (int job = wave; job < nb * ntp; job += NW) {
    const int rb = job / ntp, p0 = (job - rb * ntp) * 16;
    f32x4 acc = mm_rc(sG2T, MK, rb * 16, sY, PS, p0, MK, zero4());
    const f32x4 dd = mm_rc(sB, NS, rb * 16, sD, PS, p0, NS, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sr = rb * 16 + 4 * lg + i;
      if (sr < M) {
        const int s = sr / R;
        const float coef = sTK[s * kTok + kOmw] + (s == n - 1 ? cn : 0.f);
        p.dx[(tok0 + (size_t)s * tstep) * R * P + (size_t)(sr - s * R) * P + p0 + lr] = acc[i] + coef * dd[i];
      }
    }
  }
  // (f) whole-segment scalars: Iend' = <D', S0'>, <dS0', V_{s0-1}>, <S0', J D'> per pair
  {
    float part = 0.f;
    for (int e = tid; e < N * PS; e += NT) part += sD[e] * sS[e];
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) sRD[wave] = part;
  }
  __syncthreads();
  if (tid == 0) {
    float v = 0.f;
    for (int i = 0; i < NW; ++i) v += sRD[i];
    sRD[258] = v;
  }
  __syncthreads();
  {
    float part = 0.f;
    for (int e = tid; e < M * R; e += NT) {
      const int tr = e / R, r = e - tr * R, t = tr / R;
      float cbm = 0.f, xy = 0.f;
      for (int i = 0; i < N; ++i) cbm += sC[tr * NS + i] * sBm[r * N + i];
      for (int i = 0; i < P; ++i) xy += sXm[r * P + i] * sY[tr * PS + i];
      part += sTK[t * kTok + kEl] * cbm * xy;
    }
    for (int e = tid; e < R * N; e += NT) {
      const int r = e / N, nn = e - r * N;
      float dx = 0.f;
      for (int i = 0; i < P; ++i) dx += sD[nn * PS + i] * sXm[r * P + i];
      part += eend * sBm[e] * dx;
    }
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) sRD[8 + wave] = part;
  }
  __syncthreads();
  if (tid == 0) {
    float v = 0.f;
    for (int i = 0; i < NW; ++i) v += sRD[8 + i];
    sRD[259] = v;
  }
  for (int k = tid; k < NH; k += NT) {
    float v = 0.f;
    for (int c = 0; c < P; ++c)
      v += sS[(2 * k) * PS + c] * sD[(2 * k + 1) * PS + c] - sS[(2 * k + 1) * PS + c] * sD[(2 * k) * PS + c];
    sRD[264 + k] = v;
  }
  __syncthreads();
  // (g) per token: dl, d gamma, d delta; then dt, lam, A (suffix sums of dl)
  for (int u = tid; u < n; u += NT) {
    float* k = sTK + u * kTok;
    float ome = 0.f, ie = 0.f;
    for (int q = 0; q < NH; ++q) {
      ome += sPB[u * NH + q];
      ie += sPI[u * NH + q];
    }
    const float omend = __expf(l_end - k[kL]) * ome;
    const float tend = k[kWend] * omend;
    k[kTend] = tend;
    k[kDl] = ie + k[kRowT] - k[kColT] - tend;
    k[kDg] = k[kColOm] + omend;
    k[kDd] = k[kColOmS] + omend;   // d delta_{u+1}
  }
  __syncthreads();
  // dt, lam, A on wave 0, lane u = token u: suffix sums of dl by lane shuffles
  if (wave == 0) {
    const bool in = lane < n;
    const float* k = sTK + (in ? lane : 0) * kTok;
    float tsum = in ? k[kTend] : 0.f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tsum += __shfl_xor(tsum, off);
    float suf = in ? k[kDl] : 0.f;
    if (lane == n - 1) suf += eend * sRD[258] + tsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_down(suf, d);
      if (lane + d < 64) suf += y;
    }
    const float d = in ? k[kDt] : 0.f, lm = k[kLam], dg = k[kDg];
    const float ddl = lane == 0 ? sRD[259] : sTK[(in && lane > 0 ? lane - 1 : 0) * kTok + kDd];
    if (in) {
      const size_t tok = tok0 + (size_t)lane * tstep;
      p.ddt[tok] = Ah * suf + lm * dg + (1.f - lm) * ddl;
      p.dlam[tok] = d * (dg - ddl);
    }
    float dA = d * suf;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dA += __shfl_xor(dA, off);
    if (lane == 0) atomicAdd(p.dA + g.h, dA);
  }
  // angles, over (pair, token) with the tokens of a pair in Q adjacent lanes:
  // dPhi_t = J(dB~_t, B~_t) + J(dC~_t, C~_t) (+ <K_end, J D> at the end), then
  // dphi_t = sum_{u>=t} dPhi_u
  if (p.dtheta) {
#pragma unroll
    for (int i = 0; i < I_TH; ++i) {
      const int e = tid + i * NT, k = e / Q, t = e - k * Q;
      const bool in = e < U_TH && t < n;
      const int at = in ? t * NH + k : 0;
      float ks = in ? sPK[at] : 0.f;
#pragma unroll
      for (int off = 1; off < Q; off <<= 1) ks += __shfl_xor(ks, off, Q);
      float v = in ? sPA[at] + sPC[at] : 0.f;
      if (in && t == n - 1) v += eend * sRD[264 + k] + ks;
#pragma unroll
      for (int d = 1; d < Q; d <<= 1) {
        const float y = __shfl_down(v, d, Q);
        if (t + d < Q) v += y;
      }
      if (in) p.dtheta[(tok0 + (size_t)t * tstep) * NH + k] = v;
    }
  }
  // (h) the first segment: d h0 = dS0', dV_{-1} = delta_0 dS0' -> d B_prev, d x_prev
  if (g.j == 0 && (p.dh0 || p.dBp || p.dxp)) {
    __syncthreads();   // (S0' is read above; it is replaced by dS0')
    for (int job = wave; job < (N / 16 > 0 ? N / 16 : 1) * ntp; job += NW) {
      const int nb0 = (job / ntp) * 16, p0 = (job % ntp) * 16;
      const f32x4 acc = mm_cc(sC, NS, nb0, sY, PS, p0, sEL, 1, MK, zero4());
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int nn = nb0 + 4 * lg + i, c = p0 + lr;
        if (nn < N && c < P) sS[nn * PS + c] = acc[i] + eend * sD[nn * PS + c];
      }
    }
    __syncthreads();
    if (p.dh0)
      for (int e = tid; e < N * P; e += NT) p.dh0[(size_t)g.bh * N * P + e] = sS[(e / P) * PS + e % P];
    const float dlt0 = sTK[kDlt];
    if (p.dBp) {
      for (int e = tid; e < R * N; e += NT) {
        const int r = e / N, nn = e - r * N;
        float v = 0.f;
        for (int c = 0; c < P; ++c) v += sS[nn * PS + c] * sXm[r * P + c];
        p.dBp[(size_t)g.bh * R * N + e] = dlt0 * v;
      }
    }
    if (p.dxp) {
      for (int e = tid; e < R * P; e += NT) {
        const int r = e / P, c = e - r * P;
        float v = 0.f;
        for (int i = 0; i < N; ++i) v += sS[i * PS + c] * sBm[r * N + i];
        p.dxp[(size_t)g.bh * R * P + e] = dlt0 * v;
      }
    }
  }
}

}  // namespace
}  // namespace m3

namespace m3 {
namespace {

template <typename T, int N, int P, int R>
hipError_t run_backward(const BackwardParams& p, hipStream_t s) {
  const unsigned nbh = (unsigned)(p.batch * p.H), nsg = nbh * (unsigned)p.nseg;
  const dim3 blk(bwd_threads(N, P));
  // the chunk kernel is built for one segment length per variant
  if (p.S != backward_segment(R, N, P)) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * bwd_lds(p.S, R, N, P).total;
  if (lds > (size_t)kLdsBudget) return hipErrorInvalidValue;
  // the chunk kernel's dynamic LDS may exceed the default limit: raise it once per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<int> set_once[64][2][8][4][4];
  std::atomic<int>& flag = set_once[dev][sizeof(T) == 2][ilog2(N)][ilog2(P) & 3][ilog2(R)];
  if (flag.load(std::memory_order_acquire) == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_grads_kernel<T, N, P, R>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess)
      return hipErrorInvalidValue;
    flag.store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL((fwd_maps_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  hipLaunchKernelGGL((fwd_combine_kernel<N, P>), dim3(nbh * comb_slices<N, P>()), blk, 0, s, p);
  hipLaunchKernelGGL((bwd_maps_kernel<T, N, P, R>), dim3(nsg), blk, 0, s, p);
  hipLaunchKernelGGL((bwd_combine_kernel<N, P>), dim3(nbh * comb_slices<N, P>()), blk, 0, s, p);
  hipLaunchKernelGGL((chunk_grads_kernel<T, N, P, R>), dim3(nsg), dim3(grads_threads(N, R)), lds, s, p);
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
