// m3_prefill.hip -- chunked Mamba-3 prefill for gfx950.
//
// The recurrence (explainer panels 1, 3, 4; paper page Table 1 caption)
//   H_t = alpha_t R(phi_t) H_{t-1} + beta_t R(phi_t) V_{t-1} + gamma_t V_t,
//   V_t = B_t X_t^T,  Y_t = H_t^T C_t
// is evaluated chunk by chunk as an exact rearrangement (the explainer's
// section 3.3 remark on the chunked algorithm and its structured-mask view,
// section 3.1.2-3.1.3 / Eq. 7, paper page Figure 1).  Within a chunk starting at
// token t0, with chunk-local log decay l_t = sum_{t0<=j<=t} dt_j A and chunk-local
// phase Phi_t = sum_{t0<=j<=t} phi_j (the data-dependent RoPE form, Prop. 3/4):
//
//   Y_t = exp(l_t) C~_t^T S_in
//       + sum_{t0<=s<=t} exp(l_t - l_s) m_ts (C~_t . B~_s) X_s          (1)
//   m_ts = gamma_s                      if s == t
//        = gamma_s + (1-lam_{s+1}) dt_{s+1}   if s < t
//   B~_s = R(-Phi_s) B_s,  C~_t = R(-Phi_t) C_t
//
// The second line of m_ts folds the delayed endpoint of token s+1 into column s:
// beta_{s+1} exp(l_t - l_{s+1}) = (1-lam_{s+1}) dt_{s+1} exp(l_t - l_s).  The same
// fold carries the delayed endpoint across chunk boundaries: the state handed to
// the next chunk already contains (1-lam_{t1}) dt_{t1} V_{t1-1} for that chunk's
// first token t1, so a chunk never looks at its predecessor's tokens.
//
//   S_out = a_c R(Psi_c) S_in + u_c,   a_c = exp(l_end), Psi_c = Phi_end
//   u_c   = sum_s exp(l_end - l_s) w_s R(Psi_c - Phi_s) B_s X_s^T          (2)
//   w_s   = gamma_s + (1-lam_{s+1}) dt_{s+1}  (next token's term, 0 at the end
//                                               of the sequence)
// S_in of the first chunk is h0 + (1-lam_0) dt_0 B_prev X_prev^T.
// Exponents are always differences l_t - l_s <= 0 (never a product of exp(l_t)
// and exp(-l_s), which would overflow fp32 over long chunks).
//
// Launches:  chunk_state (2) -> state_pass (scan over chunks) -> chunk_output (1).
#include "m3_device.h"

namespace m3 {
namespace {

constexpr int kThreads = 256;
constexpr int kKB = 64;            // chunk_state: contraction rows staged per LDS block

__host__ __device__ inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

// ---- LDS layouts (host and device compute them identically) ----------------
struct StateLds {            // chunk_state
  size_t W, l, cs, Xt, Bt, total;
};
__host__ __device__ inline StateLds state_lds(int Q, int N, int P, int esize) {
  StateLds o;
  o.W = 0;
  o.l = o.W + sizeof(float) * Q;
  o.cs = o.l + sizeof(float) * Q;
  o.Xt = o.cs + sizeof(float2) * (size_t)Q * (N / 2);
  o.Bt = o.Xt + (size_t)esize * P * (kKB + 8);
  o.total = o.Bt + (size_t)esize * N * (kKB + 8);
  return o;
}
struct OutputLds {           // chunk_output
  size_t l, g, w, cs, B, Xt, H, total;
};
__host__ __device__ inline OutputLds output_lds(int Q, int R, int N, int P, int esize) {
  const int QRp = round_up(Q * R, 32);
  OutputLds o;
  o.l = 0;
  o.g = o.l + sizeof(float) * Q;
  o.w = o.g + sizeof(float) * Q;
  o.cs = round_up((int)(o.w + sizeof(float) * Q), 16);
  o.B = o.cs + sizeof(float2) * (size_t)Q * (N / 2);
  o.Xt = o.B + (size_t)esize * QRp * (N + 8);
  o.H = o.Xt + (size_t)esize * P * (QRp + 8);
  o.total = o.H + (size_t)esize * P * (N + 8);
  return o;
}

__device__ __forceinline__ size_t tok_index(const PrefillParams& p, int b, int t, int h) {
  return ((size_t)b * p.L + t) * p.H + h;
}

// Inclusive scan of a[0..n) in LDS by one 256-thread block (n <= 256).
__device__ void block_scan_inclusive(float* a, int n) {
  const int tid = threadIdx.x;
  for (int off = 1; off < n; off <<= 1) {
    const float v = (tid < n && tid >= off) ? a[tid - off] : 0.f;
    __syncthreads();
    if (tid < n) a[tid] += v;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// chunk_state: u_c (eq. 2), a_c and R(Psi_c) for one (b, h, chunk).
// u_c^T [P][N] = X^T [P][rows] * Bw [rows][N] with rows = (token, rank) of the
// chunk and Bw = exp(l_end - l_s) w_s R(Psi_c - Phi_s) B_s; both operands are
// staged transposed in LDS (contraction index contiguous) 64 rows at a time.
template <typename T, int N, int P>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(PrefillParams p) {
  constexpr int NH = N / 2;
  constexpr int TP = P / 16, TN = N / 16, TT = TP * TN, TPW = (TT + 3) / 4;
  constexpr int KS = kKB + 8;      // LDS row stride (elements) of the transposed tiles
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  const int R = p.R, logR = p.logR, Q = p.Q;
  const int t0 = c * Q;
  const int nt = min(Q, p.L - t0);
  const int rows = nt << logR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  extern __shared__ __align__(16) unsigned char smem[];
  const StateLds lay = state_lds(Q, N, P, sizeof(T));
  float* s_W = reinterpret_cast<float*>(smem + lay.W);
  float* s_l = reinterpret_cast<float*>(smem + lay.l);
  float2* s_cs = reinterpret_cast<float2*>(smem + lay.cs);
  T* s_Xt = reinterpret_cast<T*>(smem + lay.Xt);
  T* s_Bt = reinterpret_cast<T*>(smem + lay.Bt);

  const float A = p.A[h];
  for (int s = tid; s < Q; s += kThreads)
    s_l[s] = s < nt ? p.dt[tok_index(p, b, t0 + s, h)] * A : 0.f;
  // raw angles of the chunk's tokens
  if (p.theta) {
    for (int i = tid; i < Q * NH; i += kThreads) {
      const int s = i / NH, k = i - s * NH;
      s_cs[i].x = s < nt ? p.theta[tok_index(p, b, t0 + s, h) * NH + k] : 0.f;
    }
  }
  __syncthreads();
  block_scan_inclusive(s_l, Q);
  const float l_end = s_l[nt - 1];
  for (int s = tid; s < Q; s += kThreads) {
    float W = 0.f;
    if (s < nt) {
      const size_t tk = tok_index(p, b, t0 + s, h);
      float w = p.lam[tk] * p.dt[tk];
      if (t0 + s + 1 < p.L) w += (1.f - p.lam[tk + p.H]) * p.dt[tk + p.H];
      W = __expf(l_end - s_l[s]) * w;
    }
    s_W[s] = W;
  }
  float2* rot_out = p.ws_rot + ((size_t)bh * p.nc + c) * NH;
  if (p.theta) {
    // exclusive suffix sums: angle still to turn from token s to the chunk end
    for (int k = tid; k < NH; k += kThreads) {
      float run = 0.f;
      for (int s = nt - 1; s >= 0; --s) {
        const float th = s_cs[s * NH + k].x;
        s_cs[s * NH + k].x = run;
        run += th;
      }
      float sn, cn;
      sincosf(run, &sn, &cn);
      rot_out[k] = make_float2(cn, sn);
    }
    __syncthreads();
    for (int i = tid; i < Q * NH; i += kThreads) {
      float sn, cn;
      sincosf(s_cs[i].x, &sn, &cn);
      s_cs[i] = make_float2(cn, sn);
    }
  } else {
    for (int i = tid; i < Q * NH; i += kThreads) s_cs[i] = make_float2(1.f, 0.f);
    for (int k = tid; k < NH; k += kThreads) rot_out[k] = make_float2(1.f, 0.f);
  }
  if (tid == 0) p.ws_decay[(size_t)bh * p.nc + c] = __expf(l_end);
  __syncthreads();

  const T* Bg = static_cast<const T*>(p.B);
  const T* Xg = static_cast<const T*>(p.x);
  f32x4 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero4();

  for (int kb = 0; kb < rows; kb += kKB) {
    for (int it = tid; it < kKB * (N / 8); it += kThreads) {
      const int rl = it / (N / 8), ng = it - rl * (N / 8);
      const int row = kb + rl;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (row < rows) {
        const int s = row >> logR, r = row & (R - 1);
        load8(Bg + (tok_index(p, b, t0 + s, h) * R + r) * N + ng * 8, v);
        const float W = s_W[s];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 cs = s_cs[s * NH + ng * 4 + j];
          const float u = v[2 * j], w = v[2 * j + 1];
          v[2 * j] = W * (cs.x * u - cs.y * w);
          v[2 * j + 1] = W * (cs.y * u + cs.x * w);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s_Bt[(ng * 8 + j) * KS + rl] = from_f<T>(v[j]);
    }
    for (int it = tid; it < kKB * (P / 8); it += kThreads) {
      const int rl = it / (P / 8), pg = it - rl * (P / 8);
      const int row = kb + rl;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (row < rows) {
        const int s = row >> logR, r = row & (R - 1);
        load8(Xg + (tok_index(p, b, t0 + s, h) * R + r) * P + pg * 8, v);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s_Xt[(pg * 8 + j) * KS + rl] = from_f<T>(v[j]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = wave + 4 * i;
      if (tile < TT) {
        const int pt = tile / TN, ntl = tile - pt * TN;
#pragma unroll
        for (int ks = 0; ks < kKB / 32; ++ks) {
          Frag<T> fa, fb;
          frag_lds8(fa, s_Xt + (pt * 16 + (lane & 15)) * KS + ks * 32 + 8 * (lane >> 4));
          frag_lds8(fb, s_Bt + (ntl * 16 + (lane & 15)) * KS + ks * 32 + 8 * (lane >> 4));
          acc[i] = mma(fa, fb, acc[i]);
        }
      }
    }
    __syncthreads();
  }

  float* out = p.ws_state + ((size_t)bh * p.nc + c) * P * N;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = wave + 4 * i;
    if (tile < TT) {
      const int pt = tile / TN, ntl = tile - pt * TN;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        out[(pt * 16 + 4 * (lane >> 4) + j) * N + ntl * 16 + (lane & 15)] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// state_pass: for one (b, h, pair k, column p) walk the chunks in order,
// S <- a_c R(Psi_c) S + u_c, leaving in slot c the state that enters chunk c.
// Slots are [P][N] fp32, so a pair (2k, 2k+1) is one float2 and consecutive
// threads (consecutive k) touch consecutive float2s.
template <typename T>
__global__ __launch_bounds__(kThreads) void state_pass_kernel(PrefillParams p) {
  const int NH = p.N / 2;
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)p.batch * p.H * NH * p.P;
  if (gid >= total) return;
  const int k = (int)(gid % NH);
  const size_t rest = gid / NH;
  const int col = (int)(rest % p.P);
  const int bh = (int)(rest / p.P);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N, P = p.P, R = p.R;

  float g0 = 0.f, g1 = 0.f;
  if (p.h0) {
    g0 = p.h0[((size_t)bh * N + 2 * k) * P + col];
    g1 = p.h0[((size_t)bh * N + 2 * k + 1) * P + col];
  }
  if (p.Bp) {
    const size_t t = tok_index(p, b, 0, h);
    const float kappa = (1.f - p.lam[t]) * p.dt[t];
    const T* Bp = static_cast<const T*>(p.Bp) + (size_t)bh * R * N;
    const T* xp = static_cast<const T*>(p.xp) + (size_t)bh * R * P;
    float v0 = 0.f, v1 = 0.f;
    for (int r = 0; r < R; ++r) {
      const float xv = to_f(xp[r * P + col]);
      v0 += to_f(Bp[r * N + 2 * k]) * xv;
      v1 += to_f(Bp[r * N + 2 * k + 1]) * xv;
    }
    g0 += kappa * v0;
    g1 += kappa * v1;
  }
  float2* slot = reinterpret_cast<float2*>(p.ws_state + (size_t)bh * p.nc * P * N) + (size_t)col * NH + k;
  const size_t stride = (size_t)P * NH;            // float2 per chunk slot
  const float* dec = p.ws_decay + (size_t)bh * p.nc;
  const float2* rot = p.ws_rot + (size_t)bh * p.nc * NH + k;
  int c = 0;
  for (; c + 4 <= p.nc; c += 4) {
    float2 u[4], cs[4];
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[i] = slot[(c + i) * stride];
      cs[i] = rot[(size_t)(c + i) * NH];
      a[i] = dec[c + i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      slot[(c + i) * stride] = make_float2(g0, g1);
      const float r0 = cs[i].x * g0 - cs[i].y * g1, r1 = cs[i].y * g0 + cs[i].x * g1;
      g0 = a[i] * r0 + u[i].x;
      g1 = a[i] * r1 + u[i].y;
    }
  }
  for (; c < p.nc; ++c) {
    const float2 u = slot[c * stride];
    const float2 cs = rot[(size_t)c * NH];
    const float a = dec[c];
    slot[c * stride] = make_float2(g0, g1);
    const float r0 = cs.x * g0 - cs.y * g1, r1 = cs.y * g0 + cs.x * g1;
    g0 = a * r0 + u.x;
    g1 = a * r1 + u.y;
  }
  if (p.h_out) {
    p.h_out[((size_t)bh * N + 2 * k) * P + col] = g0;
    p.h_out[((size_t)bh * N + 2 * k + 1) * P + col] = g1;
  }
}

// ---------------------------------------------------------------------------
// chunk_output: equation (1) for one (b, h, chunk).
// Rows of the flattened chunk are (token, rank) pairs, 16 per MFMA tile.  Each
// wave owns output row tiles; for a row tile it
//   - builds C~ fragments straight from global memory (rotated in registers),
//   - reads the entering state out of LDS:  Y = diag(exp(l_t)) C~ S_in,
//   - walks the causal 32-row blocks of B~:  S^T = B~ C~^T on MFMA, applies
//     the decay x two-band mask elementwise in registers, and feeds the masked
//     tile straight back as the A operand of (mask o S) X.
template <typename T, int N, int P>
__global__ __launch_bounds__(kThreads) void chunk_output_kernel(PrefillParams p) {
  constexpr int NH = N / 2;
  constexpr int NK = (N + 31) / 32;        // 32-wide slices of the state dimension
  constexpr int TP = P / 16;
  constexpr int NS = N + 8;                // LDS row stride of B~ and S_in^T
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh - b * p.H;
  const int R = p.R, logR = p.logR, Q = p.Q;
  const int QRp = round_up(Q << logR, 32);
  const int XS = QRp + 8;                  // LDS row stride of X^T
  const int t0 = c * Q;
  const int nt = min(Q, p.L - t0);
  const int rows = nt << logR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  extern __shared__ __align__(16) unsigned char smem[];
  const OutputLds lay = output_lds(Q, R, N, P, sizeof(T));
  float* s_l = reinterpret_cast<float*>(smem + lay.l);
  float* s_g = reinterpret_cast<float*>(smem + lay.g);
  float* s_w = reinterpret_cast<float*>(smem + lay.w);
  float2* s_cs = reinterpret_cast<float2*>(smem + lay.cs);
  T* s_B = reinterpret_cast<T*>(smem + lay.B);
  T* s_Xt = reinterpret_cast<T*>(smem + lay.Xt);
  T* s_H = reinterpret_cast<T*>(smem + lay.H);

  const float A = p.A[h];
  for (int s = tid; s < Q; s += kThreads) {
    float lv = 0.f, gv = 0.f, wv = 0.f;
    if (s < nt) {
      const size_t tk = tok_index(p, b, t0 + s, h);
      const float d = p.dt[tk];
      lv = d * A;
      gv = p.lam[tk] * d;
      wv = gv;
      if (s + 1 < nt) wv += (1.f - p.lam[tk + p.H]) * p.dt[tk + p.H];
    }
    s_l[s] = lv; s_g[s] = gv; s_w[s] = wv;
  }
  if (p.theta) {
    for (int i = tid; i < Q * NH; i += kThreads) {
      const int s = i / NH, k = i - s * NH;
      s_cs[i].x = s < nt ? p.theta[tok_index(p, b, t0 + s, h) * NH + k] : 0.f;
    }
  }
  // entering state S_in^T [P][N] -> LDS in the compute type
  {
    const float* Sg = p.ws_state + ((size_t)bh * p.nc + c) * P * N;
    for (int i = tid; i < P * (N / 4); i += kThreads) {
      const int pp = i / (N / 4), n4 = i - pp * (N / 4);
      const float4 v = *reinterpret_cast<const float4*>(Sg + (size_t)pp * N + 4 * n4);
      T* d = s_H + pp * NS + 4 * n4;
      d[0] = from_f<T>(v.x); d[1] = from_f<T>(v.y); d[2] = from_f<T>(v.z); d[3] = from_f<T>(v.w);
    }
  }
  __syncthreads();
  block_scan_inclusive(s_l, Q);
  if (p.theta) {
    for (int k = tid; k < NH; k += kThreads) {
      float run = 0.f;
      for (int s = 0; s < nt; ++s) {
        run += s_cs[s * NH + k].x;
        s_cs[s * NH + k].x = run;
      }
    }
    __syncthreads();
    for (int i = tid; i < Q * NH; i += kThreads) {
      float sn, cn;
      sincosf(s_cs[i].x, &sn, &cn);
      s_cs[i] = make_float2(cn, sn);
    }
  } else {
    for (int i = tid; i < Q * NH; i += kThreads) s_cs[i] = make_float2(1.f, 0.f);
  }
  __syncthreads();

  const T* Bg = static_cast<const T*>(p.B);
  const T* Cg = static_cast<const T*>(p.C);
  const T* Xg = static_cast<const T*>(p.x);
  // B~ rows (token, rank) -> LDS row-major; X -> LDS transposed.
  for (int it = tid; it < QRp * (N / 8); it += kThreads) {
    const int row = it / (N / 8), ng = it - row * (N / 8);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < rows) {
      const int s = row >> logR, r = row & (R - 1);
      load8(Bg + (tok_index(p, b, t0 + s, h) * R + r) * N + ng * 8, v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float2 cs = s_cs[s * NH + ng * 4 + j];     // R(-Phi_s)
        const float u = v[2 * j], w = v[2 * j + 1];
        v[2 * j] = cs.x * u + cs.y * w;
        v[2 * j + 1] = -cs.y * u + cs.x * w;
      }
    }
    T* d = s_B + row * NS + ng * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = from_f<T>(v[j]);
  }
  for (int it = tid; it < QRp * (P / 8); it += kThreads) {
    const int row = it / (P / 8), pg = it - row * (P / 8);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < rows) {
      const int s = row >> logR, r = row & (R - 1);
      load8(Xg + (tok_index(p, b, t0 + s, h) * R + r) * P + pg * 8, v);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_Xt[(pg * 8 + j) * XS + row] = from_f<T>(v[j]);
  }
  __syncthreads();

  T* Yg = static_cast<T*>(p.y);
  const int MT = QRp / 16;
  for (int it = wave; it < MT && it * 16 < rows; it += 4) {
    // this lane's row of C~ (and column of S^T)
    const int row_a = it * 16 + l16;
    const bool va = row_a < rows;
    const int ta = row_a >> logR, ra = row_a & (R - 1);
    Frag<T> cf[NK];
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
      const int n0 = kn * 32 + 8 * g4;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (va && n0 < N) {
        load8(Cg + (tok_index(p, b, t0 + ta, h) * R + ra) * N + n0, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 cs = s_cs[ta * NH + n0 / 2 + j];  // R(-Phi_t)
          const float u = v[2 * j], w = v[2 * j + 1];
          v[2 * j] = cs.x * u + cs.y * w;
          v[2 * j + 1] = -cs.y * u + cs.x * w;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) frag_set(cf[kn], j, v[j]);
    }

    // entering-state term: Y = C~ S_in, rows scaled by exp(l_t)
    f32x4 yacc[TP];
#pragma unroll
    for (int pn = 0; pn < TP; ++pn) {
      yacc[pn] = zero4();
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        const int n0 = kn * 32 + 8 * g4;
        Frag<T> hf;
        if (n0 < N) frag_lds8(hf, s_H + (pn * 16 + l16) * NS + n0);
        else frag_zero(hf);
        yacc[pn] = mma(cf[kn], hf, yacc[pn]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = it * 16 + 4 * g4 + j;
      const float e = row < rows ? __expf(s_l[row >> logR]) : 0.f;
#pragma unroll
      for (int pn = 0; pn < TP; ++pn) yacc[pn][j] *= e;
    }

    // intra-chunk causal blocks of 32 source rows
    const int last_row = min(it * 16 + 15, rows - 1);
    const int sbmax = last_row >= 0 ? last_row / 32 : -1;
    const float l_t = va ? s_l[ta] : 0.f;
    for (int sb = 0; sb <= sbmax; ++sb) {
      f32x4 st0 = zero4(), st1 = zero4();
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        const int n0 = kn * 32 + 8 * g4;
        Frag<T> a0, a1;
        if (n0 < N) {
          frag_lds8(a0, s_B + (sb * 32 + l16) * NS + n0);
          frag_lds8(a1, s_B + (sb * 32 + 16 + l16) * NS + n0);
        } else {
          frag_zero(a0);
          frag_zero(a1);
        }
        st0 = mma(a0, cf[kn], st0);
        st1 = mma(a1, cf[kn], st1);
      }
      Frag<T> pf;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int srow = sb * 32 + hh * 16 + 4 * g4 + j;
          const int s = srow >> logR;
          float m = 0.f;
          if (va && srow < rows && s <= ta)
            m = __expf(l_t - s_l[s]) * (s < ta ? s_w[s] : s_g[s]);
          frag_set(pf, hh * 4 + j, (hh ? st1[j] : st0[j]) * m);
        }
      }
#pragma unroll
      for (int pn = 0; pn < TP; ++pn) {
        Frag<T> xf;
        const T* xr = s_Xt + (pn * 16 + l16) * XS + sb * 32 + 4 * g4;
        frag_lds4x2(xf, xr, xr + 16);
        yacc[pn] = mma(pf, xf, yacc[pn]);
      }
    }

#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = it * 16 + 4 * g4 + j;
      if (row < rows) {
        const int t = row >> logR, r = row & (R - 1);
        T* yo = Yg + (tok_index(p, b, t0 + t, h) * R + r) * P + l16;
#pragma unroll
        for (int pn = 0; pn < TP; ++pn) yo[pn * 16] = from_f<T>(yacc[pn][j]);
      }
    }
  }
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Raises a kernel's dynamic-LDS limit to the whole per-CU budget, once per
// kernel instantiation (the planner never asks for more than that).
template <void (*Kernel)(PrefillParams)>
hipError_t set_lds(size_t bytes) {
  static bool done = false;
  if (bytes <= 64 * 1024 || done) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
  if (e == hipSuccess) done = true;
  return e;
}

template <typename T, int N, int P>
hipError_t run_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream) {
  const dim3 grid(p.nc, p.batch * p.H), block(kThreads);
  hipError_t e;
  if ((e = set_lds<chunk_state_kernel<T, N, P>>(plan.lds_state)) != hipSuccess) return e;
  if ((e = set_lds<chunk_output_kernel<T, N, P>>(plan.lds_output)) != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_state_kernel<T, N, P>), grid, block, plan.lds_state, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t lanes = (size_t)p.batch * p.H * (N / 2) * P;
  hipLaunchKernelGGL((state_pass_kernel<T>), dim3((unsigned)((lanes + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_output_kernel<T, N, P>), grid, block, plan.lds_output, stream, p);
  return hipGetLastError();
}

template <typename T, int N>
hipError_t dispatch_p(const PrefillParams& p, const PrefillPlan& plan, hipStream_t s) {
  switch (p.P) {
    case 16: return run_prefill<T, N, 16>(p, plan, s);
    case 32: return run_prefill<T, N, 32>(p, plan, s);
    case 64: return run_prefill<T, N, 64>(p, plan, s);
    case 128: return run_prefill<T, N, 128>(p, plan, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t dispatch_n(const PrefillParams& p, const PrefillPlan& plan, hipStream_t s) {
  switch (p.N) {
    case 16: return dispatch_p<T, 16>(p, plan, s);
    case 32: return dispatch_p<T, 32>(p, plan, s);
    case 64: return dispatch_p<T, 64>(p, plan, s);
    case 128: return dispatch_p<T, 128>(p, plan, s);
    case 256: return dispatch_p<T, 256>(p, plan, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t chunk_state_lds_bytes(int Q, int R, int N, int P, int esize) {
  (void)R;
  return state_lds(Q, N, P, esize).total;
}
size_t chunk_output_lds_bytes(int Q, int R, int N, int P, int esize) {
  return output_lds(Q, R, N, P, esize).total;
}

hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, int dtype,
                          hipStream_t stream) {
  return dtype == M3_BF16 ? dispatch_n<bf16>(p, plan, stream) : dispatch_n<float>(p, plan, stream);
}

hipError_t launch_copy_or_zero(float* dst, const float* src, size_t n, hipStream_t stream) {
  if (n == 0 || dst == src) return hipSuccess;
  hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     dst, src, n);
  return hipGetLastError();
}

}  // namespace m3
