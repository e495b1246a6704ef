// m3_decode.hip -- single-token Mamba-3 decode step for gfx950.
//
// Per (sequence, head) the N x P state (fp32, or bf16 between steps: the paper
// page's Table 6 benchmarks decode with either) is read once and written once:
//   H <- R(phi)[alpha H + beta B_prev X_prev^T] + gamma B X^T,   Y = H^T C
// (Mamba-3 explainer, panel 3 physical-frame loop with the two-endpoint rule of
// panel 1 and the rank-R write/readout of panel 4 / Eqs. 12-14).  Decode is
// bound by moving the state (the explainer's section 3.3 argument and the
// paper's Table 2 intensity model), so the kernel is organised around one
// coalesced pass over it; the R-fold MIMO work rides on each loaded element.
//
// Work unit = (pair k, quad q): rows 2k and 2k+1, columns 4q..4q+3.  Consecutive
// lanes take consecutive quads of the same row pair, so every load/store
// instruction covers whole 16-byte-aligned runs of a row (8-byte runs for a
// bf16 state).  The rotation of a pair is lane-local because both of its rows
// sit in the same unit.
// The coefficients are folded into the small operands once per workgroup:
//   H <- [alpha R(phi)] H + sum_r (beta R(phi) B_prev)[:, r] x_prev[r]^T + (gamma B)[:, r] x[r]^T
// so each state element costs one 2x2 rotation and one 2R-long FMA chain.  The
// small operands are staged in LDS as fp32; the readout Y = H^T C is reduced
// across lanes that share a quad (xor shuffles within the wave, then LDS
// across waves).  The gated entry point contracts the ranks of Y with the
// rank-expanded SiLU gate in the same final pass and writes one value per
// head column instead of R.  The prologue entry point normalises the B, C and
// B_prev columns (with their biases) and scales the raw angles by dt while
// the small operands are staged.
#include "m3_device.h"

namespace m3 {
namespace {

// Raw 8-element loads (bf16: one 16-byte load; fp32: two).
template <typename T> struct Raw;
template <> struct Raw<bf16> { uint4 v[1]; };
template <> struct Raw<float> { uint4 v[2]; };
__device__ __forceinline__ void raw_zero(Raw<bf16>& r) { r.v[0] = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw_zero(Raw<float>& r) { r.v[0] = r.v[1] = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw_load(Raw<bf16>& r, const bf16* p) { r.v[0] = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void raw_load(Raw<float>& r, const float* p) {
  r.v[0] = *reinterpret_cast<const uint4*>(p);
  r.v[1] = *reinterpret_cast<const uint4*>(p + 4);
}
__device__ __forceinline__ void raw_unpack(const Raw<bf16>& r, float (&v)[8]) {
  const uint32_t w[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_unpack(const Raw<float>& r, float (&v)[8]) {
  v[0] = __uint_as_float(r.v[0].x); v[1] = __uint_as_float(r.v[0].y);
  v[2] = __uint_as_float(r.v[0].z); v[3] = __uint_as_float(r.v[0].w);
  v[4] = __uint_as_float(r.v[1].x); v[5] = __uint_as_float(r.v[1].y);
  v[6] = __uint_as_float(r.v[1].z); v[7] = __uint_as_float(r.v[1].w);
}

// The small per-token operands of one (sequence, head), as 8-element items:
// [B | C | B_prev] (R*N/8 items each), [x | x_prev] (R*P/8 each), then the
// angles (4 per item).  A NULL source reads as zeros.  A B_prev item also
// carries the angles of its 4 row pairs (it is rotated when staged).
// (Pointers are passed one by one: a struct of them selected by a run-time
// index would be placed in private memory.)
template <typename T>
struct Item { Raw<T> raw; uint4 th; uint4 b0, b1; bool ok, tok, bok; };   // masks applied when staged

// Branch-free on purpose: every item issues its loads unconditionally from a
// clamped address (B stands in for a missing source) and masks the result, so
// the compiler need not wait for a load at a control-flow merge and the state
// loads issued after these stay in flight.
__device__ __forceinline__ uint4 mask4(uint4 v, bool ok) {
  const uint32_t m = ok ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

template <typename T>
__device__ __forceinline__ Item<T> load_item(const T* B, const T* C, const T* Bp, const T* X,
                                             const T* Xp, const float* theta, int N,
                                             int nb8, int nx8, int nitems, int i,
                                             const float* biasB = nullptr, const float* biasC = nullptr) {
  const int nbB = 3 * nb8, nbX = nbB + 2 * nx8;
  const bool isB = i < nbB, isX = !isB && i < nbX, isT = !isB && !isX && i < nitems;
  const int wb = isB ? i / nb8 : 0;
  const int wx = isX ? (i - nbB) / nx8 : 0;
  const int j = isB ? i - wb * nb8 : (isX ? i - nbB - wx * nx8 : 0);
  const T* src = isB ? (wb == 0 ? B : (wb == 1 ? C : Bp)) : (wx == 0 ? X : Xp);
  const bool ok = (isB || isX) && src != nullptr;
  Item<T> it;
  raw_load(it.raw, ok ? src + 8 * j : B);
  // angles: the 4 row pairs of a B_prev item, or an angle item
  const bool tb = isB && wb == 2 && src != nullptr && theta != nullptr;
  const bool tok = tb || (isT && theta != nullptr);
  const int toff = tb ? (8 * j - ((8 * j) / N) * N) / 2 : 4 * (i - nbX);
  it.th = *reinterpret_cast<const uint4*>(tok ? theta + toff : reinterpret_cast<const float*>(B));
  // prologue biases of a B / C / B_prev item (B_prev takes B's)
  const float* bsrc = isB ? (wb == 1 ? biasC : biasB) : nullptr;
  const bool bok = ok && bsrc != nullptr;
  const uint4* bp = reinterpret_cast<const uint4*>(bok ? bsrc + 8 * j : reinterpret_cast<const float*>(B));
  it.b0 = bp[0];
  it.b1 = bp[1];
  it.ok = ok;
  it.tok = tok;
  it.bok = bok;
  return it;
}

// Prologue: the RMS-norm factor of a B / C / B_prev item's column (the N/8
// items of one (rank, tensor) column sit in consecutive lanes), computed by
// every lane; items of other kinds get a factor they do not use.
template <typename T>
__device__ __forceinline__ float item_norm(const Item<T>& it, int N, float eps) {
  Raw<T> raw = it.raw;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(raw.v) / sizeof(uint4)); ++k) raw.v[k] = mask4(raw.v[k], it.ok);
  float v[8];
  raw_unpack(raw, v);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  for (int off = 1; off < N / 8; off <<= 1) ss += __shfl_xor(ss, off);
  return rsqrtf(ss / (float)N + eps);
}

// Widens an item to fp32 into LDS:
//   sW [N][2R]: (beta R(phi) B_prev) in slots 0..R-1, (gamma B) in R..2R-1
//   sC [N][R], sXX [2R][P]: x_prev rows then x rows, sCS [N/2]: alpha (cos, sin).
// scale, tsc: the prologue's norm factor of the item's column and the angle
// multiplier (dt); 1 without the prologue.
template <typename T, int R>
__device__ __forceinline__ void stage_item(float* sW, float* sC, float* sXX, float2* sCS,
                                           int N, int P, int nb8, int nx8, int nitems,
                                           float alpha, float beta, float gamma,
                                           int i, const Item<T>& it, float scale = 1.f, float tsc = 1.f) {
  Raw<T> raw = it.raw;
#pragma unroll
  for (int k = 0; k < (int)(sizeof(raw.v) / sizeof(uint4)); ++k) raw.v[k] = mask4(raw.v[k], it.ok);
  const uint4 tm = mask4(it.th, it.tok);
  const float4 th = make_float4(tsc * __uint_as_float(tm.x), tsc * __uint_as_float(tm.y),
                                tsc * __uint_as_float(tm.z), tsc * __uint_as_float(tm.w));
  float v[8];
  raw_unpack(raw, v);
  if (i < 3 * nb8) {
    const uint4 b0 = mask4(it.b0, it.bok), b1 = mask4(it.b1, it.bok);
    const float bias[8] = {__uint_as_float(b0.x), __uint_as_float(b0.y), __uint_as_float(b0.z), __uint_as_float(b0.w),
                           __uint_as_float(b1.x), __uint_as_float(b1.y), __uint_as_float(b1.z), __uint_as_float(b1.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * scale + bias[e];
    const int which = i / nb8, j = i - which * nb8;
    const int rr = (8 * j) / N, n0 = 8 * j - rr * N;
    if (which == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sW[(n0 + e) * 2 * R + R + rr] = gamma * v[e];
    } else if (which == 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sC[(n0 + e) * R + rr] = v[e];
    } else {
      const float a[4] = {th.x, th.y, th.z, th.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = __cosf(a[e]), sn = __sinf(a[e]);
        const float u = v[2 * e], w = v[2 * e + 1];
        sW[(n0 + 2 * e) * 2 * R + rr] = beta * (c * u - sn * w);
        sW[(n0 + 2 * e + 1) * 2 * R + rr] = beta * (sn * u + c * w);
      }
    }
  } else if (i < 3 * nb8 + 2 * nx8) {
    const int k = i - 3 * nb8;
    const int which = k / nx8, j = k - which * nx8;
    const int rr = (8 * j) / P, p0 = 8 * j - rr * P;
    float* dst = sXX + (which == 0 ? R + rr : rr) * P + p0;
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else if (i < nitems) {
    const int j = i - 3 * nb8 - 2 * nx8;
    const float a[4] = {th.x, th.y, th.z, th.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) sCS[4 * j + e] = make_float2(alpha * __cosf(a[e]), alpha * __sinf(a[e]));
  }
}

// Threads per workgroup and units per thread for an N x P state: one unit per
// thread up to 512 threads, then more units per thread.  A bf16 state, or a
// rank of 4 or more with at most 512 units, takes half as many threads with
// twice the units each: a thread then has 64 bytes of state in flight (as an
// fp32 state at 512 threads and two units does), which measured 12-19% faster
// for the bf16 state and 6-23% for N=64 at R=4 and R=8; N=128 fp32 and rank
// 1-2 were unchanged by it.
constexpr int decode_units(int N, int P) { return (N / 2) * (P / 4); }
constexpr int decode_threads_base(int N, int P) {
  return decode_units(N, P) >= 512 ? 512 : decode_units(N, P) <= 64 ? 64 : (decode_units(N, P) + 63) / 64 * 64;
}
template <typename S, int R>
constexpr int decode_threads(int N, int P) {
  return decode_threads_base(N, P) >= 128 && (sizeof(S) == 2 || (R >= 4 && decode_units(N, P) <= 512))
             ? decode_threads_base(N, P) / 2
             : decode_threads_base(N, P);
}

// N and P are template parameters: the index arithmetic then needs no integer
// division at run time.
// State access: fp32, or bf16 (4 values in 8 bytes, rounded to nearest even
// when stored).  Non-temporal: the state is touched once per step.
__device__ __forceinline__ float4 ld_state(const float* p) { return ld_stream4(p); }
__device__ __forceinline__ void st_state(float* p, float4 v) { st_stream4(p, v); }
__device__ __forceinline__ float4 ld_state(const bf16* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                     __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
}
__device__ __forceinline__ void st_state(bf16* p, float4 v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  auto b = [](float f) { return (unsigned)__builtin_bit_cast(uint16_t, static_cast<bf16>(f)); };
  const u32x2 w = {b(v.x) | (b(v.y) << 16), b(v.z) | (b(v.w) << 16)};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(p));
}

template <typename T, typename S, int R, int N, int P>
__global__ __launch_bounds__((decode_threads<S, R>(N, P))) void decode_kernel(DecodeParams p) {
  constexpr int NT = decode_threads<S, R>(N, P);
  constexpr int UPT = (decode_units(N, P) + NT - 1) / NT;
  const int bh = blockIdx.x;
  const int h_idx = bh % p.H;
  constexpr int QP = P >> 2;             // quads per row
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int nwaves = NT >> 6;

  extern __shared__ float smem[];
  float* sW = smem;                      // [N][2R]
  float* sC = sW + 2 * N * R;            // [N][R]
  float* sXX = sC + N * R;               // [2R][P]
  float2* sCS = reinterpret_cast<float2*>(sXX + 2 * R * P);   // [N/2]
  float* sRed = reinterpret_cast<float*>(sCS + (N >> 1));     // [nwaves][R][P]

  const int q = tid % QP;                // constant across this thread's units
  constexpr int units = (N >> 1) * QP;
  S* hg = static_cast<S*>(p.h) + (size_t)bh * N * P;

  const T* Bg = static_cast<const T*>(p.B) + (size_t)bh * R * N;
  const T* Cg = static_cast<const T*>(p.C) + (size_t)bh * R * N;
  const T* Xg = static_cast<const T*>(p.x) + (size_t)bh * R * P;
  const T* Bpg = p.Bp ? static_cast<const T*>(p.Bp) + (size_t)bh * R * N : nullptr;
  const T* Xpg = p.xp ? static_cast<const T*>(p.xp) + (size_t)bh * R * P : nullptr;
  const float* thg = p.theta ? p.theta + (size_t)bh * (N >> 1) : nullptr;

  // Small operands first (at most two items per thread), then the state.  Loads
  // complete in order, so the operands are staged into LDS and the barrier is
  // passed while the state is still in flight.
  constexpr int nb8 = (R * N) >> 3, nx8 = (R * P) >> 3;
  const int nth4 = thg ? (N >> 3) : 0;
  const int nitems = 3 * nb8 + 2 * nx8 + nth4;
  const float d = p.dt[bh], lm = p.lam[bh], Ah = p.A[h_idx];
  const float* bBh = p.pro && p.biasB ? p.biasB + (size_t)h_idx * R * N : nullptr;
  const float* bCh = p.pro && p.biasC ? p.biasC + (size_t)h_idx * R * N : nullptr;
  const Item<T> it0 = load_item(Bg, Cg, Bpg, Xg, Xpg, thg, N, nb8, nx8, nitems, tid, bBh, bCh);
  const Item<T> it1 = load_item(Bg, Cg, Bpg, Xg, Xpg, thg, N, nb8, nx8, nitems, tid + NT, bBh, bCh);

  // (unconditional, from a clamped unit: a load under a branch would make the
  // compiler wait for everything at the merge)
  float4 h0v[UPT], h1v[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int k = min(tid + i * NT, units - 1) / QP;
    h0v[i] = ld_state(hg + (size_t)(2 * k) * P + 4 * q);
    h1v[i] = ld_state(hg + (size_t)(2 * k + 1) * P + 4 * q);
  }

  const float alpha = __expf(d * Ah);
  const float beta = (1.f - lm) * d * alpha;
  const float gamma = lm * d;
  // prologue: column norm factors (lane shuffles: every lane takes part) and
  // angles scaled by dt
  float sc0 = 1.f, sc1 = 1.f;
  if (p.pro) {
    sc0 = item_norm(it0, N, p.eps);
    sc1 = item_norm(it1, N, p.eps);
  }
  const float tsc = p.pro ? d : 1.f;
  stage_item<T, R>(sW, sC, sXX, sCS, N, P, nb8, nx8, nitems, alpha, beta, gamma, tid, it0, sc0, tsc);
  stage_item<T, R>(sW, sC, sXX, sCS, N, P, nb8, nx8, nitems, alpha, beta, gamma, tid + NT, it1, sc1, tsc);
  // large shapes (more than two items per thread): the rest, loaded and staged
  // here, every lane through every round
  for (int base = 2 * NT; base < nitems; base += NT) {
    const int i = base + tid;
    const Item<T> it = load_item(Bg, Cg, Bpg, Xg, Xpg, thg, N, nb8, nx8, nitems, i, bBh, bCh);
    const float sc = p.pro ? item_norm(it, N, p.eps) : 1.f;
    if (i < nitems) stage_item<T, R>(sW, sC, sXX, sCS, N, P, nb8, nx8, nitems, alpha, beta, gamma, i, it, sc, tsc);
  }
  if (!thg)
    for (int k = tid; k < (N >> 1); k += NT) sCS[k] = make_float2(alpha, 0.f);
  __syncthreads();

  float4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);

#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u < units) {
      const int k = u / QP;
      const float2 cs = sCS[k];          // alpha (cos, sin) of pair k
      const float4 a = h0v[i], b = h1v[i];
      float4 n0, n1;
      n0.x = cs.x * a.x - cs.y * b.x; n1.x = cs.y * a.x + cs.x * b.x;
      n0.y = cs.x * a.y - cs.y * b.y; n1.y = cs.y * a.y + cs.x * b.y;
      n0.z = cs.x * a.z - cs.y * b.z; n1.z = cs.y * a.z + cs.x * b.z;
      n0.w = cs.x * a.w - cs.y * b.w; n1.w = cs.y * a.w + cs.x * b.w;
      const float* w0 = sW + (2 * k) * 2 * R;
      const float* w1 = w0 + 2 * R;
#pragma unroll
      for (int j = 0; j < 2 * R; ++j) {
        // x_prev / x columns 4q..4q+3 are re-read from LDS per unit (same address
        // across the lanes of a quad; keeps them out of the register budget)
        const float4 xx = *reinterpret_cast<const float4*>(sXX + j * P + 4 * q);
        const float c0 = w0[j], c1 = w1[j];
        n0.x += c0 * xx.x; n0.y += c0 * xx.y; n0.z += c0 * xx.z; n0.w += c0 * xx.w;
        n1.x += c1 * xx.x; n1.y += c1 * xx.y; n1.z += c1 * xx.z; n1.w += c1 * xx.w;
      }
      st_state(hg + (size_t)(2 * k) * P + 4 * q, n0);
      st_state(hg + (size_t)(2 * k + 1) * P + 4 * q, n1);
      const float* c0 = sC + (2 * k) * R;
      const float* c1 = c0 + R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        acc[r].x += n0.x * c0[r] + n1.x * c1[r];
        acc[r].y += n0.y * c0[r] + n1.y * c1[r];
        acc[r].z += n0.z * c0[r] + n1.z * c1[r];
        acc[r].w += n0.w * c0[r] + n1.w * c1[r];
      }
    }
  }

  // Reduce over the lanes of this wave that hold the same quad q.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    for (int off = QP; off < 64; off <<= 1) {
      acc[r].x += __shfl_xor(acc[r].x, off);
      acc[r].y += __shfl_xor(acc[r].y, off);
      acc[r].z += __shfl_xor(acc[r].z, off);
      acc[r].w += __shfl_xor(acc[r].w, off);
    }
  }
  if (lane < QP) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      *reinterpret_cast<float4*>(sRed + (wave * R + r) * P + 4 * q) = acc[r];
  }
  __syncthreads();
  if (p.out) {
    // gated readout: out[c] = sum_r w_y[r][c] Y[c][r] silu(w_z[r][c] z[c])
    T* og = static_cast<T*>(p.out) + (size_t)bh * P;
    const T* zg = p.z ? static_cast<const T*>(p.z) + (size_t)bh * P : nullptr;
    const float* wyh = p.wy ? p.wy + (size_t)h_idx * R * P : nullptr;
    const float* wzh = p.wz ? p.wz + (size_t)h_idx * R * P : nullptr;
    for (int c = tid; c < P; c += NT) {
      const float zc = zg ? to_f(zg[c]) : 0.f;
      float o = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += sRed[(w * R + r) * P + c];
        if (wyh) s *= wyh[r * P + c];
        if (zg) {
          const float v = (wzh ? wzh[r * P + c] : 1.f) * zc;
          s *= v / (1.f + __expf(-v));
        }
        o += s;
      }
      og[c] = from_f<T>(o);
    }
    return;
  }
  T* yg = static_cast<T*>(p.y) + (size_t)bh * R * P;
  for (int i = tid; i < R * P; i += NT) {
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += sRed[w * R * P + i];
    yg[i] = from_f<T>(s);
  }
}

template <typename T, typename S, int R, int N, int P>
hipError_t dispatch_shape(const DecodeParams& p, hipStream_t stream) {
  constexpr int nt = decode_threads<S, R>(N, P);
  constexpr int nwaves = nt / 64;
  const size_t lds = sizeof(float) * (3 * (size_t)N * R + 2 * (size_t)R * P + N +
                                      (size_t)nwaves * R * P);   // sW, sC, sXX, sCS, sRed
  hipLaunchKernelGGL((decode_kernel<T, S, R, N, P>), dim3(p.batch * p.H), dim3(nt), lds, stream, p);
  return hipGetLastError();
}

template <typename T, typename S, int R, int N>
hipError_t dispatch_p(const DecodeParams& p, hipStream_t stream) {
  switch (p.P) {
    case 16: return dispatch_shape<T, S, R, N, 16>(p, stream);
    case 32: return dispatch_shape<T, S, R, N, 32>(p, stream);
    case 64: return dispatch_shape<T, S, R, N, 64>(p, stream);
    case 128: return dispatch_shape<T, S, R, N, 128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename S, int R>
hipError_t dispatch_n(const DecodeParams& p, hipStream_t stream) {
  switch (p.N) {
    case 16: return dispatch_p<T, S, R, 16>(p, stream);
    case 32: return dispatch_p<T, S, R, 32>(p, stream);
    case 64: return dispatch_p<T, S, R, 64>(p, stream);
    case 128: return dispatch_p<T, S, R, 128>(p, stream);
    case 256: return dispatch_p<T, S, R, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename S>
hipError_t dispatch_rank(const DecodeParams& p, hipStream_t stream) {
  switch (p.R) {
    case 1: return dispatch_n<T, S, 1>(p, stream);
    case 2: return dispatch_n<T, S, 2>(p, stream);
    case 4: return dispatch_n<T, S, 4>(p, stream);
    case 8: return dispatch_n<T, S, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// A bf16 state is supported with bf16 inputs (the API rejects other pairings).
hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream) {
  if (p.batch == 0 || p.H == 0) return hipSuccess;
  if (p.state_bf16) return dtype == M3_BF16 ? dispatch_rank<bf16, bf16>(p, stream) : hipErrorInvalidValue;
  return dtype == M3_BF16 ? dispatch_rank<bf16, float>(p, stream) : dispatch_rank<float, float>(p, stream);
}

}  // namespace m3
