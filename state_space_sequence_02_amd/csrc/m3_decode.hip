// m3_decode.hip -- single-token Mamba-3 decode step for gfx950.
//
// Per (sequence, head) the N x P fp32 state is read once and written once:
//   H <- R(phi)[alpha H + beta B_prev X_prev^T] + gamma B X^T,   Y = H^T C
// (Mamba-3 explainer, panel 3 physical-frame loop with the two-endpoint rule of
// panel 1 and the rank-R write/readout of panel 4 / Eqs. 12-14).  Decode is
// bound by moving the state (the explainer's section 3.3 argument and the
// paper's Table 2 intensity model), so the kernel is organised around one
// coalesced pass over it; the R-fold MIMO work rides on each loaded element.
//
// Work unit = (pair k, quad q): rows 2k and 2k+1, columns 4q..4q+3.  Consecutive
// lanes take consecutive quads of the same row pair, so every load/store
// instruction covers whole 16-byte-aligned runs of a row.  The rotation of a
// pair is lane-local because both of its rows sit in the same unit.
// All small per-token operands (B, C, B_prev, x, x_prev, cos/sin) are staged in
// LDS as fp32 first; the readout Y = H^T C is reduced across lanes that share a
// quad (xor shuffles within the wave, then LDS across waves).
#include "m3_device.h"

namespace m3 {
namespace {

template <typename T, int R, int UPT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  const int bh = blockIdx.x;
  const int h_idx = bh % p.H;
  const int N = p.N, P = p.P;
  const int QP = P >> 2;                 // quads per row
  const int NT = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = NT >> 6;

  extern __shared__ float smem[];
  float* sB = smem;                      // [N][R]  current B, pair-friendly layout
  float* sC = sB + N * R;                // [N][R]
  float* sBp = sC + N * R;               // [N][R]  previous B
  float* sX = sBp + N * R;               // [R][P]
  float* sXp = sX + R * P;               // [R][P]
  float2* sCS = reinterpret_cast<float2*>(sXp + R * P);     // [N/2] cos, sin
  float* sRed = reinterpret_cast<float*>(sCS + (N >> 1));   // [nwaves][R][P]

  const int q = tid % QP;                // constant across this thread's units
  const int units = (N >> 1) * QP;
  float* hg = p.h + (size_t)bh * N * P;

  // The state is the only large operand: issue all of this thread's state loads
  // first, so their latency overlaps the staging of the small per-token
  // operands below instead of following it.
  float4 h0v[UPT], h1v[UPT];
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u < units) {
      const int k = u / QP;
      h0v[i] = ld_stream4(hg + (size_t)(2 * k) * P + 4 * q);
      h1v[i] = ld_stream4(hg + (size_t)(2 * k + 1) * P + 4 * q);
    }
  }

  const T* Bg = static_cast<const T*>(p.B) + (size_t)bh * R * N;
  const T* Cg = static_cast<const T*>(p.C) + (size_t)bh * R * N;
  const T* Xg = static_cast<const T*>(p.x) + (size_t)bh * R * P;
  const T* Bpg = p.Bp ? static_cast<const T*>(p.Bp) + (size_t)bh * R * N : nullptr;
  const T* Xpg = p.xp ? static_cast<const T*>(p.xp) + (size_t)bh * R * P : nullptr;

  for (int i = tid; i < R * N; i += NT) {
    const int r = i / N, n = i - r * N;
    sB[n * R + r] = to_f(Bg[i]);
    sC[n * R + r] = to_f(Cg[i]);
    sBp[n * R + r] = Bpg ? to_f(Bpg[i]) : 0.f;
  }
  for (int i = tid; i < R * P; i += NT) {
    sX[i] = to_f(Xg[i]);
    sXp[i] = Xpg ? to_f(Xpg[i]) : 0.f;
  }
  for (int k = tid; k < (N >> 1); k += NT) {
    float c = 1.f, s = 0.f;
    if (p.theta) sincosf(p.theta[(size_t)bh * (N >> 1) + k], &s, &c);
    sCS[k] = make_float2(c, s);
  }
  const float d = p.dt[bh], lm = p.lam[bh];
  const float alpha = __expf(d * p.A[h_idx]);
  const float beta = (1.f - lm) * d * alpha;
  const float gamma = lm * d;
  __syncthreads();

  float4 xr[R], xpr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    xr[r] = *reinterpret_cast<const float4*>(sX + r * P + 4 * q);
    xpr[r] = *reinterpret_cast<const float4*>(sXp + r * P + 4 * q);
  }
  float4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);

#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = tid + i * NT;
    if (u < units) {
      const int k = u / QP;
      const float* b0 = sB + (2 * k) * R;  const float* b1 = b0 + R;
      const float* p0 = sBp + (2 * k) * R; const float* p1 = p0 + R;
      float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0, w0 = v0, w1 = v0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // previous write rows 2k, 2k+1 and current write rows 2k, 2k+1
        w0.x += p0[r] * xpr[r].x; w0.y += p0[r] * xpr[r].y; w0.z += p0[r] * xpr[r].z; w0.w += p0[r] * xpr[r].w;
        w1.x += p1[r] * xpr[r].x; w1.y += p1[r] * xpr[r].y; w1.z += p1[r] * xpr[r].z; w1.w += p1[r] * xpr[r].w;
        v0.x += b0[r] * xr[r].x;  v0.y += b0[r] * xr[r].y;  v0.z += b0[r] * xr[r].z;  v0.w += b0[r] * xr[r].w;
        v1.x += b1[r] * xr[r].x;  v1.y += b1[r] * xr[r].y;  v1.z += b1[r] * xr[r].z;  v1.w += b1[r] * xr[r].w;
      }
      const float2 cs = sCS[k];
      float4 a0, a1, n0, n1;
      a0.x = alpha * h0v[i].x + beta * w0.x; a0.y = alpha * h0v[i].y + beta * w0.y;
      a0.z = alpha * h0v[i].z + beta * w0.z; a0.w = alpha * h0v[i].w + beta * w0.w;
      a1.x = alpha * h1v[i].x + beta * w1.x; a1.y = alpha * h1v[i].y + beta * w1.y;
      a1.z = alpha * h1v[i].z + beta * w1.z; a1.w = alpha * h1v[i].w + beta * w1.w;
      n0.x = cs.x * a0.x - cs.y * a1.x + gamma * v0.x; n1.x = cs.y * a0.x + cs.x * a1.x + gamma * v1.x;
      n0.y = cs.x * a0.y - cs.y * a1.y + gamma * v0.y; n1.y = cs.y * a0.y + cs.x * a1.y + gamma * v1.y;
      n0.z = cs.x * a0.z - cs.y * a1.z + gamma * v0.z; n1.z = cs.y * a0.z + cs.x * a1.z + gamma * v1.z;
      n0.w = cs.x * a0.w - cs.y * a1.w + gamma * v0.w; n1.w = cs.y * a0.w + cs.x * a1.w + gamma * v1.w;
      st_stream4(hg + (size_t)(2 * k) * P + 4 * q, n0);
      st_stream4(hg + (size_t)(2 * k + 1) * P + 4 * q, n1);
      const float* c0 = sC + (2 * k) * R; const float* c1 = c0 + R;
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
  T* yg = static_cast<T*>(p.y) + (size_t)bh * R * P;
  for (int i = tid; i < R * P; i += NT) {
    float s = 0.f;
    for (int w = 0; w < nwaves; ++w) s += sRed[w * R * P + i];
    yg[i] = from_f<T>(s);
  }
}

template <typename T, int R>
hipError_t dispatch_upt(const DecodeParams& p, hipStream_t stream) {
  const int units = (p.N / 2) * (p.P / 4);
  const int nt = units >= 256 ? 256 : (units <= 64 ? 64 : ((units + 63) / 64) * 64);
  const int upt = (units + nt - 1) / nt;
  const int nwaves = nt / 64;
  const size_t lds = sizeof(float) * (3 * (size_t)p.N * R + 2 * (size_t)R * p.P + p.N +
                                      (size_t)nwaves * R * p.P);
  const dim3 grid(p.batch * p.H), block(nt);
  switch (upt) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, R, 1>), grid, block, lds, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, R, 2>), grid, block, lds, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, R, 4>), grid, block, lds, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<T, R, 8>), grid, block, lds, stream, p); break;
    case 16: hipLaunchKernelGGL((decode_kernel<T, R, 16>), grid, block, lds, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_rank(const DecodeParams& p, hipStream_t stream) {
  switch (p.R) {
    case 1: return dispatch_upt<T, 1>(p, stream);
    case 2: return dispatch_upt<T, 2>(p, stream);
    case 4: return dispatch_upt<T, 4>(p, stream);
    case 8: return dispatch_upt<T, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream) {
  if (p.batch == 0 || p.H == 0) return hipSuccess;
  return dtype == M3_BF16 ? dispatch_rank<bf16>(p, stream) : dispatch_rank<float>(p, stream);
}

}  // namespace m3
