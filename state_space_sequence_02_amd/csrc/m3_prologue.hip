// m3_prologue.hip -- the prologue as a stage of its own, for the shapes whose
// fused prologue prefill variant the library does not launch.
//
// The pre-processing is the fused prologue's (the explainer's sec. 3.4 and
// Table 5(a) remark: RMS normalization of B and C followed by learned
// head-specific channel biases; Prop. 2: the step's rotation is dt times the
// generator's angle): every (token, head, rank) column of B, of C and of
// B_prev (N values) is divided by sqrt(mean of its squares + eps) and gets
// bias[h, r, :] added (B_prev takes B's bias), and the step angle of pair k is
// dt_t * theta_raw[.., k].  The results go to the caller's workspace in the
// inputs' layouts and dtype (bf16 values rounded to nearest even), and the plain
// prefill then runs on them.  Both kernels are HBM streams: each input element
// is read once and each result written once.
#include "m3_device.h"
#include "m3_prologue.h"

namespace m3 {
namespace {

constexpr int kNormThreads = 256;

__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Rows [0, nrows) of a [.., H, R, N] array: row i belongs to head (i / R) % H
// and rank i % R.  N / 8 lanes share a row, 8 consecutive values each; the
// sum of squares is reduced over those lanes with xor shuffles (the groups
// are aligned, so no shuffle leaves its row).
template <typename T, int N>
__global__ __launch_bounds__(kNormThreads) void bcnorm_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                              size_t nrows, int H, int R, float eps,
                                                              const float* __restrict__ bias) {
  constexpr int LPR = N / 8;
  constexpr int RPB = kNormThreads / LPR;   // rows per block
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int g = threadIdx.x % LPR;
  if (row >= nrows) return;   // (whole row groups leave together: the shuffles stay inside live groups)
  float v[8];
  load8(src + row * N + g * 8, v);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.f / sqrtf(ss / (float)N + eps);
  float b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (bias) {
    const int r = (int)(row % (size_t)R), h = (int)((row / (size_t)R) % (size_t)H);
    load8(bias + ((size_t)h * R + r) * N + g * 8, b);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * inv + b[i];
  store8(dst + row * N + g * 8, v);
}

// phi[t, k] = dt[t] * theta[t, k] over n4 groups of 4 pairs (NH = N / 2 pairs
// per token, a multiple of 4).
__global__ __launch_bounds__(256) void angle_scale_kernel(const float* __restrict__ dt, const float* __restrict__ theta,
                                                          float* __restrict__ phi, size_t n4, int NH) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float d = dt[(i * 4) / (size_t)NH];
  float4 t = reinterpret_cast<const float4*>(theta)[i];
  t.x *= d; t.y *= d; t.z *= d; t.w *= d;
  reinterpret_cast<float4*>(phi)[i] = t;
}

template <typename T, int N>
hipError_t launch_norm(const void* src, void* dst, size_t nrows, int H, int R, float eps, const float* bias,
                       hipStream_t stream) {
  if (nrows == 0) return hipSuccess;
  constexpr int RPB = kNormThreads / (N / 8);
  const size_t blocks = (nrows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bcnorm_kernel<T, N>), dim3((unsigned)blocks), dim3(kNormThreads), 0, stream,
                     static_cast<const T*>(src), static_cast<T*>(dst), nrows, H, R, eps, bias);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_norm_n(int N, const void* src, void* dst, size_t nrows, int H, int R, float eps, const float* bias,
                         hipStream_t stream) {
  switch (N) {
    case 16: return launch_norm<T, 16>(src, dst, nrows, H, R, eps, bias, stream);
    case 32: return launch_norm<T, 32>(src, dst, nrows, H, R, eps, bias, stream);
    case 64: return launch_norm<T, 64>(src, dst, nrows, H, R, eps, bias, stream);
    case 128: return launch_norm<T, 128>(src, dst, nrows, H, R, eps, bias, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prologue_stage(const PrologueStage& p, hipStream_t stream) {
  const size_t rows = (size_t)p.tokens * p.R;   // (token, head) pairs x ranks
  struct { const void* src; void* dst; size_t n; const float* bias; } jobs[] = {
      {p.B, p.Bn, rows, p.biasB}, {p.C, p.Cn, rows, p.biasC}, {p.Bp, p.Bpn, p.Bp ? (size_t)p.pairs * p.R : 0, p.biasB}};
  for (const auto& j : jobs) {
    const hipError_t e = p.dtype == M3_BF16 ? launch_norm_n<bf16>(p.N, j.src, j.dst, j.n, p.H, p.R, p.eps, j.bias, stream)
                                            : launch_norm_n<float>(p.N, j.src, j.dst, j.n, p.H, p.R, p.eps, j.bias, stream);
    if (e != hipSuccess) return e;
  }
  if (p.theta) {
    const size_t n4 = (size_t)p.tokens * (p.N / 2) / 4;
    if (n4 > 0) {
      hipLaunchKernelGGL(angle_scale_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream,
                         p.dt, p.theta, p.phi, n4, p.N / 2);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace m3
