// m3_fused_kernel.h -- single-pass chunked Mamba-3 prefill kernel for gfx950.
//
// One workgroup per (sequence, chunk): 8 waves for N <= 64, 16 for N >= 128
// (where a chunk needs a whole CU's LDS).  Each input element is read from HBM
// once; besides the outputs a chunk writes one N x P fp32 state (and, when its
// predecessor's state was not yet published, its own affine map).
//
// The arithmetic is the exact chunked rearrangement of the recurrence
//   H_t = alpha_t R(phi_t) H_{t-1} + beta_t R(phi_t) V_{t-1} + gamma_t V_t,
//   V_t = B_t X_t^T,  Y_t = H_t^T C_t
// (Mamba-3 explainer panels 1, 3, 4; its chunked-algorithm remark in sec. 3.3;
// the decay x two-band structured mask of the paper page's Figure 1 and the
// explainer's Eq. 7; data-dependent RoPE, Prop. 3/4 and Eq. 11).  With
// chunk-local l_t = sum_{t0<=j<=t} dt_j A and Phi_t = sum_{t0<=j<=t} phi_j:
//
//   Y_t  = exp(l_t) C~_t^T S_in + sum_{t0<=s<=t} exp(l_t-l_s) m_ts (C~_t . B~_s) X_s
//   m_ts = gamma_s (s == t),  gamma_s + (1-lam_{s+1}) dt_{s+1} (s < t)
//   S_out = a_c R(Psi_c) S_in + U_c,   U_c = R(Psi_c) sum_s exp(l_end-l_s) w_s B~_s X_s^T
//   w_s  = gamma_s + (1-lam_{s+1}) dt_{s+1}   (the next token's delayed endpoint,
//          zero after the last token of the sequence)
//   B~_s = R(-Phi_s) B_s,  C~_t = R(-Phi_t) C_t,  a_c = exp(l_end), Psi_c = Phi_end
// S_in of the first chunk is h0 + (1-lam_0) dt_0 B_prev X_prev^T; S_out of the
// last chunk is the final state.  Exponents are differences l_t - l_s <= 0.
//
// Passing states between chunks (the setupai page's "hardware-aware parallel
// scan"): chunk c's map S -> a_c R(Psi_c) S + U_c is affine, so a chunk whose
// predecessor has not finished composes the predecessors' maps itself
// (decoupled look-back).  Flags per chunk: 1 = map published, 2 = S_out
// published, tagged with the call's epoch (a flag of another call reads as 0).
// Wave 0 reads the predecessors' flags once before the look-back proper (at
// the start when maps are in use, else after staging); a chunk publishes its
// map only when maps are in use and its predecessor's state was not there.
// Workgroups take chunk-major tickets from an atomic counter, so every chunk a
// workgroup looks back at holds a lower ticket and is already running: every
// wait ends.  A bounded spin turns a wait that never ends into NaN outputs.
// Maps and states move as 16-byte buffer loads/stores with the cache policy of
// device-scope atomics, each lane's values in register order; flags and the
// per-chunk records are device-scope relaxed atomics.  A wave waits for its
// stores to complete (s_waitcnt 0) and the last wave to finish raises the flag
// (an LDS counter), so no cache-wide write-back/invalidate and no workgroup
// barrier is needed to publish.
//
// Work order inside a workgroup:
//   A  all global loads issued (raw buffer loads, rows past the sequence end
//      read as zeros); chunk-local cumulative log decay and phases: each
//      thread scans its own tokens in registers, lanes combine with shuffles,
//      waves with one barrier; cos/sin table of Phi in LDS
//   B  stage B~ (rotated) and X in LDS; the wave's C~ rows are kept in
//      registers as MFMA operands; wave 0 polls the predecessors' flags
//      (when maps are in use, this poll is issued with the loads in A)
//   C  U = R(Psi) sum_s W_s B~_s^T X_s on MFMA (operands by LDS transpose reads);
//      publish the map if needed
//   D  look back for S_in; S_out = a R(Psi) S_in + U; stores issued
//   E  outputs of the wave's 16-row tiles, together: C~ S_in, then per 32-row
//      source block the masked intra-chunk products on MFMA (each B~ / X read
//      serves every tile of the wave); flag 2 raised; y stored.
//
// Variants (template flags): G, the gated readout, replaces the y store by the
// rank contraction with the rank-expanded SiLU gate (its operands loaded
// during phase C and written to the free tail of the cos/sin region once the
// table is dead); PRO, the prologue,
// normalises B and C rows (and B_prev) with their biases while they are
// staged and scales the raw angles by dt before the phase scan.
//
// Column order: X is staged in LDS with its columns permuted so that the
// 16-column MFMA tile pt holds head columns TPt*l + pt (l = 0..15, TPt = P/16).
// U, the chunk states in the workspace (stored in register order), S_in^T and
// the output accumulators all follow that order; a lane then holds TPt
// consecutive head columns of each of its output rows, and y leaves as full
// row segments.  h0, h_out, x_prev and y are read/written in the head's own
// column order.
#pragma once

#include <algorithm>
#include <atomic>

#include "m3_device.h"

namespace m3 {
namespace fused {

constexpr int kMaxBatch = 12;         // 16-byte B/X loads per thread per batch, at most
constexpr int kMapGroup = 1;        // predecessor maps loaded per round trip
constexpr int kAngleCap = kFusedAngleCap;   // max Q * N/2 angles per chunk


__host__ __device__ constexpr int round_up_i(int a, int b) { return (a + b - 1) / b * b; }

__host__ __device__ constexpr size_t max_sz(size_t a, size_t b) { return a > b ? a : b; }

struct Lds {
  size_t row, rw, W, csH, B, X, misc, pb, total;
  size_t segl, sega;   // scan scratch, inside B (used only before B~ is staged)
};
// LDS row stride (elements) of the X tile.  bf16 X is read with 8-byte
// transposing reads in which 16 lanes take 4 columns of 4 consecutive rows:
// a stride of 8 or 24 banks (16 or 48 elements mod 64) puts the 4 rows on
// disjoint banks.  fp32 X is read one element per lane along a row.
__host__ __device__ constexpr int x_stride(int P, int esize) {
  return esize == 2 ? (P == 16 ? 16 : P + 16) : P + 8;
}

// row: per (token, rank) row float4 {l, w, gamma, W}
// rw: per row exp(l_be - l) w with be the last row of the row's 32-row block
//     (the factored decay of the off-diagonal mask blocks);  W: per row W
// csH: cos/sin of Phi [Q][N/2 + 1] while B~, C~ and R(Psi) are formed, then S_in^T [P][N+8].
//      Within a row, pair k = 4g + j is at column j * N/8 + g: the 16 lanes of an
//      access that take consecutive groups g of one row read consecutive entries.
// B: B~ [QRp][N+8];  X: X [QRp][P+8] (permuted columns)
// segl: kWaves floats, sega: kWaves x N/8 float4 (per-wave scan totals)
// misc: 8 ints of workgroup scalars, then (prologue) the R column-norm factors of B_prev
// pb: the prologue's bias tables [2][R][N] fp32 (B's, then C's), only when pro.
__host__ __device__ constexpr Lds lds_layout(int Q, int R, int N, int P, int esize, int pro = 0) {
  const int QRp = round_up_i(Q * R, 32);
  const int kWaves = fused_threads(N) / 64;
  const size_t scan = sizeof(float) * kWaves + sizeof(float4) * (size_t)kWaves * (N / 8);
  Lds o{};
  o.row = 0;
  o.rw = o.row + sizeof(float4) * QRp;
  o.W = o.rw + sizeof(float) * QRp;
  o.csH = o.W + sizeof(float) * QRp;
  o.B = o.csH + round_up_i((int)max_sz(sizeof(float2) * (size_t)Q * (N / 2 + 1), (size_t)esize * P * (N + 8)), 16);
  o.X = o.B + round_up_i((int)max_sz((size_t)esize * QRp * (N + 8), scan), 16);
  o.misc = o.X + (size_t)esize * QRp * x_stride(P, esize);
  o.pb = o.misc + 64;
  o.total = o.pb + (pro ? sizeof(float) * (size_t)R * (2 * N + 4) : 0);   // B's [R][N], C's [R][N + 4]
  o.segl = o.B;
  o.sega = o.B + sizeof(float) * kWaves;
  return o;
}

__device__ __forceinline__ size_t tok_index(const FusedParams& p, int b, int t, int h) {
  return ((size_t)b * p.L + t) * p.H + h;
}

// Device-scope relaxed 8-byte load/store of two floats.
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const unsigned long long v =
      __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}
__device__ __forceinline__ void st_dev2(float* p, float a, float b) {
  const unsigned long long v = (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this wave issued has completed.
__device__ __forceinline__ void mem_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Every one of the workgroup's `nwaves` waves calls this once after
// mem_done(); the last one to arrive raises flag `f` to `val`.  `ctr` is an
// LDS counter starting at 0.
__device__ __forceinline__ void arrive_and_flag(int* ctr, unsigned long long* f, unsigned long long val, int nwaves,
                                                bool lane0 = (threadIdx.x & 63) == 0) {
  if (lane0) {
    const int n = atomicAdd(ctr, 1);
    if (n == nwaves - 1) __hip_atomic_store(f, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Raw 8-element loads (bf16: 16 B, fp32: 32 B).
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { uint4 v; };
template <> struct Raw8<float> { uint4 v[2]; };
__device__ __forceinline__ void raw_load(Raw8<bf16>& r, const bf16* p) { r.v = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void raw_load(Raw8<float>& r, const float* p) {
  r.v[0] = *reinterpret_cast<const uint4*>(p);
  r.v[1] = *reinterpret_cast<const uint4*>(p + 4);
}
__device__ __forceinline__ void raw_zero(Raw8<bf16>& r) { r.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw_zero(Raw8<float>& r) { r.v[0] = r.v[1] = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void raw_store(bf16* d, const Raw8<bf16>& r) { *reinterpret_cast<uint4*>(d) = r.v; }
__device__ __forceinline__ void raw_store(float* d, const Raw8<float>& r) {
  reinterpret_cast<uint4*>(d)[0] = r.v[0];
  reinterpret_cast<uint4*>(d)[1] = r.v[1];
}
__device__ __forceinline__ void raw_unpack(const Raw8<bf16>& r, float (&v)[8]) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void raw_unpack(const Raw8<float>& r, float (&v)[8]) {
  v[0] = __uint_as_float(r.v[0].x); v[1] = __uint_as_float(r.v[0].y);
  v[2] = __uint_as_float(r.v[0].z); v[3] = __uint_as_float(r.v[0].w);
  v[4] = __uint_as_float(r.v[1].x); v[5] = __uint_as_float(r.v[1].y);
  v[6] = __uint_as_float(r.v[1].z); v[7] = __uint_as_float(r.v[1].w);
}
template <typename T> __device__ __forceinline__ void store8(T* d, const float (&v)[8]);
template <> __device__ __forceinline__ void store8<bf16>(bf16* d, const float (&v)[8]) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = static_cast<bf16>(v[j]);
  *reinterpret_cast<bf16x8*>(d) = o;
}
template <> __device__ __forceinline__ void store8<float>(float* d, const float (&v)[8]) {
  reinterpret_cast<float4*>(d)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(d)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// R(-phi) on the 4 pairs of 8 consecutive state entries (even start); the
// cos/sin of pair j are at cs[j * stride].
__device__ __forceinline__ void rotate_neg(float (&v)[8], const float2* cs, int stride) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float2 q = cs[j * stride];
    const float u = v[2 * j], w = v[2 * j + 1];
    v[2 * j] = q.x * u + q.y * w;
    v[2 * j + 1] = -q.y * u + q.x * w;
  }
}

// MFMA operand fragment for column c0 + lane%16 of a row-major [row][col] LDS
// tile, holding rows r0..r0+3 in slots 0..3 and r1..r1+3 in slots 4..7 (r0, r1
// may depend on the lane's group lane/16).  bf16: two ds_read_b64_tr_b16 (within
// each 16-lane group, lane i supplies row r + i/4, columns c0 + 4*(i%4)..+3, and
// lane l receives rows r..r+3 of column c0 + l).  fp32: eight scalar reads.
// (i: the lane's index within its 16-lane group, lane % 16)
__device__ __forceinline__ void frag_tr(Frag<bf16>& f, const bf16* base, int stride, int r0, int r1, int c0,
                                        int i = threadIdx.x & 15) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const bf16* p0 = base + (r0 + (i >> 2)) * stride + c0 + 4 * (i & 3);
  const bf16* p1 = base + (r1 + (i >> 2)) * stride + c0 + 4 * (i & 3);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  const v4i16 ab[2] = {a, b};
  f.v = *reinterpret_cast<const bf16x8*>(ab);
}
__device__ __forceinline__ void frag_tr(Frag<float>& f, const float* base, int stride, int r0, int r1, int c0) {
  const int c = c0 + (threadIdx.x & 15);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = base[(r0 + e) * stride + c];
    f.v[4 + e] = base[(r1 + e) * stride + c];
  }
}

// Raw buffer access: a descriptor with a byte extent; loads at offsets past
// the extent return zeros.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kCpolDevice = 16;   // sc1: the coherence bit of device-scope atomic accesses
__device__ __forceinline__ Rsrc buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float buf_load_f32(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float4 buf_load_f32x4(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void raw_load_buf(Raw8<bf16>& d, Rsrc r, uint32_t off) {
  d.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void raw_load_buf(Raw8<float>& d, Rsrc r, uint32_t off) {
  d.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  d.v[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
}

// 16-byte loads/stores with the cache policy of device-scope atomics (sc1):
// written by one workgroup, read by another after a flag.
__device__ __forceinline__ f32x4 buf_load_dev4(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ void buf_store_dev4(Rsrc r, uint32_t off, f32x4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCpolDevice);
}

// Stores the 8 head columns c0..c0+7 of one X row into the permuted LDS row:
// head column c goes to LDS column (c % TPt) * 16 + c / TPt.  The 8/TPt
// columns that land side by side go out as one store (c0 is a multiple of 8,
// so such a run starts on a multiple of its own size).
template <int TPt, typename T>
__device__ __forceinline__ void store_x_permuted(T* row, int c0, const Raw8<T>& r) {
  T v[8];
  static_assert(sizeof(Raw8<T>) == sizeof(v), "raw size");
  __builtin_memcpy(v, &r, sizeof(v));
  constexpr int RUN = TPt < 8 ? 8 / TPt : 1;   // consecutive LDS columns per store
#pragma unroll
  for (int t = 0; t < (TPt < 8 ? TPt : 8); ++t) {
    T* d = row + t * 16 + c0 / TPt;
    T run[RUN];
#pragma unroll
    for (int m = 0; m < RUN; ++m) run[m] = v[t + m * TPt];
    if constexpr (RUN * sizeof(T) == 4) {
      uint32_t w;
      __builtin_memcpy(&w, run, 4);
      *reinterpret_cast<uint32_t*>(d) = w;
    } else if constexpr (RUN * sizeof(T) == 8) {
      uint2 w;
      __builtin_memcpy(&w, run, 8);
      *reinterpret_cast<uint2*>(d) = w;
    } else if constexpr (RUN * sizeof(T) == 16) {
      uint4 w;
      __builtin_memcpy(&w, run, 16);
      *reinterpret_cast<uint4*>(d) = w;
    } else {
#pragma unroll
      for (int m = 0; m < RUN; ++m) d[m] = run[m];
    }
  }
}

// Stores n (= TPt) consecutive outputs of one row.
template <typename T, int TPt>
__device__ __forceinline__ void store_row(T* d, const float (&v)[TPt]) {
  if constexpr (sizeof(T) == 2 && TPt % 2 == 0) {
    uint32_t w[TPt / 2];
#pragma unroll
    for (int i = 0; i < TPt / 2; ++i) {
      const bf16 lo = static_cast<bf16>(v[2 * i]), hi = static_cast<bf16>(v[2 * i + 1]);
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    if constexpr (TPt == 2) *reinterpret_cast<uint32_t*>(d) = w[0];
    else if constexpr (TPt == 4) *reinterpret_cast<uint2*>(d) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint4*>(d) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (sizeof(T) == 4 && TPt % 4 == 0) {
#pragma unroll
    for (int i = 0; i < TPt / 4; ++i)
      reinterpret_cast<float4*>(d)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < TPt; ++i) d[i] = from_f<T>(v[i]);
  }
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 sub4(float4 a, float4 b) { return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w); }
// v of the lane kRor places before this one, cyclically, within its row of
// 16 lanes (DPP row_ror; every lane of the row must be active).
template <int kRor>
__device__ __forceinline__ float dpp_row_ror(float v) {
  static_assert(kRor >= 1 && kRor <= 15, "row_ror takes 1..15");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + kRor, 0xF, 0xF, false));
}
__device__ __forceinline__ float4 shfl_up4(float4 v, int off) {
  return make_float4(__shfl_up(v.x, off), __shfl_up(v.y, off), __shfl_up(v.z, off), __shfl_up(v.w, off));
}

// RT: output row tiles per wave (the chunk has at most RT * 16 * kWaves rows);
// register arrays are sized by it.
// Waves per SIMD the register allocation must allow: a 1024-thread workgroup
// needs 4 (128 VGPRs); a 512-thread one asks for 4 too, so two workgroups share
// a CU, unless at the largest chunk it takes two would not fit the CU's LDS
// anyway -- then 2 (256 VGPRs), which keeps those variants free of spills.
template <typename T, int N, int P, int R, int RT, bool PRO>
constexpr int prefill_waves_per_simd() {
  if (fused_threads(N) == 1024) return 4;
  if (N > 64 || RT > 2) return 2;
  constexpr int kQmax = RT * 16 * (fused_threads(N) / 64) / R;
  return 2 * lds_layout(kQmax, R, N, P, (int)sizeof(T), PRO ? 1 : 0).total > (size_t)kLdsBudget ? 2 : 4;
}

// G: the gated readout (out [b,L,H,P]) replaces the y store.  PRO: the fused
// prologue (B, C, B_prev column RMS norm + biases; angle = dt x raw angle).
template <typename T, int N, int P, int R, int RT, bool G, bool PRO>
__global__ __launch_bounds__(fused_threads(N), (prefill_waves_per_simd<T, N, P, R, RT, PRO>())) void prefill_kernel(FusedParams p) {
  constexpr int kThreads = fused_threads(N);
  constexpr int kWaves = kThreads / 64;
  constexpr int NH = N / 2;
  constexpr int NG = NH / 4;                  // 4-pair column groups of the angle table
  constexpr int CSS = NH + 1;                 // angle table row stride (float2): rows 2 banks apart
  // angle table column of pair k (4-pair group k/4, slot k%4)
  auto cs_col = [](int k) { return (k & 3) * NG + (k >> 2); };
  constexpr int NK = (N + 31) / 32;           // 32-wide slices of the state dimension
  constexpr int TPt = P / 16;                 // 16-column tiles of the head dimension
  constexpr int TNt = N / 16;                 // 16-row tiles of the state dimension
  // state tiles (phases C, D): wave w owns n-tiles nslot + NGRP*i and p-tiles pslot + WPN*j
  constexpr int NGRP = TNt < kWaves ? TNt : kWaves;
  constexpr int NPW = TNt / NGRP;
  constexpr int WPN = kWaves / NGRP;
  constexpr int PTW = (TPt + WPN - 1) / WPN;
  constexpr int NS = N + 8;                   // LDS row stride of B~ and S_in^T
  constexpr int XS = x_stride(P, sizeof(T));  // LDS row stride of X
  constexpr int LOGR = R == 1 ? 0 : R == 2 ? 1 : R == 4 ? 2 : 3;
  constexpr int RTW = RT;                     // max output row tiles per wave
  // B/X loads per thread per batch: the whole chunk in one batch when it fits
  constexpr int kBatchRaw = (round_up_i(RT * 16 * kWaves * (N / 8), kThreads) + RT * 16 * kWaves * (P / 8) +
                             kThreads - 1) / kThreads;
  constexpr int kBatch = kBatchRaw < kMaxBatch ? kBatchRaw : kMaxBatch;
  const int tid = threadIdx.x;

  extern __shared__ __align__(16) unsigned char smem[];
  const int Q = p.Q;
  const Lds lay = lds_layout(Q, R, N, P, sizeof(T), PRO ? 1 : 0);
  float* s_pb = reinterpret_cast<float*>(smem + lay.pb);   // prologue biases (PRO)
  float4* s_row = reinterpret_cast<float4*>(smem + lay.row);
  float* s_rw = reinterpret_cast<float*>(smem + lay.rw);
  float* s_W = reinterpret_cast<float*>(smem + lay.W);
  float* s_segl = reinterpret_cast<float*>(smem + lay.segl);
  float4* s_sega = reinterpret_cast<float4*>(smem + lay.sega);
  float2* s_cs = reinterpret_cast<float2*>(smem + lay.csH);
  T* s_H = reinterpret_cast<T*>(smem + lay.csH);
  T* s_B = reinterpret_cast<T*>(smem + lay.B);
  T* s_X = reinterpret_cast<T*>(smem + lay.X);
  int* s_misc = reinterpret_cast<int*>(smem + lay.misc);

  // ---- ticket: chunk-major order over all sequences ----
  // (the taker of the last ticket readies the control word for the next call:
  // count 0, next epoch.  A count past the last ticket only arises in a
  // workspace that was not zero-filled: the workgroup records the error and
  // computes nothing.)
  const int nbh = p.batch * p.H;
  if (tid == 0) {
    const unsigned total = (unsigned)(nbh * p.nc);
    const unsigned long long w = atomicAdd(p.ctl, 1ull);
    const unsigned cnt = (unsigned)(w & kTicketMask);
    const unsigned long long epoch = w >> kTicketBits;
    if (cnt == total - 1)
      __hip_atomic_store(p.ctl, (epoch + 1) << kTicketBits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (cnt >= total)
      __hip_atomic_fetch_or(p.err, (unsigned long long)kErrControl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_misc[0] = cnt < total ? (int)cnt : -1;
    s_misc[6] = (int)(unsigned)(epoch + 1);
    s_misc[7] = (int)(unsigned)((epoch + 1) >> 32);
  }
  __syncthreads();
  // (read into a scalar register: the chunk's indices and addresses derived
  // from it are then scalar too)
  const int ticket = __builtin_amdgcn_readfirstlane(s_misc[0]);
  if (ticket < 0) return;   // (uniform: the whole workgroup leaves)
  // this call's flag tag; flag_state() reads a flag of another call as 0
  const unsigned long long tag = ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane(s_misc[7]) << 32) |
                                 (unsigned)__builtin_amdgcn_readfirstlane(s_misc[6]);
  auto flag_state = [&](unsigned long long f) { return (f >> 2) == tag ? (unsigned)(f & 3u) : 0u; };
  const int QRp = round_up_i(Q * R, 32);
  const int MT = QRp / 16;
  const size_t tstride = (size_t)p.H;           // token step in [b, L, H] arrays
  const size_t rowstepB = tstride * R * N, rowstepX = tstride * R * P;
  constexpr uint32_t kOff = 0x80000000u;        // an offset past every extent
  const uint32_t tsb = (uint32_t)tstride * 4;   // token step of [b, L, H] fp32 arrays, bytes
  const uint32_t esz = sizeof(T);
  const uint32_t rsB = (uint32_t)rowstepB * esz, rsX = (uint32_t)rowstepX * esz;
  float dv, lmv, dnv, lmnv_raw;
  // tokens per angle thread, at most (NSEG = min(threads / NG, Q) segments of
  // Q / NSEG tokens; Q * R rows fill at most RT row tiles per wave)
  constexpr int kQmaxT = RT * 16 * kWaves / R;
  constexpr int kAL0 = kQmaxT / (kThreads / NG) > 1 ? kQmaxT / (kThreads / NG) : 1;
  constexpr int kAL = kAL0 < 4 ? kAL0 : 4;
  float4 th4[kAL];
  float thdt[kAL];        // PRO: dt of the angle tokens
  float4 pbv0, pbv1;      // PRO: this thread's bias items (B's, C's)
  Raw8<T> raw[kBatch];
  Raw8<T> craw[RTW][NK];
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int nslot = wave % NGRP, pslot = wave / NGRP;
  // head column held by lane l16 in 16-column tile pt (the permuted order)
  auto hcol = [&](int pt) { return l16 * TPt + pt; };
  // output row tiles of this wave, paired (w, MT-1-w) for balance
  const int ntiles_w = (MT + kWaves - 1 - wave) / kWaves;
  // (one tile per wave: the second half of the waves takes the tiles in reverse
  // order, so waves w and w + 4 -- one SIMD when waves go round-robin over the
  // four -- hold a light and a heavy tile)
  const bool rev = RT == 1 && MT == kWaves && wave >= kWaves / 2;
  auto tile_of = [&](int k) {
    if (rev) return MT - 1 - (wave - kWaves / 2);
    const int pair = k >> 1;
    return (k & 1) ? MT - 1 - (wave + 2 * kWaves * pair) : wave + 2 * kWaves * pair;
  };
  // angles: thread -> (segment sg, column group cg): tokens sg*ALEN .. +ALEN-1,
  // pairs 4cg .. 4cg+3 (ALEN <= 4 since Q * N/2 <= kAngleCap)
  const int NSEG = min(kThreads / NG, Q);
  const int ALEN = Q / NSEG;
  const int cg = tid % NG, sg = tid / NG;
  // B items are padded to a multiple of the workgroup size so every item slot
  // of a batch reads one tensor (a uniform descriptor).
  const int nbi = QRp * (N / 8), nxi = QRp * (P / 8);
  const int nbp = round_up_i(nbi, kThreads), ntot = nbp + nxi;

  // ---- A: every global load of the chunk is issued before any of it is used ----
  // Raw buffer loads: 32-bit offsets from per-chunk descriptors whose extent
  // ends after the chunk's last valid token, so rows past the sequence end (and
  // unused item slots) read as zeros without masks or branches.  (A load under
  // a branch merged with a default value would make the compiler wait for it at
  // the merge and serialise the batch.)
  auto batch_loads = [&](Rsrc rB, Rsrc rX, int base) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kThreads;
      if (base - tid + u * kThreads < nbp) {     // uniform: this slot reads B
        const int row = i / (N / 8), g = i - row * (N / 8);
        raw_load_buf(raw[u], rB, i < nbi ? (uint32_t)(row >> LOGR) * rsB + ((row & (R - 1)) * N + g * 8) * esz : kOff);
      } else {
        const int j = i - nbp;
        const int row = j / (P / 8), g = j - row * (P / 8);
        raw_load_buf(raw[u], rX, j < nxi ? (uint32_t)(row >> LOGR) * rsX + ((row & (R - 1)) * P + g * 8) * esz : kOff);
      }
    }
  };
  auto issue_chunk = [&](int tk) {
    const int c = tk / nbh, bh = tk - c * nbh;
    const int b = bh / p.H, h = bh - b * p.H;
    const int t0 = c * Q;
    const int nt = min(Q, p.L - t0);
    const size_t tok0 = tok_index(p, b, t0, h);
    const Rsrc rD = buf_rsrc(p.dt + tok0, (nt - 1) * tsb + 4);
    const Rsrc rL = buf_rsrc(p.lam + tok0, (nt - 1) * tsb + 4);
    const int nnext = min(nt, p.L - t0 - 1);    // tokens whose successor exists
    const Rsrc rDn = buf_rsrc(p.dt + tok0 + tstride, nnext > 0 ? (nnext - 1) * tsb + 4 : 0);
    const Rsrc rLn = buf_rsrc(p.lam + tok0 + tstride, nnext > 0 ? (nnext - 1) * tsb + 4 : 0);
    if constexpr (PRO) {   // first, so they are back before the rest
      constexpr int kPb = R * N / 4;                      // float4 items per bias table
      const Rsrc rBB = buf_rsrc(p.biasB ? p.biasB + (size_t)h * R * N : nullptr, p.biasB ? R * N * 4 : 0);
      const Rsrc rBC = buf_rsrc(p.biasC ? p.biasC + (size_t)h * R * N : nullptr, p.biasC ? R * N * 4 : 0);
      pbv0 = buf_load_f32x4(rBB, tid < kPb ? 16u * tid : kOff);
      pbv1 = buf_load_f32x4(rBC, tid < kPb ? 16u * tid : kOff);
    }
    const uint32_t toff = tid < Q ? tid * tsb : kOff;
    dv = buf_load_f32(rD, toff);
    lmv = buf_load_f32(rL, toff);
    dnv = buf_load_f32(rDn, toff);
    lmnv_raw = buf_load_f32(rLn, toff);
    const Rsrc rT = buf_rsrc(p.theta ? p.theta + tok0 * NH : nullptr, p.theta ? (nt - 1) * tsb * NH + NH * 4 : 0);
#pragma unroll
    for (int j = 0; j < kAL; ++j) {
      const bool ok = j < ALEN && sg < NSEG;
      th4[j] = buf_load_f32x4(rT, ok ? (uint32_t)(sg * ALEN + j) * tsb * NH + 16 * cg : kOff);
    }
    if constexpr (PRO) {
#pragma unroll
      for (int j = 0; j < kAL; ++j) {
        const bool ok = j < ALEN && sg < NSEG;
        thdt[j] = buf_load_f32(rD, ok ? (uint32_t)(sg * ALEN + j) * tsb : kOff);
      }
    }
    const uint32_t extB = (uint32_t)(nt - 1) * rsB + R * N * esz;
    batch_loads(buf_rsrc(static_cast<const T*>(p.B) + tok0 * R * N, extB),
                buf_rsrc(static_cast<const T*>(p.x) + tok0 * R * P, (uint32_t)(nt - 1) * rsX + R * P * esz), tid);
    const Rsrc rC = buf_rsrc(static_cast<const T*>(p.C) + tok0 * R * N, extB);
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
      const int row_a = (k < ntiles_w ? tile_of(k) : 0) * 16 + l16;
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        const int n0 = kn * 32 + 8 * g4;
        const bool ok = k < ntiles_w && n0 < N;
        raw_load_buf(craw[k][kn], rC, ok ? (uint32_t)(row_a >> LOGR) * rsB + ((row_a & (R - 1)) * N + n0) * esz : kOff);
      }
    }
  };
  issue_chunk(ticket);
  const int c = ticket / nbh, bh = ticket - c * nbh;
  const int b = bh / p.H, h = bh - b * p.H;
  const int t0 = c * Q;
  const int nt = min(Q, p.L - t0);
  const int rows = nt * R;
  const size_t tok0 = tok_index(p, b, t0, h);
  unsigned long long* flags = p.flags + (size_t)bh * p.nc;
  // With maps, wave 0 reads the predecessors' flags right away: the answer
  // (whether the predecessor's state is there, i.e. whether to publish a map)
  // is then in before the map is done, and serves as the look-back's first step.
  const int W0 = min(c, 64);
  unsigned fpoll = 1u;
  if (p.use_maps && wave == 0 && lane < W0)
    fpoll = flag_state(__hip_atomic_load(flags + c - 1 - lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const T* Bg = static_cast<const T*>(p.B) + tok0 * R * N;
  const T* Xg = static_cast<const T*>(p.x) + tok0 * R * P;
  const float A = p.A[h];
  if (tid == 0) {
    s_misc[3] = 0;      // wave counter: map published
    s_misc[4] = 0;      // wave counter: state published
  }
  float* s_bps = reinterpret_cast<float*>(s_misc + 8);   // PRO: B_prev column norm factors [R]
  if constexpr (PRO) {
    constexpr int kPb = R * N / 4;
    if (tid < kPb) {
      *reinterpret_cast<float4*>(s_pb + 4 * tid) = pbv0;
      *reinterpret_cast<float4*>(s_pb + R * N + (4 * tid / N) * (N + 4) + 4 * tid % N) = pbv1;
    }
    // a sequence's first chunk: wave 0 reduces B_prev's column norms now, into
    // LDS, so the state set-up after the look-back holds no extra registers
    if (c == 0 && p.Bp && wave == 0) {
      const T* Bp0 = static_cast<const T*>(p.Bp) + (size_t)bh * R * N;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float ss = 0.f;
        for (int n = lane; n < N; n += 64) {
          const float t = to_f(Bp0[r * N + n]);
          ss += t * t;
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        if (lane == 0) s_bps[r] = rsqrtf(ss / (float)N + p.eps);
      }
    }
  }
  const float lmnv = (t0 + tid + 1 < p.L && tid < nt) ? lmnv_raw : 1.f;   // (only multiplies dnv = 0 otherwise)

  // chunk-local cumulative log decay (token tid) and phases (this thread's
  // tokens and pairs): in-register / in-wave scans, one barrier across waves
  float gv = 0.f, wv = 0.f, lsc = 0.f;
  if (tid < Q) {
    gv = lmv * dv;
    wv = gv + (1.f - lmnv) * dnv;
    lsc = dv * A;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(lsc, off);
    if (lane >= off) lsc += u;
  }
  if constexpr (PRO) {   // raw angles: the step's angle is dt x theta
#pragma unroll
    for (int j = 0; j < kAL; ++j) {
      const float d = thdt[j];
      th4[j] = make_float4(d * th4[j].x, d * th4[j].y, d * th4[j].z, d * th4[j].w);
    }
  }
#pragma unroll
  for (int j = 1; j < kAL; ++j)
    if (j < ALEN) th4[j] = add4(th4[j], th4[j - 1]);
  float4 atot = th4[0];   // this thread's segment total (constant indices only:
#pragma unroll               // a run-time index would put th4 in private memory)
  for (int j = 1; j < kAL; ++j)
    if (j < ALEN) atot = th4[j];
  float4 ainc = atot;
#pragma unroll
  for (int off = NG; off < 64; off <<= 1) {
    const float4 u = shfl_up4(ainc, off);
    if (lane >= off) ainc = add4(ainc, u);
  }
  if (lane == 63) s_segl[wave] = lsc;
  if (lane >= 64 - NG) s_sega[wave * NG + cg] = ainc;
  __syncthreads();
  float lbase = 0.f, l_end = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float t = s_segl[w];
    if (w < wave) lbase += t;
    l_end += t;
  }
  float4 abase = sub4(ainc, atot);
  for (int w = 0; w < wave; ++w) abase = add4(abase, s_sega[w * NG + cg]);
  __syncthreads();   // scan scratch (inside B's space) is dead after this
  if (tid < Q) {
    const float lv = lsc + lbase;
    const float W = tid < nt ? __expf(l_end - lv) * wv : 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s_row[tid * R + r] = make_float4(lv, wv, gv, W);
      s_W[tid * R + r] = W;
    }
  }
  for (int i = Q * R + tid; i < QRp; i += kThreads) {
    s_row[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    s_W[i] = 0.f;
  }
  if (sg < NSEG) {
#pragma unroll
    for (int j = 0; j < kAL; ++j) {
      if (j < ALEN) {
        const float4 ph = add4(abase, th4[j]);
        float s0, c0, s1, c1, s2, c2, s3, c3;
        __sincosf(ph.x, &s0, &c0);
        __sincosf(ph.y, &s1, &c1);
        __sincosf(ph.z, &s2, &c2);
        __sincosf(ph.w, &s3, &c3);
        float2* d = s_cs + (sg * ALEN + j) * CSS + cg;
        d[0] = make_float2(c0, s0);
        d[NG] = make_float2(c1, s1);
        d[2 * NG] = make_float2(c2, s2);
        d[3 * NG] = make_float2(c3, s3);
      }
    }
  }
  __syncthreads();   // angles done
  // Off-diagonal mask blocks use exp(l_t - l_s) = exp(l_t - l_be) exp(l_be - l_s)
  // with be the last valid row of the source block (s <= be <= t: both factors
  // <= 1); the second factor times the two-band weight is kept per row.
  for (int k = tid; k < QRp; k += kThreads) {
    float v = 0.f;
    if (k < rows) {
      const float4 rk = s_row[k];
      v = __expf(s_row[min(k | 31, rows - 1)].x - rk.x) * rk.y;
    }
    s_rw[k] = v;
  }

  // ---- B: stage B~ = R(-Phi_s) B_s and X (permuted columns) ----
  // PRO: the B items of one thread (tid + multiples of kThreads) all have the
  // same rank and 8-column group, so its 8 bias values are read once
  static_assert(kThreads % (N / 8) == 0 && (kThreads / (N / 8)) % R == 0, "B item -> (rank, columns) per thread");
  float bbr[8];
  if constexpr (PRO) {
    const float* bb = s_pb + ((tid / (N / 8)) & (R - 1)) * N + (tid % (N / 8)) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) bbr[e] = bb[e];
  }
  for (int base = tid; base < ntot; base += kThreads * kBatch) {
    if (base != tid)
      batch_loads(buf_rsrc(Bg, (uint32_t)(nt - 1) * rsB + R * N * esz),
                  buf_rsrc(Xg, (uint32_t)(nt - 1) * rsX + R * P * esz), base);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + u * kThreads;
      float pscale = 1.f;
      if constexpr (PRO) {   // every lane: a B row's N/8 items sit in consecutive lanes
        float v[8];
        raw_unpack(raw[u], v);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        if constexpr (N / 8 == 16) {   // a row is one 16-lane DPP row: rotate-and-add
          ss += dpp_row_ror<8>(ss);
          ss += dpp_row_ror<4>(ss);
          ss += dpp_row_ror<2>(ss);
          ss += dpp_row_ror<1>(ss);
        } else {
#pragma unroll
          for (int off = 1; off < N / 8; off <<= 1) ss += __shfl_xor(ss, off);
        }
        pscale = rsqrtf(ss / (float)N + p.eps);
      }
      if (i < nbi) {
        const int row = i / (N / 8), ng = i - row * (N / 8);
        float v[8];
        raw_unpack(raw[u], v);
        if constexpr (PRO) {
          if (row < rows) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * pscale + bbr[e];
          }
        }
        if (row < rows) rotate_neg(v, s_cs + (row >> LOGR) * CSS + ng, NG);
        store8<T>(s_B + row * NS + ng * 8, v);
      } else if (i >= nbp && i < ntot) {
        const int j = i - nbp;
        const int row = j / (P / 8), pg = j - row * (P / 8);
        store_x_permuted<TPt>(s_X + row * XS, pg * 8, raw[u]);
      }
    }
  }
  // C~ fragments of this wave's output rows (rotated by -Phi_t)
  Frag<T> cf[RTW][NK];
#pragma unroll
  for (int k = 0; k < RTW; ++k) {
    const int row_a = (k < ntiles_w ? tile_of(k) : 0) * 16 + l16;
    const int ta = row_a < rows ? row_a >> LOGR : 0;
    float cscale = 1.f;
    if constexpr (PRO) {   // a C row: NK slices in this lane, 4 lane groups (g4)
      float ss = 0.f;
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        float v[8];
        raw_unpack(craw[k][kn], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      cscale = rsqrtf(ss / (float)N + p.eps);
    }
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
      const int n0 = kn * 32 + 8 * g4;
      float v[8];
      raw_unpack(craw[k][kn], v);
      if constexpr (PRO) {
        if (n0 < N && row_a < rows) {
          const float* bc = s_pb + R * N + (row_a & (R - 1)) * (N + 4) + n0;   // (rows 4 banks apart)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * cscale + bc[e];
        }
      }
      if (n0 < N) rotate_neg(v, s_cs + ta * CSS + n0 / 8, NG);
#pragma unroll
      for (int e = 0; e < 8; ++e) frag_set(cf[k][kn], e, v[e]);
    }
  }
  __syncthreads();
  // Without maps, wave 0 reads the flags of up to 64 predecessors (lane k:
  // chunk c-1-k) now, for the first step of the look-back (with maps this
  // was done at the start, see there).
  if (!p.use_maps && wave == 0 && lane < W0)
    fpoll = flag_state(__hip_atomic_load(flags + c - 1 - lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));

  // Gated readout: the gate operands (w_y, w_z [R][P] fp32, this chunk's z
  // [nt][P]) go to LDS behind S_in^T in the cos/sin region when they fit.  One
  // round of loads is issued here and arrives during C's products; it is
  // written to LDS once the cos/sin table is dead (after the map decision),
  // together with any remaining rounds.  Otherwise the output stage reads them
  // from global memory.
  constexpr uint32_t kSinTB = (uint32_t)round_up_i((int)(sizeof(T) * P * NS), 16);
  constexpr uint32_t kGwB = 2u * R * P * 4u;
  constexpr int kWi = R * P / 4;                          // float4 items per weight table
  constexpr int kZi = P / 8;                              // 8-element items per z row
  const bool gate_lds = G && (uint32_t)(lay.B - lay.csH) >= kSinTB + kGwB + (uint32_t)(Q * P * sizeof(T));
  float* s_gw = reinterpret_cast<float*>(smem + lay.csH + kSinTB);
  T* s_gz = reinterpret_cast<T*>(smem + lay.csH + kSinTB + kGwB);
  const int gnz = (G && p.z) ? nt * kZi : 0;
  const size_t gzstep = tstride * P;
  const Rsrc rWy = buf_rsrc((G && p.wy) ? p.wy + (size_t)h * R * P : nullptr, (G && p.wy) ? R * P * 4 : 0);
  const Rsrc rWz = buf_rsrc((G && p.wz) ? p.wz + (size_t)h * R * P : nullptr, (G && p.wz) ? R * P * 4 : 0);
  const Rsrc rZ = buf_rsrc((G && p.z) ? static_cast<const T*>(p.z) + tok0 * P : nullptr,
                           (G && p.z) ? (uint32_t)(((nt - 1) * gzstep + P) * sizeof(T)) : 0);
  float4 gwa, gwb;
  Raw8<T> gzv[2];
  auto gate_load = [&](int rd) {       // round rd: weight item tid + rd*kThreads, z items 2 per thread
    const int iw = tid + rd * kThreads;
    gwa = buf_load_f32x4(rWy, iw < kWi ? 16u * iw : kOff);
    gwb = buf_load_f32x4(rWz, iw < kWi ? 16u * iw : kOff);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + (2 * rd + u) * kThreads, t = i / kZi, cc = (i - t * kZi) * 8;
      raw_load_buf(gzv[u], rZ, i < gnz ? (uint32_t)((t * gzstep + cc) * sizeof(T)) : kOff);
    }
  };
  auto gate_store = [&](int rd) {
    const int iw = tid + rd * kThreads;
    if (iw < kWi) {
      *reinterpret_cast<float4*>(s_gw + 4 * iw) = gwa;
      *reinterpret_cast<float4*>(s_gw + R * P + 4 * iw) = gwb;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + (2 * rd + u) * kThreads, t = i / kZi, cc = (i - t * kZi) * 8;
      if (i < gnz) *reinterpret_cast<Raw8<T>*>(s_gz + t * P + cc) = gzv[u];
    }
  };
  if constexpr (G) {
    if (gate_lds) gate_load(0);
  }

  // ---- C: U[n][p] = R(Psi) sum_k W_k B~[k][n] X[k][p] ----
  // Lane layout of a (state tile ntl, column tile pt): rows n = 16 ntl + 4 g4 + j
  // (two whole rotation pairs), column p = 16 pt + l16.
  f32x4 uacc[NPW][PTW];
#pragma unroll
  for (int i = 0; i < NPW; ++i)
#pragma unroll
    for (int j = 0; j < PTW; ++j) uacc[i][j] = zero4();
  for (int ks = 0; ks < QRp; ks += 32) {
    const int r0 = ks + 8 * g4;
    const float4 w0 = *reinterpret_cast<const float4*>(s_W + r0);
    const float4 w1 = *reinterpret_cast<const float4*>(s_W + r0 + 4);
    const float Wk[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    Frag<T> xf[PTW];
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int pt = pslot + WPN * j;
      if (pt < TPt) frag_tr(xf[j], s_X, XS, r0, r0 + 4, pt * 16);
    }
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int ntl = nslot + NGRP * i;
      Frag<T> bt;
      frag_tr(bt, s_B, NS, r0, r0 + 4, ntl * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) frag_set(bt, e, Wk[e] * frag_get(bt, e));
#pragma unroll
      for (int j = 0; j < PTW; ++j)
        if (pslot + WPN * j < TPt) uacc[i][j] = mma(bt, xf[j], uacc[i][j]);
    }
  }
  float2 psi[NPW][2];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int k0 = ((nslot + NGRP * i) * 16 + 4 * g4) >> 1;
    psi[i][0] = s_cs[(nt - 1) * CSS + cs_col(k0)];
    psi[i][1] = s_cs[(nt - 1) * CSS + cs_col(k0 + 1)];
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      f32x4& u = uacc[i][j];
      const float u0 = psi[i][0].x * u[0] - psi[i][0].y * u[1], u1 = psi[i][0].y * u[0] + psi[i][0].x * u[1];
      const float u2 = psi[i][1].x * u[2] - psi[i][1].y * u[3], u3 = psi[i][1].y * u[2] + psi[i][1].x * u[3];
      u[0] = u0; u[1] = u1; u[2] = u2; u[3] = u3;
    }
  }
  const float a_c = __expf(l_end);
  // chunk maps and states: stored in register order, each lane's 4 values of a
  // state tile contiguous (a wave writes or reads 1 KB runs), with the cache
  // policy of device-scope atomics
  constexpr uint32_t SLOT = fused_slot_floats(N, P);
  auto slot_off = [&](int i, int jj) { return (uint32_t)(((i * PTW + jj) * kThreads + tid) * 16); };
  const size_t chunk_id = (size_t)bh * p.nc + c;
  // Publish the map only if the predecessor's state was not there at the poll.
  if (wave == 0) {
    int need_map = 0;
    if (p.use_maps) need_map = c > 0 && (__ballot(lane < W0 && fpoll == 2u) & 1ull) == 0;
    if (lane == 0) {
      s_misc[2] = need_map;
      if (need_map) st_dev2(p.recs + chunk_id * (2 * NH + 2), a_c, 0.f);   // the record's decay
    }
  }
  __syncthreads();   // s_misc[2] visible; every read of the cos/sin table is done
  if constexpr (G) {
    if (gate_lds) {
      gate_store(0);
      const int nround = max((kWi + kThreads - 1) / kThreads, (gnz + 2 * kThreads - 1) / (2 * kThreads));
      for (int rd = 1; rd < nround; ++rd) {
        gate_load(rd);
        gate_store(rd);
      }
    }
  }
  if (s_misc[2]) {
    const Rsrc rU = buf_rsrc(p.maps + chunk_id * SLOT, SLOT * 4);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
      float* rec = p.recs + chunk_id * (2 * NH + 2);
      if (pslot == 0 && l16 == 0) {   // R(Psi) of this lane's two pairs
        st_dev2(rec + 2 + n0, psi[i][0].x, psi[i][0].y);
        st_dev2(rec + 2 + n0 + 2, psi[i][1].x, psi[i][1].y);
      }
#pragma unroll
      for (int j = 0; j < PTW; ++j) {
        const int pt = pslot + WPN * j;
        if (pt < TPt) buf_store_dev4(rU, slot_off(i, j), uacc[i][j]);
      }
    }
    mem_done();
    arrive_and_flag(&s_misc[3], flags + c, tag << 2 | 1u, kWaves);
  }

  // ---- D: S_in by look-back; S_out = a R(Psi) S_in + U ----
  float FA = 1.f;
  float2 Fpsi[NPW][2];
  // FU: the composed maps' additive part; once the chain ends it holds S_in
  f32x4 FU[NPW][PTW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    Fpsi[i][0] = Fpsi[i][1] = make_float2(1.f, 0.f);
#pragma unroll
    for (int j = 0; j < PTW; ++j) FU[i][j] = zero4();
  }
  bool chain_ok = true;
  if (c == 0) {
    float kappa0 = 0.f;
    if (p.Bp) kappa0 = (1.f - p.lam[tok0]) * p.dt[tok0];
    const T* Bp = p.Bp ? static_cast<const T*>(p.Bp) + (size_t)bh * R * N : nullptr;
    const T* xp = p.xp ? static_cast<const T*>(p.xp) + (size_t)bh * R * P : nullptr;
    float bps[R];   // PRO: B_prev column norm factors (reduced in phase A, in LDS)
#pragma unroll
    for (int r = 0; r < R; ++r) bps[r] = 1.f;
    if constexpr (PRO) {
      if (Bp) {
#pragma unroll
        for (int r = 0; r < R; ++r) bps[r] = s_bps[r];
      }
    }
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
#pragma unroll
      for (int j = 0; j < PTW; ++j) {
        const int pt = pslot + WPN * j;
        if (pt < TPt) {
          const int hc = hcol(pt);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = p.h0 ? p.h0[((size_t)bh * N + n0 + e) * P + hc] : 0.f;
            if (Bp) {
              float acc = 0.f;
#pragma unroll
              for (int r = 0; r < R; ++r) {
                float bv = to_f(Bp[r * N + n0 + e]);
                if constexpr (PRO) bv = bv * bps[r] + s_pb[r * N + n0 + e];
                acc += bv * to_f(xp[r * P + hc]);
              }
              v += kappa0 * acc;
            }
            FU[i][j][e] = v;
          }
        }
      }
    }
  } else {
    // Wave 0 polls the flags of up to 64 predecessors at once (lane k: chunk
    // hi - k).  The nearest published state ends the walk once every chunk
    // after it has published at least its map; a chunk with neither is waited
    // for.  Maps are then loaded together and composed newest first:
    // F <- F o f_j, i.e. FU += FA R(Fpsi) U_j, Fpsi <- Fpsi + Psi_j, FA <- FA a_j.
    int hi = c - 1;
    bool first = true;   // the early poll covers the first window (hi = c - 1)
    while (true) {
      if (wave == 0) {
        const int W = min(hi + 1, 64);
        unsigned spins = 0;
        int nmap = 0, state = 0;
        while (true) {
          unsigned f = 1u;
          if (first) f = lane < W ? fpoll : 1u;
          else if (lane < W) f = flag_state(__hip_atomic_load(flags + hi - lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          first = false;
          const unsigned long long m2 = __ballot(lane < W && f == 2u);
          const unsigned long long m0 = __ballot(lane < W && f == 0u);
          const int k2 = m2 ? __builtin_ctzll(m2) : W;    // nearest state (W: none in window)
          const int k0 = m0 ? __builtin_ctzll(m0) : 64;   // nearest chunk with nothing yet
          if (k0 > k2 || (k2 == W && k0 >= W)) { nmap = k2; state = k2 < W; break; }
          if (k0 > 0) { nmap = k0; state = 0; break; }   // compose what is there, then wait
          __builtin_amdgcn_s_sleep(1);
          if (++spins > p.spin_limit) { nmap = -1; break; }
        }
        if (lane == 0) { s_misc[1] = nmap; s_misc[5] = state; }
      }
      __syncthreads();
      const int nmap = s_misc[1], state = s_misc[5];
      __syncthreads();
      if (nmap < 0) { chain_ok = false; break; }
      // the state (if any) is loaded alongside the maps
      f32x4 sx[NPW][PTW];
      if (state) {
        const Rsrc rS = buf_rsrc(p.states + ((size_t)bh * p.nc + hi - nmap) * SLOT, SLOT * 4);
#pragma unroll
        for (int i = 0; i < NPW; ++i)
#pragma unroll
          for (int jj = 0; jj < PTW; ++jj)
            if (pslot + WPN * jj < TPt) sx[i][jj] = buf_load_dev4(rS, slot_off(i, jj));
      }
      for (int m0 = 0; m0 < nmap; m0 += kMapGroup) {
        f32x4 ux[kMapGroup][NPW][PTW];
        float2 rx[kMapGroup][NPW][2];
        float ax[kMapGroup];
#pragma unroll
        for (int g = 0; g < kMapGroup; ++g) {
          if (m0 + g < nmap) {
            const size_t jid = (size_t)bh * p.nc + hi - m0 - g;
            const Rsrc rU = buf_rsrc(p.maps + jid * SLOT, SLOT * 4);
            const float* rec = p.recs + jid * (2 * NH + 2);
            ax[g] = ld_dev2(rec).x;
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
              const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
              rx[g][i][0] = ld_dev2(rec + 2 + n0);
              rx[g][i][1] = ld_dev2(rec + 2 + n0 + 2);
#pragma unroll
              for (int jj = 0; jj < PTW; ++jj)
                if (pslot + WPN * jj < TPt) ux[g][i][jj] = buf_load_dev4(rU, slot_off(i, jj));
            }
          }
        }
#pragma unroll
        for (int g = 0; g < kMapGroup; ++g) {
          if (m0 + g < nmap) {
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
#pragma unroll
              for (int jj = 0; jj < PTW; ++jj) {
                const float2 x01 = make_float2(ux[g][i][jj][0], ux[g][i][jj][1]);
                const float2 x23 = make_float2(ux[g][i][jj][2], ux[g][i][jj][3]);
                FU[i][jj][0] += FA * (Fpsi[i][0].x * x01.x - Fpsi[i][0].y * x01.y);
                FU[i][jj][1] += FA * (Fpsi[i][0].y * x01.x + Fpsi[i][0].x * x01.y);
                FU[i][jj][2] += FA * (Fpsi[i][1].x * x23.x - Fpsi[i][1].y * x23.y);
                FU[i][jj][3] += FA * (Fpsi[i][1].y * x23.x + Fpsi[i][1].x * x23.y);
              }
              const float2 a0 = Fpsi[i][0], a1 = Fpsi[i][1], r0 = rx[g][i][0], r1 = rx[g][i][1];
              Fpsi[i][0] = make_float2(a0.x * r0.x - a0.y * r0.y, a0.y * r0.x + a0.x * r0.y);
              Fpsi[i][1] = make_float2(a1.x * r1.x - a1.y * r1.y, a1.y * r1.x + a1.x * r1.y);
            }
            FA *= ax[g];
          }
        }
      }
      if (state) {
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
#pragma unroll
          for (int jj = 0; jj < PTW; ++jj) {
            const float2 x01 = make_float2(sx[i][jj][0], sx[i][jj][1]);
            const float2 x23 = make_float2(sx[i][jj][2], sx[i][jj][3]);
            FU[i][jj][0] += FA * (Fpsi[i][0].x * x01.x - Fpsi[i][0].y * x01.y);
            FU[i][jj][1] += FA * (Fpsi[i][0].y * x01.x + Fpsi[i][0].x * x01.y);
            FU[i][jj][2] += FA * (Fpsi[i][1].x * x23.x - Fpsi[i][1].y * x23.y);
            FU[i][jj][3] += FA * (Fpsi[i][1].y * x23.x + Fpsi[i][1].x * x23.y);
          }
        }
        break;
      }
      hi -= nmap;
    }
  }
  const float nanv = __builtin_nanf("");
  if (!chain_ok && tid == 0)   // the wait gave up: recorded for m3_prefill_status
    __hip_atomic_fetch_or(p.err, (unsigned long long)kErrLookback, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool publish = c + 1 < p.nc;
  const Rsrc rSo = buf_rsrc(p.states + chunk_id * SLOT, publish ? SLOT * 4 : 0);
  // S_in^T goes into the (now free) cos/sin region for the readout
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int pt = pslot + WPN * j;
      if (pt < TPt) {
        const int pc = pt * 16 + l16;
        f32x4 si = FU[i][j];
        if (!chain_ok) si[0] = si[1] = si[2] = si[3] = nanv;
        const float sv4[4] = {si[0], si[1], si[2], si[3]};
        store_row<T, 4>(s_H + pc * NS + n0, sv4);
        const float q0 = a_c * si[0], q1 = a_c * si[1], q2 = a_c * si[2], q3 = a_c * si[3];
        const f32x4 u = uacc[i][j];
        const float o0 = psi[i][0].x * q0 - psi[i][0].y * q1 + u[0];
        const float o1 = psi[i][0].y * q0 + psi[i][0].x * q1 + u[1];
        const float o2 = psi[i][1].x * q2 - psi[i][1].y * q3 + u[2];
        const float o3 = psi[i][1].y * q2 + psi[i][1].x * q3 + u[3];
        if (publish) {
          buf_store_dev4(rSo, slot_off(i, j), f32x4{o0, o1, o2, o3});
        } else if (p.h_out) {
          float* ho = p.h_out + ((size_t)bh * N + n0) * P + hcol(pt);
          ho[0] = o0; ho[P] = o1; ho[2 * P] = o2; ho[3 * P] = o3;
        }
      }
    }
  }
  __syncthreads();   // S_in^T complete in LDS

  // ---- E: outputs of this wave's 16-row tiles (up to RTW), all together ----
  int itk[RTW], sbm[RTW];
  bool vk[RTW];
#pragma unroll
  for (int k = 0; k < RTW; ++k) {
    itk[k] = k < ntiles_w ? tile_of(k) : 0;
    vk[k] = k < ntiles_w && itk[k] * 16 < rows;
    sbm[k] = vk[k] ? min(itk[k] * 16 + 15, rows - 1) / 32 : -1;
  }
  int sbmax = -1;
#pragma unroll
  for (int k = 0; k < RTW; ++k) sbmax = max(sbmax, sbm[k]);
  // inter-chunk term C~_t^T S_in, scaled by exp(l_t)
  f32x4 yacc[RTW][TPt];
#pragma unroll
  for (int k = 0; k < RTW; ++k)
#pragma unroll
    for (int pn = 0; pn < TPt; ++pn) yacc[k][pn] = zero4();
#pragma unroll
  for (int pn = 0; pn < TPt; ++pn) {
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
      const int n0 = kn * 32 + 8 * g4;
      Frag<T> hf;
      if (n0 < N) frag_lds8(hf, s_H + (pn * 16 + l16) * NS + n0);
      else frag_zero(hf);
#pragma unroll
      for (int k = 0; k < RTW; ++k)
        if (vk[k]) yacc[k][pn] = mma(cf[k][kn], hf, yacc[k][pn]);
    }
  }
  float l_t[RTW];
#pragma unroll
  for (int k = 0; k < RTW; ++k) {
    if (!vk[k]) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = itk[k] * 16 + 4 * g4 + j;
      const float e = row < rows ? __expf(s_row[row].x) : 0.f;
#pragma unroll
      for (int pn = 0; pn < TPt; ++pn) yacc[k][pn][j] *= e;
    }
    const int row_a = itk[k] * 16 + l16;
    l_t[k] = row_a < rows ? s_row[row_a].x : 0.f;
  }
  // the state stores were issued before the inter term: wait for them and
  // raise the flag before the intra-chunk work
  if (publish) {
    mem_done();
    arrive_and_flag(&s_misc[4], flags + c, tag << 2 | 2u, kWaves);
  }
  for (int sb = 0; sb <= sbmax; ++sb) {
    // S^T block = B~[32 rows of block sb] C~[tile]^T, for every tile of the wave
    f32x4 st[RTW][2];
#pragma unroll
    for (int k = 0; k < RTW; ++k) st[k][0] = st[k][1] = zero4();
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
#pragma unroll
      for (int k = 0; k < RTW; ++k) {
        if (sb <= sbm[k]) {
          st[k][0] = mma(a0, cf[k][kn], st[k][0]);
          st[k][1] = mma(a1, cf[k][kn], st[k][1]);
        }
      }
    }
    // decay x two-band mask on each score tile
    Frag<T> pf[RTW];
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
      if (sb > sbm[k]) continue;
      const int row_a = itk[k] * 16 + l16;
      const bool va = row_a < rows;
      if (sb * 32 + 32 <= itk[k] * 16) {
        // source block wholly before this tile: every s < t, one exp per lane
        const int be = min(sb * 32 + 31, rows - 1);
        const float et = va ? __expf(l_t[k] - s_row[be].x) : 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float4 rw = *reinterpret_cast<const float4*>(s_rw + sb * 32 + hh * 16 + 4 * g4);
          const float r4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) frag_set(pf[k], hh * 4 + j, et * r4[j] * st[k][hh][j]);
        }
      } else {
        // the block holding this tile: elementwise; a lane's 4 rows in each
        // 16-row half are min(R, 4)-row groups of one token
        constexpr int RG = R < 4 ? R : 4;
        const int ta = row_a >> LOGR;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int rb = sb * 32 + hh * 16 + 4 * g4;
#pragma unroll
          for (int q = 0; q < 4; q += RG) {
            const int srow = rb + q;
            const int s = srow >> LOGR;
            float m = 0.f;
            if (va && srow < rows && s <= ta) {
              const float4 rw = s_row[srow];
              m = __expf(l_t[k] - rw.x) * (s < ta ? rw.y : rw.z);
            }
#pragma unroll
            for (int j = q; j < q + RG; ++j) frag_set(pf[k], hh * 4 + j, m * st[k][hh][j]);
          }
        }
      }
    }
    // (mask o S) X, each X fragment shared by the tiles
#pragma unroll
    for (int pn = 0; pn < TPt; ++pn) {
      Frag<T> xf;
      frag_tr(xf, s_X, XS, sb * 32 + 4 * g4, sb * 32 + 16 + 4 * g4, pn * 16);
#pragma unroll
      for (int k = 0; k < RTW; ++k)
        if (sb <= sbm[k]) yacc[k][pn] = mma(pf[k], xf, yacc[k][pn]);
    }
  }
  // y: a lane holds head columns TPt*l16 .. TPt*l16+TPt-1 of 4 rows per tile
  if constexpr (!G) {
    T* Yg = static_cast<T*>(p.y) + tok0 * R * P;
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
      if (!vk[k]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = itk[k] * 16 + 4 * g4 + j;
        if (row < rows) {
          float v[TPt];
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) v[pn] = chain_ok ? yacc[k][pn][j] : nanv;
          store_row<T, TPt>(Yg + (row >> LOGR) * rowstepX + (row & (R - 1)) * P + TPt * l16, v);
        }
      }
    }
  } else {
    // gated readout out[t][c] = sum_r w_y[r][c] y[(t, r)][c] silu(w_z[r][c] z[t][c]):
    // a lane's 4 rows are whole tokens' ranks for R <= 4 (RG rows per token);
    // at R = 8 they are half a token's, and the lane 16 apart holds the rest
    const size_t rowstepO = tstride * P;
    T* Og = static_cast<T*>(p.out) + tok0 * P;
    const T* Zg = p.z ? static_cast<const T*>(p.z) + tok0 * P : nullptr;
    const float* wyh = p.wy ? p.wy + (size_t)h * R * P + TPt * l16 : nullptr;
    const float* wzh = p.wz ? p.wz + (size_t)h * R * P + TPt * l16 : nullptr;
    const float* swy = s_gw + TPt * l16;
    const float* swz = s_gw + R * P + TPt * l16;
    constexpr int RG = R < 4 ? R : 4;
#pragma unroll
    for (int k = 0; k < RTW; ++k) {
      if (!vk[k]) continue;
#pragma unroll
      for (int q = 0; q < 4; q += RG) {
        const int row0 = itk[k] * 16 + 4 * g4 + q;
        const bool valid = row0 < rows;
        const int tk = row0 >> LOGR;
        float zv[TPt], o[TPt];
#pragma unroll
        for (int pn = 0; pn < TPt; ++pn) {
          zv[pn] = !(Zg && valid) ? 0.f
                   : gate_lds ? to_f(s_gz[tk * P + TPt * l16 + pn]) : to_f(Zg[tk * rowstepO + TPt * l16 + pn]);
          o[pn] = 0.f;
        }
#pragma unroll
        for (int j = q; j < q + RG; ++j) {
          const int r = (row0 + j - q) & (R - 1);
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) {
            float v = yacc[k][pn][j];
            if (wyh) v *= gate_lds ? swy[r * P + pn] : wyh[r * P + pn];
            if (Zg) {
              const float gz = (wzh ? (gate_lds ? swz[r * P + pn] : wzh[r * P + pn]) : 1.f) * zv[pn];
              v *= gz * __builtin_amdgcn_rcpf(1.f + __expf(-gz));   // silu (1-ulp reciprocal)
            }
            o[pn] += v;
          }
        }
        if constexpr (R == 8) {
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) o[pn] += __shfl_xor(o[pn], 16);
        }
        if (valid && (R != 8 || (g4 & 1) == 0)) {
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) o[pn] = chain_ok ? o[pn] : nanv;
          store_row<T, TPt>(Og + tk * rowstepO + TPt * l16, o);
        }
      }
    }
  }
}

template <typename T, int N, int P, int R, int RT, bool G, bool PRO>
hipError_t launch(const FusedParams& p, size_t lds, hipStream_t stream) {
  // A variant that uses scratch is never launched (the host plan already
  // refuses the ones the build report lists; this checks the loaded code).
  static std::atomic<int> scratch_state{0};   // 0 unknown, 1 none, 2 uses scratch
  int st = scratch_state.load(std::memory_order_relaxed);
  if (st == 0) {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(prefill_kernel<T, N, P, R, RT, G, PRO>)) != hipSuccess)
      return hipErrorInvalidDeviceFunction;
    st = fa.localSizeBytes > 0 ? 2 : 1;
    scratch_state.store(st, std::memory_order_relaxed);
  }
  if (st == 2) return hipErrorNotSupported;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  // The LDS limit is raised once per instantiation and device (one bit per
  // device; callers racing on the first launch just set it twice).
  static std::atomic<unsigned long long> lds_set{0};
  if (lds > 64 * 1024 && (dev < 0 || !(lds_set.load(std::memory_order_acquire) >> dev & 1ull))) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_kernel<T, N, P, R, RT, G, PRO>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (e != hipSuccess) return e;
    if (dev >= 0) lds_set.fetch_or(1ull << dev, std::memory_order_acq_rel);
  }
  const size_t grid = (size_t)p.batch * p.H * p.nc;
  // Maps let a chunk finish before its predecessor's state exists; they pay off
  // only when many chunks of one sequence are in flight at once (few sequences
  // x heads for the workgroups resident on the device): then consecutive
  // chunks start closer together than a state takes to pass from one to the
  // next.  With at most 4 in flight the state chain keeps up, and the maps'
  // stores and waits would only cost time.
  // (resident workgroups per device, cached with the LDS size they were
  // computed for: one 64-bit word per device, so concurrent callers never see
  // half an update)
  static std::atomic<unsigned long long> cache[64];
  int resident = 0;
  const unsigned long long hit = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0ull;
  if (hit != 0 && (hit >> 32) == (unsigned long long)lds) {
    resident = (int)(hit & 0xffffffffull);
  } else {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(prefill_kernel<T, N, P, R, RT, G, PRO>), fused_threads(N), lds) == hipSuccess)
      resident = cus * per;
    if (dev >= 0 && resident > 0)
      cache[dev].store(((unsigned long long)lds << 32) | (unsigned)resident, std::memory_order_relaxed);
  }
  FusedParams q = p;
  const size_t nbh = (size_t)p.batch * p.H;
  q.use_maps = !(resident > 0 && (size_t)resident <= 4 * nbh);
  hipLaunchKernelGGL((prefill_kernel<T, N, P, R, RT, G, PRO>), dim3((unsigned)grid), dim3(fused_threads(N)), lds, stream, q);
  return hipGetLastError();
}


template <typename T, int N, int P, int R>
hipError_t launch_rt(const FusedParams& p, size_t lds, hipStream_t s) {
  const int rt = fused_row_tiles(p.Q, R, N);
  constexpr int kWaves = fused_threads(N) / 64;
  constexpr int kMaxRT = (fused_rows_cap(N) / 16 + kWaves - 1) / kWaves;
  // variants: plain, gated readout, prologue (not both)
  if (p.out && p.pro) return hipErrorInvalidValue;
  if (p.out) {
    if (rt <= 1) return launch<T, N, P, R, 1, true, false>(p, lds, s);
    if (rt <= 2 && kMaxRT >= 2) return launch<T, N, P, R, (kMaxRT >= 2 ? 2 : 1), true, false>(p, lds, s);
    if (rt <= 4 && kMaxRT >= 4) return launch<T, N, P, R, (kMaxRT >= 4 ? 4 : 1), true, false>(p, lds, s);
    return hipErrorInvalidValue;
  }
  if (p.pro) {   // (one output tile per wave only: the host rejects larger chunks)
    if (rt <= 1) return launch<T, N, P, R, 1, false, true>(p, lds, s);
    return hipErrorInvalidValue;
  }
  if (rt <= 1) return launch<T, N, P, R, 1, false, false>(p, lds, s);
  if (rt <= 2 && kMaxRT >= 2) return launch<T, N, P, R, (kMaxRT >= 2 ? 2 : 1), false, false>(p, lds, s);
  if (rt <= 4 && kMaxRT >= 4) return launch<T, N, P, R, (kMaxRT >= 4 ? 4 : 1), false, false>(p, lds, s);
  return hipErrorInvalidValue;
}

template <typename T, int N>
hipError_t launch_n(const FusedParams& p, size_t lds, hipStream_t s) {
#define M3_R_CASES(PP)                                          \
  switch (p.R) {                                                \
    case 1: return launch_rt<T, N, PP, 1>(p, lds, s);           \
    case 2: return launch_rt<T, N, PP, 2>(p, lds, s);           \
    case 4: return launch_rt<T, N, PP, 4>(p, lds, s);           \
    case 8: return launch_rt<T, N, PP, 8>(p, lds, s);           \
    default: return hipErrorInvalidValue;                       \
  }
  switch (p.P) {
    case 16: M3_R_CASES(16)
    case 32: M3_R_CASES(32)
    case 64: M3_R_CASES(64)
    case 128: M3_R_CASES(128)
    default: return hipErrorInvalidValue;
  }
#undef M3_R_CASES
}

}  // namespace fused
}  // namespace m3

// One translation unit per (dtype, N) instantiates the kernels for all P and R.
#define M3_FUSED_INSTANTIATE(TYPE, TNAME, NN)                                                   \
  namespace m3 {                                                                                \
  hipError_t launch_fused_##TNAME##_##NN(const FusedParams& p, size_t lds, hipStream_t s) {    \
    return fused::launch_n<TYPE, NN>(p, lds, s);                                                \
  }                                                                                             \
  }
