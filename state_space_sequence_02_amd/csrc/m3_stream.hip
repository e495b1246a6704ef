// m3_stream.hip -- persistent, streaming single-pass prefill for gfx950 on the
// hot shapes: bf16 inputs, P = 64, N = 64 or 128, R = 1, 2 or 4, chunks of
// 128 or 256 (token, rank) rows.
//
// It computes what prefill_kernel (m3_fused_kernel.h) computes -- the exact
// chunked rearrangement of the recurrence (Mamba-3 explainer panels 1, 3, 4,
// its sec. 3.3 chunked-algorithm remark; the paper page's Figure 1 decay x
// two-band mask; data-dependent RoPE, explainer Prop. 3/4 and Eq. 11), with
// the same decoupled look-back between chunks and the same workspace -- but
// organised so that the loads of one chunk overlap the arithmetic of another:
//
//  * persistent: one 1024-thread workgroup per compute unit takes chunk
//    tickets (chunk-major over all sequences, as the per-chunk kernel does)
//    until they run out.  The next chunk's ticket is taken at the start of the
//    current one, and its first source blocks are loaded during the current
//    chunk's last blocks, so they are in flight while its look-back and
//    output stage run.
//  * streaming: B and X pass through a two-slot LDS ring in 32-row source
//    blocks, the next PRE blocks' loads in flight in registers (one 16-byte
//    item per thread per block).  Each block, once staged (B rotated by
//    -Phi_s, X with permuted columns), feeds the chunk map U (every wave owns
//    one 16-row state tile and PTW column tiles of it) and the masked
//    intra-chunk products of every wave's 16-row output tile.  No wave waits
//    for a whole chunk's B and X, and a chunk needs ~67 KB of LDS instead of
//    ~154 KB.
//  * the tail of a chunk: U turned by Psi, the map published when the
//    predecessor's state was not there at the poll (maps in use), the
//    look-back for S_in, S_out = a R(Psi) S_in + U stored and flagged, then
//    the inter-chunk term exp(l_t) C~_t^T S_in added to the accumulated intra
//    term, and y stored.
//
// With PRO (m3_scan_prefill_prologue) the prologue is applied where the
// operands are staged: each B row is RMS-normalised over its N values (the
// row's N/8 items sit in consecutive lanes: DPP row rotations at N = 128, xor
// shuffles at N = 64) and gets the head's B bias, each C row likewise when its
// MFMA fragments are formed (4 lane groups), a sequence's first chunk scales
// B_prev by column norms wave 0 takes into LDS, and the angle threads multiply
// the raw angles by their tokens' dt before the phase scan.  The head's bias
// tables ([R][N] each) are loaded one chunk ahead with the scalars.
//
// Termination and the control words: a workgroup whose ticket is past the
// call's last one stops; it then counts itself in the exit counter (the
// workspace's third 8-byte word), and the last of the grid to stop resets the
// ticket count to 0 with the next epoch and the exit counter to 0, so the
// zero-filled workspace stays ready for the next call (flags carry the epoch,
// as with the per-chunk kernel).  A ticket past the last one by more than the
// grid size cannot happen in a zero-filled workspace: it sets the error word's
// control bit.
//
// Every look-back waits only on chunks with lower tickets; the lowest ticket
// not yet finished is always some workgroup's current chunk (a workgroup's
// next ticket is larger than its current one), and its own predecessors are
// finished, so every wait ends.
#include "m3_fused_kernel.h"

namespace m3 {
namespace stream {
using namespace fused;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
#ifndef M3_STREAM_MAP_GROUP
#define M3_STREAM_MAP_GROUP 3
#endif
constexpr int kMapGroup = M3_STREAM_MAP_GROUP;   // maps loaded at once in the look-back

// LDS: per-row data, cos/sin of Phi (then U while the look-back runs), the
// two-slot ring (then S_in^T for the readout), every lane's C~ fragments
// (its wave's output rows; read back only by that lane), scalars.
struct SLds {
  size_t row, rw, W, cs, ring, blk, cfr, misc, pb, total;
  size_t segl, sega;   // scan scratch, inside the ring (before a chunk's first block is staged)
};
// pro: the fused prologue's tables behind the rest: the head's B and C biases
// [R][N] each, then B_prev's column norm factors [R] (a sequence's first chunk)
__host__ __device__ constexpr SLds lds_of(int Q, int R, int N, int P, bool pro = false, bool gate = false) {
  SLds o{};
  const int QR = Q * R;
  o.row = 0;
  o.rw = o.row + sizeof(float4) * QR;
  o.W = o.rw + sizeof(float) * QR;
  o.cs = o.W + sizeof(float) * QR;
  o.ring = o.cs + round_up_i((int)max_sz(sizeof(float2) * (size_t)Q * (N / 2 + 1), sizeof(float) * (size_t)N * P), 16);
  o.blk = round_up_i(2 * 32 * (N + 8) + 2 * 32 * x_stride(P, 2), 16);   // B~ [32][N+8], X [32][XS] (bf16)
  o.cfr = o.ring + 2 * o.blk;     // [N/32][kThreads] 16-byte fragments
  o.misc = o.cfr + 16 * (size_t)kThreads * (N / 32);
  o.pb = o.misc + 64;
  // (gate: the head's w_y and w_z [R][P] each in the same place)
  o.total = o.pb + (pro ? sizeof(float) * (size_t)R * (2 * N + 4) : gate ? sizeof(float) * (size_t)R * 2 * P : 0);
  o.segl = o.ring;
  o.sega = o.ring + sizeof(float) * kWaves;
  return o;
}

// The kernel's argument as a pointer into the kernarg segment that passes
// through an empty asm: fields read through it are loaded afresh (scalar loads)
// where they are used, so the compiler cannot keep them live from one chunk's
// iteration into the next (hoisted out of the persistent loop, the ~30
// pointers and sizes overflow the scalar registers and spill).
typedef const __attribute__((opencl_constant)) FusedParams* KParams;
__device__ __forceinline__ KParams reload_params() {
  KParams kp = (KParams)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return kp;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 inside each 16-lane row (lanes before the shift read 0), then
// lane 15 of each row added into rows 1 and 3, then lane 31 into rows 2 and 3.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_mv(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, BOUND));
}
__device__ __forceinline__ float wave_scan_add(float v) {
  v += dpp_mv<0x111, 0xF, true>(v);    // row_shr:1
  v += dpp_mv<0x112, 0xF, true>(v);    // row_shr:2
  v += dpp_mv<0x114, 0xF, true>(v);    // row_shr:4
  v += dpp_mv<0x118, 0xF, true>(v);    // row_shr:8
  v += dpp_mv<0x142, 0xA, false>(v);   // row_bcast:15, into rows 1 and 3
  v += dpp_mv<0x143, 0xC, false>(v);   // row_bcast:31, into rows 2 and 3
  return v;
}

// NBK: 32-row source blocks per chunk (Q * R = 32 NBK); PRE: blocks in flight;
// MAPS: chunk maps in use (many chunks of one sequence in flight at once: a
// chunk whose predecessor's state is late publishes its map, and the look-back
// composes maps); without, a chunk waits for its predecessor's state.
// PRO: the fused prologue (BCNorm of B, C and B_prev with the head's B/C
// biases, the step angle dt x theta) applied where B and C are staged and the
// angles scanned.
// GATE: the gated rank-contracted readout fused into the output stage
// (m3_scan_prefill_gated): out[t][c] = sum_r w_y[r][c] y[(t, r)][c]
// silu(w_z[r][c] z[t][c]) replaces y.
template <int N, int P, int R, int NBK, int PRE, bool MAPS, bool PRO, bool GATE>
__global__ __launch_bounds__(kThreads, 4) void stream_kernel(FusedParams p_in) {
  typedef bf16 T;
  constexpr int NH = N / 2;
  constexpr int NG = NH / 4;                  // 4-pair column groups of the angle table
  constexpr int CSS = NH + 1;                 // angle table row stride (float2)
  constexpr int NK = N / 32;                  // 32-wide slices of the state dimension
  constexpr int TPt = P / 16;                 // 16-column tiles of the head dimension
  constexpr int TNt = N / 16;                 // 16-row tiles of the state dimension
  constexpr int NGRP = TNt < kWaves ? TNt : kWaves;
  constexpr int NPW = TNt / NGRP;
  constexpr int WPN = kWaves / NGRP;
  constexpr int PTW = (TPt + WPN - 1) / WPN;
  constexpr int NS = N + 8;                   // LDS row stride of B~ and S_in^T
  constexpr int XS = x_stride(P, 2);          // LDS row stride of X
  constexpr int LOGR = R == 1 ? 0 : R == 2 ? 1 : 2;
  constexpr int QR = NBK * 32;                // (token, rank) rows per chunk
  constexpr int Q = QR / R;                   // tokens per chunk
  constexpr int MT = QR / 16;                 // 16-row output tiles per chunk
  constexpr int kBI = 32 * (N / 8), kXI = 32 * (P / 8);   // 16-byte items of a block: B, X
  constexpr int NSEG = (kThreads / NG) < Q ? (kThreads / NG) : Q;   // angle segments
  constexpr int ALEN = Q / NSEG;              // tokens per angle thread
  constexpr int kXStep = NBK - 1 - PRE;       // first loop step that loads the next chunk's blocks
  static_assert(R == 1 || R == 2 || R == 4, "rank");
  static_assert(!(PRO && GATE), "one fused stage per variant");
  static_assert(!GATE || P == 64, "the gated output stage reads 4 columns of z per lane");
  static_assert(MT <= kWaves && kBI + kXI <= kThreads && kBI % 64 == 0 && kXI % 64 == 0, "geometry");
  static_assert(NBK % PRE == 0 && kXStep >= 1, "a chunk's block 0 lands in prefetch slot 0");
  static_assert(ALEN >= 1 && ALEN <= 4 && NSEG * ALEN == Q, "angle threads");
  static_assert(kThreads % (N / 8) == 0 && NK >= 1 && TPt >= 1, "tiles");
  constexpr SLds lay = lds_of(Q, R, N, P, PRO, GATE);
  constexpr uint32_t kOff = 0x80000000u;      // an offset past every extent
  constexpr uint32_t SLOT = fused_slot_floats(N, P);
  static_assert(SLOT == (uint32_t)NPW * PTW * kThreads * 4, "slot layout");

  extern __shared__ __align__(16) unsigned char smem[];
  float4* s_row = reinterpret_cast<float4*>(smem + lay.row);
  float* s_rw = reinterpret_cast<float*>(smem + lay.rw);
  float* s_W = reinterpret_cast<float*>(smem + lay.W);
  float* s_segl = reinterpret_cast<float*>(smem + lay.segl);
  float4* s_sega = reinterpret_cast<float4*>(smem + lay.sega);
  float2* s_cs = reinterpret_cast<float2*>(smem + lay.cs);
  float* s_U = reinterpret_cast<float*>(smem + lay.cs);   // U, in slot order (after the angles)
  T* s_H = reinterpret_cast<T*>(smem + lay.ring);          // S_in^T [P][N + 8] (after the blocks)
  bf16x8* s_cf = reinterpret_cast<bf16x8*>(smem + lay.cfr);   // C~ fragments [NK][kThreads]
  int* s_misc = reinterpret_cast<int*>(smem + lay.misc);
  float* s_pb = reinterpret_cast<float*>(smem + lay.pb);   // PRO: bias tables, B_prev norms
  auto ringB = [&](int slot) { return reinterpret_cast<T*>(smem + lay.ring + slot * lay.blk); };
  auto ringX = [&](int slot) { return reinterpret_cast<T*>(smem + lay.ring + slot * lay.blk) + 32 * NS; };

  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // ---- first ticket ----
  const unsigned total0 = (unsigned)(p_in.batch * p_in.H * p_in.nc);
  if (threadIdx.x == 0) {
    const unsigned long long w = atomicAdd(p_in.ctl, 1ull);
    const unsigned cnt = (unsigned)(w & kTicketMask);
    const unsigned long long epoch = w >> kTicketBits;
    if (cnt >= total0 + gridDim.x)   // only in a workspace that was not zero-filled
      __hip_atomic_fetch_or(p_in.err, (unsigned long long)kErrControl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_misc[0] = (int)cnt;
    s_misc[6] = (int)(unsigned)(epoch + 1);
    s_misc[7] = (int)(unsigned)((epoch + 1) >> 32);
  }
  __syncthreads();
  unsigned ticket = (unsigned)__builtin_amdgcn_readfirstlane(s_misc[0]);


  Raw8<T> pre[PRE];
  float dv, lmv, dnv, lmnv_raw, av;
  float4 th4[ALEN];
  float dth[ALEN];   // PRO: dt of the angle thread's tokens
  float4 pbv;        // PRO: 4 of the head's bias values (B's [R][N] then C's);
                     // GATE: 4 of the head's gate weights (w_y's [R][P] then w_z's)
  Raw8<T> craw[NK];
  struct Ck { int c, bh, h, nt; size_t tok0; };
  Ck ck{0, 0, 0, 0, 0};
  bool first = true;
  while (true) {
    const KParams p = reload_params();
    // this call's flag tag (epoch + 1), read where it is needed: held across
    // the persistent loop it would take registers for its whole length
    const unsigned long long tag = ((unsigned long long)(unsigned)__builtin_amdgcn_readfirstlane(s_misc[7]) << 32) |
                                   (unsigned)__builtin_amdgcn_readfirstlane(s_misc[6]);
    auto flag_state = [&](unsigned long long f) { return (f >> 2) == tag ? (unsigned)(f & 3u) : 0u; };
    // thread indices, recomputed per chunk (an opaque copy of the thread
    // index): the addresses derived from them are cheap to form again, and
    // kept live across the persistent loop they would spill
    int tid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(tid));   // the lane
    tid |= wave0 << 6;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int nslot = wave % NGRP, pslot = wave / NGRP;
    auto hcol = [&](int pt) { return l16 * TPt + pt; };
    auto cs_col = [](int k) { return (k & 3) * NG + (k >> 2); };
    // this wave's output tile (at most one); with a full set of 16 the second
    // half of the waves takes them in reverse order, so each SIMD (waves w,
    // w + 4, w + 8, w + 12) holds light and heavy tiles alike
    const bool has_tile = wave < MT;
    const int tile = (MT == kWaves && wave >= kWaves / 2) ? MT - 1 - (wave - kWaves / 2) : wave;
    const int cg = tid % NG, sg = tid / NG;     // angle thread: column group, token segment
    // block items: waves below kBI / 64 load B rows, the next kXI / 64 waves X rows
    const bool ldB = wave < kBI / 64;
    const bool ldX = !ldB && wave < (kBI + kXI) / 64;
    const int nbh = p->batch * p->H;
    const unsigned total = (unsigned)(nbh * p->nc);
    const size_t tstride = (size_t)p->H;         // token step in [b, L, H] arrays
    const uint32_t tsb = (uint32_t)tstride * 4;
    const uint32_t rsB = (uint32_t)(tstride * R * N * 2), rsX = (uint32_t)(tstride * R * P * 2);
  // A chunk's indices; a ticket past the last one gives an empty chunk (nt = 0:
  // every load of it reads zeros).
  auto chunk_of = [&](unsigned tk) {
    Ck k{0, 0, 0, 0, 0};
    if (tk < total) {
      k.c = (int)tk / nbh;
      k.bh = (int)tk - k.c * nbh;
      const int b = k.bh / p->H;
      k.h = k.bh - b * p->H;
      const int t0 = k.c * Q;
      k.nt = min(Q, p->L - t0);
      k.tok0 = ((size_t)b * p->L + t0) * p->H + k.h;
    }
    return k;
  };
  // this thread's 16-byte item of source block j of the chunk at token index
  // tok0 with nt tokens
  auto blk_load = [&](Raw8<T>& r, size_t ktok0, int knt, int j) {
    const Rsrc rB = buf_rsrc(static_cast<const T*>(p->B) + ktok0 * R * N, knt > 0 ? (uint32_t)(knt - 1) * rsB + R * N * 2 : 0);
    const Rsrc rX = buf_rsrc(static_cast<const T*>(p->x) + ktok0 * R * P, knt > 0 ? (uint32_t)(knt - 1) * rsX + R * P * 2 : 0);
    uint32_t off = kOff;
    if (ldB) {
      const int row = 32 * j + tid / (N / 8), g = tid % (N / 8);
      off = (uint32_t)(row >> LOGR) * rsB + (uint32_t)(((row & (R - 1)) * N + g * 8) * 2);
    } else if (ldX) {
      const int i = tid - kBI;
      const int row = 32 * j + i / (P / 8), g = i % (P / 8);
      off = (uint32_t)(row >> LOGR) * rsX + (uint32_t)(((row & (R - 1)) * P + g * 8) * 2);
    }
    raw_load_buf(r, ldB ? rB : rX, off);
  };
  // the chunk's per-token scalars, its head's A, and its angles
  auto small_load = [&](const Ck& k) {
    const int nt = k.nt;
    const Rsrc rD = buf_rsrc(p->dt + k.tok0, nt > 0 ? (nt - 1) * tsb + 4 : 0);
    const Rsrc rL = buf_rsrc(p->lam + k.tok0, nt > 0 ? (nt - 1) * tsb + 4 : 0);
    const int t0 = k.c * Q;
    const int nnext = nt > 0 ? min(nt, p->L - t0 - 1) : 0;   // tokens whose successor exists
    const Rsrc rDn = buf_rsrc(p->dt + k.tok0 + tstride, nnext > 0 ? (nnext - 1) * tsb + 4 : 0);
    const Rsrc rLn = buf_rsrc(p->lam + k.tok0 + tstride, nnext > 0 ? (nnext - 1) * tsb + 4 : 0);
    const uint32_t toff = tid < Q ? tid * tsb : kOff;
    dv = buf_load_f32(rD, toff);
    lmv = buf_load_f32(rL, toff);
    dnv = buf_load_f32(rDn, toff);
    lmnv_raw = buf_load_f32(rLn, toff);
    av = buf_load_f32(buf_rsrc(p->A, (uint32_t)p->H * 4), nt > 0 ? (uint32_t)k.h * 4 : kOff);   // A of the head
    const Rsrc rT = buf_rsrc(p->theta ? p->theta + k.tok0 * NH : nullptr, (p->theta && nt > 0) ? (nt - 1) * tsb * NH + NH * 4 : 0);
#pragma unroll
    for (int j = 0; j < ALEN; ++j)
      th4[j] = buf_load_f32x4(rT, sg < NSEG ? (uint32_t)(sg * ALEN + j) * tsb * NH + 16 * cg : kOff);
    if constexpr (PRO) {
      // theta holds raw angles: each angle thread also takes its tokens' dt
#pragma unroll
      for (int j = 0; j < ALEN; ++j) dth[j] = buf_load_f32(rD, sg < NSEG ? (uint32_t)(sg * ALEN + j) * tsb : kOff);
      // the head's biases, one float4 per thread: B's [R][N] (threads below
      // R N / 4), then C's (the next R N / 4); a missing table reads as zeros
      constexpr int kPb4 = R * N / 4;
      const Rsrc rBb = buf_rsrc(p->biasB ? p->biasB + (size_t)k.h * R * N : nullptr, (p->biasB && nt > 0) ? R * N * 4 : 0);
      const Rsrc rCb = buf_rsrc(p->biasC ? p->biasC + (size_t)k.h * R * N : nullptr, (p->biasC && nt > 0) ? R * N * 4 : 0);
      pbv = add4(buf_load_f32x4(rBb, tid < kPb4 ? (uint32_t)tid * 16 : kOff),
                 buf_load_f32x4(rCb, tid >= kPb4 && tid < 2 * kPb4 ? (uint32_t)(tid - kPb4) * 16 : kOff));
    }
    if constexpr (GATE) {   // the head's w_y then w_z [R][P], one float4 per thread
      constexpr int kGw4 = R * P / 4;
      const Rsrc rWy = buf_rsrc(p->wy ? p->wy + (size_t)k.h * R * P : nullptr, (p->wy && nt > 0) ? R * P * 4 : 0);
      const Rsrc rWz = buf_rsrc(p->wz ? p->wz + (size_t)k.h * R * P : nullptr, (p->wz && nt > 0) ? R * P * 4 : 0);
      pbv = add4(buf_load_f32x4(rWy, tid < kGw4 ? (uint32_t)tid * 16 : kOff),
                 buf_load_f32x4(rWz, tid >= kGw4 && tid < 2 * kGw4 ? (uint32_t)(tid - kGw4) * 16 : kOff));
    }
  };
  auto c_load = [&](const Ck& k) {
    const Rsrc rC = buf_rsrc(static_cast<const T*>(p->C) + k.tok0 * R * N, k.nt > 0 ? (uint32_t)(k.nt - 1) * rsB + R * N * 2 : 0);
    const int row_a = tile * 16 + l16;
#pragma unroll
    for (int kn = 0; kn < NK; ++kn) {
      const int n0 = kn * 32 + 8 * g4;
      raw_load_buf(craw[kn], rC, has_tile ? (uint32_t)(row_a >> LOGR) * rsB + (uint32_t)(((row_a & (R - 1)) * N + n0) * 2) : kOff);
    }
  };
  // stages block j (rows 32j..32j+31 of a chunk with `rows` valid rows) from
  // this thread's item into ring slot `slot`: B rows turned by -Phi, X columns permuted
  auto stage = [&](const Raw8<T>& r, int j, int slot, int rows) {
    if (ldB) {
      const int row = tid / (N / 8), ng = tid % (N / 8);
      const int grow = 32 * j + row;
      float v[8];
      raw_unpack(r, v);
      if constexpr (PRO) {   // the row's N / 8 items sit in consecutive lanes
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        if constexpr (N / 8 == 16) {   // one 16-lane DPP row: rotate-and-add
          ss += dpp_row_ror<8>(ss);
          ss += dpp_row_ror<4>(ss);
          ss += dpp_row_ror<2>(ss);
          ss += dpp_row_ror<1>(ss);
        } else {
#pragma unroll
          for (int off = 1; off < N / 8; off <<= 1) ss += __shfl_xor(ss, off);
        }
        if (grow < rows) {   // (rows past the chunk's end stay zero)
          const float sc = rsqrtf(ss / (float)N + p->eps);
          const float* bb = s_pb + (grow & (R - 1)) * N + ng * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * sc + bb[e];
        }
      }
      // (rows past the chunk's end hold zeros: any angle will do)
      rotate_neg(v, s_cs + (min(grow, rows - 1) >> LOGR) * CSS + ng, NG);
      store8<T>(ringB(slot) + row * NS + ng * 8, v);
    } else if (ldX) {
      const int i = tid - kBI;
      const int row = i / (P / 8), pg = i % (P / 8);
      store_x_permuted<TPt>(ringX(slot) + row * XS, pg * 8, r);
    }
  };

    if (first) {   // the first chunk's loads
      first = false;
      ck = chunk_of(ticket);
      small_load(ck);
      c_load(ck);
#pragma unroll
      for (int u = 0; u < PRE; ++u) blk_load(pre[u], ck.tok0, ck.nt, u);
    }
    if (ticket >= total) break;
    const int c = ck.c, bh = ck.bh, nt = ck.nt;
    const int rows = nt * R;
    const int NB = (rows + 31) / 32;          // source blocks with valid rows
    const size_t tok0 = ck.tok0;
    unsigned long long* flags = p->flags + (size_t)bh * p->nc;
    __syncthreads();   // the previous chunk's output stage is done with s_row, S_in^T and s_misc
    // the next ticket: taken now, read by everyone after loop step kXStep - 1.
    // Nothing is computed from the atomic's result before then (it goes to LDS
    // whole, both words, so neither register of it is reused meanwhile;
    // readers mask it), so no wait for it is placed here.
    unsigned long long nextw;
    if (tid == 0) {
      s_misc[3] = 0;   // wave counter: map published
      s_misc[4] = 0;   // wave counter: state published
      nextw = atomicAdd(p->ctl, 1ull);
    }
    if constexpr (GATE) {
      if (tid < R * P / 2) *reinterpret_cast<float4*>(s_pb + 4 * tid) = pbv;
    }
    if constexpr (PRO) {
      if (tid < R * N / 2) *reinterpret_cast<float4*>(s_pb + 4 * tid) = pbv;
      // a sequence's first chunk: wave 0 reduces B_prev's column norms into
      // LDS (read when S_in is set up)
      if (c == 0 && p->Bp && wave == 0) {
        const T* Bp0 = static_cast<const T*>(p->Bp) + (size_t)bh * R * N;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float ss = 0.f;
          for (int n = lane; n < N; n += 64) {
            const float t = to_f(Bp0[r * N + n]);
            ss += t * t;
          }
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
          if (lane == 0) s_pb[2 * R * N + r] = rsqrtf(ss / (float)N + p->eps);
        }
      }
    }
    const float A = av;   // (loaded with the scalars, one chunk ahead)
    const float lmnv = (c * Q + tid + 1 < p->L && tid < nt) ? lmnv_raw : 1.f;   // (only multiplies dnv = 0 otherwise)

    // ---- chunk-local cumulative log decay (token tid) and phases ----
    float gv = 0.f, wv = 0.f, lsc = 0.f;
    if (tid < Q) {
      gv = lmv * dv;
      wv = gv + (1.f - lmnv) * dnv;
      lsc = dv * A;
    }
    lsc = wave_scan_add(lsc);
    if constexpr (PRO) {   // the step angle: dt x the raw angle
#pragma unroll
      for (int j = 0; j < ALEN; ++j)
        th4[j] = make_float4(th4[j].x * dth[j], th4[j].y * dth[j], th4[j].z * dth[j], th4[j].w * dth[j]);
    }
#pragma unroll
    for (int j = 1; j < ALEN; ++j) th4[j] = add4(th4[j], th4[j - 1]);
    const float4 atot = th4[ALEN - 1];
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
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) {   // (every read issued at once)
      const float4 t = s_sega[w * NG + cg];
      if (w < wave) abase = add4(abase, t);
    }
    __syncthreads();   // scan scratch (in the ring) is dead after this
    if (tid < Q) {
      const float lv = lsc + lbase;
      const float W = tid < nt ? __expf(l_end - lv) * wv : 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s_row[tid * R + r] = make_float4(lv, wv, gv, W);
        s_W[tid * R + r] = W;
      }
    }
    if (sg < NSEG) {
#pragma unroll
      for (int j = 0; j < ALEN; ++j) {
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
    __syncthreads();   // angles and rows done
    // factored decay of the off-diagonal mask blocks: exp(l_be - l_s) w_s,
    // be the last valid row of the row's 32-row block
    for (int k = tid; k < QR; k += kThreads) {
      float v = 0.f;
      if (k < rows) {
        const float4 rk = s_row[k];
        v = __expf(s_row[min(k | 31, rows - 1)].x - rk.x) * rk.y;
      }
      s_rw[k] = v;
    }
    // C~ fragments of this wave's output rows (turned by -Phi_t), kept in LDS:
    // each lane reads back only its own, and in registers they would not fit
    // beside the accumulators, U and the blocks in flight
    const int row_a = tile * 16 + l16;
    {
      const int ta = row_a < rows ? row_a >> LOGR : 0;
      float csc = 1.f;
      if constexpr (PRO) {   // a C row: NK slices in this lane, 4 lane groups
        float ss = 0.f;
#pragma unroll
        for (int kn = 0; kn < NK; ++kn) {
          float v[8];
          raw_unpack(craw[kn], v);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        csc = rsqrtf(ss / (float)N + p->eps);
      }
#pragma unroll
      for (int kn = 0; kn < NK; ++kn) {
        const int n0 = kn * 32 + 8 * g4;
        float v[8];
        raw_unpack(craw[kn], v);
        if constexpr (PRO) {
          if (row_a < rows) {
            const float* bc = s_pb + R * N + (row_a & (R - 1)) * N + n0;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * csc + bc[e];
          }
        }
        rotate_neg(v, s_cs + ta * CSS + n0 / 8, NG);
        Frag<T> cfk;
#pragma unroll
        for (int e = 0; e < 8; ++e) frag_set(cfk, e, v[e]);
        s_cf[kn * kThreads + tid] = cfk.v;
      }
    }
    // block 0 into slot 0; its prefetch slot takes block PRE
    stage(pre[0], 0, 0, rows);
    blk_load(pre[0], tok0, nt, PRE);
    __syncthreads();

    // ---- the source blocks ----
    const bool vk = has_tile && tile * 16 < rows;
    const int sbm = vk ? min(tile * 16 + 15, rows - 1) / 32 : -1;
    float l_t = 0.f;
    if (vk) l_t = row_a < rows ? s_row[row_a].x : 0.f;
    f32x4 uacc[NPW][PTW];
    f32x4 yacc[TPt];
#pragma unroll
    for (int i = 0; i < NPW; ++i)
#pragma unroll
      for (int jj = 0; jj < PTW; ++jj) uacc[i][jj] = zero4();
#pragma unroll
    for (int pn = 0; pn < TPt; ++pn) yacc[pn] = zero4();
    unsigned nticket = total;
    size_t ntok0 = 0;   // the next chunk's first token index and tokens (for its block loads)
    int nnt = 0;
    // blocks jb .. jb + PRE - 1 per round (the prefetch slot of block b is b % PRE)
#pragma unroll 1
    for (int jb = 0; jb < NBK; jb += PRE) {
#pragma unroll
     for (int u = 0; u < PRE; ++u) {
      const int j = jb + u;
      if (j == kXStep - 1 && tid == 0) *reinterpret_cast<unsigned long long*>(s_misc + 8) = nextw;
      if (j == kXStep) {
        nticket = (unsigned)__builtin_amdgcn_readfirstlane(s_misc[8]) & (unsigned)kTicketMask;
        const Ck nk = chunk_of(nticket);
        ntok0 = nk.tok0;
        nnt = nk.nt;
        small_load(nk);   // the next chunk's scalars and angles, in flight from here
      }
      // stage block j + 1 (loaded PRE blocks ago) into the other slot, and
      // reuse its prefetch slot for block j + 1 + PRE of this chunk, or past
      // the end, for the next chunk's first blocks
      if (j + 1 < NBK) {
        stage(pre[(u + 1) % PRE], j + 1, (j + 1) & 1, rows);
        const bool mine = j + 1 + PRE < NBK;
        blk_load(pre[(u + 1) % PRE], mine ? tok0 : ntok0, mine ? nt : nnt, mine ? j + 1 + PRE : j + 1 + PRE - NBK);
      }
      if (j < NB) {
        const T* sB = ringB(j & 1);
        const T* sX = ringX(j & 1);
        // U[n][p] += sum_k W_k B~[k][n] X[k][p] over the block's rows
        {
          const int r0 = 8 * g4;
          const float4 w0 = *reinterpret_cast<const float4*>(s_W + 32 * j + r0);
          const float4 w1 = *reinterpret_cast<const float4*>(s_W + 32 * j + r0 + 4);
          const float Wk[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
          Frag<T> xf[PTW];
#pragma unroll
          for (int jj = 0; jj < PTW; ++jj) {
            const int pt = pslot + WPN * jj;
            if (pt < TPt) frag_tr(xf[jj], sX, XS, r0, r0 + 4, pt * 16, l16);
          }
#pragma unroll
          for (int i = 0; i < NPW; ++i) {
            Frag<T> bt;
            frag_tr(bt, sB, NS, r0, r0 + 4, (nslot + NGRP * i) * 16, l16);
#pragma unroll
            for (int e = 0; e < 8; ++e) frag_set(bt, e, Wk[e] * frag_get(bt, e));
#pragma unroll
            for (int jj = 0; jj < PTW; ++jj)
              if (pslot + WPN * jj < TPt) uacc[i][jj] = mma(bt, xf[jj], uacc[i][jj]);
          }
        }
        // this wave's output tile against the block: S^T = B~ C~^T, decay x
        // two-band mask, (mask o S) X
        if (j <= sbm) {
          f32x4 st[2] = {zero4(), zero4()};
#pragma unroll
          for (int kn = 0; kn < NK; ++kn) {
            const int n0 = kn * 32 + 8 * g4;
            Frag<T> a0, a1;
            frag_lds8(a0, sB + l16 * NS + n0);
            frag_lds8(a1, sB + (16 + l16) * NS + n0);
            Frag<T> cfk;
            cfk.v = s_cf[kn * kThreads + tid];
            st[0] = mma(a0, cfk, st[0]);
            st[1] = mma(a1, cfk, st[1]);
          }
          Frag<T> pf;
          const bool va = row_a < rows;
          if (j * 32 + 32 <= tile * 16) {
            // source block wholly before the tile: every s < t, one exp per lane
            const int be = min(j * 32 + 31, rows - 1);
            const float et = va ? __expf(l_t - s_row[be].x) : 0.f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const float4 rw = *reinterpret_cast<const float4*>(s_rw + j * 32 + hh * 16 + 4 * g4);
              const float r4[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) frag_set(pf, hh * 4 + e, et * r4[e] * st[hh][e]);
            }
          } else {
            // the block holding the tile: elementwise; a lane's 4 rows in each
            // 16-row half are min(R, 4)-row groups of one token
            constexpr int RG = R < 4 ? R : 4;
            const int ta = row_a >> LOGR;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int rb = j * 32 + hh * 16 + 4 * g4;
#pragma unroll
              for (int q = 0; q < 4; q += RG) {
                const int srow = rb + q;
                const int s = srow >> LOGR;
                const float4 rw = s_row[srow];   // (srow < QR: always inside the table)
                const float mv = __expf(fminf(l_t - rw.x, 0.f)) * (s < ta ? rw.y : rw.z);
                const float m = (va && srow < rows && s <= ta) ? mv : 0.f;
#pragma unroll
                for (int e = q; e < q + RG; ++e) frag_set(pf, hh * 4 + e, m * st[hh][e]);
              }
            }
          }
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) {
            Frag<T> xf;
            frag_tr(xf, sX, XS, 4 * g4, 16 + 4 * g4, pn * 16, l16);
            yacc[pn] = mma(pf, xf, yacc[pn]);
          }
        }
      }
      __syncthreads();   // slot j & 1 is free for block j + 2
     }
    }
    const Ck nck = chunk_of(nticket);

    // ---- U turned by Psi; the map, if the predecessor's state is late ----
    float2 psi[NPW][2];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int k0 = ((nslot + NGRP * i) * 16 + 4 * g4) >> 1;
      psi[i][0] = s_cs[(nt - 1) * CSS + cs_col(k0)];
      psi[i][1] = s_cs[(nt - 1) * CSS + cs_col(k0 + 1)];
#pragma unroll
      for (int jj = 0; jj < PTW; ++jj) {
        f32x4& u = uacc[i][jj];
        const float u0 = psi[i][0].x * u[0] - psi[i][0].y * u[1], u1 = psi[i][0].y * u[0] + psi[i][0].x * u[1];
        const float u2 = psi[i][1].x * u[2] - psi[i][1].y * u[3], u3 = psi[i][1].y * u[2] + psi[i][1].x * u[3];
        u[0] = u0; u[1] = u1; u[2] = u2; u[3] = u3;
      }
    }
    const float a_c = __expf(l_end);
    auto slot_off = [&](int i, int jj) { return (uint32_t)(((i * PTW + jj) * kThreads + tid) * 16); };
    const size_t chunk_id = (size_t)bh * p->nc + c;
    // wave 0 reads the flags of up to 64 predecessors (lane k: chunk c-1-k):
    // the map decision and the look-back's first step
    const int W0 = min(c, 64);
    unsigned fpoll = 1u;
    if (wave == 0) {
      if (lane < W0)
        fpoll = flag_state(__hip_atomic_load(flags + c - 1 - lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      int need_map = 0;
      if (MAPS) need_map = c > 0 && (__ballot(lane < W0 && fpoll == 2u) & 1ull) == 0;
      if (lane == 0) {
        s_misc[2] = need_map;
        if (need_map) st_dev2(p->recs + chunk_id * (2 * NH + 2), a_c, 0.f);   // the record's decay
      }
    }
    __syncthreads();   // s_misc[2] visible; every read of the cos/sin table is done
    if (s_misc[2]) {
      const Rsrc rU = buf_rsrc(p->maps + chunk_id * SLOT, SLOT * 4);
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
        float* rec = p->recs + chunk_id * (2 * NH + 2);
        if (pslot == 0 && l16 == 0) {   // R(Psi) of this lane's two pairs
          st_dev2(rec + 2 + n0, psi[i][0].x, psi[i][0].y);
          st_dev2(rec + 2 + n0 + 2, psi[i][1].x, psi[i][1].y);
        }
#pragma unroll
        for (int jj = 0; jj < PTW; ++jj)
          if (pslot + WPN * jj < TPt) buf_store_dev4(rU, slot_off(i, jj), uacc[i][jj]);
      }
      mem_done();
      arrive_and_flag(&s_misc[3], flags + c, tag << 2 | 1u, kWaves, lane == 0);
    }
    // U waits in LDS (the dead cos/sin region) while the look-back runs: the
    // output accumulators and the next chunk's blocks already hold registers
#pragma unroll
    for (int i = 0; i < NPW; ++i)
#pragma unroll
      for (int jj = 0; jj < PTW; ++jj)
        if (pslot + WPN * jj < TPt)
          *reinterpret_cast<f32x4*>(s_U + 4 * (size_t)((i * PTW + jj) * kThreads + tid)) = uacc[i][jj];

    // ---- S_in by look-back; S_out = a R(Psi) S_in + U ----
    f32x4 FU[NPW][PTW];   // S_in
#pragma unroll
    for (int i = 0; i < NPW; ++i)
#pragma unroll
      for (int jj = 0; jj < PTW; ++jj) FU[i][jj] = zero4();
    bool chain_ok = true;
    if (c == 0) {
      // S_in = h0 + (1 - lam_0) dt_0 B_prev X_prev^T
      float kappa0 = 0.f;
      if (p->Bp) kappa0 = (1.f - p->lam[tok0]) * p->dt[tok0];
      const T* Bp = p->Bp ? static_cast<const T*>(p->Bp) + (size_t)bh * R * N : nullptr;
      const T* xp = p->xp ? static_cast<const T*>(p->xp) + (size_t)bh * R * P : nullptr;
#pragma unroll
      for (int i = 0; i < NPW; ++i) {
        const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
        float bpv[R][4];   // B_prev rows n0 .. n0 + 3 of every rank (zeros without B_prev)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint2 w = Bp ? *reinterpret_cast<const uint2*>(Bp + r * N + n0) : make_uint2(0u, 0u);
          bpv[r][0] = __uint_as_float(w.x << 16);
          bpv[r][1] = __uint_as_float(w.x & 0xffff0000u);
          bpv[r][2] = __uint_as_float(w.y << 16);
          bpv[r][3] = __uint_as_float(w.y & 0xffff0000u);
          if constexpr (PRO) {
            if (Bp) {
#pragma unroll
              for (int e = 0; e < 4; ++e) bpv[r][e] = bpv[r][e] * s_pb[2 * R * N + r] + s_pb[r * N + n0 + e];
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < PTW; ++jj) {
          const int pt = pslot + WPN * jj;
          if (pt < TPt) {
            const int hc = hcol(pt);
            float xv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) xv[r] = xp ? to_f(xp[r * P + hc]) : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float acc = 0.f;
#pragma unroll
              for (int r = 0; r < R; ++r) acc += bpv[r][e] * xv[r];
              FU[i][jj][e] = (p->h0 ? p->h0[((size_t)bh * N + n0 + e) * P + hc] : 0.f) + kappa0 * acc;
            }
          }
        }
      }
    } else if constexpr (!MAPS) {
      // without maps the predecessor publishes only its state: lane 0 of wave 0
      // waits for it (its first poll is above), then every lane loads its tiles
      if (wave == 0) {
        unsigned f = fpoll;   // (lane 0: chunk c - 1)
        unsigned spins = 0;
        int ok = 1;
        while (__builtin_amdgcn_readfirstlane(f) != 2u) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > p->spin_limit) { ok = 0; break; }
          f = flag_state(__hip_atomic_load(flags + c - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        if (lane == 0) s_misc[1] = ok;
      }
      __syncthreads();
      if (!s_misc[1]) {
        chain_ok = false;
      } else {
        const Rsrc rS = buf_rsrc(p->states + ((size_t)bh * p->nc + c - 1) * SLOT, SLOT * 4);
#pragma unroll
        for (int i = 0; i < NPW; ++i)
#pragma unroll
          for (int jj = 0; jj < PTW; ++jj)
            if (pslot + WPN * jj < TPt) FU[i][jj] = buf_load_dev4(rS, slot_off(i, jj));
      }
    } else {
      // Maps in use.  Wave 0 finds the chain: the nearest predecessor s whose
      // state is published with every chunk after it (s + 1 .. c - 1) having
      // published at least its map, polling up to 64 flags at once (lane k:
      // chunk hi - k) and waiting on a chunk that has published neither.  Then
      // every lane applies the maps oldest first to S_s:
      // X <- a_j R(Psi_j) X + U_j (one running state: few registers).
      if (wave == 0) {
        int hi = c - 1;          // the newest chunk not yet known to be in the chain
        bool first = true;       // the poll above covers the window at hi = c - 1
        int sidx = -2;
        unsigned spins = 0;
        while (hi >= 0) {
          const int W = min(hi + 1, 64);
          unsigned f = 1u;
          if (first) f = lane < W ? fpoll : 1u;
          else if (lane < W) f = flag_state(__hip_atomic_load(flags + hi - lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          first = false;
          const unsigned long long m2 = __ballot(lane < W && f == 2u);
          const unsigned long long m0 = __ballot(lane < W && f == 0u);
          const int k2 = m2 ? __builtin_ctzll(m2) : W;    // nearest state (W: none in the window)
          const int k0 = m0 ? __builtin_ctzll(m0) : 64;   // nearest chunk with nothing yet
          if (k2 < W && k0 > k2) { sidx = hi - k2; break; }   // a state behind an unbroken run of maps
          if (k0 > 0) { hi -= min(k0, W); continue; }           // maps up to the first gap (or the window's end)
          __builtin_amdgcn_s_sleep(1);                          // chunk hi has published nothing yet
          if (++spins > p->spin_limit) break;
        }
        if (lane == 0) s_misc[1] = sidx;   // (-2: the wait gave up; chunk 0 always publishes a state)
      }
      __syncthreads();
      const int sidx = s_misc[1];
      if (sidx < 0) {
        chain_ok = false;
      } else {
        const Rsrc rS = buf_rsrc(p->states + ((size_t)bh * p->nc + sidx) * SLOT, SLOT * 4);
#pragma unroll
        for (int i = 0; i < NPW; ++i)
#pragma unroll
          for (int jj = 0; jj < PTW; ++jj)
            if (pslot + WPN * jj < TPt) FU[i][jj] = buf_load_dev4(rS, slot_off(i, jj));
        // kMapGroup maps' loads at once, then applied oldest first (a slot
        // past c - 1 reloads map c - 1 and is not applied)
        for (int j0 = sidx + 1; j0 < c; j0 += kMapGroup) {
          float ax[kMapGroup];
          f32x4 r4[kMapGroup][NPW], um[kMapGroup][NPW][PTW];
#pragma unroll
          for (int g = 0; g < kMapGroup; ++g) {
            const size_t jid = (size_t)bh * p->nc + min(j0 + g, c - 1);
            const Rsrc rU = buf_rsrc(p->maps + jid * SLOT, SLOT * 4);
            // the map's record (a_j, then cos/sin Psi_j per pair) through a
            // uniform descriptor: 32-bit offsets, no per-lane 64-bit addresses
            const Rsrc rR = buf_rsrc(p->recs + jid * (2 * NH + 2), (2 * NH + 2) * 4);
            ax[g] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rR, 0, 0, kCpolDevice));
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
              const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
              r4[g][i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rR, (uint32_t)(2 + n0) * 4, 0, kCpolDevice));
#pragma unroll
              for (int jj = 0; jj < PTW; ++jj)
                um[g][i][jj] = pslot + WPN * jj < TPt ? buf_load_dev4(rU, slot_off(i, jj)) : zero4();
            }
          }
#pragma unroll
          for (int g = 0; g < kMapGroup; ++g) {
            if (j0 + g >= c) break;
#pragma unroll
            for (int i = 0; i < NPW; ++i) {
              const f32x4 q = r4[g][i];
#pragma unroll
              for (int jj = 0; jj < PTW; ++jj) {
                const f32x4 u = um[g][i][jj];
                f32x4& x = FU[i][jj];
                const float x0 = ax[g] * (q[0] * x[0] - q[1] * x[1]) + u[0];
                const float x1 = ax[g] * (q[1] * x[0] + q[0] * x[1]) + u[1];
                const float x2 = ax[g] * (q[2] * x[2] - q[3] * x[3]) + u[2];
                const float x3 = ax[g] * (q[3] * x[2] + q[2] * x[3]) + u[3];
                x[0] = x0; x[1] = x1; x[2] = x2; x[3] = x3;
              }
            }
          }
        }
      }
    }
    const float nanv = __builtin_nanf("");
    if (!chain_ok && tid == 0)   // the wait gave up: recorded for m3_prefill_status
      __hip_atomic_fetch_or(p->err, (unsigned long long)kErrLookback, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool publish = c + 1 < p->nc;
    const Rsrc rSo = buf_rsrc(p->states + chunk_id * SLOT, publish ? SLOT * 4 : 0);
    // S_in^T goes into the (now free) ring for the readout
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int n0 = (nslot + NGRP * i) * 16 + 4 * g4;
#pragma unroll
      for (int jj = 0; jj < PTW; ++jj) {
        const int pt = pslot + WPN * jj;
        if (pt < TPt) {
          const int pc = pt * 16 + l16;
          f32x4 si = FU[i][jj];
          if (!chain_ok) si[0] = si[1] = si[2] = si[3] = nanv;
          const float sv4[4] = {si[0], si[1], si[2], si[3]};
          store_row<T, 4>(s_H + pc * NS + n0, sv4);
          const float q0 = a_c * si[0], q1 = a_c * si[1], q2 = a_c * si[2], q3 = a_c * si[3];
          const f32x4 u = *reinterpret_cast<const f32x4*>(s_U + 4 * (size_t)((i * PTW + jj) * kThreads + tid));
          const float o0 = psi[i][0].x * q0 - psi[i][0].y * q1 + u[0];
          const float o1 = psi[i][0].y * q0 + psi[i][0].x * q1 + u[1];
          const float o2 = psi[i][1].x * q2 - psi[i][1].y * q3 + u[2];
          const float o3 = psi[i][1].y * q2 + psi[i][1].x * q3 + u[3];
          if (publish) {
            buf_store_dev4(rSo, slot_off(i, jj), f32x4{o0, o1, o2, o3});
          } else if (p->h_out) {
            float* ho = p->h_out + ((size_t)bh * N + n0) * P + hcol(pt);
            ho[0] = o0; ho[P] = o1; ho[2 * P] = o2; ho[3 * P] = o3;
          }
        }
      }
    }
    // the state flag goes up once the stores are done: at once when the
    // successor is likely waiting for it, else after the readout below, which
    // runs while the stores complete
    const bool late = p->late_flag != 0;
    if (publish && !late) {
      mem_done();
      arrive_and_flag(&s_misc[4], flags + c, tag << 2 | 2u, kWaves, lane == 0);
    }
    __syncthreads();   // S_in^T complete in LDS

    // GATE: the gate input of this lane's tokens (TPt columns each), in flight
    // through the inter-chunk readout
    constexpr int kRG = R < 4 ? R : 4;   // a lane's 4 output rows: 4 / kRG tokens
    uint2 zr[4 / kRG];
    if constexpr (GATE) {
#pragma unroll
      for (int q = 0; q < 4 / kRG; ++q) {
        const int row0 = tile * 16 + 4 * g4 + q * kRG;
        zr[q] = make_uint2(0u, 0u);
        if (vk && p->z && row0 < rows)
          zr[q] = *reinterpret_cast<const uint2*>(static_cast<const T*>(p->z) + (tok0 + (size_t)(row0 >> LOGR) * tstride) * P + TPt * l16);
      }
    }
    // ---- inter-chunk term exp(l_t) C~_t^T S_in, added to the intra term; y ----
    if (vk) {
      float e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = tile * 16 + 4 * g4 + e;
        e4[e] = row < rows ? __expf(s_row[row].x) : 0.f;
      }
#pragma unroll
      for (int pn = 0; pn < TPt; ++pn) {
        f32x4 ia = zero4();
#pragma unroll
        for (int kn = 0; kn < NK; ++kn) {
          Frag<T> hf;
          frag_lds8(hf, s_H + (pn * 16 + l16) * NS + kn * 32 + 8 * g4);
          Frag<T> cfk;
          cfk.v = s_cf[kn * kThreads + tid];
          ia = mma(cfk, hf, ia);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[pn][e] += e4[e] * ia[e];
      }
    }
    if (publish && late) {
      mem_done();
      arrive_and_flag(&s_misc[4], flags + c, tag << 2 | 2u, kWaves, lane == 0);
    }
    // the next chunk's C rows (cf is dead), after the state flag (the wait
    // before a flag covers every load in flight): in flight during the y
    // stores and the next chunk's start
    c_load(nck);
    if (vk && !GATE) {
      T* Yg = static_cast<T*>(p->y) + tok0 * R * P;
      const size_t rowstepX = tstride * R * P;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = tile * 16 + 4 * g4 + e;
        if (row < rows) {
          float v[TPt];
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) v[pn] = chain_ok ? yacc[pn][e] : nanv;
          store_row<T, TPt>(Yg + (row >> LOGR) * rowstepX + (row & (R - 1)) * P + TPt * l16, v);
        }
      }
    } else if (vk) {
      // gated readout: a lane's 4 rows are whole tokens' ranks (RG rows per
      // token, R <= 4); it holds head columns TPt*l16 .. TPt*l16+TPt-1 (P = 64:
      // 4 columns, one 8-byte run of the token's gate input, loaded after the
      // block loop).  The head's w_y and w_z wait in LDS (loaded one chunk
      // ahead)
      const size_t rowstepO = tstride * P;
      T* Og = static_cast<T*>(p->out) + tok0 * P;
      const T* Zg = p->z ? static_cast<const T*>(p->z) + tok0 * P : nullptr;
      const float* wyh = p->wy ? s_pb + TPt * l16 : nullptr;           // the head's w_y, w_z in LDS
      const float* wzh = p->wz ? s_pb + R * P + TPt * l16 : nullptr;
      constexpr int RG = R < 4 ? R : 4;
#pragma unroll
      for (int q = 0; q < 4; q += RG) {
        const int row0 = tile * 16 + 4 * g4 + q;
        const bool valid = row0 < rows;
        const int tk = row0 >> LOGR;
        float zv[TPt], o[TPt];
        const uint2 zw = zr[q / RG];
        zv[0] = __uint_as_float(zw.x << 16);
        zv[1] = __uint_as_float(zw.x & 0xffff0000u);
        zv[2] = __uint_as_float(zw.y << 16);
        zv[3] = __uint_as_float(zw.y & 0xffff0000u);
#pragma unroll
        for (int pn = 0; pn < TPt; ++pn) o[pn] = 0.f;
#pragma unroll
        for (int j = q; j < q + RG; ++j) {
          const int r = (row0 + j - q) & (R - 1);
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) {
            float v = yacc[pn][j];
            if (wyh) v *= wyh[r * P + pn];
            if (Zg) {
              const float gz = (wzh ? wzh[r * P + pn] : 1.f) * zv[pn];
              v *= gz * __builtin_amdgcn_rcpf(1.f + __expf(-gz));   // silu (1-ulp reciprocal)
            }
            o[pn] += v;
          }
        }
        if (valid) {
#pragma unroll
          for (int pn = 0; pn < TPt; ++pn) o[pn] = chain_ok ? o[pn] : nanv;
          store_row<T, TPt>(Og + tk * rowstepO + TPt * l16, o);
        }
      }
    }
    ticket = nticket;
    ck = nck;
  }

  // ---- stop: the last workgroup of the grid readies the control words ----
  if (wave0 == 0 && __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0) {
    const KParams pe = reload_params();
    const unsigned long long tag = ((unsigned long long)(unsigned)s_misc[7] << 32) | (unsigned)s_misc[6];
    const unsigned long long epoch = tag - 1;   // (tag = epoch + 1)
    unsigned long long* exitctr = pe->ctl + 2;
    const unsigned long long e = atomicAdd(exitctr, 1ull);
    if (e == gridDim.x - 1) {
      __hip_atomic_store(exitctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pe->ctl, (epoch + 1) << kTicketBits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int N, int P, int R, int NBK, int PRE, bool MAPS, bool PRO, bool GATE>
hipError_t launch_v(const FusedParams& p, size_t grid, bool late, hipStream_t stream) {
  constexpr size_t lds = lds_of(NBK * 32 / R, R, N, P, PRO, GATE).total;
  const void* fn = reinterpret_cast<const void*>(stream_kernel<N, P, R, NBK, PRE, MAPS, PRO, GATE>);
  static std::atomic<int> scratch_state{0};   // 0 unknown, 1 none, 2 uses scratch
  int st = scratch_state.load(std::memory_order_relaxed);
  if (st == 0) {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess) return hipErrorInvalidDeviceFunction;
    st = fa.localSizeBytes > 0 ? 2 : 1;
    scratch_state.store(st, std::memory_order_relaxed);
  }
  if (st == 2) return hipErrorNotSupported;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  static std::atomic<unsigned long long> lds_set{0};
  if (lds > 64 * 1024 && (dev < 0 || !(lds_set.load(std::memory_order_acquire) >> dev & 1ull))) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (e != hipSuccess) return e;
    if (dev >= 0) lds_set.fetch_or(1ull << dev, std::memory_order_acq_rel);
  }
  FusedParams q = p;
  q.use_maps = MAPS ? 1 : 0;
  q.late_flag = late ? 1 : 0;
  hipLaunchKernelGGL((stream_kernel<N, P, R, NBK, PRE, MAPS, PRO, GATE>), dim3((unsigned)grid), dim3(kThreads), lds, stream, q);
  return hipGetLastError();
}

template <int N, int P, int R, int NBK, int PRE, bool PRO, bool GATE>
hipError_t launch(const FusedParams& p, hipStream_t stream) {
  constexpr size_t lds = lds_of(NBK * 32 / R, R, N, P, PRO, GATE).total;
  // resident workgroups per device (cached): the persistent grid (both map
  // modes have the same launch bounds and LDS)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  static std::atomic<int> cache[64];
  int resident = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (resident <= 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(stream_kernel<N, P, R, NBK, PRE, true, PRO, GATE>), kThreads, lds) != hipSuccess)
      return hipErrorInvalidValue;
    resident = cus * per;
    if (resident <= 0) return hipErrorInvalidValue;
    if (dev >= 0) cache[dev].store(resident, std::memory_order_relaxed);
  }
  const size_t chunks = (size_t)p.batch * p.H * p.nc;
  const size_t grid = std::min(chunks, (size_t)resident);
  // maps pay off when many chunks of one sequence are in flight at once: more
  // than 8 resident workgroups per sequence.  Without maps each chunk of a
  // sequence waits for its predecessor's state, a hand-off of ~2.2-2.5 us at
  // N = 128; with maps a chunk publishes its map and composes a run of them,
  // ~1 us more per chunk.  Measured on 65,536-token sequences (N = 128, R = 4,
  // 256 resident workgroups): 8 in flight, states only 4% faster; 16 and 32,
  // maps 1.5 and 2.2 times faster.
  if ((size_t)resident > 8 * (size_t)p.batch * p.H) return launch_v<N, P, R, NBK, PRE, true, PRO, GATE>(p, grid, false, stream);
  // States only.  With at most 4 chunks of a sequence in flight the hand-off
  // chain (~2.5 us a link) stays well inside the time a workgroup spends on its
  // chunks, so a chunk's state flag waits for the end of its readout, and the
  // state stores complete meanwhile instead of holding up the whole workgroup.
  const bool late = (size_t)resident <= 4 * (size_t)p.batch * p.H;
  return launch_v<N, P, R, NBK, PRE, false, PRO, GATE>(p, grid, late, stream);
}

}  // namespace stream

// The shapes the streaming kernel takes: bf16, P = 64, no gate or prologue;
// N = 64 with R = 1, 2 or 4 at 128 or 256 (token, rank) rows per chunk; N = 128
// at 128 rows (R = 1, 2, 4) or 256 rows (R = 4): the chunks whose LDS fits.
bool stream_supported(int dtype, int N, int P, int R, int Q, int gated, int pro) {
  if (dtype != M3_BF16 || P != 64 || (N != 64 && N != 128) || (gated && pro)) return false;
  if (R != 1 && R != 2 && R != 4) return false;
  if (Q * R != 128 && Q * R != 256) return false;
  return Q * (N / 2) <= kFusedAngleCap && stream::lds_of(Q, R, N, P, pro != 0).total <= (size_t)kLdsBudget;
}

size_t stream_lds_bytes(int Q, int R, int N, int P) { return stream::lds_of(Q, R, N, P).total; }
size_t stream_lds_bytes_pro(int Q, int R, int N, int P) { return stream::lds_of(Q, R, N, P, true).total; }

template <bool PRO, bool GATE>
hipError_t launch_stream_pro(const FusedParams& p, hipStream_t s) {
  const int rows = p.Q * p.R;
#define M3_STREAM_R(NN, NBK, PRE)                                        \
  switch (p.R) {                                                         \
    case 1: return stream::launch<NN, 64, 1, NBK, PRE, PRO, GATE>(p, s); \
    case 2: return stream::launch<NN, 64, 2, NBK, PRE, PRO, GATE>(p, s); \
    case 4: return stream::launch<NN, 64, 4, NBK, PRE, PRO, GATE>(p, s); \
    default: return hipErrorInvalidValue;                                \
  }
  if (p.P != 64) return hipErrorInvalidValue;
  if (p.N == 128) {
    // (128 tokens at R = 2, 256 rows, do not fit: the cos/sin table of 128
    // tokens, the ring and the C~ fragments of 256 rows need ~164 KB of LDS)
    if (rows == 256 && p.R == 4) return stream::launch<128, 64, 4, 8, 4, PRO, GATE>(p, s);
    if (rows == 128 && p.R == 1) return stream::launch<128, 64, 1, 4, 2, PRO, GATE>(p, s);
    if (rows == 128 && p.R == 2) return stream::launch<128, 64, 2, 4, 2, PRO, GATE>(p, s);
    if (rows == 128 && p.R == 4) return stream::launch<128, 64, 4, 4, 2, PRO, GATE>(p, s);
    return hipErrorInvalidValue;
  } else if (p.N == 64) {
    if (rows == 256) { M3_STREAM_R(64, 8, 4) }
    if (rows == 128) { M3_STREAM_R(64, 4, 2) }
  }
#undef M3_STREAM_R
  return hipErrorInvalidValue;
}

hipError_t launch_stream_prefill(const FusedParams& p, hipStream_t s) {
  if (p.pro && p.out) return hipErrorInvalidValue;   // (no entry point fuses both)
  if (p.out) return launch_stream_pro<false, true>(p, s);
  return p.pro ? launch_stream_pro<true, false>(p, s) : launch_stream_pro<false, false>(p, s);
}

}  // namespace m3
