// Drives the host side of the C ABI (include/m3.h) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU: every query over a grid of valid and
// invalid shapes, the status strings, and for each entry point the argument
// errors the host reports before any launch (NULL shape and pointers, bad
// dtype and rank, aliasing, small workspace) plus the empty-batch no-op.  The
// device pointers are fake addresses the host never dereferences.  Exits 0 and
// prints "abi ok"; a sanitizer report aborts the process.
#include <cstdint>
#include <cstdio>

#include "m3.h"

static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { std::fprintf(stderr, "FAIL: %s (line %d)\n", msg, __LINE__); ++fails; } } while (0)

static void* far(int i) { return reinterpret_cast<void*>((uintptr_t)(1ull << 44) + (uintptr_t)i * (1ull << 36)); }
static float* farf(int i) { return static_cast<float*>(far(i)); }

static void queries() {
  const int batches[] = {-1, 0, 1, 3}, lens[] = {-5, 0, 1, 63, 4096, 1 << 26}, heads[] = {0, 1, 32};
  const int hds[] = {0, 16, 48, 64, 128, 256}, sts[] = {0, 2, 16, 64, 128, 256, 512}, ranks[] = {0, 1, 3, 4, 8, 16};
  const int chunks[] = {-1, 0, 16, 64, 100, 128, 256, 512}, dts[] = {0, 1, 7};
  long n = 0;
  for (int b : batches) for (int L : lens) for (int H : heads) for (int P : hds) for (int N : sts)
    for (int R : ranks) for (int q : chunks) for (int dt : dts) {
      const m3_shape s{b, L, H, P, N, R, q, dt};
      const size_t ws = m3_prefill_workspace_bytes(&s);
      const int32_t c0 = m3_prefill_chunk_used(&s), c1 = m3_prefill_gated_chunk_used(&s);
      const int32_t c2 = m3_prefill_prologue_chunk_used(&s), cm = m3_prefill_max_chunk(&s);
      const size_t bw = m3_scan_backward_workspace_bytes(&s);
      CHECK(c0 >= 0 && c1 >= 0 && c2 >= 0 && cm >= 0, "chunk queries non-negative");
      if (q > 0 && c0 > 0) CHECK(c0 == q, "a requested chunk is exact");
      if (c0 == 0 && ws > 0 && c1 == 0 && c2 == 0) CHECK(false, "workspace for a refused shape");
      (void)bw;
      ++n;
    }
  const m3_shape* nul = nullptr;
  CHECK(m3_prefill_workspace_bytes(nul) == 0 && m3_prefill_chunk_used(nul) == 0, "NULL shape queries");
  CHECK(m3_scan_backward_workspace_bytes(nul) == 0, "NULL shape backward query");
  std::printf("%ld shapes queried\n", n);
}

static void statuses() {
  for (int st = -3; st < 12; ++st) CHECK(m3_status_str(static_cast<m3_status>(st)) != nullptr, "status string");
  CHECK(m3_version() > 0, "version");
}

static void prefill_errors() {
  const m3_shape ok{2, 64, 3, 64, 64, 1, 0, M3_BF16};
  const size_t ws = m3_prefill_workspace_bytes(&ok);
  CHECK(ws > 0, "workspace of a valid shape");
  auto call = [&](const m3_shape* s, int x_, int y_, void* wsp, size_t wsb) {
    return m3_scan_prefill(s, far(x_), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr, nullptr,
                           nullptr, far(y_), farf(8), wsp, wsb, nullptr);
  };
  CHECK(call(nullptr, 0, 7, far(9), ws) == M3_ERR_NULL, "NULL shape");
  const m3_shape bad_dt{2, 64, 3, 64, 64, 1, 0, 5};
  CHECK(call(&bad_dt, 0, 7, far(9), ws) == M3_ERR_DTYPE, "bad dtype");
  const m3_shape bad_r{2, 64, 3, 64, 64, 3, 0, M3_BF16};
  CHECK(call(&bad_r, 0, 7, far(9), ws) == M3_ERR_SHAPE, "rank 3");
  const m3_shape n256{2, 64, 3, 64, 256, 1, 0, M3_BF16};
  CHECK(call(&n256, 0, 7, far(9), 1ull << 40) == M3_ERR_SHAPE, "N = 256 prefill");
  CHECK(call(&ok, 0, 0, far(9), ws) == M3_ERR_ALIAS, "y aliases x");
  CHECK(call(&ok, 0, 7, nullptr, ws) == M3_ERR_WORKSPACE, "NULL workspace");
  CHECK(call(&ok, 0, 7, far(9), ws - 1) == M3_ERR_WORKSPACE, "small workspace");
  CHECK(m3_scan_prefill(&ok, nullptr, far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr, nullptr, nullptr,
                        far(7), farf(8), far(9), ws, nullptr) == M3_ERR_NULL, "NULL x");
  CHECK(m3_scan_prefill(&ok, far(0), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr, far(10), nullptr,
                        far(7), farf(8), far(9), ws, nullptr) == M3_ERR_NULL, "B_prev without x_prev");
  const m3_shape empty{0, 64, 3, 64, 64, 1, 0, M3_BF16};
  CHECK(m3_scan_prefill(&empty, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, nullptr, 0, nullptr) == M3_OK, "empty batch");
  const m3_shape big{64, 65536, 32, 64, 128, 4, 0, M3_BF16};
  CHECK(m3_scan_prefill_noalloc(&big, far(0), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr, nullptr,
                                nullptr, far(7), farf(8), nullptr) == M3_ERR_WORKSPACE, "noalloc oversize");
  const m3_prologue pro{1e-5f, nullptr, nullptr};
  CHECK(m3_scan_prefill_prologue(&ok, nullptr, far(0), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr,
                                 nullptr, nullptr, far(7), farf(8), far(9), ws, nullptr) == M3_ERR_NULL, "prologue NULL");
  CHECK(m3_scan_prefill_prologue(&ok, &pro, far(0), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr,
                                 nullptr, nullptr, far(0), farf(8), far(9), ws, nullptr) == M3_ERR_ALIAS,
        "prologue y aliases x");
  CHECK(m3_scan_prefill_gated(&ok, far(0), far(1), far(2), farf(3), farf(4), farf(5), farf(6), nullptr, nullptr,
                              nullptr, far(11), farf(12), farf(13), far(11), farf(8), far(9), ws, nullptr) ==
            M3_ERR_ALIAS, "gated out aliases z");
  CHECK(m3_prefill_status(nullptr, 0, nullptr) == M3_ERR_NULL, "status of NULL workspace");
}

static void decode_errors() {
  const m3_shape ok{128, 1, 32, 64, 128, 4, 0, M3_BF16};
  auto call = [&](const m3_shape* s, float* h, int Bp, int B) {
    return m3_decode_step(s, h, far(Bp), far(11), far(0), far(B), far(2), farf(3), farf(4), farf(5), farf(6), far(7),
                          nullptr);
  };
  CHECK(call(nullptr, farf(8), 10, 1) == M3_ERR_NULL, "NULL shape");
  CHECK(call(&ok, nullptr, 10, 1) == M3_ERR_NULL, "NULL state");
  CHECK(call(&ok, farf(8), 1, 1) == M3_ERR_ALIAS, "B_prev aliases B");
  const m3_shape fp32{128, 1, 32, 64, 128, 4, 0, M3_FP32};
  CHECK(m3_decode_step_bf16_state(&fp32, far(8), far(10), far(11), far(0), far(1), far(2), farf(3), farf(4),
                                  farf(5), farf(6), far(7), nullptr) == M3_ERR_DTYPE, "bf16 state with fp32 inputs");
  CHECK(m3_decode_step_gated(&ok, farf(8), far(10), far(11), far(0), far(1), far(2), farf(3), farf(4), farf(5),
                             farf(6), far(12), farf(13), farf(14), nullptr, nullptr) == M3_ERR_NULL, "gated NULL out");
  CHECK(m3_decode_step_prologue(&ok, nullptr, farf(8), far(10), far(11), far(0), far(1), far(2), farf(3), farf(4),
                                farf(5), farf(6), far(7), nullptr) == M3_ERR_NULL, "prologue NULL");
}

static void backward_errors() {
  const m3_shape ok{2, 64, 3, 64, 128, 4, 0, M3_BF16};
  const size_t ws = m3_scan_backward_workspace_bytes(&ok);
  CHECK(ws > 0, "backward workspace");
  auto call = [&](const float* theta, float* dtheta, float* dx, void* wsp, size_t wsb) {
    return m3_scan_backward(&ok, far(0), far(1), far(2), farf(3), farf(4), farf(5), theta, nullptr, nullptr,
                            nullptr, far(7), nullptr, dx, farf(9), farf(10), farf(11), farf(12), farf(13), dtheta,
                            nullptr, nullptr, nullptr, wsp, wsb, nullptr);
  };
  CHECK(call(nullptr, farf(14), farf(8), far(15), ws) == M3_ERR_NULL, "dtheta without theta");
  CHECK(call(farf(6), farf(14), nullptr, far(15), ws) == M3_ERR_NULL, "NULL dx");
  CHECK(call(farf(6), farf(14), farf(8), nullptr, ws) == M3_ERR_WORKSPACE, "NULL workspace");
  CHECK(call(farf(6), farf(14), farf(8), far(15), ws - 1) == M3_ERR_WORKSPACE, "small workspace");
  CHECK(call(farf(6), farf(14), farf(0), far(15), ws) == M3_ERR_ALIAS, "dx aliases x");
}

int main() {
  queries();
  statuses();
  prefill_errors();
  decode_errors();
  backward_errors();
  if (fails) {
    std::fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  std::printf("abi ok\n");
  return 0;
}
