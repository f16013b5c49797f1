// Calls every host-side entry point of the C ABI (abi.cpp, shapes.cpp) with
// exactly sized host buffers, linked against the launch stand-ins of
// launch_stubs.cpp, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_native_sanitizers.py).  Workspaces
// are allocated at exactly the size the ABI's size query returns, so a region
// the ABI carves past that size is an overflow the sanitizer reports.  Also
// checks the status and message of the argument errors.  (The allocation-free
// indexer lives in device code and is not part of this build.)
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "launch_stubs.h"
#include "sparse_li.h"

namespace {

int failures = 0;

#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);    \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

// An exactly sized heap buffer (malloc's alignment is 16 bytes).
struct Buf {
  void* p = nullptr;
  explicit Buf(size_t n) {
    p = malloc(n ? n : 1);
    if (!p) abort();
    memset(p, 0, n ? n : 1);
  }
  ~Buf() { free(p); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  template <class T>
  T* as() const { return static_cast<T*>(p); }
};

// A paged batch over a pool of at most 64 pages (pages are shared between
// requests: the host code never reads the cache, and the launch stand-ins
// touch the whole pool, so its size is free).
struct Batch {
  int B, max_pages, num_pages;
  std::vector<int32_t> lens, bt;
  Batch(int B_, int max_pages_, int len)
      : B(B_), max_pages(max_pages_), num_pages((int)std::min<long long>(64, (long long)B_ * max_pages_)) {
    lens.assign(B, len);
    bt.resize((size_t)B * max_pages);
    for (size_t i = 0; i < bt.size(); ++i) bt[i] = (int32_t)(i % num_pages);
  }
};

void topk_case(int B, int n_q, int qd, int kd, int max_pages, int top_k, bool expect_prefill) {
  Batch b(B, max_pages, max_pages * 64);
  const size_t T = (size_t)B * n_q, E = qd == LI_BF16 ? 2 : 1;
  Buf q(T * 64 * 128 * E), qs(T * 64 * 4), w(T * 64 * 4), k((size_t)b.num_pages * 64 * 128 * E),
      ks((size_t)b.num_pages * 64 * 4), idx(T * top_k * 4);
  const size_t wsb = li_score_topk_workspace_size(B, n_q, max_pages, top_k);
  CHECK(wsb > 0);
  Buf ws(wsb);
  g_stub.calls.clear();
  const bool fp8 = qd != LI_BF16;
  const li_status st = li_score_topk(B, n_q, b.lens.data(), b.bt.data(), max_pages, b.num_pages, qd, q.p,
                                     fp8 ? qs.as<uint8_t>() : nullptr, w.as<float>(), kd, k.p, fp8 ? ks.p : nullptr,
                                     top_k, idx.as<int32_t>(), ws.p, wsb, nullptr);
  if (st != LI_OK) fprintf(stderr, "li_score_topk: %s\n", li_last_error());
  CHECK(st == LI_OK);
  CHECK(g_stub.calls == (expect_prefill ? "idx_prefill " : "idx_decode "));
  // the workspace clear covers what the size query returned
  CHECK(li_workspace_zero(ws.p, wsb / 4 * 4, nullptr) == LI_OK);
  if (!expect_prefill) {
    // a workspace smaller than required is refused before any launch
    g_stub.calls.clear();
    CHECK(li_score_topk(B, n_q, b.lens.data(), b.bt.data(), max_pages, b.num_pages, qd, q.p,
                        fp8 ? qs.as<uint8_t>() : nullptr, w.as<float>(), kd, k.p, fp8 ? ks.p : nullptr, top_k,
                        idx.as<int32_t>(), ws.p, 64, nullptr) == LI_ERR_WORKSPACE);
    CHECK(g_stub.calls.empty() && strlen(li_last_error()) > 0);
  }
}

void sfa_case(bool prefill, int B, int n_q, int H, int kvd, int groups, int max_pages, int top_k, bool with_lse) {
  Batch b(B, max_pages, max_pages * 64);
  const size_t T = (size_t)B * n_q;
  const size_t row = kvd == LI_BF16 ? 1152 : kvd == LI_FP8 ? 576 : 640;
  Buf q(T * H * 576 * 2), kv((size_t)b.num_pages * 64 * row), kvs((size_t)b.num_pages * 64 * groups * 4),
      idx(T * top_k * 4), out(T * H * 512 * 2), lse(T * H * 4);
  const size_t wsb = sfa_workspace_size((int)T, H, top_k);
  CHECK(wsb > 0);
  Buf ws(wsb);
  g_stub.calls.clear();
  auto fn = prefill ? sfa_prefill : sfa_decode;
  const li_status st = fn(B, n_q, b.lens.data(), b.bt.data(), max_pages, b.num_pages, q.p, H, kvd, kv.p,
                          kvd == LI_BF16 ? nullptr : kvs.as<float>(), groups, idx.as<int32_t>(), top_k, 0.04f, out.p,
                          with_lse ? lse.as<float>() : nullptr, ws.p, wsb, nullptr);
  if (st != LI_OK) fprintf(stderr, "sfa: %s\n", li_last_error());
  CHECK(st == LI_OK);
  CHECK(g_stub.calls == "sfa ");
}

void step_case(int B, int n_q, int dt, int H, int max_pages, int top_k, const char* want) {
  Batch b(B, max_pages, max_pages * 64 - 7);
  const size_t T = (size_t)B * n_q, E = dt == LI_BF16 ? 2 : 1;
  const int kvd = dt == LI_BF16 ? LI_BF16 : LI_FP8;
  const size_t row = kvd == LI_BF16 ? 1152 : 576;
  Buf qi(T * 64 * 128 * E), qs(T * 64 * 4), w(T * 64 * 4), k((size_t)b.num_pages * 64 * 128 * E),
      ks((size_t)b.num_pages * 64 * 4), q(T * H * 576 * 2), kv((size_t)b.num_pages * 64 * row),
      kvs((size_t)b.num_pages * 64 * 4), idx(T * top_k * 4), out(T * H * 512 * 2), lse(T * H * 4);
  const size_t wsb = li_decode_step_workspace_size(B, n_q, max_pages, H, top_k);
  CHECK(wsb > 0);
  Buf ws(wsb);
  const bool fp8 = dt != LI_BF16;
  g_stub.calls.clear();
  const li_status st = li_decode_step(
      B, n_q, b.lens.data(), b.bt.data(), max_pages, b.num_pages, dt, qi.p, fp8 ? qs.as<uint8_t>() : nullptr,
      w.as<float>(), dt, k.p, fp8 ? ks.p : nullptr, q.p, H, kvd, kv.p, fp8 ? kvs.as<float>() : nullptr, 1, top_k,
      0.04f, idx.as<int32_t>(), out.p, lse.as<float>(), ws.p, wsb, nullptr);
  if (st != LI_OK) fprintf(stderr, "li_decode_step: %s\n", li_last_error());
  CHECK(st == LI_OK);
  if (g_stub.calls != want) fprintf(stderr, "step B=%d n_q=%d: launches '%s', expected '%s'\n", B, n_q,
                                    g_stub.calls.c_str(), want);
  CHECK(g_stub.calls == want);
}

void quant_and_append() {
  g_stub.calls.clear();
  CHECK(li_quantize_mxfp8(0, 128, nullptr, nullptr, nullptr, nullptr) == LI_OK);
  CHECK(g_stub.calls.empty());
  {
    Buf x(3 * 128 * 2), codes(3 * 128), scales(3 * 4);
    CHECK(li_quantize_mxfp8(3, 128, x.p, codes.as<uint8_t>(), scales.as<uint8_t>(), nullptr) == LI_OK);
    CHECK(li_quantize_mxfp8(3, 100, x.p, codes.as<uint8_t>(), scales.as<uint8_t>(), nullptr) == LI_ERR_INVALID_ARG);
  }
  const int kinds[][4] = {// k_dtype, kv_dtype, groups, n_q
                          {LI_BF16, LI_BF16, 1, 1},
                          {LI_FP8, LI_FP8, 5, 2},
                          {LI_MXFP8, LI_FP8_ROPE_BF16, 4, 1},
                          {LI_FP8, LI_FP8_ROPE_BF16, 1, 2}};
  for (const auto& kd : kinds) {
    Batch b(3, 4, 100);
    const int n_q = kd[3];
    const size_t T = (size_t)b.B * n_q, P = (size_t)b.num_pages * 64;
    const size_t krow = kd[0] == LI_BF16 ? 256 : 128, vrow = kd[1] == LI_BF16 ? 1152 : kd[1] == LI_FP8 ? 576 : 640;
    Buf kn(T * 128 * 2), kc(P * krow), ksc(P * 4), vn(T * 576 * 2), vc(P * vrow), vsc(P * kd[2] * 4);
    const bool kf = kd[0] != LI_BF16, vf = kd[1] != LI_BF16;
    g_stub.calls.clear();
    CHECK(li_cache_append(b.B, n_q, b.lens.data(), b.bt.data(), b.max_pages, b.num_pages, kn.p, kd[0], kc.p,
                          kf ? ksc.p : nullptr, vn.p, kd[1], vc.p, vf ? vsc.as<float>() : nullptr, kd[2],
                          nullptr) == LI_OK);
    CHECK(g_stub.calls == "append ");
    // only one of the two caches
    CHECK(li_cache_append(b.B, n_q, b.lens.data(), b.bt.data(), b.max_pages, b.num_pages, nullptr, 0, nullptr,
                          nullptr, vn.p, kd[1], vc.p, vf ? vsc.as<float>() : nullptr, kd[2], nullptr) == LI_OK);
  }
}

// argument errors: status, message, and nothing launched
void errors() {
  Batch b(2, 4, 200);
  Buf big(1 << 20), ws(1 << 20);
  void* P = big.p;
  const int32_t* L = b.lens.data();
  const int32_t* T = b.bt.data();
  auto topk = [&](int B, int n_q, int qd, const void* q, const uint8_t* qs, int kd, const void* ks, int top_k,
                  void* w, size_t wb) {
    g_stub.calls.clear();
    const li_status st = li_score_topk(B, n_q, L, T, 4, 8, qd, q, qs, static_cast<float*>(P), kd, P, ks, top_k,
                                       static_cast<int32_t*>(P), w, wb, nullptr);
    CHECK(g_stub.calls.empty() && strlen(li_last_error()) > 0);
    return st;
  };
  const uint8_t* S = static_cast<const uint8_t*>(P);
  CHECK(topk(0, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 0, LI_BF16, P, nullptr, LI_BF16, nullptr, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 0, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 2049, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, LI_BF16, nullptr, nullptr, LI_BF16, nullptr, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, 9, P, nullptr, 9, nullptr, 64, ws.p, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(topk(2, 1, LI_BF16, P, nullptr, LI_FP8, nullptr, 64, ws.p, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(topk(2, 1, LI_FP8, P, nullptr, LI_FP8, P, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, LI_FP8, P, S, LI_MXFP8, S + 2, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 1, LI_BF16, S + 4, nullptr, LI_BF16, nullptr, 64, ws.p, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(topk(2, 3, LI_FP8, P, S, LI_FP8, P, 64, ws.p, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(topk(2, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 64, nullptr, 1 << 20) == LI_ERR_WORKSPACE);
  CHECK(topk(2, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 64, static_cast<char*>(ws.p) + 4, (1 << 20) - 4) ==
        LI_ERR_INVALID_ARG);
  CHECK(topk(4097, 1, LI_BF16, P, nullptr, LI_BF16, nullptr, 64, ws.p, 1 << 20) == LI_ERR_UNSUPPORTED);

  auto sfa = [&](int H, int kvd, const float* kvs, int groups, float sm, size_t wb) {
    g_stub.calls.clear();
    const li_status st = sfa_decode(2, 1, L, T, 4, 8, P, H, kvd, P, kvs, groups, static_cast<int32_t*>(P), 2048, sm,
                                    P, nullptr, ws.p, wb, nullptr);
    CHECK(g_stub.calls.empty() && strlen(li_last_error()) > 0);
    return st;
  };
  const float* F = static_cast<const float*>(P);
  CHECK(sfa(48, LI_BF16, nullptr, 1, 0.1f, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(sfa(128, 7, nullptr, 1, 0.1f, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(sfa(128, LI_BF16, F, 1, 0.1f, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(sfa(128, LI_FP8, nullptr, 1, 0.1f, 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(sfa(128, LI_FP8, F, 3, 0.1f, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(sfa(128, LI_FP8_ROPE_BF16, F, 5, 0.1f, 1 << 20) == LI_ERR_UNSUPPORTED);
  CHECK(sfa(128, LI_BF16, nullptr, 1, __builtin_nanf(""), 1 << 20) == LI_ERR_INVALID_ARG);
  CHECK(sfa(128, LI_BF16, nullptr, 1, 0.1f, 16) == LI_ERR_WORKSPACE);

  g_stub.calls.clear();
  CHECK(li_decode_step(2, 3, L, T, 4, 8, LI_BF16, P, nullptr, F, LI_BF16, P, nullptr, P, 128, LI_BF16, P, nullptr, 1,
                       64, 0.1f, static_cast<int32_t*>(P), P, nullptr, ws.p, 1 << 20, nullptr) == LI_ERR_UNSUPPORTED);
  CHECK(li_decode_step(2, 1, L, T, 4, 8, LI_BF16, P, nullptr, F, LI_BF16, P, nullptr, P, 128, LI_BF16, P, nullptr, 1,
                       64, 0.1f, static_cast<int32_t*>(P), P, nullptr, ws.p, 64, nullptr) == LI_ERR_WORKSPACE);
  CHECK(g_stub.calls.empty());
  CHECK(li_workspace_zero(nullptr, 64, nullptr) == LI_ERR_INVALID_ARG);
  CHECK(li_workspace_zero(ws.p, 62, nullptr) == LI_ERR_INVALID_ARG);
  CHECK(li_cache_append(2, 1, L, T, 4, 8, nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr, nullptr, 1, nullptr) ==
        LI_ERR_INVALID_ARG);
  // size queries of nonsense shapes are 0
  CHECK(li_score_topk_workspace_size(0, 1, 4, 64) == 0 && sfa_workspace_size(1, 0, 64) == 0 &&
        li_decode_step_workspace_size(1, 3, 4, 128, 64) == 0);
}

}  // namespace

int main() {
  CHECK(strstr(li_version(), "gfx950") != nullptr);
  // decode indexer: one and two tokens, every key format, the chunk and
  // block-layout choices (small and large batches, long requests)
  topk_case(1, 1, LI_BF16, LI_BF16, 32, 256, false);
  topk_case(1, 1, LI_BF16, LI_BF16, 2048, 2048, false);
  topk_case(8, 2, LI_BF16, LI_BF16, 2048, 2048, false);
  topk_case(3, 2, LI_FP8, LI_FP8, 100, 2048, false);
  topk_case(5, 1, LI_FP8, LI_MXFP8, 64, 512, false);
  topk_case(64, 1, LI_BF16, LI_BF16, 256, 2048, false);
  topk_case(2, 2, LI_BF16, LI_BF16, 4096, 2048, false);  // 256 chunks of the smallest length
  topk_case(4096, 1, LI_BF16, LI_BF16, 2, 64, false);
  topk_case(2, 9, LI_BF16, LI_BF16, 16, 2048, true);  // prefill chunk
  // the block-layout choice: several rounds of the chip
  topk_case(64, 1, LI_BF16, LI_BF16, 1024, 2048, false);
  CHECK(g_stub.xcd_local == 1);
  topk_case(4, 1, LI_BF16, LI_BF16, 1024, 2048, false);
  CHECK(g_stub.xcd_local == 0);
  // another device (80 compute units): the per-device CU cache
  g_stub.device = 1;
  topk_case(8, 1, LI_BF16, LI_BF16, 2048, 2048, false);
  g_stub.device = 0;
  // the test hook for the exchange patience
  li_set_exchange_patience(5);
  topk_case(2, 1, LI_BF16, LI_BF16, 256, 2048, false);
  CHECK(g_stub.spin_max == 5);
  li_set_exchange_patience(-1);
  topk_case(2, 1, LI_BF16, LI_BF16, 256, 2048, false);
  CHECK(g_stub.spin_max > 5);

  // attention: every head count, latent format and scale grouping, with and
  // without lse, one split and many
  const int heads[] = {16, 32, 64, 128};
  for (int H : heads) {
    sfa_case(false, 1, 1, H, LI_BF16, 1, 32, 2048, true);
    sfa_case(false, 64, 2, H, LI_BF16, 1, 32, 2048, false);
  }
  sfa_case(false, 3, 1, 128, LI_FP8, 5, 40, 2048, true);
  sfa_case(false, 3, 1, 64, LI_FP8, 1, 40, 512, true);
  sfa_case(false, 2, 2, 128, LI_FP8_ROPE_BF16, 4, 40, 2048, true);
  sfa_case(false, 2, 1, 128, LI_FP8_ROPE_BF16, 1, 40, 100, false);
  sfa_case(true, 2, 33, 128, LI_BF16, 1, 40, 2048, true);
  sfa_case(true, 1, 5, 64, LI_FP8, 5, 8, 64, true);

  // the whole step: one launch (bf16, one token, 128 heads, a grid within one
  // round of the chip) and two launches otherwise
  step_case(8, 1, LI_BF16, 128, 2048, 2048, "step ");
  step_case(1, 1, LI_BF16, 128, 16, 2048, "step ");
  step_case(32, 1, LI_BF16, 128, 64, 512, "step ");
  step_case(64, 1, LI_BF16, 128, 2048, 2048, "idx_decode sfa ");
  step_case(4, 2, LI_BF16, 128, 512, 2048, "idx_decode sfa ");
  step_case(4, 1, LI_FP8, 128, 512, 2048, "idx_decode sfa ");
  step_case(4, 1, LI_BF16, 64, 512, 2048, "idx_decode sfa ");

  quant_and_append();
  {
    Batch b(5, 7, 300);
    Buf bad(4);
    g_stub.calls.clear();
    CHECK(li_validate_paged(b.B, b.lens.data(), b.bt.data(), b.max_pages, b.num_pages, bad.as<int32_t>(), nullptr) ==
          LI_OK);
    CHECK(g_stub.calls == "validate ");
    CHECK(li_validate_paged(0, b.lens.data(), b.bt.data(), b.max_pages, b.num_pages, bad.as<int32_t>(), nullptr) ==
          LI_ERR_INVALID_ARG);
    CHECK(li_validate_paged(b.B, b.lens.data(), b.bt.data(), b.max_pages, b.num_pages, nullptr, nullptr) ==
          LI_ERR_INVALID_ARG);
  }
  errors();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi_sanitize: ok\n");
  return 0;
}
