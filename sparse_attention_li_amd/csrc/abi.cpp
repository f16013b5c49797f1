// Host side of the C ABI declared in include/sparse_li.h: argument checks,
// workspace carving, launch-shape choice.  Every check runs before anything
// is enqueued, so a failing call leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "launch.h"
#include "sparse_li.h"

namespace {

thread_local char g_err[512] = "";

li_status fail(li_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

li_status hip_fail(hipError_t e, const char* what) {
  return fail(LI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Number of compute units of the current device (cached per device id).
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

struct IdxLayout {
  int chunk, ncm;
  size_t off_counters, off_refs, off_cnts, off_cand, total;
};

IdxLayout idx_layout(int B, int n_q, bool fp8, int max_pages) {
  IdxLayout l;
  l.chunk = sli::idx_decode_chunk(B, n_q, fp8, max_pages, device_cus());
  const long long maxlen = (long long)max_pages * 64;
  l.ncm = (int)std::max<long long>(1, (maxlen + l.chunk - 1) / l.chunk);
  const size_t T = (size_t)B * n_q;
  size_t o = 0;
  // The exchange counters sit in a fixed region at the start whatever the
  // geometry, so a workspace reused for another batch shape never finds the
  // previous call's lists where it expects zeroed counters.
  l.off_counters = o;
  o = round_up(o + (size_t)(sli::kMaxSeqs + 1) * sli::kCounterStride * 4, 256);  // + the launch line
  l.off_refs = o;
  o = round_up(o + T * l.ncm * 2 * 8, 256);
  l.off_cnts = o;
  o = round_up(o + T * l.ncm * 8, 256);
  l.off_cand = o;
  o = round_up(o + T * l.ncm * l.chunk * 8, 256);
  l.total = o;
  return l;
}

// Polls an exchange wait makes before giving up.  Only the test hook
// li_set_exchange_patience changes it (to force the exact fallbacks).
constexpr int kDefaultPatience = 20000;
std::atomic<int> g_patience{kDefaultPatience};

int spin_max() { return g_patience.load(std::memory_order_relaxed); }

// Splits of the index row so that about one workgroup per CU is busy (an
// attention workgroup fills a CU: one wave per SIMD).  Workgroups hold every
// head of a token (65 to 128 heads), or a block of 32 or 64.  Small calls
// split down to one 32-row tile per workgroup (batch 1 x 2048, top-K 256:
// 8 splits, 16.8 -> 13.5 us against two-tile splits).
void sfa_shape(int T, int H, int top_k, int& n_splits, int& split_len) {
  const int cus = device_cus();
  const int hpb = sli::sfa_heads_per_block(H);
  const int head_blocks = (H + hpb - 1) / hpb;
  const int per_split = T * head_blocks;
  int s = std::max(1, (cus + per_split - 1) / per_split);
  s = std::min(s, std::max(1, top_k / 32));
  split_len = (top_k + s - 1) / s;
  split_len = (split_len + 31) / 32 * 32;
  split_len = std::min(split_len, sli::kMaxSplitRows);
  n_splits = (top_k + split_len - 1) / split_len;
}

size_t sfa_partials_bytes(int T, int H, int n_splits) {
  if (n_splits == 1) return 256;
  return round_up((size_t)T * n_splits * H * 512 * 2, 256) + round_up((size_t)T * n_splits * H * 2 * 4, 256);
}

li_status check_paged(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                      int32_t max_pages, int32_t num_pages) {
  if (num_seqs <= 0) return fail(LI_ERR_INVALID_ARG, "num_seqs must be positive (got %d)", num_seqs);
  if (q_per_seq <= 0) return fail(LI_ERR_INVALID_ARG, "q_per_seq must be positive (got %d)", q_per_seq);
  if (max_pages <= 0 || num_pages <= 0)
    return fail(LI_ERR_INVALID_ARG, "max_pages and num_pages must be positive (got %d, %d)", max_pages, num_pages);
  if (!seq_lens || !block_table) return fail(LI_ERR_INVALID_ARG, "seq_lens and block_table must not be NULL");
  if ((long long)num_seqs * q_per_seq > (1LL << 30)) return fail(LI_ERR_UNSUPPORTED, "too many tokens");
  return LI_OK;
}

// Every check of li_score_topk except the workspace's.
li_status check_topk(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q, const uint8_t* q_scales,
                     const float* w, int32_t k_dtype, const void* k_cache, const void* k_scales, int32_t top_k,
                     const int32_t* idx_out) {
  li_status st = check_paged(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages);
  if (st != LI_OK) return st;
  if (top_k < 1 || top_k > LI_MAX_TOP_K) return fail(LI_ERR_INVALID_ARG, "top_k must be in [1, 2048] (got %d)", top_k);
  if (!q || !w || !k_cache || !idx_out) return fail(LI_ERR_INVALID_ARG, "q, w, k_cache and idx_out must not be NULL");
  if (q_dtype != LI_BF16 && q_dtype != LI_FP8) return fail(LI_ERR_UNSUPPORTED, "unknown q_dtype %d", q_dtype);
  const bool fp8 = q_dtype == LI_FP8;
  if (fp8 ? (k_dtype != LI_FP8 && k_dtype != LI_MXFP8) : k_dtype != LI_BF16)
    return fail(LI_ERR_UNSUPPORTED, "k_dtype %d does not go with q_dtype %d (BF16 with BF16; FP8 with FP8 or MXFP8)",
                k_dtype, q_dtype);
  if (fp8 && (!q_scales || !k_scales)) return fail(LI_ERR_INVALID_ARG, "FP8 needs q_scales and k_scales");
  if (!fp8 && (q_scales || k_scales)) return fail(LI_ERR_INVALID_ARG, "BF16 takes no scales (pass NULL)");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(w))
    return fail(LI_ERR_INVALID_ARG, "q, w and k_cache must be 16-byte aligned");
  if (fp8 && (reinterpret_cast<uintptr_t>(k_scales) & 3u)) return fail(LI_ERR_INVALID_ARG, "k_scales must be 4-byte aligned");
  if (q_per_seq > 2) {
    if (fp8) return fail(LI_ERR_UNSUPPORTED, "the prefill indexer is built for bf16 only");
    if ((long long)num_seqs * ((q_per_seq + 3) / 4) > 0x7fffffffLL) return fail(LI_ERR_UNSUPPORTED, "grid too large");
  } else {
    if (num_seqs > sli::kMaxSeqs) return fail(LI_ERR_UNSUPPORTED, "num_seqs %d exceeds %d", num_seqs, sli::kMaxSeqs);
    const IdxLayout l = idx_layout(num_seqs, q_per_seq, fp8, max_pages);
    if (l.ncm > sli::kMaxChunksPerSeq)
      return fail(LI_ERR_UNSUPPORTED, "max_pages*64 = %lld positions exceeds %d", (long long)max_pages * 64,
                  sli::kMaxChunksPerSeq * l.chunk);
  }
  return LI_OK;
}

// Every check of sfa_decode / sfa_prefill except the workspace's.
li_status check_sfa(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                    int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                    const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                    int32_t top_k, float sm_scale, const void* out) {
  li_status st = check_paged(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages);
  if (st != LI_OK) return st;
  if (top_k < 1 || top_k > LI_MAX_TOP_K) return fail(LI_ERR_INVALID_ARG, "top_k must be in [1, 2048] (got %d)", top_k);
  if (!q || !kv_cache || !idx || !out) return fail(LI_ERR_INVALID_ARG, "q, kv_cache, idx and out must not be NULL");
  if (num_heads != 16 && num_heads != 32 && num_heads != 64 && num_heads != 128)
    return fail(LI_ERR_UNSUPPORTED, "num_heads must be 16, 32, 64 or 128 (got %d)", num_heads);
  if (kv_dtype != LI_BF16 && kv_dtype != LI_FP8 && kv_dtype != LI_FP8_ROPE_BF16)
    return fail(LI_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
  const bool fp8 = kv_dtype != LI_BF16, rope16 = kv_dtype == LI_FP8_ROPE_BF16;
  if (fp8) {
    if (!kv_scales) return fail(LI_ERR_INVALID_ARG, "FP8 latent cache needs kv_scales");
    if (!rope16 && kv_scale_groups != 1 && kv_scale_groups != 5)
      return fail(LI_ERR_UNSUPPORTED, "kv_scale_groups must be 1 or 5 (got %d)", kv_scale_groups);
    if (rope16 && kv_scale_groups != 1 && kv_scale_groups != 4)
      return fail(LI_ERR_UNSUPPORTED, "kv_scale_groups must be 1 or 4 with a bf16 rope (got %d)", kv_scale_groups);
  } else if (kv_scales) {
    return fail(LI_ERR_INVALID_ARG, "BF16 latent cache takes no scales (pass NULL)");
  }
  if (!(sm_scale == sm_scale)) return fail(LI_ERR_INVALID_ARG, "sm_scale is NaN");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out))
    return fail(LI_ERR_INVALID_ARG, "q, kv_cache and out must be 16-byte aligned");
  return LI_OK;
}

// Shape of the single-launch decode step: the indexer's chunks of 4096
// positions, one workgroup each, which attends the positions of the
// selection in its chunk (one partial per chunk).
struct StepLayout {
  int ncm;
  size_t off_part_o, off_part_ml, total;
};

StepLayout step_layout(int B, int max_pages, int H, int top_k) {
  StepLayout s;
  (void)top_k;
  const long long maxlen = (long long)max_pages * 64;
  s.ncm = (int)std::max<long long>(1, (maxlen + 4095) / 4096);
  size_t o = round_up((size_t)(sli::kMaxSeqs + 1) * sli::kCounterStride * 4, 256);
  o = round_up(o + (size_t)B * s.ncm * 2 * 8, 256);
  o = round_up(o + (size_t)B * s.ncm * 8, 256);
  o = round_up(o + (size_t)B * s.ncm * 4096 * 8, 256);
  s.off_part_o = o;
  o = round_up(o + (size_t)B * s.ncm * H * 512 * 2, 256);
  s.off_part_ml = o;
  o = round_up(o + (size_t)B * s.ncm * H * 2 * 4, 256);
  s.total = o;
  return s;
}

// The step runs as one launch for bf16 caches, one query token per request,
// 128 heads, and a grid of at most one workgroup per compute unit.
bool step_fused(int B, int q_per_seq, int q_dtype, int k_dtype, int kv_dtype, int H, int max_pages) {
  if (q_per_seq != 1 || q_dtype != LI_BF16 || k_dtype != LI_BF16 || kv_dtype != LI_BF16 || H != 128) return false;
  const long long ncm = std::max<long long>(1, ((long long)max_pages * 64 + 4095) / 4096);
  return ncm <= 64 && (long long)(B + 7) / 8 * 8 * ncm <= device_cus();
}


// Launch part of li_score_topk (arguments already checked).
li_status run_topk(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                   int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q, const uint8_t* q_scales,
                   const float* w, int32_t k_dtype, const void* k_cache, const void* k_scales, int32_t top_k,
                   int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream) {
  const bool fp8 = q_dtype == LI_FP8;
  if (q_per_seq > 2) {
    // prefill chunk: many causal queries per request, selection state on chip
    sli::IdxPrefillArgs pa;
    pa.B = num_seqs;
    pa.n_q = q_per_seq;
    pa.max_pages = max_pages;
    pa.num_pages = num_pages;
    pa.top_k = top_k;
    pa.seq_lens = seq_lens;
    pa.block_table = block_table;
    pa.q = q;
    pa.w = w;
    pa.k = k_cache;
    pa.idx_out = idx_out;
    (void)workspace;
    (void)workspace_bytes;
    hipError_t e = sli::launch_idx_prefill(pa, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LI_OK : hip_fail(e, "prefill indexer launch");
  }
  const IdxLayout l = idx_layout(num_seqs, q_per_seq, fp8, max_pages);
  if (!workspace) return fail(LI_ERR_WORKSPACE, "workspace must not be NULL");
  if (workspace_bytes < l.total)
    return fail(LI_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, l.total);
  if (!aligned16(workspace)) return fail(LI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  sli::IdxDecodeArgs a;
  a.B = num_seqs;
  a.n_q = q_per_seq;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.top_k = top_k;
  a.n_chunks_max = l.ncm;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.q = q;
  a.q_scales = q_scales;
  a.w = w;
  a.k = k_cache;
  a.k_scales = k_scales;
  a.k_mx = k_dtype == LI_MXFP8;
  a.idx_out = idx_out;
  char* ws = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<uint32_t*>(ws + l.off_counters);
  a.refs = reinterpret_cast<uint64_t*>(ws + l.off_refs);
  a.cnts = reinterpret_cast<uint64_t*>(ws + l.off_cnts);
  a.cand = reinterpret_cast<uint64_t*>(ws + l.off_cand);
  a.spin_max = spin_max();
  a.xcd_local = sli::idx_decode_xcd_local(num_seqs, l.ncm, l.chunk, device_cus()) ? 1 : 0;
  hipError_t e = sli::launch_idx_decode(a, l.chunk, fp8, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "indexer launch");
}
}  // namespace

li_status sli::report(li_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

extern "C" {

const char* li_version(void) { return "sparse_li 0.1.0 (gfx950)"; }

const char* li_last_error(void) { return g_err; }

void li_set_exchange_patience(int32_t polls) {
  g_patience.store(polls < 0 || polls >= (1 << 30) ? kDefaultPatience : polls, std::memory_order_relaxed);
}

size_t li_score_topk_workspace_size(int32_t num_seqs, int32_t q_per_seq, int32_t max_pages, int32_t top_k) {
  if (num_seqs <= 0 || q_per_seq <= 0 || max_pages <= 0 || top_k <= 0) return 0;
  if (q_per_seq > 2) return 256;  // the prefill kernel keeps its selection state in LDS
  // (the layout depends on the chunk length, which differs between bf16 and
  // FP8 for two-token calls: the larger of the two)
  return std::max(idx_layout(num_seqs, q_per_seq, false, max_pages).total,
                  idx_layout(num_seqs, q_per_seq, true, max_pages).total);
}

li_status li_workspace_zero(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(LI_ERR_INVALID_ARG, "workspace must not be NULL");
  if (workspace_bytes % 4 != 0 || !aligned16(workspace))
    return fail(LI_ERR_INVALID_ARG, "workspace must be 16-byte aligned and a multiple of 4 bytes");
  hipError_t e = sli::launch_zero_fill(workspace, workspace_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "zero-fill launch");
}

li_status li_score_topk(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                        int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q,
                        const uint8_t* q_scales, const float* w, int32_t k_dtype, const void* k_cache,
                        const void* k_scales, int32_t top_k, int32_t* idx_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const li_status st = check_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q,
                                  q_scales, w, k_dtype, k_cache, k_scales, top_k, idx_out);
  if (st != LI_OK) return st;
  return run_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q, q_scales, w, k_dtype,
                  k_cache, k_scales, top_k, idx_out, workspace, workspace_bytes, stream);
}

size_t sfa_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t top_k) {
  if (num_tokens <= 0 || num_heads <= 0 || top_k <= 0) return 0;
  int s, len;
  sfa_shape(num_tokens, num_heads, top_k, s, len);
  return sfa_partials_bytes(num_tokens, num_heads, s);
}

static li_status sfa_common(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                            int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                            const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                            int32_t top_k, float sm_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const li_status st = check_sfa(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q, num_heads,
                                 kv_dtype, kv_cache, kv_scales, kv_scale_groups, idx, top_k, sm_scale, out);
  if (st != LI_OK) return st;
  const bool fp8 = kv_dtype != LI_BF16, rope16 = kv_dtype == LI_FP8_ROPE_BF16;
  const int T = num_seqs * q_per_seq;
  int s, len;
  sfa_shape(T, num_heads, top_k, s, len);
  sli::SfaArgs a;
  a.T = T;
  a.n_q = q_per_seq;
  a.H = num_heads;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.top_k = top_k;
  a.kv_groups = fp8 ? kv_scale_groups : 1;
  a.rope_bf16 = rope16 ? 1 : 0;
  a.n_splits = s;
  a.split_len = len;
  a.head_blocks = (num_heads + sli::sfa_heads_per_block(num_heads) - 1) / sli::sfa_heads_per_block(num_heads);
  a.sm_scale = sm_scale;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.q = q;
  a.kv = kv_cache;
  a.kv_scales = kv_scales;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (s > 1) {
    const size_t need = sfa_workspace_size(T, num_heads, top_k);
    if (!workspace) return fail(LI_ERR_WORKSPACE, "workspace must not be NULL");
    if (workspace_bytes < need)
      return fail(LI_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(LI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<__bf16*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + round_up((size_t)T * s * num_heads * 512 * 2, 256));
  }
  hipError_t e = sli::launch_sfa(a, fp8, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "attention launch");
}

li_status sfa_decode(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                     const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                     int32_t top_k, float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return sfa_common(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q, num_heads, kv_dtype, kv_cache,
                    kv_scales, kv_scale_groups, idx, top_k, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

li_status sfa_prefill(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                      int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                      const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                      int32_t top_k, float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return sfa_common(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q, num_heads, kv_dtype, kv_cache,
                    kv_scales, kv_scale_groups, idx, top_k, sm_scale, out, lse, workspace, workspace_bytes, stream);
}

size_t li_decode_step_workspace_size(int32_t num_seqs, int32_t q_per_seq, int32_t max_pages, int32_t num_heads,
                                     int32_t top_k) {
  if (num_seqs <= 0 || q_per_seq <= 0 || q_per_seq > 2 || max_pages <= 0 || num_heads <= 0 || top_k <= 0) return 0;
  // the two-launch form: the indexer's workspace, then the attention's
  const size_t two = round_up(li_score_topk_workspace_size(num_seqs, q_per_seq, max_pages, top_k), 256) +
                     sfa_workspace_size(num_seqs * q_per_seq, num_heads, top_k);
  const size_t one = q_per_seq == 1 ? step_layout(num_seqs, max_pages, num_heads, top_k).total : 0;
  return std::max(two, one);
}

li_status li_decode_step(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                         int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q_idx,
                         const uint8_t* q_scales, const float* w, int32_t k_dtype, const void* k_cache,
                         const void* k_scales, const void* q, int32_t num_heads, int32_t kv_dtype,
                         const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, int32_t top_k,
                         float sm_scale, int32_t* idx_out, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (q_per_seq > 2) return fail(LI_ERR_UNSUPPORTED, "li_decode_step takes 1 or 2 query tokens per request");
  li_status st = check_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q_idx, q_scales,
                            w, k_dtype, k_cache, k_scales, top_k, idx_out);
  if (st != LI_OK) return st;
  st = check_sfa(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q, num_heads, kv_dtype, kv_cache,
                 kv_scales, kv_scale_groups, idx_out, top_k, sm_scale, out);
  if (st != LI_OK) return st;
  const size_t need = li_decode_step_workspace_size(num_seqs, q_per_seq, max_pages, num_heads, top_k);
  if (!workspace) return fail(LI_ERR_WORKSPACE, "workspace must not be NULL");
  if (workspace_bytes < need)
    return fail(LI_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(LI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  if (!step_fused(num_seqs, q_per_seq, q_dtype, k_dtype, kv_dtype, num_heads, max_pages)) {
    // two launches on the stream: the indexer, then the attention
    const size_t wi = round_up(li_score_topk_workspace_size(num_seqs, q_per_seq, max_pages, top_k), 256);
    st = run_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q_idx, q_scales, w,
                  k_dtype, k_cache, k_scales, top_k, idx_out, ws, wi, stream);
    if (st != LI_OK) return st;
    return sfa_common(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q, num_heads, kv_dtype,
                      kv_cache, kv_scales, kv_scale_groups, idx_out, top_k, sm_scale, out, lse, ws + wi,
                      workspace_bytes - wi, stream);
  }
  const StepLayout l = step_layout(num_seqs, max_pages, num_heads, top_k);
  sli::StepArgs s;
  sli::IdxDecodeArgs& a = s.idx;
  a.B = num_seqs;
  a.n_q = 1;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.top_k = top_k;
  a.n_chunks_max = l.ncm;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.q = q_idx;
  a.q_scales = nullptr;
  a.w = w;
  a.k = k_cache;
  a.k_scales = nullptr;
  a.k_mx = false;
  a.idx_out = idx_out;
  a.spin_max = spin_max();
  // a request's chunks on one XCD: its query (read by every chunk's
  // attention) is fetched into that XCD's L2 once, not once per chunk
  a.xcd_local = 1;
  {
    size_t o = 0;
    a.counters = reinterpret_cast<uint32_t*>(ws + o);
    o = round_up(o + (size_t)(sli::kMaxSeqs + 1) * sli::kCounterStride * 4, 256);
    a.refs = reinterpret_cast<uint64_t*>(ws + o);
    o = round_up(o + (size_t)num_seqs * l.ncm * 2 * 8, 256);
    a.cnts = reinterpret_cast<uint64_t*>(ws + o);
    o = round_up(o + (size_t)num_seqs * l.ncm * 8, 256);
    a.cand = reinterpret_cast<uint64_t*>(ws + o);
  }
  sli::SfaArgs& t = s.att;
  t.T = num_seqs;
  t.n_q = 1;
  t.H = num_heads;
  t.max_pages = max_pages;
  t.num_pages = num_pages;
  t.top_k = top_k;
  t.kv_groups = 1;
  t.rope_bf16 = 0;
  t.n_splits = l.ncm;    // partial slots per token: one per chunk
  t.split_len = top_k;
  t.head_blocks = 1;
  t.sm_scale = sm_scale;
  t.seq_lens = seq_lens;
  t.block_table = block_table;
  t.q = q;
  t.kv = kv_cache;
  t.kv_scales = nullptr;
  t.idx = idx_out;
  t.out = out;
  t.lse = lse;
  t.part_o = reinterpret_cast<__bf16*>(ws + l.off_part_o);
  t.part_ml = reinterpret_cast<float*>(ws + l.off_part_ml);
  hipError_t e = sli::launch_decode_step(s, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "decode step launch");
}

li_status li_validate_paged(int32_t num_seqs, const int32_t* seq_lens, const int32_t* block_table, int32_t max_pages,
                            int32_t num_pages, int32_t* bad_out, void* stream) {
  if (num_seqs <= 0 || max_pages <= 0 || num_pages <= 0)
    return fail(LI_ERR_INVALID_ARG, "num_seqs, max_pages and num_pages must be positive (got %d, %d, %d)", num_seqs,
                max_pages, num_pages);
  if (!seq_lens || !block_table || !bad_out)
    return fail(LI_ERR_INVALID_ARG, "seq_lens, block_table and bad_out must not be NULL");
  if (reinterpret_cast<uintptr_t>(bad_out) & 3u) return fail(LI_ERR_INVALID_ARG, "bad_out must be 4-byte aligned");
  sli::ValidateArgs a;
  a.B = num_seqs;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.bad_out = bad_out;
  hipError_t e = sli::launch_validate_paged(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "validation launch");
}

li_status li_quantize_mxfp8(int32_t n_rows, int32_t row_len, const void* x, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (n_rows < 0) return fail(LI_ERR_INVALID_ARG, "n_rows must not be negative (got %d)", n_rows);
  if (row_len <= 0 || row_len % 32 != 0)
    return fail(LI_ERR_INVALID_ARG, "row_len must be a positive multiple of 32 (got %d)", row_len);
  if (n_rows == 0) return LI_OK;
  if (!x || !codes || !scales) return fail(LI_ERR_INVALID_ARG, "x, codes and scales must not be NULL");
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0)
    return fail(LI_ERR_INVALID_ARG, "x must be 16-byte aligned and codes 8-byte aligned");
  sli::QuantArgs a;
  a.n_rows = n_rows;
  a.row_len = row_len;
  a.x = x;
  a.codes = codes;
  a.scales = scales;
  hipError_t e = sli::launch_mxfp8_quant(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "MXFP8 quantisation launch");
}

li_status li_cache_append(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                          int32_t max_pages, int32_t num_pages, const void* k_new, int32_t k_dtype, void* k_cache,
                          void* k_scales, const void* kv_new, int32_t kv_dtype, void* kv_cache, float* kv_scales,
                          int32_t kv_scale_groups, void* stream) {
  li_status st = check_paged(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages);
  if (st != LI_OK) return st;
  if (!k_new && !kv_new) return fail(LI_ERR_INVALID_ARG, "k_new and kv_new must not both be NULL");
  sli::AppendArgs a;
  a.B = num_seqs;
  a.n_q = q_per_seq;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.k_new = k_new;
  a.k_fp8 = false;
  a.k_mx = false;
  a.k_cache = k_cache;
  a.k_scales = k_scales;
  a.kv_new = kv_new;
  a.kv_fp8 = false;
  a.kv_rope_bf16 = false;
  a.kv_groups = 1;
  a.kv_cache = kv_cache;
  a.kv_scales = kv_scales;
  if (k_new) {
    if (k_dtype != LI_BF16 && k_dtype != LI_FP8 && k_dtype != LI_MXFP8)
      return fail(LI_ERR_UNSUPPORTED, "unknown k_dtype %d", k_dtype);
    a.k_fp8 = k_dtype != LI_BF16;
    a.k_mx = k_dtype == LI_MXFP8;
    if (!k_cache) return fail(LI_ERR_INVALID_ARG, "k_cache must not be NULL when k_new is given");
    if (a.k_fp8 && !k_scales) return fail(LI_ERR_INVALID_ARG, "an FP8 key cache needs k_scales");
    if (k_dtype == LI_FP8 && (reinterpret_cast<uintptr_t>(k_scales) & 3u))
      return fail(LI_ERR_INVALID_ARG, "f32 k_scales must be 4-byte aligned");
    if (!aligned16(k_new) || !aligned16(k_cache)) return fail(LI_ERR_INVALID_ARG, "k_new and k_cache must be 16-byte aligned");
  }
  if (kv_new) {
    if (kv_dtype != LI_BF16 && kv_dtype != LI_FP8 && kv_dtype != LI_FP8_ROPE_BF16)
      return fail(LI_ERR_UNSUPPORTED, "unknown kv_dtype %d", kv_dtype);
    a.kv_fp8 = kv_dtype != LI_BF16;
    a.kv_rope_bf16 = kv_dtype == LI_FP8_ROPE_BF16;
    if (!kv_cache) return fail(LI_ERR_INVALID_ARG, "kv_cache must not be NULL when kv_new is given");
    if (a.kv_fp8) {
      if (!kv_scales) return fail(LI_ERR_INVALID_ARG, "an FP8 latent cache needs kv_scales");
      if (!a.kv_rope_bf16 && kv_scale_groups != 1 && kv_scale_groups != 5)
        return fail(LI_ERR_UNSUPPORTED, "kv_scale_groups must be 1 (per row) or 5 (per 128-wide tile), got %d",
                    kv_scale_groups);
      if (a.kv_rope_bf16 && kv_scale_groups != 1 && kv_scale_groups != 4)
        return fail(LI_ERR_UNSUPPORTED, "kv_scale_groups must be 1 or 4 with a bf16 rope, got %d", kv_scale_groups);
      a.kv_groups = kv_scale_groups;
    }
    if (!aligned16(kv_new) || !aligned16(kv_cache)) return fail(LI_ERR_INVALID_ARG, "kv_new and kv_cache must be 16-byte aligned");
  }
  hipError_t e = sli::launch_cache_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LI_OK : hip_fail(e, "cache append launch");
}

}  // extern "C"
