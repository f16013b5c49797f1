// Host stand-ins for the kernel launches and for the few HIP runtime calls the
// C ABI makes, so that abi.cpp and shapes.cpp can be built for the CPU with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/native/abi_sanitize.cpp).
// "Device" buffers are host allocations here.  Each launch stand-in reads or
// writes the whole extent its kernel indexes, derived from the launch
// arguments alone: a workspace region carved past the caller's allocation, or
// an extent the arguments understate, then shows up as a sanitizer report.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "launch.h"
#include "launch_stubs.h"

StubLog g_stub;

// ---- the HIP runtime calls of abi.cpp ----

hipError_t hipGetDevice(int* dev) {
  *dev = g_stub.device;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int dev) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *v = dev == 0 ? 256 : 80;
  return hipSuccess;
}

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }

namespace {

[[noreturn]] void die(const char* what) {
  fprintf(stderr, "launch stub: %s\n", what);
  abort();
}

unsigned sink = 0;

void rd(const void* p, size_t n, const char* what) {
  if (n == 0) return;
  if (!p) die(what);
  const unsigned char* b = static_cast<const unsigned char*>(p);
  unsigned s = 0;
  for (size_t i = 0; i < n; ++i) s += b[i];
  sink += s;
}

void wr(void* p, size_t n, const char* what) {
  if (n == 0) return;
  if (!p) die(what);
  memset(p, 0, n);
}

void seqs(const int32_t* seq_lens, const int32_t* bt, int B, int max_pages) {
  rd(seq_lens, (size_t)B * 4, "seq_lens");
  rd(bt, (size_t)B * max_pages * 4, "block_table");
}

void idx_decode(const sli::IdxDecodeArgs& a, int chunk, bool fp8) {
  if (chunk != 256 && chunk != 1024 && chunk != 2048 && chunk != 4096 && chunk != 8192) die("chunk length");
  if ((long long)a.n_chunks_max * chunk < (long long)a.max_pages * 64) die("chunks do not cover max_pages");
  if (a.n_chunks_max > sli::kMaxChunksPerSeq || a.B > sli::kMaxSeqs) die("grid limits");
  const size_t T = (size_t)a.B * a.n_q, E = fp8 ? 1 : 2, ncm = (size_t)a.n_chunks_max;
  seqs(a.seq_lens, a.block_table, a.B, a.max_pages);
  rd(a.q, T * 64 * 128 * E, "q");
  if (fp8) rd(a.q_scales, T * 64 * 4, "q_scales");
  rd(a.w, T * 64 * 4, "w");
  rd(a.k, (size_t)a.num_pages * 64 * 128 * E, "k");
  if (fp8) rd(a.k_scales, (size_t)a.num_pages * 64 * 4, "k_scales");
  wr(a.idx_out, T * a.top_k * 4, "idx_out");
  wr(a.counters, (size_t)(sli::kMaxSeqs + 1) * sli::kCounterStride * 4, "counters");
  wr(a.refs, T * ncm * 2 * 8, "refs");
  wr(a.cnts, T * ncm * 8, "cnts");
  wr(a.cand, T * ncm * chunk * 8, "cand");
  g_stub.spin_max = a.spin_max;
  g_stub.xcd_local = a.xcd_local;
}

void sfa(const sli::SfaArgs& a, bool fp8) {
  if (a.n_splits < 1 || (long long)a.n_splits * a.split_len < a.top_k) die("splits do not cover top_k");
  if (a.split_len > sli::kMaxSplitRows && a.n_splits > 1) die("split_len");
  if (a.T % a.n_q) die("T");
  const size_t T = (size_t)a.T, H = (size_t)a.H;
  const size_t row = a.rope_bf16 ? 640 : fp8 ? 576 : 1152;
  seqs(a.seq_lens, a.block_table, a.T / a.n_q, a.max_pages);
  rd(a.q, T * H * 576 * 2, "q");
  rd(a.kv, (size_t)a.num_pages * 64 * row, "kv");
  if (fp8) rd(a.kv_scales, (size_t)a.num_pages * 64 * a.kv_groups * 4, "kv_scales");
  rd(a.idx, T * a.top_k * 4, "idx");
  wr(a.out, T * H * 512 * 2, "out");
  if (a.lse) wr(a.lse, T * H * 4, "lse");
  if (a.n_splits > 1) {
    wr(a.part_o, T * a.n_splits * H * 512 * 2, "part_o");
    wr(a.part_ml, T * a.n_splits * H * 2 * 4, "part_ml");
  }
}

}  // namespace

namespace sli {

hipError_t launch_idx_decode(const IdxDecodeArgs& a, int chunk, bool fp8, hipStream_t) {
  g_stub.calls += "idx_decode ";
  idx_decode(a, chunk, fp8);
  return hipSuccess;
}

hipError_t launch_idx_prefill(const IdxPrefillArgs& a, hipStream_t) {
  g_stub.calls += "idx_prefill ";
  const size_t T = (size_t)a.B * a.n_q;
  seqs(a.seq_lens, a.block_table, a.B, a.max_pages);
  rd(a.q, T * 64 * 128 * 2, "q");
  rd(a.w, T * 64 * 4, "w");
  rd(a.k, (size_t)a.num_pages * 64 * 128 * 2, "k");
  wr(a.idx_out, T * a.top_k * 4, "idx_out");
  return hipSuccess;
}

hipError_t launch_sfa(const SfaArgs& a, bool fp8, hipStream_t) {
  g_stub.calls += "sfa ";
  sfa(a, fp8);
  return hipSuccess;
}

hipError_t launch_decode_step(const StepArgs& s, hipStream_t) {
  g_stub.calls += "step ";
  if (s.idx.n_q != 1 || s.att.T != s.idx.B || s.att.n_splits != s.idx.n_chunks_max) die("step shape");
  idx_decode(s.idx, 4096, false);
  // one partial slot per chunk, in use even when a request has one chunk
  const sli::SfaArgs& t = s.att;
  wr(t.part_o, (size_t)t.T * t.n_splits * t.H * 512 * 2, "part_o");
  wr(t.part_ml, (size_t)t.T * t.n_splits * t.H * 2 * 4, "part_ml");
  sfa(t, false);
  return hipSuccess;
}

hipError_t launch_validate_paged(const ValidateArgs& a, hipStream_t) {
  g_stub.calls += "validate ";
  seqs(a.seq_lens, a.block_table, a.B, a.max_pages);
  wr(a.bad_out, 4, "bad_out");
  return hipSuccess;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t) {
  g_stub.calls += "zero ";
  wr(p, bytes, "zero_fill");
  return hipSuccess;
}

hipError_t launch_mxfp8_quant(const QuantArgs& a, hipStream_t) {
  g_stub.calls += "quant ";
  rd(a.x, (size_t)a.n_rows * a.row_len * 2, "x");
  wr(a.codes, (size_t)a.n_rows * a.row_len, "codes");
  wr(a.scales, (size_t)a.n_rows * (a.row_len / 32), "scales");
  return hipSuccess;
}

hipError_t launch_cache_append(const AppendArgs& a, hipStream_t) {
  g_stub.calls += "append ";
  const size_t T = (size_t)a.B * a.n_q, P = (size_t)a.num_pages * 64;
  seqs(a.seq_lens, a.block_table, a.B, a.max_pages);
  if (a.k_new) {
    rd(a.k_new, T * 128 * 2, "k_new");
    wr(a.k_cache, P * 128 * (a.k_fp8 ? 1 : 2), "k_cache");
    if (a.k_fp8) wr(a.k_scales, P * 4, "k_scales");
  }
  if (a.kv_new) {
    rd(a.kv_new, T * 576 * 2, "kv_new");
    wr(a.kv_cache, P * (a.kv_rope_bf16 ? 640 : a.kv_fp8 ? 576 : 1152), "kv_cache");
    if (a.kv_fp8) wr(a.kv_scales, P * a.kv_groups * 4, "kv_scales");
  }
  return hipSuccess;
}

}  // namespace sli
