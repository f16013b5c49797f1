// li_score_topk without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops and harnesses
// that forbid hipMalloc).  The decode indexer's exchange workspace (arrival
// counters, per-chunk brackets and counts, band lists) lives in a file-scope
// device array instead; every other step is li_score_topk itself.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress and only
// that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "launch.h"
#include "sparse_li.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LI_NOALLOC_WORKSPACE_MAX;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device (null until set up)
std::mutex g_setup;

}  // namespace

extern "C" li_status li_score_topk_noalloc(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens,
                                           const int32_t* block_table, int32_t max_pages, int32_t num_pages,
                                           int32_t q_dtype, const void* q, const uint8_t* q_scales, const float* w,
                                           int32_t k_dtype, const void* k_cache, const void* k_scales,
                                           int32_t top_k, int32_t* idx_out, void* stream) {
  // the geometry must fit the array; invalid arguments are reported by li_score_topk
  const size_t need = li_score_topk_workspace_size(num_seqs, q_per_seq, max_pages, top_k);
  if (need == 0)
    return li_score_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q, q_scales, w,
                         k_dtype, k_cache, k_scales, top_k, idx_out, nullptr, 0, stream);
  if (need > kScratchBytes)
    return sli::report(LI_ERR_UNSUPPORTED,
                       "li_score_topk_noalloc: this geometry needs %zu bytes of exchange workspace, more than the "
                       "library array's %zu; use li_score_topk with a caller workspace",
                       need, kScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sli::report(LI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return sli::report(LI_ERR_UNSUPPORTED, "device id %d out of range", dev);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_setup);
    if (!g_scratch[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return sli::report(LI_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
      // The exchange counters must start at zero (every call leaves them so).
      // The whole array is cleared, by a kernel on the caller's stream, so
      // that no word of an earlier use can carry a later call's tag even if
      // this first call is captured and replayed.
      e = sli::launch_zero_fill(p, kScratchBytes, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return sli::report(LI_ERR_HIP, "workspace clear: %s", hipGetErrorString(e));
      g_scratch[dev] = p;
    }
    ws = g_scratch[dev];
  }
  return li_score_topk(num_seqs, q_per_seq, seq_lens, block_table, max_pages, num_pages, q_dtype, q, q_scales, w,
                       k_dtype, k_cache, k_scales, top_k, idx_out, ws, kScratchBytes, stream);
}
