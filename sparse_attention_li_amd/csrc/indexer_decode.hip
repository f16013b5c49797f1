// Decode launches of the fused lightning-indexer score + Top-K (the kernel
// body, its decomposition and its exact cross-chunk selection are described in
// indexer_decode_body.h), and the workspace fill kernel.
#include "indexer_decode_body.h"

namespace sli {

template <int NQ, int NW, int CHUNK, bool FP8, int RS>
__global__ __launch_bounds__(NW * 64) void li_decode_kernel(const IdxDecodeArgs a) {
  __shared__ IdxSmem<NQ, NW, CHUNK, FP8, RS> sm;
  __shared__ __attribute__((aligned(16))) unsigned char arena[IdxSmem<NQ, NW, CHUNK, FP8, RS>::kArena];
  __shared__ uint32_t keys[NQ * CHUNK];
  __shared__ int pages[CHUNK / 64];
  uint32_t* grid_line = a.counters + (size_t)kMaxSeqs * kCounterStride;
  const uint32_t tag = __builtin_amdgcn_readfirstlane(xload(&grid_line[kGridEpoch]) + 1u);
  int b;
  (void)li_decode_body<NQ, NW, CHUNK, FP8, RS>(a, IdxLds<NQ, NW, CHUNK, FP8, RS>{sm, arena, keys, pages}, tag, b);
  // every workgroup (those without work included) departs once; the last
  // resets the count and advances the epoch for the next call
  if (threadIdx.x == 0) {
    const uint32_t total = gridDim.x;
    const uint32_t d = __hip_atomic_fetch_add(&grid_line[kGridDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == total - 1) {
      __hip_atomic_store(&grid_line[kGridDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&grid_line[kGridEpoch], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int NQ, int NW, int CHUNK, bool FP8, int RS = 2>
static hipError_t launch_one(const IdxDecodeArgs& a, hipStream_t stream) {
  const long long blocks = a.xcd_local ? (long long)((a.B + 7) / 8) * 8 * a.n_chunks_max : (long long)a.B * a.n_chunks_max;
  dim3 grid((unsigned)blocks);
  hipLaunchKernelGGL((li_decode_kernel<NQ, NW, CHUNK, FP8, RS>), grid, dim3(NW * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_idx_decode(const IdxDecodeArgs& a, int chunk, bool fp8, hipStream_t stream) {
  if (chunk == 256) {
    if (a.n_q == 1) return fp8 ? launch_one<1, 4, 256, true>(a, stream) : launch_one<1, 4, 256, false>(a, stream);
    if (a.n_q == 2) return fp8 ? launch_one<2, 4, 256, true>(a, stream) : launch_one<2, 4, 256, false>(a, stream);
  } else if (chunk == 1024) {
    if (a.n_q == 1) return fp8 ? launch_one<1, 4, 1024, true>(a, stream) : launch_one<1, 4, 1024, false>(a, stream);
    if (a.n_q == 2) return fp8 ? launch_one<2, 4, 1024, true>(a, stream) : launch_one<2, 4, 1024, false>(a, stream);
  } else if (chunk == 2048) {
    if (a.n_q == 1) return fp8 ? launch_one<1, 4, 2048, true>(a, stream) : launch_one<1, 4, 2048, false>(a, stream);
    if (a.n_q == 2) return fp8 ? launch_one<2, 4, 2048, true>(a, stream) : launch_one<2, 4, 2048, false>(a, stream);
  } else if (chunk == 8192) {
    if (fp8 && a.n_q == 1) return launch_one<1, 4, 8192, true>(a, stream);
  } else if (chunk == 4096) {
    // FP8 grids of several rounds: four-wave workgroups (56 / 72 KiB of LDS), two per CU, so one
    // streams while the other selects (eight-wave ones fill a CU alone)
    if (fp8 && a.xcd_local)
      return a.n_q == 1 ? launch_one<1, 4, 4096, true>(a, stream) : launch_one<2, 4, 4096, true>(a, stream);
    if (a.n_q == 1) return fp8 ? launch_one<1, 8, 4096, true>(a, stream) : launch_one<1, 8, 4096, false>(a, stream);
    if (a.n_q == 2 && fp8) return launch_one<2, 8, 4096, true>(a, stream);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- workspace fill
__global__ void zero_fill_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t nb = (words + 255) / 256;
  unsigned blocks = (unsigned)(nb < 4096 ? nb : 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace sli
