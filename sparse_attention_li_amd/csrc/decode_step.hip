// The whole decode step in one launch: lightning-indexer score + Top-K, then
// sparse MLA attention over the selected rows, then the merge of the partial
// results, for bf16 caches, one query token per request and 128 heads.
//
// The pages take every step other than attention off the decode critical
// path by fusing the indexer into one operator and dispatching the layer's
// operators as one ("Day-0 Inference Adaptation and Optimization for Hybrid
// Attention Architectures", sec. 3; "Day0 Inference Adaptation and
// Performance Optimization for a Sparse Hybrid Architecture LLM", sec. 6).
// Here one workgroup per (request, 4096-position chunk) runs, in turn:
//   1. the decode indexer's chunk work (li_decode_body: score its chunk,
//      exchange brackets with the request's other chunks, write its share of
//      the request's index row, through to memory), recording the pool rows
//      of the positions it selected;
//   2. attention over exactly those rows -- the positions of the request's
//      selection that lie in its chunk, so no workgroup waits for another's
//      index writes -- giving a partial (max, sum, normalised output) per head;
//   3. once every chunk of the request has published its partial (a count),
//      merge items of 16 heads, taken from a counter by the request's
//      workgroups, combine the partials into the output and lse.
// A request of one chunk writes its output in step 2.  When the indexer's
// exchanges fell back (a workgroup gave up and the last one to arrive wrote
// the whole request), that last workgroup attends over the whole selection
// and writes the output itself; the partial count then never completes and
// the others' bounded waits end.  No wait depends on a workgroup that might
// not be running, and every wait is bounded.
#include "indexer_decode_body.h"
#include "sfa_bf16_body.h"

namespace sli {

constexpr int kStepWaves = 4;
constexpr int kStepChunk = 4096;
constexpr int kStepRing = 4;      // key tiles in flight per wave
constexpr int kStepRows = 2048;   // pool rows one workgroup attends, at most (top_k)
constexpr int kStepMergeHeads = 16;  // heads per merge item: 16 threads per head
static_assert(kStepMergeHeads * 16 == kStepWaves * 64, "one merge item per workgroup pass");

// Per-request words of the step (the request's counter line; words 0..2
// belong to the indexer's exchanges).  The launch's last workgroup to depart
// zeroes them.
enum : uint32_t { kStAttnDone = 4, kStMerge = 5 };

typedef IdxSmem<1, kStepWaves, kStepChunk, false, kStepRing> StepIdxSmem;

// LDS.  X: the indexer's key ring and keys, then the attention's four tile
// slots (all direct-to-LDS targets), and the step's broadcast words between
// the phases.  Z: the indexer's small state, then the attention's weights
// buffer and rows; the rows are written at the end of the indexer phase, so
// they lie past the indexer's state.
constexpr int kStepX = 4 * kTileBytes;
static_assert(StepIdxSmem::kArena + 4 * kStepChunk <= kStepX, "key ring and keys fit the tile slots");
struct StepIdxState {
  StepIdxSmem sm;
  int pages[kStepChunk / 64];
};
constexpr int kStepPbuf = kStepWaves * 2 * 64 * 16;
static_assert(sizeof(StepIdxState) <= kStepPbuf, "the rows lie past the indexer state");
struct StepSmall {
  union {
    StepIdxState idx;
    struct {
      char pbuf[kStepPbuf];
      int rows[kStepRows];
    } att;
  };
};
static_assert(kStepX + sizeof(StepSmall) <= 160 * 1024, "LDS of one CU");

// Polls the counter at p until it reaches `target` (bounded).
__device__ __forceinline__ bool poll_at_least(const uint32_t* p, uint32_t target, int spin_max) {
  for (int spins = 0;; ++spins) {
    if (xload(p) >= target) return true;
    if (spins >= spin_max) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Thread 0 adds 1 to the counter at p (device scope) once everything the
// workgroup wrote is complete in memory; every thread receives whether the
// count reached `target` with it.
__device__ __forceinline__ bool count_and_check(uint32_t* p, uint32_t target, uint32_t* bc) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bc[0] = old + 1u >= target ? 1u : 0u;
  }
  __syncthreads();
  const bool r = bc[0] != 0u;
  __syncthreads();
  return r;
}

// Thread 0 polls; every thread receives the outcome.
__device__ __forceinline__ bool wait_at_least(const uint32_t* p, uint32_t target, int spin_max, uint32_t* bc) {
  if (threadIdx.x == 0) bc[0] = poll_at_least(p, target, spin_max) ? 1u : 0u;
  __syncthreads();
  const bool r = bc[0] != 0u;
  __syncthreads();
  return r;
}

// Thread 0 takes the next item of the counter at p; every thread receives it.
__device__ __forceinline__ uint32_t take_item(uint32_t* p, uint32_t* bc) {
  if (threadIdx.x == 0) bc[0] = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t r = bc[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kStepWaves * 64) void li_step_kernel(const StepArgs s) {
  __shared__ __attribute__((aligned(128))) unsigned char X[kStepX];
  __shared__ __attribute__((aligned(128))) StepSmall Z;
  const IdxDecodeArgs& a = s.idx;
  uint32_t* grid_line = a.counters + (size_t)kMaxSeqs * kCounterStride;
  const uint32_t tag = __builtin_amdgcn_readfirstlane(xload(&grid_line[kGridEpoch]) + 1u);
  uint32_t* const bc = reinterpret_cast<uint32_t*>(X);  // used between the phases only

  // 1. the indexer's chunk work; the rows of what this workgroup wrote
  int b = 0, n_own = 0;
  const int st = li_decode_body<1, kStepWaves, kStepChunk, false, kStepRing, true>(
      a, IdxLds<1, kStepWaves, kStepChunk, false, kStepRing>{Z.idx.sm, X, reinterpret_cast<uint32_t*>(X + StepIdxSmem::kArena),
                                                           Z.idx.pages},
      tag, b, Z.att.rows, &n_own);
  __syncthreads();  // the indexer's LDS state is dead from here on; the rows are in place

  if (st == kBodyShare || st == kBodyAll) {
    uint32_t* rl = a.counters + (size_t)b * kCounterStride;
    const int L = max(0, min(a.seq_lens[b], a.max_pages * 64));
    const uint32_t n_chunks = (uint32_t)max(1, (L + kStepChunk - 1) / kStepChunk);
    const uint32_t ncm = (uint32_t)a.n_chunks_max;
    // the chunk of this workgroup, in the indexer's block layout
    const int c = a.xcd_local ? (int)((blockIdx.x >> 3) % ncm)
                              : (int)((blockIdx.x % ncm + ncm - (uint32_t)b % ncm) % ncm);
    // 2. attention over the rows this workgroup wrote
    const bool direct = st == kBodyAll || n_chunks == 1;
    const SfaBf16Lds lds{reinterpret_cast<char*>(X), reinterpret_cast<char*>(X + kTileBytes),
                         reinterpret_cast<char*>(X + 2 * kTileBytes), reinterpret_cast<char*>(X + 3 * kTileBytes),
                         Z.att.pbuf, Z.att.rows};
    sfa_bf16_body<kStepWaves, kStepRows, true>(s.att, lds, b, c, n_own, direct);
    // 3. merge, once every chunk's partial is out
    if (!direct) {
      const bool last = count_and_check(&rl[kStAttnDone], n_chunks, bc);
      bool merge = last || wait_at_least(&rl[kStAttnDone], n_chunks, a.spin_max, bc);
      const uint32_t n_items = (uint32_t)((s.att.H + kStepMergeHeads - 1) / kStepMergeHeads);
      while (merge) {
        const uint32_t m = take_item(&rl[kStMerge], bc);
        if (m >= n_items) break;
        // 16 threads per head, 32 columns each: every load of a split group in flight at once
        const int h = (int)m * kStepMergeHeads + (int)(threadIdx.x >> 4);
        if (h < s.att.H) sfa_merge_head<true, 4>(s.att, b, h, threadIdx.x & 15, (int)n_chunks);
      }
    }
  }

  // every workgroup departs once; the last zeroes the step words of every
  // request, resets the count and advances the epoch for the next call
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t d = __hip_atomic_fetch_add(&grid_line[kGridDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bc[1] = d == gridDim.x - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (bc[1]) {
    for (int r = threadIdx.x; r < a.B; r += blockDim.x) {
      uint32_t* rl = a.counters + (size_t)r * kCounterStride;
      __hip_atomic_store(&rl[kStAttnDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&rl[kStMerge], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
      __hip_atomic_store(&grid_line[kGridDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&grid_line[kGridEpoch], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_decode_step(const StepArgs& s, hipStream_t stream) {
  const long long blocks = s.idx.xcd_local ? (long long)((s.idx.B + 7) / 8) * 8 * s.idx.n_chunks_max
                                           : (long long)s.idx.B * s.idx.n_chunks_max;
  hipLaunchKernelGGL(li_step_kernel, dim3((unsigned)blocks), dim3(kStepWaves * 64), 0, stream, s);
  return hipGetLastError();
}

}  // namespace sli
