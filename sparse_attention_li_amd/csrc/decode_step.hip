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
//      the request's workgroups combine the partials into the output and lse,
//      in items of 16 heads dealt by arrival order at the count.
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
constexpr int kStepHeads = 128;      // query heads of the step: 8 merge items, 8 "gave up" bits
static_assert(kStepHeads / kStepMergeHeads <= 16, "one gave-up bit per item owner in the upper half-word");

// Per-request word of the step (in the request's counter line; words 0..2
// belong to the indexer's exchanges): the count of published partials in the
// low 16 bits, and from bit 16 one "gave up" bit per arrival order that owns
// merge items.  The launch's last workgroup to depart zeroes it.
enum : uint32_t { kStAttn = 4 };

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

// Thread 0 adds 1 to the count of the word at p (device scope) once
// everything the workgroup wrote is complete in memory; every thread receives
// the word as it was before.
__device__ __forceinline__ uint32_t count_in(uint32_t* p, uint32_t* bc) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) bc[0] = __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t r = bc[0];
  __syncthreads();
  return r;
}

// Thread 0 polls the count of the word at p until it reaches `target`
// (bounded); on time-out it sets the "gave up" bit `bit` and learns from the
// same atomic whether the count completed meanwhile.  Every thread receives
// whether the count is complete (the partials are all in memory).
__device__ __forceinline__ bool wait_count(uint32_t* p, uint32_t target, uint32_t bit, int spin_max, uint32_t* bc) {
  if (threadIdx.x == 0) {
    bool done = false;
    for (int spins = 0;; ++spins) {
      if ((xload(p) & 0xffffu) >= target) {
        done = true;
        break;
      }
      if (spins >= spin_max) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (!done) {
      const uint32_t w = __hip_atomic_fetch_or(p, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      done = (w & 0xffffu) >= target;  // the last arrived before the bit: it did not see it
    }
    bc[0] = done ? 1u : 0u;
  }
  __syncthreads();
  const bool r = bc[0] != 0u;
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
  // The attention's q^T operands are loaded during the indexer's exact
  // selection (LDS work only), so they are in registers when it ends.
  int b = 0, n_own = 0, n_chunks_b = 1;
  bf16x8 qpre[36];
  auto preload = [&](int bq) { sfa_load_q(s.att, bq, qpre); };
  const int st = li_decode_body<1, kStepWaves, kStepChunk, false, kStepRing, true>(
      a, IdxLds<1, kStepWaves, kStepChunk, false, kStepRing>{Z.idx.sm, X, reinterpret_cast<uint32_t*>(X + StepIdxSmem::kArena),
                                                           Z.idx.pages},
      tag, b, Z.att.rows, &n_own, &n_chunks_b, preload);
  __syncthreads();  // the indexer's LDS state is dead from here on; the rows are in place

  if (st == kBodyShare || st == kBodyAll) {
    uint32_t* rl = a.counters + (size_t)b * kCounterStride;
    // (the count comes from the indexer: a reload of the length here would
    // make every wave wait for all its stores in flight)
    const uint32_t n_chunks = (uint32_t)n_chunks_b;
    const uint32_t ncm = (uint32_t)a.n_chunks_max;
    // the chunk of this workgroup, in the indexer's block layout
    const int c = a.xcd_local ? (int)((blockIdx.x >> 3) % ncm)
                              : (int)((blockIdx.x % ncm + ncm - (uint32_t)b % ncm) % ncm);
    // 2. attention over the rows this workgroup wrote
    const bool direct = st == kBodyAll || n_chunks == 1;
    const SfaBf16Lds lds{reinterpret_cast<char*>(X), reinterpret_cast<char*>(X + kTileBytes),
                         reinterpret_cast<char*>(X + 2 * kTileBytes), reinterpret_cast<char*>(X + 3 * kTileBytes),
                         Z.att.pbuf, Z.att.rows};
    sfa_bf16_body<kStepWaves, kStepRows, true>(s.att, lds, b, c, n_own, direct, qpre);
    // 3. merge, once every chunk's partial is out.  The workgroup of arrival
    // order o at the count merges items o, o + n_chunks, ...  One that gives
    // up waiting sets its bit: the last to arrive then merges its items too,
    // unless the count completed before the bit was set, when it merges them
    // itself (exactly one of the two sees the other).  When the count never
    // completes (an exchange fell back and one workgroup wrote the whole
    // request, attending over all of it), every waiter gives up.
    if (!direct) {
      const uint32_t n_items = (uint32_t)((s.att.H + kStepMergeHeads - 1) / kStepMergeHeads);
      const uint32_t old = count_in(&rl[kStAttn], bc);
      const uint32_t o = old & 0xffffu;
      const bool last = o + 1u == n_chunks;
      auto merge_items = [&](uint32_t owner) {
        for (uint32_t m = owner; m < n_items; m += n_chunks) {
          // 16 threads per head, 32 columns each: every load of a split group in flight at once
          const int h = (int)m * kStepMergeHeads + (int)(threadIdx.x >> 4);
          if (h < s.att.H) sfa_merge_head<true, 4>(s.att, b, h, threadIdx.x & 15, (int)n_chunks);
        }
      };
      if (last) {
        merge_items(o);
        for (uint32_t g = 0; g < o && g < n_items; ++g)
          if ((old >> (16 + g)) & 1u) merge_items(g);
      } else if (o < n_items && wait_count(&rl[kStAttn], n_chunks, 1u << (16 + o), a.spin_max, bc)) {
        merge_items(o);
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
    for (int r = threadIdx.x; r < a.B; r += blockDim.x)
      __hip_atomic_store(&a.counters[(size_t)r * kCounterStride + kStAttn], 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
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
