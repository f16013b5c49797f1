// Fused lightning-indexer score + Top-K for decode (1 or 2 query tokens per
// request), gfx950.
//
// What it computes (pages: "Optimizing Inference for Hybrid Attention LLMs",
// sec. 3.1; "Day0 Inference Support and Performance Optimization for
// New-Architecture LLMs", sec. 4): for each query token t of request b and
// every visible cached position s,
//     I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:])        (64 heads x 128)
// and the min(K, visible) positions with the largest I (ties to the lower
// position).  Only the indices leave the chip.
//
// Decomposition.  One workgroup (4 waves) owns a chunk of CHUNK consecutive
// positions of one request and all of the request's query tokens, so the key
// pages are streamed from HBM exactly once.  Per 32-position tile a wave runs
//     S[head, pos] = q[head, :] . k[pos, :]   on 32x32 MFMA tiles (heads = M),
// so each lane ends up holding 16 heads of one position and the head
// reduction sum_h w*ReLU(S) is 16 in-lane FMAs plus one cross-half swap.
// Scores become order-preserving uint32 keys in LDS; they never reach HBM.
//
// Exact selection across the n chunks of a request, every workgroup writing
// its own chunk's share of the output (kappa = the K-th largest key):
//   1. chunk c takes a quota R_c with K <= sum R_c < K + n and finds, from
//      one LDS histogram of its keys, a key interval [lo_c, hi_c) holding
//      its R_c-th largest key: >= R_c of its keys are >= lo_c and < R_c are
//      >= hi_c.  Hence lo = min lo_c and hi = max hi_c bracket kappa:
//      >= sum R_c >= K keys are >= lo, and <= sum (R_c - 1) < K keys are
//      >= hi.  The quotas follow the chunks' visible positions, so every
//      bracket sits near the same quantile and the band stays narrow: whole
//      chunks split K evenly; when the last chunk holds only v < CHUNK of the
//      vis visible positions it takes floor(K v / vis) (possibly 0: then its
//      interval is empty below and ends above its largest key) and the others
//      ceil((K - that) / (n - 1)).  Chunks past the visible ones publish an
//      empty interval.  Exchange 1 publishes the intervals;
//   2. keys >= hi are selected for certain; each chunk publishes its count of
//      them and its "band" keys in [lo, hi) with their positions (exchange 2);
//   3. every workgroup loads all band keys of the request (a few per cent of
//      the positions), selects kappa among them exactly (radix select,
//      need = K - #keys >= hi), counts what the chunks before it select, and
//      writes its own selected positions at that offset, in position order.
//      In one-token grids of several rounds only the last chunk to publish
//      does this, for the whole request (merging the two sorted position
//      lists: keys >= hi and the selected band); the others leave after
//      publishing, and their CUs take the next round's chunks.
// The exchanges are arrival counters with bounded waits.  A workgroup whose
// first wait times out (its request's chunks were not all resident) publishes
// every key as band, which keeps the result exact; one whose second wait
// times out leaves its share to the last workgroup to arrive, which then
// writes the whole request from the published lists.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace sli {

constexpr int kHistBins = 4096;  // LDS histogram that brackets a chunk's R-th largest key
constexpr int kBandCap = 3584;   // band entries the final select keeps in LDS (a multiple of 512)

// Words of the fixed counter region (one 128-byte line per request, then one
// line for the whole launch).  Exchange data carries a per-call tag (the
// launch epoch + 1) in its upper 32 bits, so a reader polls the data itself:
// no counter, no fence on the common path.  The epoch is one for the whole
// workspace, so no word left by an earlier call -- for any request and any
// batch shape -- carries the current tag.  The per-request counters only
// settle the rare give-up fallback; the launch line counts departing
// workgroups, and the last one advances the epoch.
enum : uint32_t { kArrive2 = 0, kDone = 1, kState = 2 };
enum : uint32_t { kGridDone = 0, kGridEpoch = 1 };
enum : uint32_t { kStLast = 1u, kStGaveUp = 2u };
enum : uint32_t { kModeNormal = 0u, kModeFull = 1u, kModeQuit = 2u };

// LDS: a per-wave ring of two key tiles filled by direct-to-LDS loads during
// scoring; after scoring the same bytes hold the histogram and then the band
// entries of the request.
template <int NQ, int NW, int CHUNK, bool FP8, int RS>
struct IdxSmem {
  static constexpr int kTileBytes = FP8 ? 32 * 128 : 32 * 256;
  static constexpr int kSlotBytes = kTileBytes + (FP8 ? 128 : 0);  // FP8: the tile's 32 row scales follow it
  static constexpr int kRing = NW * RS * kSlotBytes;
  // after scoring: the band entries, then the per-chunk offsets and the
  // whole-request writer's bitmap (kSel bytes), or the histogram
  static constexpr int kSel = kBandCap * 8 + (3 * kMaxChunksPerSeq + 2) * 4 + CHUNK / 8;
  static constexpr int kReuse = kSel > kHistBins * 4 ? kSel : kHistBins * 4;
  static constexpr int kArena = kRing > kReuse ? kRing : kReuse;
  alignas(16) float w[NQ][64];
  uint32_t hist[256];                    // radix-select digits
  uint32_t mm[NQ][NW][2];                // per-wave min / max valid key
  uint32_t ref[NQ][2];                   // [lo, hi) of this chunk
  uint32_t sel[4];
  uint32_t scan[3 * NW];
  uint32_t flag[4];
  uint32_t next_tile;
};

// The LDS object the key DMA writes (the ring) and the ones the streaming
// loop reads or writes besides it (page ids, keys) are separate variables: the compiler's wait insertion then sees that those reads cannot
// alias a tile still in flight and does not drain the loads before them.
template <int NQ, int NW, int CHUNK, bool FP8, int RS>
struct IdxLds {
  IdxSmem<NQ, NW, CHUNK, FP8, RS>& sm;
  unsigned char* arena;  // [kArena]: key ring; after scoring the histogram, then the band entries
  uint32_t* keys;        // [NQ][CHUNK]
  int* pages;            // [CHUNK / 64]
};

template <bool FP8>
struct QOps;
template <>
struct QOps<false> {
  bf16x8 v[8];
};
template <>
struct QOps<true> {
  i32x8 v[2];
  int scale[2];
};

__device__ __forceinline__ uint64_t tagged(uint32_t v, uint32_t tag) { return (uint64_t)v | ((uint64_t)tag << 32); }

// Polls `n` tagged words until each carries `tag` (at most spin_max rounds
// of sleeping).  Returns false on time-out.
__device__ __forceinline__ bool poll_tagged(const uint64_t* p, int n, uint32_t tag, int spin_max, uint32_t* vals) {
  int spins = 0;
  for (;;) {
    bool all = true;
    for (int i = 0; i < n; ++i) {
      const uint64_t v = xload64(&p[i]);
      vals[i] = (uint32_t)v;
      all &= (uint32_t)(v >> 32) == tag;
    }
    if (all) return true;
    if (++spins > spin_max) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// What a workgroup of li_decode_body wrote of its request's index rows.
enum : int { kBodyNone = 0, kBodyShare = 1, kBodyAll = 2, kBodyQuit = 3 };

// The hook li_decode_body calls, with the request, once its chunk's keys are
// scored: callers that load nothing beside the selection pass this one.
struct NoPreload {
  __device__ void operator()(int) const {}
};

// FUSED (the single-launch decode step): the key array lives in the same LDS
// object as the key ring, so its stores are written as LDS instructions of
// their own (a compiler store there would wait for every tile in flight).
// Nothing in the launch reads the index rows (the attention takes the pool
// rows from LDS), so they are ordinary stores, whose completion a later
// memory wait does not have to await from HBM.  Returns kBodyNone (no chunk of a request), kBodyShare
// (wrote this chunk's share of the rows), kBodyAll (wrote the whole request)
// or kBodyQuit (left its share to the last workgroup); b_out = the request.
// FUSED also records, in rows_out, the physical pool row of every position
// the workgroup writes (its own selected positions, or the whole request's
// when it writes the whole request), in output order, and their number in
// n_own (every thread; at most top_k), and the request's chunk count in
// n_chunks_out (unless kBodyNone for padding past the last request).
// `preload` is called once per workgroup that goes on to write index rows,
// where the selection has no global reads left (once the band is in LDS):
// loads it issues complete under the exact selection.
template <int NQ, int NW, int CHUNK, bool FP8, int RS, bool FUSED = false, typename Pre = NoPreload>
__device__ __forceinline__ int li_decode_body(const IdxDecodeArgs& a, IdxLds<NQ, NW, CHUNK, FP8, RS> lds,
                                              const uint32_t tag, int& b_out, int* rows_out = nullptr,
                                              int* n_own = nullptr, int* n_chunks_out = nullptr,
                                              const Pre& preload = Pre{}) {
  static_assert(!FUSED || NQ == 1, "the fused step takes one query token per request");
  IdxSmem<NQ, NW, CHUNK, FP8, RS>& sm = lds.sm;
  uint32_t* s_keys = lds.keys;  // [NQ][CHUNK]

  constexpr int THREADS = NW * 64;
  constexpr int NT = CHUNK / 32;  // 32-position tiles per chunk
  static_assert(NT >= RS * NW, "each wave starts with RS tiles");
  constexpr int PER = CHUNK / THREADS;  // keys per thread (contiguous positions)
  static_assert(PER * THREADS == CHUNK && 32 % PER == 0, "chunk splits into whole bit groups per thread");
  static_assert(kMaxChunksPerSeq <= THREADS, "one thread per chunk of a request");

  // Block -> (request b, chunk c).  The hardware deals blocks to the 8 XCDs
  // in turn (block id mod 8) and each XCD starts its blocks in id order; the
  // chunks of a request must be resident together for the exchanges.
  //  - spread (grids of one round): request b owns blocks b*ncm .. b*ncm+ncm-1
  //    and chunk c runs as block b*ncm + (c + b) mod ncm, so chunk 0 of
  //    successive requests rotates over the XCDs;
  //  - XCD-local (grids of several rounds): request b's chunks all run on XCD
  //    b mod 8, as blocks 8 ((b / 8) ncm + c) + b mod 8, so a request waits
  //    only for its own XCD's earlier requests, not for the slowest XCD.
  const uint32_t ncm_u = (uint32_t)a.n_chunks_max, bid = blockIdx.x;
  int b, c;
  if (a.xcd_local) {
    const uint32_t r = bid >> 3;
    b = (int)((r / ncm_u) * 8u + (bid & 7u));
    c = (int)(r % ncm_u);
  } else {
    b = (int)(bid / ncm_u);
    c = (int)((bid % ncm_u + ncm_u - (uint32_t)b % ncm_u) % ncm_u);
  }
  b_out = b;
  if (b >= a.B) return kBodyNone;  // padding of the XCD-local grid (departs in the caller)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 31, half = lane >> 5;
  const int t0 = b * NQ;
  const int s0 = c * CHUNK;
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- prologue (one memory latency)
  // Page ids (loaded in bounds of the block table whatever the request's
  // length), the length, q, w and the exchange epoch are all requested at
  // once; the key tiles follow as soon as the page ids are in LDS.
  int pg = 0;
  if (tid < CHUNK / 64 && s0 / 64 + tid < a.max_pages) pg = bt[s0 / 64 + tid];
  int L = a.seq_lens[b];
  const float wv = tid < NQ * 64 ? a.w[(size_t)t0 * 64 + tid] : 0.f;
  QOps<FP8> qa[NQ * 2];  // A operands: the token's 64 heads as two 32-row tiles
#pragma unroll
  for (int mt = 0; mt < NQ * 2; ++mt) {
    const size_t row = (size_t)(t0 + mt / 2) * 64 + 32 * (mt & 1) + n;  // (token, head)
    if constexpr (!FP8) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + row * 128 + 64 * half);
#pragma unroll
      for (int j = 0; j < 8; ++j) qa[mt].v[j] = qp[j];
    } else {
      // The block-scaled 32x32x64 MFMA splits its k range into two blocks of
      // 32: block 0 is bytes 0..15 of both lane halves, block 1 bytes 16..31,
      // and block b takes its E8M0 scale from the lanes of half b.  So in
      // k-step j, bytes 0..15 of this lane carry d = 64j + 16 half + 0..15
      // (MX group 2j) and bytes 16..31 carry d = 64j + 32 + 16 half + 0..15
      // (MX group 2j+1); this lane supplies the scale of group 2j + half.
      const uint8_t* qp = static_cast<const uint8_t*>(a.q) + row * 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(qp + 64 * j + 16 * half);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(qp + 64 * j + 32 + 16 * half);
        qa[mt].v[j] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        qa[mt].scale[j] = a.q_scales[row * 4 + 2 * j + half];
      }
    }
  }
  uint32_t* ctr = a.counters + (size_t)b * kCounterStride;
  L = max(0, min(L, a.max_pages * 64));
  const int n_chunks = max(1, (L + CHUNK - 1) / CHUNK);
  if constexpr (FUSED) *n_chunks_out = n_chunks;
  if (c >= n_chunks) return kBodyNone;
  if (tid < CHUNK / 64) lds.pages[tid] = (s0 + 64 * tid < L) ? min(max(pg, 0), a.num_pages - 1) : 0;
  if (tid < NQ * 64) sm.w[tid / 64][tid % 64] = wv;
  const int n_valid = min(CHUNK, L - s0);     // positions of this chunk in the cache (>= 1)
  const int nt_used = (n_valid + 31) / 32;    // tiles that hold any of them
  if (tid == 0) sm.next_tile = RS * NW;
  // tiles nobody scores hold no visible position: their keys are 0
  for (int i = nt_used * 32 + tid; i < CHUNK; i += THREADS)
#pragma unroll
    for (int j = 0; j < NQ; ++j) s_keys[j * CHUNK + i] = 0u;
  // Every prologue load (q operands included) is complete before the first
  // tile is issued.  They were issued together with the page ids, which the
  // barrier waits for anyway; without this wait the compiler cannot prove the
  // q operands ready inside the streaming loop and drains every tile load in
  // flight before each tile's first MFMA.
  SLI_WAIT_VMCNT(0);
  __syncthreads();

  // ---------------------------------------------------------------- score
  // Tiles of 32 positions (inside one page) are dealt to the waves on demand
  // (an LDS counter), so the chunk's waves finish together.  Each wave moves
  // its tiles by direct-to-LDS loads into a private ring of RS slots; each DMA
  // instruction reads one contiguous kilobyte of the tile (eight lanes per
  // 128-byte line) and writes lane l's 16 bytes to slot 64i + l; inside a
  // line the 16-byte chunks are XOR-swizzled by (row & 7), so the MFMA
  // operand reads (row n, fixed column) hit distinct banks.  FP8 tiles bring
  // their 32 row scales along (one more direct-to-LDS load, 4 bytes a lane).
  constexpr int TB = IdxSmem<NQ, NW, CHUNK, FP8, RS>::kTileBytes;
  constexpr int SB = IdxSmem<NQ, NW, CHUNK, FP8, RS>::kSlotBytes;
  constexpr int DMA_PER_TILE = TB / 1024 + (FP8 ? 1 : 0);
  constexpr int ROW = FP8 ? 128 : 256;  // bytes per key row
  constexpr int RPI = 1024 / ROW;       // rows per DMA instruction
  unsigned char* ring = lds.arena + wid * RS * SB;
  // this lane's share of every DMA instruction: row (within the instruction)
  // and the 16-byte chunk of that row
  const int dma_row = lane / (64 / RPI);
  const int dma_line = FP8 ? 0 : (lane >> 3) & 1;
  auto issue = [&](int tile, int slot_i) {
    const int lp = tile * 32;  // position inside the chunk
    const size_t row0 = (size_t)lds.pages[lp >> 6] * 64 + (lp & 32);
    const char* base = static_cast<const char*>(a.k) + row0 * ROW;
    unsigned char* dst = ring + slot_i * SB;
#pragma unroll
    for (int i = 0; i < TB / 1024; ++i) {
      const int row = RPI * i + dma_row;
      const int col = 8 * dma_line + ((lane & 7) ^ (row & 7));
      __builtin_amdgcn_global_load_lds(base + row * ROW + 16 * col, (lds_void*)(dst + 1024 * i), 16, 0, 0);
    }
    if constexpr (FP8) {
      if (lane < 32)
        __builtin_amdgcn_global_load_lds(static_cast<const uint32_t*>(a.k_scales) + row0 + lane, (lds_void*)(dst + TB),
                                         4, 0, 0);
    }
  };
  // `issued` counts this wave's vector-memory instructions; mark[s] is the
  // count just after slot s's tile was issued.
  uint32_t issued = 0, mark[RS];
  auto issue_counted = [&](int tile, int slot_i) {
    issue(tile, slot_i);
    issued += DMA_PER_TILE;
    mark[slot_i] = issued;
  };
  // The tile counter is bumped by an LDS atomic written as the instruction
  // itself (with its own wait): as a compiler atomic it would make the wait
  // pass drain every direct-to-LDS load in flight first.
  const uint32_t next_addr = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)&sm.next_tile;
  auto grab = [&]() -> int {
    uint32_t t = 0;
    if (lane == 0)  // one lane: one tile
      asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(t) : "v"(next_addr), "v"(1u) : "memory");
    return (int)min(__builtin_amdgcn_readfirstlane(t), (uint32_t)nt_used);
  };
  // the first RS tiles of every wave (tq[s]: the tile in slot s, nt_used when
  // none); the one after them is dealt below
  int tq[RS];
#pragma unroll
  for (int s = 0; s < RS; ++s) {
    mark[s] = 0u;
    tq[s] = wid + NW * s < nt_used ? wid + NW * s : nt_used;
    if (tq[s] < nt_used) issue_counted(tq[s], s);
  }

  int vis[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) vis[j] = max(0, L - NQ + j + 1);
  uint32_t kmin[NQ], kmax[NQ];  // this lane's smallest / largest valid key
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    kmin[j] = 0xffffffffu;
    kmax[j] = 0u;
  }

  // LDS byte offset of (row, 16-byte chunk) inside a tile
  auto slot = [&](int row, int col) {
    return 1024 * (row / RPI) + 16 * ((64 / RPI) * (row % RPI) + 8 * (col >> 3) + ((col & 7) ^ (row & 7)));
  };

  // Scoring a tile is split in two: the MFMAs (operand reads of the slot
  // awaited inside, so the slot may be refilled right after), and the head
  // sums of their results.  acc receives S[head, pos] of the tile's 32
  // positions (two 32-head tiles per query token); ksw the FP8 row's scale
  // word: its f32 scale, or (MXFP8 keys) its four E8M0 codes, group g in byte g.
  auto scores = [&](int slot_i, f32x16 (&acc)[NQ * 2], uint32_t& ksw) {
    const unsigned char* src = ring + slot_i * SB;
#pragma unroll
    for (int mt = 0; mt < NQ * 2; ++mt) acc[mt] = (f32x16){};
    // The operand reads of the ring are LDS instructions of their own, each
    // k-step waiting for exactly its reads: the compiler cannot tell a read
    // of this slot from the direct-to-LDS loads in flight into the others and
    // would wait for all of them before a compiler-issued read.
    const uint32_t src_a = (uint32_t)(size_t)(const lds_void*)src;
    if constexpr (!FP8) {
      // k-step j: row n, bytes 128 half + 16 j = chunk 8 half + j
      bf16x8 kb[8];
#define SLI_KB_READ(J) asm volatile("ds_read_b128 %0, %1" : "=v"(kb[J]) : "v"(src_a + (uint32_t)slot(n, 8 * half + J)));
      SLI_KB_READ(0) SLI_KB_READ(1) SLI_KB_READ(2) SLI_KB_READ(3)
      SLI_KB_READ(4) SLI_KB_READ(5) SLI_KB_READ(6) SLI_KB_READ(7)
#undef SLI_KB_READ
#define SLI_KB_STEP(J)                                                                 \
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kb[J]) : "i"(7 - J));                  \
  for (int mt = 0; mt < NQ * 2; ++mt)                                                  \
    acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt].v[J], kb[J], acc[mt], 0, 0, 0);
      SLI_KB_STEP(0) SLI_KB_STEP(1) SLI_KB_STEP(2) SLI_KB_STEP(3)
      SLI_KB_STEP(4) SLI_KB_STEP(5) SLI_KB_STEP(6) SLI_KB_STEP(7)
#undef SLI_KB_STEP
      ksw = 0u;
    }
    if constexpr (FP8) {
      // k-step j: row n, bytes 64 j + 16 half (chunk 4j + half) and 64 j + 32 + 16 half
      i32x4 kr[4];
      asm volatile("ds_read_b32 %0, %1" : "=v"(ksw) : "v"(src_a + (uint32_t)(TB + 4 * n)));
      asm volatile("ds_read_b128 %0, %1" : "=v"(kr[0]) : "v"(src_a + (uint32_t)slot(n, half)));
      asm volatile("ds_read_b128 %0, %1" : "=v"(kr[1]) : "v"(src_a + (uint32_t)slot(n, 2 + half)));
      asm volatile("ds_read_b128 %0, %1" : "=v"(kr[2]) : "v"(src_a + (uint32_t)slot(n, 4 + half)));
      asm volatile("ds_read_b128 %0, %1" : "=v"(kr[3]) : "v"(src_a + (uint32_t)slot(n, 6 + half)));
      asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(ksw), "+v"(kr[0]), "+v"(kr[1]));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (j == 1) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kr[2]), "+v"(kr[3]));
        const i32x4 lo = kr[2 * j], hi = kr[2 * j + 1];
        const i32x8 kb = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        // this lane supplies the B scale of MX group 2j + half of row n (the
        // same lane-half rule as the query's A scales); 127 = 1 for row scales
        const int kbs = a.k_mx ? (int)((ksw >> (8 * (2 * j + half))) & 0xffu) : 127;
#pragma unroll
        for (int mt = 0; mt < NQ * 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt].v[j], kb, acc[mt], 0, 0, 0,
                                                                   qa[mt].scale[j], 0, kbs);
      }
    }
  };
  // Head weights of this lane's accumulator rows (rows 8g + 4 half + i of
  // head tile mh): held in registers by the single-launch step, whose
  // indexer phase has the registers of the attention phase to spare.
  float wreg[FUSED ? NQ : 1][FUSED ? 32 : 1];
  if constexpr (FUSED) {
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
      for (int mh = 0; mh < 2; ++mh)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) wreg[j][16 * mh + 4 * g + i] = sm.w[j][32 * mh + 8 * g + 4 * half + i];
  }
  // Weighted ReLU head sum of a tile's scores (four partial sums, added
  // pairwise), its key into LDS and the lane's key range.
  auto head_sums = [&](int tile, const f32x16 (&acc)[NQ * 2], uint32_t ksw) {
    const int pos0 = s0 + tile * 32;
    const float kscale = (FP8 && !a.k_mx) ? __uint_as_float(ksw) : 1.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // output rows 8g+4*half+0..3 of this 32-head tile: four consecutive heads
          f32x4 w4;
          if constexpr (FUSED) {
            w4 = (f32x4){wreg[j][16 * mh + 4 * g], wreg[j][16 * mh + 4 * g + 1], wreg[j][16 * mh + 4 * g + 2],
                         wreg[j][16 * mh + 4 * g + 3]};
          } else {
            w4 = *reinterpret_cast<const f32x4*>(&sm.w[j][32 * mh + 8 * g + 4 * half]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // bf16: four partial sums, as the single-launch step's scorer adds them
            if constexpr (FP8) p4[0] += w4[i] * fmaxf(acc[2 * j + mh][4 * g + i], 0.f);
            else p4[i] += w4[i] * fmaxf(acc[2 * j + mh][4 * g + i], 0.f);
          }
        }
      }
      float part = FP8 ? p4[0] : (p4[0] + p4[1]) + (p4[2] + p4[3]);
      part += __shfl_xor(part, 32, kWave);
      if constexpr (FP8) part *= kscale;  // positive per-row scale commutes with ReLU (1 for MXFP8 keys)
      if (half == 0) {
        const int s = pos0 + n;
        const uint32_t key = (s < vis[j]) ? score_key(part) : 0u;
        if constexpr (FUSED) {
          const uint32_t ka = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)&s_keys[j * CHUNK + tile * 32 + n];
          asm volatile("ds_write_b32 %0, %1" : : "v"(ka), "v"(key) : "memory");
        } else {
          s_keys[j * CHUNK + tile * 32 + n] = key;
        }
        if (key != 0u) {
          kmin[j] = min(kmin[j], key);
          kmax[j] = max(kmax[j], key);
        }
      }
    }
  };

  int pre = tq[RS - 1] < nt_used ? grab() : nt_used;
  // Slots are consumed in ring order; the tile dealt next refills the slot
  // just consumed.  Tiles are dealt in increasing order, so the first slot
  // found without a tile ends the loop.
  // The single-launch step (bf16, one query token, one wave per SIMD): the
  // MFMAs of one tile with the head sums of the previous tile interleaved,
  // a quarter of a 32-head block per k-step, so the wave's vector work is
  // issued while its matrix work runs (in-order issue would otherwise hold
  // the head sums behind the last MFMA of the tile).
  auto scores_overlap = [&](int slot_i, f32x16 (&acc)[NQ * 2], const f32x16 (&prev)[NQ * 2], int prev_tile,
                            bool has_prev) {
    if constexpr (!FP8 && NQ == 1 && FUSED) {
    const unsigned char* src = ring + slot_i * SB;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) acc[mt] = (f32x16){};
    const uint32_t src_a = (uint32_t)(size_t)(const lds_void*)src;
    bf16x8 kb[8];
#define SLI_KB_READ(J) asm volatile("ds_read_b128 %0, %1" : "=v"(kb[J]) : "v"(src_a + (uint32_t)slot(n, 8 * half + J)));
    SLI_KB_READ(0) SLI_KB_READ(1) SLI_KB_READ(2) SLI_KB_READ(3)
    SLI_KB_READ(4) SLI_KB_READ(5) SLI_KB_READ(6) SLI_KB_READ(7)
#undef SLI_KB_READ
    float p4[4] = {0.f, 0.f, 0.f, 0.f};
    // k-step J: the MFMAs of this tile, then the previous tile's heads of
    // block J / 4, rows 8 (J % 4) + 4 half + 0..3
#define SLI_KB_STEP_OV(J)                                                                                  \
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(kb[J]) : "i"(7 - J));                                       \
  acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0].v[J], kb[J], acc[0], 0, 0, 0);                 \
  acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1].v[J], kb[J], acc[1], 0, 0, 0);                 \
  if (has_prev) {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                         \
      p4[i] += wreg[0][4 * (J) + i] * fmaxf(prev[(J) >> 2][4 * ((J) & 3) + i], 0.f);                    \
  }                                                                                                       \
  __builtin_amdgcn_sched_barrier(0);
    SLI_KB_STEP_OV(0) SLI_KB_STEP_OV(1) SLI_KB_STEP_OV(2) SLI_KB_STEP_OV(3)
    SLI_KB_STEP_OV(4) SLI_KB_STEP_OV(5) SLI_KB_STEP_OV(6) SLI_KB_STEP_OV(7)
#undef SLI_KB_STEP_OV
    if (has_prev) {
      float part = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      part += __shfl_xor(part, 32, kWave);
      if (half == 0) {
        const int s = s0 + prev_tile * 32 + n;
        const uint32_t key = (s < vis[0]) ? score_key(part) : 0u;
        const uint32_t ka = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)&s_keys[prev_tile * 32 + n];
        asm volatile("ds_write_b32 %0, %1" : : "v"(ka), "v"(key) : "memory");
        if (key != 0u) {
          kmin[0] = min(kmin[0], key);
          kmax[0] = max(kmax[0], key);
        }
      }
    }
    }
  };

  bool more = tq[0] < nt_used;
  // The single-launch step runs one wave per SIMD, so the head sums of each
  // tile wait for the next tile's MFMAs to be issued (accumulator sets
  // alternating with the slot parity); with two waves per SIMD the other
  // wave fills those gaps and each tile is finished in turn.
  constexpr bool kOverlap = FUSED;
  static_assert(!kOverlap || RS % 2 == 0, "accumulator sets alternate with the slot parity");
  f32x16 acc0[NQ * 2], acc1[NQ * 2];
  uint32_t ksw0 = 0u, ksw1 = 0u;
  int tile0 = 0, tile1 = 0, pend = -1;  // pend: the set whose head sums are outstanding
#pragma unroll 1
  while (more) {
#pragma unroll
    for (int s = 0; s < RS; ++s) {
      if (!more || tq[s] >= nt_used) {
        more = false;
        continue;
      }
      // the tile has landed once at most the instructions issued after its
      // DMA are outstanding (wave-uniform count)
      switch (min(issued - mark[s], (uint32_t)RS * DMA_PER_TILE + 2u)) {
#define SLI_WAIT_CASE(N) case N: SLI_WAIT_VMCNT(N); break;
        SLI_WAIT_CASE(0) SLI_WAIT_CASE(1) SLI_WAIT_CASE(2) SLI_WAIT_CASE(3) SLI_WAIT_CASE(4) SLI_WAIT_CASE(5)
        SLI_WAIT_CASE(6) SLI_WAIT_CASE(7) SLI_WAIT_CASE(8) SLI_WAIT_CASE(9) SLI_WAIT_CASE(10) SLI_WAIT_CASE(11)
        SLI_WAIT_CASE(12) SLI_WAIT_CASE(13) SLI_WAIT_CASE(14) SLI_WAIT_CASE(15) SLI_WAIT_CASE(16) SLI_WAIT_CASE(17)
        SLI_WAIT_CASE(18) SLI_WAIT_CASE(19) SLI_WAIT_CASE(20) SLI_WAIT_CASE(21) SLI_WAIT_CASE(22) SLI_WAIT_CASE(23)
        SLI_WAIT_CASE(24) SLI_WAIT_CASE(25) SLI_WAIT_CASE(26) SLI_WAIT_CASE(27) SLI_WAIT_CASE(28) SLI_WAIT_CASE(29)
        SLI_WAIT_CASE(30) SLI_WAIT_CASE(31) SLI_WAIT_CASE(32) SLI_WAIT_CASE(33) SLI_WAIT_CASE(34) SLI_WAIT_CASE(35)
        SLI_WAIT_CASE(36) SLI_WAIT_CASE(37) SLI_WAIT_CASE(38) SLI_WAIT_CASE(39) SLI_WAIT_CASE(40) SLI_WAIT_CASE(41)
        SLI_WAIT_CASE(42)
#undef SLI_WAIT_CASE
        default: SLI_WAIT_VMCNT(0); break;
      }
      const int tile = tq[s];
      if constexpr (kOverlap) {
        // this tile into the set of the slot parity, the previous one's head sums beside its MFMAs
        if ((s & 1) == 0) {
          scores_overlap(s, acc0, acc1, tile1, pend == 1);
          tile0 = tile;
          pend = 0;
        } else {
          scores_overlap(s, acc1, acc0, tile0, pend == 0);
          tile1 = tile;
          pend = 1;
        }
      } else {
        scores(s, acc0, ksw0);
        head_sums(tile, acc0, ksw0);
      }
      int g = nt_used;
      if (pre < nt_used) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this slot's operand reads are done
        issue_counted(pre, s);
        g = grab();
      }
      tq[s] = pre;
      pre = g;
    }
  }
  if (pend == 0) head_sums(tile0, acc0, ksw0);
  if (pend == 1) head_sums(tile1, acc1, ksw1);
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const uint32_t mn = wave_min(kmin[j]), mx = wave_max(kmax[j]);
    if (lane == 0) {
      sm.mm[j][wid][0] = mn;
      sm.mm[j][wid][1] = mx;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // key stores written as LDS instructions are done
  __syncthreads();

  // ---------------------------------------------------------------- selection
  const int K = a.top_k;
  const size_t ncm = (size_t)a.n_chunks_max;
  // index-row stores (read only after the launch)
  auto put = [&](int32_t* p, int32_t v) { *p = v; };
  // pool row of a position of this chunk (page ids in LDS) or of any
  // position of the request (block table)
  auto own_row = [&](int pos) { return lds.pages[(pos - s0) >> 6] * 64 + (pos & 63); };
  auto any_row = [&](int pos) { return min(max(bt[pos >> 6], 0), a.num_pages - 1) * 64 + (pos & 63); };
  bool any_sel = false;
#pragma unroll
  for (int j = 0; j < NQ; ++j) any_sel |= vis[j] > K;
  // Tokens that see at most K positions keep them all: chunk c's positions go
  // to out[s0 ...] (every earlier chunk is full); the chunk holding the last
  // visible position pads the row with -1.
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    if (vis[j] > K) continue;
    int32_t* out = a.idx_out + (size_t)(t0 + j) * K;
    for (int i = tid; i < CHUNK; i += THREADS)
      if (s0 + i < vis[j]) {
        put(&out[s0 + i], s0 + i);
        if constexpr (FUSED) rows_out[i] = own_row(s0 + i);  // i < vis <= K
      }
    if (c == (vis[j] == 0 ? 0 : (vis[j] - 1) / CHUNK))
      for (int i = vis[j] + tid; i < K; i += THREADS) put(&out[i], -1);
    if constexpr (FUSED) *n_own = max(0, min(CHUNK, vis[j] - s0));
  }
  if (!any_sel) {
    preload(b);
    return kBodyShare;  // (every workgroup of the request decides alike: no exchange)
  }

  // 1. the interval [lo_c, hi_c) holding this chunk's R-th largest key, R its quota
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds.arena);  // [kHistBins] (the key ring is free now)
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    if (vis[j] <= K) continue;
    const int valid = max(0, min(CHUNK, vis[j] - s0));
    const int nv = (vis[j] + CHUNK - 1) / CHUNK;   // chunks holding visible positions (>= 1)
    const int v_last = vis[j] - (nv - 1) * CHUNK;  // visible positions of the last of them
    int R = (K + nv - 1) / nv;
    if (nv > 1 && v_last < CHUNK) {
      const int r_tail = (int)((long long)K * v_last / vis[j]);  // <= v_last (K < vis)
      R = c == nv - 1 ? r_tail : (K - r_tail + nv - 2) / (nv - 1);
    }
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mn = min(mn, sm.mm[j][w][0]);
      mx = max(mx, sm.mm[j][w][1]);
    }
    if (valid == 0) {
      // no visible position: an empty interval, neutral for min lo and max hi
      if (tid == 0) sm.ref[j][0] = 0xffffffffu, sm.ref[j][1] = 0u;
    } else if (R == 0) {
      // no quota: nothing counted at or above lo_c, and no key at or above hi_c
      if (tid == 0) sm.ref[j][0] = 0xffffffffu, sm.ref[j][1] = min(mx, 0xfffffffeu) + 1u;
    } else if (mn == mx) {
      if (tid == 0) sm.ref[j][0] = mn, sm.ref[j][1] = mn + 1u;
    } else {
      const int top = 31 - __clz(mn ^ mx);
      const int shift = max(0, top - 11);
      const uint32_t base = mn >> shift;  // bin of a key: (key >> shift) - base, < 4096
      for (int i = tid; i < kHistBins; i += THREADS) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint32_t key = s_keys[j * CHUNK + tid * PER + i];
        if (key != 0u) atomicAdd(&hist[(key >> shift) - base], 1u);
      }
      __syncthreads();
      // thread t owns bins kHistBins-1 - BPT t - r, r < BPT (descending keys)
      constexpr int BPT = kHistBins / THREADS;
      uint32_t h[BPT], sum = 0;
#pragma unroll
      for (int r = 0; r < BPT; ++r) {
        h[r] = hist[kHistBins - 1 - BPT * tid - r];
        sum += h[r];
      }
      uint32_t tot;
      const uint32_t before = block_excl_scan(sum, sm.scan, tot);
      if (before < (uint32_t)R && (uint32_t)R <= before + sum) {
        uint32_t acc = before;
#pragma unroll
        for (int r = 0; r < BPT; ++r) {
          if (acc < (uint32_t)R && (uint32_t)R <= acc + h[r]) {
            const uint32_t bin = (uint32_t)(kHistBins - 1 - BPT * tid - r) + base;
            const uint64_t up = (uint64_t)(bin + 1u) << shift;
            sm.ref[j][0] = bin << shift;
            sm.ref[j][1] = up > 0xffffffffull ? 0xffffffffu : (uint32_t)up;
          }
          acc += h[r];
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t* rp = a.refs + ((size_t)(t0 + j) * ncm + c) * 2;
      xstore64(&rp[0], tagged(sm.ref[j][0], tag));
      xstore64(&rp[1], tagged(sm.ref[j][1], tag));
    }
  }

  // exchange 1: every chunk's [lo_c, hi_c) -> the request's [lo, hi)
  uint32_t lo_ref[NQ], hi_ref[NQ];
  {
    uint32_t l[NQ], h[NQ];
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      l[j] = 0xffffffffu;
      h[j] = 0u;
      if (vis[j] > K && tid < n_chunks) {
        uint32_t v[2];
        ok &= poll_tagged(a.refs + ((size_t)(t0 + j) * ncm + tid) * 2, 2, tag, a.spin_max, v);
        l[j] = v[0];
        h[j] = v[1];
      }
    }
    const bool refs_ok = block_all(ok, sm.scan);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      l[j] = wave_min(l[j]);
      h[j] = wave_max(h[j]);
      if (lane == 0) {
        sm.mm[j][wid][0] = l[j];
        sm.mm[j][wid][1] = h[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      uint32_t lm = 0xffffffffu, hm = 0u;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        lm = min(lm, sm.mm[j][w][0]);
        hm = max(hm, sm.mm[j][w][1]);
      }
      // a workgroup that did not see every chunk's interval in time treats
      // all of its keys as band, which keeps the selection exact
      lo_ref[j] = refs_ok ? max(lm, 1u) : 1u;
      hi_ref[j] = refs_ok ? hm : 0xffffffffu;
    }
  }

  // 2. publish keys >= hi (back of the region) and the band [lo, hi) (front),
  //    both in position order, then the tagged counts
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    if (vis[j] <= K) continue;
    uint32_t kk[PER];
    uint32_t na = 0, nb = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      kk[i] = s_keys[j * CHUNK + tid * PER + i];
      na += kk[i] >= hi_ref[j] ? 1u : 0u;
      nb += (kk[i] >= lo_ref[j] && kk[i] < hi_ref[j]) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t off = block_excl_scan(na | (nb << 16), sm.scan, tot);  // both counts <= CHUNK < 2^16
    uint32_t oa = off & 0xffffu, ob = off >> 16;
    uint64_t* reg = a.cand + ((size_t)(t0 + j) * ncm + c) * CHUNK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint64_t e = (uint64_t)kk[i] | ((uint64_t)(uint32_t)(s0 + tid * PER + i) << 32);
      if (kk[i] >= hi_ref[j]) {
        xstore64(&reg[CHUNK - 1 - oa], e);
        ++oa;
      } else if (kk[i] >= lo_ref[j]) {
        xstore64(&reg[ob], e);
        ++ob;
      }
    }
    if (tid == 0) sm.flag[2 + (j & 1)] = tot;
  }
  // the lists are complete in memory before the counts that announce them
  wait_vmem();
  __syncthreads();
  uint32_t old2 = 0;
  if (tid == 0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j)
      if (vis[j] > K) xstore64(&a.cnts[(size_t)(t0 + j) * ncm + c], tagged(sm.flag[2 + (j & 1)], tag));
    old2 = __hip_atomic_fetch_add(&ctr[kArrive2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // One-token grids of several rounds (the XCD-local layout) hand the whole
  // request to the last chunk to publish: the others leave at once, so their
  // CU takes the next round's chunks instead of idling through the
  // exchange-2 wait and a selection every chunk of the request would repeat
  // (mixed-length FP8 workload 201.8 -> 195.1 us).  Two-token calls keep the
  // shared selection: there the last chunk's longer stay (two selections)
  // delays the dispatch of the next request's chunks, which then wait for it
  // at exchange 1 (128 x 128K two-token: 749 -> 823 us).  Grids of one round
  // keep every chunk busy to the end.  (Needs the keys' LDS for the two
  // position lists of the write-out.)
  const bool lastw = !FUSED && NQ == 1 && a.xcd_local && NQ * CHUNK >= 2 * K;
  uint32_t cnt_v[NQ];
  if (lastw) {
    if (tid == 0) {
      const bool last = old2 == (uint32_t)n_chunks - 1;
      if (last) __hip_atomic_store(&ctr[kArrive2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.flag[1] = last ? kModeFull : kModeQuit;
    }
    __syncthreads();
    if (sm.flag[1] == kModeQuit) return kBodyQuit;
    // every chunk has published (its count is issued before its arrival)
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      cnt_v[j] = 0u;
      if (vis[j] > K && tid < n_chunks)
        poll_tagged(&a.cnts[(size_t)(t0 + j) * ncm + tid], 1, tag, 1 << 30, &cnt_v[j]);
    }
    __syncthreads();
  } else {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      cnt_v[j] = 0u;
      if (vis[j] > K && tid < n_chunks) ok &= poll_tagged(&a.cnts[(size_t)(t0 + j) * ncm + tid], 1, tag, a.spin_max, &cnt_v[j]);
    }
    const bool all_ok = block_all(ok, sm.scan);
    if (tid == 0) {
      uint32_t mode = kModeNormal;
      const bool last = old2 == (uint32_t)n_chunks - 1;
      if (last) {
        // last to arrive: writes the whole request if some workgroup gave up
        const uint32_t st = __hip_atomic_fetch_or(&ctr[kState], kStLast, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (st & kStGaveUp) mode = kModeFull;
      } else if (!all_ok) {
        const uint32_t st = __hip_atomic_fetch_or(&ctr[kState], kStGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!(st & kStLast)) mode = kModeQuit;  // the last one has not arrived: it will write this share
      }
      sm.flag[1] = mode;
      sm.flag[0] = all_ok ? 1u : 0u;
      // done with the request's exchange state: the last to get here resets it
      const uint32_t d = __hip_atomic_fetch_add(&ctr[kDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == (uint32_t)n_chunks - 1) {
        __hip_atomic_store(&ctr[kArrive2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctr[kState], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctr[kDone], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
  const uint32_t mode = sm.flag[1];
  if (mode == kModeQuit) return kBodyQuit;
  if (!lastw && sm.flag[0] == 0u) {
    // the last one has arrived, so every count is in memory: read them again
#pragma unroll
    for (int j = 0; j < NQ; ++j)
      if (vis[j] > K && tid < n_chunks)
        poll_tagged(&a.cnts[(size_t)(t0 + j) * ncm + tid], 1, tag, 1 << 30, &cnt_v[j]);
    __syncthreads();
  }

  // 3. exact select among the band entries, then the writes
  uint32_t* s_bk = reinterpret_cast<uint32_t*>(lds.arena);       // [kBandCap] band keys
  int32_t* s_bp = reinterpret_cast<int32_t*>(s_bk + kBandCap);  // [kBandCap] their positions
  // (in the arena after the band: the key ring is dead, and sharing it lets
  // the four-wave FP8 workgroups fit three to a CU)
  uint32_t* const cbase = reinterpret_cast<uint32_t*>(s_bp + kBandCap);  // [max chunks + 1] band entries before each chunk
  uint32_t* const abase = cbase + kMaxChunksPerSeq + 1;                  // [max chunks + 1] keys >= hi before each chunk
  uint32_t* const nabove = abase + kMaxChunksPerSeq + 1;                 // [max chunks] keys >= hi per chunk
  uint32_t* const bitmap = nabove + kMaxChunksPerSeq;                    // [CHUNK / 32] one chunk's selected positions
  static_assert(IdxSmem<NQ, NW, CHUNK, FP8, RS>::kSel <= IdxSmem<NQ, NW, CHUNK, FP8, RS>::kArena, "arena layout");
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    if (vis[j] <= K) continue;
    const size_t tok = (size_t)(t0 + j);
    // A chunk's two counts fit 16 bits each (<= CHUNK), but the request's
    // band can hold every position of the request (scores that rise with
    // position put each chunk's bracket at a different key): the prefixes over
    // the chunks are taken as separate 32-bit scans.
    const uint32_t cv[2] = {cnt_v[j] & 0xffffu, cnt_v[j] >> 16};  // keys >= hi, band keys (0 past n_chunks)
    uint32_t cpre[2], ctot[2];
    block_excl_scan_n<2>(cv, sm.scan, cpre, ctot);
    if (tid < n_chunks) {
      abase[tid] = cpre[0];
      cbase[tid] = cpre[1];
      nabove[tid] = cv[0];
    }
    if (tid == 0) {
      abase[n_chunks] = ctot[0];
      cbase[n_chunks] = ctot[1];
    }
    __syncthreads();
    const uint32_t A = ctot[0], NB = ctot[1];
    const int need = K - (int)A;  // >= 1: fewer than K keys reach hi
    const bool in_lds = NB <= (uint32_t)kBandCap;
    auto gaddr = [&](int i, uint32_t sl) { return (tok * ncm + i) * CHUNK + sl; };
    // flat band entry f -> chunk (binary search over the prefix offsets)
    auto chunk_of = [&](int f) {
      int lo = 0, hi = n_chunks;  // cbase[lo] <= f < cbase[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)cbase[mid] <= f) lo = mid; else hi = mid;
      }
      return lo;
    };
    if (in_lds) {
      // up to eight loads per thread in flight at once (one memory latency
      // per 8 x blockDim entries)
      constexpr int LPT = kBandCap / THREADS < 8 ? kBandCap / THREADS : 8;
#pragma unroll 1
      for (int f0 = 0; f0 < (int)NB; f0 += LPT * THREADS) {
        uint64_t ev[LPT];
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
          const int f = f0 + tid + r * THREADS;
          ev[r] = 0ull;
          if (f < (int)NB) {
            const int i = chunk_of(f);
            ev[r] = xload64(&a.cand[gaddr(i, f - cbase[i])]);
          }
        }
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
          const int f = f0 + tid + r * THREADS;
          if (f < (int)NB) {
            s_bk[f] = (uint32_t)ev[r];
            s_bp[f] = (int32_t)(ev[r] >> 32);
          }
        }
      }
      __syncthreads();
    }
    // from here to the index stores the selection reads no global memory
    // (with the band in LDS): the caller's loads go now
    if (j == 0) preload(b);
    auto key_at = [&](int f) -> uint32_t {
      if (in_lds) return s_bk[f];
      const int i = chunk_of(f);
      return (uint32_t)xload64(&a.cand[gaddr(i, f - cbase[i])]);
    };
    int ngt;
    uint32_t tau;
    if (in_lds && NB <= 8u * kWave) {
      // the usual band (a few hundred entries): one wave selects, no block barriers
      if (wid == 0) {
        int g;
        const uint32_t tv = wave_radix_select<8>([&](int f) { return s_bk[f]; }, (int)NB, need, sm.hist, g);
        if (lane == 0) {
          sm.sel[2] = tv;
          sm.sel[3] = (uint32_t)g;
        }
      }
      __syncthreads();
      tau = sm.sel[2];
      ngt = (int)sm.sel[3];
    } else {
      // (the band in LDS is read through an accessor with no global path: a
      // read that might also be a global load makes the compiler wait for
      // every memory operation in flight before each LDS read)
      tau = in_lds ? block_radix_select<kBandCap / THREADS>([&](int f) { return s_bk[f]; }, (int)NB, need, sm.hist,
                                                            sm.sel, ngt)
                   : block_radix_select_big(key_at, (int)NB, need, sm.hist, sm.sel, ngt);
    }
    const uint32_t ties = (uint32_t)(need - ngt);  // keys equal to tau that are taken, lowest positions first
    int32_t* out = a.idx_out + tok * K;

    if (lastw) {
      // The whole request from the published lists: every chunk's keys >= hi
      // (all selected; in chunk order they are in position order) and the
      // selected band entries (> tau, or tied at tau up to `ties` of them,
      // lowest positions first; the flat band is in position order too).
      // Both lists are sorted, so a position's output slot is its rank in its
      // own list plus the number of the other list's positions below it.  The
      // keys' LDS is free (every chunk's keys are in the lists).
      int32_t* const above_pos = reinterpret_cast<int32_t*>(s_keys);  // [A]
      int32_t* const band_pos = above_pos + K;                        // [need]
      auto seg_of = [&](const uint32_t* base, int f) {  // largest i < n_chunks with base[i] <= f
        int lo = 0, hi = n_chunks;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if ((int)base[mid] <= f) lo = mid; else hi = mid;
        }
        return lo;
      };
      {
        // chunk i's keys >= hi sit at the back of its list, in position order
        // from the last slot down; eight loads per thread in flight
        constexpr int LPT = 8;
#pragma unroll 1
        for (int f0 = 0; f0 < (int)A; f0 += LPT * THREADS) {
          uint64_t ev[LPT];
#pragma unroll
          for (int r = 0; r < LPT; ++r) {
            const int f = f0 + tid + r * THREADS;
            ev[r] = 0ull;
            if (f < (int)A) {
              const int i = seg_of(abase, f);
              ev[r] = xload64(&a.cand[gaddr(i, CHUNK - 1 - (f - (int)abase[i]))]);
            }
          }
#pragma unroll
          for (int r = 0; r < LPT; ++r) {
            const int f = f0 + tid + r * THREADS;
            if (f < (int)A) above_pos[f] = (int32_t)(ev[r] >> 32);
          }
        }
      }
      // the selected band entries, compacted in order: an entry > tau, or the
      // tie of rank < ties; its slot = selected entries before it
      uint32_t n_sel = 0, eq_seen = 0;
      auto compact = [&](auto get) {
#pragma unroll 1
        for (int fb = 0; fb < (int)NB; fb += THREADS) {
          const int f = fb + tid;
          const uint64_t ev = f < (int)NB ? get(f) : 0ull;
          const uint32_t key = (uint32_t)ev;
          const bool in = f < (int)NB;
          const bool gt = in && key > tau, tie = in && key == tau;
          uint32_t gt_tot, tie_pre, tie_tot;
          const uint32_t gt_pre = block_excl_scan2(gt ? 1u : 0u, tie ? 1u : 0u, sm.scan, gt_tot, tie_pre, tie_tot);
          const uint32_t avail = ties > eq_seen ? ties - eq_seen : 0u;  // ties still to take
          if (gt || (tie && tie_pre < avail)) {
            const uint32_t slot = n_sel + gt_pre + min(tie_pre, avail);
            if (slot < (uint32_t)K) band_pos[slot] = (int32_t)(ev >> 32);
          }
          n_sel += gt_tot + min(tie_tot, avail);
          eq_seen += tie_tot;
        }
      };
      if (in_lds)
        compact([&](int f) { return (uint64_t)s_bk[f] | ((uint64_t)(uint32_t)s_bp[f] << 32); });
      else
        compact([&](int f) {
          const int i = chunk_of(f);
          return xload64(&a.cand[gaddr(i, f - cbase[i])]);
        });
      __syncthreads();
      const int n_band = min((int)n_sel, K - (int)A);  // = need
      auto below = [](const int32_t* list, int n, int p) {  // entries of a sorted list below p
        int lo = 0, hi = n;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (list[mid] < p) lo = mid + 1; else hi = mid;
        }
        return lo;
      };
      for (int f = tid; f < (int)A; f += THREADS) {
        const int p = above_pos[f];
        const int o = f + below(band_pos, n_band, p);
        if (o < K) put(&out[o], p);
      }
      for (int g = tid; g < n_band; g += THREADS) {
        const int p = band_pos[g];
        const int o = g + below(above_pos, (int)A, p);
        if (o < K) put(&out[o], p);
      }
    } else if (mode == kModeNormal) {
      // band entries before this chunk: how many are > tau, how many tie
      // (eight reads per thread in flight; the LDS and global forms are
      // separate loops, so the LDS reads wait for nothing but themselves)
      uint32_t gt = 0, eq = 0;
      const int cb = (int)cbase[c];
      constexpr int LPT = 8;
      auto count = [&](auto get) {
#pragma unroll 1
        for (int f0 = tid; f0 < cb; f0 += LPT * THREADS) {
          uint32_t kv[LPT];
#pragma unroll
          for (int r = 0; r < LPT; ++r) kv[r] = f0 + r * THREADS < cb ? get(f0 + r * THREADS) : 0u;
#pragma unroll
          for (int r = 0; r < LPT; ++r) {
            const bool in = f0 + r * THREADS < cb;
            gt += (in && kv[r] > tau) ? 1u : 0u;
            eq += (in && kv[r] == tau) ? 1u : 0u;
          }
        }
      };
      if (in_lds) count([&](int f) { return s_bk[f]; });
      else count(key_at);
      // own keys in position order: selected for certain (>= hi, or in the
      // band and > tau) or tied at tau
      uint32_t kk[PER], nd = 0, nt = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        kk[i] = s_keys[j * CHUNK + tid * PER + i];
        const bool band = kk[i] >= lo_ref[j] && kk[i] < hi_ref[j];
        nd += (kk[i] >= hi_ref[j] || (band && kk[i] > tau)) ? 1u : 0u;
        nt += (band && kk[i] == tau) ? 1u : 0u;
      }
      // one scan: totals of the earlier chunks' band (32 bits each: the band
      // may hold most of the request), prefixes of this chunk's keys (packed:
      // both <= CHUNK < 2^16)
      const uint32_t sv[3] = {gt, eq, nd | (nt << 16)};
      uint32_t spre[3], stot[3];
      block_excl_scan_n<3>(sv, sm.scan, spre, stot);
      const uint32_t gt_before = stot[0], eq_before = stot[1], pre = spre[2];
      const uint32_t avail = ties > eq_before ? ties - eq_before : 0u;  // ties left for this chunk
      uint32_t tr = pre >> 16;                                            // ties of this chunk before my keys
      const uint32_t o0 = abase[c] + gt_before + min(ties, eq_before);  // this chunk's first output
      uint32_t o = o0 + (pre & 0xffffu) + min(avail, tr);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const bool band = kk[i] >= lo_ref[j] && kk[i] < hi_ref[j];
        const bool tie = band && kk[i] == tau;
        if (kk[i] >= hi_ref[j] || (band && kk[i] > tau) || (tie && tr < avail)) {
          if constexpr (FUSED) rows_out[o - o0] = own_row(s0 + tid * PER + i);
          put(&out[o++], s0 + tid * PER + i);
        }
        tr += tie ? 1u : 0u;
      }
      if constexpr (FUSED) *n_own = (int)((stot[2] & 0xffffu) + min(avail, stot[2] >> 16));
    } else {
      // kModeFull: the whole request, chunk by chunk, from the published
      // lists (keys >= hi all taken; band entries by tau and tie rank)
      uint32_t off = 0, eq_seen = 0;
#pragma unroll 1
      for (int i = 0; i < n_chunks; ++i) {
        for (int wd = tid; wd < CHUNK / 32; wd += THREADS) bitmap[wd] = 0u;
        __syncthreads();
        const int ci0 = i * CHUNK;
        for (uint32_t e = tid; e < nabove[i]; e += THREADS) {
          const int pos = (int)(xload64(&a.cand[gaddr(i, CHUNK - 1 - e)]) >> 32);
          atomicOr(&bitmap[(pos - ci0) >> 5], 1u << ((pos - ci0) & 31));
        }
        const int f0 = (int)cbase[i], f1 = (int)cbase[i + 1];
#pragma unroll 1
        for (int fb = f0; fb < f1; fb += THREADS) {
          const int f = fb + tid;
          uint64_t ev = 0ull;
          if (f < f1)
            ev = in_lds ? ((uint64_t)s_bk[f] | ((uint64_t)(uint32_t)s_bp[f] << 32)) : xload64(&a.cand[gaddr(i, f - f0)]);
          const uint32_t key = (uint32_t)ev;
          const bool tie = f < f1 && key == tau;
          uint32_t et;
          const uint32_t rank = eq_seen + block_excl_scan(tie ? 1u : 0u, sm.scan, et);
          if (f < f1 && (key > tau || (tie && rank < ties))) {
            const int pos = (int)(ev >> 32);
            atomicOr(&bitmap[(pos - ci0) >> 5], 1u << ((pos - ci0) & 31));
          }
          eq_seen += et;
        }
        __syncthreads();
        // emit in position order: thread t owns bits PER*t .. PER*t + PER-1
        const uint32_t word = bitmap[(PER * tid) >> 5];
        const uint32_t bits = (word >> ((PER * tid) & 31)) & ((1u << PER) - 1u);
        uint32_t et;
        uint32_t o = off + block_excl_scan((uint32_t)__popc(bits), sm.scan, et);
#pragma unroll
        for (int r = 0; r < PER; ++r)
          if ((bits >> r) & 1u) {
            if constexpr (FUSED) rows_out[o] = any_row(ci0 + PER * tid + r);
            put(&out[o++], ci0 + PER * tid + r);
          }
        off += et;
        __syncthreads();
      }
      if constexpr (FUSED) *n_own = (int)off;
    }
    __syncthreads();  // LDS band arrays and offsets are reused by the next token
  }
  return mode == kModeFull ? kBodyAll : kBodyShare;
}

}  // namespace sli
