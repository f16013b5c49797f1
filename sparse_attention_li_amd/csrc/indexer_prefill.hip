// Fused lightning-indexer score + Top-K for a prefill chunk (many causal
// query tokens of one request), gfx950.
//
// Same operation as the decode kernel (pages: "Optimizing Inference for
// Hybrid Attention LLMs", sec. 3.1 -- the fused indexer serves both prefill
// and decode; "Day-0 Inference Adaptation and Optimization for Hybrid
// Attention Architectures", sec. 3), with causal visibility per query:
// query j of request b sees positions s <= L_b - n_q + j.
//
// Decomposition.  A workgroup owns 4 consecutive queries of one request and
// streams every key position any of them can see, one 64-position page per
// step.  The page is moved once into an LDS ring by direct-to-LDS loads (two
// 1 KiB instructions per wave) and read by all 8 waves: wave (query, half)
// multiplies all 64 heads of its query (two 32-row MFMA blocks, q held in
// registers) with the 32 positions of its half of the page, so key traffic
// from L2 is divided by the 4 queries and no partial head sums cross waves
// inside a page.  The weighted ReLU head sum of page t (head weights in
// registers) is taken while the MFMAs of page t+1 run, so the vector work
// hides behind the matrix cores.  The two lane halves of each wave hold
// different heads; their partial sums go to LDS and the query's first wave
// adds them when it filters the page one step later.
//
// Exact streaming Top-K per query, kept in LDS: positions arrive in
// increasing order and a position is appended to the query's candidate
// buffer (key, position) if its key reaches the running threshold tau.  An
// append also counts the key in a 256-bin histogram over [tau, max key].
// When the buffer nears capacity the histogram alone gives a new tau -- the
// lower edge of the bin holding the K-th largest key, so at least K seen keys
// stay above it -- and one in-order pass drops the keys below it.  Only when
// that frees too little (the first fill, heavy ties) does the wave run an
// exact radix selection, which keeps exactly the top K (ties to the lower,
// earlier, position) and makes tau strict: a later position with an equal
// key ranks behind every kept one.  The buffer therefore always holds the top
// K of the positions seen so far plus later contenders, in position order; a
// final exact selection writes the indices.  Scores never leave the chip.
#include "device_common.h"
#include "launch.h"

namespace sli {

typedef __attribute__((address_space(3))) void lds_void;
#define SLI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N)&15) | (((N) >> 4) << 14) | 0x70 | 0xF00)

constexpr int kPfQueries = 4;             // queries per workgroup
constexpr int kPfWaves = 2 * kPfQueries;  // one wave per (query, position half)
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfTile = 64;               // positions per key tile = one page
constexpr int kPfRing = 3;                // key tiles: one read, one landed, one in flight
constexpr int kPfCap = 3328;              // candidate slots per query (fills the LDS)
constexpr int kPfRoom = 640;              // a threshold-only compaction must leave this many free

struct PfSmem {
  alignas(16) unsigned char ring[kPfRing][kPfTile * 256];
  uint64_t buf[kPfQueries][kPfCap];         // key | position << 32, position order
  float xs[2][kPfQueries][2][kPfTile];      // [tile parity][query][lane half][position]
  uint32_t hist[kPfQueries][256];
};

// LDS byte offset of (row, 16-byte chunk) in a 64 x 256-byte key tile: rows
// are contiguous, chunks XOR-swizzled by row & 15, so 16 lanes reading the
// same chunk of 16 consecutive rows hit 16 distinct bank groups.
__device__ __forceinline__ int pf_slot(int row, int col) { return 256 * row + 16 * (col ^ (row & 15)); }

// LDS atomic add written as the instruction itself: the compiler's wait
// insertion cannot tell an atomic apart from the key-ring DMA and would drain
// every tile load in flight before it.  LDS operations of a wave complete in
// order, so later reads of the same wave see the sum; other waves read the
// histogram only after an lgkmcnt(0) wait and a barrier.
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
  const uint32_t off = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)p;
  asm volatile("ds_add_u32 %0, %1" ::"v"(off), "v"(v) : "memory");
}

// max(x, 0) as one integer max on the bits: a negative float (or -0) is a
// negative integer.  fmaxf would add a NaN-quieting canonicalisation.
__device__ __forceinline__ float relu(float x) { return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0)); }

__device__ __forceinline__ int lane_rank(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Wave-level exact selection over buf[0..n), n > k >= 1: tau = the k-th
// largest key, ties = how many entries equal to tau rank within the top k
// (the earliest ones, buf being in position order).  hist is 256 words of
// scratch.
__device__ void pf_select(const uint64_t* buf, int n, int k, uint32_t* hist, uint32_t& tau, uint32_t& ties) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = lane; i < n; i += kWave) {
    const uint32_t v = (uint32_t)buf[i];
    lo = min(lo, v);
    hi = max(hi, v);
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  uint32_t prefix, remaining = (uint32_t)k;
  if (lo == hi) {
    prefix = lo;
  } else {
    int top = 31 - __clz(lo ^ hi);
    prefix = lo & ~((2u << top) - 1u);
    while (top >= 0) {
      const int shift = top >= 7 ? top - 7 : 0;
      const int width = top - shift + 1;
      const uint32_t above = top == 31 ? 0u : ~((2u << top) - 1u);
#pragma unroll
      for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      for (int base = 0; base < n; base += 4 * kWave) {
        uint32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kWave + lane;
          v[u] = i < n ? (uint32_t)buf[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = base + u * kWave + lane;
          if (i < n && (v[u] & above) == prefix) atomicAdd(&hist[(v[u] >> shift) & ((1u << width) - 1u)], 1u);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = hist[255 - 4 * lane - i];
      const uint32_t sum = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
      const bool mine = excl < remaining && remaining <= incl;
      uint32_t dsel = 0, rsel = 0;
      if (mine) {
        uint32_t acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (acc < remaining && remaining <= acc + h[i]) {
            dsel = 255u - 4u * lane - i;
            rsel = remaining - acc;
          }
          acc += h[i];
        }
      }
      const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;  // exactly one lane
      dsel = __shfl(dsel, src, kWave);
      rsel = __shfl(rsel, src, kWave);
      prefix |= dsel << shift;
      remaining = rsel;
      top = shift - 1;
    }
  }
  tau = prefix;
  ties = remaining;
}

// In-order compaction of buf[0..n): keeps keys > thr, and of the keys equal
// to thr all of them (kEqAll) or the first `ties`.  With `rebuild`, counts
// every kept key into hist (already zero) over bins of width 2^hsh from
// hbase, the last bin open-ended.  Returns the new count.
template <bool kEqAll>
__device__ int pf_compact_pass(uint64_t* buf, int n, uint32_t thr, uint32_t ties, uint32_t* hist, uint32_t hbase,
                               int hsh, bool rebuild) {
  const int lane = threadIdx.x & (kWave - 1);
  int out = 0;
  uint32_t ties_seen = 0;
  for (int base = 0; base < n; base += 4 * kWave) {
    uint64_t e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * kWave + lane;
      e[u] = i < n ? buf[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = base + u * kWave + lane < n;
      const uint32_t key = (uint32_t)e[u];
      bool keep;
      if (kEqAll) {
        keep = valid && key >= thr;
      } else {
        const bool eq = valid && key == thr;
        const uint64_t tie_mask = __ballot(eq);
        keep = valid && (key > thr || (eq && ties_seen + (uint32_t)lane_rank(tie_mask) < ties));
        ties_seen += (uint32_t)__popcll(tie_mask);
      }
      const uint64_t keep_mask = __ballot(keep);
      if (keep) {
        buf[out + lane_rank(keep_mask)] = e[u];  // slot <= read index: never ahead of the reads
        if (rebuild) atomicAdd(&hist[min(255u, (key - hbase) >> hsh)], 1u);
      }
      out += __popcll(keep_mask);
    }
  }
  return out;
}

__global__ __launch_bounds__(kPfThreads) void li_prefill_kernel(const IdxPrefillArgs a) {
  __shared__ PfSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wid & (kPfQueries - 1), ph = wid / kPfQueries;  // query of this wave, position half
  const int n = lane & 31, half = lane >> 5;

  // heaviest query blocks first
  const int nqb = (a.n_q + kPfQueries - 1) / kPfQueries;
  const int item = gridDim.x - 1 - blockIdx.x;
  const int b = item / nqb, qb = item % nqb;
  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * kPfTile));
  const int j0 = qb * kPfQueries;
  const int nq_here = min(kPfQueries, a.n_q - j0);
  const int* bt = a.block_table + (size_t)b * a.max_pages;
  // visible positions of each query of the block; the block streams the largest
  const int vis_last = max(0, min(L, L - a.n_q + j0 + nq_here));
  const int n_tiles = (vis_last + kPfTile - 1) / kPfTile;
  const bool q_ok = qw < nq_here;
  const int vis_q = q_ok ? max(0, min(L, L - a.n_q + j0 + qw + 1)) : 0;
  const bool fin = ph == 0 && q_ok;  // this wave filters and selects for its query
  // The filtering wave carries the longer path of each step (its filter, then
  // its MFMA chains): it issues first when both waves of its SIMD are ready
  // (3.568 -> 3.546 ms; the other way round, 3.652).
  if (fin) __builtin_amdgcn_s_setprio(1);

  // A operands: heads 32*blk + n of this wave's query; k-step j = d 64*half+8j .. +8.
  // Head weights of the accumulator rows this lane holds: 32*blk + 8*(v/4) + 4*half + v%4.
  bf16x8 qa[2][8];
  float wv[2][16];
  {
    const size_t tok = (size_t)b * a.n_q + j0 + (q_ok ? qw : 0);
    const __bf16 keep = q_ok ? (__bf16)1.f : (__bf16)0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const bf16x8* qp =
          reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + (tok * 64 + 32 * blk + n) * 128 + 64 * half);
#pragma unroll
      for (int j = 0; j < 8; ++j) qa[blk][j] = qp[j] * keep;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(a.w + tok * 64 + 32 * blk + 8 * g + 4 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[blk][4 * g + i] = w4[i];
      }
    }
  }
  if (fin) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.hist[qw][4 * lane + i] = 0;
  }
  SLI_WAIT_VMCNT(0);  // register operands are in before the DMA accounting starts

  // Direct-to-LDS load of tile t: wave w copies rows 4i..4i+3 for i = w, w+8,
  // through a buffer resource spanning exactly the tile's page (the hardware
  // returns zeros for any offset outside it).  The block table is read
  // through the constant address space, so the wave-uniform page id comes
  // from a scalar load and leaves the vector memory counter to the tiles.
  typedef __attribute__((address_space(4))) const int const_int;
  const_int* btc = (const_int*)bt;
  auto page = [&](int t) { return min(max(btc[min(t, n_tiles - 1)], 0), a.num_pages - 1); };
  uint32_t dma_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 4 * (wid + kPfWaves * h) + (lane >> 4);
    dma_off[h] = (uint32_t)(row * 256 + 16 * ((lane & 15) ^ (row & 15)));
  }
  auto issue = [&](int t, int pg) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(a.k)) + (size_t)pg * (kPfTile * 256), (short)0, kPfTile * 256, 0x00020000);
    unsigned char* dst = sm.ring[(uint32_t)t % kPfRing];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + 1024 * (wid + kPfWaves * h)), 16, dma_off[h], 0, 0, 0);
  };
  // B operands: row 32*ph + n of the tile, chunk 8*half + j for k-step j
  uint32_t kb_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kb_off[j] = (uint32_t)pf_slot(32 * ph + n, 8 * half + j);

  // selection state of the query (meaningful in the filtering wave only)
  int cnt = 0;
  uint32_t tau = 0u, hbase = 0u;
  int hsh = 24;  // bins of the top 8 key bits until the first compaction
  bool strict = false;
  uint64_t* qbuf = sm.buf[qw];
  uint32_t* qhist = sm.hist[qw];

  // Bin holding the K-th largest key, counting from the top bin (the buffer
  // holds more than K keys, all binned), and how many keys lie in it or above.
  auto kth_bin = [&](uint32_t (&h)[4], uint32_t& bsel, uint32_t& kept) {
    const uint32_t K = (uint32_t)a.top_k;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = qhist[255 - 4 * lane - i];
    const uint32_t sum = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t excl = incl - sum;
    const bool mine = excl < K && K <= incl;
    bsel = 0;
    kept = 0;
    if (mine) {
      uint32_t acc = excl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (acc < K && K <= acc + h[i]) {
          bsel = 255u - 4u * lane - i;
          kept = acc + h[i];
        }
        acc += h[i];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    bsel = __shfl(bsel, src, kWave);
    kept = __shfl(kept, src, kWave);
  };
  // Between compactions (every 16 steps) the threshold follows the histogram: the lower edge
  // of the K-th key's bin has at least K seen keys at or above it.  Keys
  // below it stay in the buffer (and their bins) until the next compaction.
  auto raise = [&]() {
    uint32_t h[4], bsel, kept;
    kth_bin(h, bsel, kept);
    const uint32_t edge = hbase + (bsel << hsh);
    if (edge > tau) {
      tau = edge;
      strict = false;
    }
  };

  auto compact = [&]() {
    const uint32_t K = (uint32_t)a.top_k;
    uint32_t h[4], bsel, kept;
    kth_bin(h, bsel, kept);
    const uint32_t sum = h[0] + h[1] + h[2] + h[3];
    // highest non-empty bin bounds the largest key (unless it is the open top bin)
    const int top_lane = __ffsll((unsigned long long)__ballot(sum != 0)) - 1;
    uint32_t btop = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i)
      if (h[i] != 0) btop = 255u - 4u * lane - i;
    btop = __shfl(btop, top_lane, kWave);
    const uint32_t old_base = hbase;
    const int old_sh = hsh;
    uint32_t thr, ties = 0;
    bool eq_all;
    if (bsel >= 1 && kept <= (uint32_t)(kPfCap - kPfRoom)) {
      thr = hbase + (bsel << hsh);  // lower edge of that bin: >= K seen keys reach it
      eq_all = true;
      strict = false;
    } else {
      pf_select(qbuf, cnt, (int)K, qhist, thr, ties);
      eq_all = false;
      strict = true;
    }
    tau = thr;
    hbase = thr;
    uint32_t kmax;
    if (btop < 255u) {
      kmax = (uint32_t)min((uint64_t)0xffffffffu, (uint64_t)old_base + ((uint64_t)(btop + 1u) << old_sh) - 1u);
    } else {
      kmax = 0u;
      for (int i = lane; i < cnt; i += kWave) kmax = max(kmax, (uint32_t)qbuf[i]);
      kmax = wave_max(kmax);
    }
    const uint32_t range = kmax - thr;
    hsh = range > 255u ? 24 - __clz(range) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) qhist[4 * lane + i] = 0;
    __builtin_amdgcn_s_waitcnt(0xC07F);
    cnt = eq_all ? pf_compact_pass<true>(qbuf, cnt, thr, 0u, qhist, hbase, hsh, true)
                 : pf_compact_pass<false>(qbuf, cnt, thr, ties, qhist, hbase, hsh, true);
  };

  // filter tile u of this query (both lane halves' partial sums) and append
  auto finish = [&](int u) {
    const float sc = sm.xs[u & 1][qw][0][lane] + sm.xs[u & 1][qw][1][lane];
    const int p = kPfTile * u + lane;
    const uint32_t key = score_key(sc);
    const bool take = p < vis_q && (strict ? key > tau : key >= tau);
    const uint64_t m = __ballot(take);
    if (m != 0) {
      if (take) {  // (bounded indices into sm, one 64-bit store: the compiler sees these miss the key ring)
        sm.buf[qw][min((uint32_t)(cnt + lane_rank(m)), (uint32_t)kPfCap - 1u)] = ((uint64_t)p << 32) | key;
        lds_add(&sm.hist[qw][min(255u, (key - hbase) >> hsh)], 1u);
      }
      cnt += __popcll(m);
    }
  };

  int pg_next = 0;   // page of the next tile to load
  float part0 = 0.f; // head-block-0 partial sum of the previous tile (this lane's heads, position 32*ph + n)
  f32x16 acc0, acc1; // head blocks 0 and 1 of the tile being multiplied

  // Step t (tile t's B operands are already in registers): wait until tile
  // t+1 has landed (tile t+2 may be in flight); a raw barrier (no fence: it
  // would also wait for the prefetch) makes it and the partial sums of tile
  // t-1 visible to every wave and frees the slot of tile t, read during step
  // t-1, for tile t+3.  Then
  //   phase A: MFMA chain of head block 0 of tile t, with the head-block-1
  //            weighted ReLU sum of tile t-1 (its partial goes to LDS);
  //   phase B: MFMA chain of head block 1 of tile t, with the LDS reads of
  //            tile t+1 and the head-block-0 sum of tile t.
  // Each k-step's MFMA is followed by a small share of vector work that the
  // wave issues while the MFMA runs; the scheduling fences keep it there.
  // The query's first wave filters tile t-2 (both partials visible since the
  // barrier) before its phase A: its SIMD's other wave, which does not
  // filter, has the matrix pipe to itself meanwhile, and the filter no
  // longer trails the step (3.634 -> 3.575 ms against filtering after phase B).
  auto step = [&](int t, const bf16x8 (&kc)[8], bf16x8 (&kn)[8], bool steady) {
    if (steady || t + 2 < n_tiles) SLI_WAIT_VMCNT(2);
    else SLI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    if (steady || t + 3 < n_tiles) issue(t + 3, pg_next);
    // the next page id (a scalar load) is requested now, so its latency
    // passes under this step's matrix work rather than at the next step's
    // wait, which also covers scalar loads
    pg_next = page(t + 4);
    const bool cur = steady || t < n_tiles;
    const bool prev = steady || (t >= 1 && t - 1 < n_tiles);
    const bool next = steady || t + 1 < n_tiles;
    if (fin && (steady || (t >= 2 && t - 2 < n_tiles))) finish(t - 2);
    if (fin && cnt > kPfCap - kPfTile) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      compact();
    } else if (fin && (t & 15) == 15 && cnt > a.top_k) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      raise();
    }
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (cur) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][j], kc[j], j ? acc0 : (f32x16){}, 0, 0, 0);
      if (prev) {
#pragma unroll
        for (int v = 2 * j; v < 2 * j + 2; ++v) s[v & 3] += wv[1][v] * relu(acc1[v]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (prev) sm.xs[(t - 1) & 1][qw][half][32 * ph + n] = part0 + ((s[0] + s[1]) + (s[2] + s[3]));
    float s0[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (cur) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][j], kc[j], j ? acc1 : (f32x16){}, 0, 0, 0);
      if (next) kn[j] = *reinterpret_cast<const bf16x8*>(sm.ring[(uint32_t)(t + 1) % kPfRing] + kb_off[j]);
      if (cur) {
#pragma unroll
        for (int v = 2 * j; v < 2 * j + 2; ++v) s0[v & 3] += wv[0][v] * relu(acc0[v]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    part0 = (s0[0] + s0[1]) + (s0[2] + s0[3]);
  };

  if (n_tiles > 0) {
    bf16x8 kbA[8], kbB[8];  // B operands of tile t: kbA for even t, kbB for odd t
    for (int i = 0; i < 3 && i < n_tiles; ++i) issue(i, page(i));
    pg_next = page(3);
    // tile 0 landed (tiles 1 and 2 may be in flight)
    if (n_tiles > 2) SLI_WAIT_VMCNT(4);
    else if (n_tiles > 1) SLI_WAIT_VMCNT(2);
    else SLI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int j = 0; j < 8; ++j) kbA[j] = *reinterpret_cast<const bf16x8*>(sm.ring[0] + kb_off[j]);
    step(0, kbA, kbB, false);
    step(1, kbB, kbA, false);
    int t = 2;
#pragma unroll 1
    for (; t + 4 < n_tiles; t += 2) {
      step(t, kbA, kbB, true);
      step(t + 1, kbB, kbA, true);
    }
#pragma unroll 1
    for (; t < n_tiles + 2; t += 2) {
      step(t, kbA, kbB, false);
      if (t + 1 < n_tiles + 2) step(t + 1, kbB, kbA, false);
    }
  }

  // final selection and output (ascending positions, -1 padded)
  if (fin) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (cnt > a.top_k) {
      uint32_t thr, ties;
      pf_select(qbuf, cnt, a.top_k, qhist, thr, ties);
      cnt = pf_compact_pass<false>(qbuf, cnt, thr, ties, qhist, 0u, 0, false);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    int32_t* out = a.idx_out + ((size_t)b * a.n_q + j0 + qw) * a.top_k;
    for (int i = lane; i < a.top_k; i += kWave) out[i] = i < cnt ? (int32_t)(qbuf[i] >> 32) : -1;
  }
}

hipError_t launch_idx_prefill(const IdxPrefillArgs& a, hipStream_t stream) {
  const int nqb = (a.n_q + kPfQueries - 1) / kPfQueries;
  hipLaunchKernelGGL(li_prefill_kernel, dim3(a.B * nqb), dim3(kPfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sli
