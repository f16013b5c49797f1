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
// Exact selection across workgroups without writing the scores out:
//   1. each workgroup sorts a copy of its chunk's keys in LDS and publishes
//      order statistics: the key at descending rank 32i-1 certifies that the
//      chunk holds >= 32i keys >= it;
//   2. after every chunk of the request has published (a bounded wait on an
//      arrival counter), the m-th largest sample, m = ceil(K/32), is a lower
//      bound tau on the K-th largest score of the request: the samples above
//      it certify >= K keys >= tau;
//   3. each workgroup appends only its keys >= tau (in position order) to its
//      own candidate region -- about K + 32 per chunk in all, not the scores;
//   4. the last workgroup to finish runs an exact radix select over the
//      candidates and writes the indices in ascending position order.
// If the wait times out (the request's chunks were not co-resident) the
// workgroup falls back to tau = "every valid key", which keeps the result
// exact and only costs candidate bytes.
#include "device_common.h"
#include "launch.h"

namespace sli {

typedef __attribute__((address_space(3))) void lds_void;
#define SLI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N)&15) | (((N) >> 4) << 14) | 0x70 | 0xF00)

constexpr int kIdxThreads = 256;
constexpr int kRun = 256;               // keys one wave sorts in registers
constexpr int kCandCap = 4096;          // candidates the final select keeps in LDS
constexpr unsigned kSpinMax = 20000;    // ~1 ms of s_sleep(2) before falling back

constexpr int kSampleCap = 4096;        // samples of one request the bound search keeps in LDS

// LDS: a per-wave ring of two key tiles filled by direct-to-LDS loads during
// scoring; after scoring the same bytes hold the request's samples (bound
// search) and, in the last workgroup, the candidates of the final select.
template <int NQ, int CHUNK, bool FP8>
struct IdxSmem {
  static constexpr int kTileBytes = FP8 ? 32 * 128 : 32 * 256;
  static constexpr int kRing = (kIdxThreads / kWave) * 2 * kTileBytes;
  static constexpr int kReuse = kSampleCap * 4 > kCandCap * 8 ? kSampleCap * 4 : kCandCap * 8;
  static constexpr int kArena = kRing > kReuse ? kRing : kReuse;
  alignas(16) unsigned char arena[kArena];
  uint32_t keys[NQ * CHUNK];
  alignas(16) float w[NQ][64];
  float kscale[FP8 ? CHUNK : 1];
  int pages[CHUNK / 64];
  uint32_t hist[256];
  uint32_t cbase[kMaxChunksPerSeq + 1];
  uint32_t sel[2];
  uint32_t scan[16];
  uint32_t flag[4];
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

template <int NQ, int CHUNK, bool FP8>
__global__ __launch_bounds__(kIdxThreads) void li_decode_kernel(const IdxDecodeArgs a) {
  __shared__ IdxSmem<NQ, CHUNK, FP8> sm;
  uint32_t* s_keys = sm.keys;                                  // [NQ][CHUNK]
  uint32_t* s_smp = reinterpret_cast<uint32_t*>(sm.arena);     // [kSampleCap] samples (after scoring)

  constexpr int NS = CHUNK / kSampleEvery;  // samples per chunk (CHUNK/kRun runs of kRun/kSampleEvery)
  constexpr int NT = CHUNK / 32;            // 32-position tiles per chunk
  constexpr int NW = kIdxThreads / kWave;
  static_assert(NT % NW == 0, "tiles must split evenly over waves");
  constexpr int RUNS = CHUNK / (NW * kRun);  // sorted runs per wave
  static_assert(RUNS * NW * kRun == CHUNK, "the chunk splits into whole runs per wave");

  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 31, half = lane >> 5;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int n_chunks = max(1, (L + CHUNK - 1) / CHUNK);
  if (c >= n_chunks) return;
  const int t0 = b * NQ;
  const int s0 = c * CHUNK;
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- stage q, w, page ids
  for (int i = tid; i < NQ * 64; i += kIdxThreads) sm.w[i / 64][i % 64] = a.w[(size_t)(t0 + i / 64) * 64 + i % 64];
  for (int i = tid; i < CHUNK / 64; i += kIdxThreads) {
    const int lp = s0 / 64 + i;
    const int pg = lp < a.max_pages ? bt[lp] : 0;  // in bounds whatever L is: no wait on seq_lens first
    sm.pages[i] = lp * 64 < L ? min(max(pg, 0), a.num_pages - 1) : 0;
  }
  if constexpr (FP8) {
    __syncthreads();
    for (int i = tid; i < CHUNK; i += kIdxThreads)
      sm.kscale[i] = s0 + i < L ? a.k_scales[(size_t)sm.pages[i >> 6] * 64 + (i & 63)] : 0.f;
  }

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
  __syncthreads();

  int vis[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) vis[j] = max(0, L - NQ + j + 1);

  // ---------------------------------------------------------------- score
  // Wave w scores tiles w, w+NW, ... (32 positions each, inside one page).
  // Tiles are moved by direct-to-LDS loads into a two-slot ring private to
  // the wave.  Each DMA instruction reads one contiguous kilobyte of the tile
  // (eight lanes per 128-byte line) and writes lane l's 16 bytes to slot
  // 64i + l; inside a line the 16-byte chunks are XOR-swizzled by (row & 7),
  // so the MFMA operand reads (row n, fixed column) hit distinct banks.
  // Tiles past the end of the request copy a valid (clamped) tile and are
  // masked afterwards.
  constexpr int TB = IdxSmem<NQ, CHUNK, FP8>::kTileBytes;
  constexpr int DMA_PER_TILE = TB / 1024;
  constexpr int NIT = NT / NW;
  constexpr int ROW = FP8 ? 128 : 256;             // bytes per key row
  constexpr int RPI = 1024 / ROW;                  // rows per DMA instruction
  unsigned char* ring = sm.arena + wid * 2 * TB;
  auto tile_pos0 = [&](int it) { return s0 + (wid + NW * it) * 32; };
  // this lane's share of every DMA instruction: row (within the instruction)
  // and the 16-byte chunk of that row
  const int dma_row = lane / (64 / RPI);
  const int dma_line = FP8 ? 0 : (lane >> 3) & 1;
  auto issue = [&](int it) {
    const int pos0 = tile_pos0(it);
    const int lp = max(min(pos0, L - 1) - s0, 0);  // position inside the chunk, clamped
    const char* base =
        static_cast<const char*>(a.k) + ((size_t)sm.pages[lp >> 6] * 64 + (lp & 32)) * ROW;
    unsigned char* dst = ring + (it & 1) * TB;
#pragma unroll
    for (int i = 0; i < DMA_PER_TILE; ++i) {
      const int row = RPI * i + dma_row;
      const int col = 8 * dma_line + ((lane & 7) ^ (row & 7));
      __builtin_amdgcn_global_load_lds(base + row * ROW + 16 * col, (lds_void*)(dst + 1024 * i), 16, 0, 0);
    }
  };
  // LDS byte offset of (row, 16-byte chunk) inside a tile
  auto slot = [&](int row, int col) {
    return 1024 * (row / RPI) + 16 * ((64 / RPI) * (row % RPI) + 8 * (col >> 3) + ((col & 7) ^ (row & 7)));
  };

  auto compute = [&](int it) {
    const int tile = wid + NW * it;
    const int pos0 = s0 + tile * 32;
    const unsigned char* src = ring + (it & 1) * TB;
    f32x16 acc[NQ * 2];
#pragma unroll
    for (int mt = 0; mt < NQ * 2; ++mt) acc[mt] = (f32x16){};
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // k-step j: row n, bytes 128 half + 16 j = chunk 8 half + j
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(src + slot(n, 8 * half + j));
#pragma unroll
        for (int mt = 0; mt < NQ * 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt].v[j], kb, acc[mt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // k-step j: row n, bytes 64 j + 16 half (chunk 4j + half) and 64 j + 32 + 16 half
        const i32x4 lo = *reinterpret_cast<const i32x4*>(src + slot(n, 4 * j + half));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(src + slot(n, 4 * j + 2 + half));
        const i32x8 kb = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int mt = 0; mt < NQ * 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt].v[j], kb, acc[mt], 0, 0, 0,
                                                                   qa[mt].scale[j], 0, 127);
      }
    }
    const float kscale = FP8 ? sm.kscale[min(tile * 32 + n, CHUNK - 1)] : 1.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float part = 0.f;
#pragma unroll
      for (int mh = 0; mh < 2; ++mh) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // output rows 8g+4*half+0..3 of this 32-head tile: four consecutive heads
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(&sm.w[j][32 * mh + 8 * g + 4 * half]);
#pragma unroll
          for (int i = 0; i < 4; ++i) part += w4[i] * fmaxf(acc[2 * j + mh][4 * g + i], 0.f);
        }
      }
      part += __shfl_xor(part, 32, kWave);
      if constexpr (FP8) part *= kscale;  // positive per-row scale commutes with ReLU
      if (half == 0) {
        const int s = pos0 + n;
        s_keys[j * CHUNK + tile * 32 + n] = (s < vis[j]) ? score_key(part) : 0u;
      }
    }
  };

  issue(0);
  if (NIT > 1) issue(1);
#pragma unroll 1
  for (int it = 0; it < NIT; ++it) {
    // tile it has landed once at most the next tile's loads are outstanding
    if (it + 1 < NIT) SLI_WAIT_VMCNT(DMA_PER_TILE);
    else SLI_WAIT_VMCNT(0);
    compute(it);
    if (it + 2 < NIT) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this slot's reads are done
      issue(it + 2);
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- samples
  // Wave w sorts runs w, w+NW, ... (kRun consecutive keys each) in registers
  // and publishes, per run, the keys at descending ranks 16i-1, i = 1..16:
  // each certifies that the run holds >= 16i keys >= it.
  const size_t ncm = (size_t)a.n_chunks_max;
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
#pragma unroll 1
    for (int r0 = 0; r0 < RUNS; ++r0) {
      const int run = wid + NW * r0;
      uint32_t v[kRun / kWave];
#pragma unroll
      for (int r = 0; r < kRun / kWave; ++r) v[r] = s_keys[j * CHUNK + kRun * run + (kRun / kWave) * lane + r];
      wave_bitonic_sort_desc<kRun / kWave>(v);
      // rank e = 4*lane + r; samples at e = 16i - 1, i.e. lanes 4i+3, register 3
      uint32_t* smp = a.samples + ((size_t)(t0 + j) * ncm + c) * NS + (kRun / kSampleEvery) * run;
      if ((lane & 3) == 3) xstore(&smp[lane >> 2], v[3]);
    }
  }
  wait_vmem();
  __syncthreads();
  // Publish: the block barrier orders every thread's sample stores before
  // thread 0's agent-scope release; the wait polls with relaxed loads and
  // acquires once.  One fence pair per workgroup, not per thread or per poll.
  uint32_t* ctr = a.counters + (size_t)b * kCounterStride;
  if (tid == 0) {
    fence_release_agent();
    atomic_add_acq_rel(&ctr[0], 1u);
    unsigned spins = 0, timed_out = 0;
    while (atomic_load_relaxed(&ctr[0]) < (uint32_t)n_chunks) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinMax) {
        timed_out = 1;
        break;
      }
    }
    fence_acquire_agent();
    if (timed_out) atomic_add_acq_rel(&ctr[2], 1u);
    sm.flag[0] = timed_out;
  }
  __syncthreads();
  const bool timed_out = sm.flag[0] != 0;

  // ---------------------------------------------------------------- lower bound and emission
  const int m_need = (a.top_k + kSampleEvery - 1) / kSampleEvery;
  constexpr int PER = CHUNK / kIdxThreads;
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    uint32_t tau = 1u;
    const int n_samples = n_chunks * NS;
    if (!timed_out && m_need <= n_samples) {
      const uint32_t* smp = a.samples + (size_t)(t0 + j) * ncm * NS;
      int ngt;
      if (n_samples <= kSampleCap) {
        // all loads in flight at once (a loop with one load per trip would
        // pay the memory latency once per trip)
        constexpr int PERS = kSampleCap / kIdxThreads;
        uint32_t sv[PERS];
#pragma unroll
        for (int r = 0; r < PERS; ++r) {
          const int i = tid + r * kIdxThreads;
          sv[r] = i < n_samples ? xload(&smp[i]) : 0u;
        }
#pragma unroll
        for (int r = 0; r < PERS; ++r) {
          const int i = tid + r * kIdxThreads;
          if (i < n_samples) s_smp[i] = sv[r];
        }
        __syncthreads();
        tau = block_radix_select<kSampleCap / kIdxThreads>([&](int i) { return s_smp[i]; }, n_samples, m_need, sm.hist,
                                                           sm.sel, ngt);
      } else {
        tau = block_radix_select_big([&](int i) { return xload(&smp[i]); }, n_samples, m_need, sm.hist, sm.sel, ngt);
      }
      tau = max(tau, 1u);
    }
    uint32_t kk[PER];
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      kk[i] = s_keys[j * CHUNK + tid * PER + i];
      cnt += kk[i] >= tau ? 1u : 0u;
    }
    uint32_t total;
    uint32_t off = block_excl_scan(cnt, sm.scan, total);
    const size_t region = ((size_t)(t0 + j) * ncm + c) * CHUNK;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (kk[i] >= tau) {
        xstore(&a.cand_key[region + off], kk[i]);
        xstore(&a.cand_pos[region + off], s0 + tid * PER + i);
        ++off;
      }
    }
    if (tid == 0) xstore(&a.cand_cnt[(size_t)(t0 + j) * ncm + c], total);
    __syncthreads();  // s_smp is reused by the next token's bound search
  }
  wait_vmem();
  __syncthreads();
  if (tid == 0) {
    fence_release_agent();
    const bool last = atomic_add_acq_rel(&ctr[1], 1u) == (uint32_t)n_chunks - 1;
    if (last) fence_acquire_agent();
    sm.flag[1] = last ? 1u : 0u;
  }
  __syncthreads();
  if (!sm.flag[1]) return;

  // ---------------------------------------------------------------- exact select (last workgroup)
  uint32_t* s_ck = reinterpret_cast<uint32_t*>(sm.arena);  // [kCandCap] (the key ring is free now)
  int* s_cp = reinterpret_cast<int*>(s_ck + kCandCap);       // [kCandCap]
  const int K = a.top_k;
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    const size_t tok = (size_t)(t0 + j);
    uint32_t cc = tid < n_chunks ? xload(&a.cand_cnt[tok * ncm + tid]) : 0u;
    uint32_t N;
    uint32_t base = block_excl_scan(cc, sm.scan, N);
    if (tid < n_chunks) sm.cbase[tid] = base;
    if (tid == 0) sm.cbase[n_chunks] = N;
    __syncthreads();
    // flat candidate f -> (chunk, slot) by binary search over the prefix offsets
    // (only for the out-of-LDS fallback)
    auto locate = [&](int f) {
      int lo = 0, hi = n_chunks;  // cbase[lo] <= f < cbase[hi]
      while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if ((int)sm.cbase[mid] <= f) lo = mid; else hi = mid;
      }
      return (tok * ncm + lo) * CHUNK + (f - sm.cbase[lo]);
    };
    const bool in_lds = N <= (uint32_t)kCandCap;
    if (in_lds) {
      // Chunk by chunk: thread i takes slot i (+256, ...) of each chunk's
      // region, with the loads of 8 chunks in flight at once.
      constexpr int GB = 8;
#pragma unroll 1
      for (int c0 = 0; c0 < n_chunks; c0 += GB) {
        uint32_t maxc = 0;
        for (int u = 0; u < GB && c0 + u < n_chunks; ++u) maxc = max(maxc, sm.cbase[c0 + u + 1] - sm.cbase[c0 + u]);
#pragma unroll 1
        for (uint32_t s0 = 0; s0 < maxc; s0 += kIdxThreads) {
          uint32_t kv[GB];
          int32_t pv[GB];
#pragma unroll
          for (int u = 0; u < GB; ++u) {
            const int cc2 = c0 + u;
            const uint32_t sl = s0 + tid;
            const bool ok = cc2 < n_chunks && sl < sm.cbase[min(cc2 + 1, n_chunks)] - sm.cbase[min(cc2, n_chunks)];
            const size_t ga = (tok * ncm + cc2) * CHUNK + sl;
            kv[u] = ok ? xload(&a.cand_key[ga]) : 0u;
            pv[u] = ok ? xload(&a.cand_pos[ga]) : -1;
          }
#pragma unroll
          for (int u = 0; u < GB; ++u) {
            const int cc2 = c0 + u;
            const uint32_t sl = s0 + tid;
            if (cc2 < n_chunks && sl < sm.cbase[cc2 + 1] - sm.cbase[cc2]) {
              s_ck[sm.cbase[cc2] + sl] = kv[u];
              s_cp[sm.cbase[cc2] + sl] = pv[u];
            }
          }
        }
      }
      __syncthreads();
    }
    auto key_at = [&](int f) { return in_lds ? s_ck[f] : xload(&a.cand_key[locate(f)]); };
    auto pos_at = [&](int f) { return in_lds ? s_cp[f] : xload(&a.cand_pos[locate(f)]); };

    uint32_t tau = 0u;
    int ties = 0;
    const bool take_all = N <= (uint32_t)K;
    if (!take_all) {
      int ngt;
      tau = in_lds ? block_radix_select<kCandCap / kIdxThreads>(key_at, (int)N, K, sm.hist, sm.sel, ngt)
                   : block_radix_select_big(key_at, (int)N, K, sm.hist, sm.sel, ngt);
      ties = K - ngt;
    }
    int32_t* out = a.idx_out + tok * K;
    uint32_t written;
    if (in_lds) {
      // In position order, 256 candidates per round: wave ballots rank the
      // ties at tau and then the selected candidates inside each wave, and
      // per-wave counts (double-buffered by round parity) rank the waves.
      const int wid_ = tid >> 6;
      constexpr int NWV = kIdxThreads / kWave;
      uint32_t base = 0, ties_before = 0;
      for (int f0 = 0, rnd = 0; f0 < (int)N; f0 += kIdxThreads, ++rnd) {
        const int f = f0 + tid;
        const uint32_t key = f < (int)N ? s_ck[f] : 0u;
        const bool gt = f < (int)N && (take_all || key > tau);
        const bool tie = f < (int)N && !take_all && key == tau;
        uint32_t* cnts = sm.scan + 8 * (rnd & 1);
        const uint64_t mt = __ballot(tie);
        if (lane == 0) cnts[wid_] = (uint32_t)__popcll(mt);
        __syncthreads();
        uint32_t tb = 0, tt = 0;
        for (int w2 = 0; w2 < NWV; ++w2) {
          const uint32_t x = cnts[w2];
          tb += w2 < wid_ ? x : 0u;
          tt += x;
        }
        const uint32_t tie_rank =
            ties_before + tb + __builtin_amdgcn_mbcnt_hi((uint32_t)(mt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mt, 0u));
        const bool sel = gt || (tie && tie_rank < (uint32_t)ties);
        const uint64_t m = __ballot(sel);
        if (lane == 0) cnts[NWV + wid_] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t before = 0, tot = 0;
        for (int w2 = 0; w2 < NWV; ++w2) {
          const uint32_t x = cnts[NWV + w2];
          before += w2 < wid_ ? x : 0u;
          tot += x;
        }
        if (sel) {
          const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          out[base + before + r] = s_cp[f];
        }
        base += tot;
        ties_before += tt;
      }
      written = base;
    } else {
      // Each thread walks a contiguous segment of the (position-ordered)
      // candidates: one scan ranks the ties at tau, one places the selected.
      const int seg = ((int)N + kIdxThreads - 1) / kIdxThreads;
      const int f_lo = min((int)N, tid * seg), f_hi = min((int)N, f_lo + seg);
      uint32_t my_ties = 0;
      if (!take_all)
        for (int f = f_lo; f < f_hi; ++f) my_ties += key_at(f) == tau ? 1u : 0u;
      uint32_t tie_tot;
      uint32_t tie_rank = block_excl_scan(my_ties, sm.scan, tie_tot);
      uint32_t my_sel = 0;
      {
        uint32_t tr = tie_rank;
        for (int f = f_lo; f < f_hi; ++f) {
          const uint32_t key = key_at(f);
          const bool tie = !take_all && key == tau;
          my_sel += (take_all || key > tau || (tie && tr < (uint32_t)ties)) ? 1u : 0u;
          tr += tie ? 1u : 0u;
        }
      }
      uint32_t o = block_excl_scan(my_sel, sm.scan, written);
      {
        uint32_t tr = tie_rank;
        for (int f = f_lo; f < f_hi; ++f) {
          const uint32_t key = key_at(f);
          const bool tie = !take_all && key == tau;
          if (take_all || key > tau || (tie && tr < (uint32_t)ties)) out[o++] = pos_at(f);
          tr += tie ? 1u : 0u;
        }
      }
    }
    for (int i = (int)written + tid; i < K; i += kIdxThreads) out[i] = -1;
    __syncthreads();
  }
  if (tid == 0) {
    __hip_atomic_store(&ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NQ, int CHUNK, bool FP8>
static hipError_t launch_one(const IdxDecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.n_chunks_max, a.B);
  hipLaunchKernelGGL((li_decode_kernel<NQ, CHUNK, FP8>), grid, dim3(kIdxThreads), 0, stream, a);
  return hipGetLastError();
}

// Positions per workgroup.  Larger chunks when the grid would not otherwise
// fit on the chip at once (two workgroups per CU): with every workgroup of a
// request resident, the cross-workgroup bound, the candidate exchange and the
// final select run after the streaming instead of under its memory latency.
int idx_decode_chunk(int B, int n_q, int max_pages, int cus) {
  (void)n_q;
  const long long maxlen = (long long)max_pages * 64;
  const long long wgs1k = (long long)B * ((maxlen + 1023) / 1024);
  return wgs1k > 2LL * cus ? 2048 : 1024;
}

hipError_t launch_idx_decode(const IdxDecodeArgs& a, int chunk, bool fp8, hipStream_t stream) {
  if (chunk == 1024) {
    if (a.n_q == 1) return fp8 ? launch_one<1, 1024, true>(a, stream) : launch_one<1, 1024, false>(a, stream);
    if (a.n_q == 2) return fp8 ? launch_one<2, 1024, true>(a, stream) : launch_one<2, 1024, false>(a, stream);
  } else if (chunk == 2048) {
    if (a.n_q == 1) return fp8 ? launch_one<1, 2048, true>(a, stream) : launch_one<1, 2048, false>(a, stream);
    if (a.n_q == 2) return fp8 ? launch_one<2, 2048, true>(a, stream) : launch_one<2, 2048, false>(a, stream);
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
