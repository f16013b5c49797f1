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

constexpr int kIdxThreads = 256;
constexpr int kSampleEvery = 32;
constexpr int kCandCap = 4096;          // candidates the final select keeps in LDS
constexpr unsigned kSpinMax = 20000;    // ~1 ms of s_sleep(2) before falling back

template <int NQ, int CHUNK>
struct IdxSmem {
  static constexpr int kPhaseA = (NQ * CHUNK + CHUNK) * 4;
  static constexpr int kPhaseB = kCandCap * 8;
  static constexpr int kArena = kPhaseA > kPhaseB ? kPhaseA : kPhaseB;
  alignas(16) unsigned char arena[kArena];
  alignas(16) float w[NQ][64];
  uint32_t hist[256];
  uint32_t cbase[kMaxChunksPerSeq + 1];
  uint32_t sel[2];
  uint32_t scan[8];
  uint32_t flag[4];
};

template <bool FP8>
struct KTile;  // B-operand registers of one 32-position tile

template <>
struct KTile<false> {
  bf16x8 v[8];
};
template <>
struct KTile<true> {
  i32x8 v[2];
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
  __shared__ IdxSmem<NQ, CHUNK> sm;
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(sm.arena);   // [NQ][CHUNK]
  uint32_t* s_sorted = s_keys + NQ * CHUNK;                    // [CHUNK]

  constexpr int NS = CHUNK / kSampleEvery;  // samples per chunk
  constexpr int NT = CHUNK / 32;            // 32-position tiles per chunk
  constexpr int NW = kIdxThreads / kWave;
  static_assert(NT % NW == 0, "tiles must split evenly over waves");

  const int c = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, half = lane >> 5;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int n_chunks = max(1, (L + CHUNK - 1) / CHUNK);
  if (c >= n_chunks) return;
  const int t0 = b * NQ;
  const int s0 = c * CHUNK;
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- stage q, w
  for (int i = tid; i < NQ * 64; i += kIdxThreads) sm.w[i / 64][i % 64] = a.w[(size_t)(t0 + i / 64) * 64 + i % 64];

  QOps<FP8> qa[NQ * 2];
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
  auto tile_pos0 = [&](int it) { return s0 + (wid + NW * it) * 32; };
  auto issue = [&](int it, KTile<FP8>& kt, float& kscale) {
    const int pos0 = tile_pos0(it);
    if (pos0 >= L) return;
    int page = bt[pos0 >> 6];
    page = min(max(page, 0), a.num_pages - 1);
    const size_t rowi = (size_t)page * 64 + (pos0 & 63) + n;
    if constexpr (!FP8) {
      const bf16x8* kp = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.k) + rowi * 128 + 64 * half);
#pragma unroll
      for (int j = 0; j < 8; ++j) kt.v[j] = __builtin_nontemporal_load(kp + j);
    } else {
      const uint8_t* kp = static_cast<const uint8_t*>(a.k) + rowi * 128;
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // same k-slot order as the query operand
        const i32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kp + 64 * j + 16 * half));
        const i32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kp + 64 * j + 32 + 16 * half));
        kt.v[j] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      kscale = a.k_scales[rowi];
    }
  };

  auto compute = [&](int it, const KTile<FP8>& kt, float kscale) {
    const int tile = wid + NW * it;
    const int pos0 = s0 + tile * 32;
    if (pos0 >= L) {
      if (half == 0) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) s_keys[j * CHUNK + tile * 32 + n] = 0u;
      }
      return;
    }
    f32x16 acc[NQ * 2];
#pragma unroll
    for (int mt = 0; mt < NQ * 2; ++mt) acc[mt] = (f32x16){};
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int mt = 0; mt < NQ * 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt].v[j], kt.v[j], acc[mt], 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < NQ * 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt].v[j], kt.v[j], acc[mt], 0, 0, 0,
                                                                   qa[mt].scale[j], 0, 127);
    }
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

  {
    KTile<FP8> kt0, kt1;
    float ks0 = 1.f, ks1 = 1.f;
    issue(0, kt0, ks0);
#pragma unroll
    for (int it = 0; it < NT / NW; it += 2) {
      if (it + 1 < NT / NW) issue(it + 1, kt1, ks1);
      compute(it, kt0, ks0);
      if (it + 1 < NT / NW) {
        if (it + 2 < NT / NW) issue(it + 2, kt0, ks0);
        compute(it + 1, kt1, ks1);
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- samples
  const size_t ncm = (size_t)a.n_chunks_max;
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    for (int i = tid; i < CHUNK; i += kIdxThreads) s_sorted[i] = s_keys[j * CHUNK + i];
    __syncthreads();
    lds_bitonic_sort_desc<CHUNK>(s_sorted);
    uint32_t* smp = a.samples + ((size_t)(t0 + j) * ncm + c) * NS;
    for (int i = tid; i < NS; i += kIdxThreads) smp[i] = s_sorted[kSampleEvery * (i + 1) - 1];
    __syncthreads();
  }
  uint32_t* ctr = a.counters + (size_t)b * kCounterStride;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    atomic_add_acq_rel(&ctr[0], 1u);
    unsigned spins = 0, timed_out = 0;
    while (atomic_load_acquire(&ctr[0]) < (uint32_t)n_chunks) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinMax) {
        timed_out = 1;
        break;
      }
    }
    if (timed_out) atomic_add_acq_rel(&ctr[2], 1u);
    sm.flag[0] = timed_out;
  }
  __syncthreads();
  __threadfence();
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
      tau = block_radix_select([&](int i) { return smp[i]; }, n_samples, m_need, sm.hist, sm.sel, ngt);
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
        a.cand_key[region + off] = kk[i];
        a.cand_pos[region + off] = s0 + tid * PER + i;
        ++off;
      }
    }
    if (tid == 0) a.cand_cnt[(size_t)(t0 + j) * ncm + c] = total;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) sm.flag[1] = (atomic_add_acq_rel(&ctr[1], 1u) == (uint32_t)n_chunks - 1) ? 1u : 0u;
  __syncthreads();
  if (!sm.flag[1]) return;
  __threadfence();

  // ---------------------------------------------------------------- exact select (last workgroup)
  uint32_t* s_ck = reinterpret_cast<uint32_t*>(sm.arena);  // [kCandCap]
  int* s_cp = reinterpret_cast<int*>(s_ck + kCandCap);       // [kCandCap]
  const int K = a.top_k;
#pragma unroll 1
  for (int j = 0; j < NQ; ++j) {
    const size_t tok = (size_t)(t0 + j);
    uint32_t cc = tid < n_chunks ? a.cand_cnt[tok * ncm + tid] : 0u;
    uint32_t N;
    uint32_t base = block_excl_scan(cc, sm.scan, N);
    if (tid < n_chunks) sm.cbase[tid] = base;
    if (tid == 0) sm.cbase[n_chunks] = N;
    __syncthreads();
    // flat candidate f -> (chunk, slot) by binary search over the prefix offsets
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
      for (int f = tid; f < (int)N; f += kIdxThreads) {
        size_t g = locate(f);
        s_ck[f] = a.cand_key[g];
        s_cp[f] = a.cand_pos[g];
      }
      __syncthreads();
    }
    auto key_at = [&](int f) { return in_lds ? s_ck[f] : a.cand_key[locate(f)]; };
    auto pos_at = [&](int f) { return in_lds ? s_cp[f] : a.cand_pos[locate(f)]; };

    uint32_t tau = 0u;
    int ties = 0;
    const bool take_all = N <= (uint32_t)K;
    if (!take_all) {
      int ngt;
      tau = block_radix_select(key_at, (int)N, K, sm.hist, sm.sel, ngt);
      ties = K - ngt;
    }
    int32_t* out = a.idx_out + tok * K;
    uint32_t written = 0, ties_seen = 0;
    for (int f0 = 0; f0 < (int)N; f0 += kIdxThreads) {
      const int f = f0 + tid;
      uint32_t key = 0;
      int pos = -1;
      if (f < (int)N) {
        key = key_at(f);
        pos = pos_at(f);
      }
      const bool valid = f < (int)N;
      uint32_t is_tie = (valid && !take_all && key == tau) ? 1u : 0u;
      uint32_t nt_tot;
      uint32_t tie_rank = ties_seen + block_excl_scan(is_tie, sm.scan, nt_tot);
      const bool sel = valid && (take_all || key > tau || (is_tie && tie_rank < (uint32_t)ties));
      uint32_t ns_tot;
      uint32_t o = written + block_excl_scan(sel ? 1u : 0u, sm.scan, ns_tot);
      if (sel) out[o] = pos;
      written += ns_tot;
      ties_seen += nt_tot;
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

int idx_decode_chunk(int B, int n_q, int max_pages) {
  (void)B;
  (void)n_q;
  (void)max_pages;
  return 1024;
}

hipError_t launch_idx_decode(const IdxDecodeArgs& a, int chunk, bool fp8, hipStream_t stream) {
  if (chunk != 1024) return hipErrorInvalidValue;
  if (a.n_q == 1) return fp8 ? launch_one<1, 1024, true>(a, stream) : launch_one<1, 1024, false>(a, stream);
  if (a.n_q == 2) return fp8 ? launch_one<2, 1024, true>(a, stream) : launch_one<2, 1024, false>(a, stream);
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
