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
// streams every key position any of them can see.  Each query is handled by
// a pair of waves, one per half of the 64 indexer heads (MFMA rows), and the
// 8 waves share each 32-position key tile: it is moved once into an LDS ring
// by direct-to-LDS loads (one 1 KiB instruction per wave), so key traffic
// from L2 is divided by the number of queries in flight.  Workgroups on the
// same XCD stream the same positions at about the same time and share them
// through L2; query blocks are scheduled heaviest (latest) first.
//
// Exact streaming Top-K per query, kept entirely in LDS: positions arrive in
// increasing order; a position is appended to the query's candidate buffer
// (key, position) if its key beats the running threshold.  When the buffer
// nears capacity one wave compacts it to exactly the current top K (register
// radix select, ties to the lower -- earlier -- position) and the threshold
// becomes that K-th key, compared strictly from then on: a later position
// with an equal key ranks behind every kept one.  The buffer therefore always
// holds the top K of the positions seen so far plus later contenders, in
// position order; a final compaction writes the indices.  Scores never leave
// the chip.
#include "device_common.h"
#include "launch.h"

namespace sli {

typedef __attribute__((address_space(3))) void lds_void;
#define SLI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N)&15) | (((N) >> 4) << 14) | 0x70 | 0xF00)

constexpr int kPfQueries = 4;             // queries per workgroup
constexpr int kPfWaves = 2 * kPfQueries;  // one wave per (query, head half)
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfCap = 3072;              // candidate slots per query
constexpr int kPfRing = 3;                // key tiles in flight + in use

struct PfSmem {
  alignas(16) unsigned char ring[kPfRing][8192];  // 32 positions x 256 bytes
  uint32_t key[kPfQueries][kPfCap];
  int32_t pos[kPfQueries][kPfCap];
  float xsum[2][kPfQueries][2][32];  // per-head-half partial scores of a tile
  alignas(16) float w[kPfQueries][64];
  uint32_t hist[kPfQueries][256];
  int count[kPfQueries];
  uint32_t tau[kPfQueries];
  int strict[kPfQueries];
  int pages[kMaxPrefillPages];
};

// LDS byte offset of (row, 16-byte chunk) inside a 32 x 256-byte key tile
// written by 8 direct-to-LDS loads of one kilobyte each (four rows per load,
// chunk position XOR-swizzled by row & 7).
__device__ __forceinline__ int pf_slot(int row, int col) {
  return 1024 * (row >> 2) + 16 * (16 * (row & 3) + 8 * (col >> 3) + ((col & 7) ^ (row & 7)));
}

// Wave-level exact selection over the query's buffer: finds the k-th largest
// key (ties to the lower index), keeps exactly min(k, n) entries in order and
// returns the new count; tau = the k-th key when n > k.
__device__ int pf_compact(uint32_t* key, int32_t* pos, int n, int k, uint32_t* hist, uint32_t& tau, bool& cut) {
  const int lane = threadIdx.x & (kWave - 1);
  if (n <= k) {
    cut = false;
    return n;
  }
  // --- radix select of the k-th largest key over key[0..n) (wave-local)
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = lane; i < n; i += kWave) {
    lo = min(lo, key[i]);
    hi = max(hi, key[i]);
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
      for (int i = lane; i < 256; i += kWave) hist[i] = 0;
      __builtin_amdgcn_s_waitcnt(0xC07F);
      for (int i = lane; i < n; i += kWave) {
        const uint32_t v = key[i];
        if ((v & above) == prefix) atomicAdd(&hist[(v >> shift) & ((1u << width) - 1u)], 1u);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = hist[255 - 4 * lane - i];
      const uint32_t sum = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
      uint32_t dsel = 0, rsel = 0;
      if (excl < remaining && remaining <= incl) {
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
      // exactly one lane found the digit
      const uint64_t who = __ballot(excl < remaining && remaining <= incl);
      const int src = __ffsll((unsigned long long)who) - 1;
      dsel = __shfl(dsel, src, kWave);
      rsel = __shfl(rsel, src, kWave);
      prefix |= dsel << shift;
      remaining = rsel;
      top = shift - 1;
    }
  }
  tau = prefix;
  const uint32_t ties = remaining;  // entries equal to tau that stay (the earliest ones)
  // --- in-order compaction to the front
  int out = 0;
  uint32_t ties_seen = 0;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    uint32_t v = 0;
    int p = 0;
    if (i < n) {
      v = key[i];
      p = pos[i];
    }
    const bool tie = i < n && v == tau;
    const uint64_t tie_mask = __ballot(tie);
    const uint32_t tie_rank = ties_seen + __builtin_amdgcn_mbcnt_hi((uint32_t)(tie_mask >> 32),
                                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)tie_mask, 0u));
    const bool keep = i < n && (v > tau || (tie && tie_rank < ties));
    const uint64_t keep_mask = __ballot(keep);
    const int slot = out + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(keep_mask >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)keep_mask, 0u));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // every lane has read its entry before any write
    if (keep) {
      key[slot] = v;
      pos[slot] = p;
    }
    out += __popcll(keep_mask);
    ties_seen += (uint32_t)__popcll(tie_mask);
  }
  cut = true;
  return out;
}

__global__ __launch_bounds__(kPfThreads) void li_prefill_kernel(const IdxPrefillArgs a) {
  __shared__ PfSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wid >> 1, part = wid & 1;  // query of this wave, head half
  const int n = lane & 31, half = lane >> 5;

  // heaviest query blocks first
  const int nqb = (a.n_q + kPfQueries - 1) / kPfQueries;
  const int item = gridDim.x - 1 - blockIdx.x;
  const int b = item / nqb, qb = item % nqb;
  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int j0 = qb * kPfQueries;
  const int nq_here = min(kPfQueries, a.n_q - j0);
  const int* bt = a.block_table + (size_t)b * a.max_pages;
  // visible positions of each query of the block; the block streams the largest
  const int vis_last = max(0, min(L, L - a.n_q + j0 + nq_here));
  const int n_tiles = (vis_last + 31) / 32;
  const int n_pages = (vis_last + 63) / 64;

  for (int i = tid; i < n_pages; i += kPfThreads) sm.pages[i] = min(max(bt[i], 0), a.num_pages - 1);
  for (int i = tid; i < kPfQueries * 64; i += kPfThreads) {
    const int qi = i / 64;
    sm.w[qi][i % 64] = qi < nq_here ? a.w[((size_t)b * a.n_q + j0 + qi) * 64 + i % 64] : 0.f;
  }
  if (tid < kPfQueries) {
    sm.count[tid] = 0;
    sm.tau[tid] = 0u;
    sm.strict[tid] = 0;
  }
  const bool q_ok = qw < nq_here;
  const int vis_q = q_ok ? max(0, min(L, L - a.n_q + j0 + qw + 1)) : 0;

  // A operands: this wave's 32 heads of its query, k-step j = d 64*half+8j .. +8
  bf16x8 qa[8];
  {
    const size_t row = ((size_t)b * a.n_q + j0 + (q_ok ? qw : 0)) * 64 + 32 * part + n;
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + row * 128 + 64 * half);
    const __bf16 keep = q_ok ? (__bf16)1.f : (__bf16)0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) qa[j] = qp[j] * keep;
  }
  __syncthreads();

  // direct-to-LDS load of tile t: wave w copies rows 4w..4w+3 (one kilobyte)
  const int dma_row = 4 * wid + (lane >> 4);
  const int dma_col = 8 * ((lane >> 3) & 1) + ((lane & 7) ^ (dma_row & 7));
  auto issue = [&](int t) {
    const int p0 = min(32 * t, max(vis_last - 1, 0));
    const size_t rowi = (size_t)sm.pages[p0 >> 6] * 64 + (p0 & 32) + dma_row;
    const char* src = static_cast<const char*>(a.k) + rowi * 256 + 16 * dma_col;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(sm.ring[t % kPfRing] + 1024 * wid), 16, 0, 0);
  };

  // the first wave of each query finalises scores of a tile and appends
  auto finish_tile = [&](int t) {
    if (part != 0 || !q_ok) return;
    const float s = sm.xsum[t & 1][qw][0][n] + sm.xsum[t & 1][qw][1][n];
    const int p = 32 * t + n;
    const uint32_t k = score_key(s);
    const uint32_t tau = sm.tau[qw];
    const bool strict = sm.strict[qw] != 0;
    const bool take = half == 0 && p < vis_q && (strict ? k > tau : k >= tau);
    const uint64_t m = __ballot(take);
    const int c = sm.count[qw];
    if (take) {
      const int slot = c + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      sm.key[qw][slot] = k;
      sm.pos[qw][slot] = p;
    }
    int cnt = c + __popcll(m);
    if (cnt > kPfCap - 32) {
      __builtin_amdgcn_s_waitcnt(0xC07F);
      uint32_t nt;
      bool cut;
      cnt = pf_compact(sm.key[qw], sm.pos[qw], cnt, a.top_k, sm.hist[qw], nt, cut);
      if (cut && lane == 0) {
        sm.tau[qw] = nt;
        sm.strict[qw] = 1;
      }
    }
    if (lane == 0) sm.count[qw] = cnt;
  };

  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
#pragma unroll 1
  for (int t = 0; t < n_tiles; ++t) {
    // tile t has landed for this wave (only tile t+1 may be in flight) and
    // its LDS writes are done; a raw barrier (no fence: a fence would also
    // wait for the prefetch) then makes both visible to every wave
    if (t + 1 < n_tiles) SLI_WAIT_VMCNT(1);
    else SLI_WAIT_VMCNT(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    if (t > 0) finish_tile(t - 1);
    const unsigned char* T = sm.ring[t % kPfRing];
    bf16x8 kb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kb[j] = *reinterpret_cast<const bf16x8*>(T + pf_slot(n, 8 * half + j));
    f32x16 acc = (f32x16){};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[j], kb[j], acc, 0, 0, 0);
    float ps = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(&sm.w[qw][32 * part + 8 * g + 4 * half]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ps += w4[i] * fmaxf(acc[4 * g + i], 0.f);
    }
    ps += __shfl_xor(ps, 32, kWave);
    if (half == 0) sm.xsum[t & 1][qw][part][n] = ps;
    if (t + 2 < n_tiles) issue(t + 2);
  }
  __syncthreads();
  if (n_tiles > 0) finish_tile(n_tiles - 1);

  // final selection and output (ascending positions, -1 padded)
  if (part == 0 && q_ok) {
    uint32_t nt;
    bool cut;
    int cnt = sm.count[qw];
    cnt = pf_compact(sm.key[qw], sm.pos[qw], cnt, a.top_k, sm.hist[qw], nt, cut);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    int32_t* out = a.idx_out + ((size_t)b * a.n_q + j0 + qw) * a.top_k;
    for (int i = lane; i < a.top_k; i += kWave) out[i] = i < cnt ? sm.pos[qw][i] : -1;
  }
}

hipError_t launch_idx_prefill(const IdxPrefillArgs& a, hipStream_t stream) {
  const int nqb = (a.n_q + kPfQueries - 1) / kPfQueries;
  hipLaunchKernelGGL(li_prefill_kernel, dim3(a.B * nqb), dim3(kPfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sli
