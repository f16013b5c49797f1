// Sparse MLA attention over the selected latent rows (decode and prefill),
// gfx950.
//
// What it computes ("Day0 Inference Adaptation and Performance Optimization
// for a Sparse Hybrid Architecture LLM", sec. 1 and 2.1: attention reads only
// the KV of the positions the indexer selected; the branch is built on MLA,
// whose cache row is one 576-wide latent shared by every query head):
//     l_j = sm_scale * q[t,h,:] . c[idx_j,:],   p = softmax_j(l),
//     o[t,h,:] = sum_j p_j c[idx_j, 0:512],     lse[t,h] = log sum_j exp(l_j).
//
// Decomposition.  A workgroup owns one token, a block of up to 64 heads and a
// contiguous slice of the token's index row (a "split").  Each 32-head group
// is handled by a pair of waves, one per SIMD: for the logits each wave of the
// pair takes half of the 576-wide contraction (and the pair adds partials
// through LDS), for the output each takes 256 of the 512 columns, so the
// query operands (72 VGPRs) and the fp32 output accumulators (128) stay in
// registers for the whole slice.  Per 32-row tile:
//   - the selected rows are gathered into LDS: bf16 rows by direct
//     global-to-LDS loads through a three-deep ring (two tiles in flight while
//     one is consumed), FP8 rows through registers, dequantised on the way in
//     (block scale x E4M3 code);
//   - logits are computed transposed, S^T[pos, head] = C_tile . q^T, on 32x32
//     MFMA tiles.  In this layout a lane owns one head, so the running max,
//     the running sum and the rescale of the output accumulators are per-lane
//     scalars;
//   - the output is accumulated transposed as well, O^T[d, head] += C^T . P^T:
//     P^T comes straight from the S^T registers (the MFMA k-slot order is
//     chosen to match the S^T output layout) and C^T is read from the LDS tile
//     with the gfx950 transpose read ds_read_b64_tr_b16.
// When a token's index row is split over several workgroups, each writes an
// unnormalised fp32 partial and (max, sum) per head, and a combine kernel
// merges them.
#include "device_common.h"
#include "launch.h"

namespace sli {

constexpr int kTileRows = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tile layout.  A tile holds 32 rows x 72 chunks of 16 bytes (one chunk =
// 8 bf16), 36 KiB, filled by 36 wave-wide direct-to-LDS loads.  Load i copies
// one 128-byte line (chunks 8g..8g+7, g = i/4) of the eight rows 8(i%4)..+7:
// eight lanes per row, so every load reads whole cache lines.  Lane l of load
// i lands at byte 16(64i + l); inside its row the chunk is placed at
// position (chunk & 7) ^ f(row), a swizzle under which both operand reads are
// conflict-free: the logit operand read (eight rows, one chunk) and the
// transposed read (four consecutive rows, two adjacent chunks).
constexpr int kTileBytes = 36 * 1024;
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return 16 * (64 * (4 * (chunk >> 3) + (row >> 3)) + 8 * (row & 7) + ((chunk & 7) ^ swz(row)));
}

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at max).
#define SLI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N)&15) | (((N) >> 4) << 14) | 0x70 | 0xF00)

__device__ __forceinline__ void fp8x16_to_bf16(const i32x4& raw, float scale, bf16x8& lo8, bf16x8& hi8) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    auto a = __builtin_amdgcn_cvt_pk_f32_fp8(raw[i], false);  // codes 4i, 4i+1
    auto b = __builtin_amdgcn_cvt_pk_f32_fp8(raw[i], true);   // codes 4i+2, 4i+3
    bf16x8& d = i < 2 ? lo8 : hi8;
    const int o = 4 * (i & 1);
    d[o + 0] = (__bf16)(a[0] * scale);
    d[o + 1] = (__bf16)(a[1] * scale);
    d[o + 2] = (__bf16)(b[0] * scale);
    d[o + 3] = (__bf16)(b[1] * scale);
  }
}

// One workgroup = NW waves, wave w owns heads 32w .. 32w+31 of one token and
// the index slice [split*split_len, ...) of that token.  One wave per SIMD:
// the 576-wide q^T operands (144 VGPRs) and the 32x512 fp32 output
// accumulators (256 registers) stay resident for the whole slice.
template <int NHG, int WPH, bool FP8>
__global__ __launch_bounds__(NHG * WPH * 64) void sfa_kernel(const SfaArgs a) {
  constexpr int NW = NHG * WPH;     // waves
  constexpr int KS = 36 / WPH;      // 16-wide logit k-steps per wave
  constexpr int MI = 16 / WPH;      // 32-column output tiles per wave
  __shared__ __attribute__((aligned(128))) char tile0[kTileBytes];
  __shared__ __attribute__((aligned(128))) char tile1[kTileBytes];
  __shared__ __attribute__((aligned(128))) char tile2[kTileBytes];
  __shared__ int rows[kMaxSplitRows];
  __shared__ int s_fallback;
  __shared__ __attribute__((aligned(64))) f32x16 xbuf[WPH > 1 ? NHG * WPH : 1][kWave];
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, half = lane >> 5;
  // Work item (split, token, head block).  Blocks are numbered so that the
  // head blocks of one (split, token) are 8 apart: the hardware deals
  // workgroups round-robin over the 8 XCDs, so they share an L2 and the
  // second gather of each row hits it.
  const int id = blockIdx.x;
  const int hb = (id >> 3) % a.head_blocks;
  const int rest = (id / (8 * a.head_blocks)) * 8 + (id & 7);
  if (rest >= a.n_splits * a.T) return;
  const int split = rest % a.n_splits, t = rest / a.n_splits;
  const int b = t / a.n_q;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int i0 = split * a.split_len;
  const int cnt = max(0, min(a.split_len, a.top_k - i0));
  const int n_tiles = (cnt + kTileRows - 1) / kTileRows;
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- rows of this slice
  // Each batch has all of its index loads in flight at once, then all of its
  // block-table loads: two memory latencies per batch of 8 rows per thread.
  if (tid == 0) s_fallback = 0x7fffffff;
  constexpr int RPB = 8;
  const int n_rows = n_tiles * kTileRows;
  __syncthreads();  // s_fallback initialised
#pragma unroll 1
  for (int i0b = 0; i0b < n_rows; i0b += RPB * NT) {
    int pos_v[RPB], page_v[RPB];
#pragma unroll
    for (int r = 0; r < RPB; ++r) {
      const int i = i0b + tid + r * NT;
      pos_v[r] = i < cnt ? a.idx[(size_t)t * a.top_k + i0 + i] : -1;
    }
#pragma unroll
    for (int r = 0; r < RPB; ++r) page_v[r] = (pos_v[r] >= 0 && pos_v[r] < L) ? bt[pos_v[r] >> 6] : -1;
#pragma unroll
    for (int r = 0; r < RPB; ++r) {
      const int i = i0b + tid + r * NT;
      if (i < n_rows) {
        int rr = -1;
        if (pos_v[r] >= 0 && pos_v[r] < L) {
          rr = min(max(page_v[r], 0), a.num_pages - 1) * 64 + (pos_v[r] & 63);
          atomicMin(&s_fallback, rr);
        }
        rows[i] = rr;
      }
    }
  }

  // ---------------------------------------------------------------- q^T operands
  const int hg = wid / WPH, part = wid % WPH;
  const int head = 32 * (NHG * hb + hg) + n;
  const bool head_ok = head < a.H;
  bf16x8 qb[KS];
  {
    const bf16x8* qp =
        reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + ((size_t)t * a.H + (head_ok ? head : 0)) * 576);
    const __bf16 keep = head_ok ? (__bf16)1.f : (__bf16)0.f;  // padded heads get a zero query
#pragma unroll
    for (int k = 0; k < KS; ++k) qb[k] = qp[2 * (KS * part + k) + half] * keep;
  }
  __syncthreads();
  const int fallback = s_fallback;
  const bool any_valid = fallback != 0x7fffffff;

  auto bufs = [&](int i) -> char* { return i == 0 ? tile0 : (i == 1 ? tile1 : tile2); };

  // ---------------------------------------------------------------- gathers
  // BF16: wave w issues loads w, w+NW, ... of the tile; lane l copies row
  // 8(i%4) + l/8, chunk 8(i/4) + ((l & 7) ^ f(row)).
  constexpr int DMA_PER_WAVE = 36 / NW;
  auto issue_dma = [&](int tile, char* dst) {
#pragma unroll
    for (int k = 0; k < DMA_PER_WAVE; ++k) {
      const int i = wid + NW * k;
      const int row = 8 * (i & 3) + (lane >> 3);
      const int chunk = 8 * (i >> 2) + ((lane & 7) ^ swz(row));
      int pr = rows[tile * kTileRows + row];
      pr = pr >= 0 ? pr : fallback;
      const char* src = static_cast<const char*>(a.kv) + (size_t)pr * 1152 + 16 * chunk;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 1024 * i), 16, 0, 0);
    }
  };
  // FP8: codes go through registers, are scaled to bf16 and stored swizzled.
  constexpr int F8_CHUNKS = kTileRows * 36;  // 16-code chunks per tile
  constexpr int F8_PER = (F8_CHUNKS + NT - 1) / NT;
  i32x4 f8_stage[FP8 ? F8_PER : 1];
  auto load_f8 = [&](int tile) {
#pragma unroll
    for (int r = 0; r < F8_PER; ++r) {
      const int f = tid + r * NT;
      f8_stage[r] = (i32x4){0, 0, 0, 0};
      if (f < F8_CHUNKS) {
        const int row = f / 36, ch = f % 36;
        const int pr = rows[tile * kTileRows + row];
        if (pr >= 0)
          f8_stage[r] = __builtin_nontemporal_load(
              reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(a.kv) + (size_t)pr * 576) + ch);
      }
    }
  };
  auto store_f8 = [&](int tile, char* dst) {
#pragma unroll
    for (int r = 0; r < F8_PER; ++r) {
      const int f = tid + r * NT;
      if (f < F8_CHUNKS) {
        const int row = f / 36, ch = f % 36;
        const int pr = rows[tile * kTileRows + row];
        const float sc =
            pr >= 0 ? a.kv_scales[(size_t)pr * a.kv_groups + (a.kv_groups == 1 ? 0 : min(ch >> 3, 4))] : 0.f;
        bf16x8 lo8, hi8;
        fp8x16_to_bf16(f8_stage[r], sc, lo8, hi8);
        *reinterpret_cast<bf16x8*>(dst + tile_off(row, 2 * ch)) = lo8;
        *reinterpret_cast<bf16x8*>(dst + tile_off(row, 2 * ch + 1)) = hi8;
      }
    }
  };

  // ---------------------------------------------------------------- main loop
  f32x16 o[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) o[i] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.sm_scale * kLog2e;
  const int gi = lane & 15;

  const int tiles = any_valid ? n_tiles : 0;
  if constexpr (!FP8) {
    if (tiles > 0) issue_dma(0, bufs(0));
    if (tiles > 1) issue_dma(1, bufs(1));
  } else {
    if (tiles > 0) {
      load_f8(0);
      store_f8(0, bufs(0));
    }
    __syncthreads();
  }
#pragma unroll 1
  for (int tile = 0; tile < tiles; ++tile) {
    const char* T = bufs(tile % 3);
    if constexpr (!FP8) {
      if (tile + 2 < tiles) {
        issue_dma(tile + 2, bufs((tile + 2) % 3));
        SLI_WAIT_VMCNT(2 * DMA_PER_WAVE);
      } else if (tile + 1 < tiles) {
        SLI_WAIT_VMCNT(DMA_PER_WAVE);
      } else {
        SLI_WAIT_VMCNT(0);
      }
      __builtin_amdgcn_s_barrier();
    } else {
      if (tile + 1 < tiles) load_f8(tile + 1);
    }

    // logits S^T[pos, head] over this wave's share of the 576-wide contraction
    // all operand reads are issued before the MFMA chain (one wave per SIMD:
    // nothing else would hide the LDS latency)
    bf16x8 av[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) av[k] = *reinterpret_cast<const bf16x8*>(T + tile_off(n, 2 * (KS * part + k) + half));
    // bf16: two independent accumulator chains (even and odd k-steps) halve
    // the dependent MFMA latency of the logits; the FP8 variant keeps one
    // chain (its staging registers leave no room for the second)
    f32x16 s = (f32x16){};
    if constexpr (!FP8) {
      f32x16 s_odd = (f32x16){};
#pragma unroll
      for (int k = 0; k < KS; k += 2) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], qb[k], s, 0, 0, 0);
        if (k + 1 < KS) s_odd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k + 1], qb[k + 1], s_odd, 0, 0, 0);
      }
      s += s_odd;
    } else {
#pragma unroll
      for (int k = 0; k < KS; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], qb[k], s, 0, 0, 0);
    }
    if constexpr (WPH > 1) {
      xbuf[wid][lane] = s;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the partial is in LDS
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int p = 1; p < WPH; ++p) s += xbuf[hg * WPH + (part + p) % WPH][lane];
    }

    // online softmax; this lane owns head n and positions 8(v/4) + 4 half + v%4
    // valid positions of the tile as one wave-uniform mask (lanes 32..63
    // repeat lanes 0..31)
    const uint32_t vmask = (uint32_t)__ballot(rows[tile * kTileRows + n] >= 0);
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int pos = 8 * (v >> 2) + 4 * half + (v & 3);
      const float x = ((vmask >> pos) & 1u) ? s[v] * sl2 : -INFINITY;
      s[v] = x;
      mt = fmaxf(mt, x);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    // Online softmax with a lazy reference: the running reference m_run is
    // raised (and the accumulators rescaled) only when some head's tile
    // maximum exceeds it by more than 2^8; otherwise the weights exp2(x -
    // m_run) stay below 256, harmless in fp32 sums and bf16 operands.  The
    // decision is wave-uniform, so most tiles skip the rescale entirely.
    // (The FP8 single-head-group variant keeps the branch-free update: its
    // staging registers leave no room for the branch.)
    if (FP8 && NHG == 1 ? true : __ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MI; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    float rs = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = exp2f(s[v] - m_run);
      rs += p;
      pb[v >> 3][v & 7] = (__bf16)p;
    }
    l_run += rs + __shfl_xor(rs, 32, kWave);

    // O^T[d, head] += C^T[d, pos] . P^T[pos, head].  The 16-lane group of the
    // wave reads rows r0..r0+3 (and r0+8..r0+11) of columns 32mi + 16((lane>>4)&1)
    // + 0..15 (two chunks); lane gi receives one column, four consecutive rows.
    const int tr_row = 4 * half + (gi >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x4 lo[MI], hi[MI];
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int r0 = 16 * kk + tr_row, c0 = 4 * (MI * part + m) + tr_chunk;
        lo[m] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(T + tile_off(r0, c0) + 8 * (gi & 1)));
        hi[m] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(T + tile_off(r0 + 8, c0) + 8 * (gi & 1)));
      }
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const bf16x8 cv = (bf16x8){lo[m][0], lo[m][1], lo[m][2], lo[m][3], hi[m][0], hi[m][1], hi[m][2], hi[m][3]};
        o[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv, pb[kk], o[m], 0, 0, 0);
      }
    }
    if constexpr (FP8) {
      if (tile + 1 < tiles) store_f8(tile + 1, bufs((tile + 1) % 3));
      __syncthreads();
    } else {
      __builtin_amdgcn_s_barrier();
    }
  }

  // ---------------------------------------------------------------- write out
  if (!head_ok) return;
  const size_t th = (size_t)t * a.H + head;
  if (a.n_splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    __bf16* op = static_cast<__bf16*>(a.out) + th * 512;
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * (MI * part + m) + 8 * g + 4 * half;
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[m][4 * g + i] * inv);
        *reinterpret_cast<bf16x4*>(op + d) = v4;
      }
    if (a.lse && half == 0 && part == 0) a.lse[th] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  } else {
    const size_t ps = ((size_t)t * a.n_splits + split) * a.H + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    __bf16* op = a.part_o + ps * 512;
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * (MI * part + m) + 8 * g + 4 * half;
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[m][4 * g + i] * inv);
        *reinterpret_cast<bf16x4*>(op + d) = v4;
      }
    if (half == 0 && part == 0) {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 latent rows, every head of the token in one workgroup.
//
// Wave w owns heads 32w .. 32w+31 from end to end: the full 576-wide logits
// (its q^T operands, 144 VGPRs, stay resident) and all 512 output columns (16
// accumulator tiles), so the waves share only the gathered tile and each
// selected row crosses the memory system once per slice.  Tiles move through
// a four-slot LDS ring, so three tiles are in flight while one is consumed
// (logits on two independent MFMA chains, online softmax, output product).
#ifndef SLI_NO_PINS
#define SLI_PIN_V(x) asm volatile("" : "+v"(x))
#define SLI_PIN_A(x) asm volatile("" : "+a"(x))
#else
#define SLI_PIN_V(x)
#define SLI_PIN_A(x)
#endif
template <int NW>
__global__ __launch_bounds__(NW * 64) void sfa_bf16_kernel(const SfaArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KS = 36;        // 16-wide k-steps of the 576-wide logits
  constexpr int MI = 16;        // 32-column output tiles
  constexpr int PVS = 2 * MI;   // output MFMAs per tile
  constexpr int DPW = 36 / NW;  // direct-to-LDS loads per wave per tile
  constexpr int PD = 2;         // transposed-read pairs issued this many steps ahead
  constexpr int PDL = 4;        // logit operand reads issued this many steps ahead
  static_assert(36 % NW == 0, "the 36 loads of a tile are dealt evenly over the waves");
  static_assert(2 * DPW <= 63, "two tiles of loads in flight per wave");
  static_assert(DPW <= PVS, "a wave's loads of a tile fit between the output MFMAs");
  static_assert(PD <= 4 && PDL <= 4, "explicit LDS-read waits cover at most 4 steps in flight");
  // four ring slots as separate LDS objects: the compiler can then tell a read
  // of one slot from a direct-to-LDS load into another and does not make the
  // read wait for every load in flight
  __shared__ __attribute__((aligned(128))) char slot0[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot1[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot2[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot3[kTileBytes];
  __shared__ int rows[kMaxSplitRows];
  __shared__ int s_fallback;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, half = lane >> 5, gi = lane & 15;

  // Work item.  The hardware deals workgroups round-robin over the 8 XCDs
  // (id % 8); XCD x takes a contiguous range of tokens with all of their
  // splits, so the splits of a token share one L2 for the token's q (and
  // neighbouring prefill tokens, which select mostly the same rows, share it
  // for the rows).
  const int x = blockIdx.x & 7, g = blockIdx.x >> 3;
  const int tpx = (a.T + 7) / 8;
  const int t = x * tpx + g / a.n_splits;
  const int split = g % a.n_splits;
  if (t >= a.T) return;
  const int b = t / a.n_q;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int i0 = split * a.split_len;
  const int cnt = max(0, min(a.split_len, a.top_k - i0));
  const int n_tiles = (cnt + kTileRows - 1) / kTileRows;
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- rows of this slice, q^T operands
  // The index entries and then the page ids are loaded (two dependent memory
  // latencies); the q loads are issued while the page ids are in flight, so
  // they overlap with the rows' resolution and with the first tiles' loads.
  if (tid == 0) s_fallback = 0x7fffffff;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  constexpr int RPT = kMaxSplitRows / NT;  // rows per thread: one pass covers any slice
  const int n_rows = n_tiles * kTileRows;
  int pos_v[RPT], page_v[RPT];
  if (cnt > 0) {
    const int32_t* ip = a.idx + (size_t)t * a.top_k + i0;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = tid + r * NT;
      const int v = ip[min(i, cnt - 1)];
      pos_v[r] = i < cnt ? v : -1;
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const bool valid = pos_v[r] >= 0 && pos_v[r] < L;
      page_v[r] = bt[valid ? pos_v[r] >> 6 : 0];
    }
  }

  const int head = 32 * wid + n;
  const bool head_ok = head < a.H;
  bf16x8 qb[KS];
  {
    // padded heads (head >= H) run on head 0's query; nothing of theirs is stored
    const bf16x8* qp =
        reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + ((size_t)t * a.H + (head_ok ? head : 0)) * 576);
#pragma unroll
    for (int k = 0; k < KS; ++k) qb[k] = qp[2 * k + half];
  }
  // the page ids are first used here, after the q loads have been issued
#pragma unroll
  for (int r = 0; r < RPT; ++r) asm volatile("" : "+v"(page_v[r]) : : "memory");

  if (cnt > 0) {
    int fb = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = tid + r * NT;
      if (i < n_rows) {
        const bool valid = pos_v[r] >= 0 && pos_v[r] < L;
        const int rr = valid ? min(max(page_v[r], 0), a.num_pages - 1) * 64 + (pos_v[r] & 63) : -1;
        rows[i] = rr;
        if (valid) fb = min(fb, rr);
      }
    }
    if (fb != 0x7fffffff) atomicMin(&s_fallback, fb);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const int fallback = __builtin_amdgcn_readfirstlane(s_fallback);  // uniform: kept in a scalar register
  const int tiles = fallback != 0x7fffffff ? n_tiles : 0;
  // row read in place of skipped entries (and by the prologue's loads past
  // the last tile): a valid row of the slice, else the pool's first row
  const int fb_row = tiles > 0 ? fallback : 0;

  // ---------------------------------------------------------------- gathers
  // Wave w issues loads w, w+NW, ... of a tile; lane l of load i copies row
  // 8(i%4) + l/8, chunk 8(i/4) + ((l & 7) ^ f(row)).  With NW dividing 4 a
  // lane meets only 4/NW distinct rows, and f(row) depends on l alone, so
  // each load is one per-row base address plus an immediate offset.
  const int c_lane = (lane & 7) ^ swz(lane >> 3);
  auto ring = [&](int tile) -> char* {
    const int i = tile & 3;
    return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3;
  };
  constexpr int RPW = 4 / NW;
  // the row ids a lane's loads of a tile use (read ahead of the loads)
  auto tile_rows = [&](int tile, int (&pr)[4]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) pr[r] = rows[tile * kTileRows + 8 * (wid + NW * r) + (lane >> 3)];
  };
  // load k of this wave for `tile` (tile < tiles unless it is a prologue load)
  auto load_one = [&](int tile, const int (&pr)[4], int k) {
    const int i = wid + NW * k;  // (i % 4) = wid + NW (k % RPW), i / 4 = k / RPW
    const int r = RPW == 1 ? pr[0] : RPW == 2 ? ((k & 1) ? pr[1] : pr[0]) : pr[k & 3];
    const int row = (r >= 0 && tile < tiles) ? r : fb_row;
    const char* src = static_cast<const char*>(a.kv) + ((size_t)row * 72 + c_lane) * 16 + 128 * (k / RPW);
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(ring(tile) + 1024 * i), 16, 0, 0);
  };
  auto issue = [&](int tile) {
    int pr[4];
    tile_rows(tile, pr);
#pragma unroll
    for (int k = 0; k < DPW; ++k) load_one(tile, pr, k);
  };

  // ---------------------------------------------------------------- operand reads
  // Byte offsets inside a tile (tile_off with the swizzle resolved per lane):
  // logits k-step k of lane (n, half) = row n, chunk 2k + half
  //   = abase[k % 4] + 4096 (k / 4);
  // output product j (k-block kk = j / 16, column tile m = j % 16): the
  // 16-lane group reads rows r0..r0+3 and r0+8..r0+11 (r0 = 16 kk + tr_row)
  // of two adjacent chunks, lane gi receiving one column, four consecutive
  // rows per read; the low read sits at pbase[m % 2] + 4096 (m / 2) + 2048 kk
  // and the high one 1024 bytes further.
  int abase[4], pbase[2];
  {
    const int tr_row = 4 * half + (gi >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) abase[j] = 16 * (64 * (n >> 3) + 8 * (n & 7) + ((2 * j + half) ^ swz(n)));
#pragma unroll
    for (int j = 0; j < 2; ++j) pbase[j] = 16 * (8 * tr_row + ((4 * j + tr_chunk) ^ swz(tr_row))) + 8 * (gi & 1);
  }
  // The transposed reads are issued as instructions of their own: the wait
  // pass cannot tell the intrinsic's LDS read from the direct-to-LDS loads in
  // flight into other slots and would drain them all first.  Their results
  // are awaited explicitly (tr_wait) before use.
  auto lds_addr = [](const char* p) -> uint32_t { return (uint32_t)(uintptr_t)(const lds_void*)p; };
  auto pv_issue = [&](uint32_t c, int j, bf16x4& lo, bf16x4& hi) {
    const int kk = j / MI, m = j % MI;
    const uint32_t p = c + pbase[m & 1];
    switch (4096 * (m >> 1) + 2048 * kk) {
#define SLI_TR_CASE(OFF)                                                                   \
  case OFF:                                                                                \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(p), "i"(OFF));     \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(p), "i"(OFF + 1024)); \
    break;
      SLI_TR_CASE(0) SLI_TR_CASE(2048) SLI_TR_CASE(4096) SLI_TR_CASE(6144)
      SLI_TR_CASE(8192) SLI_TR_CASE(10240) SLI_TR_CASE(12288) SLI_TR_CASE(14336)
      SLI_TR_CASE(16384) SLI_TR_CASE(18432) SLI_TR_CASE(20480) SLI_TR_CASE(22528)
      SLI_TR_CASE(24576) SLI_TR_CASE(26624) SLI_TR_CASE(28672) SLI_TR_CASE(30720)
#undef SLI_TR_CASE
    }
  };

  f32x16 o[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) o[i] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.sm_scale * kLog2e;
  bf16x8 pb[2];  // P^T of the previous tile (k-blocks 0 and 1)
  pb[0] = pb[1] = (bf16x8){};

  // Online softmax of one tile's S^T, in stages that the output product of
  // the previous tile interleaves with its MFMAs.  This lane owns head n and
  // positions 8(v/4) + 4 half + v%4.  Entries past the slice or invalid were
  // gathered from a valid row of the slice, so their (finite) logits may
  // enter the maximum, which is only the reference of the exponentials; their
  // weights are zeroed.  The running reference is raised (and the
  // accumulators rescaled) only when some head's tile maximum exceeds it by
  // more than 2^8, so weights stay below 256 (harmless in fp32 sums and bf16
  // operands) and most tiles skip the rescale.
  struct Sm {
    f32x16 x;        // scaled logits
    float mt;        // tile maximum (both lane halves)
    float m_new, alpha, rs;
    bool need;       // the reference moves (wave-uniform)
    bf16x8 p[2];     // weights, the next output product's B operands
  } sm;
  // the two lane halves hold the same head: combine across them
  auto halves = [](float v, bool is_max) -> float {
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return is_max ? fmaxf(a, b) : a + b;
  };
  auto sm_stage = [&](int st, const f32x16& sv) {
    if (st == 0) {
#pragma unroll
      for (int v = 0; v < 8; ++v) sm.x[v] = sv[v] * sl2;
    } else if (st == 1) {
#pragma unroll
      for (int v = 8; v < 16; ++v) sm.x[v] = sv[v] * sl2;
    } else if (st == 2) {
      float m = fmaxf(fmaxf(sm.x[0], sm.x[1]), fmaxf(sm.x[2], sm.x[3]));
#pragma unroll
      for (int v = 4; v < 16; v += 2) m = fmaxf(m, fmaxf(sm.x[v], sm.x[v + 1]));
      sm.mt = m;
    } else if (st == 3) {
      sm.mt = halves(sm.mt, true);
      sm.need = __ballot(sm.mt > m_run + 8.f) != 0;
      sm.m_new = sm.need ? fmaxf(m_run, sm.mt) : m_run;
      sm.alpha = __builtin_amdgcn_exp2f(m_run - sm.m_new);
      sm.rs = 0.f;
    } else if (st >= 4 && st < 12) {
      const int v = 2 * (st - 4);
      const float p0 = __builtin_amdgcn_exp2f(sm.x[v] - sm.m_new);
      const float p1 = __builtin_amdgcn_exp2f(sm.x[v + 1] - sm.m_new);
      sm.rs += p0 + p1;
      sm.p[v >> 3][v & 7] = (__bf16)p0;
      sm.p[v >> 3][(v & 7) + 1] = (__bf16)p1;
    }
  };
  constexpr int SM_STAGES = 12;
  // finishes the tile's softmax once the previous output product is done:
  // zero the weights of invalid entries (rare), rescale, fold the sum
  auto sm_finish = [&](uint32_t vmask) {
    if (vmask != 0xffffffffu) {
      float rs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int pos = 8 * (v >> 2) + 4 * half + (v & 3);
        const float p = ((vmask >> pos) & 1u) ? (float)sm.p[v >> 3][v & 7] : 0.f;
        sm.p[v >> 3][v & 7] = (__bf16)p;
        rs += p;
      }
      sm.rs = rs;
    }
    if (sm.need) {
      if (__ballot(m_run > -1e29f) != 0) {  // accumulators hold something
        // (the accumulators stay in the accumulation registers around the
        // scaling; without the pins the allocator moves them and spills q)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          asm volatile("" : "+a"(o[i]));
          o[i] *= sm.alpha;
          asm volatile("" : "+a"(o[i]));
        }
      }
      l_run *= sm.alpha;
      m_run = sm.m_new;
    }
    l_run += halves(sm.rs, false);
    pb[0] = sm.p[0];
    pb[1] = sm.p[1];
  };

  // logits S^T[pos, head] of one tile (one accumulator chain: a second one
  // would not fit beside q and the output accumulators).  The operand reads
  // are instructions of their own, like the transposed reads below.
  auto av_issue = [&](uint32_t c, int k, bf16x8& v) {
    const uint32_t p = c + abase[k & 3];
    switch (4096 * (k >> 2)) {
#define SLI_AV_CASE(OFF)                                                            \
  case OFF:                                                                         \
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(p), "i"(OFF));      \
    break;
      SLI_AV_CASE(0) SLI_AV_CASE(4096) SLI_AV_CASE(8192) SLI_AV_CASE(12288) SLI_AV_CASE(16384)
      SLI_AV_CASE(20480) SLI_AV_CASE(24576) SLI_AV_CASE(28672) SLI_AV_CASE(32768)
#undef SLI_AV_CASE
    }
  };
  // The next tile's loads are spread over the chain (one every KS / DPW
  // steps), so a load whose issue stalls on a full memory queue does so
  // while MFMAs are in flight.
  auto logits = [&](const char* C, int ld_tile, const int (&pr)[4]) -> f32x16 {
    const uint32_t c = lds_addr(C);
    bf16x8 av[KS];
    f32x16 s0 = (f32x16){};
#pragma unroll
    for (int k = 0; k < PDL; ++k) av_issue(c, k, av[k]);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
#ifdef SLI_LOADS_IN_LOGITS
      if (k % (KS / DPW) == 0 && ld_tile < tiles) load_one(ld_tile, pr, k / (KS / DPW));
#endif
      if (k + PDL < KS) av_issue(c, k + PDL, av[k + PDL]);
      switch (min(PDL, KS - 1 - k)) {
#define SLI_AV_WAIT(N)                                                              \
  case N:                                                                           \
    asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(av[k]));                         \
    break;
        SLI_AV_WAIT(0) SLI_AV_WAIT(1) SLI_AV_WAIT(2) SLI_AV_WAIT(3) SLI_AV_WAIT(4)
#undef SLI_AV_WAIT
      }
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], qb[k], s0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return s0;
  };
  // output product O^T[d, head] += C^T[d, pos] . P^T[pos, head] of the
  // previous tile (do_pv), with the current tile's softmax stages (do_sm)
  // interleaved between its MFMAs
  auto outprod = [&](const char* C, bool do_pv, const f32x16& sv, bool do_sm, int ld_tile, const int (&pr)[4]) {
    const uint32_t c = lds_addr(C);
    int kld = 0;
    bf16x4 lo[PVS], hi[PVS];
    if (do_pv) {
#pragma unroll
      for (int j = 0; j < PD; ++j) pv_issue(c, j, lo[j], hi[j]);
    }
#pragma unroll
    for (int j = 0; j < PVS; ++j) {
      if (do_pv) {
        if (j + PD < PVS) pv_issue(c, j + PD, lo[j + PD], hi[j + PD]);
        // reads issued after step j's pair: 2 per later step in flight
        switch (2 * min(PD, PVS - 1 - j)) {
#define SLI_TR_WAIT(N)                                                                     \
  case N:                                                                                  \
    asm volatile("s_waitcnt lgkmcnt(" #N ")" : "+v"(lo[j]), "+v"(hi[j]));                   \
    break;
          SLI_TR_WAIT(0) SLI_TR_WAIT(2) SLI_TR_WAIT(4) SLI_TR_WAIT(6) SLI_TR_WAIT(8)
#undef SLI_TR_WAIT
        }
        const bf16x8 cv = (bf16x8){lo[j][0], lo[j][1], lo[j][2], lo[j][3], hi[j][0], hi[j][1], hi[j][2], hi[j][3]};
        o[j % MI] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv, pb[j / MI], o[j % MI], 0, 0, 0);
        SLI_PIN_A(o[j % MI]);
      }
      if (do_sm && j % 2 == 1 && j / 2 < SM_STAGES) sm_stage(j / 2, sv);
#ifndef SLI_LOADS_IN_LOGITS
      // The next tile's loads go between these independent MFMAs, and the
      // waves take turns (wave w from step (PVS / NW) w on): the CU accepts
      // one direct-to-LDS load every ~15 cycles, so loads issued by all waves
      // at once would keep each of them waiting for the others'.
      if (ld_tile < tiles && ((j - (PVS / NW) * wid) & (PVS - 1)) < DPW) {
        load_one(ld_tile, pr, kld);  // (kld counts this wave's loads of the tile)
        ++kld;
      }
#endif
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---------------------------------------------------------------- main loop
  // Iteration t: wait for tile t, load tile t + 2 into the slot of tile t - 2,
  // logits of tile t, then the output product of tile t - 1 with tile t's
  // softmax interleaved.  Two tiles are in flight while two are consumed.
  // The prologue always issues tiles 0 and 1 (past the last tile with the
  // fallback row), so the count is exact: waiting for all but those loads
  // completes the q loads issued before them, and the loop needs no wait for q.
  issue(0);
  issue(1);
  SLI_WAIT_VMCNT(2 * DPW);
  // row ids of the tile loaded next, and the valid-entry mask of the tile
  // consumed next, both read one iteration ahead
  int pr_next[4] = {0, 0, 0, 0};
  if (2 < tiles) tile_rows(2, pr_next);
  uint32_t vmask = tiles > 0 ? (uint32_t)__ballot(rows[n] >= 0) : 0u;
  auto step = [&](int tile, bool prev) {
    if (tile + 1 < tiles) {
      SLI_WAIT_VMCNT(DPW);
    } else {
      SLI_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    const int pr[4] = {pr_next[0], pr_next[1], pr_next[2], pr_next[3]};
    const f32x16 sv = logits(ring(tile), tile + 2, pr);
    if (tile + 3 < tiles) tile_rows(tile + 3, pr_next);
    const uint32_t vm_next = tile + 1 < tiles ? (uint32_t)__ballot(rows[(tile + 1) * kTileRows + n] >= 0) : 0u;
    outprod(ring(tile - 1), prev, sv, true, tile + 2, pr);
    sm_finish(vmask);
    vmask = vm_next;
  };
  if (tiles > 0) step(0, false);
#pragma unroll 1
  for (int tile = 1; tile < tiles; ++tile) step(tile, true);
  if (tiles > 0) outprod(ring(tiles - 1), true, (f32x16){}, false, tiles, pr_next);

  // ---------------------------------------------------------------- write out
  // The wave's O^T tile (32 heads x 512) is staged in LDS (its own ring slot,
  // rows padded to 1040 bytes) so that each global store writes one whole
  // 1 KiB head row.
  SLI_WAIT_VMCNT(0);  // (prologue loads past the last tile included)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();  // every wave is done with the last tile
  constexpr int kStageRow = 1040;
  char* stage = ring(wid);
  {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int m = 0; m < MI; ++m)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * m + 8 * q4 + 4 * half;
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[m][4 * q4 + i] * inv);
        *reinterpret_cast<bf16x4*>(stage + n * kStageRow + 2 * d) = v4;
      }
  }
  const size_t th = (size_t)t * a.H + head;
  const size_t ps = ((size_t)t * a.n_splits + split) * a.H + head;
  if (head_ok && half == 0) {
    if (a.n_splits == 1) {
      if (a.lse) a.lse[th] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    } else {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_run;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const int rows_out = min(32, a.H - 32 * wid);
  __bf16* obase = a.n_splits == 1 ? static_cast<__bf16*>(a.out) + ((size_t)t * a.H + 32 * wid) * 512
                                  : a.part_o + (((size_t)t * a.n_splits + split) * a.H + 32 * wid) * 512;
#pragma unroll 4
  for (int r = 0; r < rows_out; ++r) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(stage + r * kStageRow + 16 * lane);
    *reinterpret_cast<i32x4*>(obase + (size_t)r * 512 + 8 * lane) = v;
  }
}

// Merges the split partials of one (token, head).  Split s holds its output
// normalised by its own sum, O_s, with (m_s, l_s); with w_s = 2^(m_s - M) l_s,
// o = sum_s w_s O_s / sum_s w_s.  A workgroup takes 4 heads of a token, 64
// threads per head, 8 columns (16 bytes) per thread.  Splits are taken 8 at a
// time with every load of the group in flight at once (one memory latency
// per group); a later group rescales the running sums to its larger maximum.
__global__ __launch_bounds__(256) void sfa_combine_kernel(const SfaArgs a) {
  constexpr int G = 8;
  const int t = blockIdx.y, h = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (h >= a.H) return;
  const int S = a.n_splits;
  const size_t row0 = (size_t)t * S * a.H + h;  // (token, split 0, head); splits are H rows apart
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += G) {
    float2 ml[G];
    bf16x8 v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int s = min(s0 + i, S - 1);
      const size_t row = row0 + (size_t)s * a.H;
      ml[i] = *reinterpret_cast<const float2*>(a.part_ml + 2 * row);
      v[i] = *reinterpret_cast<const bf16x8*>(a.part_o + row * 512 + 8 * l);
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (s0 + i < S && ml[i].y > 0.f) Mg = fmaxf(Mg, ml[i].x);
    Mg = Mg == -INFINITY ? 0.f : Mg;  // nothing valid so far: every weight is 0
    const float r = exp2f(M - Mg);     // rescale of the earlier groups (0 when none)
    den *= r;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= r;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wgt = (s0 + i < S && ml[i].y > 0.f) ? exp2f(ml[i].x - Mg) * ml[i].y : 0.f;
      den += wgt;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += wgt * (float)v[i][j];
    }
    M = den > 0.f ? Mg : -INFINITY;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)(acc[j] * inv);
  *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.out) + ((size_t)t * a.H + h) * 512 + 8 * l) = r;
  if (a.lse && l == 0) a.lse[(size_t)t * a.H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

static hipError_t launch_combine(const SfaArgs& a, hipStream_t stream) {
  if (a.n_splits == 1) return hipSuccess;
  hipLaunchKernelGGL(sfa_combine_kernel, dim3((a.H + 3) / 4, a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Workgroups of up to 64 heads (one or two 32-head groups): FP8 rows, and
// bf16 rows when the token has at most 64 heads.
template <int NHG, bool FP8>
static hipError_t launch_sfa_blocks(const SfaArgs& a, hipStream_t stream) {
  const int items = a.n_splits * a.T;
  dim3 grid(((items + 7) / 8) * 8 * a.head_blocks);
  hipLaunchKernelGGL((sfa_kernel<NHG, 2, FP8>), grid, dim3(NHG * 2 * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_combine(a, stream);
}

// bf16 rows, every head of the token (up to 128) in one workgroup.
static hipError_t launch_sfa_bf16(const SfaArgs& a, hipStream_t stream) {
  dim3 grid(8 * ((a.T + 7) / 8) * a.n_splits);
  hipLaunchKernelGGL((sfa_bf16_kernel<4>), grid, dim3(4 * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_combine(a, stream);
}

int sfa_heads_per_block(int H, bool fp8) { return (fp8 || H <= 64) ? (H <= 32 ? 32 : 64) : 128; }

hipError_t launch_sfa(const SfaArgs& a, bool fp8, hipStream_t stream) {
  if (fp8) return a.H <= 32 ? launch_sfa_blocks<1, true>(a, stream) : launch_sfa_blocks<2, true>(a, stream);
  if (a.H <= 32) return launch_sfa_blocks<1, false>(a, stream);
  if (a.H <= 64) return launch_sfa_blocks<2, false>(a, stream);
  return launch_sfa_bf16(a, stream);
}

}  // namespace sli
