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
// Tokens with 65 to 128 heads run the all-heads kernels (sfa_bf16_kernel,
// sfa_f8_kernel: the body in sfa_bf16_body.h, one workgroup per token and
// split holding every head, so each selected row is gathered once per
// split).  Up to 64 heads run the generic kernel below.
//
// Decomposition.  A workgroup owns one token, a block of up to 64 heads and a
// contiguous slice of the token's index row (a "split").  Each 32-head group
// is handled by WPH waves: for the logits each takes 1/WPH of the 576-wide
// contraction (the group's waves add partials through LDS), for the output
// 512/WPH of the columns, so its share of the query operands and of the fp32
// output accumulators stays in registers for the whole slice.  bf16 rows use
// two waves per group (one per SIMD, 72 + 128 registers); FP8 rows four (two
// per SIMD, 36 + 64 registers), whose second wave on each SIMD covers the
// dequantisation and the exposed gather latency of the first.  Per 32-row tile:
//   - the selected rows are gathered into LDS: bf16 rows by direct
//     global-to-LDS loads through a three-deep ring (two tiles in flight while
//     one is consumed), FP8 rows through registers (codes and block scales
//     of the next tile loaded while the current one is consumed), dequantised
//     on the way in (block scale x E4M3 code);
//   - logits are computed transposed, S^T[pos, head] = C_tile . q^T, on 32x32
//     MFMA tiles.  In this layout a lane owns one head, so the running max,
//     the running sum and the rescale of the output accumulators are per-lane
//     scalars;
//   - the output is accumulated transposed as well, O^T[d, head] += C^T . P^T:
//     P^T comes straight from the S^T registers (the MFMA k-slot order is
//     chosen to match the S^T output layout) and C^T is read from the LDS tile
//     with the gfx950 transpose read ds_read_b64_tr_b16.
// When a token's index row is split over several workgroups, each writes its
// output normalised by its own sum (bf16) and (max in log2 units, sum) per
// head, and a combine kernel merges them.
#include "sfa_bf16_body.h"

namespace sli {

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
template <int NHG, int WPH, bool FP8, bool ROPE16 = false>
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
  // A row is 36 16-byte units of codes (576 bytes), or with ROPE16 32 units
  // of latent codes followed by 8 units of bf16 rope (640 bytes), the rope
  // units landing unchanged in tile chunks 64..71.
  constexpr int F8_UNITS = ROPE16 ? 40 : 36;
  constexpr int F8_ROW = 16 * F8_UNITS;
  constexpr int F8_CHUNKS = kTileRows * F8_UNITS;  // 16-byte units per tile
  constexpr int F8_PER = (F8_CHUNKS + NT - 1) / NT;
  i32x4 f8_stage[FP8 ? F8_PER : 1];
  float f8_sc[FP8 ? F8_PER : 1];  // block scale of each staged unit, loaded with it
  auto load_f8 = [&](int tile) {
#pragma unroll
    for (int r = 0; r < F8_PER; ++r) {
      const int f = tid + r * NT;
      f8_stage[r] = (i32x4){0, 0, 0, 0};
      f8_sc[r] = 0.f;
      if (f < F8_CHUNKS) {
        const int row = f / F8_UNITS, ch = f % F8_UNITS;
        const int pr = rows[tile * kTileRows + row];
        if (pr >= 0) {
          f8_stage[r] = __builtin_nontemporal_load(
              reinterpret_cast<const i32x4*>(static_cast<const uint8_t*>(a.kv) + (size_t)pr * F8_ROW) + ch);
          if (!(ROPE16 && ch >= 32))
            f8_sc[r] = a.kv_scales[(size_t)pr * a.kv_groups + (a.kv_groups == 1 ? 0 : min(ch >> 3, 4))];
        }
      }
    }
  };
  auto store_f8 = [&](int tile, char* dst) {
#pragma unroll
    for (int r = 0; r < F8_PER; ++r) {
      const int f = tid + r * NT;
      if (f < F8_CHUNKS) {
        const int row = f / F8_UNITS, ch = f % F8_UNITS;
        if (ROPE16 && ch >= 32) {  // eight bf16 rope elements (zero for a skipped entry)
          *reinterpret_cast<i32x4*>(dst + tile_off(row, 32 + ch)) = f8_stage[r];
          continue;
        }
        bf16x8 lo8, hi8;
        fp8x16_to_bf16(f8_stage[r], f8_sc[r], lo8, hi8);
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
  // the two lane halves hold the same head: combine across them with one
  // lane swap (no LDS round trip, as a shuffle would take); the exponentials
  // are the hardware's, and the tile's valid-row mask is read a tile ahead
  // (FP8 two-token workload 427.2 -> 392.1 us, mixed-length 123.3 -> 112.8 us;
  // identical outputs)
  auto halves = [](float v, bool is_max) -> float {
    float x = v, y = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
    return is_max ? fmaxf(x, y) : x + y;
  };
  uint32_t vm_cur = tiles > 0 ? (uint32_t)__ballot(rows[n] >= 0) : 0u;
#pragma unroll 1
  for (int tile = 0; tile < tiles; ++tile) {
    const char* T = bufs(tile % 3);
    const uint32_t vm_next = tile + 1 < tiles ? (uint32_t)__ballot(rows[(tile + 1) * kTileRows + n] >= 0) : 0u;
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
    // the dependent MFMA latency of the logits; the FP8 variant (four waves
    // per group, nine k-steps each) measured no faster with two and keeps one
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
    // repeat lanes 0..31), read one tile ahead
    const uint32_t vmask = vm_cur;
    float mt = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int pos = 8 * (v >> 2) + 4 * half + (v & 3);
      const float x = ((vmask >> pos) & 1u) ? s[v] * sl2 : -INFINITY;
      s[v] = x;
      mt = fmaxf(mt, x);
    }
    mt = halves(mt, true);
    // Online softmax with a lazy reference: the running reference m_run is
    // raised (and the accumulators rescaled) only when some head's tile
    // maximum exceeds it by more than 2^8; otherwise the weights exp2(x -
    // m_run) stay below 256, harmless in fp32 sums and bf16 operands.  The
    // decision is wave-uniform, so most tiles skip the rescale entirely.
    if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MI; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    float rs = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(s[v] - m_run);
      rs += p;
      pb[v >> 3][v & 7] = (__bf16)p;
    }
    l_run += halves(rs, false);

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
    vm_cur = vm_next;
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

// Merges the split partials of every (token, head) (sfa_merge_head).
__global__ __launch_bounds__(256) void sfa_combine_kernel(const SfaArgs a) {
  const int t = blockIdx.y, h = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (h >= a.H) return;
  sfa_merge_head<false>(a, t, h, l, a.n_splits);
}

static hipError_t launch_combine(const SfaArgs& a, hipStream_t stream) {
  if (a.n_splits == 1) return hipSuccess;
  hipLaunchKernelGGL(sfa_combine_kernel, dim3((a.H + 3) / 4, a.T), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Workgroups of up to 64 heads (one or two 32-head groups): FP8 rows (four
// waves per group), and bf16 rows when the token has at most 64 heads (two).
template <int NHG, bool FP8, bool ROPE16 = false>
static hipError_t launch_sfa_blocks(const SfaArgs& a, hipStream_t stream) {
  const int items = a.n_splits * a.T;
  dim3 grid(((items + 7) / 8) * 8 * a.head_blocks);
  constexpr int WPH = FP8 ? 4 : 2;
  hipLaunchKernelGGL((sfa_kernel<NHG, WPH, FP8, ROPE16>), grid, dim3(NHG * WPH * 64), 0, stream, a);
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

// FP8 latent rows (E4M3 codes with block scales apart; R16: with the rope in
// bf16), every head of the token in one workgroup: the same body and block
// layout, with three bf16 slots that the waves fill by converting their own
// gathered rows.
template <bool R16>
__global__ __launch_bounds__(256) void sfa_f8_kernel(const SfaArgs a) {
  __shared__ __attribute__((aligned(128))) char slot0[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot1[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot2[kTileBytes];
  __shared__ __attribute__((aligned(128))) char raw[4 * kF8Wave];
  __shared__ __attribute__((aligned(128))) char raw_sc[4 * 256];
  __shared__ __attribute__((aligned(128))) char qsave[4 * kF8QLds * 1024];
  __shared__ __attribute__((aligned(128))) char pbuf[4 * 2 * 64 * 16];
  __shared__ int rows[kMaxSplitRows];
  const int x = blockIdx.x & 7, g = blockIdx.x >> 3;
  const int tpx = (a.T + 7) / 8;
  const int t = x * tpx + g / a.n_splits;
  const int split = g % a.n_splits;
  if (t >= a.T) return;
  sfa_bf16_body<4, kMaxSplitRows, false, true, R16>(
      a, SfaBf16Lds{slot0, slot1, slot2, nullptr, pbuf, rows, raw, raw_sc, qsave}, t, split);
}

// FP8 rows (576 bytes, or 640 with a bf16 rope), every head of the token
// (65 to 128) in one workgroup.
template <bool R16>
static hipError_t launch_sfa_f8(const SfaArgs& a, hipStream_t stream) {
  dim3 grid(8 * ((a.T + 7) / 8) * a.n_splits);
  hipLaunchKernelGGL((sfa_f8_kernel<R16>), grid, dim3(4 * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  return e != hipSuccess ? e : launch_combine(a, stream);
}

hipError_t launch_sfa(const SfaArgs& a, bool fp8, hipStream_t stream) {
  if (fp8 && a.H > 64) return a.rope_bf16 ? launch_sfa_f8<true>(a, stream) : launch_sfa_f8<false>(a, stream);
  if (fp8 && a.rope_bf16)
    return a.H <= 32 ? launch_sfa_blocks<1, true, true>(a, stream) : launch_sfa_blocks<2, true, true>(a, stream);
  if (fp8) return a.H <= 32 ? launch_sfa_blocks<1, true>(a, stream) : launch_sfa_blocks<2, true>(a, stream);
  if (a.H <= 32) return launch_sfa_blocks<1, false>(a, stream);
  if (a.H <= 64) return launch_sfa_blocks<2, false>(a, stream);
  return launch_sfa_bf16(a, stream);
}

}  // namespace sli
