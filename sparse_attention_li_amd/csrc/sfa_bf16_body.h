// Sparse MLA attention over bf16 latent rows, or FP8 rows of 576 bytes
// (E4M3 codes with block scales, converted to bf16 in LDS), every head (up
// to 128) of a token in one four-wave workgroup: the device body shared by
// the attention launches (sfa.hip) and the single-launch decode step
// (decode_step.hip).  What it computes and the split merge are described in
// sfa.hip.
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace sli {

constexpr int kTileRows = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

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

// ---------------------------------------------------------------------------
// bf16 latent rows, every head of the token in one workgroup.
//
// Wave w computes the full 576-wide logits and the online softmax of heads
// 32w .. 32w+31 (its q^T operands, 144 VGPRs, stay resident), and the output
// of all the heads for latent columns 128w .. 128w+127 (16 accumulator tiles):
// a wave reads a quarter of each tile transposed, instead of all of it, and
// the softmax weights of every head reach every wave through an 8 KiB LDS
// buffer, laid out as the output MFMA's operand registers.  Each selected row
// crosses the memory system once per slice.  Tiles move through a four-slot
// LDS ring: two tiles are in flight while two are consumed (the logits of one,
// the output product of the one before).
// Read schedule of the bf16 kernel's output product (32 MFMAs per tile and
// wave; MFMA j uses k-block kk = j / 16, column tile mm = (j / 4) % 4 and head
// block hb = j % 4, i.e. transposed pair pi = 4 kk + mm and weights
// P(kk, hb)).  LDS reads in issue order: P(0, 0..3), pairs 0 .. A-1; pair
// pi + A just before the first MFMA of pair pi; P(1, hb) just after the last
// MFMA that uses P(0, hb).  LDS reads of one wave complete in order, so MFMA
// j waits until no more than issued - needed of them are outstanding.
// reads issued before MFMA j's wait (its own pair issue included)
__host__ __device__ constexpr int sfa_pv_issued(int ahead, int j) {
  int cnt = 4 + 2 * ahead;
  for (int i = 0; i <= j; ++i) {
    const int kk = i >> 4, mm = (i >> 2) & 3, pi = 4 * kk + mm;
    if ((i & 3) == 0 && pi + ahead < 8) cnt += 2;
    if (i < j && kk == 0 && mm == 3) cnt += 1;
  }
  return cnt;
}
// one past the issue index of the last read MFMA j needs
__host__ __device__ constexpr int sfa_pv_needed(int ahead, int j) {
  const int kk = j >> 4, mm = (j >> 2) & 3, hb = j & 3, pi = 4 * kk + mm;
  const int p_at = kk == 0 ? hb : sfa_pv_issued(ahead, 12 + hb);
  const int pair_last = pi < ahead ? 5 + 2 * pi : sfa_pv_issued(ahead, 4 * (pi - ahead)) - 1;
  return (p_at > pair_last ? p_at : pair_last) + 1;
}
__host__ __device__ constexpr int sfa_pv_outstanding(int ahead, int j) {
  return sfa_pv_issued(ahead, j) - sfa_pv_needed(ahead, j);
}
__host__ __device__ constexpr bool sfa_pv_schedule_ok(int ahead) {
  for (int j = 0; j < 32; ++j) {
    const int w = sfa_pv_outstanding(ahead, j);
    if (w < 0 || w > 8) return false;
  }
  return sfa_pv_outstanding(ahead, 31) == 0;  // everything awaited by the last MFMA
}
constexpr int kPvAhead = 1;  // transposed pairs read ahead of their first MFMA
static_assert(sfa_pv_schedule_ok(1) && sfa_pv_schedule_ok(2), "output-product read schedule");

// keep a value in a vector / an accumulation register across the statement
#define SLI_PIN_V(x) asm volatile("" : "+v"(x))
#define SLI_PIN_A(x) asm volatile("" : "+a"(x))
// LDS of the all-heads body: four ring slots of one tile each (the targets
// of the direct-to-LDS gathers; no C++ access may touch a slot while loads
// into any slot are in flight), the weights buffer and the slice's row ids.
// FP8 rows use three bf16 slots (slot3 unused) and a raw slot: the codes of
// the next tile (4 x kF8Wave bytes) and their block scales (4 x 256 bytes).
struct SfaBf16Lds {
  char* slot0;
  char* slot1;
  char* slot2;
  char* slot3;
  char* pbuf;  // 4 * 2 * 64 * 16 bytes
  int* rows;   // ROWS entries
  char* raw = nullptr;
  char* raw_sc = nullptr;
  char* qsave = nullptr;  // FP8: the first kF8QLds k-steps' q operands (4 x kF8QLds x 1 KiB)
};
constexpr int kF8Wave = 5 * 1024;  // raw bytes per wave: its 8 rows x 576 (4.5 KiB) + padding
constexpr int kF8QLds = 3;         // q operands the FP8 logits read from LDS (registers for the conversion)

// Schedule of the dequantisation that the FP8 variant interleaves with the
// 36 logit MFMAs (steps 0..35) of the current tile.  Unit j (of five per
// lane) is converted and stored a quarter (8 bytes of bf16) per step at
// steps 1 + 7j .. 4 + 7j.  Its codes, block
// scale and the pool row of the same unit of the tile after next are read
// at step 7j - 3 (before step 0 for unit 0; the row of the scale gather with
// unit 4) and awaited at step 7j; its gather of the tile after next goes out
// at step 7j + 1, into the bytes just read, and the scale gather at step 29,
// after the last scale read.  DS operations in issue order: before step 0
// unit 0's three reads, the reads of the first kF8QLds k-steps' q operands
// (kept in LDS: their registers hold the conversion) and the first PDL logit
// operand reads; at step s the
// operand read of k-step s + PDL, then a unit's reads, then the step's store.
// Each step's wait leaves in flight only operations issued after everything
// that step and the next one use.
__host__ __device__ constexpr bool sfa_f8_store_at(int s) { return s >= 1 && (s - 1) % 7 < 4 && (s - 1) / 7 < 5; }
__host__ __device__ constexpr bool sfa_f8_read_at(int s) { return s >= 4 && (s + 3) % 7 == 0 && (s + 3) / 7 <= 4; }
__host__ __device__ constexpr int sfa_f8_reads_at(int s) { return sfa_f8_read_at(s) ? ((s + 3) / 7 == 4 ? 4 : 3) : 0; }
__host__ __device__ constexpr int sfa_f8_ops_at(int pdl, int s) {
  return (s + pdl < 36 ? 1 : 0) + sfa_f8_reads_at(s) + (sfa_f8_store_at(s) ? 1 : 0);
}
__host__ __device__ constexpr int sfa_f8_ops_before(int pdl, int s) {
  int n = 3 + kF8QLds + pdl;
  for (int i = 0; i < s; ++i) n += sfa_f8_ops_at(pdl, i);
  return n;
}
// position of the last operation the wait at step k must see completed
__host__ __device__ constexpr int sfa_f8_need(int pdl, int k) {
  int need = k < pdl ? 3 + kF8QLds + k : sfa_f8_ops_before(pdl, k - pdl);  // logit operand k
  if (k >= 7 && k <= 28 && k % 7 == 0) {  // unit k / 7: its reads at step k - 3
    const int idx = sfa_f8_ops_before(pdl, k - 3) + (k - 3 + pdl < 36 ? 1 : 0) + sfa_f8_reads_at(k - 3) - 1;
    need = need > idx ? need : idx;
  }
  return need;
}
__host__ __device__ constexpr int sfa_f8_outstanding(int pdl, int k) {
  return sfa_f8_ops_before(pdl, k + 1) - sfa_f8_need(pdl, k) - 1;
}
__host__ __device__ constexpr bool sfa_f8_schedule_ok(int pdl) {
  for (int k = 0; k < 36; ++k) {
    const int w = sfa_f8_outstanding(pdl, k);
    if (w < 0 || w > 15) return false;
  }
  return true;
}

// This lane's q^T operands of the logits (all 36 k-steps): wave w holds heads
// 32w .. 32w+31, lane (n, half) head 32w + n, k-step k its 8 elements
// 16k + 8 half .. +7.  Padded heads (head >= H) run on head 0's query;
// nothing of theirs is stored.
__device__ __forceinline__ void sfa_load_q(const SfaArgs& a, const int t, bf16x8 (&qb)[36]) {
  const int lane = threadIdx.x & 63, head = 32 * (threadIdx.x >> 6) + (lane & 31), half = lane >> 5;
  const bf16x8* qp =
      reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + ((size_t)t * a.H + (head < a.H ? head : 0)) * 576);
#pragma unroll
  for (int k = 0; k < 36; ++k) qb[k] = qp[2 * k + half];
}

// Token t, index-row slice `split` (ROWS >= the slice's rows rounded up to
// whole tiles).  FUSED (the single-launch step): the caller has written the
// pool rows to attend, own_cnt of them (all valid), into lds.rows, and has
// loaded this lane's q^T operands (sfa_load_q) into qpre; with `direct` the
// result is the token's output, else the partial of slot `split`, written
// through to memory for the workgroup that merges it.
template <int NW, int ROWS, bool FUSED, bool F8 = false, bool R16 = false>
__device__ __forceinline__ void sfa_bf16_body(const SfaArgs& a, const SfaBf16Lds& lds, const int t, const int split,
                                              const int own_cnt = 0, const bool direct = false,
                                              const bf16x8* qpre = nullptr) {
  constexpr int NT = NW * 64;
  constexpr int KS = 36;        // 16-wide k-steps of the 576-wide logits
  constexpr int MI = 16;        // 32-column output tiles
  constexpr int PVS = 2 * MI;   // output MFMAs per tile
  constexpr int DPW = 36 / NW;  // direct-to-LDS loads per wave per tile
  constexpr int PDL = 4;        // logit operand reads issued this many steps ahead
  static_assert(36 % NW == 0, "the 36 loads of a tile are dealt evenly over the waves");
  static_assert(2 * DPW <= 63, "two tiles of loads in flight per wave");
  static_assert(3 * DPW <= PVS, "a wave's loads of a tile fit between the output MFMAs");
  static_assert(PDL <= 4, "explicit LDS-read waits cover at most 4 steps in flight");
  static_assert(NW == 4, "four head blocks and four column quarters");
  static_assert(ROWS % NT == 0, "row ids resolved in whole passes");
  static_assert(!(F8 && FUSED), "FP8 rows only in the attention launch");
  static_assert(!F8 || sfa_f8_schedule_ok(PDL), "dequantisation schedule");
  char* const slot0 = lds.slot0;
  char* const slot1 = lds.slot1;
  char* const slot2 = lds.slot2;
  char* const slot3 = lds.slot3;
  char* const pbuf = lds.pbuf;
  int* const rows = lds.rows;
  // The last 4 KiB of a slot hold the tile's rope columns, read only by the
  // logits; once every wave is past them they carry the tile's softmax
  // rescale factors (128 floats at +0, one flag per head block at +512).  The
  // prologue's minimum row sits there in the last slot (no tile has been
  // loaded yet).
  constexpr int kRope = 32768;
  int* const s_fallback = reinterpret_cast<int*>((F8 ? slot2 : slot3) + kRope);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 31, half = lane >> 5, gi = lane & 15;
  const int b = t / a.n_q;

  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_pages * 64));
  const int i0 = split * a.split_len;
  const int cnt = FUSED ? own_cnt : max(0, min(a.split_len, a.top_k - i0));
  const int n_tiles = (cnt + kTileRows - 1) / kTileRows;
  const bool whole = FUSED ? direct : a.n_splits == 1;  // the result is the output itself
  const int* bt = a.block_table + (size_t)b * a.max_pages;

  // ---------------------------------------------------------------- rows of this slice, q^T operands
  // The index entries and then the page ids are loaded (two dependent memory
  // latencies); the q loads are issued while the page ids are in flight, so
  // they overlap with the rows' resolution and with the first tiles' loads.
  if (tid == 0) *s_fallback = FUSED && cnt > 0 ? rows[0] : 0x7fffffff;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  constexpr int RPT = ROWS / NT;  // rows per thread: one pass covers any slice
  const int n_rows = n_tiles * kTileRows;
  int pos_v[RPT], page_v[RPT];
  if (FUSED) {
    // rows already resolved by the caller: only the last tile's tail is skipped
    if (tid < n_rows - cnt) rows[cnt + tid] = -1;
  } else if (cnt > 0) {
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
  if constexpr (FUSED) {
#pragma unroll
    for (int k = 0; k < KS; ++k) qb[k] = qpre[k];
  } else {
    sfa_load_q(a, t, qb);
  }
  // the page ids are first used here, after the q loads have been issued
  if (!FUSED) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) asm volatile("" : "+v"(page_v[r]) : : "memory");
  }

  if (!FUSED && cnt > 0) {
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
    if (fb != 0x7fffffff) atomicMin(s_fallback, fb);
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  const int fallback = __builtin_amdgcn_readfirstlane(*s_fallback);  // uniform: kept in a scalar register
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
    if constexpr (F8) {
      const int i = tile % 3;
      return i == 0 ? slot0 : i == 1 ? slot1 : slot2;
    }
    const int i = tile & 3;
    return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3;
  };
  constexpr int RPW = 4 / NW;
  // the row ids a lane's loads of a tile use (read ahead of the loads)
  auto tile_rows = [&](int tile, int (&pr)[4]) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) pr[r] = rows[tile * kTileRows + 8 * (wid + NW * r) + (lane >> 3)];
  };
  // With four waves a lane copies one row per tile (tile < tiles unless it
  // is a prologue load): the lane's address is its row's start plus its
  // chunk plus load k's 128-byte step.  (64-bit addresses: a pool may exceed
  // the 4 GiB a buffer resource spans.  The step is added to the address, not
  // given as the instruction's offset, which would move the LDS destination
  // too.)
  static_assert(RPW == 1, "one row per lane and tile");
  const uint32_t c16 = 16 * c_lane;
  const int wid_s = __builtin_amdgcn_readfirstlane(wid);
  auto tile_row = [&](int tile, const int (&pr)[4]) -> int { return (pr[0] >= 0 && tile < tiles) ? pr[0] : fb_row; };
  auto row_src = [&](int row) -> const char* { return static_cast<const char*>(a.kv) + (size_t)row * 1152 + c16; };
  // load k of this wave into the tile at dst (= its slot + 1 KiB x wave)
  auto load_one = [&](char* dst, const char* src, int k) {
    __builtin_amdgcn_global_load_lds(src + 128 * k, (lds_void*)(dst + 1024 * NW * k), 16, 0, 0);
  };
  auto issue = [&](int tile) {
    int pr[4];
    tile_rows(tile, pr);
    const char* src = row_src(tile_row(tile, pr));
    char* dst = ring(tile) + 1024 * wid_s;
#pragma unroll
    for (int k = 0; k < DPW; ++k) load_one(dst, src, k);
  };

  // FP8 rows: 576 bytes = 36 16-byte units of E4M3 codes (512 latent, 64
  // rope), with kv_groups f32 block scales per row kept apart; with R16, 640
  // bytes = 32 units of latent codes + 8 units of bf16 rope (copied as they
  // are).  Wave w gathers its own rows 8w .. 8w+7 of a tile (lane l,
  // h = l / 32, c = l % 32: loads j = 0..3 take latent unit c of row h + 2j,
  // load 4 rope unit 32 + l % 4 of row (l % 32) / 4, its upper lanes fetching
  // the lower lanes' units again into padding; with R16 rope unit 32 + l % 8
  // of row l / 8) and their scales into its part of the raw slot,
  // and later converts exactly those bytes into the bf16 tile: a wave never
  // waits for another wave's gather, and the raw slot needs no barrier.  (The
  // mapping keeps the per-unit offsets to shifts and masks: the conversion
  // runs between dependent MFMAs, where every vector instruction counts.)
  // (the per-lane unit offsets are recomputed where used, from a lane index
  // the compiler cannot hoist: kept live across the loop they would push the
  // q operands out of registers)
  const int G = F8 ? a.kv_groups : 1;
  auto f8_lane = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // row (in the wave's eight) and 16-byte unit of this lane's load j
  auto f8_row = [](int j, int ln) -> int { return j < 4 ? (ln >> 5) + 2 * j : (R16 ? ln >> 3 : (ln & 31) >> 2); };
  auto f8_ch = [](int j, int ln) -> int { return j < 4 ? (ln & 31) : 32 + (R16 ? ln & 7 : ln & 3); };
  constexpr int F8_ROW = R16 ? 640 : 576;
  // block scale of a unit (units 32..35 are the rope codes, scale group 4;
  // a bf16 rope unit has none, and reads an unused entry)
  auto f8_group = [&](int ch) -> int { return G == 1 ? 0 : min(ch >> 3, 4); };
  // this lane's scale entry: row 8w + sl / G, group sl % G (sl = min(lane, 8G - 1), G = 1, 4 or 5)
  auto f8_sl_row = [&](int sl) -> int { return G == 1 ? sl : (G == 4 ? sl >> 2 : sl / 5); };
  auto f8_sl_grp = [&](int sl) -> int { return G == 1 ? 0 : (G == 4 ? sl & 3 : sl % 5); };
  int f8_pr[6];  // pool rows of this lane's five units and of its scale entry
  auto f8_rows = [&](int tile) {
    const int ln = f8_lane(), sl = min(ln, 8 * G - 1);
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      const int rw = j < 5 ? f8_row(j, ln) : f8_sl_row(sl);
      const int pr = tile < tiles ? rows[tile * kTileRows + 8 * wid + rw] : -1;
      f8_pr[j] = pr >= 0 ? pr : fb_row;
    }
  };
  // gather j (0..4: codes, 5: scales) of the tile whose rows f8_rows resolved
  auto f8_load = [&](int j, int ln) {
    if (j < 5) {
      const char* src = static_cast<const char*>(a.kv) + (size_t)f8_pr[j] * F8_ROW + 16 * f8_ch(j, ln);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds.raw + kF8Wave * wid_s + 1024 * j), 16, 0, 0);
    } else {
      const int sl = min(ln, 8 * G - 1);
      const float* src = a.kv_scales + (size_t)f8_pr[5] * G + f8_sl_grp(sl);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds.raw_sc + 256 * wid_s), 4, 0, 0);
    }
  };
  const uint32_t f8_raw_lane = (uint32_t)(uintptr_t)(const lds_void*)lds.raw + kF8Wave * wid + 16 * lane;
  auto f8_sc_addr = [&](int j, int ln) -> uint32_t {
    return (uint32_t)(uintptr_t)(const lds_void*)lds.raw_sc + 256 * wid +
           4 * (f8_row(j, ln) * G + f8_group(f8_ch(j, ln)));
  };
  // LDS byte offset (in a bf16 tile) of the low half of unit j; the high
  // half sits 16 bytes away (the two chunks 2 ch, 2 ch + 1 differ in the
  // lowest bit of their swizzled position).  For the latent loads this is
  // tile_off(8w + h + 2j, 2c) with the swizzle of row h + 2j written out:
  // 2h + 4 (j % 2) + j / 2, bit-disjoint from 2h's neighbours, so one XOR.
  auto f8_dst = [&](int j, int ln) -> uint32_t {
    if (j < 4) {
      const int c = ln & 31, h = ln >> 5, kj = 4 * (j & 1) + (j >> 1);
      return (uint32_t)(16 * (256 * (c >> 2) + 64 * wid + 8 * h + 16 * j + (((2 * (c & 3)) ^ (2 * h)) ^ kj)));
    }
    if constexpr (R16) return (uint32_t)tile_off(8 * wid + (ln >> 3), 64 + (ln & 7));  // one bf16 chunk
    const int l = ln & 31;
    return (uint32_t)tile_off(8 * wid + (l >> 2), 2 * (32 + (l & 3)));
  };
  // half (r % 2) of a bf16 rope unit, unchanged
  auto f8_rope_half = [](const i32x4& u, int r) -> bf16x4 {
    const uint64_t v = (uint64_t)(uint32_t)u[2 * (r & 1)] | ((uint64_t)(uint32_t)u[2 * (r & 1) + 1] << 32);
    return __builtin_bit_cast(bf16x4, v);
  };
  // four codes of a unit, scaled (block scale x E4M3 value), as bf16
  auto f8_quarter = [](int code4, float sc, bf16x4& v) {
    const auto x = __builtin_amdgcn_cvt_pk_f32_fp8(code4, false);
    const auto y = __builtin_amdgcn_cvt_pk_f32_fp8(code4, true);
    v[0] = (__bf16)(x[0] * sc);
    v[1] = (__bf16)(x[1] * sc);
    v[2] = (__bf16)(y[0] * sc);
    v[3] = (__bf16)(y[1] * sc);
  };

  // ---------------------------------------------------------------- operand reads
  // Byte offsets inside a tile (tile_off with the swizzle resolved per lane):
  // logits k-step k of lane (n, half) = row n, chunk 2k + half
  //   = (abase ^ 32 (k % 4)) + 4096 (k / 4);
  // output column tile m (32 columns) at k-block kk: the 16-lane group reads
  // rows r0..r0+3 and r0+8..r0+11 (r0 = 16 kk + tr_row) of two adjacent
  // chunks, lane gi receiving one column, four consecutive rows per read; the
  // low read sits at (pbase ^ 64 (m % 2)) + 4096 (m / 2) + 2048 kk and the
  // high one 1024 bytes further.  This wave's column tiles are
  // m = 4 wid .. 4 wid + 3.  (The swizzle only permutes chunks inside an
  // aligned group of 8 or 4, so the per-step offsets are XORs of one base;
  // slot bases are multiples of 128 and keep those bits clear.)
  int abase, pbase;
  {
    const int tr_row = 4 * half + (gi >> 2);
    const int tr_chunk = 2 * ((lane >> 4) & 1) + ((gi & 3) >> 1);
    abase = 16 * (64 * (n >> 3) + 8 * (n & 7) + (half ^ swz(n)));
    pbase = 16 * (8 * tr_row + (tr_chunk ^ swz(tr_row))) + 8 * (gi & 1);
  }
  // The LDS operand reads are issued as instructions of their own: the wait
  // pass cannot tell an LDS read from the direct-to-LDS loads in flight into
  // other slots and would drain them all first.  Their results are awaited
  // explicitly before use.
  auto lds_addr = [](const char* p) -> uint32_t { return (uint32_t)(uintptr_t)(const lds_void*)p; };
  // transposed pair of this wave's column tile mm (0..3) at k-block kk
  auto pv_issue = [&](uint32_t c, int kk, int mm, bf16x4& lo, bf16x4& hi) {
    const uint32_t p = (c + pbase) ^ (64 * (mm & 1));
    switch (4096 * (mm >> 1) + 2048 * kk) {
#define SLI_TR_CASE(OFF)                                                                   \
  case OFF:                                                                                \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(p), "i"(OFF));     \
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(p), "i"(OFF + 1024)); \
    break;
      SLI_TR_CASE(0) SLI_TR_CASE(2048) SLI_TR_CASE(4096) SLI_TR_CASE(6144)
#undef SLI_TR_CASE
    }
  };
  // P^T operand of head block hb at k-block kk (16 bytes per lane)
  const uint32_t p_lane = lds_addr(pbuf) + 16 * lane;
  auto pp_issue = [&](int kk, int hb, bf16x8& v) {
    switch (1024 * (2 * hb + kk)) {
#define SLI_PP_CASE(OFF)                                                             \
  case OFF:                                                                          \
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(p_lane), "i"(OFF)); \
    break;
      SLI_PP_CASE(0) SLI_PP_CASE(1024) SLI_PP_CASE(2048) SLI_PP_CASE(3072)
      SLI_PP_CASE(4096) SLI_PP_CASE(5120) SLI_PP_CASE(6144) SLI_PP_CASE(7168)
#undef SLI_PP_CASE
    }
  };
  // rescale of this wave's heads to publish with the weights (sm_finish)
  bool pub_need = false;
  float pub_alpha = 1.f;

  f32x16 o[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) o[i] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.sm_scale * kLog2e;
  bf16x8 pb[2];  // P^T of the previous tile (k-blocks 0 and 1)
  pb[0] = pb[1] = (bf16x8){};

  // Online softmax of one tile's S^T, in steps that the output product of
  // the previous tile interleaves with its MFMAs, one step per MFMA.  This
  // lane owns head n and positions 8(v/4) + 4 half + v%4.  Entries past the
  // slice or invalid were gathered from a valid row of the slice, so their
  // (finite) logits may enter the maximum, which is only the reference of the
  // exponentials; their weights are zeroed.  The running reference is raised
  // (and the accumulators rescaled) only when some head's tile maximum exceeds
  // it by more than 2^8, so weights stay below 256 (harmless in fp32 sums and
  // bf16 operands) and most tiles skip the rescale.
  struct Sm {
    float mt0, mt1;  // partial maxima of the tile (unscaled)
    float mt;        // tile maximum, scaled (both lane halves)
    float m_new, alpha, rs;
    bool need;       // the reference moves (wave-uniform)
    float x[16];     // exponent arguments
    float e[16];     // weights in fp32
    float s2[8];     // pair sums
    bf16x8 p[2];     // weights, the next output product's B operands
  } sm;
  // the two lane halves hold the same head: combine across them
  auto halves = [](float v, bool is_max) -> float {
    float a = v, b = v;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return is_max ? fmaxf(a, b) : a + b;
  };
  // Step j of the softmax.  The logits stay unscaled in sv: the scale (> 0)
  // is applied to the maximum and folded into the exponentials' argument.
  // A step takes at most one exponential and three other vector operations,
  // none of which uses a result of the same step: the in-order issue then
  // never holds the next MFMA behind a dependent chain, and the work fits in
  // the shadow of the MFMA before it.  Value v's argument is formed at step
  // 8 + v, its exponential at 9 + v; the weights of pair q are summed at
  // 11 + 2q, and the sum is added and the pair converted to bf16 at 12 + 2q.
  auto sm_step = [&](int j, const f32x16& sv) {
    // (each result is pinned where it is made: the compiler would otherwise
    // gather the arithmetic next to its first use, many steps later)
    if (j == 0) {
      sm.mt0 = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
      sm.mt1 = fmaxf(fmaxf(sv[3], sv[4]), sv[5]);
      SLI_PIN_V(sm.mt0);
      SLI_PIN_V(sm.mt1);
    } else if (j == 1) {
      sm.mt0 = fmaxf(fmaxf(sm.mt0, sv[6]), sv[7]);
      sm.mt1 = fmaxf(fmaxf(sm.mt1, sv[8]), sv[9]);
      SLI_PIN_V(sm.mt0);
      SLI_PIN_V(sm.mt1);
    } else if (j == 2) {
      sm.mt0 = fmaxf(fmaxf(sm.mt0, sv[10]), sv[11]);
      sm.mt1 = fmaxf(fmaxf(sm.mt1, sv[12]), sv[13]);
      SLI_PIN_V(sm.mt0);
      SLI_PIN_V(sm.mt1);
    } else if (j == 3) {
      sm.mt0 = fmaxf(fmaxf(sm.mt0, sv[14]), sv[15]);
      SLI_PIN_V(sm.mt0);
    } else if (j == 4) {
      sm.mt = fmaxf(sm.mt0, sm.mt1) * sl2;
      SLI_PIN_V(sm.mt);
    } else if (j == 5) {
      sm.mt = halves(sm.mt, true);
      SLI_PIN_V(sm.mt);
    } else if (j == 6) {
      sm.need = __ballot(sm.mt > m_run + 8.f) != 0;
      sm.m_new = sm.need ? fmaxf(m_run, sm.mt) : m_run;
      SLI_PIN_V(sm.m_new);
    } else if (j == 7) {
      sm.alpha = __builtin_amdgcn_exp2f(m_run - sm.m_new);
      sm.rs = 0.f;
      SLI_PIN_V(sm.alpha);
    }
    if (j >= 8 && j < 24) {
      sm.x[j - 8] = __builtin_fmaf(sv[j - 8], sl2, -sm.m_new);
      SLI_PIN_V(sm.x[j - 8]);
    }
    if (j >= 9 && j < 25) {
      sm.e[j - 9] = __builtin_amdgcn_exp2f(sm.x[j - 9]);
      SLI_PIN_V(sm.e[j - 9]);
    }
    if (j >= 11 && j < 26 && (j - 11) % 2 == 0) {
      const int q = (j - 11) / 2;
      sm.s2[q] = sm.e[2 * q] + sm.e[2 * q + 1];
      SLI_PIN_V(sm.s2[q]);
    }
    if (j >= 12 && j < 27 && (j - 12) % 2 == 0) {
      const int q = (j - 12) / 2, v = 2 * q;
      sm.rs += sm.s2[q];
      sm.p[v >> 3][v & 7] = (__bf16)sm.e[v];
      sm.p[v >> 3][(v & 7) + 1] = (__bf16)sm.e[v + 1];
      SLI_PIN_V(sm.rs);
      SLI_PIN_V(sm.p[v >> 3]);
    }
  };
  constexpr int SM_STEPS = 27;
  static_assert(SM_STEPS <= PVS, "the softmax steps fit between the output MFMAs");
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
    // The accumulators of this wave's heads are held by every wave: the
    // rescale factor is published with the weights and applied by each wave
    // before the tile's output product (not at all while nothing has been
    // accumulated).
    pub_need = sm.need && __ballot(m_run > -1e29f) != 0;
    pub_alpha = sm.alpha;
    if (sm.need) {
      l_run *= sm.alpha;
      m_run = sm.m_new;
    }
    l_run += halves(sm.rs, false);
    pb[0] = sm.p[0];
    pb[1] = sm.p[1];
  };

  // Writes the weights and rescale factors of `tile` (finished in registers
  // by sm_finish) where every wave reads them; the caller waits for the
  // writes and a barrier makes them visible.
  auto publish = [&](int tile) {
    const uint32_t pa = lds_addr(pbuf) + 2048 * wid + 16 * lane;
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024" : : "v"(pa), "v"(pb[0]), "v"(pb[1]) : "memory");
    const uint32_t ra = lds_addr(ring(tile)) + kRope;
    if (pub_need && half == 0)
      asm volatile("ds_write_b32 %0, %1" : : "v"(ra + 4 * (32 * wid + n)), "v"(pub_alpha) : "memory");
    if (lane == 0) asm volatile("ds_write_b32 %0, %1 offset:512" : : "v"(ra + 4 * wid), "v"(pub_need ? 1 : 0) : "memory");
  };
  // Rescales the accumulators of the head blocks whose reference moved with
  // `tile` (after the barrier that follows publish).
  auto apply_rescale = [&](int tile) {
    const uint32_t ra = lds_addr(ring(tile)) + kRope;
    i32x4 fl;
    asm volatile("ds_read_b128 %0, %1 offset:512\n\ts_waitcnt lgkmcnt(0)" : "=v"(fl) : "v"(ra) : "memory");
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      if (__builtin_amdgcn_readfirstlane(fl[hb]) != 0) {
        float al;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(al) : "v"(ra + 4 * (32 * hb + n)) : "memory");
        // (the accumulators stay in the accumulation registers around the
        // scaling; without the pins the allocator moves them and spills q)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          asm volatile("" : "+a"(o[4 * mm + hb]));
          o[4 * mm + hb] *= al;
          asm volatile("" : "+a"(o[4 * mm + hb]));
        }
      }
    }
  };

  // logits S^T[pos, head] of one tile (one accumulator chain: a second one
  // would not fit beside q and the output accumulators).  The operand reads
  // are instructions of their own, like the transposed reads below.
  auto av_issue = [&](uint32_t c, int k, bf16x8& v) {
    const uint32_t p = (c + abase) ^ (32 * (k & 3));
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
  auto logits = [&](const char* C) -> f32x16 {
    const uint32_t c = lds_addr(C);
    bf16x8 av[KS];
    f32x16 s0 = (f32x16){};
#pragma unroll
    for (int k = 0; k < PDL; ++k) av_issue(c, k, av[k]);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
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
  // FP8: the same logits, with the next tile's dequantisation into the bf16
  // slot `D` and the gathers of the tile after it (do_ld, row ids from tile
  // `ld_tile`) between the MFMAs, on the schedule described at
  // sfa_f8_schedule_ok.
  auto logits_f8 = [&](const char* C, const char* D, bool do_ld, int ld_tile) -> f32x16 {
    const uint32_t c = lds_addr(C), d = lds_addr(D);
    bf16x8 av[KS];
    i32x4 code[5];
    float sc[5];
    int rowv[6];
    bf16x4 qv;
    f32x16 s0 = (f32x16){};
    const int ln = f8_lane();
    const uint32_t raw_lane = f8_raw_lane;
    const uint32_t rbase =
        lds_addr(reinterpret_cast<const char*>(rows)) + 4 * (min(ld_tile, (ROWS / kTileRows) - 1) * kTileRows + 8 * wid);
    // row (in the wave's eight) of unit j, or of this lane's scale entry (j = 5)
    auto row_of = [&](int j) -> int {
      const int sl = min(ln, 8 * G - 1);
      return j < 5 ? f8_row(j, ln) : f8_sl_row(sl);
    };
#define SLI_F8_READS(J)                                                                             \
  do {                                                                                              \
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(code[J]) : "v"(raw_lane), "i"(1024 * (J))); \
    asm volatile("ds_read_b32 %0, %1" : "=v"(sc[J]) : "v"(f8_sc_addr(J, ln)));                      \
    asm volatile("ds_read_b32 %0, %1" : "=v"(rowv[J]) : "v"(rbase + 4 * row_of(J)));                \
    if constexpr ((J) == 4) asm volatile("ds_read_b32 %0, %1" : "=v"(rowv[5]) : "v"(rbase + 4 * row_of(5))); \
  } while (0)
    SLI_WAIT_VMCNT(0);  // this wave's gathers of the next tile are in LDS
    SLI_F8_READS(0);
    bf16x8 ql[kF8QLds];
    {
      const uint32_t qa = lds_addr(lds.qsave) + 1024 * kF8QLds * wid + 16 * ln;
      asm volatile("ds_read_b128 %0, %1" : "=v"(ql[0]) : "v"(qa));
      asm volatile("ds_read_b128 %0, %1 offset:1024" : "=v"(ql[1]) : "v"(qa));
      asm volatile("ds_read_b128 %0, %1 offset:2048" : "=v"(ql[2]) : "v"(qa));
    }
#pragma unroll
    for (int k = 0; k < PDL; ++k) av_issue(c, k, av[k]);
    static_for<KS>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k + PDL < KS) av_issue(c, k + PDL, av[k + PDL]);
      if constexpr (sfa_f8_read_at(k)) SLI_F8_READS((k + 3) / 7);
      // unit j = (k - 1) / 7: quarter r converted and stored at step 1 + 7j + r
      constexpr int j = (k - 1) / 7, r = (k - 1) % 7;
      if constexpr (k >= 1 && j < 5 && r < 4) {
        uint32_t qa;
        if constexpr (R16 && j == 4) {
          // bf16 rope: the unit's two halves as they are (written twice, so
          // that every unit takes four stores)
          qv = f8_rope_half(code[4], r);
          qa = d + f8_dst(j, ln) + 8u * (r & 1);
        } else {
          f8_quarter(code[j][r], sc[j], qv);
          qa = ((d + f8_dst(j, ln)) ^ (r >= 2 ? 16u : 0u)) + 8u * (r & 1);
        }
        asm volatile("ds_write_b64 %0, %1" : : "v"(qa), "v"(qv) : "memory");
      }
      constexpr int w = sfa_f8_outstanding(PDL, k);
      if constexpr (k == 0) {
        asm volatile("s_waitcnt lgkmcnt(%7)"
                     : "+v"(av[0]), "+v"(code[0]), "+v"(sc[0]), "+v"(rowv[0]), "+v"(ql[0]), "+v"(ql[1]), "+v"(ql[2])
                     : "i"(w));
      } else if constexpr (k == 28) {
        asm volatile("s_waitcnt lgkmcnt(%5)"
                     : "+v"(av[k]), "+v"(code[4]), "+v"(sc[4]), "+v"(rowv[4]), "+v"(rowv[5])
                     : "i"(w));
      } else if constexpr (k >= 7 && k % 7 == 0) {
        asm volatile("s_waitcnt lgkmcnt(%4)"
                     : "+v"(av[k]), "+v"(code[k / 7]), "+v"(sc[k / 7]), "+v"(rowv[k / 7])
                     : "i"(w));
      } else {
        asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(av[k]) : "i"(w));
      }
      if constexpr (k < kF8QLds) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], ql[k], s0, 0, 0, 0);
      } else {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], qb[k], s0, 0, 0, 0);
      }
      // unit j's gather of the tile after next, into the bytes just read
      if constexpr (k % 7 == 1 && k / 7 < 5) {
        if (do_ld) {
          constexpr int g = k / 7;
          f8_pr[g] = rowv[g] >= 0 ? rowv[g] : fb_row;
          f8_load(g, ln);
        }
      }
      if constexpr (k == 29) {
        if (do_ld) {
          f8_pr[5] = rowv[5] >= 0 ? rowv[5] : fb_row;
          f8_load(5, ln);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#undef SLI_F8_READS
    return s0;
  };
  // FP8 prologue: tile 0 gathered, awaited and converted in one go
  auto f8_convert_all = [&](const char* D) {
    const uint32_t d = lds_addr(D);
    const int ln = f8_lane();
    i32x4 code[5];
    float sc[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      switch (j) {
#define SLI_F8_RD(J)                                                                                  \
  case J:                                                                                             \
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(code[J]) : "v"(f8_raw_lane), "i"(1024 * J)); \
    break;
        SLI_F8_RD(0) SLI_F8_RD(1) SLI_F8_RD(2) SLI_F8_RD(3) SLI_F8_RD(4)
#undef SLI_F8_RD
      }
      asm volatile("ds_read_b32 %0, %1" : "=v"(sc[j]) : "v"(f8_sc_addr(j, ln)));
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(code[0]), "+v"(code[1]), "+v"(code[2]), "+v"(code[3]), "+v"(code[4]), "+v"(sc[0]),
                   "+v"(sc[1]), "+v"(sc[2]), "+v"(sc[3]), "+v"(sc[4]));
#pragma unroll
    for (int j = 0; j < 5; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 qv;
        uint32_t qa;
        if (R16 && j == 4) {
          qv = f8_rope_half(code[4], q);
          qa = d + f8_dst(j, ln) + 8u * (q & 1);
        } else {
          f8_quarter(code[j][q], sc[j], qv);
          qa = ((d + f8_dst(j, ln)) ^ (q >= 2 ? 16u : 0u)) + 8u * (q & 1);
        }
        asm volatile("ds_write_b64 %0, %1" : : "v"(qa), "v"(qv) : "memory");
      }
  };
  // Output product O^T[d, head] += C^T[d, pos] . P^T[pos, head] of the
  // previous tile (do_pv) for this wave's 128 columns and every head, with the
  // current tile's softmax stages (do_sm) interleaved between its MFMAs.  MFMA
  // j: k-block kk = j / 16, column tile mm = (j / 4) % 4, head block
  // hb = j % 4; the read schedule and its waits are described at
  // sfa_pv_wait.
  auto outprod = [&](const char* C, bool do_pv, const f32x16& sv, bool do_sm, int ld_tile, const int (&pr)[4]) {
    const uint32_t c = lds_addr(C) + 8192 * wid;
    const char* const ld_src = row_src(tile_row(ld_tile, pr));
    const bool do_ld = ld_tile < tiles;
    char* const ld_dst = ring(ld_tile) + 1024 * wid_s;
    bf16x4 lo[8], hi[8];
    bf16x8 pv[2][4];
    bf16x8 cv;  // the transposed pair of the current column tile, one operand
    if (do_pv) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pp_issue(0, hb, pv[0][hb]);
#pragma unroll
      for (int pi = 0; pi < kPvAhead; ++pi) pv_issue(c, 0, pi, lo[pi], hi[pi]);
    }
    static_for<PVS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int kk = j >> 4, mm = (j >> 2) & 3, hb = j & 3, pi = 4 * kk + mm;
      if (do_pv) {
        if constexpr (hb == 0 && pi + kPvAhead < 8)
          pv_issue(c, (pi + kPvAhead) >> 2, (pi + kPvAhead) & 3, lo[pi + kPvAhead], hi[pi + kPvAhead]);
        constexpr int w = sfa_pv_outstanding(kPvAhead, j);
        // The pair is awaited (and joined into one operand) by the first of
        // its four MFMAs only: a wait naming it again would make the compiler
        // assume the halves changed and copy them together before every MFMA.
        if constexpr (hb == 0) {
          asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(lo[pi]), "+v"(hi[pi]), "+v"(pv[kk][hb]) : "i"(w));
          cv = (bf16x8){lo[pi][0], lo[pi][1], lo[pi][2], lo[pi][3], hi[pi][0], hi[pi][1], hi[pi][2], hi[pi][3]};
        } else {
          asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(pv[kk][hb]) : "i"(w));
        }
        o[4 * mm + hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cv, pv[kk][hb], o[4 * mm + hb], 0, 0, 0);
        SLI_PIN_A(o[4 * mm + hb]);
        if constexpr (kk == 0 && mm == 3) pp_issue(1, hb, pv[1][hb]);
      }
      if constexpr (j < SM_STEPS) {
        if (do_sm) sm_step(j, sv);
      }
      // The next tile's loads go between these independent MFMAs, one every
      // third step (four waves then issue one about every 25 cycles, within
      // the ~15 cycles per direct-to-LDS load the CU accepts).
      if constexpr (!F8 && j % 3 == 1 && j / 3 < DPW) {
        if (do_ld) load_one(ld_dst, ld_src, j / 3);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---------------------------------------------------------------- main loop
  // Iteration t: wait for tile t, load tile t + 2 into the slot of tile t - 2,
  // logits of tile t, then the output product of tile t - 1 with tile t's
  // softmax interleaved.  Two tiles are in flight while two are consumed.
  // The prologue always issues tiles 0 and 1 (past the last tile with the
  // fallback row), so the count is exact: waiting for all but those loads
  // completes the q loads issued before them, and the loop needs no wait for q.
  // FP8: tile 0 is gathered and converted here, tile 1 gathered; iteration
  // t converts tile t + 1 (gathered during iteration t - 1) inside its logits
  // and gathers tile t + 2 there.  Three bf16 slots: the logits' tile, the
  // output product's (the one before) and the one being converted.
  if constexpr (F8) {
    if (tiles > 0) {
#pragma unroll
      for (int k = 0; k < kF8QLds; ++k)
        *reinterpret_cast<bf16x8*>(lds.qsave + 1024 * (kF8QLds * wid + k) + 16 * lane) = qb[k];
      asm volatile("" : : : "memory");  // (stored before the explicit reads of them)
      f8_rows(0);
#pragma unroll
      for (int j = 0; j < 6; ++j) f8_load(j, lane);
      SLI_WAIT_VMCNT(0);
      f8_convert_all(ring(0));
      if (tiles > 1) {
        f8_rows(1);
#pragma unroll
        for (int j = 0; j < 6; ++j) f8_load(j, lane);
      }
    }
  } else {
    issue(0);
    issue(1);
    SLI_WAIT_VMCNT(2 * DPW);
  }
  // row ids of the tile loaded next, and the valid-entry mask of the tile
  // consumed next, both read one iteration ahead
  int pr_next[4] = {0, 0, 0, 0};
  if (!F8 && 2 < tiles) tile_rows(2, pr_next);
  uint32_t vmask = tiles > 0 ? (uint32_t)__ballot(rows[n] >= 0) : 0u;
  auto step = [&](int tile, bool prev) {
    if constexpr (F8) {
    } else if (tile + 1 < tiles) {
      SLI_WAIT_VMCNT(DPW);
    } else {
      SLI_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    // every wave is past tile - 2's output product (the weights buffer is
    // free) and tile - 1's logits (its rope columns are free)
    if (prev) {
      publish(tile - 1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
      apply_rescale(tile - 1);
    }
    const int pr[4] = {pr_next[0], pr_next[1], pr_next[2], pr_next[3]};
    f32x16 sv;
    if constexpr (F8) {
      // (tile + 1 is converted even past the last tile, into a free slot, so
      // that the schedule's LDS operation count never changes)
      sv = logits_f8(ring(tile), ring(tile + 1), tile + 2 < tiles, tile + 2);
    } else {
      sv = logits(ring(tile));
      if (tile + 3 < tiles) tile_rows(tile + 3, pr_next);
    }
    const uint32_t vm_next = tile + 1 < tiles ? (uint32_t)__ballot(rows[(tile + 1) * kTileRows + n] >= 0) : 0u;
    outprod(ring(tile - 1), prev, sv, true, tile + 2, pr);
    sm_finish(vmask);
    vmask = vm_next;
  };
  if (tiles > 0) step(0, false);
#pragma unroll 1
  for (int tile = 1; tile < tiles; ++tile) step(tile, true);
  if (tiles > 0) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    publish(tiles - 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    apply_rescale(tiles - 1);
    outprod(ring(tiles - 1), true, (f32x16){}, false, tiles, pr_next);
  }

  // ---------------------------------------------------------------- write out
  // 1 / sum of every head reaches every wave through the weights buffer; the
  // output (every head, this wave's 128 columns) is staged in LDS, head block
  // hb in slot hb (rows padded to 1040 bytes), so that each global store
  // writes one whole 1 KiB head row.
  SLI_WAIT_VMCNT(0);  // (prologue loads past the last tile included)
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();  // every wave is done with the last tile and the weights
  float* const s_inv = reinterpret_cast<float*>(pbuf);
  if (half == 0) s_inv[32 * wid + n] = l_run > 0.f ? 1.f / l_run : 0.f;
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  constexpr int kStageRow = 1040;
  constexpr int NSTAGE = F8 ? 3 : NW;  // head blocks staged at once
  float inv[NW];
#pragma unroll
  for (int hb = 0; hb < NW; ++hb) inv[hb] = s_inv[32 * hb + n];
  auto stage_hb = [&](int hb, char* dst) {
#pragma unroll
    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * (4 * wid + mm) + 8 * q4 + 4 * half;
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (__bf16)(o[4 * mm + hb][4 * q4 + i] * inv[hb]);
        *reinterpret_cast<bf16x4*>(dst + n * kStageRow + 2 * d) = v4;
      }
  };
#pragma unroll
  for (int hb = 0; hb < NSTAGE; ++hb) stage_hb(hb, ring(hb));
  const size_t th = (size_t)t * a.H + head;
  const size_t ps = ((size_t)t * a.n_splits + split) * a.H + head;
  if (head_ok && half == 0) {
    if (whole) {
      if (a.lse) a.lse[th] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    } else if (FUSED) {
      xstore64(reinterpret_cast<uint64_t*>(a.part_ml + 2 * ps),
               (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_run) << 32));
    } else {
      a.part_ml[2 * ps] = m_run;
      a.part_ml[2 * ps + 1] = l_run;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();  // head block wid's rows were staged by every wave
  if constexpr (F8) {
    // head blocks 0..2 by waves 0..2, then head block 3 through slot 0
    const int hb = wid;
    const int rows_out = min(32, a.H - 32 * hb);
    __bf16* obase = whole ? static_cast<__bf16*>(a.out) + ((size_t)t * a.H + 32 * hb) * 512
                          : a.part_o + (((size_t)t * a.n_splits + split) * a.H + 32 * hb) * 512;
    if (hb < NSTAGE) {
      const char* stage = ring(hb);
#pragma unroll 4
      for (int r = 0; r < rows_out; ++r) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(stage + r * kStageRow + 16 * lane);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * 512 + 8 * lane) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();  // slot 0 read out
    stage_hb(NW - 1, ring(0));
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    if (hb == NW - 1) {
#pragma unroll 4
      for (int r = 0; r < rows_out; ++r) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(ring(0) + r * kStageRow + 16 * lane);
        *reinterpret_cast<i32x4*>(obase + (size_t)r * 512 + 8 * lane) = v;
      }
    }
    return;
  }
  const char* stage = ring(wid);
  const int rows_out = min(32, a.H - 32 * wid);
  __bf16* obase = whole ? static_cast<__bf16*>(a.out) + ((size_t)t * a.H + 32 * wid) * 512
                        : a.part_o + (((size_t)t * a.n_splits + split) * a.H + 32 * wid) * 512;
  if (FUSED && !whole) {
    // partials for the merge, written through to memory
    const uint32_t ob = (uint32_t)((obase - a.part_o) * 2);
#pragma unroll 4
    for (int r = 0; r < rows_out; ++r)
      xstore128(a.part_o, ob + (uint32_t)r * 1024u + 16u * lane,
                *reinterpret_cast<const i32x4*>(stage + r * kStageRow + 16 * lane));
    return;
  }
#pragma unroll 4
  for (int r = 0; r < rows_out; ++r) {
    const i32x4 v = *reinterpret_cast<const i32x4*>(stage + r * kStageRow + 16 * lane);
    *reinterpret_cast<i32x4*>(obase + (size_t)r * 512 + 8 * lane) = v;
  }
}

// bf16 latent rows, every head of the token in one workgroup: work item =
// (token, split) of blockIdx.  The hardware deals workgroups round-robin
// over the 8 XCDs (id % 8); XCD x takes a contiguous range of tokens with all
// of their splits, so the splits of a token share one L2 for the token's q
// (and neighbouring prefill tokens, which select mostly the same rows, share
// it for the rows).
template <int NW>
__global__ __launch_bounds__(NW * 64) void sfa_bf16_kernel(const SfaArgs a) {
  // four ring slots as separate LDS objects: the compiler can then tell a read
  // of one slot from a direct-to-LDS load into another and does not make the
  // read wait for every load in flight
  __shared__ __attribute__((aligned(128))) char slot0[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot1[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot2[kTileBytes];
  __shared__ __attribute__((aligned(128))) char slot3[kTileBytes];
  // P^T operands of one tile for every head: 16 bytes per (head block, k-block, lane)
  __shared__ __attribute__((aligned(128))) char pbuf[NW * 2 * 64 * 16];
  __shared__ int rows[kMaxSplitRows];
  const int x = blockIdx.x & 7, g = blockIdx.x >> 3;
  const int tpx = (a.T + 7) / 8;
  const int t = x * tpx + g / a.n_splits;
  const int split = g % a.n_splits;
  if (t >= a.T) return;
  sfa_bf16_body<NW, kMaxSplitRows, false>(a, SfaBf16Lds{slot0, slot1, slot2, slot3, pbuf, rows}, t, split);
}

// Merges the split partials of one (token, head).  Split s holds its output
// normalised by its own sum, O_s, with (m_s, l_s); with w_s = 2^(m_s - M) l_s,
// o = sum_s w_s O_s / sum_s w_s.  A thread takes NC groups of 8 columns of
// head h (columns 8 NC l .. 8 NC l + 8 NC - 1).  Splits are taken 8 at a time
// with every load of the group in flight at once (one memory latency per
// group); a later group rescales the running sums to its larger maximum.  The
// partials of token t sit in slots 0 .. S-1 of its a.n_splits slots.
template <bool FUSED, int NC = 1>
__device__ __forceinline__ void sfa_merge_head(const SfaArgs& a, const int t, const int h, const int l, const int S) {
  constexpr int G = 8;
  const size_t row0 = (size_t)t * a.n_splits * a.H + h;  // (token, slot 0, head); slots are H rows apart
  float M = -INFINITY, den = 0.f;
  float acc[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[c][j] = 0.f;
  for (int s0 = 0; s0 < S; s0 += G) {
    float2 ml[G];
    bf16x8 v[G][NC];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int s = min(s0 + i, S - 1);
      const size_t row = row0 + (size_t)s * a.H;
      if constexpr (FUSED) {
        const uint64_t w = xload64(reinterpret_cast<const uint64_t*>(a.part_ml + 2 * row));
        ml[i] = make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
#pragma unroll
        for (int c = 0; c < NC; ++c)
          v[i][c] = __builtin_bit_cast(bf16x8, xload128(a.part_o, (uint32_t)((row * 512 + 8 * (NC * l + c)) * 2)));
      } else {
        ml[i] = *reinterpret_cast<const float2*>(a.part_ml + 2 * row);
#pragma unroll
        for (int c = 0; c < NC; ++c) v[i][c] = *reinterpret_cast<const bf16x8*>(a.part_o + row * 512 + 8 * (NC * l + c));
      }
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (s0 + i < S && ml[i].y > 0.f) Mg = fmaxf(Mg, ml[i].x);
    Mg = Mg == -INFINITY ? 0.f : Mg;  // nothing valid so far: every weight is 0
    const float r = exp2f(M - Mg);     // rescale of the earlier groups (0 when none)
    den *= r;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[c][j] *= r;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float wgt = (s0 + i < S && ml[i].y > 0.f) ? exp2f(ml[i].x - Mg) * ml[i].y : 0.f;
      den += wgt;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[c][j] += wgt * (float)v[i][c][j];
    }
    M = den > 0.f ? Mg : -INFINITY;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)(acc[c][j] * inv);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.out) + ((size_t)t * a.H + h) * 512 + 8 * (NC * l + c)) = r;
  }
  if (a.lse && l == 0) a.lse[(size_t)t * a.H + h] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace sli
