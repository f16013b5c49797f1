// Internal interface between the host-side C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sparse_li.h"

namespace sli {

constexpr int kCounterStride = 32;     // uint32 words per request (one 128-byte line)
constexpr int kMaxSeqs = 4096;         // requests per call; sizes the fixed counter region
constexpr int kMaxChunksPerSeq = 256;  // positions per request <= 256 chunks
constexpr int kMaxSplitRows = 2048;    // index entries one attention workgroup may own

struct IdxDecodeArgs {
  int B, n_q, max_pages, num_pages, top_k, n_chunks_max;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const void* q;
  const uint8_t* q_scales;
  const float* w;
  const void* k;
  const void* k_scales;  // 4 bytes per key row: f32 scale (FP8), or 4 E8M0 codes (k_mx)
  bool k_mx;             // FP8 keys with one E8M0 scale per 32 elements
  int32_t* idx_out;
  int spin_max;        // polls (each ~64 cycles of sleep) before an exchange wait gives up
  int xcd_local;       // block layout: a request's chunks on one XCD (grids of several rounds)
  // workspace
  uint32_t* counters;  // [B][kCounterStride]: arrivals, departures, give-up state, epoch
  uint64_t* refs;      // [T][n_chunks_max][2]  per chunk lo, hi (each tagged with the call's epoch)
  uint64_t* cnts;      // [T][n_chunks_max]     per chunk: keys >= hi | band keys << 16 (tagged)
  uint64_t* cand;      // [T][n_chunks_max][chunk] (key | position << 32): band from the front, keys >= hi from the back
};


struct IdxPrefillArgs {
  int B, n_q, max_pages, num_pages, top_k;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const void* q;
  const float* w;
  const void* k;
  int32_t* idx_out;
};

struct SfaArgs {
  int T, n_q, H, max_pages, num_pages, top_k, kv_groups;
  int rope_bf16;  // FP8 latent rows of 640 bytes: 512 codes + 64 bf16 rope (scales over the latent only)
  int n_splits, split_len, head_blocks;
  float sm_scale;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const void* q;
  const void* kv;
  const float* kv_scales;
  const int32_t* idx;
  void* out;
  float* lse;
  __bf16* part_o;  // [T][n_splits][H][512] split output normalised by its own sum
  float* part_ml;  // [T][n_splits][H][2]   (running max in log2 units, sum)
};

// The single-launch decode step: the indexer's arguments and workspace
// (n_q = 1, bf16, 4096-position chunks, one workgroup per chunk) and the
// attention's (T = B, 128 heads, split partials in the workspace).
struct StepArgs {
  IdxDecodeArgs idx;
  SfaArgs att;
};

struct QuantArgs {
  int n_rows, row_len;  // row_len % 32 == 0
  const void* x;        // bf16 [n_rows][row_len]
  uint8_t* codes;       // [n_rows][row_len] E4M3
  uint8_t* scales;      // [n_rows][row_len / 32] E8M0
};

struct AppendArgs {
  int B, n_q, max_pages, num_pages;
  const int32_t* seq_lens;
  const int32_t* block_table;
  const void* k_new;  // bf16 [T][128] or null
  bool k_fp8;
  bool k_mx;          // FP8 key rows with E8M0 scales per 32 elements
  void* k_cache;      // [num_pages][64][128] bf16 or E4M3
  void* k_scales;     // [num_pages][64] f32 (FP8) or [num_pages][64][4] E8M0 (k_mx)
  const void* kv_new; // bf16 [T][576] or null
  bool kv_fp8;
  bool kv_rope_bf16;  // FP8 latent rows of 640 bytes with the 64 rope elements in bf16
  int kv_groups;      // 1 or 5 (FP8), 1 or 4 (kv_rope_bf16)
  void* kv_cache;     // [num_pages][64][576] bf16 or E4M3
  float* kv_scales;   // [num_pages][64][kv_groups] (FP8)
};

struct ValidateArgs {
  int B, max_pages, num_pages;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t* bad_out;  // one int32: the count of problems found
};

// Records a failure message for li_last_error() (printf format) and returns s.
li_status report(li_status s, const char* fmt, ...);

hipError_t launch_mxfp8_quant(const QuantArgs& a, hipStream_t stream);
hipError_t launch_cache_append(const AppendArgs& a, hipStream_t stream);

int idx_decode_chunk(int B, int n_q, bool fp8, int max_pages, int cus);
bool idx_decode_xcd_local(int B, int n_chunks_max, int chunk, int cus);
hipError_t launch_idx_decode(const IdxDecodeArgs& a, int chunk, bool fp8, hipStream_t stream);
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_idx_prefill(const IdxPrefillArgs& a, hipStream_t stream);
hipError_t launch_sfa(const SfaArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_decode_step(const StepArgs& s, hipStream_t stream);
hipError_t launch_validate_paged(const ValidateArgs& a, hipStream_t stream);
int sfa_heads_per_block(int H);

}  // namespace sli
