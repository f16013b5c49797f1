/*
 * sparse_li.h -- C ABI of the MI355X (gfx950) sparse-attention hot path.
 *
 * The path has three steps, all described on the pages about the hybrid
 * model's sparse-attention branch:
 *   1. a lightning indexer scores every cached position of a request,
 *        I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:])      (64 heads x 128)
 *      ("Day-0 Inference Adaptation and Optimization for Hybrid Attention
 *      Architectures", sec. 1; "Optimizing Inference for Hybrid Attention
 *      LLMs", sec. 3.1 -- the pages name per-head scoring and a cross-head
 *      weighted sum; the ReLU is our reading of the unnamed nonlinearity);
 *   2. Top-K keeps the K best positions, on chip, writing back only indices
 *      (same sections; "Day0 Inference Support and Performance Optimization
 *      for New-Architecture LLMs", sec. 4);
 *   3. sparse attention over the MLA latent cache reads only those rows
 *      ("Day0 Inference Adaptation and Performance Optimization for a Sparse
 *      Hybrid Architecture LLM", sec. 1 and 2.1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers on the current HIP device, except
 *   where noted.  The caller owns every buffer; the library never allocates
 *   device memory and keeps no state between calls.
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *   asynchronous: buffers must stay valid until the stream has passed them.
 * - Requests and tokens.  There are B = num_seqs requests with n_q =
 *   q_per_seq new query tokens each, T = B*n_q tokens in all; token
 *   t = b*n_q + j.  seq_lens[b] = L_b counts the cached positions of request b
 *   INCLUDING its n_q new tokens, so token (b, j) sits at absolute position
 *   L_b - n_q + j and sees positions s <= L_b - n_q + j (causal; this one rule
 *   covers decode, multi-token verification and a prefill chunk).
 * - Paged caches.  Position s of request b lives in physical page
 *   block_table[b*max_pages + s/64], slot s%64; page size is 64.  Pools are
 *   arrays of num_pages pages.  Block-table entries must lie in
 *   [0, num_pages) and L_b <= max_pages*64; the kernels clamp out-of-range
 *   values (so a bad table gives wrong results, never an out-of-bounds access).
 * - Formats.  LI_BF16: bfloat16 bit patterns.  LI_FP8: OCP FP8 E4M3FN codes
 *   with block scales (positive f32 for caches, E8M0 for the indexer query).
 *   LI_MXFP8 (indexer key only): E4M3FN codes with one E8M0 scale per 32
 *   elements, like the query.  LI_FP8_ROPE_BF16 (latent only): FP8 latent
 *   with the 64 rope elements kept in bf16.  The pages' quantised layouts ("Optimizing
 *   Inference for Hybrid Attention LLMs", sec. 4 table): indexer q MXFP8 with
 *   one E8M0 scale per 32 elements, the indexer key with group-32 scales too;
 *   FP8 caches with one f32 scale per 128-element block.
 * - Return values: LI_OK, or a negative li_status; on failure nothing has been
 *   enqueued and li_last_error() describes the problem (thread-local).
 * - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef SPARSE_LI_H
#define SPARSE_LI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LI_OK = 0,
  LI_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, top_k out of range */
  LI_ERR_UNSUPPORTED = -2, /* shape or format this build does not implement */
  LI_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  LI_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} li_status;

typedef enum { LI_BF16 = 0, LI_FP8 = 1, LI_MXFP8 = 2, LI_FP8_ROPE_BF16 = 3 } li_dtype;

#define LI_PAGE_SIZE 64
#define LI_INDEX_HEADS 64
#define LI_INDEX_DIM 128
#define LI_LATENT_DIM 576 /* 512 latent + 64 rope, one head shared by all query heads */
#define LI_VALUE_DIM 512
#define LI_MAX_TOP_K 2048

/* Version string of the library (static storage).  Library housekeeping:
 * no passage of the pages defines it. */
const char* li_version(void);

/* Message of the last failing call on this thread (static thread-local
 * storage).  Library housekeeping: no passage of the pages defines it. */
const char* li_last_error(void);

/*
 * Test hook (not for production use): the number of polls (about 64 cycles of
 * sleep each) a cross-workgroup exchange wait of li_score_topk makes before it
 * gives up and takes its exact fallback; default 20000, a negative value
 * restores the default.  Lowering it forces the fallbacks, which changes
 * timing only, never results.  Process-wide, read at each call.  The exchange
 * is this library's way of keeping the selection on chip ("Day0 Inference
 * Support and Performance Optimization for New-Architecture LLMs", sec. 4:
 * Top-K without writing the scores back); the pages define no such knob.
 */
void li_set_exchange_patience(int32_t polls);

/*
 * Bytes of workspace li_score_topk needs for this geometry.  max_pages bounds
 * every L_b (L_b <= max_pages*64).  Returns 0 for invalid arguments.  The
 * workspace holds the on-chip selection's exchange state, not scores (the
 * pages keep the score matrix out of memory: "Day0 Inference Support and
 * Performance Optimization for New-Architecture LLMs", sec. 4).
 */
size_t li_score_topk_workspace_size(int32_t num_seqs, int32_t q_per_seq, int32_t max_pages, int32_t top_k);

/*
 * Zero-fills a workspace on `stream` with a kernel (no hipMemset, so it may be
 * captured in a HIP graph).  A workspace must be zero before its first use by
 * li_score_topk; every li_score_topk call leaves it zero again.  Library
 * housekeeping for the workspace above: no passage of the pages defines it.
 */
li_status li_workspace_zero(void* workspace, size_t workspace_bytes, void* stream);

/*
 * li_score_topk -- fused indexer score + Top-K selection.  The score is the
 * per-head q.k, ReLU, and the head-weighted sum over the 64 indexer heads;
 * the selection keeps the top_k positions per query token, on chip ("Day-0
 * Inference Adaptation and Optimization for Hybrid Attention Architectures",
 * sec. 1 and 3; "Optimizing Inference for Hybrid Attention LLMs", sec. 3.1;
 * "Day0 Inference Support and Performance Optimization for New-Architecture
 * LLMs", sec. 4).  The FP8 forms follow the quantised indexer layouts of
 * "Optimizing Inference for Hybrid Attention LLMs", sec. 4 table.
 *
 *   q         [T,64,128]  indexer query; LI_BF16 bits, or LI_FP8 E4M3 codes with
 *   q_scales  [T,64,4]    E8M0 scales (one per 32 consecutive elements; LI_FP8 only,
 *                         must be NULL for LI_BF16)
 *   w         [T,64]      f32 per-token head weights (any sign)
 *   k_cache   [num_pages,64,128] indexer key pool; LI_BF16 bits, or E4M3 codes with
 *   k_scales  LI_FP8:   [num_pages,64]   one positive f32 scale per 128-element row;
 *             LI_MXFP8: [num_pages,64,4] uint8 E8M0 codes, one per 32 elements
 *             (0..254); 4-byte aligned; NULL for LI_BF16
 *   k_dtype   LI_BF16 with a LI_BF16 query; LI_FP8 or LI_MXFP8 with a LI_FP8 query.
 *   top_k     1..2048
 *   idx_out   [T,top_k] int32: the min(top_k, visible) positions with the largest
 *             score, ties going to the lower position, written in ascending
 *             position order; the rest of the row is -1.
 *   workspace li_score_topk_workspace_size(...) bytes, zero before its first use
 *             (see li_workspace_zero).  Its first 512 KiB + 128 bytes hold
 *             per-request exchange counters and one launch-wide epoch at a fixed
 *             place for any geometry; each call leaves the counters zero and
 *             advances the epoch, so one workspace can serve calls of different
 *             shapes.  Calls that share a workspace must not overlap in time.
 *             num_seqs <= 4096.
 *
 * Scores live only on chip: the intermediates in HBM are, per chunk of
 * positions, two bounds on the K-th score, the positions above the upper bound
 * and the (key, position) band between the bounds.
 * Supported: q_per_seq in {1, 2} (decode, two-token verification; bf16 or
 * FP8) and q_per_seq >= 3 (prefill chunk; bf16, the workspace is not used
 * and may be NULL).
 */
li_status li_score_topk(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                        int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q,
                        const uint8_t* q_scales, const float* w, int32_t k_dtype, const void* k_cache,
                        const void* k_scales, int32_t top_k, int32_t* idx_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Bytes of the library-owned exchange workspace of li_score_topk_noalloc, per GPU. */
#define LI_NOALLOC_WORKSPACE_MAX (128u << 20)

/*
 * li_score_topk_noalloc -- li_score_topk without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc).  Same arguments,
 * layouts, results and errors as li_score_topk, minus the workspace.  It
 * allocates nothing: the exchange workspace is a device array of
 * LI_NOALLOC_WORKSPACE_MAX bytes inside the library, one per GPU, held until
 * the process ends.
 *   - Geometries whose li_score_topk_workspace_size exceeds that size return
 *     LI_ERR_UNSUPPORTED (e.g. 128 requests x 2 tokens x 131072 positions).
 *   - The first call on a device also clears the array, with a fill kernel
 *     enqueued on `stream` before the indexer.
 *   - Every call on one GPU uses the same array (each call leaves its
 *     counters zero for the next): calls that overlap in time on one GPU --
 *     other streams, other host threads -- race and give wrong results.
 */
li_status li_score_topk_noalloc(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens,
                                const int32_t* block_table, int32_t max_pages, int32_t num_pages, int32_t q_dtype,
                                const void* q, const uint8_t* q_scales, const float* w, int32_t k_dtype,
                                const void* k_cache, const void* k_scales, int32_t top_k, int32_t* idx_out,
                                void* stream);

/*
 * Bytes of workspace sfa_decode / sfa_prefill need: the partial results when
 * a token's index row is split over several workgroups (our decomposition of
 * the attention of "Day0 Inference Adaptation and Performance Optimization
 * for a Sparse Hybrid Architecture LLM", sec. 2.1; the pages do not split).
 */
size_t sfa_workspace_size(int32_t num_tokens, int32_t num_heads, int32_t top_k);

/*
 * sfa_decode -- sparse MLA attention over the selected latent rows: each
 * query head attends only to the rows of its token's index row, through the
 * one 576-wide latent row MLA keeps per position, keys the whole row and
 * values its first 512 elements ("Day0 Inference Adaptation and Performance
 * Optimization for a Sparse Hybrid Architecture LLM", sec. 1 and 2.1; FP8
 * cache layouts: "Optimizing Inference for Hybrid Attention LLMs", sec. 4
 * table; "Day-0 Inference Adaptation and Optimization for Hybrid Attention
 * Architectures", sec. 4).
 *
 *   q          [T,H,576] bf16 query (latent-absorbed 512 + rope 64), H in {16,32,64,128}
 *   kv_cache   [num_pages,64,576] latent pool; LI_BF16 bits, or LI_FP8 codes with
 *   kv_scales  [num_pages,64,G] positive f32 scales, G = kv_scale_groups:
 *              1 = one scale per row, 5 = one per 128-wide tile (the 5th is 64 wide);
 *              or LI_FP8_ROPE_BF16: [num_pages,64,640] bytes per row, the 512 latent
 *              elements as E4M3 codes then the 64 rope elements as bf16, with
 *              G = 1 (one scale per row) or 4 (one per 128-wide latent tile)
 *   idx        [T,top_k] int32 logical positions of the token's request; entries
 *              < 0 or >= L_b are skipped
 *   sm_scale   softmax scale applied to q.c
 *   out        [T,H,512] bf16:  sum_j softmax_j(sm_scale * q.c_j) * c_j[0:512]
 *   lse        [T,H] f32 natural-log sum of exp of the scaled logits, or NULL;
 *              a row with no valid index gives out = 0 and lse = -inf
 *   workspace  sfa_workspace_size(T, H, top_k) bytes (no initialisation needed)
 */
li_status sfa_decode(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                     const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                     int32_t top_k, float sm_scale, void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * sfa_prefill -- the same operation for a prefill chunk (many query tokens
 * per request, each with its own causal index row: "Day0 Inference Adaptation
 * and Performance Optimization for a Sparse Hybrid Architecture LLM", sec. 2.1
 * -- prefill and decode attention over the selected rows); same arguments,
 * layouts and results as sfa_decode, and the same kernels and launch choice:
 * the split of a token's index row over workgroups follows from the token
 * count, so a chunk of many tokens runs unsplit.
 */
li_status sfa_prefill(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                      int32_t max_pages, int32_t num_pages, const void* q, int32_t num_heads, int32_t kv_dtype,
                      const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, const int32_t* idx,
                      int32_t top_k, float sm_scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace li_decode_step needs (q_per_seq 1 or 2); 0 for invalid
 * arguments.
 */
size_t li_decode_step_workspace_size(int32_t num_seqs, int32_t q_per_seq, int32_t max_pages, int32_t num_heads,
                                     int32_t top_k);

/*
 * li_decode_step -- one whole decode step of the sparse-attention path:
 * li_score_topk followed by sfa_decode on the same stream, as one launch
 * where the shape allows it.  The pages take every step other than attention
 * off the decode critical path by fusing the indexer into one operator and
 * dispatching the layer as one kernel ("Day-0 Inference Adaptation and
 * Optimization for Hybrid Attention Architectures", sec. 3; "Day0 Inference
 * Adaptation and Performance Optimization for a Sparse Hybrid Architecture
 * LLM", sec. 6).
 *
 *   Arguments: those of li_score_topk (q_idx = its q) and of sfa_decode (q =
 *   the MLA query), sharing num_seqs .. num_pages and top_k; idx_out receives
 *   the index rows and is read back by the attention.
 *   workspace  li_decode_step_workspace_size(...) bytes, zero before its first
 *              use (li_workspace_zero); every call leaves it so.  The same
 *              contract as li_score_topk's workspace; calls that share a
 *              workspace must not overlap in time.
 * One launch for bf16 query, keys and latent, q_per_seq = 1, num_heads = 128
 * and at most one 4096-position chunk per compute unit (num_seqs *
 * ceil(max_pages * 64 / 4096) <= CUs, <= 64 chunks per request): each
 * chunk's workgroup scores its chunk, writes its share of the index row,
 * attends to the selected positions that lie in its chunk (one partial per
 * chunk), and the request's workgroups merge the partials once every chunk
 * has published its own, in the same launch.  Other shapes run li_score_topk
 * and sfa_decode back to back.  idx_out is identical to li_score_topk's; out
 * and lse equal sfa_decode's up to the rounding of the partials (the fused
 * launch splits the index row by chunk, not by rank).
 */
li_status li_decode_step(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                         int32_t max_pages, int32_t num_pages, int32_t q_dtype, const void* q_idx,
                         const uint8_t* q_scales, const float* w, int32_t k_dtype, const void* k_cache,
                         const void* k_scales, const void* q, int32_t num_heads, int32_t kv_dtype,
                         const void* kv_cache, const float* kv_scales, int32_t kv_scale_groups, int32_t top_k,
                         float sm_scale, int32_t* idx_out, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * li_validate_paged -- checks the paged-cache metadata on the device (debug
 * aid; no kernel depends on it).  The conventions above require block-table
 * entries in [0, num_pages) and 0 <= L_b <= max_pages*64; the kernels clamp
 * violations, so a bad table gives wrong results rather than an access
 * outside the pools, and this call finds them.  Library housekeeping: no
 * passage of the pages defines it.
 *   seq_lens     [num_seqs] int32, block_table [num_seqs, max_pages] int32 (device)
 *   bad_out      one int32 (device, 4-byte aligned): set to the number of
 *                requests whose length lies outside [0, max_pages*64] plus the
 *                number of pages in use (p < ceil(L_b/64), L_b held to that
 *                range) whose id lies outside [0, num_pages)
 * Asynchronous on `stream` (a fill kernel clears bad_out first; no memset).
 */
li_status li_validate_paged(int32_t num_seqs, const int32_t* seq_lens, const int32_t* block_table, int32_t max_pages,
                            int32_t num_pages, int32_t* bad_out, void* stream);

/*
 * li_quantize_mxfp8 -- MXFP8 quantisation of bf16 rows, e.g. the indexer
 * query before li_score_topk ("Day-0 Inference Adaptation and Optimization
 * for Hybrid Attention Architectures", sec. 4: MXFP8 indexer query, group 32;
 * "Optimizing Inference for Hybrid Attention LLMs", sec. 4 table).
 *
 *   x       [n_rows,row_len] bf16, row_len a positive multiple of 32, 16-byte aligned
 *   codes   [n_rows,row_len] E4M3 codes out (8-byte aligned)
 *   scales  [n_rows,row_len/32] E8M0 codes out
 * Per group of 32 consecutive elements: X = 2^(floor(log2 amax) - 8) (E8M0
 * code floor(log2 amax) - 8 + 127, held to 0..254; an all-zero group takes
 * X = 1), element codes = x / X rounded to the nearest E4M3 value (ties to
 * the even code), saturating at 448.  n_rows = 0 is a no-op.  Asynchronous
 * on `stream`; the caller owns every buffer.
 */
li_status li_quantize_mxfp8(int32_t n_rows, int32_t row_len, const void* x, uint8_t* codes, uint8_t* scales,
                            void* stream);

/*
 * li_cache_append -- writes the new tokens' indexer-key and latent rows into
 * the paged caches (the pages' per-step cache update before the indexer and
 * attention read them; quantised layouts: same sections as above, FP8 KV with
 * per-token-head-tile scales of tile 128).
 *
 * Token t = b*q_per_seq + j (its request's j-th new token) is written at
 * position L_b - q_per_seq + j: page block_table[b][pos/64], slot pos%64.
 * Tokens whose position falls outside [0, max_pages*64) are skipped.
 *   k_new     [T,128] bf16 indexer-key rows, or NULL (no key cache update)
 *   k_dtype   LI_BF16 (copied), LI_FP8 (codes; k_scales[page][slot] = amax/448
 *             of the row, 1 for an all-zero row; codes = fl32(x/scale) to the
 *             nearest E4M3, ties to even, saturating; f32 k_scales 4-byte
 *             aligned) or LI_MXFP8 (per 32 elements, as li_quantize_mxfp8;
 *             k_scales [num_pages,64,4] uint8 E8M0)
 *   kv_new    [T,576] bf16 latent rows (512 latent + 64 rope), or NULL
 *   kv_dtype  LI_BF16 or LI_FP8 with kv_scale_groups 1 (one scale per row) or 5
 *             (one per 128-wide tile, the fifth 64 wide); scales as for the key;
 *             or LI_FP8_ROPE_BF16 (640-byte rows, the rope copied as bf16) with
 *             kv_scale_groups 1 or 4 over the 512 latent elements
 * Caches and scales as in li_score_topk / sfa_decode.  Asynchronous on
 * `stream`; rows of other positions are left untouched.
 */
li_status li_cache_append(int32_t num_seqs, int32_t q_per_seq, const int32_t* seq_lens, const int32_t* block_table,
                          int32_t max_pages, int32_t num_pages, const void* k_new, int32_t k_dtype, void* k_cache,
                          void* k_scales, const void* kv_new, int32_t kv_dtype, void* kv_cache, float* kv_scales,
                          int32_t kv_scale_groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_LI_H */
