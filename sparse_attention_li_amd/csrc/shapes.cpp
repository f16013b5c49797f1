// Launch-shape choices of the kernels (plain host code, no device code, so
// the C ABI's host logic can be built and checked on a machine without a GPU).
#include "launch.h"

namespace sli {

// Positions per workgroup.  256 when even at that length the grid fits one
// round of the chip (small calls: a few requests of up to 65536 positions,
// the most chunks a request may have): a chunk's 64 KiB of bf16 keys are then
// in flight at once, and a small call streams in one memory round trip
// instead of four.  4096 (eight waves, one workgroup per CU) when
// the grid still gives every CU a workgroup: each CU then streams the same
// amount and the request's chunks finish together.  FP8 one-token grids that
// would take more than one round of the chip at 4096 (three four-wave
// workgroups per CU) use 8192: half the workgroups, so fewer requests wait at
// their exchanges for chunks dispatched in a later round.  Smaller chunks
// (four waves, two workgroups per CU) for small batches, and for bf16
// two-token calls, whose keys and key ring would not fit beside each other in
// LDS.
int idx_decode_chunk(int B, int n_q, bool fp8, int max_pages, int cus) {
  const long long maxlen = (long long)max_pages * 64;
  auto wgs = [&](long long ch) { return (long long)B * ((maxlen + ch - 1) / ch); };
  if (fp8 && n_q == 1 && wgs(4096) > 3LL * cus) return 8192;
  if (wgs(256) <= cus && maxlen <= 256LL * kMaxChunksPerSeq) return 256;
  if ((n_q == 1 || fp8) && wgs(4096) >= cus) return 4096;
  return wgs(1024) > 2LL * cus ? 2048 : 1024;
}

// XCD-local block layout when the grid takes several rounds of the chip (one
// workgroup per CU counted), a request's chunks fit in one XCD's CUs at once,
// and there are enough requests (>= 2 per XCD) to balance the XCDs.
bool idx_decode_xcd_local(int B, int n_chunks_max, int chunk, int cus) {
  (void)chunk;
  return B >= 16 && n_chunks_max <= cus / 8 && (long long)B * n_chunks_max > cus;
}

// Heads per attention workgroup: every head of the token (65 to 128), or a
// block of 32 or 64 for small head counts.
int sfa_heads_per_block(int H) { return H <= 64 ? (H <= 32 ? 32 : 64) : 128; }

}  // namespace sli
