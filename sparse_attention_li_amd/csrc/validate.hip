// Check of the paged-cache metadata on the device: the kernels clamp
// out-of-range page ids and lengths (a bad table gives wrong results, never
// an access outside the pools); this count lets a caller find such tables.
#include "launch.h"

namespace sli {

// One thread per (request, logical page).  A request whose length lies
// outside [0, max_pages*64] counts once (on its page 0); every page a request
// uses (p < ceil(L/64), L held to that range) whose id lies outside
// [0, num_pages) counts once.
__global__ void validate_paged_kernel(const ValidateArgs a) {
  const long long total = (long long)a.B * a.max_pages;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int b = (int)(i / a.max_pages), p = (int)(i % a.max_pages);
    const int L = a.seq_lens[b];
    const long long cap = (long long)a.max_pages * 64;
    uint32_t bad = 0;
    if (p == 0 && (L < 0 || (long long)L > cap)) ++bad;
    const long long Lc = L < 0 ? 0 : ((long long)L > cap ? cap : L);
    if ((long long)p * 64 < Lc) {
      const int pg = a.block_table[i];
      if (pg < 0 || pg >= a.num_pages) ++bad;
    }
    if (bad) atomicAdd(reinterpret_cast<uint32_t*>(a.bad_out), bad);
  }
}

hipError_t launch_validate_paged(const ValidateArgs& a, hipStream_t stream) {
  hipError_t e = launch_zero_fill(a.bad_out, 4, stream);
  if (e != hipSuccess) return e;
  const long long total = (long long)a.B * a.max_pages;
  const long long nb = (total + 255) / 256;
  const unsigned blocks = (unsigned)(nb < 1024 ? (nb > 0 ? nb : 1) : 1024);
  hipLaunchKernelGGL(validate_paged_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sli
