// Device primitives shared by the gfx950 kernels of the sparse-attention path:
// vector types, MFMA wrappers, order-preserving score keys, wave/block scans,
// a block-wide radix select and an LDS bitonic sort.  Wavefront size is 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sli {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- score keys
// Order-preserving map from fp32 to uint32: larger float -> larger key.
// -0.0 is folded into +0.0 first.  Key 0 is reserved for "no position" (it is
// the image of a negative NaN, which the path never produces).
__device__ __forceinline__ uint32_t score_key(float x) {
  x = x + 0.0f;
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- scans
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Block-wide exclusive scan of one value per thread.  s_tmp needs
// blockDim.x/64 entries.  Every thread receives the block total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tmp, uint32_t& total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) s_tmp[wid] = incl;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    uint32_t x = s_tmp[i];
    off += (i < wid) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// ---------------------------------------------------------------- radix select
// Finds the k-th largest key (1 <= k <= N) among N keys given by get(i).  On
// return every thread holds tau and n_greater = number of keys > tau (so
// k - n_greater keys equal to tau belong to the top k).  Four 8-bit digit
// passes with LDS histograms; wave 0 locates each digit with a suffix scan.
// s_hist needs 256 entries, s_sel 2.
template <class Get>
__device__ uint32_t block_radix_select(Get get, int N, int k, uint32_t* s_hist, uint32_t* s_sel, int& n_greater) {
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
      uint32_t key = get(i);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = s_hist[255 - 4 * lane - i];
      uint32_t sum = h[0] + h[1] + h[2] + h[3];
      uint32_t incl = wave_incl_scan(sum);
      uint32_t excl = incl - sum;
      if (excl < remaining && remaining <= incl) {
        uint32_t acc = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (acc < remaining && remaining <= acc + h[i]) {
            s_sel[0] = 255u - 4u * lane - i;
            s_sel[1] = remaining - acc;
          }
          acc += h[i];
        }
      }
    }
    __syncthreads();
    uint32_t digit = s_sel[0];
    remaining = s_sel[1];
    prefix |= digit << shift;
    mask |= 255u << shift;
  }
  n_greater = k - (int)remaining;
  return prefix;
}

// ---------------------------------------------------------------- bitonic sort
// Sorts N (power of two) keys in LDS into descending order.  All threads of
// the block must call it.
template <int N>
__device__ void lds_bitonic_sort_desc(uint32_t* s) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = threadIdx.x; p < N / 2; p += blockDim.x) {
        const int i = 2 * j * (p / j) + (p % j);
        const int ixj = i + j;
        uint32_t a = s[i], b = s[ixj];
        const bool desc = (i & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          s[i] = b;
          s[ixj] = a;
        }
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- cross-workgroup flags
__device__ __forceinline__ uint32_t atomic_load_acquire(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sli
