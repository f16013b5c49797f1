// Device primitives shared by the gfx950 kernels of the sparse-attention path:
// vector types, MFMA wrappers, order-preserving score keys, wave/block scans,
// a block-wide radix select and an LDS bitonic sort.  Wavefront size is 64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace sli {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt left at max).
#define SLI_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N)&15) | (((N) >> 4) << 14) | 0x70 | 0xF00)

// Calls f(std::integral_constant<int, J>) for J = 0 .. N-1: the body is
// instantiated once per J, so everything indexed by J is a constant.
template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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
// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves (no LDS
// round trip): Hillis-Steele inside each 16-lane row, then the row totals are
// broadcast into the following rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_xor(v, d, kWave);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_xor(v, d, kWave);
    v = v < o ? v : o;
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

// Two exclusive scans with one pair of barriers.  s_tmp needs 2*blockDim.x/64
// entries.  Returns the exclusive prefix of a; b's goes to pre_b; both totals
// to every thread.
__device__ __forceinline__ uint32_t block_excl_scan2(uint32_t a, uint32_t b, uint32_t* s_tmp, uint32_t& tot_a,
                                                     uint32_t& pre_b, uint32_t& tot_b) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == kWave - 1) {
    s_tmp[wid] = ia;
    s_tmp[nw + wid] = ib;
  }
  __syncthreads();
  uint32_t oa = 0, ta = 0, ob = 0, tb = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t xa = s_tmp[i], xb = s_tmp[nw + i];
    oa += (i < wid) ? xa : 0u;
    ta += xa;
    ob += (i < wid) ? xb : 0u;
    tb += xb;
  }
  __syncthreads();
  tot_a = ta;
  tot_b = tb;
  pre_b = ob + ib - b;
  return oa + ia - a;
}

// N exclusive scans of 32-bit values with one pair of barriers.  s_tmp needs
// N*blockDim.x/64 entries.  pre[i] receives the exclusive prefix of v[i],
// tot[i] its block total (every thread).
template <int N>
__device__ __forceinline__ void block_excl_scan_n(const uint32_t (&v)[N], uint32_t* s_tmp, uint32_t (&pre)[N],
                                                  uint32_t (&tot)[N]) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  uint32_t incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) incl[i] = wave_incl_scan(v[i]);
  if (lane == kWave - 1)
#pragma unroll
    for (int i = 0; i < N; ++i) s_tmp[i * nw + wid] = incl[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    uint32_t o = 0, t = 0;
    for (int w = 0; w < nw; ++w) {
      const uint32_t x = s_tmp[i * nw + w];
      o += (w < wid) ? x : 0u;
      t += x;
    }
    pre[i] = o + incl[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();
}

// Block-wide AND of a predicate, with the barrier of __syncthreads_and but
// on caller-provided LDS (one word per wave), so a kernel's LDS is all its own.
__device__ __forceinline__ bool block_all(bool p, uint32_t* s_tmp) {
  const int wid = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const bool wave_ok = __ballot(!p) == 0ull;
  if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[wid] = wave_ok ? 1u : 0u;
  __syncthreads();
  bool r = true;
  for (int i = 0; i < nw; ++i) r = r && s_tmp[i] != 0u;
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- radix select
// Finds the k-th largest key (1 <= k <= N) among N <= PER*blockDim.x keys
// given by get(i) (any values, 0 included).  On return every thread
// holds tau and n_greater = number of keys > tau (k - n_greater keys equal to
// tau belong to the top k).  The keys sit in registers; a block min/max finds
// the bits all keys share, and the select walks 8-bit windows below the
// highest differing bit, each with one LDS histogram (plain atomics) and a
// suffix scan by wave 0.  s_hist needs 256 entries, s_sel 4.
template <int PER, class Get>
__device__ uint32_t block_radix_select(Get get, int N, int k, uint32_t* s_hist, uint32_t* s_sel, int& n_greater) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave, nw = blockDim.x / kWave;
  uint32_t key[PER];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = tid + r * (int)blockDim.x;
    key[r] = i < N ? get(i) : 0u;
    if (i < N) {
      lo = key[r] < lo ? key[r] : lo;
      hi = key[r] > hi ? key[r] : hi;
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    s_hist[2 * wid] = lo;
    s_hist[2 * wid + 1] = hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
  for (int w = 0; w < nw; ++w) {
    lo = s_hist[2 * w] < lo ? s_hist[2 * w] : lo;
    hi = s_hist[2 * w + 1] > hi ? s_hist[2 * w + 1] : hi;
  }
  __syncthreads();
  const uint32_t diff = lo ^ hi;
  if (diff == 0) {  // all keys equal
    n_greater = 0;
    return lo;
  }
  int top = 31 - __clz(diff);           // highest bit where keys differ
  uint32_t prefix = lo & ~((2u << top) - 1u);  // bits above it, shared by all keys
  uint32_t remaining = (uint32_t)k;
  while (top >= 0) {
    const int shift = top >= 7 ? top - 7 : 0;
    const int width = top - shift + 1;  // <= 8
    const uint32_t above = top == 31 ? 0u : ~((2u << top) - 1u);
    for (int i = tid; i < 256; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (tid + r * (int)blockDim.x < N && (key[r] & above) == prefix)
        atomicAdd(&s_hist[(key[r] >> shift) & ((1u << width) - 1u)], 1u);
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = s_hist[255 - 4 * lane - i];
      const uint32_t sum = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
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
    prefix |= s_sel[0] << shift;
    remaining = s_sel[1];
    top = shift - 1;
  }
  n_greater = k - (int)remaining;
  return prefix;
}

// The same selection by a single wave for N <= 64*PER keys (every lane of the
// wave calls it; no block barrier): one LDS histogram of 256 words per 8-bit
// window, private to the wave, updated with atomics and read back in order
// (a wave's LDS operations complete in order).  On return every lane holds
// tau and n_greater.
template <int PER, class Get>
__device__ uint32_t wave_radix_select(Get get, int N, int k, uint32_t* s_hist, int& n_greater) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[PER];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = lane + r * kWave;
    key[r] = i < N ? get(i) : 0u;
    if (i < N) {
      lo = key[r] < lo ? key[r] : lo;
      hi = key[r] > hi ? key[r] : hi;
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lo == hi) {
    n_greater = 0;
    return lo;
  }
  int top = 31 - __clz(lo ^ hi);
  uint32_t prefix = lo & ~((2u << top) - 1u);
  uint32_t remaining = (uint32_t)k;
  while (top >= 0) {
    const int shift = top >= 7 ? top - 7 : 0;
    const int width = top - shift + 1;
    const uint32_t above = top == 31 ? 0u : ~((2u << top) - 1u);
#pragma unroll
    for (int i = 0; i < 4; ++i) s_hist[4 * lane + i] = 0u;
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (lane + r * kWave < N && (key[r] & above) == prefix)
        atomicAdd(&s_hist[(key[r] >> shift) & ((1u << width) - 1u)], 1u);
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = s_hist[255 - 4 * lane - i];
    const uint32_t sum = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t excl = incl - sum;
    const bool mine = excl < remaining && remaining <= incl;
    uint32_t dsel = 0, rsel = 0;
    if (mine) {
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
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;  // exactly one lane
    dsel = __shfl(dsel, src, kWave);
    rsel = __shfl(rsel, src, kWave);
    prefix |= dsel << shift;
    remaining = rsel;
    top = shift - 1;
  }
  n_greater = k - (int)remaining;
  return prefix;
}

// The same selection for inputs too large to hold in registers (rare
// fallback paths): four 8-bit passes, each streaming all N keys through get()
// with eight reads per thread in flight.
template <class Get>
__device__ uint32_t block_radix_select_big(Get get, int N, int k, uint32_t* s_hist, uint32_t* s_sel, int& n_greater) {
  constexpr int LPT = 8;
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) s_hist[i] = 0;
    __syncthreads();
    for (int i0 = threadIdx.x; i0 < N; i0 += LPT * (int)blockDim.x) {
      uint32_t key[LPT];
#pragma unroll
      for (int r = 0; r < LPT; ++r) {
        const int i = i0 + r * (int)blockDim.x;
        key[r] = i < N ? get(i) : 0u;
      }
#pragma unroll
      for (int r = 0; r < LPT; ++r)
        if (i0 + r * (int)blockDim.x < N && (key[r] & mask) == prefix) atomicAdd(&s_hist[(key[r] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = s_hist[255 - 4 * lane - i];
      const uint32_t sum = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t excl = incl - sum;
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
    prefix |= s_sel[0] << shift;
    remaining = s_sel[1];
    mask |= 255u << shift;
  }
  n_greater = k - (int)remaining;
  return prefix;
}

// ---------------------------------------------------------------- wave sort
// Sorts the 64*R keys held by one wave (lane l holds elements R*l .. R*l+R-1
// in v[0..R-1]) into descending order, in registers: bitonic network whose
// cross-lane steps are xor-shuffles, so no LDS and no block barrier.
template <int R>
__device__ __forceinline__ void wave_bitonic_sort_desc(uint32_t (&v)[R]) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int N = kWave * R;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((r & j) == 0) {
            const int e = R * lane + r;
            const bool desc = (e & k) == 0;
            const uint32_t a = v[r], b = v[r | j];
            const bool sw = desc ? (a < b) : (a > b);
            v[r] = sw ? b : a;
            v[r | j] = sw ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = R * lane + r;
          const uint32_t o = __shfl_xor(v[r], j / R, kWave);
          const bool desc = (e & k) == 0;
          const bool lower = (e & j) == 0;
          // the lower index of a descending pair keeps the max
          const bool keep_max = desc == lower;
          v[r] = keep_max ? (v[r] > o ? v[r] : o) : (v[r] < o ? v[r] : o);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bitonic sort
// Sorts N (power of two) keys in LDS into descending order.  All threads of
// the block must call it.
template <int N>
__device__ void lds_bitonic_sort_desc(uint32_t* s) {
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int p = threadIdx.x; p < N / 2; p += blockDim.x) {
        const int i = ((p & ~(j - 1)) << 1) | (p & (j - 1));  // j is a power of two
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

// Polling read of a counter: relaxed, so it does not invalidate caches on
// every iteration; the caller issues one acquire fence once the wait is over.
__device__ __forceinline__ uint32_t atomic_load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads and stores of data that other workgroups (possibly on other XCDs,
// each with its own L2) exchange within one launch: system-coherent accesses
// that bypass the non-coherent caches, so no reader can see a line another
// L2 kept from an earlier launch.  Only small exchange buffers use them.
__device__ __forceinline__ void xstore(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void xstore(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint32_t xload(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ int32_t xload(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void xstore64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t xload64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// 16-byte accesses of data exchanged between the workgroups of one launch,
// system-coherent like xstore / xload (cache policy sc0 sc1), through a buffer
// resource over a wave-uniform `base` with a per-lane byte offset < 2 GiB.
constexpr int kCPolSystem = 1 | 16;  // sc0 | sc1
__device__ __forceinline__ void xstore128(void* base, uint32_t off, i32x4 v) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCPolSystem);
}
__device__ __forceinline__ i32x4 xload128(const void* base, uint32_t off) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCPolSystem);
}

// Waits until this wave's outstanding vector-memory operations (stores
// included) have completed, i.e. reached L2.  Every thread runs it before the
// workgroup barrier that precedes a single thread's agent-scope release: the
// release writes L2 back, so all waves' stores must be in L2 by then.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

}  // namespace sli
