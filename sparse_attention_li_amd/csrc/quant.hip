// Cache append and quantisers: the step before the sparse-attention path in
// every decode step, gfx950.
//
// What it computes ("Day-0 Inference Adaptation and Optimization for Hybrid
// Attention Architectures", sec. 4; "Optimizing Inference for Hybrid
// Attention LLMs", sec. 4 table; "Day0 Inference Adaptation and Performance
// Optimization for a Sparse Hybrid Architecture LLM", sec. 3.1):
//  - MXFP8 quantisation of the indexer query: per group of 32 consecutive
//    elements, a power-of-two scale X = 2^(floor(log2 amax) - 8) stored as an
//    E8M0 code (8 is E4M3's largest exponent; an all-zero group takes X = 1),
//    elements x / X as E4M3 codes (nearest, ties to even, saturating at 448);
//  - the new token's indexer-key row (128) and latent row (576 = 512 + 64)
//    written into the paged caches at its position: bf16 as is, or FP8 with
//    an f32 scale amax / 448 per row or per 128-wide tile (the fifth tile of
//    a latent row being 64 wide) and codes fl32(x / scale) as E4M3, or (key
//    rows) MXFP8 like the query, or (latent rows) FP8 latent with the rope
//    kept in bf16 (scales per row or per 128-wide tile of the 512 latent).
// Token t = b * n_q + j sits at position L_b - n_q + j of request b.
#include "device_common.h"
#include "launch.h"

namespace sli {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two floats to two E4M3 codes (nearest even), saturated at +-448 first.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Eight bf16 values (one 16-byte chunk) -> eight codes (8 bytes), each value
// multiplied by `mul` (a power of two) or divided by `div` (rounded fp32
// quotient), whichever is given.
__device__ __forceinline__ uint2 encode8(const u32x4& raw, float mul, float div) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
    v[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = div != 0.f ? __fdiv_rn(v[i], div) : v[i] * mul;
  uint2 r;
  r.x = e4m3x2(v[0], v[1]) | (e4m3x2(v[2], v[3]) << 16);
  r.y = e4m3x2(v[4], v[5]) | (e4m3x2(v[6], v[7]) << 16);
  return r;
}

__device__ __forceinline__ float amax8(const u32x4& raw) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_bits_to_f32(raw[i] & 0xffffu)));
    m = fmaxf(m, fabsf(bf16_bits_to_f32(raw[i] >> 16)));
  }
  return m;
}

// max over groups of `w` consecutive lanes (w a power of two <= 64)
__device__ __forceinline__ float group_max(float v, int w) {
  for (int d = 1; d < w; d <<= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

// ---------------------------------------------------------------- MXFP8
// log2 of a group's scale X = 2^(floor(log2 amax) - 8), held to E8M0's range
// [-127, 127] (an all-zero group: X = 1; a subnormal amax: the least scale).
__device__ __forceinline__ int mx_shift(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  return e == 0 ? -127 : min(max(e - 127 - 8, -127), 127);
}

// Four lanes per 32-element group, eight elements (16 bytes) per lane.
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const QuantArgs a) {
  const size_t chunk = (size_t)blockIdx.x * 256 + threadIdx.x;  // 8-element chunk
  const size_t n_chunks = (size_t)a.n_rows * (a.row_len / 8);
  const bool ok = chunk < n_chunks;
  const u32x4 raw = ok ? reinterpret_cast<const u32x4*>(a.x)[chunk] : (u32x4){0u, 0u, 0u, 0u};
  const int sh = mx_shift(group_max(amax8(raw), 4));  // log2 X
  if (!ok) return;
  reinterpret_cast<uint2*>(a.codes)[chunk] = encode8(raw, ldexpf(1.f, -sh), 0.f);
  if ((threadIdx.x & 3) == 0) a.scales[chunk / 4] = (uint8_t)(sh + 127);
}

hipError_t launch_mxfp8_quant(const QuantArgs& a, hipStream_t stream) {
  const size_t n_chunks = (size_t)a.n_rows * (a.row_len / 8);
  const unsigned blocks = (unsigned)((n_chunks + 255) / 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- cache append
// One workgroup per new token: wave 0 writes the indexer-key row (lanes 0-15,
// eight elements each), wave 1 the latent row (lanes 0-63 the 512 latent
// elements, then lanes 0-7 the 64 rope elements).
__global__ __launch_bounds__(128) void cache_append_kernel(const AppendArgs a) {
  const int t = blockIdx.x, b = t / a.n_q, j = t % a.n_q;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int L = a.seq_lens[b];
  const int s = L - a.n_q + j;
  if (s < 0 || s >= a.max_pages * 64) return;  // no slot for this token
  const int page = min(max(a.block_table[(size_t)b * a.max_pages + (s >> 6)], 0), a.num_pages - 1);
  const size_t row = (size_t)page * 64 + (s & 63);  // physical row of the pool
  if (wid == 0) {
    if (!a.k_new) return;
    const u32x4 raw = lane < 16 ? reinterpret_cast<const u32x4*>(a.k_new)[(size_t)t * 16 + lane] : (u32x4){0u, 0u, 0u, 0u};
    if (!a.k_fp8) {
      if (lane < 16) reinterpret_cast<u32x4*>(a.k_cache)[row * 16 + lane] = raw;
      return;
    }
    if (a.k_mx) {  // MXFP8: one E8M0 scale per 32 elements (four lanes)
      const int sh = mx_shift(group_max(amax8(raw), 4));
      if (lane < 16) reinterpret_cast<uint2*>(a.k_cache)[row * 16 + lane] = encode8(raw, ldexpf(1.f, -sh), 0.f);
      if (lane < 16 && (lane & 3) == 0) static_cast<uint8_t*>(a.k_scales)[row * 4 + lane / 4] = (uint8_t)(sh + 127);
      return;
    }
    const float amax = group_max(amax8(raw), 16);
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    if (lane < 16) reinterpret_cast<uint2*>(a.k_cache)[row * 16 + lane] = encode8(raw, 1.f, sc);
    if (lane == 0) static_cast<float*>(a.k_scales)[row] = sc;
    return;
  }
  if (!a.kv_new) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.kv_new) + (size_t)t * 72;
  const u32x4 lat = src[lane];                                             // elements 8 lane .. 8 lane + 7
  const u32x4 rope = lane < 8 ? src[64 + lane] : (u32x4){0u, 0u, 0u, 0u};  // elements 512 + 8 lane ..
  if (!a.kv_fp8) {
    reinterpret_cast<u32x4*>(a.kv_cache)[row * 72 + lane] = lat;
    if (lane < 8) reinterpret_cast<u32x4*>(a.kv_cache)[row * 72 + 64 + lane] = rope;
    return;
  }
  if (a.kv_rope_bf16) {  // 640-byte rows: latent codes (scales over the latent only), then the rope as is
    const float am = group_max(amax8(lat), a.kv_groups == 1 ? 64 : 16);
    const float sc = am > 0.f ? __fdiv_rn(am, 448.f) : 1.f;
    uint8_t* dst = static_cast<uint8_t*>(a.kv_cache) + row * 640;
    reinterpret_cast<uint2*>(dst)[lane] = encode8(lat, 1.f, sc);
    if (lane < 8) reinterpret_cast<u32x4*>(dst + 512)[lane] = rope;
    float* scp = a.kv_scales + row * a.kv_groups;
    if (a.kv_groups == 1 ? lane == 0 : (lane & 15) == 0) scp[lane >> 4] = sc;
    return;
  }
  float sc_lat, sc_rope;
  if (a.kv_groups == 1) {
    const float amax = fmaxf(group_max(amax8(lat), 64), group_max(amax8(rope), 64));
    sc_lat = sc_rope = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  } else {
    const float am_lat = group_max(amax8(lat), 16);    // tile lane / 16 of 128 elements
    const float am_rope = group_max(amax8(rope), 8);   // the 64-wide fifth tile (lanes 0-7)
    sc_lat = am_lat > 0.f ? __fdiv_rn(am_lat, 448.f) : 1.f;
    sc_rope = am_rope > 0.f ? __fdiv_rn(am_rope, 448.f) : 1.f;
  }
  uint8_t* dst = static_cast<uint8_t*>(a.kv_cache) + row * 576;
  reinterpret_cast<uint2*>(dst)[lane] = encode8(lat, 1.f, sc_lat);
  if (lane < 8) reinterpret_cast<uint2*>(dst + 512)[lane] = encode8(rope, 1.f, sc_rope);
  float* scp = a.kv_scales + row * a.kv_groups;
  if (a.kv_groups == 1) {
    if (lane == 0) scp[0] = sc_lat;
  } else {
    if ((lane & 15) == 0) scp[lane >> 4] = sc_lat;
    if (lane == 0) scp[4] = sc_rope;
  }
}

hipError_t launch_cache_append(const AppendArgs& a, hipStream_t stream) {
  const int T = a.B * a.n_q;
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_append_kernel, dim3(T), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sli
