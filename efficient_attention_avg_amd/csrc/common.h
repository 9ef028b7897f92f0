// Device helpers shared by the MiTA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

constexpr int kWave = 64;
constexpr int kHeadDim = 64;

// Raw bfloat16 storage: the upper 16 bits of an fp32.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Order-preserving map of an fp32 score to uint32: a larger score gives a
// larger key.  -0.0 is folded onto +0.0 first so that the two compare equal,
// as they do as numbers.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float fast_exp(float x) {
  // e^x = 2^(x*log2 e) on the hardware exp2 unit.
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// 2-D adaptive average pooling window along one axis: [lo, hi).
// (32-bit arithmetic while (i + 1) g + mg - 1 < 2^31; 64-bit past that, for
// the widest grids the API accepts)
__host__ __device__ __forceinline__ void pool_window(int i, int g, int mg, int* lo, int* hi) {
  if ((long long)g * (mg + 1) < (1LL << 31)) {
    *lo = (i * g) / mg;
    *hi = ((i + 1) * g + mg - 1) / mg;
  } else {
    *lo = (int)(((long long)i * g) / mg);
    *hi = (int)(((long long)(i + 1) * g + mg - 1) / mg);
  }
}

}  // namespace mita
