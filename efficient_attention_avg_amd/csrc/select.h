// Reductions and scans inside a 16-lane group (one DPP row) of a wavefront.
// All 16 lanes of a group must be active together: a DPP read of an inactive
// lane returns 0 instead of that lane's value.
#pragma once

#include "common.h"
#include "mfma.h"

namespace mita {

// (bound_ctrl set: a lane whose source is past the row's end reads 0, so no
// "old" value has to be materialised in the destination first)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
// quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror: after these four
// steps every lane of a 16-lane row holds the row's reduction.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// row_shl:n gives lane t the value of lane t+n of its row (zero past the end)
constexpr int kDppShl1 = 0x101, kDppShl2 = 0x102, kDppShl4 = 0x104, kDppShl8 = 0x108;

__device__ __forceinline__ float g16_maxf(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float g16_minf(float v) {
  v = fminf(v, dpp_f<kDppXor1>(v));
  v = fminf(v, dpp_f<kDppXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  return fminf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ int g16_maxi(int v) {
  v = max(v, dpp_i<kDppXor1>(v));
  v = max(v, dpp_i<kDppXor2>(v));
  v = max(v, dpp_i<kDppHalfMirror>(v));
  return max(v, dpp_i<kDppMirror>(v));
}
__device__ __forceinline__ int g16_addi(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  return v + dpp_i<kDppMirror>(v);
}
// inclusive suffix sum over the row: lane t gets sum over t' >= t
__device__ __forceinline__ int g16_suffix(int v) {
  v += dpp_i<kDppShl1>(v);
  v += dpp_i<kDppShl2>(v);
  v += dpp_i<kDppShl4>(v);
  return v + dpp_i<kDppShl8>(v);
}
__device__ __forceinline__ uint32_t g16_ballot(bool p, int g) {
  return (uint32_t)(__ballot(p) >> (16 * g)) & 0xFFFFu;
}
// This lane's 16-lane group's bits of a wave ballot.
__device__ __forceinline__ uint32_t g16_bits(uint64_t ballot, int g) {
  return (uint32_t)(ballot >> (16 * g)) & 0xFFFFu;
}
__device__ __forceinline__ float g16_sumf(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
// inclusive prefix sum over the row: lane t gets sum over t' <= t (row_shr:n
// hands lane t the value of lane t-n, zero before the row start)
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
__device__ __forceinline__ int g16_prefix(int v) {
  v += dpp_i<kDppShr1>(v);
  v += dpp_i<kDppShr2>(v);
  v += dpp_i<kDppShr4>(v);
  return v + dpp_i<kDppShr8>(v);
}
// (value, index) argmax over the row, ties to the lower index (empty lanes
// hold -inf and INT_MAX)
__device__ __forceinline__ void g16_argmax(float& v, int& i) {
#define MITA_G16_ARGMAX_STEP(CTRL)                 \
  {                                                \
    const float ov = dpp_f<CTRL>(v);               \
    const int oi = dpp_i<CTRL>(i);                 \
    if (ov > v || (ov == v && oi < i)) {           \
      v = ov;                                      \
      i = oi;                                      \
    }                                              \
  }
  MITA_G16_ARGMAX_STEP(kDppXor1)
  MITA_G16_ARGMAX_STEP(kDppXor2)
  MITA_G16_ARGMAX_STEP(kDppHalfMirror)
  MITA_G16_ARGMAX_STEP(kDppMirror)
#undef MITA_G16_ARGMAX_STEP
}

// Lane c16 <-> c16 ^ 8 of each 16-lane row (DPP row rotate by 8); the vector
// form moves each element by value (a bit cast applied to the element
// expression v[i] itself was compiled as a read of element 0).
constexpr int kDppRor8 = 0x128;
__device__ __forceinline__ int swap8(int v) { return dpp_i<kDppRor8>(v); }
__device__ __forceinline__ f32x4 swap8(f32x4 v) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __int_as_float(swap8(__float_as_int(v[i])));
  return r;
}

}  // namespace mita
