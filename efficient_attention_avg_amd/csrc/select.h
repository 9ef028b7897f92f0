// Reductions and scans inside a 16-lane group (one DPP row) of a wavefront.
// All 16 lanes of a group must be active together: a DPP read of an inactive
// lane returns 0 instead of that lane's value.
#pragma once

#include "common.h"
#include "mfma.h"

namespace mita {

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
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

}  // namespace mita
