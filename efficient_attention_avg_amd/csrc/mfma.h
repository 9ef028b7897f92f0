// CDNA4 (gfx950) matrix-core helpers: 16x16x32 bf16 / f16 MFMA with fp32
// accumulation.  Operand layout (wave64, l = lane, g = l/16, c = l%16):
//   A[16 x 32]: lane l holds A[c][8g + t], t < 8
//   B[32 x 16]: lane l holds B[8g + t][c], t < 8
//   D[16 x 16]: lane l holds D[4g + r][c], r < 4
// Only the pairing of A's and B's k slots matters, so any permutation of the
// 32 k indices applied to both operands gives the same product; the kernels
// use that to feed an accumulator straight back in as the next B operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mita {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// gfx950's transposing LDS read of 16-bit elements: in each 16-lane group,
// lane s points at four consecutive elements (row s >> 2 of a 4 x 16 tile,
// columns 4 (s & 3) ..), and lane t receives column t of the tile (rows
// 0 .. 3), i.e. four k values of an MFMA operand.  Used to read V^T
// fragments straight from V rows kept in LDS.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_tr16(const char* p) {
  const s16x4 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Byte offset of 16-byte chunk `c` (0..7) of a 128-byte row in LDS,
// XOR-swizzled so that 16 consecutive rows read at one logical chunk spread
// over the banks.
__device__ __forceinline__ int rc(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> f16 bits (round to nearest even).
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Two fp32 -> packed f16x2 (round to nearest even, one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  const f16x2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Two fp32 -> packed bf16x2 (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Pack two f16 bit patterns into one dword (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// A head's [N][64] bf16 rows as a raw buffer: 32-bit byte offsets, and an
// offset past the head's bytes reads zeros (the buffer range check), which
// stands in for padding rows without a branch or a select on the data.
// (N * 128 stays below 2^29 for N <= 2^22, so PAST is past every head.)
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int PAST = 0x40000000;
__device__ __forceinline__ Rsrc head_rows(const uint16_t* base, int N) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, N * 128, 0x00020000);
}
__device__ __forceinline__ u32x4 ld16(Rsrc r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// A head's [N][64] fp32 output rows as a raw buffer for stores: a store at an
// offset past the rows (PAST: N * 256 <= 2^30 for N <= 2^22) is dropped.
__device__ __forceinline__ Rsrc out_rows(float* base, int N) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, N * 256, 0x00020000);
}
// 16-byte store with the non-temporal hint (data not read again soon).
__device__ __forceinline__ void st16_nt(Rsrc r, f32x4 v, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 2);
}

}  // namespace mita
