// Host-side launchers of the MiTA kernels (internal to libmita.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mita {

struct Shape {
  int B, H, grid_h, grid_w, d, m_h, m_w, k;
  int N, m, BH;
  bool bf16;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// step a1: landmark pooling
hipError_t launch_pool(const void* Q, float* ql, const Shape& s, hipStream_t st);

// steps a2-a4: landmark scores, per-row top-k, landmark values
size_t landmark_scratch_bytes(const Shape& s);
hipError_t launch_landmark(const float* ql, const void* K, const void* V, int32_t* idx,
                           float* vl, void* scratch, const Shape& s, hipStream_t st);

// steps a5-a6: routing and grouping
hipError_t launch_route(const void* Q, const float* ql, int32_t* route, const Shape& s,
                        hipStream_t st);
hipError_t launch_group(const int32_t* route, int32_t* counts, int32_t* offsets, int32_t* perm,
                        const Shape& s, hipStream_t st);

// step a7: grouped expert attention
hipError_t launch_attend(const void* Q, const void* K, const void* V, const float* ql,
                         const float* vl, const int32_t* idx, const int32_t* route,
                         const int32_t* offsets, const int32_t* perm, float* out,
                         const Shape& s, hipStream_t st);

// bf16 kernels for long grids (MFMA, LDS-staged)
hipError_t launch_pool_bf16(const void* Q, float* ql, const Shape& s, hipStream_t st);
bool landmark_bf16_supported(const Shape& s);
hipError_t launch_landmark_bf16(const float* ql, const void* K, const void* V, int32_t* idx,
                                float* vl, const Shape& s, hipStream_t st);
bool route_bf16_supported(const Shape& s);
size_t route_chist_bytes(const Shape& s);
hipError_t launch_route_bf16(const void* Q, const float* ql, int32_t* route, int32_t* chist,
                             const Shape& s, hipStream_t st);
hipError_t launch_group_bf16(const int32_t* route, const int32_t* chist, int32_t* counts,
                             int32_t* offsets, int32_t* perm, const Shape& s, hipStream_t st);
bool attend_bf16_supported(const Shape& s);
hipError_t launch_attend_bf16(const void* Q, const void* K, const void* V, const float* ql,
                              const float* vl, const int32_t* idx, const int32_t* offsets,
                              const int32_t* perm, float* out, const Shape& s, hipStream_t st);

// whole pass for short grids in one persistent kernel
bool fused_supported(const Shape& s);
hipError_t launch_fused(const void* Q, const void* K, const void* V, float* out, int32_t* idx,
                        int32_t* route, float* ql, float* vl, int32_t* counts, int32_t* offsets,
                        int32_t* perm, const Shape& s, hipStream_t st);

}  // namespace mita
