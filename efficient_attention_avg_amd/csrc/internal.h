// Host-side launchers of the MiTA kernels (internal to libmita.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace mita {

struct Shape {
  int B, H, grid_h, grid_w, d, m_h, m_w, k;
  int N, m, BH;
  bool bf16;
  int s = 1;            // experts per query
  bool shared = true;   // false: the route-only variant (no shared expert)
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Lets `kernel` take up to `bytes` of dynamic LDS on the current device, once
// per (kernel, device): `done` (one per kernel and byte count, at its launch
// site) holds a bit per device id below 64, set after the attribute call
// succeeded there.  The call costs about 5 us of host time, which on every
// launch left the GPU idle between dependent kernels.  Threads racing on a
// device's first launch both make the same idempotent call; devices with ids
// of 64 and up make it on every launch.
inline hipError_t allow_lds(const void* kernel, int bytes, std::atomic<unsigned long long>& done) {
  int dev = 0;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const unsigned long long bit = dev >= 0 && dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

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
// keys split over several workgroups need this much scratch (per-chunk
// candidates and V_L partials) for the merge kernel; 0 for one chunk
size_t landmark_bf16_scratch_bytes(const Shape& s);
// stats (optional, [BH][m]): each landmark row's softmax maximum (x, tau
// units) and sum (y) over all keys
hipError_t launch_landmark_bf16(const float* ql, const void* K, const void* V, int32_t* idx,
                                float* vl, void* scratch, const Shape& s, hipStream_t st,
                                float4* stats = nullptr);
bool route_bf16_supported(const Shape& s);
size_t route_chist_bytes(const Shape& s);
hipError_t launch_route_bf16(const void* Q, const float* ql, int32_t* route, int32_t* chist,
                             const Shape& s, hipStream_t st);
hipError_t launch_group_bf16(const int32_t* route, int32_t* chist, int32_t* counts,
                             int32_t* offsets, int32_t* perm, const Shape& s, hipStream_t st);
bool attend_bf16_supported(const Shape& s);
// s > 1: the attention kernel leaves per-item partial sums in `partial`
// (attend_partial_bytes) and launch_merge combines them into out
size_t attend_partial_bytes(const Shape& s);
hipError_t launch_attend_bf16(const void* Q, const void* K, const void* V, const float* ql,
                              const float* vl, const int32_t* idx, const int32_t* offsets,
                              const int32_t* perm, float* out, void* partial, const Shape& s,
                              hipStream_t st);
hipError_t launch_merge(const void* partial, float* out, const Shape& s, hipStream_t st);

// gradients of the pass (dQ, dK, dV) given the forward's intermediates
size_t backward_scratch_bytes(const Shape& s);
// where the backward scratch keeps the landmark rows' softmax statistics: the
// forward landmark pass may fill them (stats_ready), sparing a recomputation
float4* backward_stats(void* scratch, const Shape& s);
hipError_t launch_backward(const void* Q, const void* K, const void* V, const float* dout,
                           const float* ql, const float* vl, const int32_t* idx,
                           const int32_t* route, const int32_t* offsets, const int32_t* perm,
                           float* dq, float* dk, float* dv, void* scratch, const Shape& s,
                           hipStream_t st, bool stats_ready = false);

// whole pass for short grids in one persistent kernel
bool fused_supported(const Shape& s);
hipError_t launch_fused(const void* Q, const void* K, const void* V, float* out, int32_t* idx,
                        int32_t* route, float* ql, float* vl, int32_t* counts, int32_t* offsets,
                        int32_t* perm, const Shape& s, hipStream_t st);

}  // namespace mita
