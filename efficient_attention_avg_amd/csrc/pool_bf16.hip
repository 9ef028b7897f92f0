// Step a1 for bf16 inputs on long grids -- landmark queries by 2-D adaptive
// average pooling of Q (page "NeurIPS'26：注意力也是FFN？...", landmark-query
// section: m landmark queries by local average pooling; windows are
// [floor(r*gh/mh), ceil((r+1)*gh/mh)) in each axis).
//
// HBM-bound: one workgroup per (head, landmark row r) reads the window rows
// y0..y1 of Q once, with 16-byte loads that are contiguous across threads
// (8 threads cover one 128-byte token row).  Per-column window sums go to LDS,
// then each landmark of the row sums its column range.  Overlapping windows
// re-read a few rows from L2.
#include "common.h"
#include "internal.h"

namespace mita {

__global__ __launch_bounds__(256) void pool_bf16_kernel(const uint16_t* __restrict__ Q,
                                                        float* __restrict__ ql, int gh, int gw,
                                                        int mh, int mw) {
  extern __shared__ float colsum[];  // [gw][64]
  const int r = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int N = gh * gw, m = mh * mw;
  const uint16_t* q = Q + (size_t)bh * N * kHeadDim;
  int y0, y1;
  pool_window(r, gh, mh, &y0, &y1);
  // column sums over the window rows: item = (column x, 8-channel chunk c)
  for (int it = tid; it < gw * 8; it += blockDim.x) {
    const int x = it >> 3, c = it & 7;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // eight rows' loads in flight at a time
    for (int y = y0; y < y1; y += 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (y + u < y1) v[u] = *reinterpret_cast<const uint4*>(q + (size_t)((y + u) * gw + x) * kHeadDim + 8 * c);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (y + u >= y1) break;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[2 * i] += __uint_as_float(w[i] << 16);
          a[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
        }
      }
    }
    float4* dst = reinterpret_cast<float4*>(colsum + x * kHeadDim + 8 * c);
    dst[0] = make_float4(a[0], a[1], a[2], a[3]);
    dst[1] = make_float4(a[4], a[5], a[6], a[7]);
  }
  __syncthreads();
  const float rows = (float)(y1 - y0);
  for (int it = tid; it < mw * kHeadDim; it += blockDim.x) {
    const int c = it / kHeadDim, ch = it % kHeadDim;
    int x0, x1;
    pool_window(c, gw, mw, &x0, &x1);
    float acc = 0.f;
    for (int x = x0; x < x1; ++x) acc += colsum[x * kHeadDim + ch];
    ql[((size_t)bh * m + r * mw + c) * kHeadDim + ch] = acc / (rows * (float)(x1 - x0));
  }
}

hipError_t launch_pool_bf16(const void* Q, float* ql, const Shape& s, hipStream_t st) {
  dim3 grid(s.m_h, s.BH);
  const size_t lds = (size_t)s.grid_w * kHeadDim * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  pool_bf16_kernel<<<grid, 256, lds, st>>>((const uint16_t*)Q, ql, s.grid_h, s.grid_w, s.m_h,
                                           s.m_w);
  return hipGetLastError();
}

}  // namespace mita
