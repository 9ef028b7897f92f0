// Step a1 -- landmark queries by 2-D adaptive average pooling of Q over the
// token grid (page "NeurIPS'26：注意力也是FFN？...", landmark-query section:
// m landmark queries come from local average pooling; the window rule is the
// standard adaptive one: rows [floor(r*gh/mh), ceil((r+1)*gh/mh)), same for
// columns, so windows overlap when the grid does not divide evenly).
//
// HBM-bound: every Q element is read once by the windows that cover it
// (overlapping windows re-read a few rows, from L2).  One workgroup per
// (head, landmark row r) covers all m_w landmarks of that row; a thread owns
// one channel pair so a wave reads whole 128-byte bf16 token rows.
#include "common.h"
#include "internal.h"

namespace mita {

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ Q, float* __restrict__ ql,
                                                   int gh, int gw, int mh, int mw) {
  const int r = blockIdx.x;          // landmark row
  const int bh = blockIdx.y;
  const int N = gh * gw, m = mh * mw;
  const T* q = Q + (size_t)bh * N * kHeadDim;
  int y0, y1;
  pool_window(r, gh, mh, &y0, &y1);
  // threads: (landmark column c, channel ch); loop if the block is too small
  for (int t = threadIdx.x; t < mw * kHeadDim; t += blockDim.x) {
    const int c = t / kHeadDim, ch = t % kHeadDim;
    int x0, x1;
    pool_window(c, gw, mw, &x0, &x1);
    float acc = 0.f;
    for (int y = y0; y < y1; ++y)
      for (int x = x0; x < x1; ++x) acc += to_f32(q[(size_t)(y * gw + x) * kHeadDim + ch]);
    const float cnt = (float)((y1 - y0) * (x1 - x0));
    ql[((size_t)bh * m + r * mw + c) * kHeadDim + ch] = acc / cnt;
  }
}

hipError_t launch_pool(const void* Q, float* ql, const Shape& s, hipStream_t st) {
  dim3 grid(s.m_h, s.BH);
  if (s.bf16)
    pool_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)Q, ql, s.grid_h, s.grid_w, s.m_h, s.m_w);
  else
    pool_kernel<float><<<grid, 256, 0, st>>>((const float*)Q, ql, s.grid_h, s.grid_w, s.m_h, s.m_w);
  return hipGetLastError();
}

}  // namespace mita
