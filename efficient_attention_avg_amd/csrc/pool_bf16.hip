// Step a1 for bf16 inputs on long grids -- landmark queries by 2-D adaptive
// average pooling of Q (page "NeurIPS'26：注意力也是FFN？...", landmark-query
// section: m landmark queries by local average pooling; windows are
// [floor(r*gh/mh), ceil((r+1)*gh/mh)) in each axis).
//
// grid_w <= 256: one workgroup per (head, landmark row r) reads the window rows
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
  // column sums over the window rows: item = (column x, 8-channel chunk c);
  // a thread's items go two at a time with all their row loads in flight
  for (int it0 = tid; it0 < gw * 8; it0 += 2 * blockDim.x) {
    float a[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) a[j][i] = 0.f;
    for (int y = y0; y < y1; y += 8) {
      uint4 v[2][8];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int it = it0 + j * blockDim.x, x = it >> 3, c = it & 7;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (it < gw * 8 && y + u < y1)
            v[j][u] = *reinterpret_cast<const uint4*>(q + (size_t)((y + u) * gw + x) * kHeadDim + 8 * c);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (it0 + j * (int)blockDim.x >= gw * 8 || y + u >= y1) continue;
          const uint32_t w[4] = {v[j][u].x, v[j][u].y, v[j][u].z, v[j][u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[j][2 * i] += __uint_as_float(w[i] << 16);
            a[j][2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
          }
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int it = it0 + j * blockDim.x, x = it >> 3, c = it & 7;
      if (it >= gw * 8) continue;
      float4* dst = reinterpret_cast<float4*>(colsum + x * kHeadDim + 8 * c);
      dst[0] = make_float4(a[j][0], a[j][1], a[j][2], a[j][3]);
      dst[1] = make_float4(a[j][4], a[j][5], a[j][6], a[j][7]);
    }
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

// Wide grids (grid_w > 256, e.g. one long row of tokens, where the column
// sums would not fit in LDS): one workgroup per (head, landmark) sums its own
// window.  Thread t takes channel chunk t & 7 (8 bf16, 16 bytes) of window
// cells t >> 3, t >> 3 + 32, ...; eight threads cover one 128-byte token row,
// so a 1-D window is read as one contiguous run.  Four cells per thread are in
// flight at once; the 32 partial sums per channel meet in LDS.
__global__ __launch_bounds__(256) void pool_window_bf16_kernel(const uint16_t* __restrict__ Q,
                                                               float* __restrict__ ql, int gh,
                                                               int gw, int mh, int mw) {
  __shared__ float part[32][kHeadDim + 4];
  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int r = i / mw, c = i - r * mw;
  const int N = gh * gw, m = mh * mw;
  int y0, y1, x0, x1;
  pool_window(r, gh, mh, &y0, &y1);
  pool_window(c, gw, mw, &x0, &x1);
  const int ww = x1 - x0, cells = (y1 - y0) * ww;
  const int ch = tid & 7, cg = tid >> 3;
  const uint16_t* q = Q + (size_t)bh * N * kHeadDim + 8 * ch;
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = 0.f;
  for (int c0 = cg; c0 < cells; c0 += 4 * 32) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cell = c0 + 32 * u;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      if (cell < cells) {
        const int y = y0 + cell / ww, x = x0 + cell % ww;
        v[u] = *reinterpret_cast<const uint4*>(q + (size_t)(y * gw + x) * kHeadDim);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[2 * j] += __uint_as_float(w[j] << 16);
        a[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[cg][8 * ch + j] = a[j];
  __syncthreads();
  if (tid < kHeadDim) {
    float acc = 0.f;
    for (int g = 0; g < 32; ++g) acc += part[g][tid];
    ql[((size_t)bh * m + i) * kHeadDim + tid] = acc / (float)cells;
  }
}

bool pool_bf16_wide(const Shape& s) { return s.grid_w > 256; }

hipError_t launch_pool_bf16(const void* Q, float* ql, const Shape& s, hipStream_t st) {
  if (pool_bf16_wide(s)) {
    dim3 grid(s.m, s.BH);
    pool_window_bf16_kernel<<<grid, 256, 0, st>>>((const uint16_t*)Q, ql, s.grid_h, s.grid_w,
                                                  s.m_h, s.m_w);
    return hipGetLastError();
  }
  dim3 grid(s.m_h, s.BH);
  const size_t lds = (size_t)s.grid_w * kHeadDim * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  pool_bf16_kernel<<<grid, 256, lds, st>>>((const uint16_t*)Q, ql, s.grid_h, s.grid_w, s.m_h,
                                           s.m_w);
  return hipGetLastError();
}

}  // namespace mita
