// Steps a5-a6 -- routing and grouping (page "NeurIPS'26：注意力也是FFN？...",
// landmark-query section: each query picks the routed expert of the landmark
// it matches best; Algorithm 1 then groups the queries by that route so each
// expert's keys are fetched once per group).
//
// route_n = argmax_i q_n . Q_L[i] with ties to the lowest i (a strict '>'
// scan in landmark order), or the s best landmarks in that order.  Grouping
// is a per-head stable counting sort of the routes (the N * s (query, rank)
// items when s > 1): histogram, exclusive scan, then an order-preserving
// scatter.
#include "common.h"
#include "internal.h"

namespace mita {

constexpr int kMaxS = 8;

// route[(bh * N + n) * s + j]: the j-th best landmark of query n (a strict '>'
// in landmark order keeps the lower id ahead of an equal score).
template <typename T>
__global__ __launch_bounds__(256) void route_kernel(const T* __restrict__ Q,
                                                    const float* __restrict__ ql,
                                                    int32_t* __restrict__ route, int N, int m,
                                                    int s) {
  const int bh = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const T* qr = Q + ((size_t)bh * N + n) * kHeadDim;
  float q[kHeadDim];
#pragma unroll
  for (int c = 0; c < kHeadDim; ++c) q[c] = to_f32(qr[c]);
  const float* L = ql + (size_t)bh * m * kHeadDim;
  float bv[kMaxS];
  int bi[kMaxS];
#pragma unroll
  for (int t = 0; t < kMaxS; ++t) {
    bv[t] = -INFINITY;
    bi[t] = 0;
  }
  for (int i = 0; i < m; ++i) {
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < kHeadDim; ++c) a = fmaf(q[c], L[i * kHeadDim + c], a);
    // sorted insertion into the first s slots
#pragma unroll
    for (int t = kMaxS - 1; t > 0; --t) {
      if (t >= s) continue;
      const bool up = a > bv[t - 1];
      const bool here = !up && a > bv[t];
      bv[t] = up ? bv[t - 1] : (here ? a : bv[t]);
      bi[t] = up ? bi[t - 1] : (here ? i : bi[t]);
    }
    if (a > bv[0]) {
      bv[0] = a;
      bi[0] = i;
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxS; ++t)
    if (t < s) route[((size_t)bh * N + n) * s + t] = bi[t];
}

__global__ __launch_bounds__(256) void group_kernel(const int32_t* __restrict__ route,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int N, int m) {
  extern __shared__ int gsm[];
  int* cnt = gsm;          // [m]
  int* cur = gsm + m;      // [m]
  int* cr = gsm + 2 * m;   // [256]
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int32_t* r = route + (size_t)bh * N;
  for (int e = tid; e < m; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int n = tid; n < N; n += 256) atomicAdd(&cnt[r[n]], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < m; ++e) {
      cur[e] = run;
      offsets[(size_t)bh * (m + 1) + e] = run;
      run += cnt[e];
    }
    offsets[(size_t)bh * (m + 1) + m] = run;
  }
  for (int e = tid; e < m; e += 256) counts[(size_t)bh * m + e] = cnt[e];
  __syncthreads();
  for (int n0 = 0; n0 < N; n0 += 256) {
    const int n = n0 + tid;
    const int e = n < N ? r[n] : -1;
    cr[tid] = e;
    __syncthreads();
    if (n < N) {
      int rank = 0;
      for (int j = 0; j < tid; ++j) rank += (cr[j] == e);
      perm[(size_t)bh * N + cur[e] + rank] = n;
    }
    __syncthreads();
    if (n < N) atomicAdd(&cur[e], 1);
    __syncthreads();
  }
}

hipError_t launch_route(const void* Q, const float* ql, int32_t* route, const Shape& s,
                        hipStream_t st) {
  if (s.s > kMaxS) return hipErrorInvalidValue;
  dim3 grid((s.N + 255) / 256, s.BH);
  if (s.bf16)
    route_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)Q, ql, route, s.N, s.m, s.s);
  else
    route_kernel<float><<<grid, 256, 0, st>>>((const float*)Q, ql, route, s.N, s.m, s.s);
  return hipGetLastError();
}

hipError_t launch_group(const int32_t* route, int32_t* counts, int32_t* offsets, int32_t* perm,
                        const Shape& s, hipStream_t st) {
  // the N * s (query, rank) items in item order t = n * s + j
  const size_t lds = (size_t)(2 * s.m + 256) * sizeof(int);
  group_kernel<<<s.BH, 256, lds, st>>>(route, counts, offsets, perm, s.N * s.s, s.m);
  return hipGetLastError();
}

}  // namespace mita
