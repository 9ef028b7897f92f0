// Step a7 -- grouped expert attention (page "NeurIPS'26：注意力也是FFN？...",
// landmark-query section, the s = 1 output, and Algorithm 1): a query routed
// to expert e attends the m shared entries (keys Q_L, values V_L) and the k
// raw entries of expert e (keys K[idx_e], values V[idx_e]) under ONE softmax
// over the m + k concatenated logits scaled by tau.
//
// First schedule: one wave per query, queries visited in grouped order (perm)
// so consecutive waves reuse the same expert rows from cache.  Lanes first
// own logits (one full dot product each), then own output channels.
#include "common.h"
#include "internal.h"

namespace mita {

template <typename T>
__global__ __launch_bounds__(256) void attend_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ route, const int32_t* __restrict__ perm, float* __restrict__ out,
    int N, int m, int k, float tau) {
  extern __shared__ float asm_[];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = m + k;
  float* qs = asm_ + wv * (kHeadDim + E);
  float* lg = qs + kHeadDim;
  const int bh = blockIdx.y;
  const int p = blockIdx.x * 4 + wv;
  const bool valid = p < N;
  int n = 0, e = 0;
  if (valid) {
    n = perm[(size_t)bh * N + p];
    e = route[(size_t)bh * N + n];
    qs[lane] = to_f32(Q[((size_t)bh * N + n) * kHeadDim + lane]);
  }
  __syncthreads();
  const int32_t* irow = idx + ((size_t)bh * m + e) * k;
  if (valid) {
    for (int j = lane; j < E; j += kWave) {
      float a = 0.f;
      if (j < m) {
        const float* kr = ql + ((size_t)bh * m + j) * kHeadDim;
        for (int c = 0; c < kHeadDim; ++c) a = fmaf(qs[c], kr[c], a);
      } else {
        const T* kr = K + ((size_t)bh * N + irow[j - m]) * kHeadDim;
        for (int c = 0; c < kHeadDim; ++c) a = fmaf(qs[c], to_f32(kr[c]), a);
      }
      lg[j] = a * tau;
    }
  }
  __syncthreads();
  float ps = 0.f;
  if (valid) {
    float mx = -INFINITY;
    for (int j = lane; j < E; j += kWave) mx = fmaxf(mx, lg[j]);
    mx = wave_max(mx);
    for (int j = lane; j < E; j += kWave) {
      const float pj = fast_exp(lg[j] - mx);
      lg[j] = pj;
      ps += pj;
    }
    ps = wave_sum(ps);
  }
  __syncthreads();
  if (valid) {
    float acc = 0.f;
    const float* vrow = vl + (size_t)bh * m * kHeadDim + lane;
    for (int j = 0; j < m; ++j) acc = fmaf(lg[j], vrow[(size_t)j * kHeadDim], acc);
    const T* vh = V + (size_t)bh * N * kHeadDim + lane;
    for (int j = 0; j < k; ++j) acc = fmaf(lg[m + j], to_f32(vh[(size_t)irow[j] * kHeadDim]), acc);
    out[((size_t)bh * N + n) * kHeadDim + lane] = acc / ps;
  }
}

hipError_t launch_attend(const void* Q, const void* K, const void* V, const float* ql,
                         const float* vl, const int32_t* idx, const int32_t* route,
                         const int32_t* offsets, const int32_t* perm, float* out,
                         const Shape& s, hipStream_t st) {
  (void)offsets;
  dim3 grid((s.N + 3) / 4, s.BH);
  const size_t lds = (size_t)4 * (kHeadDim + s.m + s.k) * sizeof(float);
  const float tau = 1.0f / sqrtf((float)s.d);
  if (s.bf16)
    attend_kernel<bf16_t><<<grid, 256, lds, st>>>((const bf16_t*)Q, (const bf16_t*)K,
                                                  (const bf16_t*)V, ql, vl, idx, route, perm,
                                                  out, s.N, s.m, s.k, tau);
  else
    attend_kernel<float><<<grid, 256, lds, st>>>((const float*)Q, (const float*)K,
                                                 (const float*)V, ql, vl, idx, route, perm, out,
                                                 s.N, s.m, s.k, tau);
  return hipGetLastError();
}

}  // namespace mita
