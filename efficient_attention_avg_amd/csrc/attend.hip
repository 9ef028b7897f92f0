// Step a7 -- grouped expert attention (page "NeurIPS'26：注意力也是FFN？...",
// landmark-query section, the s = 1 output, and Algorithm 1): a query routed
// to expert e attends the m shared entries (keys Q_L, values V_L) and the k
// raw entries of expert e (keys K[idx_e], values V[idx_e]) under ONE softmax
// over the m + k concatenated logits scaled by tau.  With s experts per query
// the routed part is the concatenation of its s experts' entries (no key
// merged); the route-only variant has no shared entries.
//
// Scalar schedule (fp32 inputs, and bf16 shapes past the matrix-core kernel's
// range): one wave per query.  The entries go by in chunks of 64 (lane = entry:
// one full dot product each), merged by online softmax; then lanes own
// output channels and sum the chunk's weighted value rows.  With s = 1 the
// queries are visited in grouped order (perm) so consecutive waves reuse one
// expert's rows from cache; with s > 1 in token order.
#include "common.h"
#include "internal.h"

namespace mita {

template <typename T>
__global__ __launch_bounds__(256) void attend_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ route, const int32_t* __restrict__ perm, float* __restrict__ out,
    int N, int m, int k, int s, int shared, float tau) {
  __shared__ float qs[4][kHeadDim];
  __shared__ float pw[4][64];
  __shared__ const void* prow[4][64];  // the value row of each entry of the chunk
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.y;
  const int p = blockIdx.x * 4 + wv;
  if (p >= N) return;  // (no block-wide barrier below)
  const int n = s == 1 ? perm[(size_t)bh * N + p] : p;
  qs[wv][lane] = to_f32(Q[((size_t)bh * N + n) * kHeadDim + lane]);
  __builtin_amdgcn_wave_barrier();
  const int ms = shared ? m : 0;
  const int E = ms + s * k;
  const int32_t* rt = route + ((size_t)bh * N + n) * s;
  const T* Kh = K + (size_t)bh * N * kHeadDim;
  const T* Vh = V + (size_t)bh * N * kHeadDim;
  float mref = -INFINITY, lsum = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < E; c0 += 64) {
    const int j = c0 + lane;
    float a = -INFINITY;
    const void* vrow = nullptr;
    if (j < E) {
      float dot = 0.f;
      if (j < ms) {
        const float* kr = ql + ((size_t)bh * m + j) * kHeadDim;
        for (int c = 0; c < kHeadDim; ++c) dot = fmaf(qs[wv][c], kr[c], dot);
        vrow = vl + ((size_t)bh * m + j) * kHeadDim;
      } else {
        const int jj = j - ms, e = rt[jj / k];
        const int key = idx[((size_t)bh * m + e) * k + jj % k];
        const T* kr = Kh + (size_t)key * kHeadDim;
        for (int c = 0; c < kHeadDim; ++c) dot = fmaf(qs[wv][c], to_f32(kr[c]), dot);
        vrow = Vh + (size_t)key * kHeadDim;
      }
      a = dot * tau;
    }
    const float mnew = fmaxf(mref, wave_max(a));  // finite: the chunk has an entry
    const float alpha = fast_exp(mref - mnew);
    const float pj = j < E ? fast_exp(a - mnew) : 0.f;
    lsum = lsum * alpha + wave_sum(pj);
    acc *= alpha;
    mref = mnew;
    pw[wv][lane] = pj;
    prow[wv][lane] = vrow;
    __builtin_amdgcn_wave_barrier();
    const int nc = min(64, E - c0);
    for (int t = 0; t < nc; ++t) {
      const float w = pw[wv][t];
      const float v = c0 + t < ms ? reinterpret_cast<const float*>(prow[wv][t])[lane]
                                  : to_f32(reinterpret_cast<const T*>(prow[wv][t])[lane]);
      acc = fmaf(w, v, acc);
    }
    __builtin_amdgcn_wave_barrier();
  }
  out[((size_t)bh * N + n) * kHeadDim + lane] = acc / lsum;
}

hipError_t launch_attend(const void* Q, const void* K, const void* V, const float* ql,
                         const float* vl, const int32_t* idx, const int32_t* route,
                         const int32_t* offsets, const int32_t* perm, float* out,
                         const Shape& s, hipStream_t st) {
  (void)offsets;
  dim3 grid((s.N + 3) / 4, s.BH);
  const float tau = 1.0f / sqrtf((float)s.d);
  const int sh = s.shared ? 1 : 0;
  if (s.bf16)
    attend_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)Q, (const bf16_t*)K,
                                                (const bf16_t*)V, ql, vl, idx, route, perm, out,
                                                s.N, s.m, s.k, s.s, sh, tau);
  else
    attend_kernel<float><<<grid, 256, 0, st>>>((const float*)Q, (const float*)K, (const float*)V,
                                               ql, vl, idx, route, perm, out, s.N, s.m, s.k, s.s,
                                               sh, tau);
  return hipGetLastError();
}

}  // namespace mita
