// Steps a2-a4 -- the landmark pass (page "NeurIPS'26：注意力也是FFN？...",
// landmark-query section): each landmark query is scored against every key,
// S = tau * Q_L K^T; its k best keys (ties to the lowest key id) form one
// routed expert; and the same scores, softmax-normalised over all N keys,
// weight V into the landmark value V_L (the shared expert's values).  The one
// score row feeds both the selection and the softmax, as the page notes.
//
// First schedule: one workgroup per (head, landmark).  The score row is kept
// in a scratch row in device memory (L2-resident while the workgroup runs);
// the k-th largest score is found by a 4-digit (8-bit) radix select over
// order-preserving keys, and the expert is the stable compaction of keys
// above that threshold plus the lowest-index ones equal to it.
#include "common.h"
#include "internal.h"

namespace mita {

template <typename T>
__global__ __launch_bounds__(256) void landmark_kernel(const float* __restrict__ ql,
                                                       const T* __restrict__ K,
                                                       const T* __restrict__ V,
                                                       int32_t* __restrict__ idx,
                                                       float* __restrict__ vl,
                                                       float* __restrict__ S, int N, int m, int k,
                                                       float tau) {
  const int i = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ float qs[kHeadDim];
  __shared__ float red[4];
  __shared__ float accs[4][kHeadDim];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t pick[2];
  __shared__ int wcnt[2][4];

  const size_t row = (size_t)bh * m + i;
  float* srow = S + row * N;
  const T* Kh = K + (size_t)bh * N * kHeadDim;
  const T* Vh = V + (size_t)bh * N * kHeadDim;
  if (tid < kHeadDim) qs[tid] = ql[row * kHeadDim + tid];
  __syncthreads();

  // a2: one score per key
  float mx = -INFINITY;
  for (int j = tid; j < N; j += 256) {
    const T* kr = Kh + (size_t)j * kHeadDim;
    float a = 0.f;
    for (int c = 0; c < kHeadDim; ++c) a = fmaf(qs[c], to_f32(kr[c]), a);
    a *= tau;
    srow[j] = a;
    mx = fmaxf(mx, a);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();

  // a4: softmax over all keys applied to V (wave wv takes keys wv, wv+4, ...)
  float acc = 0.f, psum = 0.f;
  for (int j = wv; j < N; j += 4) {
    const float p = fast_exp(srow[j] - mx);
    psum += p;
    acc = fmaf(p, to_f32(Vh[(size_t)j * kHeadDim + lane]), acc);
  }
  accs[wv][lane] = acc;
  if (lane == 0) red[wv] = psum;
  __syncthreads();
  if (tid < kHeadDim) {
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float a = (accs[0][tid] + accs[1][tid]) + (accs[2][tid] + accs[3][tid]);
    vl[row * kHeadDim + tid] = a / tot;
  }

  // a3: radix select of the k-th largest key, 8 bits at a time
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < N; j += 256) {
      const uint32_t u = score_key(srow[j]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, b = 255;
      for (; b > 0; --b) {
        if (cum + (int)hist[b] >= remaining) break;
        cum += (int)hist[b];
      }
      pick[0] = (uint32_t)b;
      pick[1] = (uint32_t)(remaining - cum);
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    pmask |= 255u << shift;
    remaining = (int)pick[1];
    __syncthreads();
  }
  const uint32_t T_key = prefix;  // the k-th largest key; take `remaining` of its ties

  // stable compaction in key order: all keys above T_key, then the lowest-id ties
  int base = 0, eq_seen = 0;
  int32_t* orow = idx + row * k;
  for (int j0 = 0; j0 < N; j0 += 256) {
    const int j = j0 + tid;
    const uint32_t u = j < N ? score_key(srow[j]) : 0u;
    const bool gt = j < N && u > T_key;
    const bool eq = j < N && u == T_key;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wcnt[0][wv] = __popcll(beq);
    __syncthreads();
    int eq_before = eq_seen;
    for (int w = 0; w < wv; ++w) eq_before += wcnt[0][w];
    const bool take = gt || (eq && eq_before + lanes_below(beq) < remaining);
    const uint64_t bt = __ballot(take);
    if (lane == 0) wcnt[1][wv] = __popcll(bt);
    __syncthreads();
    int pos = base;
    for (int w = 0; w < wv; ++w) pos += wcnt[1][w];
    if (take) orow[pos + lanes_below(bt)] = j;
    base += wcnt[1][0] + wcnt[1][1] + wcnt[1][2] + wcnt[1][3];
    eq_seen += wcnt[0][0] + wcnt[0][1] + wcnt[0][2] + wcnt[0][3];
    __syncthreads();
  }
}

size_t landmark_scratch_bytes(const Shape& s) {
  return align_up((size_t)s.BH * s.m * s.N * sizeof(float), 256);
}

hipError_t launch_landmark(const float* ql, const void* K, const void* V, int32_t* idx,
                           float* vl, void* scratch, const Shape& s, hipStream_t st) {
  dim3 grid(s.m, s.BH);
  const float tau = 1.0f / sqrtf((float)s.d);
  if (s.bf16)
    landmark_kernel<bf16_t><<<grid, 256, 0, st>>>(ql, (const bf16_t*)K, (const bf16_t*)V, idx, vl,
                                                  (float*)scratch, s.N, s.m, s.k, tau);
  else
    landmark_kernel<float><<<grid, 256, 0, st>>>(ql, (const float*)K, (const float*)V, idx, vl,
                                                 (float*)scratch, s.N, s.m, s.k, tau);
  return hipGetLastError();
}

}  // namespace mita
