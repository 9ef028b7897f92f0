// Steps a5-a6 for bf16 inputs on long grids -- routing and grouping (page
// "NeurIPS'26：注意力也是FFN？...", landmark-query section: each query goes to
// the routed expert of its best-matching landmark, the query-landmark scores
// being the ones the shared expert reuses; Algorithm 1 groups the queries by
// route before attending).
//
// route_bf16_kernel: one workgroup per (head, 256-query chunk).  The head's
// Q_L is staged in LDS as bf16 hi + lo; R^T = Q_L Q^T runs on bf16 MFMA with
// fp32 accumulation (near-fp32 scores, so the argmax is decided at fp32
// accuracy); the argmax scans landmarks in increasing order with a strict '>'
// and combines lanes with ties to the lower landmark.  The chunk's route
// histogram goes to the workspace.
//
// group_bf16_kernel: one workgroup per head.  Chunk histograms -> per-expert
// counts and offsets -> per-chunk starting positions; each wave then places
// its chunks' queries stably: within a 64-query run, queries sharing a route
// are found by ballot and ranked by lane order.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace mita {
namespace rt {

constexpr int QC = 256;  // queries per route workgroup

__device__ __forceinline__ int rc(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

__global__ __launch_bounds__(256) void route_bf16_kernel(const uint16_t* __restrict__ Q,
                                                         const float* __restrict__ ql,
                                                         int32_t* __restrict__ route,
                                                         int32_t* __restrict__ chist, int N, int m,
                                                         int nchunks) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int mt = (m + 15) >> 4;  // landmark tiles
  char* qlh = sm;
  char* qll = sm + mt * 16 * 128;
  int* hist = reinterpret_cast<int*>(sm + 2 * mt * 16 * 128);
  const uint16_t* Qh = Q + (size_t)bh * N * 64;
  // this wave's four 16-query tiles: every Q row load is issued up front
  constexpr int TPW = QC / 16 / 4;
  u32x4 qb[TPW][2];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int n = chunk * QC + 16 * (w + 4 * i) + c16;
      qb[i][0] = n < N ? *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 8 * g) : z;
      qb[i][1] = n < N ? *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 32 + 8 * g) : z;
    }
  }
  // stage Q_L (rows past m are zero) as bf16 hi / lo, 128-byte swizzled rows
  for (int it = tid; it < mt * 16 * 16; it += 256) {
    const int row = it >> 4, q4 = it & 15;  // 4 channels per item
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < m) f = *reinterpret_cast<const float4*>(ql + ((size_t)bh * m + row) * 64 + 4 * q4);
    const float v[4] = {f.x, f.y, f.z, f.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = bf16_rne_bits(v[i]);
      l[i] = bf16_rne_bits(v[i] - bf16_bits_to_f32(h[i]));
    }
    const int off = rc(row, q4 >> 1) + (q4 & 1) * 8;
    *reinterpret_cast<u32x2*>(qlh + off) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *reinterpret_cast<u32x2*>(qll + off) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  }
  for (int e = tid; e < m; e += 256) hist[e] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tt = w + 4 * i;
    const int n = chunk * QC + 16 * tt + c16;  // this lane's query column
    const bool ok = n < N;
    const u32x4 b0 = qb[i][0], b1 = qb[i][1];
    float best = -INFINITY;
    int bi = 0;
    for (int lt = 0; lt < mt; ++lt) {
      const int row = 16 * lt + c16;
      const u32x4 ah0 = *reinterpret_cast<const u32x4*>(qlh + rc(row, g));
      const u32x4 al0 = *reinterpret_cast<const u32x4*>(qll + rc(row, g));
      const u32x4 ah1 = *reinterpret_cast<const u32x4*>(qlh + rc(row, 4 + g));
      const u32x4 al1 = *reinterpret_cast<const u32x4*>(qll + rc(row, 4 + g));
      f32x4 c = zero4();
      c = mfma_bf16(ah0, b0, c);
      c = mfma_bf16(al0, b0, c);
      c = mfma_bf16(ah1, b1, c);
      c = mfma_bf16(al1, b1, c);
      // lane holds R[query n][landmark 16lt + 4g + r]; landmarks rise with (lt, r)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int L = 16 * lt + 4 * g + r;
        if (L < m && c[r] > best) { best = c[r]; bi = L; }
      }
    }
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ov = __shfl_xor(best, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if (g == 0 && ok) {
      route[(size_t)bh * N + n] = bi;
      atomicAdd(&hist[bi], 1);
    }
  }
  __syncthreads();
  int32_t* dst = chist + ((size_t)bh * nchunks + chunk) * m;
  for (int e = tid; e < m; e += 256) dst[e] = hist[e];
}

__global__ __launch_bounds__(1024) void group_bf16_kernel(const int32_t* __restrict__ route,
                                                         const int32_t* __restrict__ chist,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm, int N, int m,
                                                         int nchunks) {
  extern __shared__ int gsm[];
  int* cur = gsm;                   // [nchunks][m]: next free position per chunk/expert
  int* tot = gsm + nchunks * m;     // [m]
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nt = blockDim.x, nw = nt >> 6;
  const int32_t* ch = chist + (size_t)bh * nchunks * m;
  // the chunk histograms into LDS in one coalesced sweep (independent loads),
  // then per expert: totals and each chunk's count before it
  for (int it = tid; it < nchunks * m; it += nt) cur[it] = ch[it];
  __syncthreads();
  for (int e = tid; e < m; e += nt) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = cur[c * m + e];
      cur[c * m + e] = run;
      run += v;
    }
    tot[e] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < m; ++e) {
      const int t = tot[e];
      offsets[(size_t)bh * (m + 1) + e] = run;
      counts[(size_t)bh * m + e] = t;
      tot[e] = run;  // now the expert's offset
      run += t;
    }
    offsets[(size_t)bh * (m + 1) + m] = run;
  }
  __syncthreads();
  for (int it = tid; it < nchunks * m; it += nt) cur[it] += tot[it % m];
  __syncthreads();
  // stable scatter: wave w takes chunks w, w + nw, ...; runs of 64 queries in order
  const int32_t* r = route + (size_t)bh * N;
  int32_t* pm = perm + (size_t)bh * N;
  for (int c = w; c < nchunks; c += nw) {
    int* cc = cur + c * m;
    for (int base = c * QC; base < min(N, (c + 1) * QC); base += 64) {
      const int n = base + lane;
      const int e = n < N ? r[n] : -1;
      uint64_t left = __ballot(e >= 0);
      while (left) {
        const int src = __ffsll((unsigned long long)left) - 1;
        const int v = __shfl(e, src, 64);
        const uint64_t same = __ballot(e == v);
        const int at = cc[v];  // read by every lane before the update below
        if (e == v) pm[at + __popcll(same & ((1ull << lane) - 1ull))] = n;
        __builtin_amdgcn_wave_barrier();
        if (lane == src) cc[v] = at + __popcll(same);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        left &= ~same;
      }
    }
  }
}

}  // namespace rt

bool route_bf16_supported(const Shape& s) {
  const size_t nchunks = (s.N + rt::QC - 1) / rt::QC;
  return s.bf16 && s.m <= 512 && (nchunks * s.m + s.m) * 4 <= 160 * 1024;
}

size_t route_chist_bytes(const Shape& s) {
  const int nchunks = (s.N + rt::QC - 1) / rt::QC;
  return (size_t)s.BH * nchunks * s.m * 4;
}

hipError_t launch_route_bf16(const void* Q, const float* ql, int32_t* route, int32_t* chist,
                             const Shape& s, hipStream_t st) {
  const int nchunks = (s.N + rt::QC - 1) / rt::QC;
  const int mt = (s.m + 15) / 16;
  const size_t lds = (size_t)2 * mt * 16 * 128 + (size_t)s.m * 4;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)rt::route_bf16_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  dim3 grid(nchunks, s.BH);
  rt::route_bf16_kernel<<<grid, 256, lds, st>>>((const uint16_t*)Q, ql, route, chist, s.N, s.m,
                                                nchunks);
  return hipGetLastError();
}

hipError_t launch_group_bf16(const int32_t* route, const int32_t* chist, int32_t* counts,
                             int32_t* offsets, int32_t* perm, const Shape& s, hipStream_t st) {
  const int nchunks = (s.N + rt::QC - 1) / rt::QC;
  const size_t lds = ((size_t)nchunks * s.m + s.m) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)rt::group_bf16_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  rt::group_bf16_kernel<<<s.BH, 1024, lds, st>>>(route, chist, counts, offsets, perm, s.N, s.m,
                                                 nchunks);
  return hipGetLastError();
}

}  // namespace mita
