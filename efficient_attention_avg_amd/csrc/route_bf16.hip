// Steps a5-a6 for bf16 inputs on long grids -- routing and grouping (page
// "NeurIPS'26：注意力也是FFN？...", landmark-query section: each query goes to
// the routed expert of its best-matching landmark, the query-landmark scores
// being the ones the shared expert reuses; Algorithm 1 groups the queries by
// route before attending).
//
// route_bf16_kernel: a few workgroups per head, each owning a chunk of qc
// queries (a multiple of the run length R, itself a multiple of 64).  The head's Q_L is staged once in LDS as bf16
// hi + lo; R^T = Q_L Q^T runs on bf16 MFMA with fp32 accumulation
// (near-fp32 scores, so the argmax is decided at fp32 accuracy); the argmax
// scans landmarks in increasing order with a strict '>' and combines lanes
// with ties to the lower landmark.  Each of the eight waves walks its
// 16-query tiles with the next tile's Q rows already loading; routes collect
// in LDS and go out once, with the route histogram of each R-query run, at
// the end.
//
// group_bf16_kernel: one workgroup per head.  Run histograms -> per-expert
// counts and offsets -> per-run starting positions; the sixteen waves then
// place the runs' queries stably, 64 at a time: queries sharing a route are
// found by ballot and ranked by lane order.  With few heads (fewer than 128)
// the workgroup only writes the starting positions back over the run
// histograms, and group_place_kernel places each run's queries with a wave
// of its own, so that the placement spreads over the GPU.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace mita {
namespace rt {



constexpr int RW = 8;  // waves per route workgroup

// A lane's best landmarks for its query column, best first (MS slots; the
// first s of them are the answer): landmarks arrive in increasing id order,
// so a strict '>' keeps the lower id ahead of an equal score.
template <int MS>
struct TopS {
  float v[MS];
  int i[MS];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int t = 0; t < MS; ++t) {
      v[t] = -INFINITY;
      i[t] = 0x7FFFFFFF;
    }
  }
  __device__ __forceinline__ void insert(float x, int L) {
#pragma unroll
    for (int t = MS - 1; t > 0; --t) {
      const bool up = x > v[t - 1];           // x goes above slot t - 1
      const bool here = !up && x > v[t];
      v[t] = up ? v[t - 1] : (here ? x : v[t]);
      i[t] = up ? i[t - 1] : (here ? L : i[t]);
    }
    const bool top = x > v[0];
    v[0] = top ? x : v[0];
    i[0] = top ? L : i[0];
  }
  // drops slot 0 (taken by the merge)
  __device__ __forceinline__ void pop(bool p) {
#pragma unroll
    for (int t = 0; t < MS - 1; ++t) {
      v[t] = p ? v[t + 1] : v[t];
      i[t] = p ? i[t + 1] : i[t];
    }
    v[MS - 1] = p ? -INFINITY : v[MS - 1];
    i[MS - 1] = p ? 0x7FFFFFFF : i[MS - 1];
  }
};

// Best (score, id) of the four lane groups holding one query's landmarks,
// ties to the lower landmark id.
__device__ __forceinline__ void best_of_groups(float& v, int& i) {
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// MS = 1: the argmax; MS > 1: the best s <= MS landmarks per query, written
// best first as items t = n * s + j.
template <int MS>
__global__ __launch_bounds__(64 * RW) void route_bf16_kernel(const uint16_t* __restrict__ Q,
                                                         const float* __restrict__ ql,
                                                         int32_t* __restrict__ route,
                                                         int32_t* __restrict__ chist, int N, int m,
                                                         int nruns, int qc, int R, int s) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int mt = (m + 15) >> 4;  // landmark tiles
  char* qlh = sm;
  char* qll = sm + mt * 16 * 128;
  const int cruns = qc / R;  // runs per chunk
  int* hist = reinterpret_cast<int*>(sm + 2 * mt * 16 * 128);  // [cruns][m] (items per run)
  int* rbuf = hist + cruns * m;  // the chunk's routes, s per query
  const uint16_t* Qh = Q + (size_t)bh * N * 64;
  const int base = chunk * qc, ntile = qc >> 4;
  // Q_L (rows past m are zero): all of this thread's loads first, before the
  // Q rows (vector memory counters drain in issue order)
  constexpr int SU = 4;  // staging items per thread (up to 128 landmark rows)
  float4 qlv[SU];
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int it = tid + 64 * RW * u, row = it >> 4, q4 = it & 15;
    qlv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (it < mt * 16 * 16 && row < m)
      qlv[u] = *reinterpret_cast<const float4*>(ql + ((size_t)bh * m + row) * 64 + 4 * q4);
  }
  // the first tile's Q rows (B operand: lane = query column c16, channels
  // 8g.. and 32 + 8g..)
  const u32x4 z = {0u, 0u, 0u, 0u};
  auto load_q = [&](int tt, u32x4& b0, u32x4& b1) {
    const int n = base + 16 * tt + c16;
    b0 = n < N ? *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 8 * g) : z;
    b1 = n < N ? *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 32 + 8 * g) : z;
  };
  u32x4 nb0, nb1;
  load_q(w, nb0, nb1);
  // ... then as bf16 hi / lo into 128-byte swizzled rows
#pragma unroll
  for (int u = 0; u < SU; ++u) {
    const int it = tid + 64 * RW * u, row = it >> 4, q4 = it & 15;
    if (it >= mt * 16 * 16) break;
    const float v[4] = {qlv[u].x, qlv[u].y, qlv[u].z, qlv[u].w};
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
  // landmark tiles beyond what the unrolled items cover (m > 128)
  for (int it = tid + 64 * RW * SU; it < mt * 16 * 16; it += 64 * RW) {
    const int row = it >> 4, q4 = it & 15;
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
  for (int e = tid; e < cruns * m; e += 64 * RW) hist[e] = 0;
  __syncthreads();
  for (int tt = w; tt < ntile; tt += RW) {
    const int n = base + 16 * tt + c16;  // this lane's query column
    const bool ok = n < N;
    const u32x4 b0 = nb0, b1 = nb1;
    if (tt + RW < ntile) load_q(tt + RW, nb0, nb1);
    float best = -INFINITY;
    int bi = 0;
    TopS<MS> top;
    if constexpr (MS > 1) top.init();
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
        if constexpr (MS == 1) {
          if (L < m && c[r] > best) { best = c[r]; bi = L; }
        } else {
          top.insert(L < m ? c[r] : -INFINITY, L < m ? L : 0x7FFFFFFF);
        }
      }
    }
    if constexpr (MS == 1) {
      best_of_groups(best, bi);
      if (g == 0 && ok) {
        rbuf[16 * tt + c16] = bi;
        atomicAdd(&hist[(16 * tt / R) * m + bi], 1);
      }
    } else {
      // s rounds: the best head of the four groups' lists is the next route;
      // the group holding it drops it
      for (int j = 0; j < s; ++j) {
        float v = top.v[0];
        int i = top.i[0];
        best_of_groups(v, i);
        top.pop(top.i[0] == i);
        // (an empty slot can win only when scores are NaN; keep the id in
        // range so such input cannot index past the histogram)
        i = i < m ? i : m - 1;
        if (g == 0 && ok) {
          rbuf[(16 * tt + c16) * s + j] = i;
          atomicAdd(&hist[(16 * tt / R) * m + i], 1);
        }
      }
    }
  }
  __syncthreads();
  const int nq = min(qc, N - base) * s;
  for (int i = tid; i < nq; i += 64 * RW) route[((size_t)bh * N + base) * s + i] = rbuf[i];
  const int run0 = chunk * cruns, nr = min(cruns, nruns - run0);
  int32_t* dst = chist + ((size_t)bh * nruns + run0) * m;
  for (int e = tid; e < nr * m; e += 64 * RW) dst[e] = hist[e];
}

// PLACE: place the queries here (else write each run's starting positions
// over its histogram for group_place_kernel).
template <bool PLACE>
__global__ __launch_bounds__(1024) void group_bf16_kernel(const int32_t* __restrict__ route,
                                                         int32_t* __restrict__ chist,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm, int N, int m,
                                                         int nchunks, int qc) {
  // here a "chunk" is one run of qc = R queries
  extern __shared__ int gsm[];
  int* cur = gsm;                   // [nchunks][m]: next free position per chunk/expert
  int* tot = gsm + nchunks * m;     // [m]
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nt = blockDim.x, nw = nt >> 6;
  int32_t* ch = chist + (size_t)bh * nchunks * m;
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
  if (!PLACE) {
    for (int it = tid; it < nchunks * m; it += nt) ch[it] = cur[it];
    return;
  }
  __syncthreads();
  // stable scatter: wave w takes chunks w, w + nw, ...; runs of 64 queries in order
  const int32_t* r = route + (size_t)bh * N;
  int32_t* pm = perm + (size_t)bh * N;
  for (int c = w; c < nchunks; c += nw) {
    int* cc = cur + c * m;
    for (int base = c * qc; base < min(N, (c + 1) * qc); base += 64) {
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

// One wave per (run, head): the run's qc items placed stably from its
// starting positions (written by group_bf16_kernel<false>), 64 at a time,
// with the routes of the next GU steps requested together.
constexpr int GU = 4;

__global__ __launch_bounds__(64) void group_place_kernel(const int32_t* __restrict__ route,
                                                         const int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ perm, int N, int m,
                                                         int nruns, int qc) {
  extern __shared__ int cc[];  // [m]: next free position per expert
  const int run = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int32_t* ps = pos + ((size_t)bh * nruns + run) * m;
  for (int e = lane; e < m; e += 64) cc[e] = ps[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int32_t* r = route + (size_t)bh * N;
  int32_t* pm = perm + (size_t)bh * N;
  const int lo = run * qc, hi = min(N, lo + qc);
  for (int b0 = lo; b0 < hi; b0 += 64 * GU) {
    int ev[GU];
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int n = b0 + 64 * u + lane;
      ev[u] = n < hi ? r[n] : -1;
    }
#pragma unroll
    for (int u = 0; u < GU; ++u) {
      const int n = b0 + 64 * u + lane, e = ev[u];
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

// Grouping in two kernels (starting positions per head, then one wave per
// run placing its queries) when there are too few heads for one workgroup
// per head to fill the GPU.
static bool group_split(const Shape& s) { return s.BH < 128; }

// Run length R: a multiple of 64, doubled until a head's run histograms fit
// in 64 KB of LDS (128 KB when the grouping is split: that workgroup then
// holds nothing else, and shorter runs give the routing and placement
// kernels more workgroups).  Queries per route workgroup qc: a multiple of R
// such that about 768 workgroups cover all heads.
static void route_chunking(const Shape& s, int& qc, int& nchunks, int& R, int& nruns) {
  const size_t budget = (group_split(s) ? 128 : 64) * 1024;
  R = 64;
  while ((size_t)((s.N + R - 1) / R) * s.m * 4 > budget && R < s.N) R *= 2;
  nruns = (s.N + R - 1) / R;
  int parts = (768 + s.BH - 1) / s.BH;
  if (parts > nruns) parts = nruns;
  if (parts < 1) parts = 1;
  qc = (((s.N + parts - 1) / parts) + R - 1) / R * R;
  nchunks = (s.N + qc - 1) / qc;
}

static size_t route_lds(const Shape& s, int qc, int R) {
  const int mt = (s.m + 15) / 16;
  return (size_t)2 * mt * 16 * 128 + (size_t)(qc / R) * s.m * 4 + (size_t)qc * s.s * 4;
}

bool route_bf16_supported(const Shape& s) {
  int qc, nchunks, R, nruns;
  route_chunking(s, qc, nchunks, R, nruns);
  return s.bf16 && s.m <= 512 && s.s <= 8 && ((size_t)nruns * s.m + s.m) * 4 <= 160 * 1024 &&
         route_lds(s, qc, R) <= 160 * 1024;
}

size_t route_chist_bytes(const Shape& s) {
  int qc, nchunks, R, nruns;
  route_chunking(s, qc, nchunks, R, nruns);
  return (size_t)s.BH * nruns * s.m * 4;
}

hipError_t launch_route_bf16(const void* Q, const float* ql, int32_t* route, int32_t* chist,
                             const Shape& s, hipStream_t st) {
  int qc, nchunks, R, nruns;
  route_chunking(s, qc, nchunks, R, nruns);
  const size_t lds = route_lds(s, qc, R);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  // the smallest list that holds s routes
  const int form = s.s == 1 ? 0 : s.s == 2 ? 1 : s.s <= 4 ? 2 : 3;
  auto kernel = form == 0 ? rt::route_bf16_kernel<1>
                : form == 1 ? rt::route_bf16_kernel<2>
                : form == 2 ? rt::route_bf16_kernel<4> : rt::route_bf16_kernel<8>;
  static std::atomic<unsigned long long> lds_set[4];
  if (const hipError_t e = allow_lds((const void*)kernel, 160 * 1024, lds_set[form]); e != hipSuccess)
    return e;
  dim3 grid(nchunks, s.BH);
  kernel<<<grid, 64 * rt::RW, lds, st>>>((const uint16_t*)Q, ql, route, chist, s.N, s.m, nruns,
                                         qc, R, s.s);
  return hipGetLastError();
}

hipError_t launch_group_bf16(const int32_t* route, int32_t* chist, int32_t* counts,
                             int32_t* offsets, int32_t* perm, const Shape& s, hipStream_t st) {
  int qc, nchunks, R, nruns;
  route_chunking(s, qc, nchunks, R, nruns);
  const size_t lds = ((size_t)nruns * s.m + s.m) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const bool split = group_split(s);
  auto kernel = split ? rt::group_bf16_kernel<false> : rt::group_bf16_kernel<true>;
  static std::atomic<unsigned long long> lds_set[2];
  if (const hipError_t e = allow_lds((const void*)kernel, 160 * 1024, lds_set[split ? 1 : 0]);
      e != hipSuccess)
    return e;
  // the sort runs over the N * s (query, rank) items, R * s of them per run
  kernel<<<s.BH, 1024, lds, st>>>(route, chist, counts, offsets, perm, s.N * s.s, s.m, nruns,
                                  R * s.s);
  if (!split) return hipGetLastError();
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  rt::group_place_kernel<<<dim3(nruns, s.BH), 64, (size_t)s.m * 4, st>>>(
      route, chist, perm, s.N * s.s, s.m, nruns, R * s.s);
  return hipGetLastError();
}

}  // namespace mita
