// Gradients of the MiTA pass: dQ, dK, dV of sum(dOut * out), with the top-k
// sets and routes of the forward held fixed (they are discrete choices,
// constant under small changes of the inputs).  The pages time training
// with this attention (page "NeurIPS'26：注意力也是FFN？...", long-sequence
// section, Table 5 and the route-only ablation) but do not describe its
// backward; it is the chain rule through the forward's steps in reverse:
//   7  out_n = sum_j w_nj val_j, w_n = softmax(tau q_n . key_j) over the
//      query's entries (the m shared ones with keys Q_L and values V_L, and
//      its experts' k routed ones with keys K[idx], values V[idx]):
//        dz_nj = tau w_nj (dOut_n . val_j - dOut_n . out_n)
//        dq_n += sum_j dz_nj key_j,  dkey_j += dz_nj q_n,  dval_j += w_nj dOut_n
//   4  V_L = A V, A = softmax_row(S), S = tau Q_L K^T:
//        dS_ij = A_ij (dV_L_i . V_j - dV_L_i . V_L_i)
//        dV += A^T dV_L,  dQ_L += tau dS K,  dK += tau dS^T Q_L
//   1  Q_L = window means of Q:  dQ_t += sum over windows i holding t of
//      dQ_L_i / |window i|.
//
// Kernels (fp32 accumulation, fp32 gradients; inputs bf16 or fp32):
//   tile      (s = 1, at most 128 entry columns) the query, expert and shared
//             steps below in one kernel on MFMA: workgroups walk a head's
//             experts, 16 queries at a time; otherwise:
//   query     one wave per query: two sweeps over its entries in chunks of
//             64 (lane = entry for dot products, lane = channel for sums):
//             the softmax and out_n (online), then w and dz per entry, which
//             go to a per-entry buffer, and dq_n;
//   expert    one workgroup per (head, expert): its key slots' dK and dV
//             rows summed over the expert's (query, rank) items from that
//             buffer, then added to dK, dV with one atomic per element (an
//             expert's keys may be another expert's too);
//   shared    dQ_L, dV_L from the buffer's shared entries, per 16 landmarks;
//   landmark  (m <= 64) on fp32 MFMA, per run of four 64-key blocks: A and
//             dS for every landmark, the blocks' dV and dK rows (owned by the
//             workgroup, added in place) and its share of dQ_L (one atomic
//             per element); for m > 64 a scalar form per 64-key block, after
//   stats     each landmark row's softmax maximum and sum over all keys (the
//             forward's MFMA landmark pass leaves them when it runs);
//   pool      dQ += each token's windows' dQ_L.
// Float additions into global memory use the hardware's float atomics
// (unsafeAtomicAdd: the buffers are ordinary device memory, where they are
// exact adds), not a compare-and-swap loop.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

#include <algorithm>
#include <type_traits>

namespace mita {
namespace bwd {

// a . row over 64 channels (`a` in LDS, read by every lane of the wave alike;
// one row per lane).  (16-byte row loads measured slower: 2.0 -> 2.5 ms.)
template <typename T>
__device__ __forceinline__ float dot64(const float* a, const T* row) {
  float acc = 0.f;
#pragma unroll 16
  for (int c = 0; c < kHeadDim; ++c) acc = fmaf(a[c], to_f32(row[c]), acc);
  return acc;
}

// Where entry j of query n lives: its key and value rows (fp32 for the shared
// entries, T for the routed ones).
template <typename T>
struct Entry {
  const void* key;
  const void* val;
  bool sh;
};

template <typename T>
__device__ __forceinline__ Entry<T> entry_of(int j, int ms, int k, const float* qlh,
                                             const float* vlh, const int32_t* rt,
                                             const int32_t* idxh, const T* Kh, const T* Vh) {
  Entry<T> e;
  if (j < ms) {
    e.key = qlh + (size_t)j * kHeadDim;
    e.val = vlh + (size_t)j * kHeadDim;
    e.sh = true;
  } else {
    const int jj = j - ms;
    const int key = idxh[(size_t)rt[jj / k] * k + jj % k];
    e.key = Kh + (size_t)key * kHeadDim;
    e.val = Vh + (size_t)key * kHeadDim;
    e.sh = false;
  }
  return e;
}

template <typename T>
__device__ __forceinline__ float dot_entry(const float* a, const void* row, bool sh) {
  return sh ? dot64<float>(a, reinterpret_cast<const float*>(row))
            : dot64<T>(a, reinterpret_cast<const T*>(row));
}

template <typename T>
__device__ __forceinline__ float elem(const void* row, bool sh, int c) {
  return sh ? reinterpret_cast<const float*>(row)[c] : to_f32(reinterpret_cast<const T*>(row)[c]);
}

// ---------------------------------------------------------------- query
template <typename T>
__global__ __launch_bounds__(256) void query_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ route, const int32_t* __restrict__ perm,
    const float* __restrict__ dout, float* __restrict__ dq, float2* __restrict__ G, int N, int m,
    int k, int s, int shared, float tau) {
  __shared__ float qs[4][kHeadDim];
  __shared__ float gs[4][kHeadDim];
  __shared__ float pw[4][64];
  __shared__ const void* prow[4][64];
  __shared__ bool psh[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bh = blockIdx.y;
  const int p = blockIdx.x * 4 + wv;
  if (p >= N) return;  // (wave-level synchronisation only below)
  // s = 1: queries in grouped order, so that neighbouring waves read one
  // expert's rows from cache
  const int n = s == 1 ? perm[(size_t)bh * N + p] : p;
  const size_t row = (size_t)bh * N + n;
  qs[wv][lane] = to_f32(Q[row * kHeadDim + lane]);
  const float g = dout[row * kHeadDim + lane];
  gs[wv][lane] = g;
  __builtin_amdgcn_wave_barrier();
  const int ms = shared ? m : 0, E = ms + s * k;
  const float* qlh = ql + (size_t)bh * m * kHeadDim;
  const float* vlh = vl + (size_t)bh * m * kHeadDim;
  const int32_t* rt = route + row * s;
  const int32_t* idxh = idx + (size_t)bh * m * k;
  const T* Kh = K + (size_t)bh * N * kHeadDim;
  const T* Vh = V + (size_t)bh * N * kHeadDim;
  // sweep 1: the softmax's maximum and sum, and out_n (lane = channel)
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < E; c0 += 64) {
    const int j = c0 + lane;
    float a = -INFINITY;
    Entry<T> e{nullptr, nullptr, false};
    if (j < E) {
      e = entry_of<T>(j, ms, k, qlh, vlh, rt, idxh, Kh, Vh);
      a = tau * dot_entry<T>(qs[wv], e.key, e.sh);
    }
    const float mnew = fmaxf(M, wave_max(a));
    const float alpha = fast_exp(M - mnew);
    const float p = j < E ? fast_exp(a - mnew) : 0.f;
    L = L * alpha + wave_sum(p);
    acc *= alpha;
    M = mnew;
    pw[wv][lane] = p;
    prow[wv][lane] = e.val;
    psh[wv][lane] = e.sh;
    __builtin_amdgcn_wave_barrier();
    const int nc = min(64, E - c0);
#pragma unroll 8
    for (int t = 0; t < nc; ++t) acc = fmaf(pw[wv][t], elem<T>(prow[wv][t], psh[wv][t], lane), acc);
    __builtin_amdgcn_wave_barrier();
  }
  const float inv = 1.0f / L;
  const float D = wave_sum(acc * inv * g);  // dOut_n . out_n
  // sweep 2: w and dz per entry (to the buffer), dq_n (lane = channel)
  float dqa = 0.f;
  float2* Gr = G + row * E;
  for (int c0 = 0; c0 < E; c0 += 64) {
    const int j = c0 + lane;
    float dz = 0.f;
    Entry<T> e{nullptr, nullptr, false};
    if (j < E) {
      e = entry_of<T>(j, ms, k, qlh, vlh, rt, idxh, Kh, Vh);
      const float a = tau * dot_entry<T>(qs[wv], e.key, e.sh);
      const float w = fast_exp(a - M) * inv;
      const float dw = dot_entry<T>(gs[wv], e.val, e.sh);
      dz = tau * w * (dw - D);
      Gr[j] = make_float2(w, dz);
    }
    pw[wv][lane] = dz;
    prow[wv][lane] = e.key;
    psh[wv][lane] = e.sh;
    __builtin_amdgcn_wave_barrier();
    const int nc = min(64, E - c0);
#pragma unroll 8
    for (int t = 0; t < nc; ++t) dqa = fmaf(pw[wv][t], elem<T>(prow[wv][t], psh[wv][t], lane), dqa);
    __builtin_amdgcn_wave_barrier();
  }
  dq[row * kHeadDim + lane] = dqa;
}

// ---------------------------------------------------------------- expert
// Workgroup (expert e, head bh); 64 key slots at a time: wave w takes slots
// 16 w .. 16 w + 15 and lane c channel c, summing dz q and w dOut over the
// expert's items (staged 16 at a time); each slot's row then goes out as one
// atomic instruction over 64 contiguous floats (two cache lines).
template <typename T>
__global__ __launch_bounds__(256) void expert_kernel(
    const T* __restrict__ Q, const float* __restrict__ dout, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float2* __restrict__ G, float* __restrict__ dK, float* __restrict__ dV, int N, int m,
    int k, int s, int ms) {
  constexpr int IT = 16;
  __shared__ float qs[IT][kHeadDim];
  __shared__ float gs[IT][kHeadDim];
  __shared__ float2 ws[IT][64];
  const int e = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int E = ms + s * k;
  const int q0 = offsets[(size_t)bh * (m + 1) + e], cnt = offsets[(size_t)bh * (m + 1) + e + 1] - q0;
  if (cnt == 0) return;
  const int32_t* ph = perm + (size_t)bh * N * s + q0;
  const int lane = tid & 63, w = tid >> 6;
  for (int j0 = 0; j0 < k; j0 += 64) {
    float ak[16], av[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) ak[c] = av[c] = 0.f;
    for (int i0 = 0; i0 < cnt; i0 += IT) {
      __syncthreads();
      for (int it = tid; it < IT * kHeadDim; it += 256) {
        const int i = it >> 6, c = it & 63;
        float qv = 0.f, gv = 0.f;
        if (i0 + i < cnt) {
          const int t = ph[i0 + i], n = t / s;
          qv = to_f32(Q[((size_t)bh * N + n) * kHeadDim + c]);
          gv = dout[((size_t)bh * N + n) * kHeadDim + c];
        }
        qs[i][c] = qv;
        gs[i][c] = gv;
      }
      for (int it = tid; it < IT * 64; it += 256) {
        const int i = it >> 6, j = it & 63;
        float2 v = make_float2(0.f, 0.f);
        if (i0 + i < cnt && j0 + j < k) {
          const int t = ph[i0 + i], n = t / s, r = t - n * s;
          v = G[((size_t)bh * N + n) * E + ms + r * k + j0 + j];
        }
        ws[i][j] = v;
      }
      __syncthreads();
      const int ni = min(IT, cnt - i0);
      for (int i = 0; i < ni; ++i) {
        const float qv = qs[i][lane], gv = gs[i][lane];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float2 wz = ws[i][16 * w + j];
          ak[j] = fmaf(wz.y, qv, ak[j]);
          av[j] = fmaf(wz.x, gv, av[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int slot = j0 + 16 * w + j;
      if (slot < k) {
        const int key = idx[((size_t)bh * m + e) * k + slot];
        unsafeAtomicAdd(dK + ((size_t)bh * N + key) * kHeadDim + lane, ak[j]);
        unsafeAtomicAdd(dV + ((size_t)bh * N + key) * kHeadDim + lane, av[j]);
      }
    }
  }
}

// ---------------------------------------------------------------- tile
// The query, expert and shared steps in one kernel on fp32 MFMA (16x16x4),
// for s = 1 with at most 128 entry columns (the m shared entries, then the k
// routed ones, each padded to a multiple of 16).  Workgroup (expert e, head
// bh), four waves; the expert's queries go 16 at a time (a tile) and wave w
// owns the entry column tiles w and w + 4 (16 entries each):
//   S = Q E_key^T and dW = dOut E_val^T, the wave's entry rows held in
//     registers as B operands (lane (g, j): entry 16 t + j, channels 16 g ..
//     16 g + 15, one per k-step) and the tile's rows read from LDS;
//   the softmax maximum, the sum of weights and dOut . out = sum w dw per
//     query, each a 16-lane reduction and a sum over the waves through LDS;
//   dz = tau w (dw - dOut . out);
//   dE_key += dz^T Q and dE_val += w^T dOut, with the S accumulators as the
//     A operands as they stand (k-step r pairs lane group g with query
//     4 g + r), kept in registers over the expert's tiles;
//   dq = dz E_key over the wave's entries (dz transposed through LDS, the
//     entry rows from an LDS copy), summed over the waves in LDS and stored
//     once per query.
// At the end each entry row goes out with float atomics: routed entries into
// dK, dV (row = key id), shared ones into dQ_L, dV_L.
constexpr int TILE_EP = 128;   // entry columns at most
constexpr int KE_STRIDE = 80;  // floats per LDS entry row (rows 16 banks apart)
constexpr int ZT_STRIDE = 17;  // floats per transposed dz row

// 16 floats of a row (fp32 or bf16) from channel c0
__device__ __forceinline__ void load16(const float* row, int c0, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 f = *reinterpret_cast<const float4*>(row + c0 + 4 * q);
    v[4 * q] = f.x;
    v[4 * q + 1] = f.y;
    v[4 * q + 2] = f.z;
    v[4 * q + 3] = f.w;
  }
}
__device__ __forceinline__ void load16(const bf16_t* row, int c0, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const u32x4 b = *reinterpret_cast<const u32x4*>(row + c0 + 8 * q);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * q + 2 * t] = __uint_as_float(b[t] << 16);
      v[8 * q + 2 * t + 1] = __uint_as_float(b[t] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// NTW: entry column tiles per wave (1 when the entries fit 64 columns: fewer
// registers and LDS, three workgroups per CU).  Workgroup (p, head bh) walks
// the head's experts p, p + P, ..; its tiles run back to back, each tile's
// successor's query rows (the next tile of the expert, or the next expert's
// first) requested while it is computed.  (Requesting the next expert's
// routed rows early too needed 32 more registers, which at three workgroups
// per CU spilled: 1005 us against 945 us per DeiT-S backward without.)  The
// shared entries' gradients accumulate over all of the workgroup's experts
// and go out once at the end; the routed ones go out after each expert.
template <typename T, int NTW>
__global__ __launch_bounds__(256, NTW == 1 ? 3 : 2) void tile_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ ql, const float* __restrict__ vl, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    const float* __restrict__ dout, float* __restrict__ dq, float* __restrict__ dK,
    float* __restrict__ dV, float* __restrict__ dql, float* __restrict__ dvl, int N, int m, int k,
    int ms, int msp, int ep, int P, float tau) {
  // bf16 inputs with two column tiles per wave: S and dW on bf16 MFMA
  // 16x16x32 (Q, K and V are exact in bf16; dOut and the shared entries' Q_L,
  // V_L split into bf16 hi + lo).  Otherwise all on fp32 MFMA (measured: the
  // one-tile form, bound by its loads' latency, ran 10% slower with the
  // splits, the two-tile form 30% faster).
  constexpr bool BF = std::is_same<T, bf16_t>::value && NTW == 2;
  __shared__ __attribute__((aligned(16))) float qt[16][68];
  __shared__ __attribute__((aligned(16))) uint16_t qtb[16][72];
  __shared__ __attribute__((aligned(16))) uint16_t gth[16][72];
  __shared__ __attribute__((aligned(16))) uint16_t gtl[16][72];
  __shared__ __attribute__((aligned(16))) float gt[16][68];
  __shared__ __attribute__((aligned(16))) float ke[4][16 * NTW][KE_STRIDE];
  __shared__ float zt[4][16 * NTW][ZT_STRIDE];
  __shared__ __attribute__((aligned(16))) float dqp[4][16][68];
  __shared__ __attribute__((aligned(16))) float red[3][16][4];
  __shared__ int qid[16];
  const int p = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
  const float kl2 = tau * 1.4426950408889634f;  // logits in the base-2 domain
  const int ntile = ep >> 4;
  // this wave's entry column tiles: w and w + 4 (nt of them)
  const int nt = (w < ntile ? 1 : 0) + (NTW > 1 && w + 4 < ntile ? 1 : 0);
  const int32_t* offh = offsets + (size_t)bh * (m + 1);
  const int32_t* permh = perm + (size_t)bh * N;
  // the first non-empty expert at or after e0 in this workgroup's sequence
  // (m when none): its query range [q0, q0 + cnt)
  auto next_expert = [&](int e0, int& q0, int& cnt) {
    for (int e = e0; e < m; e += P) {
      q0 = offh[e];
      cnt = offh[e + 1] - q0;
      if (cnt > 0) return e;
    }
    q0 = cnt = 0;
    return m;
  };
  // a tile's rows: thread -> (query rq, channels rc0 ..)  (bf16: qv.x, qv.y
  // carry the four raw bf16 values)
  const int rq = tid >> 4, rc0 = 4 * (tid & 15);
  auto fetch = [&](int q0, int t0, int cnt, float4& qv, float4& gv, int& id) {
    qv = gv = make_float4(0.f, 0.f, 0.f, 0.f);
    id = -1;
    if (t0 + rq < cnt) {
      id = permh[q0 + t0 + rq];
      const size_t r = ((size_t)bh * N + id) * kHeadDim + rc0;
      if constexpr (BF) {
        const u32x2 b = *reinterpret_cast<const u32x2*>(Q + r);
        qv.x = __uint_as_float(b[0]);
        qv.y = __uint_as_float(b[1]);
      } else {
        qv = make_float4(to_f32(Q[r]), to_f32(Q[r + 1]), to_f32(Q[r + 2]), to_f32(Q[r + 3]));
      }
      gv = *reinterpret_cast<const float4*>(dout + r);
    }
  };
  // The wave's entry rows as B operands.  fp32: kb/vb hold channels 16 g ..
  // 16 g + 15 (one per 16x16x4 k-step); bf16: kh/vh (hi, or the exact bf16
  // row) and kl/vlo (lo; zero for routed entries) hold channels 32 ks + 8 g
  // .. + 7 for k-steps ks = 0, 1 of 16x16x32.  Shared tiles' rows (Q_L, V_L)
  // are the same for every expert; routed tiles' rows are the expert's keys.
  float kb[BF ? 1 : NTW][16], vb[BF ? 1 : NTW][16];
  u32x4 kh[NTW][2], kl[NTW][2], vh[NTW][2], vlo[NTW][2];
  bool valid[NTW], sht[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    sht[i] = 16 * (w + 4 * i) < msp;
    const int col = 16 * (w + 4 * i) + j;
    valid[i] = i < nt && (sht[i] ? col < ms : col - msp < k);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) kh[i][ks] = kl[i][ks] = vh[i][ks] = vlo[i][ks] = u32x4{0u, 0u, 0u, 0u};
    if constexpr (!BF) {
#pragma unroll
      for (int c = 0; c < 16; ++c) kb[i][c] = vb[i][c] = 0.f;
    }
  }
  // rows of tile i for expert e (shared tiles: e is ignored) into the operand
  // registers, and their key channels into the wave's LDS copy for dq
  auto load_entries = [&](int i, int e) {
    const int col = 16 * (w + 4 * i) + j;
    const float* srow_k = nullptr;
    const float* srow_v = nullptr;
    const T* rrow_k = nullptr;
    const T* rrow_v = nullptr;
    if (sht[i]) {
      srow_k = ql + ((size_t)bh * m + col) * kHeadDim;
      srow_v = vl + ((size_t)bh * m + col) * kHeadDim;
    } else if (valid[i]) {
      const size_t r = ((size_t)bh * N + idx[((size_t)bh * m + e) * k + col - msp]) * kHeadDim;
      rrow_k = K + r;
      rrow_v = V + r;
    }
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = 32 * ks + 8 * g;
        if (valid[i] && sht[i]) {
          float a[8], b[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 fa = *reinterpret_cast<const float4*>(srow_k + c0 + 4 * h);
            const float4 fb = *reinterpret_cast<const float4*>(srow_v + c0 + 4 * h);
            a[4 * h] = fa.x; a[4 * h + 1] = fa.y; a[4 * h + 2] = fa.z; a[4 * h + 3] = fa.w;
            b[4 * h] = fb.x; b[4 * h + 1] = fb.y; b[4 * h + 2] = fb.z; b[4 * h + 3] = fb.w;
          }
          uint32_t hk[8], lk[8], hv[8], lv[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            hk[t] = bf16_rne_bits(a[t]);
            lk[t] = bf16_rne_bits(a[t] - bf16_bits_to_f32(hk[t]));
            hv[t] = bf16_rne_bits(b[t]);
            lv[t] = bf16_rne_bits(b[t] - bf16_bits_to_f32(hv[t]));
          }
          kh[i][ks] = u32x4{pack2(hk[0], hk[1]), pack2(hk[2], hk[3]), pack2(hk[4], hk[5]), pack2(hk[6], hk[7])};
          kl[i][ks] = u32x4{pack2(lk[0], lk[1]), pack2(lk[2], lk[3]), pack2(lk[4], lk[5]), pack2(lk[6], lk[7])};
          vh[i][ks] = u32x4{pack2(hv[0], hv[1]), pack2(hv[2], hv[3]), pack2(hv[4], hv[5]), pack2(hv[6], hv[7])};
          vlo[i][ks] = u32x4{pack2(lv[0], lv[1]), pack2(lv[2], lv[3]), pack2(lv[4], lv[5]), pack2(lv[6], lv[7])};
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<float4*>(&ke[w][16 * i + j][c0 + 4 * h]) =
                make_float4(a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]);
        } else {
          u32x4 kk = u32x4{0u, 0u, 0u, 0u}, vv = kk;
          if (valid[i]) {
            kk = *reinterpret_cast<const u32x4*>(rrow_k + c0);
            vv = *reinterpret_cast<const u32x4*>(rrow_v + c0);
          }
          kh[i][ks] = kk;
          vh[i][ks] = vv;
#pragma unroll
          for (int h = 0; h < 2; ++h)
            *reinterpret_cast<float4*>(&ke[w][16 * i + j][c0 + 4 * h]) =
                make_float4(__uint_as_float(kk[2 * h] << 16), __uint_as_float(kk[2 * h] & 0xFFFF0000u),
                            __uint_as_float(kk[2 * h + 1] << 16),
                            __uint_as_float(kk[2 * h + 1] & 0xFFFF0000u));
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 16; ++c) kb[i][c] = vb[i][c] = 0.f;
      if (valid[i]) {
        if (sht[i]) {
          load16(srow_k, 16 * g, kb[i]);
          load16(srow_v, 16 * g, vb[i]);
        } else {
          load16(rrow_k, 16 * g, kb[i]);
          load16(rrow_v, 16 * g, vb[i]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(&ke[w][16 * i + j][16 * g + 4 * q]) =
            make_float4(kb[i][4 * q], kb[i][4 * q + 1], kb[i][4 * q + 2], kb[i][4 * q + 3]);
    }
  };
  f32x4 adk[NTW][4], adv[NTW][4];
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) adk[i][c4] = adv[i][c4] = zero4();
  // the entries' rows go out: lane (g, j) holds [entry 16 (w + 4i) + 4g + r]
  // [channel 16 c4 + j]; SH selects the shared tiles (else the routed ones)
  auto flush = [&](bool sh_tiles, int e) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      if (i >= nt || sht[i] != sh_tiles) continue;
      const int base = 16 * (w + 4 * i);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = base + 4 * g + r;
        float* dk = nullptr;
        float* dv = nullptr;
        if (sh_tiles) {
          if (col < ms) {
            dk = dql + ((size_t)bh * m + col) * kHeadDim;
            dv = dvl + ((size_t)bh * m + col) * kHeadDim;
          }
        } else if (col - msp < k) {
          const size_t row = ((size_t)bh * N + idx[((size_t)bh * m + e) * k + col - msp]) * kHeadDim;
          dk = dK + row;
          dv = dV + row;
        }
        if (dk) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            unsafeAtomicAdd(dk + 16 * c4 + j, adk[i][c4][r]);
            unsafeAtomicAdd(dv + 16 * c4 + j, adv[i][c4][r]);
          }
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) adk[i][c4][r] = adv[i][c4][r] = 0.f;
      }
    }
  };

  int qa, ca, qb, cb;
  int ea = next_expert(p, qa, ca);
  if (ea >= m) return;
  int eb = next_expert(ea + P, qb, cb);
#pragma unroll
  for (int i = 0; i < NTW; ++i)
    if (i < nt) load_entries(i, ea);
  float4 qv, gv;
  int qidv;
  fetch(qa, 0, ca, qv, gv, qidv);

  while (ea < m) {
    for (int t0 = 0; t0 < ca; t0 += 16) {
      const int nq = min(16, ca - t0);
      __syncthreads();  // the previous tile's LDS is spent
      if constexpr (BF) {
        *reinterpret_cast<u32x2*>(&qtb[rq][rc0]) = u32x2{__float_as_uint(qv.x), __float_as_uint(qv.y)};
        const float gf[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t hh[4], ll[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          hh[t] = bf16_rne_bits(gf[t]);
          ll[t] = bf16_rne_bits(gf[t] - bf16_bits_to_f32(hh[t]));
        }
        *reinterpret_cast<u32x2*>(&gth[rq][rc0]) = u32x2{pack2(hh[0], hh[1]), pack2(hh[2], hh[3])};
        *reinterpret_cast<u32x2*>(&gtl[rq][rc0]) = u32x2{pack2(ll[0], ll[1]), pack2(ll[2], ll[3])};
      } else {
        *reinterpret_cast<float4*>(&qt[rq][rc0]) = qv;
      }
      *reinterpret_cast<float4*>(&gt[rq][rc0]) = gv;
      if ((tid & 15) == 0) qid[rq] = qidv;
      // the next tile's rows fly while this one is computed
      if (t0 + 16 < ca)
        fetch(qa, t0 + 16, ca, qv, gv, qidv);
      else if (eb < m)
        fetch(qb, 0, cb, qv, gv, qidv);
      __syncthreads();
      // S and dW: lane (g, j) holds [query 4g + r][entry 16 (w + 4i) + j]
      f32x4 sa[NTW], sw[NTW];
#pragma unroll
      for (int i = 0; i < NTW; ++i) sa[i] = sw[i] = zero4();
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&qtb[j][32 * ks + 8 * g]);
          const u32x4 ah = *reinterpret_cast<const u32x4*>(&gth[j][32 * ks + 8 * g]);
          const u32x4 al = *reinterpret_cast<const u32x4*>(&gtl[j][32 * ks + 8 * g]);
#pragma unroll
          for (int i = 0; i < NTW; ++i)
            if (i < nt) {
              sa[i] = mfma_bf16(a, kh[i][ks], sa[i]);
              sw[i] = mfma_bf16(ah, vh[i][ks], sw[i]);
              sw[i] = mfma_bf16(al, vh[i][ks], sw[i]);
              if (sht[i]) {
                sa[i] = mfma_bf16(a, kl[i][ks], sa[i]);
                sw[i] = mfma_bf16(ah, vlo[i][ks], sw[i]);
              }
            }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a4 = *reinterpret_cast<const float4*>(&qt[j][16 * g + 4 * q]);
          const float4 d4 = *reinterpret_cast<const float4*>(&gt[j][16 * g + 4 * q]);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w}, dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < NTW; ++i)
              if (i < nt) {
                sa[i] = mfma_f32(av[u], kb[i][4 * q + u], sa[i]);
                sw[i] = mfma_f32(dv[u], vb[i][4 * q + u], sw[i]);
              }
        }
      }
      // logits (base 2; -inf for padding entries) and the row maxima
      float x[NTW][4];
      float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[i][r] = valid[i] ? sa[i][r] * kl2 : -INFINITY;
          mx[r] = fmaxf(mx[r], x[i][r]);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        mx[r] = g16_maxf(mx[r]);
        if (j == r) red[0][4 * g + r][w] = mx[r];
      }
      __syncthreads();
      float ps[4], pd[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 m4 = *reinterpret_cast<const float4*>(&red[0][4 * g + r][0]);
        mx[r] = fmaxf(fmaxf(m4.x, m4.y), fmaxf(m4.z, m4.w));
        ps[r] = pd[r] = 0.f;
      }
      float pw[NTW][4];
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[i][r] = __builtin_amdgcn_exp2f(x[i][r] - mx[r]);  // 0 at -inf
          ps[r] += pw[i][r];
          pd[r] = fmaf(pw[i][r], sw[i][r], pd[r]);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ps[r] = g16_sumf(ps[r]);
        pd[r] = g16_sumf(pd[r]);
        if (j == r) {
          red[1][4 * g + r][w] = ps[r];
          red[2][4 * g + r][w] = pd[r];
        }
      }
      __syncthreads();
      // w = p / L, dz = tau w (dw - D), D = sum p dw / L
      float wt[NTW][4], dz[NTW][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 l4 = *reinterpret_cast<const float4*>(&red[1][4 * g + r][0]);
        const float4 d4 = *reinterpret_cast<const float4*>(&red[2][4 * g + r][0]);
        const float inv = 1.0f / ((l4.x + l4.y) + (l4.z + l4.w));
        const float D = ((d4.x + d4.y) + (d4.z + d4.w)) * inv;
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          wt[i][r] = pw[i][r] * inv;
          dz[i][r] = tau * wt[i][r] * (sw[i][r] - D);
        }
      }
      // dE_key += dz^T Q, dE_val += w^T dOut (k-step r: lane group g with
      // query 4g + r); dz transposed into the wave's LDS rows for dq
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          float bq;
          if constexpr (BF)
            bq = bf16_bits_to_f32(qtb[4 * g + r][16 * c4 + j]);
          else
            bq = qt[4 * g + r][16 * c4 + j];
          const float bg = gt[4 * g + r][16 * c4 + j];
#pragma unroll
          for (int i = 0; i < NTW; ++i)
            if (i < nt) {
              adk[i][c4] = mfma_f32(dz[i][r], bq, adk[i][c4]);
              adv[i][c4] = mfma_f32(wt[i][r], bg, adv[i][c4]);
            }
        }
#pragma unroll
        for (int i = 0; i < NTW; ++i)
          if (i < nt) zt[w][16 * i + j][4 * g + r] = dz[i][r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // dq share over this wave's entries: lane (g, j) -> [query 4g + r][channel 16 c4 + j]
      f32x4 aq[4];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) aq[c4] = zero4();
#pragma unroll
      for (int i = 0; i < NTW; ++i)
        if (i < nt) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const float a = zt[w][16 * i + 4 * ks + g][j];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
              aq[c4] = mfma_f32(a, ke[w][16 * i + 4 * ks + g][16 * c4 + j], aq[c4]);
          }
        }
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
        for (int r = 0; r < 4; ++r) dqp[w][4 * g + r][16 * c4 + j] = aq[c4][r];
      __syncthreads();
      {
        const int qi = tid >> 4, c0 = 4 * (tid & 15);
        if (qi < nq) {
          float4 sum = *reinterpret_cast<const float4*>(&dqp[0][qi][c0]);
#pragma unroll
          for (int ww = 1; ww < 4; ++ww) {
            const float4 v = *reinterpret_cast<const float4*>(&dqp[ww][qi][c0]);
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
          }
          *reinterpret_cast<float4*>(dq + ((size_t)bh * N + qid[qi]) * kHeadDim + c0) = sum;
        }
      }
    }
    // the expert's routed rows go out; then on to the next expert
    flush(false, ea);
    ea = eb;
    qa = qb;
    ca = cb;
    if (ea >= m) break;
    eb = next_expert(ea + P, qb, cb);
    // (the wave's own LDS copy of its key rows: its reads of the previous
    // expert's are done)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int i = 0; i < NTW; ++i)
      if (i < nt && !sht[i]) load_entries(i, ea);
  }
  // the shared entries' rows, summed over the workgroup's experts
  flush(true, 0);
}

// ---------------------------------------------------------------- shared
// dQ_L[i] = sum_n dz_ni q_n, dV_L[i] = sum_n w_ni dOut_n for 16 landmarks per
// workgroup (thread: landmark tid/16, channels 4 (tid%16) ..); then each
// row's dV_L . V_L for the landmark step.
template <typename T>
__global__ __launch_bounds__(256) void shared_kernel(
    const T* __restrict__ Q, const float* __restrict__ dout, const float2* __restrict__ G,
    const float* __restrict__ vl, float* __restrict__ dql, float* __restrict__ dvl,
    float4* __restrict__ stats, int N, int m, int E) {
  constexpr int NB = 32;
  __shared__ float qs[NB][kHeadDim];
  __shared__ float gs[NB][kHeadDim];
  __shared__ float2 ws[NB][16];
  __shared__ float red[16][16];
  const int i0 = blockIdx.x * 16, bh = blockIdx.y, tid = threadIdx.x;
  const int li = tid >> 4, c0 = 4 * (tid & 15);
  float aq[4] = {0.f, 0.f, 0.f, 0.f}, av[4] = {0.f, 0.f, 0.f, 0.f};
  for (int n0 = 0; n0 < N; n0 += NB) {
    __syncthreads();
    for (int it = tid; it < NB * kHeadDim; it += 256) {
      const int i = it >> 6, c = it & 63;
      const bool ok = n0 + i < N;
      const size_t r = (size_t)bh * N + n0 + i;
      qs[i][c] = ok ? to_f32(Q[r * kHeadDim + c]) : 0.f;
      gs[i][c] = ok ? dout[r * kHeadDim + c] : 0.f;
    }
    for (int it = tid; it < NB * 16; it += 256) {
      const int i = it >> 4, l = it & 15;
      ws[i][l] = (n0 + i < N && i0 + l < m) ? G[((size_t)bh * N + n0 + i) * E + i0 + l]
                                            : make_float2(0.f, 0.f);
    }
    __syncthreads();
    const int nn = min(NB, N - n0);
    for (int i = 0; i < nn; ++i) {
      const float2 wz = ws[i][li];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        aq[c] = fmaf(wz.y, qs[i][c0 + c], aq[c]);
        av[c] = fmaf(wz.x, gs[i][c0 + c], av[c]);
      }
    }
  }
  const int i = i0 + li;
  float part = 0.f;
  if (i < m) {
    const size_t r = ((size_t)bh * m + i) * kHeadDim + c0;
    *reinterpret_cast<float4*>(dql + r) = make_float4(aq[0], aq[1], aq[2], aq[3]);
    *reinterpret_cast<float4*>(dvl + r) = make_float4(av[0], av[1], av[2], av[3]);
#pragma unroll
    for (int c = 0; c < 4; ++c) part = fmaf(av[c], vl[r + c], part);
  }
  red[li][tid & 15] = part;
  __syncthreads();
  if (tid < 16 && i0 + tid < m) {
    float c = 0.f;
    for (int q = 0; q < 16; ++q) c += red[tid][q];
    stats[(size_t)bh * m + i0 + tid].z = c;
  }
}

// ---------------------------------------------------------------- stats
// Each landmark row's maximum and sum of exp(S - max) over all keys, with
// S = tau Q_L . K: 16 rows per workgroup (thread: row tid/16, keys tid%16 +
// 16 q of each staged 64-key block); with dvl given, also the row's
// dV_L . V_L (otherwise left as the shared step wrote it).
template <typename T>
__global__ __launch_bounds__(256) void stats_kernel(const float* __restrict__ ql,
                                                    const T* __restrict__ K,
                                                    const float* __restrict__ dvl,
                                                    const float* __restrict__ vl,
                                                    float4* __restrict__ stats, int N, int m,
                                                    float tau, int with_ml) {
  __shared__ float kb[64][kHeadDim + 1];
  __shared__ float qr[16][kHeadDim];
  const int i0 = blockIdx.x * 16, bh = blockIdx.y, tid = threadIdx.x;
  const int li = tid >> 4, lk = tid & 15;
  for (int it = tid; it < 16 * kHeadDim; it += 256) {
    const int i = it >> 6, c = it & 63;
    qr[i][c] = i0 + i < m ? ql[((size_t)bh * m + i0 + i) * kHeadDim + c] : 0.f;
  }
  float M = -INFINITY, L = 0.f;
  for (int b0 = 0; b0 < (with_ml ? N : 0); b0 += 64) {
    __syncthreads();
    for (int it = tid; it < 64 * kHeadDim; it += 256) {
      const int j = it >> 6, c = it & 63;
      kb[j][c] = b0 + j < N ? to_f32(K[((size_t)bh * N + b0 + j) * kHeadDim + c]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = lk + 16 * q;
      if (b0 + j >= N) continue;
      float a = 0.f;
#pragma unroll 16
      for (int c = 0; c < kHeadDim; ++c) a = fmaf(qr[li][c], kb[j][c], a);
      a *= tau;
      const float mn = fmaxf(M, a);
      L = L * fast_exp(M - mn) + fast_exp(a - mn);
      M = mn;
    }
  }
  // combine the 16 threads of a row (lanes 16 li .. 16 li + 15 of one wave)
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float oM = __shfl_xor(M, o, 64), oL = __shfl_xor(L, o, 64);
    const float mn = fmaxf(M, oM);
    L = (M > -INFINITY ? L * fast_exp(M - mn) : 0.f) + (oM > -INFINITY ? oL * fast_exp(oM - mn) : 0.f);
    M = mn;
  }
  float z = 0.f;
  if (dvl && i0 + li < m) {
    const size_t r = ((size_t)bh * m + i0 + li) * kHeadDim + 4 * lk;
#pragma unroll
    for (int c = 0; c < 4; ++c) z = fmaf(dvl[r + c], vl[r + c], z);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) z += __shfl_xor(z, o, 64);
  if (lk == 0 && i0 + li < m) {
    float4* st = stats + (size_t)bh * m + i0 + li;
    if (with_ml) {
      st->x = M;
      st->y = L;
    }
    if (dvl) st->z = z;
  }
}

// ---------------------------------------------------------------- landmark
// Workgroup (64-key block, head): landmark rows 32 at a time; A_ij and dS_ij
// for the rows and the block's keys into LDS; then the block's dV, dK rows
// (thread: key tid/4, channels 16 (tid%4) ..) and the rows' dQ_L share
// (thread: row tid/8, channels 8 (tid%8) .., atomics).
template <typename T>
__global__ __launch_bounds__(256) void landmark_kernel(
    const float* __restrict__ ql, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ dvl, const float4* __restrict__ stats, float* __restrict__ dql,
    float* __restrict__ dK, float* __restrict__ dV, int N, int m, float tau) {
  constexpr int MR = 32;
  __shared__ float kb[64][kHeadDim + 1];
  __shared__ float vb[64][kHeadDim + 1];
  __shared__ float qr[MR][kHeadDim + 1];
  __shared__ float dr[MR][kHeadDim + 1];
  __shared__ float A[MR][65];
  __shared__ float dS[MR][65];
  const int b0 = blockIdx.x * 64, bh = blockIdx.y, tid = threadIdx.x;
  for (int it = tid; it < 64 * kHeadDim; it += 256) {
    const int j = it >> 6, c = it & 63;
    const bool ok = b0 + j < N;
    const size_t r = ((size_t)bh * N + b0 + j) * kHeadDim + c;
    kb[j][c] = ok ? to_f32(K[r]) : 0.f;
    vb[j][c] = ok ? to_f32(V[r]) : 0.f;
  }
  const int kj = tid >> 2, kc = 16 * (tid & 3);
  float adv[16], adk[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) adv[c] = adk[c] = 0.f;
  for (int i0 = 0; i0 < m; i0 += MR) {
    __syncthreads();
    for (int it = tid; it < MR * kHeadDim; it += 256) {
      const int i = it >> 6, c = it & 63;
      const bool ok = i0 + i < m;
      qr[i][c] = ok ? ql[((size_t)bh * m + i0 + i) * kHeadDim + c] : 0.f;
      dr[i][c] = ok ? dvl[((size_t)bh * m + i0 + i) * kHeadDim + c] : 0.f;
    }
    __syncthreads();
    for (int it = tid; it < MR * 64; it += 256) {
      const int i = it >> 6, j = it & 63;
      float a = 0.f, ds = 0.f;
      if (i0 + i < m && b0 + j < N) {
        const float4 st = stats[(size_t)bh * m + i0 + i];
        float sc = 0.f, da = 0.f;
#pragma unroll 16
        for (int c = 0; c < kHeadDim; ++c) {
          sc = fmaf(qr[i][c], kb[j][c], sc);
          da = fmaf(dr[i][c], vb[j][c], da);
        }
        a = fast_exp(tau * sc - st.x) / st.y;
        ds = a * (da - st.z);
      }
      A[i][j] = a;
      dS[i][j] = ds;
    }
    __syncthreads();
    const int nr = min(MR, m - i0);
    for (int i = 0; i < nr; ++i) {
      const float a = A[i][kj], ds = dS[i][kj];
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        adv[c] = fmaf(a, dr[i][kc + c], adv[c]);
        adk[c] = fmaf(ds, qr[i][kc + c], adk[c]);
      }
    }
    {
      // wave w: rows w, w + 4, ..; lane: channel (one atomic instruction per
      // row over 64 contiguous floats)
      const int lane = tid & 63, wv = tid >> 6;
      float aq[MR / 4];
#pragma unroll
      for (int q = 0; q < MR / 4; ++q) aq[q] = 0.f;
      for (int j = 0; j < 64; ++j) {
        const float kv = kb[j][lane];
#pragma unroll
        for (int q = 0; q < MR / 4; ++q) aq[q] = fmaf(dS[wv + 4 * q][j], kv, aq[q]);
      }
#pragma unroll
      for (int q = 0; q < MR / 4; ++q) {
        const int ri = wv + 4 * q;
        if (ri < nr) unsafeAtomicAdd(dql + ((size_t)bh * m + i0 + ri) * kHeadDim + lane, tau * aq[q]);
      }
    }
  }
  if (b0 + kj < N) {
    // the block's rows belong to this workgroup alone: add in place
    float* dv = dV + ((size_t)bh * N + b0 + kj) * kHeadDim + kc;
    float* dk = dK + ((size_t)bh * N + b0 + kj) * kHeadDim + kc;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      dv[c] += adv[c];
      dk[c] += tau * adk[c];
    }
  }
}

// ---------------------------------------------------------------- landmark (MFMA)
// m <= 64, on fp32 MFMA 16x16x4.  Workgroup (run of LMK_BLOCKS 64-key blocks,
// head): the landmark rows' Q_L, dV_L, statistics and dV_L . V_L are staged
// once; then per 64-key block wave w owns keys 16 w .. 16 w + 15 (their K and
// V rows in registers as B operands: lane (g, j) holds key j, channels 16 g ..
// 16 g + 15; the next block's rows are requested while this one is computed).
// Per 16-row tile of landmarks:
//   S = Q_L K_w^T and dA = dV_L V_w^T (Q_L and dV_L rows from LDS as A);
//   A = exp(tau S - M) / L and dS = A (dA - dV_L . V_L), with the rows'
//     statistics (zero past m and at keys past N);
//   dV_w += A^T dV_L and dK_w += dS^T Q_L (the accumulators as A operands as
//     they stand: k-step r pairs lane group g with row 4 g + r);
//   dQ_L += dS K_w (dS transposed through LDS), held in registers over the
//     blocks.
// The blocks' dK, dV rows belong to this workgroup and are added in place;
// dQ_L, the four waves' shares summed in LDS, goes out with one float atomic
// per element per workgroup (tau applied to dK and dQ_L on the way out).
constexpr int LMK_BLOCKS = 4;

template <typename T>
__global__ __launch_bounds__(256, 2) void landmark_mfma_kernel(
    const float* __restrict__ ql, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ dvl, const float* __restrict__ vl, const float4* __restrict__ stats,
    float* __restrict__ dql, float* __restrict__ dK, float* __restrict__ dV, int N, int m,
    float tau) {
  __shared__ __attribute__((aligned(16))) float qs[64][68];
  __shared__ __attribute__((aligned(16))) float gs[64][68];
  __shared__ __attribute__((aligned(16))) float acc_q[64][68];
  __shared__ __attribute__((aligned(16))) float kt[4][16][KE_STRIDE];
  __shared__ float zt[4][16][ZT_STRIDE];
  __shared__ float rst[3][64];  // M, 1 / L, dV_L . V_L per row
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
  const int mt = (m + 15) >> 4;
  const int blk0 = blockIdx.x * LMK_BLOCKS, blk1 = min((N + 63) >> 6, blk0 + LMK_BLOCKS);
  // this wave's keys of block blk: K and V rows (zero past N)
  auto load_rows = [&](int blk, float (&kk)[16], float (&vv)[16]) {
    const int key = 64 * blk + 16 * w + j;
#pragma unroll
    for (int c = 0; c < 16; ++c) kk[c] = vv[c] = 0.f;
    if (key < N) {
      load16(K + ((size_t)bh * N + key) * kHeadDim, 16 * g, kk);
      load16(V + ((size_t)bh * N + key) * kHeadDim, 16 * g, vv);
    }
  };
  float kr[16], vr[16], kn[16], vn[16];
  load_rows(blk0, kr, vr);
  // this wave's dQ_L share: lane (g, j) -> [row 16 rt + 4g + r][channel 16 c4 + j]
  f32x4 aq[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) aq[rt][c4] = zero4();
  // rows (zero past m), the dQ_L sums, the rows' statistics; every load of a
  // thread goes out before any is used.  Thread (row tid / 4, channels
  // 16 (tid % 4) ..): its Q_L, dV_L and V_L chunks, and dV_L . V_L
  {
    const int r = tid >> 2, c0 = 16 * (tid & 3);
    float4 q[4], d[4], v[4];
    float4 st = make_float4(0.f, 1.f, 0.f, 0.f);
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = d[u] = v[u] = z4;
    if (r < m) {
      const size_t o = ((size_t)bh * m + r) * kHeadDim + c0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        q[u] = *reinterpret_cast<const float4*>(ql + o + 4 * u);
        d[u] = *reinterpret_cast<const float4*>(dvl + o + 4 * u);
        v[u] = *reinterpret_cast<const float4*>(vl + o + 4 * u);
      }
      st = stats[(size_t)bh * m + r];
    }
    float z = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<float4*>(&qs[r][c0 + 4 * u]) = q[u];
      *reinterpret_cast<float4*>(&gs[r][c0 + 4 * u]) = d[u];
      *reinterpret_cast<float4*>(&acc_q[r][c0 + 4 * u]) = z4;
      z = fmaf(d[u].x, v[u].x, fmaf(d[u].y, v[u].y, fmaf(d[u].z, v[u].z, fmaf(d[u].w, v[u].w, z))));
    }
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    if ((tid & 3) == 0) {
      rst[0][r] = st.x;
      rst[1][r] = r < m ? 1.0f / st.y : 0.f;
      rst[2][r] = z;
    }
  }
  __syncthreads();
  for (int blk = blk0; blk < blk1; ++blk) {
    if (blk + 1 < blk1) load_rows(blk + 1, kn, vn);
    const bool kok = 64 * blk + 16 * w + j < N;
    // the wave's key rows for dQ_L's B operand (its own LDS slot: the previous
    // block's reads are done)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(&kt[w][j][16 * g + 4 * q]) =
          make_float4(kr[4 * q], kr[4 * q + 1], kr[4 * q + 2], kr[4 * q + 3]);
    f32x4 adk[4], adv[4];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) adk[c4] = adv[c4] = zero4();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt >= mt) break;
      // S and dA: lane (g, j) holds [row 16 rt + 4g + r][key j of the wave]
      f32x4 sa = zero4(), sd = zero4();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a4 = *reinterpret_cast<const float4*>(&qs[16 * rt + j][16 * g + 4 * q]);
        const float4 d4 = *reinterpret_cast<const float4*>(&gs[16 * rt + j][16 * g + 4 * q]);
        sa = mfma_f32(a4.x, kr[4 * q], sa);
        sd = mfma_f32(d4.x, vr[4 * q], sd);
        sa = mfma_f32(a4.y, kr[4 * q + 1], sa);
        sd = mfma_f32(d4.y, vr[4 * q + 1], sd);
        sa = mfma_f32(a4.z, kr[4 * q + 2], sa);
        sd = mfma_f32(d4.z, vr[4 * q + 2], sd);
        sa = mfma_f32(a4.w, kr[4 * q + 3], sa);
        sd = mfma_f32(d4.w, vr[4 * q + 3], sd);
      }
      float aw[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * rt + 4 * g + r;
        const float a = kok ? fast_exp(tau * sa[r] - rst[0][row]) * rst[1][row] : 0.f;
        aw[r] = a;
        ds[r] = a * (sd[r] - rst[2][row]);
        zt[w][j][4 * g + r] = ds[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          adv[c4] = mfma_f32(aw[r], gs[16 * rt + 4 * g + r][16 * c4 + j], adv[c4]);
          adk[c4] = mfma_f32(ds[r], qs[16 * rt + 4 * g + r][16 * c4 + j], adk[c4]);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float a = zt[w][4 * ks + g][j];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
          aq[rt][c4] = mfma_f32(a, kt[w][4 * ks + g][16 * c4 + j], aq[rt][c4]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // the wave's dK, dV rows: lane (g, j) holds [key 16 w + 4g + r][channel 16 c4 + j]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 64 * blk + 16 * w + 4 * g + r;
      if (kk < N) {
        float* dk = dK + ((size_t)bh * N + kk) * kHeadDim;
        float* dv = dV + ((size_t)bh * N + kk) * kHeadDim;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          dk[16 * c4 + j] += tau * adk[c4][r];
          dv[16 * c4 + j] += adv[c4][r];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      kr[c] = kn[c];
      vr[c] = vn[c];
    }
  }
  // the waves' dQ_L shares summed in LDS, then one atomic per element
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (rt >= mt) break;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc_q[16 * rt + 4 * g + r][16 * c4 + j] += aq[rt][c4][r];
      }
    }
    __syncthreads();
  }
  for (int it = tid; it < m * kHeadDim; it += 256) {
    const int r = it >> 6, c = it & 63;
    unsafeAtomicAdd(dql + ((size_t)bh * m + r) * kHeadDim + c, tau * acc_q[r][c]);
  }
}

// ---------------------------------------------------------------- pool
// dQ[t] += sum over the windows i holding token t of dQ_L[i] / |window i|;
// along an axis of g cells pooled to mg windows, cell y lies in windows
// floor(y mg / g) .. ceil((y + 1) mg / g) - 1.  Thread: (token, 16 channels):
// float4s sub, sub + 4, sub + 8, sub + 12 of the row (sub = thread % 4), so
// that a token's four threads read 64 contiguous bytes per instruction.
__global__ __launch_bounds__(256) void pool_kernel(const float* __restrict__ dql,
                                                   float* __restrict__ dq, int gh, int gw,
                                                   int mh, int mw) {
  const int N = gh * gw, m = mh * mw;
  const long long it = (long long)blockIdx.x * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (it >= (long long)N * 4) return;
  const int n = (int)(it >> 2), c0 = 4 * (int)(it & 3);
  // (32-bit arithmetic when every product below stays under 2^31, which holds
  // for all but extreme grids; 64-bit otherwise, a uniform branch)
  const int y = n / gw, x = n - y * gw;
  int r0, r1, cl, ch;
  if ((long long)gh * (mh + 1) < (1LL << 31) && (long long)gw * (mw + 1) < (1LL << 31)) {
    r0 = (y * mh) / gh;
    r1 = ((y + 1) * mh + gh - 1) / gh - 1;
    cl = (x * mw) / gw;
    ch = ((x + 1) * mw + gw - 1) / gw - 1;
  } else {
    r0 = (int)(((long long)y * mh) / gh);
    r1 = (int)(((long long)(y + 1) * mh + gh - 1) / gh) - 1;
    cl = (int)(((long long)x * mw) / gw);
    ch = (int)(((long long)(x + 1) * mw + gw - 1) / gw) - 1;
  }
  float4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r = r0; r <= r1; ++r) {
    int y0, y1;
    pool_window(r, gh, mh, &y0, &y1);
    for (int cc = cl; cc <= ch; ++cc) {
      int x0, x1;
      pool_window(cc, gw, mw, &x0, &x1);
      const float inv = 1.0f / (float)((y1 - y0) * (x1 - x0));
      const float4* src =
          reinterpret_cast<const float4*>(dql + ((size_t)bh * m + r * mw + cc) * kHeadDim + c0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = src[4 * q];
        acc[q].x = fmaf(v.x, inv, acc[q].x);
        acc[q].y = fmaf(v.y, inv, acc[q].y);
        acc[q].z = fmaf(v.z, inv, acc[q].z);
        acc[q].w = fmaf(v.w, inv, acc[q].w);
      }
    }
  }
  float4* dst = reinterpret_cast<float4*>(dq + ((size_t)bh * N + n) * kHeadDim + c0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float4 d = dst[4 * q];
    d.x += acc[q].x;
    d.y += acc[q].y;
    d.z += acc[q].z;
    d.w += acc[q].w;
    dst[4 * q] = d;
  }
}

// Clears two buffers of n4 float4s each (16-byte stores, grid-stride).
__global__ __launch_bounds__(256) void zero_kernel(float4* __restrict__ a, float4* __restrict__ b,
                                                   long long n4) {
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (long long)gridDim.x * 256) {
    a[i] = z;
    b[i] = z;
  }
}

static unsigned zero_grid(long long n4) {
  const long long g = (n4 + 255) / 256;
  return (unsigned)(g < 4096 ? g : 4096);
}

}  // namespace bwd

// The tile kernel's case: s = 1 and at most 128 entry columns (m and k each
// padded to 16).
static bool bwd_tiled(const Shape& s) {
  const int ms = s.shared ? s.m : 0;
  return s.s == 1 && ((ms + 15) & ~15) + ((s.k + 15) & ~15) <= bwd::TILE_EP;
}

// Scratch: the landmark rows' statistics, dQ_L, dV_L, and (outside the tile
// kernel's case) the per-entry (w, dz) buffer.
size_t backward_scratch_bytes(const Shape& s) {
  const size_t E = (size_t)(s.shared ? s.m : 0) + (size_t)s.s * s.k;
  return align_up((size_t)s.BH * s.m * 16, 256) + 2 * align_up((size_t)s.BH * s.m * 64 * 4, 256) +
         (bwd_tiled(s) ? 0 : align_up((size_t)s.BH * s.N * E * 8, 256));
}

float4* backward_stats(void* scratch, const Shape& s) {
  (void)s;
  return (float4*)scratch;
}

template <typename T>
static hipError_t run_backward(const T* Q, const T* K, const T* V, const float* dout,
                               const float* ql, const float* vl, const int32_t* idx,
                               const int32_t* route, const int32_t* offsets,
                               const int32_t* perm, float* dq, float* dk, float* dv,
                               void* scratch, const Shape& s, hipStream_t st, bool stats_ready) {
  const int ms = s.shared ? s.m : 0;
  const int E = ms + s.s * s.k;
  const float tau = 1.0f / sqrtf((float)s.d);
  char* p = (char*)scratch;
  float4* stats = backward_stats(scratch, s);
  p += align_up((size_t)s.BH * s.m * 16, 256);
  float* dql = (float*)p;
  p += align_up((size_t)s.BH * s.m * 64 * 4, 256);
  float* dvl = (float*)p;
  p += align_up((size_t)s.BH * s.m * 64 * 4, 256);
  float2* G = (float2*)p;  // (outside the tile kernel's case)
  const long long nel = (long long)s.BH * s.N * 64;
  bwd::zero_kernel<<<bwd::zero_grid(nel / 4), 256, 0, st>>>((float4*)dk, (float4*)dv, nel / 4);
  const dim3 rows((s.m + 15) / 16, s.BH);
  if (bwd_tiled(s)) {
    // one kernel for the query, expert and shared steps; dQ_L and dV_L then
    // collect float atomics
    const int msp = (ms + 15) & ~15, ep = msp + ((s.k + 15) & ~15);
    if (s.shared) {
      const long long nl = (long long)s.BH * s.m * 64;
      bwd::zero_kernel<<<bwd::zero_grid(nl / 4), 256, 0, st>>>((float4*)dql, (float4*)dvl, nl / 4);
    }
    // workgroups per head: one-tile form, enough for about six per CU in all
    // (the shared entries' sums then go out once per workgroup); two-tile
    // form, one per expert (measured at 3136 tokens: 715 us against 754 us
    // with eight per head)
    const int P = ep <= 64 ? std::max(1, std::min(s.m, (1536 + s.BH - 1) / s.BH)) : s.m;
    auto tile = ep <= 64 ? bwd::tile_kernel<T, 1> : bwd::tile_kernel<T, 2>;
    tile<<<dim3(P, s.BH), 256, 0, st>>>(Q, K, V, ql, vl, idx, offsets, perm, dout, dq, dk, dv,
                                        dql, dvl, s.N, s.m, s.k, ms, msp, ep, P, tau);
  } else {
    bwd::query_kernel<T><<<dim3((s.N + 3) / 4, s.BH), 256, 0, st>>>(
        Q, K, V, ql, vl, idx, route, perm, dout, dq, G, s.N, s.m, s.k, s.s, s.shared ? 1 : 0, tau);
    bwd::expert_kernel<T><<<dim3(s.m, s.BH), 256, 0, st>>>(Q, dout, idx, offsets, perm, G, dk, dv,
                                                           s.N, s.m, s.k, s.s, ms);
    if (s.shared)
      bwd::shared_kernel<T><<<rows, 256, 0, st>>>(Q, dout, G, vl, dql, dvl, stats, s.N, s.m, E);
  }
  if (s.shared) {
    if (s.m <= 64) {
      // statistics from the forward pass, or recomputed here; dV_L . V_L
      // inside the landmark kernel
      if (!stats_ready)
        bwd::stats_kernel<T><<<rows, 256, 0, st>>>(ql, K, nullptr, vl, stats, s.N, s.m, tau, 1);
      const int runs = ((s.N + 63) / 64 + bwd::LMK_BLOCKS - 1) / bwd::LMK_BLOCKS;
      bwd::landmark_mfma_kernel<T><<<dim3(runs, s.BH), 256, 0, st>>>(
          ql, K, V, dvl, vl, stats, dql, dk, dv, s.N, s.m, tau);
    } else {
      bwd::stats_kernel<T><<<rows, 256, 0, st>>>(ql, K, bwd_tiled(s) ? dvl : nullptr, vl, stats,
                                                 s.N, s.m, tau, stats_ready ? 0 : 1);
      bwd::landmark_kernel<T><<<dim3((s.N + 63) / 64, s.BH), 256, 0, st>>>(
          ql, K, V, dvl, stats, dql, dk, dv, s.N, s.m, tau);
    }
    bwd::pool_kernel<<<dim3((unsigned)(((long long)s.N * 4 + 255) / 256), s.BH), 256, 0, st>>>(
        dql, dq, s.grid_h, s.grid_w, s.m_h, s.m_w);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const void* Q, const void* K, const void* V, const float* dout,
                           const float* ql, const float* vl, const int32_t* idx,
                           const int32_t* route, const int32_t* offsets, const int32_t* perm,
                           float* dq, float* dk, float* dv, void* scratch, const Shape& s,
                           hipStream_t st, bool stats_ready) {
  if (s.bf16)
    return run_backward<bf16_t>((const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, dout, ql, vl,
                                idx, route, offsets, perm, dq, dk, dv, scratch, s, st, stats_ready);
  return run_backward<float>((const float*)Q, (const float*)K, (const float*)V, dout, ql, vl, idx,
                             route, offsets, perm, dq, dk, dv, scratch, s, st, stats_ready);
}

}  // namespace mita
