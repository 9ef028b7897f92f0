// Steps a2-a4 for bf16 inputs on long grids -- the landmark pass (page
// "NeurIPS'26：注意力也是FFN？...", landmark-query section: every landmark
// query scores all keys; its k best keys, ties to the lowest key id, form a
// routed expert; the same scores, softmax-normalised over all N keys, weight V
// into the landmark values V_L).
//
// Two streaming kernels over one head's keys, each workgroup owning 16*NW
// landmark rows (16 per wave), keys in 64-key blocks staged through LDS with
// the next block prefetched into registers:
//   values: S^T = K Q_L^T on bf16 MFMA (Q_L split hi + lo: fp32-accurate
//     scores), an online softmax folded into V_L^T = V^T P^T on f16 MFMA (the
//     normaliser from an all-ones MFMA over the same f16 weights), and each
//     row's min and max score;
//   select: recomputes S from K (now in L2).  Pass 1 counts the row's scores
//     in 256 equal bins over [min, max] and finds the bin holding the k-th
//     best.  Pass 2 collects the keys in that bin or above (typically k plus
//     a few) into the row's LDS buffer; one exact selection (ties to the lower
//     key id) keeps k, emitted in ascending key order via a bitmap.  Should the
//     boundary bin overflow the buffer, pass 2 cuts the buffer back to its
//     exact k best whenever it fills and only admits later keys above the
//     k-th kept score, so the result stays exact.
// Workgroups of one head are launched on the same XCD so K and V come from
// HBM once and are re-read from that XCD's L2.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

namespace mita {
namespace lmk {

constexpr int KB = 64;                    // keys per block
constexpr int KST_BYTES = KB * 128;       // K block: 64 bf16 rows, XOR-swizzled chunks
constexpr int VT_STRIDE = KB * 2 + 16;    // bytes per V^T row: 64 f16 keys + pad
constexpr int VT_BYTES = 64 * VT_STRIDE;
constexpr int HIST_BYTES = 512;           // one row's 256 packed 16-bit bins
constexpr int HIST_STRIDE = 528;          // rows 4 banks apart: the 16 rows' atomics spread

__device__ __forceinline__ int rc(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

struct Args {
  const float* ql;
  const uint16_t* K;
  const uint16_t* V;
  int32_t* idx;
  float* vl;
  float* minmax;  // [BH][m][2] row min and max score
  int BH, N, m, k, cap, rblocks;  // rblocks = workgroups per head
};

// K block (and, for the values kernel, the V block) for one 64-key block.
template <int NW, bool WITH_V>
struct Pf {
  static constexpr int KC = 8 / NW;               // 16-byte K chunks per thread
  static constexpr int VC = WITH_V ? 4 / NW : 0;  // V key-pair chunks per thread
  u32x4 k[KC], v0[VC > 0 ? VC : 1], v1[VC > 0 ? VC : 1];
};

template <int NW, bool WITH_V>
__device__ __forceinline__ void load_block(Pf<NW, WITH_V>& pf, const uint16_t* Kh,
                                           const uint16_t* Vh, int blk, int N, int tid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < Pf<NW, WITH_V>::KC; ++i) {
    const int id = tid + 64 * NW * i, row = id >> 3, c = id & 7, key = blk * KB + row;
    pf.k[i] = key < N ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * 64 + 8 * c) : z;
  }
#pragma unroll
  for (int i = 0; i < Pf<NW, WITH_V>::VC; ++i) {
    const int id = tid + 64 * NW * i, p = id & 31, c = id >> 5;  // 32 key pairs x 8 chunks
    const int j0 = blk * KB + 2 * p, j1 = j0 + 1;
    pf.v0[i] = j0 < N ? *reinterpret_cast<const u32x4*>(Vh + (size_t)j0 * 64 + 8 * c) : z;
    pf.v1[i] = j1 < N ? *reinterpret_cast<const u32x4*>(Vh + (size_t)j1 * 64 + 8 * c) : z;
  }
}

template <int NW, bool WITH_V>
__device__ __forceinline__ void store_block(const Pf<NW, WITH_V>& pf, char* kst, char* vt,
                                            int tid) {
#pragma unroll
  for (int i = 0; i < Pf<NW, WITH_V>::KC; ++i) {
    const int id = tid + 64 * NW * i, row = id >> 3, c = id & 7;
    *reinterpret_cast<u32x4*>(kst + rc(row, c)) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < Pf<NW, WITH_V>::VC; ++i) {
    const int id = tid + 64 * NW * i, p = id & 31, c = id >> 5;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t a = (pf.v0[i][t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
      const uint32_t b = (pf.v1[i][t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(vt + (8 * c + t) * VT_STRIDE + 4 * p) =
          pk_f16(bf16_bits_to_f32(a), bf16_bits_to_f32(b));
    }
  }
}

// Q_L row `row` as the B operand (lane: landmark c16, channels 32ks + 8g ..),
// split into bf16 hi and lo; zero for rows past m.
__device__ __forceinline__ void load_ql_b(const float* ql, int bh, int m, int row, int g,
                                          u32x4 (&bqh)[2], u32x4 (&bql)[2]) {
  const bool ok = row < m;
  const float* qr = ql + ((size_t)bh * m + (ok ? row : 0)) * 64;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const float4 f0 = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * g);
    const float4 f1 = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * g + 4);
    const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = ok ? f[i] : 0.f;
      h[i] = bf16_rne_bits(v);
      l[i] = bf16_rne_bits(v - bf16_bits_to_f32(h[i]));
    }
    bqh[ks] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    bql[ks] = u32x4{l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16)};
  }
}

// Scores of the staged block: lane holds key 64blk + 16kt + 4g + r of its row
// (tau-scaled; -inf past N).
__device__ __forceinline__ void block_scores(const char* kst, const u32x4 (&bqh)[2],
                                             const u32x4 (&bql)[2], int blk, int N, int g,
                                             int c16, float (&s)[4][4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(kst + rc(16 * kt + c16, g));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(kst + rc(16 * kt + c16, 4 + g));
    f32x4 c = zero4();
    c = mfma_bf16(a0, bqh[0], c);
    c = mfma_bf16(a0, bql[0], c);
    c = mfma_bf16(a1, bqh[1], c);
    c = mfma_bf16(a1, bql[1], c);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = blk * KB + 16 * kt + 4 * g + r;
      s[kt][r] = key < N ? c[r] * 0.125f : -INFINITY;
    }
  }
}

__device__ __forceinline__ void head_of_block(const Args& a, int& bh, int& rb) {
  // round-robin dispatch puts workgroup b on XCD b % 8: keep a head's
  // workgroups on one XCD so its K and V stay in that XCD's L2
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  bh = xcd + 8 * (slot / a.rblocks);
  rb = slot % a.rblocks;
}

// ---------------------------------------------------------------- values
template <int NW>
__global__ __launch_bounds__(64 * NW) void lmk_values_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char sm[KST_BYTES + VT_BYTES];
  char* kst = sm;
  char* vt = sm + KST_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int bh, rb;
  head_of_block(a, bh, rb);
  if (bh >= a.BH) return;
  const int N = a.N;
  const uint16_t* Kh = a.K + (size_t)bh * N * 64;
  const uint16_t* Vh = a.V + (size_t)bh * N * 64;
  const int myrow = rb * 16 * NW + 16 * w + c16;
  u32x4 bqh[2], bql[2];
  load_ql_b(a.ql, bh, a.m, myrow, g, bqh, bql);
  const float l2e = 1.4426950408889634f;
  float mrun = -INFINITY, mn = INFINITY;
  f32x4 accv[4] = {zero4(), zero4(), zero4(), zero4()};
  f32x4 lsum = zero4();
  const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  // one block computes while the next two are in flight
  auto compute = [&](int blk) {
    float s[4][4];
    block_scores(kst, bqh, bql, blk, N, g, c16, s);
    float bmax = s[0][0];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bmax = fmaxf(bmax, s[kt][r]);
        if (s[kt][r] > -INFINITY) mn = fminf(mn, s[kt][r]);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float mnew = fmaxf(mrun, bmax);
    const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * l2e);
    mrun = mnew;
    u32x4 bp[2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f((s[2 * sp][r] - mnew) * l2e);
        p[4 + r] = __builtin_amdgcn_exp2f((s[2 * sp + 1][r] - mnew) * l2e);
      }
      bp[sp] = u32x4{pk_f16(p[0], p[1]), pk_f16(p[2], p[3]), pk_f16(p[4], p[5]), pk_f16(p[6], p[7])};
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const char* vrow = vt + (16 * ct + c16) * VT_STRIDE;
      f32x4 acc = accv[ct] * alpha;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vrow + (32 * sp + 4 * g) * 2);
        const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vrow + (32 * sp + 16 + 4 * g) * 2);
        acc = mfma_f16(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, bp[sp], acc);
      }
      accv[ct] = acc;
    }
    lsum = mfma_f16(ones, bp[0], lsum * alpha);
    lsum = mfma_f16(ones, bp[1], lsum);
  };
  Pf<NW, true> pfa, pfb;
  const int nblk = (N + KB - 1) / KB;
  load_block<NW, true>(pfa, Kh, Vh, 0, N, tid);
  if (nblk > 1) load_block<NW, true>(pfb, Kh, Vh, 1, N, tid);
  for (int blk = 0; blk < nblk; blk += 2) {
    __syncthreads();
    store_block<NW, true>(pfa, kst, vt, tid);
    __syncthreads();
    if (blk + 2 < nblk) load_block<NW, true>(pfa, Kh, Vh, blk + 2, N, tid);
    compute(blk);
    if (blk + 1 < nblk) {
      __syncthreads();
      store_block<NW, true>(pfb, kst, vt, tid);
      __syncthreads();
      if (blk + 3 < nblk) load_block<NW, true>(pfb, Kh, Vh, blk + 3, N, tid);
      compute(blk + 1);
    }
  }
  mn = fminf(mn, __shfl_xor(mn, 16, 64));
  mn = fminf(mn, __shfl_xor(mn, 32, 64));
  if (myrow < a.m) {
    const float inv = 1.0f / lsum[0];
    float* dst = a.vl + ((size_t)bh * a.m + myrow) * 64;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      *reinterpret_cast<float4*>(dst + 16 * ct + 4 * g) =
          make_float4(accv[ct][0] * inv, accv[ct][1] * inv, accv[ct][2] * inv, accv[ct][3] * inv);
    if (g == 0) {
      a.minmax[((size_t)bh * a.m + myrow) * 2 + 0] = mn;
      a.minmax[((size_t)bh * a.m + myrow) * 2 + 1] = mrun;
    }
  }
}

// ---------------------------------------------------------------- select
template <int NW>
struct SelLayout {
  static constexpr int ROWS = 16 * NW;
  static constexpr int OFF_K = 0;
  static constexpr int OFF_HIST = OFF_K + KST_BYTES;              // [ROWS] x HIST_STRIDE
  static constexpr int OFF_CNT = OFF_HIST + ROWS * HIST_STRIDE;   // [ROWS] int
  static constexpr int OFF_THR = OFF_CNT + ROWS * 4;              // [ROWS] float
  static constexpr int OFF_BSTAR = OFF_THR + ROWS * 4;            // [ROWS] int
  static constexpr int OFF_BUF = OFF_BSTAR + ROWS * 4;
  static size_t bytes(int cap) { return (size_t)OFF_BUF + (size_t)ROWS * cap * 8; }
};

// Cut rows' candidate buffers back (final == false: only rows whose buffer is
// nearly full) to their exact k best, or emit each row's exact k best in
// ascending key order (final == true).  Group g handles rows 4*batch + g.
template <int NW, int NV>
__device__ void select_rows(char* sm, const Args& a, int bh, int row0, int w, int g, int t,
                            bool final) {
  using L = SelLayout<NW>;
  const int cnt_limit = a.cap - KB;
#pragma unroll 1
  for (int batch = 0; batch < 4; ++batch) {
    const int lr = 16 * w + 4 * batch + g;
    const int row = row0 + lr;
    const bool active = row < a.m;
    int* cntp = reinterpret_cast<int*>(sm + L::OFF_CNT) + lr;
    const int cnt = active ? *cntp : 0;
    const bool work = final ? active : (active && cnt > cnt_limit);
    if (__ballot(work) == 0) continue;
    char* hist = sm + L::OFF_HIST + lr * HIST_STRIDE;
    float* vals = reinterpret_cast<float*>(sm + L::OFF_BUF + (size_t)lr * a.cap * 8);
    int* keys = reinterpret_cast<int*>(vals + a.cap);
    float sv[NV], x[NV];
    int kk[NV];
    uint32_t cand = 0u;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = t + 16 * u;
      const bool ok = work && e < cnt;
      sv[u] = ok ? vals[e] : -INFINITY;
      kk[u] = ok ? keys[e] : 0;
      x[u] = sv[u];
      cand |= (ok ? 1u : 0u) << u;
    }
    const uint32_t take = group_topk<NV>(x, kk, cand, a.k, hist, t, g);
    if (!final) {
      int run = 0;
      float kmin = INFINITY;
      const uint32_t below = (1u << t) - 1u;
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const bool bit = take >> u & 1u;
        const uint32_t gm = g16_ballot(bit, g);
        const int pos = run + __popc(gm & below);
        if (bit) {
          vals[pos] = sv[u];
          keys[pos] = kk[u];
          kmin = fminf(kmin, sv[u]);
        }
        run += __popc(gm);
      }
      kmin = g16_minf(kmin);
      if (work && t == 0) {
        *cntp = run;
        reinterpret_cast<float*>(sm + L::OFF_THR)[lr] = run >= a.k ? kmin : -INFINITY;
      }
    } else {
      uint32_t* bm = reinterpret_cast<uint32_t*>(vals);
      const int nw = (a.N + 31) >> 5;
      for (int q = t; q < nw; q += 16) bm[q] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (take >> u & 1u) atomicOr(&bm[kk[u] >> 5], 1u << (kk[u] & 31));
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const int wpl = (nw + 15) >> 4;
      const int q0 = t * wpl, q1 = min(nw, q0 + wpl);
      int mine = 0;
      for (int q = q0; q < q1; ++q) mine += __popc(bm[q]);
      const int total = g16_addi(mine);
      int pos = total - g16_suffix(mine);
      int32_t* out = a.idx + ((size_t)bh * a.m + row) * a.k;
      if (active) {
        for (int q = q0; q < q1; ++q) {
          uint32_t wbits = bm[q];
          while (wbits) {
            const int b = __ffs(wbits) - 1;
            wbits &= wbits - 1u;
            if (pos < a.k) out[pos] = 32 * q + b;
            ++pos;
          }
        }
      }
    }
  }
}

template <int NW, int NV>
__global__ __launch_bounds__(64 * NW) void lmk_select_kernel(Args a) {
  using L = SelLayout<NW>;
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int bh, rb;
  head_of_block(a, bh, rb);
  if (bh >= a.BH) return;
  const int N = a.N, row0 = rb * L::ROWS;
  const uint16_t* Kh = a.K + (size_t)bh * N * 64;
  const int lr = 16 * w + c16;  // this lane's row (column c16 of the S^T tiles)
  const int myrow = row0 + lr;
  const bool rowok = myrow < a.m;
  u32x4 bqh[2], bql[2];
  load_ql_b(a.ql, bh, a.m, myrow, g, bqh, bql);
  // 256 equal bins over the row's [min, max]
  float lo = 0.f, hi = 0.f;
  if (rowok) {
    lo = a.minmax[((size_t)bh * a.m + myrow) * 2 + 0];
    hi = a.minmax[((size_t)bh * a.m + myrow) * 2 + 1];
  }
  const float scale = hi > lo ? 256.0f / (hi - lo) : 0.f;
  char* myhist = sm + L::OFF_HIST + lr * HIST_STRIDE;
  for (int i = tid; i < L::ROWS * HIST_STRIDE / 16; i += 64 * NW)
    reinterpret_cast<u32x4*>(sm + L::OFF_HIST)[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid < L::ROWS) {
    reinterpret_cast<int*>(sm + L::OFF_CNT)[tid] = 0;
    reinterpret_cast<float*>(sm + L::OFF_THR)[tid] = -INFINITY;
  }
  const int nblk = (N + KB - 1) / KB;
  Pf<NW, false> pfa, pfb;
  // Streams the head's keys with two blocks in flight, calling body(blk)
  // with block blk staged in LDS.
  auto stream = [&](auto&& body) {
    load_block<NW, false>(pfa, Kh, nullptr, 0, N, tid);
    for (int blk = 0; blk < nblk; ++blk) {
      __syncthreads();
      store_block<NW, false>(pfa, sm + L::OFF_K, nullptr, tid);
      __syncthreads();
      if (blk + 1 < nblk) load_block<NW, false>(pfa, Kh, nullptr, blk + 1, N, tid);
      body(blk);
    }
  };
  // ---- pass 1: histogram
  stream([&](int blk) {
    float s[4][4];
    block_scores(sm + L::OFF_K, bqh, bql, blk, N, g, c16, s);
    if (rowok) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (s[kt][r] > -INFINITY) {
            const int b = min(255, max(0, (int)((s[kt][r] - lo) * scale)));
            atomicAdd(reinterpret_cast<uint32_t*>(myhist + (b >> 1) * 4), 1u << (16 * (b & 1)));
          }
    }
  });
  __syncthreads();
  // ---- the bin holding each row's k-th best (group g of wave w: rows 4*batch + g)
  for (int batch = 0; batch < 4; ++batch) {
    const int r2 = 16 * w + 4 * batch + g;
    const char* hrow = sm + L::OFF_HIST + r2 * HIST_STRIDE;
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(hrow + 32 * c16);
    const u32x4 d1 = *reinterpret_cast<const u32x4*>(hrow + 32 * c16 + 16);
    int local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      local += (int)((d0[q] & 0xFFFFu) + (d0[q] >> 16) + (d1[q] & 0xFFFFu) + (d1[q] >> 16));
    const int suf = g16_suffix(local);
    const int above = suf - local;
    const int need = a.k;
    const bool mine = above < need && need <= suf;
    int bstar = 0;
    if (mine) {
      int acc = above;
      bool found = false;
#pragma unroll
      for (int q = 15; q >= 0; --q) {
        const uint32_t dw = (q < 8 ? d0 : d1)[(q & 7) >> 1];
        const int cq = (q & 1) ? (int)(dw >> 16) : (int)(dw & 0xFFFFu);
        if (!found) {
          if (acc + cq >= need) {
            found = true;
            bstar = 16 * c16 + q;
          } else {
            acc += cq;
          }
        }
      }
    }
    bstar = g16_addi(mine ? bstar : 0);
    if (c16 == 0) reinterpret_cast<int*>(sm + L::OFF_BSTAR)[r2] = bstar;
  }
  __syncthreads();
  const int mybstar = reinterpret_cast<const int*>(sm + L::OFF_BSTAR)[lr];
  float thr = -INFINITY;
  const int cnt_limit = a.cap - KB;
  // ---- pass 2: collect the keys in the k-th best's bin or above
  stream([&](int blk) {
    float s[4][4];
    block_scores(sm + L::OFF_K, bqh, bql, blk, N, g, c16, s);
    bool inb[4][4];
    bool any = false;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int b = min(255, max(0, (int)((s[kt][r] - lo) * scale)));
        inb[kt][r] = rowok && s[kt][r] > -INFINITY && b >= mybstar;
        any |= inb[kt][r] && s[kt][r] > thr;
      }
    if (__ballot(any) != 0) {
      const int* cnt = reinterpret_cast<const int*>(sm + L::OFF_CNT);
      const bool full = rowok && cnt[lr] > cnt_limit;
      if (__ballot(full) != 0) {
        select_rows<NW, NV>(sm, a, bh, row0, w, g, c16, false);
        thr = reinterpret_cast<const float*>(sm + L::OFF_THR)[lr];
      }
      int* cntw = reinterpret_cast<int*>(sm + L::OFF_CNT) + lr;
      float* vals = reinterpret_cast<float*>(sm + L::OFF_BUF + (size_t)lr * a.cap * 8);
      int* keys = reinterpret_cast<int*>(vals + a.cap);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (inb[kt][r] && s[kt][r] > thr) {
            const int pos = atomicAdd(cntw, 1);
            vals[pos] = s[kt][r];
            keys[pos] = blk * KB + 16 * kt + 4 * g + r;
          }
    }
  });
  __syncthreads();
  select_rows<NW, NV>(sm, a, bh, row0, w, g, c16, true);
}

}  // namespace lmk

bool landmark_bf16_supported(const Shape& s) {
  // the select kernel's per-row buffer: k kept plus one block, and room for a
  // bitmap of N keys at the end
  int need = s.k + 2 * lmk::KB;
  if (need < (s.N + 63) / 64) need = (s.N + 63) / 64;
  return s.bf16 && need <= 512;
}

size_t landmark_minmax_bytes(const Shape& s) { return (size_t)s.BH * s.m * 2 * sizeof(float); }

template <int NW, int NV>
static hipError_t launch_select(const lmk::Args& a0, const Shape& s, hipStream_t st) {
  lmk::Args a = a0;
  a.cap = 16 * NV;
  a.rblocks = (s.m + 16 * NW - 1) / (16 * NW);
  const size_t lds = lmk::SelLayout<NW>::bytes(a.cap);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)lmk::lmk_select_kernel<NW, NV>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  const int grid = ((s.BH + 7) / 8) * 8 * a.rblocks;
  lmk::lmk_select_kernel<NW, NV><<<grid, 64 * NW, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_landmark_bf16(const float* ql, const void* K, const void* V, int32_t* idx,
                                float* vl, float* minmax, const Shape& s, hipStream_t st) {
  lmk::Args a{ql, (const uint16_t*)K, (const uint16_t*)V, idx, vl, minmax,
              s.BH, s.N, s.m, s.k, 0, 0};
  // values: 64 rows per workgroup (16 per wave)
  {
    constexpr int NW = 4;
    a.rblocks = (s.m + 16 * NW - 1) / (16 * NW);
    const int grid = ((s.BH + 7) / 8) * 8 * a.rblocks;
    lmk::lmk_values_kernel<NW><<<grid, 64 * NW, 0, st>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // select: per-row buffer of k + 128 entries (one block of slack plus room
  // for the boundary bin, so the exact cut-back is rarely needed), at least
  // N/64 (the final bitmap); 32 rows per workgroup, 16 for big buffers
  int need = s.k + 2 * lmk::KB;
  if (need < (s.N + 63) / 64) need = (s.N + 63) / 64;
  if (need <= 128) return launch_select<2, 8>(a, s, st);
  if (need <= 192) return launch_select<2, 12>(a, s, st);
  if (need <= 256) return launch_select<2, 16>(a, s, st);
  if (need <= 384) return launch_select<1, 24>(a, s, st);
  if (need <= 512) return launch_select<1, 32>(a, s, st);
  return hipErrorInvalidValue;
}

}  // namespace mita
