// The whole MiTA forward for one (batch, head) in one workgroup, for short
// token grids (N <= 208, m <= 32, k <= 32, d = 64, bf16 inputs): the DeiT-T /
// DeiT-S shape (14x14 patches, 5x5 landmarks, k = 25) of the page
// "NeurIPS'26：注意力也是FFN？从快权重出发，重新理解高效注意力", section
// "用少量地标查询，同时构造全局概括与细节专家" and Algorithm 1.
//
// A persistent grid of 8-wave workgroups, two per CU, each walking heads.  A
// head needs 79 KB of LDS, so two heads are in flight per CU and one's
// barrier-bound phases overlap the other's work.  K rows for the scores and
// the routing and expert tiles' Q rows are read straight from global memory
// (L2 after first touch) as MFMA operands; the head's Q rows (for pooling),
// then its scores, then its V rows (f16), histograms, a copy of K for the
// expert tiles and small tables live in LDS:
//   B  landmark pooling from the Q rows -> Q_L (fp32), split bf16 hi + lo;
//   C  S^T = K Q_L^T on bf16 MFMA (hi + lo: near-fp32 scores, so top-k sets
//      and routes are decided at fp32 accuracy), into the shared region X;
//   D  per landmark row, exact top-k: one 128-bin histogram over the row's
//      range, every key above the k-th best's bin taken, that bin's keys by
//      rank (ties to the lower key id); then P = exp(S - max) in f16;
//   V  V rows (f16, one padded 144-byte row per key) replace the scores in
//      X; E and G take V^T fragments from them with the transposing LDS read
//      (four keys of one channel per lane and instruction), so an expert's
//      scattered key rows are gathered eight bytes per lane at a time;
//   E  V_L^T = V^T P^T on f16 MFMA, normalised by the row sums;
//   E' R^T = Q_L Q^T per token tile: routes by a 16-lane argmax (ties to the
//      lower landmark);
//   F  stable counting sort of the queries by route (popcounts of each
//      expert's query bitmap) into 16-query tiles of the sorted order;
//   G  per tile: logits^T = [Q_L; K_e] Q_g^T (bf16 MFMA; the shared half
//      recomputed from Q_L, K_e rows gathered from the LDS copy of K), one
//      softmax over the m + k entries per query, and out^T = [V_L; V_e]^T P^T
//      (f16 MFMA, P fed straight from the logits' accumulators), in fp32,
//      stored in whole 128-byte lines.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

namespace mita {
namespace fused {

constexpr int MAXNT = 13;           // 16-token tiles
constexpr int NP = MAXNT * 16;      // 208 padded tokens
constexpr int KPMAX = 224;          // keys padded to a multiple of 32 (P V k-steps)
constexpr int THREADS = 512;
constexpr int NWAVES = THREADS / 64;
constexpr int TPW = (MAXNT + NWAVES - 1) / NWAVES;  // 16-token tiles per wave
constexpr int VITEMS = (8 * (KPMAX / 2) + THREADS - 1) / THREADS;  // V pair items per thread
constexpr int MMAX = 32, KMAX = 32;

constexpr int V_STRIDE = 144;       // bytes per Q / V row (64 16-bit channels + pad: rows 4 banks apart)
constexpr int S_STRIDE = 212;       // floats per score row
constexpr int H_STRIDE = 528;       // bytes per histogram / P row
constexpr int BLIST = 16;           // boundary-bin entries ranked through a list
constexpr int TBM_WORDS = (16 * MAXNT + 63) / 32;  // key bitmap words (+1 for a 2-word read)
static_assert(8 * BLIST + 4 * TBM_WORDS <= 512, "list and bitmap fit in a histogram row");
constexpr int VLT_STRIDE = 80;      // bytes per V_L^T row (f16 landmarks)

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int X_BYTES = cmax(MMAX * S_STRIDE * 4, KPMAX * V_STRIDE);
constexpr int OFF_X = 0;                          // Q rows (B), S (C, D), then V rows (E, G)
constexpr int OFF_H = OFF_X + X_BYTES;
// H: histograms and P rows (D, E), then the head's K rows, bf16 and
// chunk-swizzled like Q_L, for the expert tiles (G)
constexpr int H_BYTES = MMAX * H_STRIDE > NP * 128 ? MMAX * H_STRIDE : NP * 128;
constexpr int OFF_QLH = OFF_H + H_BYTES;
constexpr int OFF_QLL = OFF_QLH + MMAX * 128;
constexpr int OFF_VLT = OFF_QLL + MMAX * 128;
constexpr int OFF_IDX = OFF_VLT + 64 * VLT_STRIDE;
constexpr int OFF_ROUTE = OFF_IDX + MMAX * KMAX * 4;
constexpr int OFF_PERM = OFF_ROUTE + 256 * 4;
constexpr int OFF_BM = OFF_PERM + 256 * 4;        // [32 experts][8] words: query bitmaps
constexpr int OFF_OFFS = OFF_BM + MMAX * 8 * 4;   // [33] int: expert offsets in PERM
constexpr int OFF_STAT = OFF_OFFS + 48 * 4;       // the non-empty experts' bit mask
constexpr int OFF_WB = OFF_STAT + 16;             // [MMAX][4][8] window-membership bytes
constexpr int OFF_LUT = OFF_WB + MMAX * 4 * 8;    // [16] x 4 bf16: a nibble's bits as 0 / 1
constexpr int OFF_INVC = OFF_LUT + 16 * 8;        // [MMAX] 1 / pooling window size
constexpr int LDS_BYTES = OFF_INVC + MMAX * 4;
static_assert(2 * LDS_BYTES <= 160 * 1024, "two workgroups per gfx950 CU");
static_assert(OFF_H % 16 == 0 && OFF_QLH % 16 == 0 && OFF_VLT % 16 == 0 && OFF_IDX % 16 == 0 &&
                  OFF_BM % 16 == 0,
              "16-byte aligned LDS regions");

struct Outputs {
  float* out;
  int32_t* idx;
  int32_t* route;
  float* ql;
  float* vl;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
};

__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// This thread's coordinates, re-derived through an opaque zero at the start of
// each phase: the compiler then recomputes them (a few cheap instructions)
// instead of holding them, and values built from them, across phases.
#define FUSED_IDS                                                              \
  const int tid = threadIdx.x + opaque_zero(), lane = tid & 63, w = tid >> 6; \
  const int g = lane >> 4, c16 = lane & 15;                                    \
  (void)lane;                                                                  \
  (void)w;                                                                     \
  (void)g;                                                                     \
  (void)c16

template <typename P>
__device__ __forceinline__ P* lds(char* base, int off) {
  return reinterpret_cast<P*>(base + off);
}

// Q_L fragments (hi, lo) for both 16-landmark tiles and both 32-channel
// steps: lane holds Q_L[16lt + c16][32ks + 8g .. +8].  They serve as the B
// operand of S^T and R and as the A operand of the shared logits.
__device__ __forceinline__ void load_ql(char* sm, u32x4 (&qlh)[2][2], u32x4 (&qll)[2][2], int g,
                                        int c16) {
#pragma unroll
  for (int lt = 0; lt < 2; ++lt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      qlh[lt][ks] = *lds<u32x4>(sm, OFF_QLH + rc(16 * lt + c16, 4 * ks + g));
      qll[lt][ks] = *lds<u32x4>(sm, OFF_QLL + rc(16 * lt + c16, 4 * ks + g));
    }
}

// A head's Q or V rows as items: key pairs (2p, 2p+1) of 8-channel chunk c,
// items tid + THREADS i (c = item % 8, p = item / 8: eight threads read one
// 128-byte row, and their 16-byte LDS stores spread over the banks).
struct VRows {
  u32x4 v0[VITEMS], v1[VITEMS];
};

__device__ __forceinline__ void load_v(VRows& vr, Rsrc rows, int N, int tid) {
#pragma unroll
  for (int i = 0; i < VITEMS; ++i) {
    const int id = tid + THREADS * i;
    const int c = id & 7, p = id >> 3;
    const int j0 = 2 * p, j1 = 2 * p + 1;
    vr.v0[i] = ld16(rows, p < KPMAX / 2 && j0 < N ? j0 * 128 + c * 16 : PAST);
    vr.v1[i] = ld16(rows, p < KPMAX / 2 && j1 < N ? j1 * 128 + c * 16 : PAST);
  }
}

// V rows (f16) over X from the same items: each key's 8-channel chunk c as one
// 16-byte store.
__device__ __forceinline__ void store_v(const VRows& vr, char* sm, int tid) {
#pragma unroll
  for (int i = 0; i < VITEMS; ++i) {
    const int id = tid + THREADS * i;
    const int c = id & 7, p = id >> 3;
    if (p < KPMAX / 2) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 x = h ? vr.v1[i] : vr.v0[i];
        u32x4 f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          f[q] = pk_f16(__uint_as_float(x[q] << 16), __uint_as_float(x[q] & 0xFFFF0000u));
        *lds<u32x4>(sm, OFF_X + (2 * p + h) * V_STRIDE + 16 * c) = f;
      }
    }
  }
}

// Q rows (bf16, as loaded) over X from the same register layout: each token's
// 8-channel chunk c as one 16-byte store.  (Pooling reads Q^T fragments from
// them with the transposing LDS read.)
__device__ __forceinline__ void store_q(const VRows& qr, char* sm, int tid) {
#pragma unroll
  for (int i = 0; i < VITEMS; ++i) {
    const int id = tid + THREADS * i;
    const int c = id & 7, p = id >> 3;
    if (p < KPMAX / 2) {
      *lds<u32x4>(sm, OFF_X + (2 * p) * V_STRIDE + 16 * c) = qr.v0[i];
      *lds<u32x4>(sm, OFF_X + (2 * p + 1) * V_STRIDE + 16 * c) = qr.v1[i];
    }
  }
}

// EXTRAS: whether any of the optional intermediate outputs is requested; the
// plain forward is compiled without their stores and branches.
template <bool EXTRAS>
__global__ __launch_bounds__(THREADS, 4) void mita_fused_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, Outputs o, int BH, int gh, int gw, int mh, int mw, int k) {
  __shared__ __attribute__((aligned(16))) char sm[LDS_BYTES];
  const int N = gh * gw, m = mh * mw;
  const int nt = (N + 15) >> 4;
  const int KP = (N + 31) & ~31;
  const float kLogitScale = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) * log2(e): base-2 softmax
  const size_t head_elems = (size_t)N * 64;
  const u32x4 z = {0u, 0u, 0u, 0u};
  static_assert(NWAVES == 8, "pooling: one 16-channel x 16-landmark tile per wave");

  // expert key slots past k stay 0 for every head (top-k fills slots < k)
  for (int q = threadIdx.x; q < MMAX * KMAX; q += THREADS) *lds<int>(sm, OFF_IDX + q * 4) = 0;
  // each landmark's window (rows y0 .. y1, columns x0 .. x1) once, into the
  // histogram region (spent long before the first head's top-k), and 1 /
  // its size (0 past m)
  if (threadIdx.x < MMAX) {
    const int L = threadIdx.x;
    float inv_cnt = 0.f;
    int y0 = 0, y1 = 0, x0 = 0, x1 = 0;
    if (L < m) {
      pool_window(L / mw, gh, mh, &y0, &y1);
      pool_window(L % mw, gw, mw, &x0, &x1);
      inv_cnt = 1.0f / (float)((y1 - y0) * (x1 - x0));
    }
    *lds<i32x4>(sm, OFF_H + L * 16) = i32x4{y0, y1, x0, x1};
    *lds<float>(sm, OFF_INVC + L * 4) = inv_cnt;
  }
  // bf16 1.0 / 0 for each bit of a nibble, pairs packed as the MFMA operand
  if (threadIdx.x < 16) {
    const uint32_t n = threadIdx.x, one = 0x3F80u;
    *lds<u32x2>(sm, OFF_LUT + n * 8) = u32x2{(n & 1u ? one : 0u) | (n & 2u ? one << 16 : 0u),
                                             (n & 4u ? one : 0u) | (n & 8u ? one << 16 : 0u)};
  }
  __syncthreads();
  // which tokens each landmark window holds (the same for every head): byte
  // [L][g][ks] has bit t set when token 32ks + 8g + t lies in L's window, so a
  // lane's bytes for every k-step of the pooling product are one 8-byte read
  static_assert(KPMAX / 32 <= 8, "one byte per k-step");
  for (int it = threadIdx.x; it < MMAX * 4 * 8; it += THREADS) {
    const int L = it >> 5, gg = (it >> 3) & 3, ks = it & 7, o = 4 * ks + gg;
    uint32_t bits = 0;
    if (L < m && 8 * o < KPMAX) {
      const i32x4 wd = *lds<i32x4>(sm, OFF_H + L * 16);
      // tokens 8o .. 8o + 7: one division, then step along the row
      int y = (8 * o) / gw, x = 8 * o - y * gw;
      for (int t = 0; t < 8; ++t) {
        bits |= (8 * o + t < N && y >= wd[0] && y < wd[1] && x >= wd[2] && x < wd[3] ? 1u : 0u) << t;
        if (++x == gw) {
          x = 0;
          ++y;
        }
      }
    }
    *lds<uint8_t>(sm, OFF_WB + it) = (uint8_t)bits;
  }

  // a head's Q rows are requested while the previous head runs its expert tiles
  VRows qr;
  if (blockIdx.x < BH) load_v(qr, head_rows(Q + (size_t)blockIdx.x * head_elems, N), N, threadIdx.x);

  for (int bh = blockIdx.x; bh < BH; bh += gridDim.x) {
    // Thread coordinates are re-derived through an opaque zero every head so
    // that the compiler recomputes per-thread LDS addresses inside each phase
    // instead of hoisting them all out of the loop and pinning registers.
    const int tid = threadIdx.x + opaque_zero(), lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const uint16_t* Qh = Q + bh * head_elems;
    const Rsrc rQ = head_rows(Qh, N), rK = head_rows(K + bh * head_elems, N);
    __syncthreads();  // the previous head is done with LDS
    store_q(qr, sm, tid);
    if (tid < MMAX * 8) *lds<uint32_t>(sm, OFF_BM + tid * 4) = 0u;
    // C's K rows, issued after the Q row store so that its wait does not cover them
    u32x4 ka[TPW][2];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int key = 16 * (w + NWAVES * j) + c16;
      const int off = key < N ? key * 128 + 16 * g : PAST;
      ka[j][0] = ld16(rK, off);
      ka[j][1] = ld16(rK, off + 64);
    }
    __syncthreads();

    // The head's short, barrier-separated phases (B to F and the V_L step)
    // issue at a raised wave priority, the expert tiles (G) at the normal
    // one: the other workgroup on the CU is then most often in its tiles, and
    // its instructions fill the gaps of this workgroup's barrier-bound path
    // instead of delaying it (DeiT-S: 67.0 -> 64.9 us per step; priority 1
    // gave 65.1, a higher level for top-k and routing alone none).
    __builtin_amdgcn_s_setprio(3);
    // ---------------- B: landmark pooling as a contraction over tokens,
    // Q_L^T = Q^T W (W: 0/1 window membership) on bf16 MFMA, then / window size
    {
      FUSED_IDS;
      const int ct = w & 3, L = 16 * (w >> 2) + c16;
      f32x4 acc = zero4();
      const u32x2 wb = *lds<u32x2>(sm, OFF_WB + (L * 4 + g) * 8);
      const int nks = KP / 32 + opaque_zero();  // per-step tests made here, not held
      // Q^T[channels 16ct ..][tokens 32ks + 8g ..]: lane (g, c16) points at
      // token 32ks + 8g + (c16 >> 2) (+ 4), channels 16ct + 4 (c16 & 3) ..
      const int qa = OFF_X + (8 * g + (c16 >> 2)) * V_STRIDE + 32 * ct + 8 * (c16 & 3);
#pragma unroll
      for (int ks = 0; ks < KPMAX / 32; ++ks) {
        if (ks < nks) {
          const u32x2 lo = lds_tr16(sm + qa + 32 * ks * V_STRIDE);
          const u32x2 hi = lds_tr16(sm + qa + (32 * ks + 4) * V_STRIDE);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          // B = W[tokens 32ks + 8g .. +7][landmark L]: one membership byte, two nibbles
          const uint32_t byte = (wb[ks >> 2] >> (8 * (ks & 3))) & 0xFFu;
          const u32x2 b01 = *lds<u32x2>(sm, OFF_LUT + (byte & 15u) * 8);
          const u32x2 b23 = *lds<u32x2>(sm, OFF_LUT + (byte >> 4) * 8);
          const u32x4 b = {b01[0], b01[1], b23[0], b23[1]};
          acc = mfma_bf16(a, b, acc);
        }
      }
      // lane holds Q_L[landmark L][channels 16ct + 4g .. +3]: fp32, then bf16 hi + lo
      const float inv_cnt = *lds<float>(sm, OFF_INVC + L * 4);
      const float q0 = acc[0] * inv_cnt, q1 = acc[1] * inv_cnt;
      const float q2 = acc[2] * inv_cnt, q3 = acc[3] * inv_cnt;
      // the LDS copy carries tau * log2(e): scores, routing scores and shared
      // logits then come out of the products in the base-2 softmax domain
      const float s0 = q0 * kLogitScale, s1 = q1 * kLogitScale;
      const float s2 = q2 * kLogitScale, s3 = q3 * kLogitScale;
      const uint32_t h01 = pk_bf16(s0, s1), h23 = pk_bf16(s2, s3);
      const uint32_t l01 = pk_bf16(s0 - bf16_bits_to_f32(h01 & 0xFFFFu), s1 - bf16_bits_to_f32(h01 >> 16));
      const uint32_t l23 = pk_bf16(s2 - bf16_bits_to_f32(h23 & 0xFFFFu), s3 - bf16_bits_to_f32(h23 >> 16));
      const int off = rc(L, 2 * ct + (g >> 1)) + (g & 1) * 8;
      *lds<u32x2>(sm, OFF_QLH + off) = u32x2{h01, h23};
      *lds<u32x2>(sm, OFF_QLL + off) = u32x2{l01, l23};
      if (EXTRAS && o.ql && L < m)
        *reinterpret_cast<float4*>(o.ql + ((size_t)bh * m + L) * 64 + 16 * ct + 4 * g) =
            make_float4(q0, q1, q2, q3);
    }
    __syncthreads();

    // ---------------- C: S^T = K Q_L^T (K rows from global memory) -> S rows in X,
    // and (same Q_L fragments) the routing scores of E'
    {
      FUSED_IDS;
      u32x4 qlh[2][2], qll[2][2];
      load_ql(sm, qlh, qll, g, c16);
      // every key column up to 16 * MAXNT is written: keys past N get -inf
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tt = w + NWAVES * j;
        if (tt < MAXNT) {
          const int kb = 16 * tt + 4 * g;
#pragma unroll
          for (int lt = 0; lt < 2; ++lt) {
            f32x4 c = zero4();
            if (tt < nt) {
              c = mfma_bf16(ka[j][0], qlh[lt][0], c);
              c = mfma_bf16(ka[j][0], qll[lt][0], c);
              c = mfma_bf16(ka[j][1], qlh[lt][1], c);
              c = mfma_bf16(ka[j][1], qll[lt][1], c);
            }
            // lane holds S^T[key kb + r][landmark 16lt + c16]
            *lds<float4>(sm, OFF_X + ((16 * lt + c16) * S_STRIDE + kb) * 4) =
                make_float4(kb < N ? c[0] : -INFINITY, kb + 1 < N ? c[1] : -INFINITY,
                            kb + 2 < N ? c[2] : -INFINITY, kb + 3 < N ? c[3] : -INFINITY);
          }
        }
      }
    }
    // the routing phase's query rows fly while the rows' top-k runs
    u32x4 qb[TPW][2];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int tok = 16 * (w + NWAVES * j) + c16;
      const int off = tok < N ? tok * 128 + 16 * g : PAST;
      qb[j][0] = ld16(rQ, off);
      qb[j][1] = ld16(rQ, off + 64);
    }
    __syncthreads();

    // ---------------- D: exact top-k of each landmark row; then P = exp(S - max) in f16
    {
      FUSED_IDS;
      static_assert(4 * NWAVES == MMAX, "one landmark row per 16-lane group");
      const int i = 4 * w + g;  // landmark row of this 16-lane group
      const bool active = i < m;
      if (__ballot(active) != 0) {
        const int t = c16, key0 = MAXNT * t;  // this lane owns keys key0 .. key0 + 12
        // scores (-inf at padding keys; rows past m hold zeros and are
        // computed but never used)
        float v[MAXNT];
#pragma unroll
        for (int u = 0; u < MAXNT; ++u) v[u] = *lds<float>(sm, OFF_X + (i * S_STRIDE + key0 + u) * 4);
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int u = 0; u < MAXNT; ++u) {
          lo = fminf(lo, key0 + u < N ? v[u] : INFINITY);
          hi = fmaxf(hi, v[u]);
        }
        lo = g16_minf(lo);
        hi = g16_maxf(hi);
        const float rmax = hi;
        // 128 equal bins over [lo, hi]: f = (x - lo) * 128 / (hi - lo), bin =
        // floor(f) clamped to [0, 127] (A > 0, so padding has f = -inf and
        // lands in bin 0, whose counter starts at minus the padding count).
        // Lane t owns the 32-bit counters of bins 8t .. 8t+7.
        const float A = hi > lo ? fminf(128.0f / (hi - lo), 1e30f) : 1.f, B = -lo * A;
        float f[MAXNT];
#pragma unroll
        for (int u = 0; u < MAXNT; ++u) f[u] = __builtin_fmaf(v[u], A, B);
        char* hrow = sm + OFF_H + i * H_STRIDE;
        uint32_t* hist = reinterpret_cast<uint32_t*>(hrow);
        // (constants through an opaque zero: built here, not held in
        // registers across the head loop)
        const uint32_t z0 = (uint32_t)opaque_zero();
        const float c127 = 127.0f + (float)opaque_zero();
        *reinterpret_cast<u32x4*>(hrow + 32 * t) = u32x4{t == 0 ? (uint32_t)(N - 16 * MAXNT) : z0, z0, z0, z0};
        *reinterpret_cast<u32x4*>(hrow + 32 * t + 16) = u32x4{z0, z0, z0, z0};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < MAXNT; ++u) atomicAdd(hist + (int)__builtin_amdgcn_fmed3f(f[u], 0.f, c127), 1u);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // the boundary bin b*: the bin holding the k-th largest score; `above`
        // keys lie in higher bins, `inb` in b* itself
        int bstar = 0, above = 0, inb = 0;
        {
          const u32x4 d0 = *reinterpret_cast<const u32x4*>(hrow + 32 * t);
          const u32x4 d1 = *reinterpret_cast<const u32x4*>(hrow + 32 * t + 16);
          const int cb[8] = {(int)d0[0], (int)d0[1], (int)d0[2], (int)d0[3],
                             (int)d1[0], (int)d1[1], (int)d1[2], (int)d1[3]};
          int local = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q) local += cb[q];
          // keys in bins above this lane's (higher lane = higher bins)
          int acc = g16_suffix(local) - local;
          int hit_b = 0, hit_a = 0, hit_n = 0;
#pragma unroll
          for (int q = 7; q >= 0; --q) {
            const bool h = acc < k && acc + cb[q] >= k;
            hit_b = h ? 8 * t + q : hit_b;
            hit_a = h ? acc : hit_a;
            hit_n = h ? cb[q] : hit_n;
            acc += cb[q];
          }
          // exactly one lane of an active group hits: masked group sums broadcast
          const bool mine = active && hit_n > 0;
          bstar = g16_addi(mine ? hit_b : 0);
          above = g16_addi(mine ? hit_a : 0);
          inb = g16_addi(mine ? hit_n : 0);
        }
        // bin > b* <=> f >= b* + 1 and bin == b* <=> f in [b*, b* + 1), with the
        // clamped end bins open-ended
        const float th = bstar == 127 ? INFINITY : (float)(bstar + 1);
        const float tl = bstar == 0 ? -1e30f : (float)bstar;
        uint32_t take = 0, bnd = 0;
#pragma unroll
        for (int u = 0; u < MAXNT; ++u) {
          take |= (f[u] >= th ? 1u : 0u) << u;
          bnd |= (f[u] >= tl && f[u] < th ? 1u : 0u) << u;
        }
        // the boundary bin supplies k - above keys: all of them when that is
        // its whole count, else the best first (larger score, then lower key
        // id), one per round
        int need = active ? k - above : 0;
        if (active && need == inb) {
          take |= bnd;
          need = 0;
        }
        if (__ballot(need > 0 && inb > BLIST) == 0) {
          // every boundary bin of the wave fits a BLIST-entry list: the bin's
          // keys are listed in the row's spent histogram, lane t ranks entry t
          // against the list (larger score first, then lower key id), and the
          // entries ranked below `need` are marked in a key bitmap from which
          // each lane takes its own bits
          float* lst_v = reinterpret_cast<float*>(hrow);
          int* lst_k = reinterpret_cast<int*>(hrow + 4 * BLIST);
          uint32_t* tbm = reinterpret_cast<uint32_t*>(hrow + 8 * BLIST);
          const bool sel = need > 0;
          const int nbl = sel ? __popc(bnd) : 0;
          int p = g16_prefix(nbl) - nbl;
          // (the histogram has been read: its row now takes the list)
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          // scores re-read from the score rows by key (a lane holds one or two)
          // (the group's bnd bits number exactly inb <= BLIST; the bound on p
          // keeps the writes inside the list regardless)
          for (uint32_t bb = sel ? bnd : 0u; bb != 0u && p < BLIST; bb &= bb - 1u, ++p) {
            const int key = key0 + __builtin_ctz(bb);
            lst_v[p] = *lds<float>(sm, OFF_X + (i * S_STRIDE + key) * 4);
            lst_k[p] = key;
          }
          if (t < TBM_WORDS) tbm[t] = 0u;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (sel && t < inb) {
            const float ev = lst_v[t];
            const int ek = lst_k[t];
            int r = 0;
            for (int j = 0; j < inb; ++j) {
              const float jv = lst_v[j];
              r += (jv > ev || (jv == ev && lst_k[j] < ek)) ? 1 : 0;
            }
            if (r < need) atomicOr(tbm + (ek >> 5), 1u << (ek & 31));
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (sel) {
            const int w0 = key0 >> 5;
            const uint64_t two = (uint64_t)tbm[w0] | ((uint64_t)tbm[w0 + 1] << 32);
            take |= (uint32_t)(two >> (key0 & 31)) & ((1u << MAXNT) - 1u);
          }
          need = 0;
        } else if (__ballot(need > 0) != 0) {
          // each lane's best boundary candidate (descending scan: ties keep the
          // lower key); a lane rescans only after its candidate is taken and
          // it holds more
          auto best_of = [&](float& bv, int& bk) {
            bv = -INFINITY;
            bk = 0x7FFFFFFF;
#pragma unroll
            for (int u = MAXNT - 1; u >= 0; --u) {
              const bool c = (bnd >> u & 1u) && v[u] >= bv;
              bv = c ? v[u] : bv;
              bk = c ? key0 + u : bk;
            }
          };
          float bv;
          int bk;
          best_of(bv, bk);
          for (; __ballot(need > 0) != 0; --need) {
            float wv = bv;
            int wk = bk;
            g16_argmax(wv, wk);
            const bool win = need > 0 && wk == bk && bk != 0x7FFFFFFF;
            if (win) {
              const int u = bk - key0;
              take |= 1u << u;
              bnd &= ~(1u << u);
              bv = -INFINITY;
              bk = 0x7FFFFFFF;
            }
            if (__ballot(win && bnd != 0) != 0) {
              if (win && bnd != 0) best_of(bv, bk);
            }
          }
        }
        // the expert: kept key ids in ascending order (lane-major, since each
        // lane owns a contiguous key range); lanes without a key to write
        // (and, as a guard, any position past the row's slots) aim at their
        // own word of the spent histogram
        {
          const int cnt = __popc(take);
          int pos = g16_prefix(cnt) - cnt;
#pragma unroll
          for (int u = 0; u < MAXNT; ++u) {
            const bool bit = take >> u & 1u;
            const int off = bit && pos < KMAX ? OFF_IDX + (i * KMAX + pos) * 4 : OFF_H + i * H_STRIDE + 4 * t;
            *lds<int>(sm, off) = key0 + u;
            pos += bit ? 1 : 0;
          }
        }
        // P row (f16) over this row's bytes, zero past the owned keys up to the
        // padded width (its sum comes out of the V_L products)
        uint16_t* prow = reinterpret_cast<uint16_t*>(hrow);
        const float moff = active ? -rmax : 0.f;  // scores are in the base-2 domain
#pragma unroll
        for (int u = 0; u < MAXNT; ++u)
          prow[key0 + u] = (uint16_t)f16_bits(__builtin_amdgcn_exp2f(v[u] + moff));
        static_assert(MAXNT * 16 + 16 == KPMAX, "one zero column per lane past the owned keys");
        prow[MAXNT * 16 + t] = 0;
      }
    }
    // ---------------- E': R^T = Q_L Q^T per token tile (Q rows from global memory): routes
    {
      FUSED_IDS;
      u32x4 qlh[2][2], qll[2][2];
      load_ql(sm, qlh, qll, g, c16);
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tt = w + NWAVES * j;
        if (tt >= nt) break;
        const int tok = 16 * tt + c16;
        f32x4 acc[2];
#pragma unroll
        for (int lt = 0; lt < 2; ++lt) {
          f32x4 c = zero4();
          c = mfma_bf16(qlh[lt][0], qb[j][0], c);
          c = mfma_bf16(qll[lt][0], qb[j][0], c);
          c = mfma_bf16(qlh[lt][1], qb[j][1], c);
          c = mfma_bf16(qll[lt][1], qb[j][1], c);
          acc[lt] = c;  // lane holds R[token tok][landmark 16lt + 4g + r]
        }
        float best = -INFINITY;
        int bi = 0;
#pragma unroll
        for (int lt = 0; lt < 2; ++lt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int L = 16 * lt + 4 * g + r;  // increasing: strict '>' keeps the lowest
            const float v = L < m ? acc[lt][r] : -INFINITY;
            if (v > best) { best = v; bi = L; }
          }
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
          const float ov = __shfl_xor(best, off, 64);
          const int oi = __shfl_xor(bi, off, 64);
          if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
        }
        if (g == 0 && tok < N) {
          *lds<int>(sm, OFF_ROUTE + tok * 4) = bi;
          atomicOr(lds<uint32_t>(sm, OFF_BM + (bi * 8 + (tok >> 5)) * 4), 1u << (tok & 31));
          if (EXTRAS && o.route) o.route[(size_t)bh * N + tok] = bi;
        }
      }
    }
    // the V rows fly while the queries are grouped
    VRows vr;
    load_v(vr, head_rows(V + bh * head_elems, N), N, tid);
    __syncthreads();

    if (EXTRAS && o.idx) {
      for (int q = tid; q < m * k; q += THREADS)
        o.idx[(size_t)bh * m * k + q] = *lds<int>(sm, OFF_IDX + ((q / k) * KMAX + q % k) * 4);
    }

    // ---------------- F: group the queries by route (stable): expert counts and
    // offsets from the route bitmaps, then each query's place in PERM
    {
      FUSED_IDS;
      if (w == 0) {
        int cnt = 0;
        if (lane < m) {
          const u32x4 b0 = *lds<u32x4>(sm, OFF_BM + lane * 32);
          const u32x4 b1 = *lds<u32x4>(sm, OFF_BM + lane * 32 + 16);
          cnt = __popc(b0[0]) + __popc(b0[1]) + __popc(b0[2]) + __popc(b0[3]) + __popc(b1[0]) +
                __popc(b1[1]) + __popc(b1[2]) + __popc(b1[3]);
        }
        int incl = cnt;  // inclusive scan over the wave (lanes past m hold 0)
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int x = __shfl_up(incl, off, 64);
          if (lane >= off) incl += x;
        }
        const int off_e = incl - cnt;  // lane m holds N
        if (lane <= m) *lds<int>(sm, OFF_OFFS + lane * 4) = off_e;
        const uint64_t ne = __ballot(cnt > 0);
        if (lane == 0) *lds<uint32_t>(sm, OFF_STAT) = (uint32_t)ne;
        if (EXTRAS && lane < m) {
          if (o.counts) o.counts[(size_t)bh * m + lane] = cnt;
          if (o.offsets) o.offsets[(size_t)bh * (m + 1) + lane] = off_e;
        }
        if (EXTRAS && lane == m && o.offsets) o.offsets[(size_t)bh * (m + 1) + m] = N;
      }
      __syncthreads();
      if (tid < N) {
        // rank among the expert's queries = its bitmap bits below tid
        const int e = *lds<int>(sm, OFF_ROUTE + tid * 4);
        const u32x4 b0 = *lds<u32x4>(sm, OFF_BM + e * 32);
        const u32x4 b1 = *lds<u32x4>(sm, OFF_BM + e * 32 + 16);
        const uint32_t bw[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const int word = tid >> 5;
        int rank = 0;
#pragma unroll
        for (int q = 0; q < 7; ++q) {
          const uint32_t part = q < word ? bw[q] : (q == word ? bw[q] & ((1u << (tid & 31)) - 1u) : 0u);
          rank += __popc(part);
        }
        const int pos = *lds<int>(sm, OFF_OFFS + e * 4) + rank;
        *lds<int>(sm, OFF_PERM + pos * 4) = tid;
        if (EXTRAS && o.perm) o.perm[(size_t)bh * N + pos] = tid;
      }
      __syncthreads();
    }

    // ---------------- V: V rows (f16) over the score region
    {
      FUSED_IDS;
      store_v(vr, sm, tid);
    }
    __syncthreads();

    // the K rows for the expert tiles' LDS copy fly while V_L is formed
    constexpr int KITEMS = (NP * 8 + THREADS - 1) / THREADS;
    u32x4 kst[KITEMS];
#pragma unroll
    for (int i = 0; i < KITEMS; ++i) {
      const int id = tid + THREADS * i, row = id >> 3;
      kst[i] = ld16(rK, row < N ? row * 128 + 16 * (id & 7) : PAST);
    }

    // ---------------- E: V_L^T = V^T P^T (16-channel x 16-landmark tiles)
    {
      FUSED_IDS;
  #pragma unroll 1
      for (int tile = w; tile < 8; tile += NWAVES) {
        const int ct = tile & 3, lt = tile >> 2;
        // the row sums of the same f16 weights: an all-ones A operand
        const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
        f32x4 acc = zero4(), tot = zero4();
        // V^T[channels 16ct ..][keys 32ks + 8g ..]: lane (g, c16) points at key
        // 32ks + 8g + (c16 >> 2) (+ 4), channels 16ct + 4 (c16 & 3) ..
        const int va = OFF_X + (8 * g + (c16 >> 2)) * V_STRIDE + 32 * ct + 8 * (c16 & 3);
        for (int ks = 0; ks < KP / 32; ++ks) {
          const u32x2 lo = lds_tr16(sm + va + 32 * ks * V_STRIDE);
          const u32x2 hi = lds_tr16(sm + va + (32 * ks + 4) * V_STRIDE);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          const u32x4 b = *lds<u32x4>(sm, OFF_H + (16 * lt + c16) * H_STRIDE + (32 * ks + 8 * g) * 2);
          acc = mfma_f16(a, b, acc);
          tot = mfma_f16(ones, b, tot);
        }
        const int L = 16 * lt + c16;
        const bool ok = L < m;
        const float inv = ok ? __builtin_amdgcn_rcpf(tot[0]) : 0.f;
        float vl4[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          vl4[r] = ok ? acc[r] * inv : 0.f;
          *lds<uint16_t>(sm, OFF_VLT + (16 * ct + 4 * g + r) * VLT_STRIDE + L * 2) =
              (uint16_t)f16_bits(vl4[r]);
        }
        if (EXTRAS && ok && o.vl) {
          *reinterpret_cast<float4*>(o.vl + ((size_t)bh * m + L) * 64 + 16 * ct + 4 * g) =
              make_float4(vl4[0], vl4[1], vl4[2], vl4[3]);
        }
      }

    }
    __syncthreads();  // the P rows are spent
    {
      FUSED_IDS;
#pragma unroll
      for (int i = 0; i < KITEMS; ++i) {
        const int id = tid + THREADS * i, row = id >> 3;
        if (row < NP) *lds<u32x4>(sm, OFF_H + rc(row, id & 7)) = kst[i];
      }
    }
    __syncthreads();

    __builtin_amdgcn_s_setprio(0);
    // ---------------- G: grouped expert attention over 16-query tiles of the
    // sorted order; a tile spans the experts of its queries, each column
    // taking the routed half of its own expert
    {
      FUSED_IDS;
      // (the last head re-reads its own rows, which are in cache, so that the
      // registers are written on every path)
      load_v(qr, head_rows(bh + (int)gridDim.x < BH ? Qh + (size_t)gridDim.x * head_elems : Qh, N), N, tid);
      const uint32_t nonempty =
          __builtin_amdgcn_readfirstlane(*lds<uint32_t>(sm, OFF_STAT));
      const int nqt = (N + 15) >> 4;
      const Rsrc outr = out_rows(o.out + (size_t)bh * N * 64, N);
      // expert e's key rows for this lane's two slot tiles, from the LDS copy
      // (slots past k hold key 0: their logits are masked)
      auto load_k = [&](int e, u32x4 (&ak)[2][2]) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int key = *lds<int>(sm, OFF_IDX + (e * KMAX + 16 * st + c16) * 4);
          ak[st][0] = *lds<u32x4>(sm, OFF_H + rc(key, g));
          ak[st][1] = *lds<u32x4>(sm, OFF_H + rc(key, g + 4));
        }
      };
      // whether this lane's routed slots 4g + r and 16 + 4g + r hold keys
      // (lane masks, fixed for the head: computed once, not per expert)
      bool ok0[4], ok1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ok0[r] = 4 * g + r < k;
        ok1[r] = 16 + 4 * g + r < k;
      }
      for (int tile = w; tile < nqt; tile += NWAVES) {
        const int p0 = 16 * tile, p = p0 + c16;
        const bool live = p < N;  // columns past N compute on the tile's first query
        const int qi = *lds<int>(sm, OFF_PERM + (live ? p : p0) * 4);
        const int ce = *lds<int>(sm, OFF_ROUTE + qi * 4);
        const int e_lo = __builtin_amdgcn_readfirstlane(
            *lds<int>(sm, OFF_ROUTE + *lds<int>(sm, OFF_PERM + p0 * 4) * 4));
        const int e_hi = __builtin_amdgcn_readfirstlane(
            *lds<int>(sm, OFF_ROUTE + *lds<int>(sm, OFF_PERM + min(p0 + 15, N - 1) * 4) * 4));
        // the tile's experts: the non-empty ones in [e_lo, e_hi] (sorted order)
        const uint32_t blocks = nonempty & ((e_hi >= 31 ? ~0u : (2u << e_hi) - 1u) & ~((1u << e_lo) - 1u));
        const u32x4 bq0 = ld16(rQ, qi * 128 + 16 * g);
        const u32x4 bq1 = ld16(rQ, qi * 128 + 16 * g + 64);
        u32x4 ak[2][2];
        // shared logits^T = Q_L Q_g^T (hi + lo; Q_L carries the log2-domain scale)
        float x[16];
        {
          u32x4 qlh[2][2], qll[2][2];
          load_ql(sm, qlh, qll, g, c16);
#pragma unroll
          for (int lt = 0; lt < 2; ++lt) {
            f32x4 c = zero4();
            c = mfma_bf16(qlh[lt][0], bq0, c);
            c = mfma_bf16(qll[lt][0], bq0, c);
            c = mfma_bf16(qlh[lt][1], bq1, c);
            c = mfma_bf16(qll[lt][1], bq1, c);
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * lt + r] = 16 * lt + 4 * g + r < m ? c[r] : -INFINITY;
          }
        }
        // routed logits^T = K_e Q_g^T per expert, kept for the expert's columns
#pragma unroll
        for (int q = 8; q < 16; ++q) x[q] = -INFINITY;
        for (uint32_t bl = blocks; bl != 0;) {
          const int e = __builtin_ctz(bl);
          bl &= bl - 1u;
          load_k(e, ak);
          f32x4 lr[2];
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            f32x4 c = zero4();
            c = mfma_bf16(ak[st][0], bq0, c);
            c = mfma_bf16(ak[st][1], bq1, c);
            lr[st] = c;
          }
          // the expert's columns take its valid slots' logits (the other
          // slots stay -inf)
          const bool mine = ce == e;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[8 + r] = mine && ok0[r] ? lr[0][r] * kLogitScale : x[8 + r];
            x[12 + r] = mine && ok1[r] ? lr[1][r] * kLogitScale : x[12 + r];
          }
        }
        float mx = x[0];
#pragma unroll
        for (int q = 1; q < 16; ++q) mx = fmaxf(mx, x[q]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
#pragma unroll
        for (int q = 0; q < 16; ++q) x[q] = __builtin_amdgcn_exp2f(x[q] - mx);
        // P^T as the B operand: entries {4g+r, 16+4g+r} of each half, query c16
        u32x4 bps, bpr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bps[q] = pk_f16(x[2 * q], x[2 * q + 1]);
          bpr[q] = pk_f16(x[8 + 2 * q], x[8 + 2 * q + 1]);
        }
        // softmax normaliser of the same f16 weights the products use: an
        // all-ones A operand sums every entry column into each output row
        const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
        f32x4 tot = mfma_f16(ones, bps, zero4());
        tot = mfma_f16(ones, bpr, tot);
        const float inv = __builtin_amdgcn_rcpf(tot[0]);
        // out^T = V_L^T P_s^T + sum over the tile's experts of V_e^T P_r^T
        // (P_r^T columns of other experts zeroed)
        f32x4 acc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          // V_L^T[ch 16ct + c16][landmarks 4g..4g+3, 16+4g..16+4g+3]
          const int rowb = OFF_VLT + (16 * ct + c16) * VLT_STRIDE;
          const u32x2 lo2 = *lds<u32x2>(sm, rowb + (4 * g) * 2);
          const u32x2 hi2 = *lds<u32x2>(sm, rowb + (16 + 4 * g) * 2);
          acc[ct] = mfma_f16(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, bps, zero4());
        }
        for (uint32_t bl = blocks; bl != 0;) {
          const int e = __builtin_ctz(bl);
          bl &= bl - 1u;
          const bool mine = ce == e;
          const u32x4 bpe = {mine ? bpr[0] : 0u, mine ? bpr[1] : 0u, mine ? bpr[2] : 0u, mine ? bpr[3] : 0u};
          // V_e^T fragments by transposing reads of the expert's V rows: lane
          // (g, c16) points at the row of slot 4g + (c16 >> 2) (and 16 + 4g +
          // ..), channels 16ct + 4 (c16 & 3) .., and receives channel 16ct +
          // c16 of slots 4g .. 4g + 3 (and 16 + 4g ..).  (Slots past k hold
          // key 0, weighted 0.)
          const int k0 = *lds<int>(sm, OFF_IDX + (e * KMAX + 4 * g + (c16 >> 2)) * 4);
          const int k1 = *lds<int>(sm, OFF_IDX + (e * KMAX + 16 + 4 * g + (c16 >> 2)) * 4);
          const int a0 = OFF_X + k0 * V_STRIDE + 8 * (c16 & 3);
          const int a1 = OFF_X + k1 * V_STRIDE + 8 * (c16 & 3);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const u32x2 lo = lds_tr16(sm + a0 + 32 * ct), hi = lds_tr16(sm + a1 + 32 * ct);
            acc[ct] = mfma_f16(u32x4{lo[0], lo[1], hi[0], hi[1]}, bpe, acc[ct]);
          }
        }
        // lanes c16 and c16 ^ 8 trade their odd channel tiles, so that each
        // store writes whole 128-byte lines: in one instruction the 8 lanes
        // (g, c) and (g, c ^ 8) cover channels 0..31 (or 32..63) of one query
        // (non-temporal: the output is not read again here); a column past N
        // stores past the buffer's range, which the hardware drops
        {
          const f32x4 v0 = acc[0] * inv, v2 = acc[2] * inv;
          const f32x4 r1 = swap8(acc[1] * inv), r3 = swap8(acc[3] * inv);
          const int rqi = swap8(qi);
          const bool rlive = swap8(live ? 1 : 0) != 0;
          const bool lo = c16 < 8;
          const int own = live ? qi * 256 + 16 * g : PAST;
          const int other = rlive ? rqi * 256 + 16 * g : PAST;
          st16_nt(outr, lo ? v0 : r1, lo ? own : other + 64);
          st16_nt(outr, lo ? r1 : v0, lo ? other + 64 : own);
          st16_nt(outr, lo ? v2 : r3, lo ? own + 128 : other + 192);
          st16_nt(outr, lo ? r3 : v2, lo ? other + 192 : own + 128);
        }
      }
    }
  }
}

}  // namespace fused

bool fused_supported(const Shape& s) {
  return s.bf16 && s.s == 1 && s.shared && s.d == 64 && s.N <= fused::NP && s.m <= fused::MMAX &&
         s.k <= fused::KMAX;
}

static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

hipError_t launch_fused(const void* Q, const void* K, const void* V, float* out, int32_t* idx,
                        int32_t* route, float* ql, float* vl, int32_t* counts, int32_t* offsets,
                        int32_t* perm, const Shape& s, hipStream_t st) {
  fused::Outputs o{out, idx, route, ql, vl, counts, offsets, perm};
  // two resident workgroups per CU, each walking heads
  const int slots = 2 * device_cu_count();
  const int grid = s.BH < slots ? s.BH : slots;
  const bool extras = idx || route || ql || vl || counts || offsets || perm;
  auto kernel = extras ? fused::mita_fused_kernel<true> : fused::mita_fused_kernel<false>;
  kernel<<<grid, fused::THREADS, 0, st>>>((const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, o,
                                          s.BH, s.grid_h, s.grid_w, s.m_h, s.m_w, s.k);
  return hipGetLastError();
}

}  // namespace mita
