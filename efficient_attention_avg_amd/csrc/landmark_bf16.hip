// Steps a2-a4 for bf16 inputs on long grids -- the landmark pass (page
// "NeurIPS'26：注意力也是FFN？...", landmark-query section: every landmark
// query scores all keys; its k best keys, ties to the lowest key id, form a
// routed expert; the same scores, softmax-normalised over all N keys, weight V
// into the landmark values V_L).
//
// One kernel.  A workgroup owns 32 landmark rows of one head (two 16-row MFMA
// tiles, so every K block loaded feeds both); its four waves split the head's
// keys (wave w takes the 64-key blocks w, w+4, ...).  Raw scores
// c = Q_L . K (the scale tau = 1/8 is a power of two, so it is folded into the
// softmax and bin constants without changing any order) run on bf16 MFMA
// with K rows loaded straight into the A operand and Q_L split hi + lo
// (fp32-accurate).  Phases, separated by workgroup barriers:
//   V  values: per wave, an online softmax of its keys' scores folded into
//      V_L^T = V^T P^T (f16 MFMA; V staged transposed in the wave's own LDS
//      slot; the running maximum is only raised when a score exceeds it by
//      more than 2^8 in weight, so most blocks skip the rescale); the four
//      partial results merge by log-sum-exp into V_L, and each row's score
//      min and max fix 256 equal histogram bins;
//   H  histogram: the waves recompute their scores (K now in L2) and count
//      them per row in LDS; the bin holding the k-th best is found per row;
//   C  collect: scores in that bin or above go to the row's LDS buffer
//      (k + 64 entries).  The histogram says beforehand whether a row's
//      candidates fit; when one does not (many equal scores), the collection
//      runs one block at a time and cuts such buffers back to their exact k
//      best whenever the next block could overflow them, later keys having to
//      beat the k-th kept one in (value, lower key id) order;
//   F  final: the keys above the boundary bin are all taken, the boundary
//      bin's by rank among themselves (ties to the lower key id); the k ids
//      are written ascending through a bitmap in the row's histogram space
//      (or, for N > 8192, by counting).
// Workgroups of one head are launched on one XCD so its K and V come from HBM
// once and are re-read from that XCD's L2.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

#include <type_traits>

namespace mita {
namespace lmk {

constexpr int KB = 64;                  // keys per block
constexpr int NW = 4;                   // waves per workgroup
constexpr int TL = 2;                   // 16-row MFMA tiles per workgroup
constexpr int ROWS = 16 * TL;           // landmark rows per workgroup
constexpr int VT_STRIDE = KB * 2 + 16;  // bytes per V^T row: 64 f16 keys + pad
constexpr int VT_BYTES = 64 * VT_STRIDE;
constexpr int HIST_STRIDE = 1040;       // one row's 256 32-bit bins + pad (rows 4 banks apart)
constexpr int SPARE_BIN = 256;          // pad word: counts the keys past N of a ragged block
constexpr int BITMAP_MAX_N = 8192;      // keys whose bitmap fits in a histogram row
constexpr int LIST_MAX = 128;           // boundary entries listed in a histogram row
constexpr int MERGE_STRIDE = 68;        // floats per (wave, row): 64 acc, max, sum, min, max
constexpr float kTauLog2e = 0.125f * 1.4426950408889634f;
constexpr float kSlack = 8.0f;          // log2 headroom of the lazily raised maximum

// per-row state in LDS
struct RowState {
  float lo, A, B;     // bin(c) = clamp(fma(c, A, B), 0, 255): 256 bins over [lo, hi]
  float bthr;         // collect when fma(c, A, B) >= bthr (the boundary bin or above)
  int bstar, above;   // boundary bin, count strictly above it
  int cnt;            // entries in the row's buffer
  float thr;          // admission bound (k-th kept), -inf while unbounded
  int thrkey;         // key id of the k-th kept entry
  int over;           // candidates may not fit: collect block by block
  int pad[2];
};

constexpr int OFF_HIST = 0;
constexpr int OFF_ROW = OFF_HIST + ROWS * HIST_STRIDE;
constexpr int OFF_FLAG = OFF_ROW + ROWS * (int)sizeof(RowState);
constexpr int OFF_QL = (OFF_FLAG + 16 + 15) & ~15;  // Q_L B operands: [tl][ks][hi, lo][lane] x 16 B
constexpr int OFF_UNION = OFF_QL + TL * 2 * 2 * 64 * 16;
constexpr int VALUES_BYTES = NW * VT_BYTES;  // phase V staging (the merge area aliases it)
static_assert(NW * ROWS * MERGE_STRIDE * 4 <= VALUES_BYTES, "merge area fits in the staging");
static_assert(BITMAP_MAX_N / 8 <= HIST_STRIDE && LIST_MAX * 8 <= HIST_STRIDE, "row space");
static_assert((SPARE_BIN + 1) * 4 <= HIST_STRIDE, "the spare counter sits in the row's pad");

struct Args {
  const float* ql;
  const uint16_t* K;
  const uint16_t* V;
  int32_t* idx;
  float* vl;
  int BH, N, m, k, cap, tiles;
};

__host__ __device__ constexpr size_t lds_bytes(int cap) {
  return (size_t)OFF_UNION + ((size_t)ROWS * cap * 8 > (size_t)VALUES_BYTES
                                  ? (size_t)ROWS * cap * 8
                                  : (size_t)VALUES_BYTES);
}

// A operands of one 64-key block: lane (g, c16) holds key 16kt + c16,
// channels 8g.. (k-step 0) and 32 + 8g.. (k-step 1).  Keys past N read zeros
// (their scores are masked).
struct KRegs {
  u32x4 a[4][2];
};

__device__ __forceinline__ void load_k(KRegs& kr, Rsrc Kh, int blk, int N, int g, int c16) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = blk * KB + 16 * kt + c16;
    const int off = key < N ? key * 128 + 16 * g : PAST;
    kr.a[kt][0] = ld16(Kh, off);
    kr.a[kt][1] = ld16(Kh, off + 64);
  }
}

// V block for the transposed LDS copy: lane holds keys 4p..4p+3 of chunk c
// (8 channels) for items it = lane, lane + 64 (p = it >> 3, c = it & 7).
// Keys past N read zeros (their weights are 0).
struct VRegs {
  u32x4 v[2][4];
};

__device__ __forceinline__ void load_v(VRegs& vr, Rsrc Vh, int blk, int N, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int it = lane + 64 * j, p = it >> 3, c = it & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = blk * KB + 4 * p + i;
      vr.v[j][i] = ld16(Vh, key < N ? key * 128 + 16 * c : PAST);
    }
  }
}

// V^T (f16) into the wave's slot: row = channel, 64 keys per row.
__device__ __forceinline__ void store_vt(const VRegs& vr, char* vt, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int it = lane + 64 * j, p = it >> 3, c = it & 7;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f[i] = bf16_bits_to_f32((vr.v[j][i][t >> 1] >> (16 * (t & 1))) & 0xFFFFu);
      *reinterpret_cast<u32x2*>(vt + (8 * c + t) * VT_STRIDE + 8 * p) =
          u32x2{pk_f16(f[0], f[1]), pk_f16(f[2], f[3])};
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
    bqh[ks] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    bql[ks] = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
  }
}

// This lane's Q_L B operands of tile tl, kept in LDS (each lane its own
// 16-byte slots) rather than in registers across the passes.
__device__ __forceinline__ void ql_slot_store(char* sm, int tl, int lane, const u32x4 (&bqh)[2],
                                              const u32x4 (&bql)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    *reinterpret_cast<u32x4*>(sm + OFF_QL + (((tl * 2 + ks) * 2 + 0) * 64 + lane) * 16) = bqh[ks];
    *reinterpret_cast<u32x4*>(sm + OFF_QL + (((tl * 2 + ks) * 2 + 1) * 64 + lane) * 16) = bql[ks];
  }
}

// This lane's Q_L B operands of both tiles, read back from its LDS slots into
// registers for the length of one pass.
struct QLRegs {
  u32x4 h[TL][2], l[TL][2];
};
__device__ __forceinline__ void ql_load(QLRegs& q, const char* sm, int lane) {
#pragma unroll
  for (int tl = 0; tl < TL; ++tl)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      q.h[tl][ks] = *reinterpret_cast<const u32x4*>(sm + OFF_QL + (((tl * 2 + ks) * 2 + 0) * 64 + lane) * 16);
      q.l[tl][ks] = *reinterpret_cast<const u32x4*>(sm + OFF_QL + (((tl * 2 + ks) * 2 + 1) * 64 + lane) * 16);
    }
}

// Raw scores of one block: lane holds key 64blk + 16kt + 4g + r of row c16.
// Every phase computes them with this same sequence, so a score is
// bit-identical wherever it is recomputed.
__device__ __forceinline__ void block_scores(const KRegs& kr, const QLRegs& q, int tl,
                                             float (&s)[4][4]) {
  const u32x4 (&bqh)[2] = q.h[tl];
  const u32x4 (&bql)[2] = q.l[tl];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4 c = zero4();
    c = mfma_bf16(kr.a[kt][0], bqh[0], c);
    c = mfma_bf16(kr.a[kt][0], bql[0], c);
    c = mfma_bf16(kr.a[kt][1], bqh[1], c);
    c = mfma_bf16(kr.a[kt][1], bql[1], c);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[kt][r] = c[r];
  }
}

__device__ __forceinline__ int key_of(int blk, int kt, int g, int r) {
  return blk * KB + 16 * kt + 4 * g + r;
}

__device__ __forceinline__ int bin_of(float c, float A, float B) {
  return (int)__builtin_amdgcn_fmed3f(__builtin_fmaf(c, A, B), 0.f, 255.f);
}

// Candidate order: larger score first, ties to the lower key id.
__device__ __forceinline__ bool better(float va, int ka, float vb, int kb) {
  return va > vb || (va == vb && ka < kb);
}

// Number of the n entries at `list` (interleaved score, key) that rank
// before (v, key).  The 16 lanes of a group read the same entries.
__device__ __forceinline__ int rank_in_list(const float* list, int n, float v, int key) {
  int r = 0;
  int j = 0;
  for (; j + 2 <= n; j += 2) {
    const float4 e = *reinterpret_cast<const float4*>(list + 2 * j);
    r += better(e.x, __float_as_int(e.y), v, key) + better(e.z, __float_as_int(e.w), v, key);
  }
  if (j < n) r += better(list[2 * j], __float_as_int(list[2 * j + 1]), v, key);
  return r;
}

// Same over the row's buffer (separate score and key arrays).
__device__ __forceinline__ int rank_in(const float* vals, const int* keys, int n, float v,
                                       int key) {
  int r = 0;
  int j = 0;
  for (; j + 4 <= n; j += 4) {
    const float4 vv = *reinterpret_cast<const float4*>(vals + j);
    const int4 kk = *reinterpret_cast<const int4*>(keys + j);
    r += better(vv.x, kk.x, v, key) + better(vv.y, kk.y, v, key) + better(vv.z, kk.z, v, key) +
         better(vv.w, kk.w, v, key);
  }
  for (; j < n; ++j) r += better(vals[j], keys[j], v, key);
  return r;
}

__device__ __forceinline__ void group_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cuts row lr's buffer back to its exact k best (kept in buffer order) and
// sets the admission bound to the k-th of them.  Lane t of the group takes
// entries t, t + 16, ...
__device__ void row_cut(char* sm, const Args& a, int lr, bool work, int t, int g) {
  RowState* rs = reinterpret_cast<RowState*>(sm + OFF_ROW) + lr;
  float* vals = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)lr * a.cap * 8);
  int* keys = reinterpret_cast<int*>(vals + a.cap);
  const int cnt = work ? rs->cnt : 0;
  uint32_t keep = 0u;
  float tv = -INFINITY;
  int tk = 0;
  for (int u = 0; 16 * u < cnt; ++u) {
    const int e = t + 16 * u;
    if (e < cnt) {
      const float v = vals[e];
      const int key = keys[e];
      const int r = rank_in(vals, keys, cnt, v, key);
      keep |= (r < a.k ? 1u : 0u) << u;
      if (r == a.k - 1) {
        tv = v;
        tk = key + 1;
      }
    }
  }
  // exactly one lane holds the k-th kept entry
  tv = g16_maxf(tv);
  tk = g16_addi(tk) - 1;
  group_sync();
  // stable in-place filter, 16 entries at a time (writes land at or below
  // the entries read in the same step)
  const uint32_t below = (1u << t) - 1u;
  int run = 0;
  for (int u = 0; 16 * u < cnt; ++u) {
    const int e = t + 16 * u;
    const bool kp = e < cnt && (keep >> u & 1u);
    const float v = kp ? vals[e] : 0.f;
    const int key = kp ? keys[e] : 0;
    const uint32_t gm = g16_ballot(kp, g);
    group_sync();
    if (kp) {
      vals[run + __popc(gm & below)] = v;
      keys[run + __popc(gm & below)] = key;
    }
    run += __popc(gm);
  }
  if (work && t == 0) {
    rs->cnt = run;
    rs->thr = tv;
    rs->thrkey = tk;
  }
}

// Row lr's k best of its buffer, written ascending to `out`.
__device__ void row_final(char* sm, const Args& a, int lr, bool work, int t, int g,
                          int32_t* out) {
  RowState* rs = reinterpret_cast<RowState*>(sm + OFF_ROW) + lr;
  float* vals = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)lr * a.cap * 8);
  int* keys = reinterpret_cast<int*>(vals + a.cap);
  float* list = reinterpret_cast<float*>(sm + OFF_HIST + lr * HIST_STRIDE);
  const int cnt = work ? rs->cnt : 0;
  const float A = rs->A, B = rs->B;
  const int bstar = rs->bstar, above = rs->above;
  // entries above the boundary bin are in; the boundary bin's are ranked
  // among themselves, in a compact list when it fits
  const float upthr = bstar < 255 ? (float)(bstar + 1) : INFINITY;
  const int nb = cnt - above;
  const bool listed = nb <= LIST_MAX;
  const uint32_t below = (1u << t) - 1u;
  uint32_t up = 0u;
  int run = 0;
  for (int u = 0; 16 * u < cnt; ++u) {
    const int e = t + 16 * u;
    bool inb = false;
    if (e < cnt) {
      const bool isup = __builtin_fmaf(vals[e], A, B) >= upthr;
      up |= (isup ? 1u : 0u) << u;
      inb = !isup;
    }
    const uint32_t gm = g16_ballot(inb, g);
    if (listed && inb) {
      const int pos = run + __popc(gm & below);
      list[2 * pos] = vals[e];
      list[2 * pos + 1] = __int_as_float(keys[e]);
    }
    run += __popc(gm);
  }
  group_sync();
  uint32_t take = up;
  const int need = a.k - above;
  const int nw = (a.N + 31) >> 5;
  // a short list is ranked entry by entry (lane t: entries t and t + 16) and
  // its winners' keys kept in registers for the bitmap and their slots;
  // otherwise every buffer entry outside `up` is ranked where it sits
  const bool short_list = listed && nb <= 32 && a.N <= BITMAP_MAX_N && nw * 6 <= HIST_STRIDE;
  int win[2] = {-1, -1};
  if (short_list) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = t + 16 * j;
      if (i < nb) {
        const float v = list[2 * i];
        const int key = __float_as_int(list[2 * i + 1]);
        if (rank_in_list(list, nb, v, key) < need) win[j] = key;
      }
    }
  } else {
    for (int u = 0; 16 * u < cnt; ++u) {
      const int e = t + 16 * u;
      if (e < cnt && !(up >> u & 1u)) {
        const float v = vals[e];
        const int key = keys[e];
        const int r = listed ? rank_in_list(list, nb, v, key) : rank_in(vals, keys, cnt, v, key) - above;
        take |= (r < need ? 1u : 0u) << u;
      }
    }
  }
  group_sync();
  if (a.N <= BITMAP_MAX_N) {
    // bitmap of the taken keys in the row's histogram space; slot = number of
    // taken keys below
    uint32_t* bm = reinterpret_cast<uint32_t*>(list);
    for (int q = t; q < nw; q += 16) bm[q] = 0u;
    group_sync();
    for (int u = 0; 16 * u < cnt; ++u) {
      const int e = t + 16 * u;
      if (e < cnt && (take >> u & 1u)) atomicOr(&bm[keys[e] >> 5], 1u << (keys[e] & 31));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (win[j] >= 0) atomicOr(&bm[win[j] >> 5], 1u << (win[j] & 31));
    group_sync();
    if (nw * 6 <= HIST_STRIDE) {
      // taken keys before each bitmap word (16-bit, after the bitmap), lane t
      // taking words t, t + 16, ...; then every taken entry writes its own
      // slot: the taken keys before its word plus those below it in the word
      uint16_t* wpre = reinterpret_cast<uint16_t*>(bm + nw);
      int run = 0;
      for (int r0 = 0; r0 < nw; r0 += 16) {
        const int q = r0 + t;
        const int c = q < nw ? __popc(bm[q]) : 0;
        const int tot = g16_addi(c);
        if (q < nw) wpre[q] = (uint16_t)(run + tot - g16_suffix(c));
        run += tot;
      }
      group_sync();
      if (work) {
        auto emit = [&](int key) {
          const int wq = key >> 5;
          const int pos = wpre[wq] + __popc(bm[wq] & ((1u << (key & 31)) - 1u));
          if (pos < a.k) out[pos] = key;
        };
        for (int u = 0; 16 * u < cnt; ++u) {
          const int e = t + 16 * u;
          if (e < cnt && (take >> u & 1u)) emit(keys[e]);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (win[j] >= 0) emit(win[j]);
      }
    } else {
      const int wpl = (nw + 15) >> 4;
      const int q0 = t * wpl, q1 = min(nw, q0 + wpl);
      int mine = 0;
      for (int q = q0; q < q1; ++q) mine += __popc(bm[q]);
      int pos = g16_addi(mine) - g16_suffix(mine);
      if (work) {
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
  } else {
    // slot = number of taken keys below, counted over the buffer with the
    // untaken keys replaced by INT_MAX (the scores are no longer needed)
    int* tkeys = reinterpret_cast<int*>(vals);
    for (int u = 0; 16 * u < cnt; ++u) {
      const int e = t + 16 * u;
      if (e < cnt) tkeys[e] = (take >> u & 1u) ? keys[e] : 0x7FFFFFFF;
    }
    group_sync();
    for (int u0 = 0; 16 * u0 < cnt; u0 += 4) {
      int kq[4], pos[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = t + 16 * (u0 + i);
        kq[i] = (e < cnt && (take >> (u0 + i) & 1u)) ? tkeys[e] : -1;
      }
      int j = 0;
      for (; j + 4 <= cnt; j += 4) {
        const int4 kk = *reinterpret_cast<const int4*>(tkeys + j);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pos[i] += (kk.x < kq[i]) + (kk.y < kq[i]) + (kk.z < kq[i]) + (kk.w < kq[i]);
      }
      for (; j < cnt; ++j) {
        const int kj = tkeys[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) pos[i] += kj < kq[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (work && kq[i] >= 0) out[pos[i]] = kq[i];
    }
  }
}

__global__ __launch_bounds__(64 * NW) void landmark_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // round-robin dispatch puts workgroup b on XCD b % 8: keep a head's
  // workgroups on one XCD so its K and V stay in that XCD's L2
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int bh = xcd + 8 * (slot / a.tiles), row0 = (slot % a.tiles) * ROWS;
  if (bh >= a.BH) return;
  const int N = a.N, nblk = (N + KB - 1) / KB;
  const bool ragged = (N % KB) != 0;  // the last block has keys past N
  const Rsrc Kh = head_rows(a.K + (size_t)bh * N * 64, N);
  const Rsrc Vh = head_rows(a.V + (size_t)bh * N * 64, N);
  RowState* rows = reinterpret_cast<RowState*>(sm + OFF_ROW);
  int* flag = reinterpret_cast<int*>(sm + OFF_FLAG);

  for (int i = tid; i < ROWS * HIST_STRIDE / 16; i += 64 * NW)
    reinterpret_cast<u32x4*>(sm + OFF_HIST)[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) flag[0] = 0;

  // this lane's rows: 16 * tl + c16 of the workgroup's rows (column c16 of
  // tile tl of S^T)
  // (every wave writes the same values into the same slots)
#pragma unroll
  for (int tl = 0; tl < TL; ++tl) {
    u32x4 bqh[2], bql[2];
    load_ql_b(a.ql, bh, a.m, row0 + 16 * tl + c16, g, bqh, bql);
    ql_slot_store(sm, tl, lane, bqh, bql);
  }

  // each pass's first K block is requested before the previous pass's tail
  // (merge, bin search), so that its latency hides behind that work
  KRegs kpre;
  // ------------------------------------------------------------ V: values
  {
    char* vt = sm + OFF_UNION + w * VT_BYTES;
    float mref[TL], mn[TL], mx[TL];
    f32x4 accv[TL][4], lsum[TL];
#pragma unroll
    for (int tl = 0; tl < TL; ++tl) {
      mref[tl] = -INFINITY;
      mn[tl] = INFINITY;
      mx[tl] = -INFINITY;
      lsum[tl] = zero4();
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) accv[tl][ct] = zero4();
    }
    const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    QLRegs qlr;
    ql_load(qlr, sm, lane);  // (this lane's own slots: no barrier needed)
    KRegs kr;
    VRegs vr;
    if (w < nblk) {
      load_k(kr, Kh, w, N, g, c16);
      load_v(vr, Vh, w, N, lane);
    }
    for (int blk = w; blk < nblk; blk += NW) {
      // the V registers are free once stored and the K registers once the
      // scores are out: the next block's loads go out right after each
      store_vt(vr, vt, lane);
      if (blk + NW < nblk) load_v(vr, Vh, blk + NW, N, lane);
      group_sync();
      // the block's V^T A operands, shared by both row tiles:
      // V^T[channel 16ct + c16][keys 32sp + 4g .., 32sp + 16 + 4g ..]
      u32x4 av[4][2];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const char* vrow = vt + (16 * ct + c16) * VT_STRIDE;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vrow + (32 * sp + 4 * g) * 2);
          const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vrow + (32 * sp + 16 + 4 * g) * 2);
          av[ct][sp] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        }
      }
      const bool last = ragged && blk == nblk - 1;
      // one tile at a time keeps one tile's scores and weights live
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        float s[4][4];
        block_scores(kr, qlr, tl, s);
        if (tl == TL - 1 && blk + NW < nblk) load_k(kr, Kh, blk + NW, N, g, c16);
        if (last) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool ok = key_of(blk, kt, g, r) < N;
              if (ok) mn[tl] = fminf(mn[tl], s[kt][r]);
              if (!ok) s[kt][r] = -INFINITY;
            }
        } else {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) mn[tl] = fminf(mn[tl], s[kt][r]);
        }
        float bmax = s[0][0];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) bmax = fmaxf(bmax, s[kt][r]);
        mx[tl] = fmaxf(mx[tl], bmax);
        // raise the reference maximum only when some weight would exceed 2^8
        const bool raise = (bmax - mref[tl]) * kTauLog2e > kSlack;
        if (__ballot(raise) != 0) {
          float m2 = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
          m2 = fmaxf(m2, __shfl_xor(m2, 32, 64));
          const float mnew = fmaxf(mref[tl], m2);
          const float alpha = __builtin_amdgcn_exp2f((mref[tl] - mnew) * kTauLog2e);
          mref[tl] = mnew;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) accv[tl][ct] = accv[tl][ct] * alpha;
          lsum[tl] = lsum[tl] * alpha;
        }
        const float moff = -mref[tl] * kTauLog2e;
        u32x4 bp[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          float p[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * sp][r], kTauLog2e, moff));
            p[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * sp + 1][r], kTauLog2e, moff));
          }
          bp[sp] = u32x4{pk_f16(p[0], p[1]), pk_f16(p[2], p[3]), pk_f16(p[4], p[5]),
                         pk_f16(p[6], p[7])};
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          f32x4 acc = accv[tl][ct];
#pragma unroll
          for (int sp = 0; sp < 2; ++sp) acc = mfma_f16(av[ct][sp], bp[sp], acc);
          accv[tl][ct] = acc;
        }
        lsum[tl] = mfma_f16(ones, bp[0], lsum[tl]);
        lsum[tl] = mfma_f16(ones, bp[1], lsum[tl]);
      }
      group_sync();
    }
#pragma unroll
    for (int tl = 0; tl < TL; ++tl) {
      mn[tl] = fminf(mn[tl], __shfl_xor(mn[tl], 16, 64));
      mn[tl] = fminf(mn[tl], __shfl_xor(mn[tl], 32, 64));
      mx[tl] = fmaxf(mx[tl], __shfl_xor(mx[tl], 16, 64));
      mx[tl] = fmaxf(mx[tl], __shfl_xor(mx[tl], 32, 64));
    }
    __syncthreads();  // every wave is done with its staging slot
    // partials: acc[tl][ct][r] = V_L^T[channel 16ct + 4g + r][row 16tl + c16],
    // relative to exp2((c - mref) tau log2e); mref <= the true maximum mx
#pragma unroll
    for (int tl = 0; tl < TL; ++tl) {
      float* part =
          reinterpret_cast<float*>(sm + OFF_UNION) + (w * ROWS + 16 * tl + c16) * MERGE_STRIDE;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        *reinterpret_cast<float4*>(part + 16 * ct + 4 * g) =
            make_float4(accv[tl][ct][0], accv[tl][ct][1], accv[tl][ct][2], accv[tl][ct][3]);
      if (g == 0) {
        part[64] = mref[tl];
        part[65] = lsum[tl][0];
        part[66] = mn[tl];
        part[67] = mx[tl];
      }
    }
    if (w < nblk) load_k(kpre, Kh, w, N, g, c16);
    __syncthreads();
    // merge: thread -> (row, 4 channels), ROWS * 16 items
    const float* base = reinterpret_cast<const float*>(sm + OFF_UNION);
    for (int it = tid; it < ROWS * 16; it += 64 * NW) {
      const int r = it >> 4, c4 = (it & 15) * 4;
      float M = -INFINITY, lo = INFINITY, hi = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* pw = base + (ww * ROWS + r) * MERGE_STRIDE;
        M = fmaxf(M, pw[64]);
        lo = fminf(lo, pw[66]);
        hi = fmaxf(hi, pw[67]);
      }
      float L = 0.f;
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* pw = base + (ww * ROWS + r) * MERGE_STRIDE;
        const float mw = pw[64];
        const float f = mw > -INFINITY ? __builtin_amdgcn_exp2f((mw - M) * kTauLog2e) : 0.f;
        L += f * pw[65];
        const float4 v = *reinterpret_cast<const float4*>(pw + c4);
        o.x += f * v.x;
        o.y += f * v.y;
        o.z += f * v.z;
        o.w += f * v.w;
      }
      if (row0 + r < a.m) {
        const float inv = 1.0f / L;
        *reinterpret_cast<float4*>(a.vl + ((size_t)bh * a.m + row0 + r) * 64 + c4) =
            make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      }
      if (c4 == 0) {
        // capped so that fma(c, A, B) stays finite
        const float A = hi > lo ? fminf(256.0f / (hi - lo), 1e30f) : 0.f;
        rows[r].lo = lo;
        rows[r].A = A;
        rows[r].B = -lo * A;
      }
    }
    __syncthreads();
  }
  float A[TL], B[TL];
#pragma unroll
  for (int tl = 0; tl < TL; ++tl) {
    A[tl] = rows[16 * tl + c16].A;
    B[tl] = rows[16 * tl + c16].B;
  }

  // ------------------------------------------------------------ H: histogram
  {
    QLRegs qlr;
    ql_load(qlr, sm, lane);
    KRegs kr = kpre;
    for (int blk = w; blk < nblk; blk += NW) {
      // keys past N of a ragged last block count into the spare word past
      // the 256 bins (no branch per score)
      uint32_t spare = 0u;
      if (ragged && blk == nblk - 1) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) spare |= (key_of(blk, kt, g, r) < N ? 0u : 1u) << (4 * kt + r);
      }
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        float s[4][4];
        block_scores(kr, qlr, tl, s);
        if (tl == TL - 1 && blk + NW < nblk) load_k(kr, Kh, blk + NW, N, g, c16);
        uint32_t* myhist =
            reinterpret_cast<uint32_t*>(sm + OFF_HIST + (16 * tl + c16) * HIST_STRIDE);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int bin = bin_of(s[kt][r], A[tl], B[tl]);
            atomicAdd(myhist + ((spare >> (4 * kt + r) & 1u) ? SPARE_BIN : bin), 1u);
          }
      }
    }
  }
  if (w < nblk) load_k(kpre, Kh, w, N, g, c16);
  __syncthreads();
  // the bin holding each row's k-th best: group g of wave w takes rows
  // 4w + g + 16i
#pragma unroll
  for (int i = 0; i < TL; ++i) {
    const int r = 4 * w + g + 16 * i;
    const uint32_t* hrow = reinterpret_cast<const uint32_t*>(sm + OFF_HIST + r * HIST_STRIDE);
    uint32_t cb[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 d = *reinterpret_cast<const u32x4*>(hrow + 16 * c16 + 4 * q);
      cb[4 * q] = d[0];
      cb[4 * q + 1] = d[1];
      cb[4 * q + 2] = d[2];
      cb[4 * q + 3] = d[3];
    }
    int local = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) local += (int)cb[q];
    const int suf = g16_suffix(local);
    const int above_lane = suf - local;
    const int need = a.k;
    const bool mine = above_lane < need && need <= suf;
    int bstar = 0, above = 0, inbin = 0;
    if (mine) {
      int acc = above_lane;
      bool found = false;
#pragma unroll
      for (int q = 15; q >= 0; --q) {
        const int cq = (int)cb[q];
        if (!found) {
          if (acc + cq >= need) {
            found = true;
            bstar = 16 * c16 + q;
            above = acc;
            inbin = cq;
          } else {
            acc += cq;
          }
        }
      }
    }
    bstar = g16_addi(mine ? bstar : 0);
    above = g16_addi(mine ? above : 0);
    inbin = g16_addi(mine ? inbin : 0);
    if (c16 == 0) {
      const bool real = row0 + r < a.m;
      const bool over = real && above + inbin > a.cap;
      rows[r].bstar = bstar;
      rows[r].above = above;
      // padding rows collect nothing
      rows[r].bthr = !real ? INFINITY : (bstar == 0 ? -INFINITY : (float)bstar);
      rows[r].cnt = 0;
      rows[r].thr = -INFINITY;
      rows[r].thrkey = 0x7FFFFFFF;
      rows[r].over = over ? 1 : 0;
      if (over) atomicOr(flag, 1);
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ C: collect
  {
    QLRegs qlr;
    ql_load(qlr, sm, lane);
    float bthr[TL];
#pragma unroll
    for (int tl = 0; tl < TL; ++tl) bthr[tl] = rows[16 * tl + c16].bthr;
    // appends the block's scores of tile tl that are in the boundary bin or
    // above (and, when bounded, beat the admission bound (thr, thrkey))
    // the bits (4kt + r) of this lane's keys of block blk that lie below N
    auto valid_bits = [&](int blk) {
      uint32_t vb = 0u;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) vb |= (key_of(blk, kt, g, r) < N ? 1u : 0u) << (4 * kt + r);
      return vb;
    };
    // appends the block's scores of tile tl that are in the boundary bin or
    // above (and, with BOUNDED, beat the admission bound (thr, thrkey));
    // `valid` masks the keys past N of a ragged last block
    auto collect = [&](auto bounded, const float (&s)[4][4], int tl, int blk, uint32_t valid,
                       float thr, int thrkey) {
      constexpr bool BOUNDED = decltype(bounded)::value;
      const int lr = 16 * tl + c16;
      uint32_t msk = 0u;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = s[kt][r];
          bool q = __builtin_fmaf(v, A[tl], B[tl]) >= bthr[tl];
          if constexpr (BOUNDED) {
            const int key = key_of(blk, kt, g, r);
            q = q && (v > thr || (v == thr && key < thrkey));
          }
          msk |= (q ? 1u : 0u) << (4 * kt + r);
        }
      msk &= valid;
      if (__ballot(msk != 0u) == 0) return;
      // each lane reserves its own run of slots (the order of entries in a
      // row's buffer does not matter: they are ranked by score and key id)
      const int c = __popc(msk);
      int pos = 0;
      if (c > 0) pos = atomicAdd(&rows[lr].cnt, c);
      float* vals = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)lr * a.cap * 8);
      int* keys = reinterpret_cast<int*>(vals + a.cap);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (msk >> (4 * kt + r) & 1u) {
            vals[pos] = s[kt][r];
            keys[pos] = key_of(blk, kt, g, r);
            ++pos;
          }
    };
    if (flag[0] == 0) {
      // every row's candidates fit: one streaming pass
      KRegs kr = kpre;
      for (int blk = w; blk < nblk; blk += NW) {
        const uint32_t valid = ragged && blk == nblk - 1 ? valid_bits(blk) : 0xFFFFu;
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) {
          float s[4][4];
          block_scores(kr, qlr, tl, s);
          if (tl == TL - 1 && blk + NW < nblk) load_k(kr, Kh, blk + NW, N, g, c16);
          collect(std::false_type{}, s, tl, blk, valid, 0.f, 0);
        }
      }
    } else {
      // one block at a time (its owner wave appends, at most KB entries per
      // row); rows that could overflow on the next block are cut back first
      for (int blk = 0; blk < nblk; ++blk) {
        if (blk % NW == w) {
          const uint32_t valid = ragged && blk == nblk - 1 ? valid_bits(blk) : 0xFFFFu;
          KRegs kr;
          load_k(kr, Kh, blk, N, g, c16);
#pragma unroll
          for (int tl = 0; tl < TL; ++tl) {
            float s[4][4];
            block_scores(kr, qlr, tl, s);
            const int lr = 16 * tl + c16;
            collect(std::true_type{}, s, tl, blk, valid, rows[lr].thr, rows[lr].thrkey);
          }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TL; ++i) {
          const int r = 4 * w + g + 16 * i;
          const bool work = row0 + r < a.m && rows[r].over && rows[r].cnt > a.cap - KB;
          if (__ballot(work) != 0) row_cut(sm, a, r, work, c16, g);
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ F: final
#pragma unroll 1
  for (int i = 0; i < TL; ++i) {
    const int r = 4 * w + g + 16 * i;
    const bool work = row0 + r < a.m;
    int32_t* out = a.idx + ((size_t)bh * a.m + (work ? row0 + r : 0)) * a.k;
    row_final(sm, a, r, work, c16, g, out);
  }
}

}  // namespace lmk

// The row buffer holds k plus one block of candidates (k + 64 entries, at
// most 512: one bit each in the selection masks).
static int landmark_cap(const Shape& s) {
  const int cap = (s.k + lmk::KB + 15) & ~15;
  return cap <= 512 ? cap : 0;
}

bool landmark_bf16_supported(const Shape& s) {
  return s.bf16 && landmark_cap(s) > 0 && lmk::lds_bytes(landmark_cap(s)) <= 160 * 1024;
}

hipError_t launch_landmark_bf16(const float* ql, const void* K, const void* V, int32_t* idx,
                                float* vl, const Shape& s, hipStream_t st) {
  lmk::Args a{ql, (const uint16_t*)K, (const uint16_t*)V, idx, vl, s.BH, s.N, s.m, s.k,
              landmark_cap(s), (s.m + lmk::ROWS - 1) / lmk::ROWS};
  if (a.cap == 0) return hipErrorInvalidValue;
  const size_t lds = lmk::lds_bytes(a.cap);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)lmk::landmark_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  const int grid = ((s.BH + 7) / 8) * 8 * a.tiles;
  lmk::landmark_kernel<<<grid, 64 * lmk::NW, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace mita
