// Steps a2-a4 for bf16 inputs on long grids -- the landmark pass (page
// "NeurIPS'26：注意力也是FFN？...", landmark-query section: every landmark
// query scores all keys; its k best keys, ties to the lowest key id, form a
// routed expert; the same scores, softmax-normalised over all N keys, weight V
// into the landmark values V_L).
//
// One kernel.  A workgroup owns 32 landmark rows of one head (two 16-row MFMA
// tiles, so every K block loaded feeds both); its four waves (eight where the
// candidate buffers of a large k already leave one workgroup per CU) split
// the head's keys (wave w takes the 64-key blocks w, w+NW, ...).  Raw scores
// c = Q_L . K (the scale tau = 1/8 is a power of two, so it is folded into the
// softmax and bin constants without changing any order) run on bf16 MFMA
// with K rows loaded straight into the A operand and Q_L split hi + lo
// (fp32-accurate).  Phases, separated by workgroup barriers:
//   V  values: per wave, an online softmax of its keys' scores folded into
//      V_L^T = V^T P^T (f16 MFMA; the block's V rows staged as f16 in the
//      wave's own LDS slot and read back as V^T fragments by the transposing
//      LDS read; the running maximum is only raised when a score exceeds it by
//      more than 2^8 in weight, so most blocks skip the rescale); the four
//      partial results merge by log-sum-exp into V_L.  For k <= 128 the
//      same scores are counted into each row's 256-bin histogram as they
//      stream by, on bins fixed from the waves' first blocks (each wave
//      streams a contiguous quarter, so the samples spread over the keys);
//   H  (k > 128) histogram: the rows' exact score ranges from pass V fix the
//      bins, and the waves recompute their scores (K now in L2) to count
//      them; either way the bin holding the k-th best is found per row;
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
// once and are re-read from that XCD's L2 (with fewer than 8 heads they
// alternate over the XCDs, so that every XCD has work).
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

#include <type_traits>

namespace mita {
namespace lmk {

constexpr int KB = 64;                  // keys per block
constexpr int NW4 = 4;                  // waves per workgroup (8 where one workgroup fills a CU's LDS)
constexpr int TL = 2;                   // 16-row MFMA tiles per workgroup
constexpr int ROWS = 16 * TL;           // landmark rows per workgroup
constexpr int V_STRIDE = 64 * 2 + 16;  // bytes per staged V row: 64 f16 channels + pad
constexpr int VT_BYTES = KB * V_STRIDE;  // a wave's staging slot: one block's V rows
constexpr int HIST_STRIDE = 1040;       // one row's 256 32-bit bins + pad (rows 4 banks apart)
constexpr int SPARE_BIN = 256;          // pad word: counts the keys past N of a ragged block
constexpr int BITMAP_MAX_N = 8192;      // keys whose bitmap fits in a histogram row
constexpr int LIST_MAX = 128;           // boundary entries listed in a histogram row
constexpr int CHUNK_BLOCKS = 64;        // key blocks per chunk at most (4096 keys)
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
// The union holds phase V's staging (one VT_BYTES slot per wave; the merge
// area aliases it), then the rows' candidate buffers; the [wave][row]
// first-block (min, max) samples follow it.
__host__ __device__ constexpr int union_bytes(int cap, int nw) {
  return ROWS * cap * 8 > nw * VT_BYTES ? ROWS * cap * 8 : nw * VT_BYTES;
}
static_assert(ROWS * MERGE_STRIDE * 4 <= VT_BYTES, "a wave's merge area fits in its staging slot");
static_assert(BITMAP_MAX_N / 8 <= HIST_STRIDE && LIST_MAX * 8 <= HIST_STRIDE, "row space");
// a chunk's key bitmap, padded to whole 16-byte groups, and its 16-bit word
// prefixes share one row's space
static_assert(6 * ((CHUNK_BLOCKS * KB / 32 + 3) & ~3) <= HIST_STRIDE, "bitmap and prefixes fit a row");
static_assert((SPARE_BIN + 1) * 4 <= HIST_STRIDE, "the spare counter sits in the row's pad");

struct Args {
  const float* ql;
  const uint16_t* K;
  const uint16_t* V;
  int32_t* idx;
  float* vl;
  int BH, N, m, k, cap, tiles;
  // keys split into nch chunks of cblk blocks (nch > 1: each workgroup writes
  // its chunk's top-k as (score, key) pairs and its unnormalised V_L partial,
  // and merge_kernel or merge_row_kernel finishes both)
  int nch, cblk;
  // 1: the histogram is built during the values pass on bins fixed from
  // each wave's first block; 0: a third pass builds it on the exact range
  int fuse_h;
  float* cand_s;   // [BH][m][nch][k] scores of each chunk's top-k
  int32_t* cand_k; // [BH][m][nch][k] their key ids, ascending within a chunk
  float* vlpart;   // [BH][m][nch][PART_STRIDE]: 64 sums, reference max, sum
  // optional [BH][m]: each row's softmax statistics over all N keys, x = the
  // reference maximum tau * c_max and y = the sum of exp(tau c - x) (the
  // backward pass reuses them)
  float4* stats;
};

constexpr int PART_STRIDE = 68;

// This workgroup's keys: blocks [blk0, blk1), keys [kbase, kend); it selects
// kk = min(k, kend - kbase) of them.
struct Chunk {
  int chunk, blk0, blk1, kbase, kend, kk;
};

__host__ __device__ constexpr size_t lds_bytes(int cap, int nw) {
  return (size_t)OFF_UNION + (size_t)union_bytes(cap, nw) + (size_t)nw * ROWS * 8;
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

// V block for the wave's LDS staging: lane holds keys 4p..4p+3 of chunk c
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

// The block's V rows (f16) into the wave's slot: row = key, chunk c of a
// key as one 16-byte store.  (The products read V^T fragments from them with
// the transposing LDS read.)
__device__ __forceinline__ void store_v(const VRegs& vr, char* vt, int lane) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int it = lane + 64 * j, p = it >> 3, c = it & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 x = vr.v[j][i];
      u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f[q] = pk_f16(__uint_as_float(x[q] << 16), __uint_as_float(x[q] & 0xFFFF0000u));
      *reinterpret_cast<u32x4*>(vt + (4 * p + i) * V_STRIDE + 16 * c) = f;
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

// Number of the n entries at `list` (interleaved score, key: a row's
// candidate buffer or boundary list) that rank before (v, key).  The 16 lanes
// of a group read the same entries.
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

__device__ __forceinline__ void group_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cuts row lr's buffer back to its exact k best (kept in buffer order) and
// sets the admission bound to the k-th of them.  Lane t of the group takes
// entries t, t + 16, ...
__device__ void row_cut(char* sm, const Args& a, int kk, int lr, bool work, int t, int g) {
  RowState* rs = reinterpret_cast<RowState*>(sm + OFF_ROW) + lr;
  float* buf = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)lr * a.cap * 8);  // (score, key)
  const int cnt = work ? rs->cnt : 0;
  uint32_t keep = 0u;
  float tv = -INFINITY;
  int tk = 0;
  for (int u = 0; 16 * u < cnt; ++u) {
    const int e = t + 16 * u;
    if (e < cnt) {
      const float2 ev = *reinterpret_cast<const float2*>(buf + 2 * e);
      const float v = ev.x;
      const int key = __float_as_int(ev.y);
      const int r = rank_in_list(buf, cnt, v, key);
      keep |= (r < kk ? 1u : 0u) << u;
      if (r == kk - 1) {
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
    const float2 ev = kp ? *reinterpret_cast<const float2*>(buf + 2 * e) : make_float2(0.f, 0.f);
    const uint32_t gm = g16_ballot(kp, g);
    group_sync();
    if (kp) *reinterpret_cast<float2*>(buf + 2 * (run + __popc(gm & below))) = ev;
    run += __popc(gm);
  }
  if (work && t == 0) {
    rs->cnt = run;
    rs->thr = tv;
    rs->thrkey = tk;
  }
}

// Rows lr[j]'s kk best of their buffers, each written ascending by key id to
// out[j], and (when outs[j] is not null) their scores beside them.  The
// chunk's keys have a bitmap of (kend - kbase) bits in each row's histogram
// space.  The R rows of a lane group go through every step together, so that
// one group barrier serves them all and their LDS round trips overlap.
template <int R>
__device__ void rows_final(char* sm, const Args& a, const Chunk& ch, const int (&lr)[R],
                           const bool (&work)[R], int t, int g, int32_t* const (&out)[R],
                           float* const (&outs)[R]) {
  float* buf[R];   // (score, key) pairs
  float* list[R];
  int cnt[R], bstar[R], above[R], nb[R], need[R];
  float A[R], B[R], upthr[R];
  bool listed[R], short_list[R];
  const int nw = (ch.kend - ch.kbase + 31) >> 5;
  int cmax = 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const RowState* rs = reinterpret_cast<const RowState*>(sm + OFF_ROW) + lr[j];
    buf[j] = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)lr[j] * a.cap * 8);
    list[j] = reinterpret_cast<float*>(sm + OFF_HIST + lr[j] * HIST_STRIDE);
    cnt[j] = work[j] ? rs->cnt : 0;
    A[j] = rs->A;
    B[j] = rs->B;
    bstar[j] = rs->bstar;
    above[j] = rs->above;
    // entries above the boundary bin are in; the boundary bin's are ranked
    // among themselves, in a compact list when it fits
    upthr[j] = bstar[j] < 255 ? (float)(bstar[j] + 1) : INFINITY;
    nb[j] = cnt[j] - above[j];
    listed[j] = nb[j] <= LIST_MAX;
    need[j] = ch.kk - above[j];
    // a short list is ranked entry by entry (lane t: entries t and t + 16)
    // and its winners' keys kept in registers for the bitmap and their
    // slots; otherwise every buffer entry outside `up` is ranked where it sits
    short_list[j] = listed[j] && nb[j] <= 32 && nw * 6 <= HIST_STRIDE;
    cmax = max(cmax, cnt[j]);
  }
  const uint32_t below = (1u << t) - 1u;
  uint32_t up[R], take[R];
  int run[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    up[j] = 0u;
    run[j] = 0;
  }
  for (int u = 0; 16 * u < cmax; ++u) {
    const int e = t + 16 * u;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      bool inb = false;
      float2 ev = make_float2(0.f, 0.f);
      if (e < cnt[j]) {
        ev = *reinterpret_cast<const float2*>(buf[j] + 2 * e);
        const bool isup = __builtin_fmaf(ev.x, A[j], B[j]) >= upthr[j];
        up[j] |= (isup ? 1u : 0u) << u;
        inb = !isup;
      }
      const uint32_t gm = g16_ballot(inb, g);
      if (listed[j] && inb) *reinterpret_cast<float2*>(list[j] + 2 * (run[j] + __popc(gm & below))) = ev;
      run[j] += __popc(gm);
    }
  }
  group_sync();
  int win[R][2];
  float winv[R][2];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    take[j] = up[j];
    win[j][0] = win[j][1] = -1;
    winv[j][0] = winv[j][1] = 0.f;
    if (short_list[j]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = t + 16 * h;
        if (i < nb[j]) {
          const float v = list[j][2 * i];
          const int key = __float_as_int(list[j][2 * i + 1]);
          if (rank_in_list(list[j], nb[j], v, key) < need[j]) {
            win[j][h] = key;
            winv[j][h] = v;
          }
        }
      }
    } else {
      for (int u = 0; 16 * u < cnt[j]; ++u) {
        const int e = t + 16 * u;
        if (e < cnt[j] && !(up[j] >> u & 1u)) {
          const float2 ev = *reinterpret_cast<const float2*>(buf[j] + 2 * e);
          const float v = ev.x;
          const int key = __float_as_int(ev.y);
          const int r = listed[j] ? rank_in_list(list[j], nb[j], v, key)
                                  : rank_in_list(buf[j], cnt[j], v, key) - above[j];
          take[j] |= (r < need[j] ? 1u : 0u) << u;
        }
      }
    }
  }
  group_sync();
  // bitmap of the taken keys (relative to the chunk's first key) in each
  // row's histogram space; slot = number of taken keys below (lane t clears
  // and scans four words at a time: nw4 16-byte groups, the words past nw in
  // the last group staying zero)
  const int kb = ch.kbase;
  const int nw4 = (nw + 3) >> 2;
  uint32_t* bm[R];
  uint16_t* wpre[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    bm[j] = reinterpret_cast<uint32_t*>(list[j]);
    // taken keys before each bitmap word (16-bit, after the bitmap's groups)
    wpre[j] = reinterpret_cast<uint16_t*>(bm[j] + 4 * nw4);
    for (int q4 = t; q4 < nw4; q4 += 16) reinterpret_cast<u32x4*>(bm[j])[q4] = u32x4{0u, 0u, 0u, 0u};
  }
  group_sync();
  for (int u = 0; 16 * u < cmax; ++u) {
    const int e = t + 16 * u;
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (e < cnt[j] && (take[j] >> u & 1u)) {
        const int key = __float_as_int(buf[j][2 * e + 1]);
        atomicOr(&bm[j][(key - kb) >> 5], 1u << ((key - kb) & 31));
      }
  }
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (win[j][h] >= 0) atomicOr(&bm[j][(win[j][h] - kb) >> 5], 1u << ((win[j][h] - kb) & 31));
  group_sync();
  // lane t takes word groups t, t + 16, ...; then every taken entry writes
  // its own slot: the taken keys before its word plus those below it in the
  // word
#pragma unroll
  for (int j = 0; j < R; ++j) run[j] = 0;
  for (int r0 = 0; r0 < nw4; r0 += 16) {
    const int q4 = r0 + t;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const u32x4 wv = q4 < nw4 ? reinterpret_cast<const u32x4*>(bm[j])[q4] : u32x4{0u, 0u, 0u, 0u};
      const int c0 = __popc(wv[0]), c1 = __popc(wv[1]), c2 = __popc(wv[2]), c3 = __popc(wv[3]);
      const int c = c0 + c1 + c2 + c3;
      const int tot = g16_addi(c);
      const uint32_t p0 = (uint32_t)(run[j] + tot - g16_suffix(c));
      if (q4 < nw4)
        *reinterpret_cast<u32x2*>(wpre[j] + 4 * q4) =
            u32x2{p0 | (p0 + c0) << 16, (p0 + c0 + c1) | (p0 + c0 + c1 + c2) << 16};
      run[j] += tot;
    }
  }
  group_sync();
  auto emit = [&](int j, int key, float v) {
    const int wq = (key - kb) >> 5;
    const int pos = wpre[j][wq] + __popc(bm[j][wq] & ((1u << ((key - kb) & 31)) - 1u));
    if (pos < ch.kk) {
      out[j][pos] = key;
      if (outs[j]) outs[j][pos] = v;
    }
  };
  for (int u = 0; 16 * u < cmax; ++u) {
    const int e = t + 16 * u;
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (work[j] && e < cnt[j] && (take[j] >> u & 1u)) {
        const float2 ev = *reinterpret_cast<const float2*>(buf[j] + 2 * e);
        emit(j, __float_as_int(ev.y), ev.x);
      }
  }
#pragma unroll
  for (int j = 0; j < R; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (work[j] && win[j][h] >= 0) emit(j, win[j][h], winv[j][h]);
}

// FUSE (a.fuse_h): the histogram is built during pass V; a template
// parameter so that each form gets its own register allocation.
// NW: waves per workgroup (4, or 8 where one workgroup's LDS fills a CU
// anyway); the waves split the keys, and lane group g of wave w finishes
// rows 4w + g + 4 NW i (RPG of them).
template <bool FUSE, int NW>
__global__ __launch_bounds__(64 * NW) void landmark_kernel(Args a) {
  constexpr int RPG = ROWS / (4 * NW);
  static_assert(RPG * 4 * NW == ROWS, "rows split evenly over the lane groups");
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // round-robin dispatch puts workgroup b on XCD b % 8: keep a head's
  // workgroups on one XCD so its K and V stay in that XCD's L2; with fewer
  // than 8 heads a head's workgroups alternate over the XCDs instead, so
  // that every XCD has work
  const int b = blockIdx.x;
  const int per_head = a.tiles * a.nch;
  const int bh = a.BH >= 8 ? (b & 7) + 8 * ((b >> 3) / per_head) : b % a.BH;
  const int rem = a.BH >= 8 ? (b >> 3) % per_head : b / a.BH;
  const int row0 = (rem % a.tiles) * ROWS;
  if (bh >= a.BH) return;
  const int N = a.N, nblk = (N + KB - 1) / KB;
  const bool ragged = (N % KB) != 0;  // the last block has keys past N
  Chunk ch;
  ch.chunk = rem / a.tiles;
  ch.blk0 = ch.chunk * a.cblk;
  ch.blk1 = min(nblk, ch.blk0 + a.cblk);
  ch.kbase = ch.blk0 * KB;
  ch.kend = min(N, ch.blk1 * KB);
  ch.kk = min(a.k, ch.kend - ch.kbase);
  const int blk0 = ch.blk0, blk1 = ch.blk1;
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
  float A[TL], B[TL];  // this lane's rows' histogram bins: bin = fma(c, A, B)
  // ------------------------------------------------------------ V: values
  // (and the histogram of the same scores)
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
    // in this pass wave w streams a contiguous quarter of the chunk's blocks,
    // [vb0, vb1), so that the waves' first blocks are spread over it
    const int nbc = blk1 - blk0;
    const int vb0 = blk0 + (w * nbc) / NW, vb1 = blk0 + ((w + 1) * nbc) / NW;
    if (vb0 < vb1) {
      load_k(kr, Kh, vb0, N, g, c16);
      load_v(vr, Vh, vb0, N, lane);
    }
    // the histogram bins, fixed before the scores stream by: each wave's
    // first block (spread over the chunk) samples every row's scores, and
    // the 256 bins span [hi - 1.5 r, hi + 0.5 r] around the samples' range
    // r = hi - lo; scores outside clamp into the end bins.  The bins decide
    // only how many keys the exact steps below must rank, never which keys
    // are taken.  (Without fuse the bins come from the exact range after
    // this pass, and a third pass builds the histogram.)
    if constexpr (FUSE) {
      float slo[TL], shi[TL];
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        slo[tl] = INFINITY;
        shi[tl] = -INFINITY;
      }
      if (vb0 < vb1) {
        const int blk = vb0;
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) {
          float sc[4][4];
          block_scores(kr, qlr, tl, sc);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool ok = key_of(blk, kt, g, r) < N;
              slo[tl] = ok ? fminf(slo[tl], sc[kt][r]) : slo[tl];
              shi[tl] = ok ? fmaxf(shi[tl], sc[kt][r]) : shi[tl];
            }
        }
      }
      float2* samp = reinterpret_cast<float2*>(sm + OFF_UNION + union_bytes(a.cap, NW));
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        slo[tl] = fminf(slo[tl], __shfl_xor(slo[tl], 16, 64));
        slo[tl] = fminf(slo[tl], __shfl_xor(slo[tl], 32, 64));
        shi[tl] = fmaxf(shi[tl], __shfl_xor(shi[tl], 16, 64));
        shi[tl] = fmaxf(shi[tl], __shfl_xor(shi[tl], 32, 64));
        if (g == 0) samp[w * ROWS + 16 * tl + c16] = make_float2(slo[tl], shi[tl]);
      }
      __syncthreads();
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        float lo = INFINITY, hi = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float2 v = samp[ww * ROWS + 16 * tl + c16];
          lo = fminf(lo, v.x);
          hi = fmaxf(hi, v.y);
        }
        // (the last wave always has a block, so the row has samples)
        const float r = hi > lo ? hi - lo : fmaxf(fabsf(hi), 1.0f);
        const float bot = hi - 1.5f * r;
        A[tl] = fminf(128.0f / r, 1e30f);
        B[tl] = -bot * A[tl];
        if (w == 0 && g == 0) {
          rows[16 * tl + c16].lo = bot;
          rows[16 * tl + c16].A = A[tl];
          rows[16 * tl + c16].B = B[tl];
        }
      }
    }
    // one block of this pass; LAST: the chunk's ragged last block, whose keys
    // past N get score -inf (weight 0) and count into the spare histogram
    // word (compile-time, like FUSE, so that the steady-state blocks carry
    // no per-key tests)
    auto vblock = [&](auto last_c, int blk) {
      constexpr bool LAST = decltype(last_c)::value;
      // the V registers are free once stored and the K registers once the
      // scores are out: the next block's loads go out right after each
      store_v(vr, vt, lane);
      if (blk + 1 < vb1) load_v(vr, Vh, blk + 1, N, lane);
      group_sync();
      // the block's V^T A operands, shared by both row tiles:
      // V^T[channel 16ct + c16][keys 32sp + 4g .., 32sp + 16 + 4g ..], by
      // transposing reads (lane points at key 32sp + 4g + (c16 >> 2) (+ 16),
      // channels 16ct + 4 (c16 & 3) ..)
      u32x4 av[4][2];
      const char* vtl = vt + (4 * g + (c16 >> 2)) * V_STRIDE + 8 * (c16 & 3);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
          const u32x2 lo2 = lds_tr16(vtl + 32 * sp * V_STRIDE + 32 * ct);
          const u32x2 hi2 = lds_tr16(vtl + (32 * sp + 16) * V_STRIDE + 32 * ct);
          av[ct][sp] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        }
      }
      uint32_t valid = 0xFFFFu;  // bit 4kt + r: key 64blk + 16kt + 4g + r < N
      if constexpr (LAST) {
        valid = 0u;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) valid |= (key_of(blk, kt, g, r) < N ? 1u : 0u) << (4 * kt + r);
      }
      // every tile's scores first, so that the next block's K loads go out
      // before the weights and products
      float sc[TL][4][4];
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) block_scores(kr, qlr, tl, sc[tl]);
      if (blk + 1 < vb1) load_k(kr, Kh, blk + 1, N, g, c16);
#pragma unroll
      for (int tl = 0; tl < TL; ++tl) {
        float (&s)[4][4] = sc[tl];
        uint32_t* myhist =
            reinterpret_cast<uint32_t*>(sm + OFF_HIST + (16 * tl + c16) * HIST_STRIDE);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = !LAST || (valid >> (4 * kt + r) & 1u);
            if constexpr (FUSE) atomicAdd(myhist + (ok ? bin_of(s[kt][r], A[tl], B[tl]) : SPARE_BIN), 1u);
            else mn[tl] = ok ? fminf(mn[tl], s[kt][r]) : mn[tl];
            if constexpr (LAST) s[kt][r] = ok ? s[kt][r] : -INFINITY;
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
    };
    // the ragged last block (if this wave streams it) runs on its own
    const int vsteady = ragged && vb0 < vb1 && vb1 == nblk ? vb1 - 1 : vb1;
#pragma unroll 1
    for (int blk = vb0; blk < vsteady; ++blk) vblock(std::false_type{}, blk);
    if (vsteady < vb1) vblock(std::true_type{}, vsteady);

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
    if (blk0 + w < blk1) load_k(kpre, Kh, blk0 + w, N, g, c16);
    __syncthreads();
    // merge: thread -> (row, 4 channels), ROWS * 16 items; with several
    // chunks the merged sums stay unnormalised and go out as the chunk's
    // partial (reference max M, sum L)
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
        if (a.nch == 1) {
          if (a.stats && c4 == 0) {
            float4* st = a.stats + (size_t)bh * a.m + row0 + r;
            st->x = M * 0.125f;
            st->y = L;
          }
          const float inv = 1.0f / L;
          *reinterpret_cast<float4*>(a.vl + ((size_t)bh * a.m + row0 + r) * 64 + c4) =
              make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        } else {
          float* pp = a.vlpart +
                      (((size_t)bh * a.m + row0 + r) * a.nch + ch.chunk) * PART_STRIDE;
          *reinterpret_cast<float4*>(pp + c4) = o;
          if (c4 == 0) *reinterpret_cast<float2*>(pp + 64) = make_float2(M, L);
        }
      }
      if (!FUSE && c4 == 0) {
        // 256 bins over the chunk's exact score range (capped so that
        // fma(c, A, B) stays finite)
        const float Ax = hi > lo ? fminf(256.0f / (hi - lo), 1e30f) : 0.f;
        rows[r].lo = lo;
        rows[r].A = Ax;
        rows[r].B = -lo * Ax;
      }
    }
    __syncthreads();
  }
  if constexpr (!FUSE) {
#pragma unroll
    for (int tl = 0; tl < TL; ++tl) {
      A[tl] = rows[16 * tl + c16].A;
      B[tl] = rows[16 * tl + c16].B;
    }
    // ---------------------------------------------------------- H: histogram
    {
      QLRegs qlr;
      ql_load(qlr, sm, lane);
      KRegs kr = kpre;
      for (int blk = blk0 + w; blk < blk1; blk += NW) {
        // keys past N of a ragged last block count into the spare word past
        // the 256 bins (no branch per score)
        uint32_t spare = 0u;
        if (ragged && blk == nblk - 1) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              spare |= (key_of(blk, kt, g, r) < N ? 0u : 1u) << (4 * kt + r);
        }
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) {
          float s[4][4];
          block_scores(kr, qlr, tl, s);
          if (tl == TL - 1 && blk + NW < blk1) load_k(kr, Kh, blk + NW, N, g, c16);
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
    if (blk0 + w < blk1) load_k(kpre, Kh, blk0 + w, N, g, c16);
  }

  __syncthreads();
  // the bin holding each row's k-th best: group g of wave w takes rows
  // 4w + g + 4 NW i
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    const int r = 4 * w + g + 4 * NW * i;
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
    const int need = ch.kk;
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
    // the block's scores of tile tl that are in the boundary bin or above
    // (and, with BOUNDED, beat the admission bound (thr, thrkey)), as bits
    // 4kt + r; `valid` masks the keys past N of a ragged last block
    auto cand_mask = [&](auto bounded, const float (&s)[4][4], int tl, int blk, uint32_t valid,
                         float thr, int thrkey) {
      constexpr bool BOUNDED = decltype(bounded)::value;
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
      return msk & valid;
    };
    // each lane reserves its own run of slots in its row's buffer (the order
    // of a buffer's entries does not matter: they are ranked by score and key
    // id), then writes its candidates there as (score, key) pairs
    auto reserve = [&](uint32_t msk, int tl) {
      const int c = __popc(msk);
      return c > 0 ? atomicAdd(&rows[16 * tl + c16].cnt, c) : 0;
    };
    auto append = [&](const float (&s)[4][4], int tl, int blk, uint32_t msk, int pos) {
      float* buf = reinterpret_cast<float*>(sm + OFF_UNION + (size_t)(16 * tl + c16) * a.cap * 8);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (msk >> (4 * kt + r) & 1u) {
            *reinterpret_cast<float2*>(buf + 2 * pos) =
                make_float2(s[kt][r], __int_as_float(key_of(blk, kt, g, r)));
            ++pos;
          }
    };
    if (flag[0] == 0) {
      // every row's candidates fit: one streaming pass.  The wave's blocks
      // alternate between two register sets, each refilled two blocks ahead
      // (this pass does little work per block, so one block of lead would
      // leave the loads' latency exposed).
      KRegs ka = kpre, kb;
      if (blk0 + w + NW < blk1) load_k(kb, Kh, blk0 + w + NW, N, g, c16);
      // LAST: the ragged last block (masked keys), run on its own so that
      // the steady-state blocks carry no per-key tests
      auto cblock = [&](auto last_c, int blk, KRegs& kr) {
        constexpr bool LAST = decltype(last_c)::value;
        const uint32_t valid = LAST ? valid_bits(blk) : 0xFFFFu;
        float s[TL][4][4];
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) block_scores(kr, qlr, tl, s[tl]);
        if (blk + 2 * NW < blk1) load_k(kr, Kh, blk + 2 * NW, N, g, c16);
        // both tiles reserve before either writes, so that one wait covers
        // both reservations
        uint32_t msk[TL];
        uint32_t any = 0u;
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) {
          msk[tl] = cand_mask(std::false_type{}, s[tl], tl, blk, valid, 0.f, 0);
          any |= msk[tl];
        }
        if (__ballot(any != 0u) == 0) return;
        int pos[TL];
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) pos[tl] = reserve(msk[tl], tl);
#pragma unroll
        for (int tl = 0; tl < TL; ++tl) append(s[tl], tl, blk, msk[tl], pos[tl]);
      };
      const int csteady = ragged && blk1 == nblk ? nblk - 1 : blk1;
      int blk = blk0 + w;
#pragma unroll 1
      for (; blk + NW < csteady; blk += 2 * NW) {
        cblock(std::false_type{}, blk, ka);
        cblock(std::false_type{}, blk + NW, kb);
      }
      bool in_b = false;  // the next block's rows are in kb
      if (blk < csteady) {
        cblock(std::false_type{}, blk, ka);
        in_b = true;
      }
      if (csteady < blk1 && (csteady - blk0) % NW == w) {
        if (in_b)
          cblock(std::true_type{}, csteady, kb);
        else
          cblock(std::true_type{}, csteady, ka);
      }
    } else {
      // one block at a time (its owner wave appends, at most KB entries per
      // row); rows that could overflow on the next block are cut back first
      for (int blk = blk0; blk < blk1; ++blk) {
        if ((blk - blk0) % NW == w) {
          const uint32_t valid = ragged && blk == nblk - 1 ? valid_bits(blk) : 0xFFFFu;
          KRegs kr;
          load_k(kr, Kh, blk, N, g, c16);
#pragma unroll
          for (int tl = 0; tl < TL; ++tl) {
            float s[4][4];
            block_scores(kr, qlr, tl, s);
            const int lr = 16 * tl + c16;
            const uint32_t msk = cand_mask(std::true_type{}, s, tl, blk, valid, rows[lr].thr, rows[lr].thrkey);
            if (__ballot(msk != 0u) != 0) append(s, tl, blk, msk, reserve(msk, tl));
          }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPG; ++i) {
          const int r = 4 * w + g + 4 * NW * i;
          const bool work = row0 + r < a.m && rows[r].over && rows[r].cnt > a.cap - KB;
          if (__ballot(work) != 0) row_cut(sm, a, ch.kk, r, work, c16, g);
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();

  // ------------------------------------------------------------ F: final
  // group g of wave w takes rows 4w + g + 4 NW i, all RPG of them together
  {
    int lr[RPG];
    bool work[RPG];
    int32_t* outk[RPG];
    float* outs[RPG];
#pragma unroll
    for (int i = 0; i < RPG; ++i) {
      lr[i] = 4 * w + g + 4 * NW * i;
      work[i] = row0 + lr[i] < a.m;
      const size_t row = (size_t)bh * a.m + (work[i] ? row0 + lr[i] : 0);
      if (a.nch == 1) {
        outk[i] = a.idx + row * a.k;
        outs[i] = nullptr;
      } else {
        const size_t at = (row * a.nch + ch.chunk) * a.k;
        outk[i] = a.cand_k + at;
        outs[i] = a.cand_s + at;
      }
    }
    rows_final<RPG>(sm, a, ch, lr, work, c16, g, outk, outs);
  }
}

// One wave per (head, landmark row) joins the chunks of the landmark pass.
// V_L: the chunks' unnormalised sums by log-sum-exp.  Top-k: the chunks'
// candidate lists hold n = (nch - 1) * k + kk_last (score, key) entries,
// ascending by key within a chunk and chunks in key order, so ascending over
// the whole list; the row's k best (larger score, then lower key id) are
// found by a 256-bin histogram over the entries' range: every entry above the
// boundary bin is taken and the boundary bin's entries are ranked among
// themselves (listed in LDS and ranked once: the listed entry of rank need - 1
// is the cut, and a boundary entry wins when it is at least as good; or, when
// more than LISTCAP share the bin, each against every entry in it); winners
// are written in list order, which is ascending key order.
// MW rows per workgroup (a wave each) and MU entries per lane in flight:
// every loop over the candidate list reads MU entries per lane before using
// any.  Used for many short rows (long-16k: 8,192 rows of 1,024, MW = 4,
// MU = 8); few long ones (a 1-D sequence, seq-256k: 512 rows of 16,384) go
// to merge_row_kernel below, four waves per row.
constexpr int LISTCAP = 256;

__device__ __forceinline__ int wave_suffix(int v, int lane) {
  // inclusive suffix sum over the 64 lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_down(v, o, 64);
    v += lane + o < 64 ? x : 0;
  }
  return v;
}

template <int MU, int MW>
__global__ __launch_bounds__(64 * MW) void merge_kernel(Args a) {
  __shared__ uint32_t hist[MW][256];
  __shared__ float2 blist[MW][LISTCAP];
  __shared__ int bcount[MW];
  __shared__ float2 cut[MW];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * MW + w;
  if (row >= (long long)a.BH * a.m) return;  // (wave-level work only below)
  const int nch = a.nch, k = a.k;
  // ---- V_L
  {
    const float* pp = a.vlpart + row * nch * PART_STRIDE;
    float M = -INFINITY;
    for (int c0 = 0; c0 < nch; c0 += MU) {
      float mv[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) mv[u] = c0 + u < nch ? pp[(c0 + u) * PART_STRIDE + 64] : -INFINITY;
#pragma unroll
      for (int u = 0; u < MU; ++u) M = fmaxf(M, mv[u]);
    }
    float o = 0.f, L = 0.f;
    for (int c0 = 0; c0 < nch; c0 += MU) {
      float mv[MU], ov[MU], lv[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const bool ok = c0 + u < nch;
        const float* q = pp + (ok ? c0 + u : 0) * PART_STRIDE;
        mv[u] = ok ? q[64] : -INFINITY;
        ov[u] = ok ? q[lane] : 0.f;
        lv[u] = ok ? q[65] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const float f = __builtin_amdgcn_exp2f((mv[u] - M) * kTauLog2e);
        o = fmaf(f, ov[u], o);
        L = fmaf(f, lv[u], L);
      }
    }
    a.vl[row * 64 + lane] = o / L;
    if (a.stats && lane == 0) {
      a.stats[row].x = M * 0.125f;
      a.stats[row].y = L;
    }
  }
  // ---- top-k
  const int last_keys = a.N - (nch - 1) * a.cblk * KB;
  const int n = (nch - 1) * k + min(k, last_keys);
  const float* cs = a.cand_s + row * nch * k;
  const int32_t* ck = a.cand_k + row * nch * k;
  // this lane's entries e0 + 64 u (u < MU) of a step starting at e0; past n
  // they read -inf (the min / max below skip them)
  auto load_s = [&](int e0, float (&v)[MU]) {
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      v[u] = e < n ? cs[e] : -INFINITY;
    }
  };
  float lo = INFINITY, hi = -INFINITY;
  for (int e0 = 0; e0 < n; e0 += 64 * MU) {
    float v[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      lo = fminf(lo, e0 + 64 * u + lane < n ? v[u] : INFINITY);
      hi = fmaxf(hi, v[u]);
    }
  }
  lo = wave_min_f(lo);
  hi = wave_max(hi);
  const float A = hi > lo ? fminf(256.0f / (hi - lo), 1e30f) : 0.f;
  const float B = -lo * A;
  uint32_t* h = hist[w];
#pragma unroll
  for (int q = 0; q < 4; ++q) h[4 * lane + q] = 0u;
  if (lane == 0) bcount[w] = 0;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  for (int e0 = 0; e0 < n; e0 += 64 * MU) {
    float v[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u)
      if (e0 + 64 * u + lane < n) atomicAdd(&h[bin_of(v[u], A, B)], 1u);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // boundary bin: lane l holds bins 4l .. 4l + 3
  int cb[4], local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    cb[q] = (int)h[4 * lane + q];
    local += cb[q];
  }
  const int suf = wave_suffix(local, lane);
  const int above_lane = suf - local;
  int bstar = 0, above = 0;
  if (above_lane < k && k <= suf) {
    int acc = above_lane;
    bool found = false;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (!found) {
        if (acc + cb[q] >= k) {
          found = true;
          bstar = 4 * lane + q;
          above = acc;
        } else {
          acc += cb[q];
        }
      }
    }
  }
  // exactly one lane found it
  const uint64_t who = __ballot(above_lane < k && k <= suf);
  const int src = __ffsll((unsigned long long)who) - 1;
  bstar = __shfl(bstar, src, 64);
  above = __shfl(above, src, 64);
  const int need = k - above;
  const int nb = __shfl(cb[bstar & 3], bstar >> 2, 64);
  // the boundary bin's entries into the list (when they fit)
  const bool listed = nb <= LISTCAP;
  if (listed) {
    for (int e0 = 0; e0 < n; e0 += 64 * MU) {
      float v[MU];
      load_s(e0, v);
      int kk[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int e = e0 + 64 * u + lane;
        kk[u] = e < n && bin_of(v[u], A, B) == bstar ? ck[e] : -1;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        if (kk[u] >= 0) {
          const int at = atomicAdd(&bcount[w], 1);
          blist[w][at] = make_float2(v[u], __int_as_float(kk[u]));
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // the cut: the listed entry with need - 1 entries of the list before it
    // (keys are distinct, so the ranks are 0 .. nb - 1 and one entry has it)
    for (int j = lane; j < nb; j += 64) {
      const float2 x = blist[w][j];
      int r = 0;
      for (int i = 0; i < nb; ++i) {
        const float2 y = blist[w][i];
        r += better(y.x, __float_as_int(y.y), x.x, __float_as_int(x.y)) ? 1 : 0;
      }
      if (r == need - 1) cut[w] = x;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
  const float2 cu = cut[w];  // (read only when listed)
  const float cv = cu.x;
  const int ckey = __float_as_int(cu.y);
  // winners in list order (entry e0 + 64 u + lane: u-major steps of 64)
  int32_t* out = a.idx + row * k;
  int run = 0;
  for (int e0 = 0; e0 < n; e0 += 64 * MU) {
    float v[MU];
    int key[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      key[u] = e < n ? ck[e] : 0;
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      bool win = false;
      if (e < n) {
        const int bn = bin_of(v[u], A, B);
        if (bn > bstar) {
          win = true;
        } else if (bn == bstar) {
          if (listed) {
            // the cut itself or better
            win = v[u] > cv || (v[u] == cv && key[u] <= ckey);
          } else {
            int r = 0;
            for (int j = 0; j < n; ++j) {
              const float x = cs[j];
              r += (bin_of(x, A, B) == bstar && better(x, ck[j], v[u], key[u])) ? 1 : 0;
            }
            win = r < need;
          }
        }
      }
      const uint64_t bw = __ballot(win);
      if (win) out[run + lanes_below(bw)] = key[u];
      run += __popcll(bw);
    }
  }
}

// The same join with a four-wave workgroup per row, for few long rows (a
// 1-D sequence: seq-256k has 512 rows of 16,384 candidates): wave w takes
// the contiguous quarter [w n / 4, (w + 1) n / 4) of the row's list and
// chunks w, w + 4, .. of its V_L partials; the histogram, the boundary list
// and its cut are shared in LDS, and winners are first counted per quarter,
// then written in list order from each quarter's offset.
constexpr int CW = 4;  // waves per row

template <int MU>
__global__ __launch_bounds__(64 * CW) void merge_row_kernel(Args a) {
  __shared__ uint32_t hist[256];
  __shared__ float2 blist[LISTCAP];
  __shared__ float vlo[CW][64];
  __shared__ float wred[4][CW];  // per wave: V_L max, V_L sum, score min, score max
  __shared__ int bcount, bsel[3], wcnt[CW];
  __shared__ float2 cut;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const long long row = blockIdx.x;
  if (row >= (long long)a.BH * a.m) return;  // (uniform over the workgroup)
  const int nch = a.nch, k = a.k;
  for (int i = tid; i < 256; i += 64 * CW) hist[i] = 0u;
  if (tid == 0) bcount = 0;
  // ---- V_L: this wave's chunks, then the four partials joined by wave 0
  {
    const float* pp = a.vlpart + row * nch * PART_STRIDE;
    float M = -INFINITY;
    for (int c0 = w; c0 < nch; c0 += CW * MU) {
      float mv[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int c = c0 + CW * u;
        mv[u] = c < nch ? pp[c * PART_STRIDE + 64] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) M = fmaxf(M, mv[u]);
    }
    float o = 0.f, L = 0.f;
    for (int c0 = w; c0 < nch; c0 += CW * MU) {
      float mv[MU], ov[MU], lv[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int c = c0 + CW * u;
        const bool ok = c < nch;
        const float* q = pp + (ok ? c : 0) * PART_STRIDE;
        mv[u] = ok ? q[64] : -INFINITY;
        ov[u] = ok ? q[lane] : 0.f;
        lv[u] = ok ? q[65] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        // (a wave without chunks keeps M = -inf and sums of 0)
        const float f = mv[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mv[u] - M) * kTauLog2e);
        o = fmaf(f, ov[u], o);
        L = fmaf(f, lv[u], L);
      }
    }
    vlo[w][lane] = o;
    if (lane == 0) {
      wred[0][w] = M;
      wred[1][w] = L;
    }
  }
  // ---- top-k: this wave's quarter of the list
  const int last_keys = a.N - (nch - 1) * a.cblk * KB;
  const int n = (nch - 1) * k + min(k, last_keys);
  const int q0 = (int)((long long)w * n / CW), q1 = (int)((long long)(w + 1) * n / CW);
  const float* cs = a.cand_s + row * nch * k;
  const int32_t* ck = a.cand_k + row * nch * k;
  auto load_s = [&](int e0, float (&v)[MU]) {
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      v[u] = e < q1 ? cs[e] : -INFINITY;
    }
  };
  {
    float lo = INFINITY, hi = -INFINITY;
    for (int e0 = q0; e0 < q1; e0 += 64 * MU) {
      float v[MU];
      load_s(e0, v);
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        lo = fminf(lo, e0 + 64 * u + lane < q1 ? v[u] : INFINITY);
        hi = fmaxf(hi, v[u]);
      }
    }
    lo = wave_min_f(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      wred[2][w] = lo;
      wred[3][w] = hi;
    }
  }
  __syncthreads();
  if (w == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < CW; ++i) M = fmaxf(M, wred[0][i]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const float f = wred[0][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((wred[0][i] - M) * kTauLog2e);
      o = fmaf(f, vlo[i][lane], o);
      L = fmaf(f, wred[1][i], L);
    }
    a.vl[row * 64 + lane] = o / L;
    if (a.stats && lane == 0) {
      a.stats[row].x = M * 0.125f;
      a.stats[row].y = L;
    }
  }
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    lo = fminf(lo, wred[2][i]);
    hi = fmaxf(hi, wred[3][i]);
  }
  const float A = hi > lo ? fminf(256.0f / (hi - lo), 1e30f) : 0.f;
  const float B = -lo * A;
  for (int e0 = q0; e0 < q1; e0 += 64 * MU) {
    float v[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u)
      if (e0 + 64 * u + lane < q1) atomicAdd(&hist[bin_of(v[u], A, B)], 1u);
  }
  __syncthreads();
  // the boundary bin (wave 0; lane l holds bins 4l .. 4l + 3)
  if (w == 0) {
    int cb[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cb[q] = (int)hist[4 * lane + q];
      local += cb[q];
    }
    const int suf = wave_suffix(local, lane);
    const int above_lane = suf - local;
    if (above_lane < k && k <= suf) {
      int acc = above_lane;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        if (acc + cb[q] >= k) {
          bsel[0] = 4 * lane + q;
          bsel[1] = acc;
          bsel[2] = cb[q];
          break;
        }
        acc += cb[q];
      }
    }
  }
  __syncthreads();
  const int bstar = bsel[0], above = bsel[1], nb = bsel[2];
  const int need = k - above;
  const bool listed = nb <= LISTCAP;
  if (listed) {
    for (int e0 = q0; e0 < q1; e0 += 64 * MU) {
      float v[MU];
      load_s(e0, v);
      int kk[MU];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int e = e0 + 64 * u + lane;
        kk[u] = e < q1 && bin_of(v[u], A, B) == bstar ? ck[e] : -1;
      }
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        if (kk[u] >= 0) {
          const int at = atomicAdd(&bcount, 1);
          blist[at] = make_float2(v[u], __int_as_float(kk[u]));
        }
      }
    }
    __syncthreads();
    // the cut: the listed entry with need - 1 entries of the list before it
    for (int j = tid; j < nb; j += 64 * CW) {
      const float2 x = blist[j];
      int r = 0;
      for (int i = 0; i < nb; ++i) {
        const float2 y = blist[i];
        r += better(y.x, __float_as_int(y.y), x.x, __float_as_int(x.y)) ? 1 : 0;
      }
      if (r == need - 1) cut = x;
    }
    __syncthreads();
  }
  const float cv = cut.x;  // (read only when listed)
  const int ckey = __float_as_int(cut.y);
  auto wins = [&](float v, int key) {
    const int bn = bin_of(v, A, B);
    if (bn > bstar) return true;
    if (bn < bstar) return false;
    if (listed) return v > cv || (v == cv && key <= ckey);
    int r = 0;
    for (int j = 0; j < n; ++j) {
      const float x = cs[j];
      r += (bin_of(x, A, B) == bstar && better(x, ck[j], v, key)) ? 1 : 0;
    }
    return r < need;
  };
  // winners: counted per quarter, then written in list order
  int mine = 0;
  for (int e0 = q0; e0 < q1; e0 += 64 * MU) {
    float v[MU];
    int key[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      key[u] = e < q1 ? ck[e] : 0;
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      mine += __popcll(__ballot(e < q1 && wins(v[u], key[u])));
    }
  }
  if (lane == 0) wcnt[w] = mine;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < w; ++i) run += wcnt[i];
  int32_t* out = a.idx + row * k;
  for (int e0 = q0; e0 < q1; e0 += 64 * MU) {
    float v[MU];
    int key[MU];
    load_s(e0, v);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      key[u] = e < q1 ? ck[e] : 0;
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int e = e0 + 64 * u + lane;
      const bool win = e < q1 && wins(v[u], key[u]);
      const uint64_t bw = __ballot(win);
      if (win) out[run + lanes_below(bw)] = key[u];
      run += __popcll(bw);
    }
  }
}

}  // namespace lmk

// The row buffer holds k plus one block of candidates (k + 64 entries, at
// most 512: one bit each in the selection masks).
static int landmark_cap(const Shape& s) {
  const int cap = (s.k + lmk::KB + 15) & ~15;
  return cap <= 512 ? cap : 0;
}

// Keys per workgroup: the head's blocks split into the fewest chunks of at
// most 4096 keys (a chunk's key bitmap must fit a histogram row), i.e. one
// chunk up to 4096 keys.  Measured at 3136 tokens (192 heads, 384 workgroups
// with one chunk), more chunks only cost: a workgroup's fixed work (clearing
// its histograms, staging Q_L, each pass's set-up) does not shrink with its
// share of the keys, and the landmark kernel took 107 us with one chunk, 125
// us with three (plus 19 us of merge) and 250 us with fourteen.
static void landmark_chunks(const Shape& s, int& nch, int& cblk) {
  const int nblk = (s.N + lmk::KB - 1) / lmk::KB;
  nch = (nblk + lmk::CHUNK_BLOCKS - 1) / lmk::CHUNK_BLOCKS;
  cblk = (nblk + nch - 1) / nch;
  nch = (nblk + cblk - 1) / cblk;
}

bool landmark_bf16_supported(const Shape& s) {
  return s.bf16 && landmark_cap(s) > 0 && lmk::lds_bytes(landmark_cap(s), lmk::NW4) <= 160 * 1024;
}

size_t landmark_bf16_scratch_bytes(const Shape& s) {
  int nch, cblk;
  landmark_chunks(s, nch, cblk);
  if (nch == 1) return 0;
  const size_t rows = (size_t)s.BH * s.m * nch;
  return align_up(rows * s.k * 4, 256) * 2 + rows * lmk::PART_STRIDE * 4;
}

hipError_t launch_landmark_bf16(const float* ql, const void* K, const void* V, int32_t* idx,
                                float* vl, void* scratch, const Shape& s, hipStream_t st,
                                float4* stats) {
  int nch, cblk;
  landmark_chunks(s, nch, cblk);
  const size_t rows = (size_t)s.BH * s.m * nch;
  char* sc = (char*)scratch;
  float* cand_s = nch > 1 ? (float*)sc : nullptr;
  int32_t* cand_k = nch > 1 ? (int32_t*)(sc + align_up(rows * s.k * 4, 256)) : nullptr;
  float* vlpart = nch > 1 ? (float*)(sc + 2 * align_up(rows * s.k * 4, 256)) : nullptr;
  if (nch > 1 && !scratch) return hipErrorInvalidValue;
  // the histogram rides the values pass when the candidate buffer's slack
  // (64 entries past k) is at least half of k: the sampled bins are about
  // twice as wide as exact ones, and a row whose boundary bin overflows the
  // slack sends its workgroup down the block-by-block path (measured: 3136
  // tokens, k = 64: 110 -> 100 us; long-16k, k = 256: 494 -> 733 us fused)
  const int fuse_h = s.k <= 128 ? 1 : 0;
  lmk::Args a{ql, (const uint16_t*)K, (const uint16_t*)V, idx, vl, s.BH, s.N, s.m, s.k,
              landmark_cap(s), (s.m + lmk::ROWS - 1) / lmk::ROWS, nch, cblk, fuse_h, cand_s,
              cand_k, vlpart, stats};
  if (a.cap == 0) return hipErrorInvalidValue;
  // eight waves where a four-wave workgroup's LDS (the candidate buffers for
  // k >= 128) already leaves room for only one workgroup per CU: the same
  // LDS then carries twice the waves streaming the keys
  constexpr size_t cu_lds = 160 * 1024;
  const bool wide = 2 * lmk::lds_bytes(a.cap, 4) > cu_lds && lmk::lds_bytes(a.cap, 8) <= cu_lds;
  const int nw = wide ? 8 : lmk::NW4;
  const size_t lds = lmk::lds_bytes(a.cap, nw);
  if (lds > cu_lds) return hipErrorInvalidValue;
  auto kernel = fuse_h ? (wide ? lmk::landmark_kernel<true, 8> : lmk::landmark_kernel<true, 4>)
                       : (wide ? lmk::landmark_kernel<false, 8> : lmk::landmark_kernel<false, 4>);
  static std::atomic<unsigned long long> lds_set[4];
  if (const hipError_t e = allow_lds((const void*)kernel, 160 * 1024, lds_set[fuse_h + 2 * wide]);
      e != hipSuccess)
    return e;
  const int grid = s.BH >= 8 ? ((s.BH + 7) / 8) * 8 * a.tiles * nch : s.BH * a.tiles * nch;
  kernel<<<grid, 64 * nw, lds, st>>>(a);
  if (nch == 1) return hipGetLastError();
  // many short rows: four rows per workgroup, eight entries per lane in
  // flight; few long ones: a four-wave workgroup per row
  const long long rws = (long long)s.BH * s.m;
  if (rws >= 4096)
    lmk::merge_kernel<8, 4><<<(unsigned)((rws + 3) / 4), 64 * 4, 0, st>>>(a);
  else
    lmk::merge_row_kernel<8><<<(unsigned)rws, 64 * lmk::CW, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mita
