// Step a7 for bf16 inputs on long grids -- grouped expert attention (page
// "NeurIPS'26：注意力也是FFN？...", the s = 1 output and Algorithm 1: queries
// grouped by route attend their expert's k raw key/value pairs and the m
// shared ones under one softmax; partial results merge by online softmax).
//
// Persistent workgroups, P per head, placed on the head's XCD so the head's
// K, V and Q rows are re-read from that XCD's L2 (spread over the XCDs when
// there are fewer than 8 heads).  A head's passes (runs of up to 64 of one
// expert's queries, in expert order) are cut into P contiguous ranges of
// near-equal length, one per workgroup, so that a large expert's queries are
// spread over several workgroups.  Per workgroup:
//   * load its segments' table (each a run of one expert's queries: range
//     and the expert's key ids) and the head's Q_L (bf16 hi + lo, or one f16
//     copy where that leaves the room for resident slots) and V_L^T (f16)
//     into LDS once;
//   * per segment: its expert's k key rows (bf16) and value rows (f16) sit in LDS,
//     shared by the four waves; V^T fragments come from the value rows by the
//     transposing LDS read.  While one segment is computed the
//     next one's first 64 rows (and the Q rows of its first 64 queries) are
//     already loading into registers; the segment's output stores are issued
//     only after those rows have been waited for, since stores and loads
//     drain through one counter.  For k > 64 the slots past the first 64 are
//     staged once per segment when all k fit (resident), else gathered in
//     place 64 at a time for every pass;
//   * per pass of <= 64 of the expert's queries, each wave owns 16: Q rows
//     are the B operand of logits^T = [Q_L; K_e] Q^T; an online softmax runs
//     over 32-entry chunks (shared entries first, then the expert's keys), and
//     each chunk's weights go straight from the logit accumulators into
//     out^T += [V_L; V_e]^T P^T on f16 MFMA, with the normaliser from an
//     all-ones MFMA.
// With s experts per query the grouped items are the (query, rank) pairs
// t = n * s + j: an item attends its expert's keys, plus the shared entries
// when j = 0 (masked to -inf for the others), and leaves its unnormalised
// sums and softmax reference (max, sum) in a partial buffer; merge_kernel then
// combines a query's s partials by log-sum-exp into its one softmax.  The
// route-only variant skips the shared entries.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "select.h"

namespace mita {
namespace att {

constexpr int TQ = 64;    // queries per pass (16 per wave)
constexpr int EC = 64;    // expert slots per LDS chunk
constexpr int EV_STRIDE = 64 * 2 + 16;  // bytes per staged V row (f16 channels + pad)
constexpr int MAXM = 256;

struct Args {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const float* ql;
  const float* vl;
  const int32_t* idx;
  const int32_t* offsets;
  const int32_t* perm;
  float* out;    // s = 1: the output; s > 1: unnormalised partial sums per item
  float2* pml;   // s > 1: each item's softmax reference maximum and sum
  int BH, N, m, k, parts;  // workgroups per head
  int s, shared;
  int kres;  // expert slots staged at once: k rounded up to EC (all resident), or EC
};

// Upper bound on a head's passes (TQ-item runs of one expert's items):
// sum over experts of ceil(c_e / TQ) <= (N s) / TQ + m.
__host__ __device__ inline int max_passes(int m, int N, int s) {
  return m + (int)(((long long)N * s + TQ - 1) / TQ);
}

// LDS layout; the segment table holds, per segment of the workgroup (a run
// of one expert's items), [first item's place in the expert order, count,
// k key ids]; the head's expert offsets sit beside it.
// A workgroup takes at most ceil(tmax / parts) passes, so at most that many
// segments (each holds at least one of its passes).  Q_L is held as bf16 hi +
// lo, or (ql16) as one f16 copy; kres expert slots of K and V rows are staged
// at a time.
struct Lay {
  int mp, vlt_stride, ew, ts;
  int off_qlh, off_qll, off_vlt, off_ke, off_vet, off_tab, off_elist, off_scan, off_offs, bytes;
  __host__ __device__ Lay(int m, int k, int parts, int tmax, bool ql16, int kres) {
    mp = (m + 31) & ~31;
    vlt_stride = mp * 2 + 16;
    ew = (tmax + parts - 1) / parts;
    ts = 2 + k;
    off_qlh = 0;
    off_qll = off_qlh + mp * 128;
    off_vlt = off_qll + (ql16 ? 0 : mp * 128);
    off_ke = off_vlt + 64 * vlt_stride;
    off_vet = off_ke + kres * 128;
    off_tab = off_vet + kres * EV_STRIDE;
    off_elist = off_tab + ew * ts * 4;
    off_scan = off_elist + (ew + 1) * 4;  // [10] ints: the deal's wave totals and bounds
    off_offs = off_scan + 16 * 4;         // the head's m + 1 expert offsets
    bytes = off_offs + (m + 1) * 4;
  }
};

// One softmax update over NC 32-entry chunks for this lane's query column.
// x: raw logits (q . key) of entries {32i + 4g + r, 32i + 16 + 4g + r}
// (-inf when masked); get_av(i, av) fetches chunk i's A fragments of
// [V_L; V_e]^T for the four channel tiles.  Weights are exp2((x - mref) tau log2e) against a
// reference maximum that is only raised when some weight would exceed 2^8,
// so most updates skip rescaling the accumulators.
template <int NC, class GetAv>
__device__ __forceinline__ void softmax_update(const float (&x)[8 * NC], GetAv get_av,
                                               float& mref, f32x4 (&acc)[4], f32x4& lsum) {
  constexpr float cs = 0.125f * 1.4426950408889634f;  // tau * log2(e)
  float cm = x[0];
#pragma unroll
  for (int i = 1; i < 8 * NC; ++i) cm = fmaxf(cm, x[i]);
  if (__ballot((cm - mref) * cs > 8.0f) != 0) {
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    const float mnew = fmaxf(mref, cm);
    const float alpha = __builtin_amdgcn_exp2f((mref - mnew) * cs);
    mref = mnew;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = acc[ct] * alpha;
    lsum = lsum * alpha;
  }
  const float moff = -mref * cs;
  const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * i + r], cs, moff));
    const u32x4 bp = {pk_f16(p[0], p[1]), pk_f16(p[2], p[3]), pk_f16(p[4], p[5]), pk_f16(p[6], p[7])};
    u32x4 av[4];
    get_av(i, av);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma_f16(av[ct], bp, acc[ct]);
    lsum = mfma_f16(ones, bp, lsum);
  }
}

// A pass's result for this lane's query (or item), written to row nq when
// live.
struct PassOut {
  f32x4 acc[4];
  float inv;
  float mref, lsum;
  int nq;
  bool live;
};

// The pass's output rows (non-temporal: the output is not read again here).
// Lane (g, c16) holds channels 16 ct + 4g .. + 3 of its query; the lanes
// c16 and c16 ^ 8 trade their odd channel tiles, so that each store writes
// whole 128-byte lines: in one instruction the 8 lanes (g, c) and (g, c ^ 8)
// cover channels 0..31 (or 32..63) of one query.  Stores go through a buffer
// descriptor over the head's output rows, and a lane without a query stores
// at an offset past its range, which the hardware drops (no branch).  Called
// by the whole wave.
__device__ __forceinline__ void store_out(Rsrc outr, const PassOut& o, int g, int c16) {
  const f32x4 v0 = o.acc[0] * o.inv, v1 = o.acc[1] * o.inv;
  const f32x4 v2 = o.acc[2] * o.inv, v3 = o.acc[3] * o.inv;
  const f32x4 r1 = swap8(v1), r3 = swap8(v3);
  const int rnq = swap8(o.nq);
  const bool rlive = swap8(o.live ? 1 : 0) != 0;
  const bool lo = c16 < 8;
  const int own = o.live ? o.nq * 256 + 16 * g : PAST;
  const int other = rlive ? rnq * 256 + 16 * g : PAST;
  // first store: the low half-row's own queries; second: the high half's
  st16_nt(outr, lo ? v0 : r1, lo ? own : other + 64);
  st16_nt(outr, lo ? r1 : v0, lo ? other + 64 : own);
  st16_nt(outr, lo ? v2 : r3, lo ? own + 128 : other + 192);
  st16_nt(outr, lo ? r3 : v2, lo ? other + 192 : own + 128);
}

// QL16: Q_L as one f16 copy (the shared logits on f16 MFMA, one product per
// 32 channels instead of the hi and lo products), which leaves room to keep
// all of an expert's k slots in LDS for large m and k.  The shared logits only
// weigh values: top-k sets and routes are decided elsewhere.
// RES: every slot of the expert resident in LDS (staged once per segment;
// a.kres = k rounded up to 64), else 64-slot chunks re-staged per pass.
template <bool QL16, bool RES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attend_bf16_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const Lay L(a.m, a.k, a.parts, max_passes(a.m, a.N, a.s), QL16, RES ? a.kres : EC);
  constexpr bool res = RES;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // with 8 or more heads a head's workgroups share one XCD (and its L2:
  // workgroups go to the XCDs round robin); with fewer, a head's workgroups
  // alternate over the XCDs so that every XCD has work
  const int b = blockIdx.x;
  const int bh = a.BH >= 8 ? (b & 7) + 8 * ((b >> 3) / a.parts) : b % a.BH;
  const int part = a.BH >= 8 ? (b >> 3) % a.parts : b / a.BH;
  if (bh >= a.BH) return;
  const int N = a.N, m = a.m, k = a.k, P = a.parts, S = a.s;
  const bool shared = a.shared != 0;
  // The prologue's global loads are few round trips deep: the head's expert
  // offsets (one load per thread) and the first Q_L / V_L rows go out
  // together at entry; the deal and the segments' item ranges then come
  // from the LDS copy of the offsets, and only the key and item ids (then
  // the first segment's rows) depend on them.
  int* offl = reinterpret_cast<int*>(sm + L.off_offs);
  int* scan = reinterpret_cast<int*>(sm + L.off_scan);
  const int32_t* offs = a.offsets + (size_t)bh * (m + 1);
  const int o_mine = tid <= m ? offs[tid] : 0;
  float4 fq[4], fv[4];
  auto load_qv = [&](int base) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = base + 256 * u + tid, row = it >> 4, q4 = it & 15;
      fq[u] = fv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (it < L.mp * 16 && row < m) {
        fq[u] = *reinterpret_cast<const float4*>(a.ql + ((size_t)bh * m + row) * 64 + 4 * q4);
        fv[u] = *reinterpret_cast<const float4*>(a.vl + ((size_t)bh * m + row) * 64 + 4 * q4);
      }
    }
  };
  if (shared) load_qv(0);
  for (int e = tid; e <= m; e += blockDim.x) offl[e] = e == tid ? o_mine : offs[e];
  if (tid == 0) scan[8] = scan[9] = 0;
  __syncthreads();
  // The deal: the head's passes, in expert order (expert e's passes run
  // over its items TQ at a time), are cut into P contiguous ranges of
  // floor / ceil(T / P) passes; this workgroup takes range [lo, hi), i.e. a
  // segment (one expert's run of items) of every expert that has passes in
  // it.  A large expert is so spread over several workgroups, and each
  // workgroup's pass count is within one of the mean.  Every workgroup of
  // the head computes the same cut.  One thread per expert (m <= 256).
  static_assert(MAXM <= 256, "one thread per expert");
  int* elist = reinterpret_cast<int*>(sm + L.off_elist);
  int* tab = reinterpret_cast<int*>(sm + L.off_tab);
  int nexp = 0;
  {
    const int e = tid;
    const int c = e < m ? offl[e + 1] - offl[e] : 0;
    const int pc = (c + TQ - 1) / TQ, ne1 = pc > 0 ? 1 : 0;
    // inclusive wave scans of the pass counts and of the non-empty flags
    int ip = pc, in = ne1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int xp = __shfl_up(ip, off, 64), xn = __shfl_up(in, off, 64);
      ip += lane >= off ? xp : 0;
      in += lane >= off ? xn : 0;
    }
    if (lane == 63) {
      scan[w] = ip;
      scan[4 + w] = in;
    }
    __syncthreads();
    // exclusive block prefixes: pe = passes before expert e, ne = non-empty
    // experts before it; T = the head's passes
    int pe = ip - pc, ne = in - ne1, T = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pe += i < w ? scan[i] : 0;
      ne += i < w ? scan[4 + i] : 0;
      T += scan[i];
    }
    const int lo = (int)((long long)part * T / P), hi = (int)((long long)(part + 1) * T / P);
    const int a0 = max(pe, lo), b0 = min(pe + pc, hi);
    const bool ov = pc > 0 && a0 < b0;
    // the experts holding passes lo and hi - 1 bound this workgroup's run
    // of non-empty experts (their ne and ne + 1)
    if (pc > 0 && pe <= lo && lo < pe + pc) scan[8] = ne;
    if (pc > 0 && pe < hi && hi <= pe + pc) scan[9] = ne + 1;
    __syncthreads();
    nexp = lo < hi ? scan[9] - scan[8] : 0;
    if (ov) {
      const int j = ne - scan[8];
      elist[j] = e;
      tab[j * L.ts] = offl[e] + TQ * (a0 - pe);
      tab[j * L.ts + 1] = min(TQ * (b0 - pe), c) - TQ * (a0 - pe);
    }
    __syncthreads();
  }
  const uint16_t* Qh = a.Q + (size_t)bh * N * 64;
  const uint16_t* Kh = a.K + (size_t)bh * N * 64;
  const uint16_t* Vh = a.V + (size_t)bh * N * 64;
  const int32_t* permh = a.perm + (size_t)bh * N * S;
  const int32_t* idxh = a.idx + (size_t)bh * m * k;
  // s = 1: output rows of the queries; s > 1: partial rows of the N * s items
  const Rsrc outr = out_rows(a.out + (size_t)bh * N * S * 64, N * S);
  float2* pmlh = S > 1 ? a.pml + (size_t)bh * N * S : nullptr;
  const u32x4 z = {0u, 0u, 0u, 0u};

  // ---- the segments' table: key ids of each segment's expert (its item
  // range is in place), with every load of a thread issued before any is
  // used
  {
    constexpr int U = 8;
    const int total = nexp * L.ts;
    for (int base = 0; base < total; base += 256 * U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = base + 256 * u + tid;
        v[u] = -1;
        if (it < total) {
          const int j = it / L.ts, o = it - j * L.ts, e = elist[j];
          if (o >= 2) v[u] = idxh[(size_t)e * k + (o - 2)];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = base + 256 * u + tid;
        if (it < total && it - (it / L.ts) * L.ts >= 2) tab[it] = v[u];
      }
    }
  }
  // ---- Q_L (hi / lo) and V_L^T for the head into LDS; rows past m are
  // zero.  (None for route-only.)  Run after the first expert's rows are
  // requested, so that the conversions overlap that latency; the barrier
  // before the first pass publishes them.
  auto store_qv = [&]() {
    for (int base = 0; shared && base < L.mp * 16; base += 256 * 4) {
      if (base > 0) load_qv(base);  // (the first chunk's loads went out at entry)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int it = base + 256 * u + tid, row = it >> 4, q4 = it & 15;
        if (it >= L.mp * 16) break;
        const float f4[4] = {fq[u].x, fq[u].y, fq[u].z, fq[u].w};
        const int off = rc(row, q4 >> 1) + (q4 & 1) * 8;
        if (QL16) {
          *reinterpret_cast<u32x2*>(sm + L.off_qlh + off) =
              u32x2{pk_f16(f4[0], f4[1]), pk_f16(f4[2], f4[3])};
        } else {
          uint32_t h[4], l[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[i] = bf16_rne_bits(f4[i]);
            l[i] = bf16_rne_bits(f4[i] - bf16_bits_to_f32(h[i]));
          }
          *reinterpret_cast<u32x2*>(sm + L.off_qlh + off) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          *reinterpret_cast<u32x2*>(sm + L.off_qll + off) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
        }
        const float vv[4] = {fv[u].x, fv[u].y, fv[u].z, fv[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<uint16_t*>(sm + L.off_vlt + (4 * q4 + i) * L.vlt_stride + 2 * row) =
              (uint16_t)f16_bits(vv[i]);
      }
    }
  };
  __syncthreads();  // the table is complete

  // gather items of this thread: K rows (slots tid>>3 and +32, chunk tid&7)
  // and the V slot pair (2p, 2p+1) of chunk c (p = tid>>3, c = tid&7: eight
  // threads read one 128-byte row)
  const int ksl = tid >> 3, kc = tid & 7;
  const int vp = tid >> 3, vc = tid & 7;
  struct Rows {
    u32x4 k0, k1, v0, v1, q0r, q1r;
    int it0;
  };
  // rows of slots [s0, s0 + 64) of segment j's expert, and (s0 == 0) this
  // lane's first-pass item and the Q row of its query (the item id is
  // requested first, so that the Q row's wait does not cover the key and
  // value rows)
  auto load_rows = [&](int j, int s0, Rows& r) {
    const int* te = tab + j * L.ts;
    const int* ke = te + 2;
    int t = 0;
    if (s0 == 0) {
      const int qi = 16 * w + c16;
      t = qi < te[1] ? permh[te[0] + qi] : 0;
    }
    const int a0 = s0 + ksl, a1 = a0 + 32, b0 = s0 + 2 * vp, b1 = b0 + 1;
    r.k0 = a0 < k ? *reinterpret_cast<const u32x4*>(Kh + (size_t)ke[a0] * 64 + 8 * kc) : z;
    r.k1 = a1 < k ? *reinterpret_cast<const u32x4*>(Kh + (size_t)ke[a1] * 64 + 8 * kc) : z;
    r.v0 = b0 < k ? *reinterpret_cast<const u32x4*>(Vh + (size_t)ke[b0] * 64 + 8 * vc) : z;
    r.v1 = b1 < k ? *reinterpret_cast<const u32x4*>(Vh + (size_t)ke[b1] * 64 + 8 * vc) : z;
    if (s0 == 0) {
      r.it0 = t;
      const int n = S == 1 ? t : t / S;
      r.q0r = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 8 * g);
      r.q1r = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 32 + 8 * g);
    }
  };
  // into LDS slots [base, base + 64)
  auto store_rows = [&](const Rows& r, int base) {
    *reinterpret_cast<u32x4*>(sm + L.off_ke + rc(base + ksl, kc)) = r.k0;
    *reinterpret_cast<u32x4*>(sm + L.off_ke + rc(base + ksl + 32, kc)) = r.k1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 x = h ? r.v1 : r.v0;
      u32x4 f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        f[q] = pk_f16(__uint_as_float(x[q] << 16), __uint_as_float(x[q] & 0xFFFF0000u));
      *reinterpret_cast<u32x4*>(sm + L.off_vet + (base + 2 * vp + h) * EV_STRIDE + 16 * vc) = f;
    }
  };
  // resident slots: segment j's slots past the first 64 (the first chunk is
  // prefetched), up to three chunks' loads issued before any store
  auto stage_rest = [&](int j) {
    for (int s0 = EC; s0 < k; s0 += 3 * EC) {
      Rows r[3];
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (s0 + u * EC < k) load_rows(j, s0 + u * EC, r[u]);
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (s0 + u * EC < k) store_rows(r[u], s0 + u * EC);
    }
  };

  // logits of 32 shared entries (landmarks 32c ..) into x[0..8); -inf for
  // a lane whose item does not take the shared entries (rank j > 0).  (QL16:
  // bq0 / bq1 are the query's channels as f16.)
  auto shared_logits = [&](int c, const u32x4 bq0, const u32x4 bq1, float* x, bool sh) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * c + 16 * h + c16;
      f32x4 s = zero4();
      if (QL16) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, g));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, 4 + g));
        s = mfma_f16(a0, bq0, s);
        s = mfma_f16(a1, bq1, s);
      } else {
        const u32x4 ah0 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, g));
        const u32x4 al0 = *reinterpret_cast<const u32x4*>(sm + L.off_qll + rc(row, g));
        const u32x4 ah1 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, 4 + g));
        const u32x4 al1 = *reinterpret_cast<const u32x4*>(sm + L.off_qll + rc(row, 4 + g));
        s = mfma_bf16(ah0, bq0, s);
        s = mfma_bf16(al0, bq0, s);
        s = mfma_bf16(ah1, bq1, s);
        s = mfma_bf16(al1, bq1, s);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * h + r] = s[r];
    }
    if (32 * c + 32 > m) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * c + 16 * h + 4 * g + r >= m) x[4 * h + r] = -INFINITY;
    }
    if (S > 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = sh ? x[i] : -INFINITY;
    }
  };
  auto shared_av = [&](int c, u32x4 (&av)[4]) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const char* vr = sm + L.off_vlt + (16 * ct + c16) * L.vlt_stride;
      const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + (32 * c + 4 * g) * 2);
      const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + (32 * c + 16 + 4 * g) * 2);
      av[ct] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    }
  };
  // logits of 32 routed entries (expert slots s0 + 32hs .., at LDS slots
  // lb + 32hs ..: lb = s0 when every slot is resident, else 0)
  auto routed_logits = [&](int s0, int lb, int hs, const u32x4 bq0, const u32x4 bq1, float* x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = lb + 32 * hs + 16 * h + c16;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(sm + L.off_ke + rc(row, g));
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(sm + L.off_ke + rc(row, 4 + g));
      f32x4 s = zero4();
      s = mfma_bf16(a0, bq0, s);
      s = mfma_bf16(a1, bq1, s);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * h + r] = s[r];
    }
    if (s0 + 32 * hs + 32 > k) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (s0 + 32 * hs + 16 * h + 4 * g + r >= k) x[4 * h + r] = -INFINITY;
    }
  };
  // V^T[ch 16ct + c16][slots 32hs + 4g .., 32hs + 16 + 4g ..] by transposing
  // reads: lane points at slot 32hs + 4g + (c16 >> 2) (+ 16), channels
  // 16ct + 4 (c16 & 3) ..
  auto routed_av = [&](int lb, int hs, u32x4 (&av)[4]) {
    const char* vr = sm + L.off_vet + (lb + 32 * hs + 4 * g + (c16 >> 2)) * EV_STRIDE + 8 * (c16 & 3);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const u32x2 lo2 = lds_tr16(vr + 32 * ct);
      const u32x2 hi2 = lds_tr16(vr + 16 * EV_STRIDE + 32 * ct);
      av[ct] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    }
  };

  // one pass over <= 64 queries (items) of expert j starting at p0; `item`
  // is this lane's query (s = 1) or (query, rank) item
  auto run_pass = [&](int j, int p0, int item, const u32x4 bq0, const u32x4 bq1) {
    const int* te = tab + j * L.ts;
    const int cnt = te[1];
    const int qi = p0 + 16 * w + c16;
    const bool wave_has = p0 + 16 * w < cnt;
    // (finite: a column whose shared logits are all masked must not make
    // the first rescale exp2(-inf - -inf))
    float mref = -1e30f;
    PassOut o;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o.acc[ct] = zero4();
    f32x4 lsum = zero4();
    // ---- shared entries: landmarks, 64 per softmax update (only rank 0
    // items take them when s > 1)
    const bool sh = shared && (S == 1 || item % S == 0);
    if (wave_has && __ballot(sh) != 0) {
      // (QL16: the query's channels as f16, exact for |q| < 65504)
      u32x4 sq0 = bq0, sq1 = bq1;
      if (QL16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sq0[q] = pk_f16(__uint_as_float(bq0[q] << 16), __uint_as_float(bq0[q] & 0xFFFF0000u));
          sq1[q] = pk_f16(__uint_as_float(bq1[q] << 16), __uint_as_float(bq1[q] & 0xFFFF0000u));
        }
      }
      const int nc = L.mp / 32;
      int c = 0;
      for (; c + 2 <= nc; c += 2) {
        float x[16];
        shared_logits(c, sq0, sq1, x, sh);
        shared_logits(c + 1, sq0, sq1, x + 8, sh);
        softmax_update<2>(x, [&](int i, u32x4 (&av)[4]) { shared_av(c + i, av); }, mref, o.acc,
                          lsum);
      }
      if (c < nc) {
        float x[8];
        shared_logits(c, sq0, sq1, x, sh);
        softmax_update<1>(x, [&](int, u32x4 (&av)[4]) { shared_av(c, av); }, mref, o.acc, lsum);
      }
    }
    // ---- routed entries: the expert's keys, 64 slots per step (from the
    // resident slots, or from an LDS chunk staged for the step)
    for (int s0 = 0; s0 < k; s0 += EC) {
      if (!res && k > EC && (s0 > 0 || p0 > 0)) {
        // slots past the first 64, or a later pass over a multi-chunk expert
        __syncthreads();  // the previous chunk's readers are done
        Rows r;
        load_rows(j, s0, r);
        store_rows(r, 0);
        __syncthreads();
      }
      const int lb = res ? s0 : 0;
      if (wave_has) {
        if (s0 + 32 < k) {
          float x[16];
          routed_logits(s0, lb, 0, bq0, bq1, x);
          routed_logits(s0, lb, 1, bq0, bq1, x + 8);
          softmax_update<2>(x, [&](int i, u32x4 (&av)[4]) { routed_av(lb, i, av); }, mref, o.acc,
                            lsum);
        } else {
          float x[8];
          routed_logits(s0, lb, 0, bq0, bq1, x);
          softmax_update<1>(x, [&](int, u32x4 (&av)[4]) { routed_av(lb, 0, av); }, mref, o.acc,
                            lsum);
        }
      }
    }
    o.live = qi < cnt;
    o.nq = item;
    o.inv = S == 1 ? 1.0f / lsum[0] : 1.0f;  // partials stay unnormalised
    o.mref = mref;
    o.lsum = lsum[0];
    return o;
  };
  // an item's softmax reference and sum, beside its partial row
  auto store_ml = [&](const PassOut& o) {
    if (S > 1 && g == 0 && o.live) pmlh[o.nq] = make_float2(o.mref, o.lsum);
  };

  Rows rows;
  if (nexp > 0) load_rows(0, 0, rows);
  store_qv();
  PassOut pending;
  pending.live = false;
  for (int j = 0; j < nexp; ++j) {
    const int* te = tab + j * L.ts;
    const int q0 = te[0], cnt = te[1];
    if (res) stage_rest(j);
    store_rows(rows, 0);  // waits for this segment's first rows (and the stores before them)
    const u32x4 bq0 = rows.q0r, bq1 = rows.q1r;
    const int it0 = rows.it0;
    // take the Q rows now too: a wait after the stores below would also wait
    // for the stores
    asm volatile("" ::"v"(bq0), "v"(bq1));
    store_out(outr, pending, g, c16);  // the previous expert's last pass
    store_ml(pending);
    pending.live = false;
    if (j + 1 < nexp) load_rows(j + 1, 0, rows);
    __syncthreads();
    if (cnt > 0) {
      PassOut o = run_pass(j, 0, it0, bq0, bq1);
      for (int p0 = TQ; p0 < cnt; p0 += TQ) {
        // later passes: query ids and Q rows straight from global memory
        store_out(outr, o, g, c16);
        store_ml(o);
        const int qi = p0 + 16 * w + c16;
        const int it = qi < cnt ? permh[q0 + qi] : 0;
        const int nq = S == 1 ? it : it / S;
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(Qh + (size_t)nq * 64 + 8 * g);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(Qh + (size_t)nq * 64 + 32 + 8 * g);
        o = run_pass(j, p0, it, b0, b1);
      }
      pending = o;
    }
    __syncthreads();  // readers of this expert's rows are done
  }
  store_out(outr, pending, g, c16);
  store_ml(pending);
}

// s > 1: out_n = sum_j acc_j 2^((M_j - M) tau log2e) / sum_j l_j 2^(...), over
// the query's s items (acc_j, M_j, l_j from the attention kernel), M the
// largest M_j.  One thread per (query, 4 channels).
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part,
                                                    const float2* __restrict__ pml,
                                                    float* __restrict__ out, long long nq, int s) {
  constexpr float cs = 0.125f * 1.4426950408889634f;  // tau * log2(e)
  const long long it = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long n = it >> 4;
  const int c4 = (int)(it & 15) * 4;
  if (n >= nq) return;
  float M = -INFINITY;
  for (int j = 0; j < s; ++j) M = fmaxf(M, pml[n * s + j].x);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.f;
  for (int j = 0; j < s; ++j) {
    const float2 ml = pml[n * s + j];
    const float f = __builtin_amdgcn_exp2f((ml.x - M) * cs);
    const float4 v = *reinterpret_cast<const float4*>(part + (n * s + j) * 64 + c4);
    o.x = fmaf(f, v.x, o.x);
    o.y = fmaf(f, v.y, o.y);
    o.z = fmaf(f, v.z, o.z);
    o.w = fmaf(f, v.w, o.w);
    l = fmaf(f, ml.y, l);
  }
  const float inv = 1.0f / l;
  *reinterpret_cast<float4*>(out + n * 64 + c4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

}  // namespace att

bool attend_bf16_supported(const Shape& s) {
  // the partial rows of the N * s items are addressed by 32-bit byte offsets
  return s.bf16 && s.m <= att::MAXM && (long long)s.N * s.s <= (1 << 22);
}

size_t attend_partial_bytes(const Shape& s) {
  if (s.s == 1) return 0;
  return (size_t)s.BH * s.N * s.s * (64 * 4 + 8);
}

static int attend_parts(const Shape& s) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  // about three resident workgroups per CU in total, at least one per head,
  // no more than the head can have passes
  int parts = (3 * ncu + s.BH - 1) / s.BH;
  const int tmax = att::max_passes(s.m, s.N, s.s);
  if (parts > tmax) parts = tmax;
  if (parts < 1) parts = 1;
  return parts;
}

namespace {
struct AttCfg {
  int parts, kres, bytes;
  bool ql16;
};
}  // namespace

// The LDS layout: the one that leaves the most resident workgroups per CU (up
// to the three the register budget allows); on a tie, all of an expert's
// slots resident before 64-slot chunks re-staged per pass, and Q_L as bf16
// hi + lo before one f16 copy.  A layout that does not fit may take more
// workgroups per head (a smaller segment table): up to twice as many for the
// resident layouts, as many as the head has passes for the chunked one.
static AttCfg attend_config(const Shape& s) {
  constexpr int cap = 160 * 1024;
  const int base = attend_parts(s), tmax = att::max_passes(s.m, s.N, s.s);
  const int kfull = (s.k + att::EC - 1) / att::EC * att::EC;
  struct Opt {
    bool ql16;
    int kres, pmax;
  };
  const int p2 = 2 * base < tmax ? 2 * base : tmax;
  const Opt opts[3] = {{false, kfull, p2}, {true, kfull, p2}, {false, att::EC, tmax}};
  AttCfg best{0, 0, 0, false};
  int best_occ = 0;
  for (const Opt& o : opts) {
    int p = base;
    while (att::Lay(s.m, s.k, p, tmax, o.ql16, o.kres).bytes > cap && p < o.pmax) ++p;
    const int bytes = att::Lay(s.m, s.k, p, tmax, o.ql16, o.kres).bytes;
    if (bytes > cap) continue;
    const int occ = cap / bytes < 3 ? cap / bytes : 3;
    if (occ > best_occ) {
      best_occ = occ;
      best = AttCfg{p, o.kres, bytes, o.ql16};
    }
  }
  return best;  // parts == 0: no layout fits
}

hipError_t launch_attend_bf16(const void* Q, const void* K, const void* V, const float* ql,
                              const float* vl, const int32_t* idx, const int32_t* offsets,
                              const int32_t* perm, float* out, void* partial, const Shape& s,
                              hipStream_t st) {
  const AttCfg c = attend_config(s);
  if (c.parts == 0) return hipErrorInvalidValue;
  // (f16 Q_L is only chosen with resident slots: three instances)
  const bool res = c.kres > att::EC;
  auto kernel = c.ql16 ? att::attend_bf16_kernel<true, true>
                : res  ? att::attend_bf16_kernel<false, true>
                       : att::attend_bf16_kernel<false, false>;
  const int form = c.ql16 ? 2 : res ? 1 : 0;
  static std::atomic<unsigned long long> lds_set[3];
  if (const hipError_t e = allow_lds((const void*)kernel, 160 * 1024, lds_set[form]);
      e != hipSuccess)
    return e;
  if (s.s > 1 && !partial) return hipErrorInvalidValue;
  float* part = s.s > 1 ? (float*)partial : out;
  float2* pml = s.s > 1 ? (float2*)((char*)partial + (size_t)s.BH * s.N * s.s * 64 * 4) : nullptr;
  att::Args a{(const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, ql, vl, idx, offsets,
              perm, part, pml, s.BH, s.N, s.m, s.k, c.parts, s.s, s.shared ? 1 : 0, c.kres};
  const int grid = s.BH >= 8 ? ((s.BH + 7) / 8) * 8 * c.parts : s.BH * c.parts;
  kernel<<<grid, 256, c.bytes, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_merge(const void* partial, float* out, const Shape& s, hipStream_t st) {
  const long long nq = (long long)s.BH * s.N;
  const float* part = (const float*)partial;
  const float2* pml = (const float2*)((const char*)partial + (size_t)nq * s.s * 64 * 4);
  const long long threads = nq * 16;
  att::merge_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(part, pml, out, nq, s.s);
  return hipGetLastError();
}

}  // namespace mita
