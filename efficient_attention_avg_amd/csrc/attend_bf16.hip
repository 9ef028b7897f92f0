// Step a7 for bf16 inputs on long grids -- grouped expert attention (page
// "NeurIPS'26：注意力也是FFN？...", the s = 1 output and Algorithm 1: queries
// grouped by route attend their expert's k raw key/value pairs and the m
// shared ones under one softmax; partial results merge by online softmax).
//
// Persistent workgroups, P per head, placed on the head's XCD so the head's
// K, V and Q rows are re-read from that XCD's L2.  A head's experts are dealt
// to its P workgroups in a snake, largest pass count first.  Per workgroup:
//   * load its experts' table (query range, key ids, first 64 query ids)
//     and the head's Q_L (bf16 hi + lo) and V_L^T (f16) into LDS once;
//   * per expert: its k key rows (bf16) and value rows (f16, transposed) sit
//     in LDS, shared by the four waves.  While one expert is computed the
//     next one's rows (and the Q rows of its first 64 queries) are already
//     loading into registers; the expert's output stores are issued only
//     after those rows have been waited for, since stores and loads drain
//     through one counter.  For k > 64 the slots past the first 64 are
//     gathered in place, 64 at a time;
//   * per pass of <= 64 of the expert's queries, each wave owns 16: Q rows
//     are the B operand of logits^T = [Q_L; K_e] Q^T; an online softmax runs
//     over 32-entry chunks (shared entries first, then the expert's keys), and
//     each chunk's weights go straight from the logit accumulators into
//     out^T += [V_L; V_e]^T P^T on f16 MFMA, with the normaliser from an
//     all-ones MFMA.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace mita {
namespace att {

constexpr int TQ = 64;    // queries per pass (16 per wave)
constexpr int EC = 64;    // expert slots per LDS chunk
constexpr int EVT_STRIDE = EC * 2 + 16;
constexpr int MAXM = 256;

__device__ __forceinline__ int rc(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

struct Args {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const float* ql;
  const float* vl;
  const int32_t* idx;
  const int32_t* offsets;
  const int32_t* perm;
  float* out;
  int BH, N, m, k, parts;  // workgroups per head
};

// LDS layout; the expert table holds, per expert of the workgroup,
// [q0, count, k key ids, first TQ query ids].
struct Lay {
  int mp, vlt_stride, ew, ts;
  int off_qlh, off_qll, off_vlt, off_ke, off_vet, off_tab, off_elist, bytes;
  __host__ __device__ Lay(int m, int k, int parts) {
    mp = (m + 31) & ~31;
    vlt_stride = mp * 2 + 16;
    ew = (m + parts - 1) / parts;
    ts = 2 + k + TQ;
    off_qlh = 0;
    off_qll = off_qlh + mp * 128;
    off_vlt = off_qll + mp * 128;
    off_ke = off_vlt + 64 * vlt_stride;
    off_vet = off_ke + EC * 128;
    off_tab = off_vet + 64 * EVT_STRIDE;
    off_elist = off_tab + ew * ts * 4;
    bytes = off_elist + (ew + 1) * 4;
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

// A pass's result for this lane's query, written to out row nq when live.
struct PassOut {
  f32x4 acc[4];
  float inv;
  int nq;
  bool live;
};

// Lane c16 <-> c16 ^ 8 of each 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ int swap8(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);
}
__device__ __forceinline__ f32x4 swap8(f32x4 v) {
  // (element by value: a bit cast applied to the element expression v[i]
  // itself was compiled as a read of element 0)
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __int_as_float(swap8(__float_as_int(v[i])));
  return r;
}

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

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attend_bf16_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const Lay L(a.m, a.k, a.parts);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int bh = xcd + 8 * (slot / a.parts), part = slot % a.parts;
  if (bh >= a.BH || part >= a.m) return;
  const int N = a.N, m = a.m, k = a.k, P = a.parts;
  // The head's experts are dealt to its P workgroups in a snake (0, 1, ..,
  // P-1, P-1, .., 0, ...) in order of their passes (then queries, then id),
  // largest first, so that the workgroups' pass totals even out; every
  // workgroup of the head computes the same deal.
  int* elist = reinterpret_cast<int*>(sm + L.off_elist);
  {
    int* ecnt = reinterpret_cast<int*>(sm + L.off_tab);  // (the table is filled after)
    for (int e = tid; e < m; e += blockDim.x) ecnt[e] = a.offsets[(size_t)bh * (m + 1) + e + 1] -
                                                      a.offsets[(size_t)bh * (m + 1) + e];
    __syncthreads();
    for (int e = tid; e < m; e += blockDim.x) {
      const int c = ecnt[e], pc = (c + TQ - 1) / TQ;
      int rank = 0;
      for (int e2 = 0; e2 < m; ++e2) {
        const int c2 = ecnt[e2], p2 = (c2 + TQ - 1) / TQ;
        rank += (p2 > pc || (p2 == pc && (c2 > c || (c2 == c && e2 < e)))) ? 1 : 0;
      }
      const int round = rank / P, pos = rank - round * P;
      if (((round & 1) ? P - 1 - pos : pos) == part) elist[round] = e;
    }
    __syncthreads();
  }
  // this workgroup's experts: one per full round, plus one in the last
  // (partial) round when the deal reaches it there
  const int full = m / P, rest = m - full * P;
  const int nexp = full + ((full & 1) ? (part >= P - rest ? 1 : 0) : (part < rest ? 1 : 0));
  const uint16_t* Qh = a.Q + (size_t)bh * N * 64;
  const uint16_t* Kh = a.K + (size_t)bh * N * 64;
  const uint16_t* Vh = a.V + (size_t)bh * N * 64;
  const int32_t* offs = a.offsets + (size_t)bh * (m + 1);
  const int32_t* permh = a.perm + (size_t)bh * N;
  const int32_t* idxh = a.idx + (size_t)bh * m * k;
  const Rsrc outr = out_rows(a.out + (size_t)bh * N * 64, N);
  int* tab = reinterpret_cast<int*>(sm + L.off_tab);
  const u32x4 z = {0u, 0u, 0u, 0u};

  // ---- the experts' table: query ranges first, then key ids and first
  // query ids with every load of a thread issued before any is used
  if (tid < nexp) {
    const int e = elist[tid];
    const int q0 = offs[e];
    tab[tid * L.ts] = q0;
    tab[tid * L.ts + 1] = offs[e + 1] - q0;
  }
  __syncthreads();
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
          if (o >= 2 && o < 2 + k) {
            v[u] = idxh[(size_t)e * k + (o - 2)];
          } else if (o >= 2 + k) {
            const int q0 = tab[j * L.ts], cnt = tab[j * L.ts + 1];
            if (o - 2 - k < cnt) v[u] = permh[q0 + (o - 2 - k)];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = base + 256 * u + tid;
        if (it < total && it - (it / L.ts) * L.ts >= 2) tab[it] = v[u];
      }
    }
  }
  // ---- Q_L (hi / lo) and V_L^T for the head; rows past m are zero.  All of
  // a thread's loads go out before any is used.
  for (int base = 0; base < L.mp * 16; base += 256 * 4) {
    float4 fq[4], fv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = base + 256 * u + tid, row = it >> 4, q4 = it & 15;
      fq[u] = fv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (it < L.mp * 16 && row < m) {
        fq[u] = *reinterpret_cast<const float4*>(a.ql + ((size_t)bh * m + row) * 64 + 4 * q4);
        fv[u] = *reinterpret_cast<const float4*>(a.vl + ((size_t)bh * m + row) * 64 + 4 * q4);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int it = base + 256 * u + tid, row = it >> 4, q4 = it & 15;
      if (it >= L.mp * 16) break;
      const float f4[4] = {fq[u].x, fq[u].y, fq[u].z, fq[u].w};
      uint32_t h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = bf16_rne_bits(f4[i]);
        l[i] = bf16_rne_bits(f4[i] - bf16_bits_to_f32(h[i]));
      }
      const int off = rc(row, q4 >> 1) + (q4 & 1) * 8;
      *reinterpret_cast<u32x2*>(sm + L.off_qlh + off) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *reinterpret_cast<u32x2*>(sm + L.off_qll + off) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      const float vv[4] = {fv[u].x, fv[u].y, fv[u].z, fv[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint16_t*>(sm + L.off_vlt + (4 * q4 + i) * L.vlt_stride + 2 * row) =
            (uint16_t)f16_bits(vv[i]);
    }
  }
  __syncthreads();

  // gather items of this thread: K rows (slots tid>>3 and +32, chunk tid&7)
  // and the V slot pair (2p, 2p+1) of chunk c
  const int ksl = tid >> 3, kc = tid & 7;
  const int vp = tid & 31, vc = tid >> 5;
  struct Rows {
    u32x4 k0, k1, v0, v1, q0r, q1r;
  };
  // rows of slots [s0, s0 + 64) of expert j, and (s0 == 0) the Q row of this
  // lane's first-pass query
  auto load_rows = [&](int j, int s0, Rows& r) {
    const int* te = tab + j * L.ts;
    const int* ke = te + 2;
    const int a0 = s0 + ksl, a1 = a0 + 32, b0 = s0 + 2 * vp, b1 = b0 + 1;
    r.k0 = a0 < k ? *reinterpret_cast<const u32x4*>(Kh + (size_t)ke[a0] * 64 + 8 * kc) : z;
    r.k1 = a1 < k ? *reinterpret_cast<const u32x4*>(Kh + (size_t)ke[a1] * 64 + 8 * kc) : z;
    r.v0 = b0 < k ? *reinterpret_cast<const u32x4*>(Vh + (size_t)ke[b0] * 64 + 8 * vc) : z;
    r.v1 = b1 < k ? *reinterpret_cast<const u32x4*>(Vh + (size_t)ke[b1] * 64 + 8 * vc) : z;
    if (s0 == 0) {
      const int n = max(te[2 + k + 16 * w + c16], 0);
      r.q0r = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 8 * g);
      r.q1r = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 32 + 8 * g);
    }
  };
  auto store_rows = [&](const Rows& r) {
    *reinterpret_cast<u32x4*>(sm + L.off_ke + rc(ksl, kc)) = r.k0;
    *reinterpret_cast<u32x4*>(sm + L.off_ke + rc(ksl + 32, kc)) = r.k1;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t x0 = (r.v0[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      const uint32_t x1 = (r.v1[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
      *reinterpret_cast<uint32_t*>(sm + L.off_vet + (8 * vc + q) * EVT_STRIDE + 4 * vp) =
          pk_f16(bf16_bits_to_f32(x0), bf16_bits_to_f32(x1));
    }
  };

  // logits of 32 shared entries (landmarks 32c ..) into x[0..8)
  auto shared_logits = [&](int c, const u32x4 bq0, const u32x4 bq1, float* x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * c + 16 * h + c16;
      const u32x4 ah0 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, g));
      const u32x4 al0 = *reinterpret_cast<const u32x4*>(sm + L.off_qll + rc(row, g));
      const u32x4 ah1 = *reinterpret_cast<const u32x4*>(sm + L.off_qlh + rc(row, 4 + g));
      const u32x4 al1 = *reinterpret_cast<const u32x4*>(sm + L.off_qll + rc(row, 4 + g));
      f32x4 s = zero4();
      s = mfma_bf16(ah0, bq0, s);
      s = mfma_bf16(al0, bq0, s);
      s = mfma_bf16(ah1, bq1, s);
      s = mfma_bf16(al1, bq1, s);
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
  // logits of 32 routed entries (LDS slots 32hs .., expert slots s0 + 32hs ..)
  auto routed_logits = [&](int s0, int hs, const u32x4 bq0, const u32x4 bq1, float* x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * hs + 16 * h + c16;
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
  auto routed_av = [&](int hs, u32x4 (&av)[4]) {
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const char* vr = sm + L.off_vet + (16 * ct + c16) * EVT_STRIDE;
      const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + (32 * hs + 4 * g) * 2);
      const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + (32 * hs + 16 + 4 * g) * 2);
      av[ct] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    }
  };

  // one pass over <= 64 queries of expert j starting at p0
  auto run_pass = [&](int j, int p0, int nq, const u32x4 bq0, const u32x4 bq1) {
    const int* te = tab + j * L.ts;
    const int cnt = te[1];
    const int qi = p0 + 16 * w + c16;
    const bool wave_has = p0 + 16 * w < cnt;
    float mref = -INFINITY;
    PassOut o;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o.acc[ct] = zero4();
    f32x4 lsum = zero4();
    // ---- shared entries: landmarks, 64 per softmax update
    if (wave_has) {
      const int nc = L.mp / 32;
      int c = 0;
      for (; c + 2 <= nc; c += 2) {
        float x[16];
        shared_logits(c, bq0, bq1, x);
        shared_logits(c + 1, bq0, bq1, x + 8);
        softmax_update<2>(x, [&](int i, u32x4 (&av)[4]) { shared_av(c + i, av); }, mref, o.acc,
                          lsum);
      }
      if (c < nc) {
        float x[8];
        shared_logits(c, bq0, bq1, x);
        softmax_update<1>(x, [&](int, u32x4 (&av)[4]) { shared_av(c, av); }, mref, o.acc, lsum);
      }
    }
    // ---- routed entries: the expert's keys, 64 slots per LDS chunk
    for (int s0 = 0; s0 < k; s0 += EC) {
      if (k > EC && (s0 > 0 || p0 > 0)) {
        // slots past the first 64, or a later pass over a multi-chunk expert
        __syncthreads();  // the previous chunk's readers are done
        Rows r;
        load_rows(j, s0, r);
        store_rows(r);
        __syncthreads();
      }
      if (wave_has) {
        if (s0 + 32 < k) {
          float x[16];
          routed_logits(s0, 0, bq0, bq1, x);
          routed_logits(s0, 1, bq0, bq1, x + 8);
          softmax_update<2>(x, [&](int i, u32x4 (&av)[4]) { routed_av(i, av); }, mref, o.acc,
                            lsum);
        } else {
          float x[8];
          routed_logits(s0, 0, bq0, bq1, x);
          softmax_update<1>(x, [&](int, u32x4 (&av)[4]) { routed_av(0, av); }, mref, o.acc, lsum);
        }
      }
    }
    o.live = qi < cnt;
    o.nq = nq;
    o.inv = 1.0f / lsum[0];
    return o;
  };

  Rows rows;
  if (nexp > 0) load_rows(0, 0, rows);
  PassOut pending;
  pending.live = false;
  for (int j = 0; j < nexp; ++j) {
    const int* te = tab + j * L.ts;
    const int q0 = te[0], cnt = te[1];
    store_rows(rows);  // waits for this expert's rows (and the stores before them)
    const u32x4 bq0 = rows.q0r, bq1 = rows.q1r;
    // take the Q rows now too: a wait after the stores below would also wait
    // for the stores
    asm volatile("" ::"v"(bq0), "v"(bq1));
    store_out(outr, pending, g, c16);  // the previous expert's last pass
    pending.live = false;
    if (j + 1 < nexp) load_rows(j + 1, 0, rows);
    __syncthreads();
    if (cnt > 0) {
      const int n0 = te[2 + k + 16 * w + c16];
      PassOut o = run_pass(j, 0, max(n0, 0), bq0, bq1);
      for (int p0 = TQ; p0 < cnt; p0 += TQ) {
        // later passes: query ids and Q rows straight from global memory
        store_out(outr, o, g, c16);
        const int qi = p0 + 16 * w + c16;
        const int nq = qi < cnt ? permh[q0 + qi] : 0;
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(Qh + (size_t)nq * 64 + 8 * g);
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(Qh + (size_t)nq * 64 + 32 + 8 * g);
        o = run_pass(j, p0, nq, b0, b1);
      }
      pending = o;
    }
    __syncthreads();  // readers of this expert's rows are done
  }
  store_out(outr, pending, g, c16);
}

}  // namespace att

bool attend_bf16_supported(const Shape& s) {
  return s.bf16 && s.m <= att::MAXM;
}

static int attend_parts(const Shape& s) {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  // about three resident workgroups per CU in total, at least one per head,
  // at most one per expert
  int parts = (3 * ncu + s.BH - 1) / s.BH;
  if (parts > s.m) parts = s.m;
  if (parts < 1) parts = 1;
  return parts;
}

hipError_t launch_attend_bf16(const void* Q, const void* K, const void* V, const float* ql,
                              const float* vl, const int32_t* idx, const int32_t* offsets,
                              const int32_t* perm, float* out, const Shape& s, hipStream_t st) {
  int parts = attend_parts(s);
  // the table must fit next to the rest: fewer experts per workgroup if not
  while (att::Lay(s.m, s.k, parts).bytes > 160 * 1024 && parts < s.m) ++parts;
  const att::Lay L(s.m, s.k, parts);
  if (L.bytes > 160 * 1024) return hipErrorInvalidValue;
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)att::attend_bf16_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  att::Args a{(const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, ql, vl, idx, offsets,
              perm, out, s.BH, s.N, s.m, s.k, parts};
  const int grid = ((s.BH + 7) / 8) * 8 * parts;
  att::attend_bf16_kernel<<<grid, 256, L.bytes, st>>>(a);
  return hipGetLastError();
}

}  // namespace mita
