// Step a7 for bf16 inputs on long grids -- grouped expert attention (page
// "NeurIPS'26：注意力也是FFN？...", the s = 1 output and Algorithm 1: queries
// grouped by route attend their expert's k raw key/value pairs and the m
// shared ones under one softmax; partial results merge by online softmax).
//
// Persistent workgroups, several per head, placed on the head's XCD so the
// head's K, V and Q rows are re-read from that XCD's L2.  Per workgroup:
//   * stage the head's Q_L (bf16 hi + lo) and V_L^T (f16) once;
//   * derive the tile list from the group offsets: tiles of <= 64 queries of
//     one expert; the workgroup takes tiles p, p + P, ...;
//   * per tile, each wave owns 16 queries: Q rows are the B operand of
//     logits^T = [Q_L; K_e] Q^T; an online softmax runs over 32-entry chunks
//     (shared entries first, then the expert's keys), and each chunk's weights
//     go straight from the logit accumulators into out^T += [V_L; V_e]^T P^T
//     on f16 MFMA, with the normaliser from an all-ones MFMA;
//   * the expert's K rows (bf16) and V rows (f16, transposed) are gathered
//     into LDS 64 slots at a time and shared by the four waves.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace mita {
namespace att {

constexpr int TQ = 64;    // queries per tile (16 per wave)
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
  int BH, N, m, k, parts;
};

struct Lay {
  int mp, vlt_stride;
  int off_qlh, off_qll, off_vlt, off_ke, off_vet, off_tstart, bytes;
  __host__ __device__ Lay(int m) {
    mp = (m + 31) & ~31;
    vlt_stride = mp * 2 + 16;
    off_qlh = 0;
    off_qll = off_qlh + mp * 128;
    off_vlt = off_qll + mp * 128;
    off_ke = off_vlt + 64 * vlt_stride;
    off_vet = off_ke + EC * 128;
    off_tstart = off_vet + 64 * EVT_STRIDE;
    bytes = off_tstart + (MAXM + 1) * 4;
  }
};

// One 32-entry chunk of the online softmax for this lane's query column.
// x: base-2 logits of entries {4g+r, 16+4g+r} (-inf when masked); av: the
// chunk's A fragments of [V_L; V_e]^T for the four channel tiles.
__device__ __forceinline__ void chunk_update(const float (&x)[8], const u32x4 (&av)[4], float& mx,
                                             f32x4 (&acc)[4], f32x4& lsum) {
  float cm = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) cm = fmaxf(cm, x[i]);
  cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
  cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
  const float mnew = fmaxf(mx, cm);
  const float alpha = __builtin_amdgcn_exp2f(mx - mnew);
  mx = mnew;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
  const u32x4 bp = {pk_f16(p[0], p[1]), pk_f16(p[2], p[3]), pk_f16(p[4], p[5]), pk_f16(p[6], p[7])};
  const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma_f16(av[ct], bp, acc[ct] * alpha);
  lsum = mfma_f16(ones, bp, lsum * alpha);
}

__global__ __launch_bounds__(256) void attend_bf16_kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const Lay L(a.m);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int bh = xcd + 8 * (slot / a.parts), part = slot % a.parts;
  if (bh >= a.BH) return;
  const int N = a.N, m = a.m, k = a.k;
  const float cs = 0.125f * 1.4426950408889634f;  // tau * log2(e)

  // ---- stage Q_L (hi / lo) and V_L^T for the head; rows past m are zero
  for (int it = tid; it < L.mp * 16; it += 256) {
    const int row = it >> 4, q4 = it & 15;
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f), v = f;
    if (row < m) {
      f = *reinterpret_cast<const float4*>(a.ql + ((size_t)bh * m + row) * 64 + 4 * q4);
      v = *reinterpret_cast<const float4*>(a.vl + ((size_t)bh * m + row) * 64 + 4 * q4);
    }
    const float fv[4] = {f.x, f.y, f.z, f.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = bf16_rne_bits(fv[i]);
      l[i] = bf16_rne_bits(fv[i] - bf16_bits_to_f32(h[i]));
    }
    const int off = rc(row, q4 >> 1) + (q4 & 1) * 8;
    *reinterpret_cast<u32x2*>(sm + L.off_qlh + off) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *reinterpret_cast<u32x2*>(sm + L.off_qll + off) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint16_t*>(sm + L.off_vlt + (4 * q4 + i) * L.vlt_stride + 2 * row) =
          (uint16_t)f16_bits(vv[i]);
  }
  // ---- tile list: expert e owns tiles tstart[e] .. tstart[e+1]-1
  const int32_t* offs = a.offsets + (size_t)bh * (m + 1);
  int* tstart = reinterpret_cast<int*>(sm + L.off_tstart);
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < m; ++e) {
      tstart[e] = run;
      run += (offs[e + 1] - offs[e] + TQ - 1) / TQ;
    }
    tstart[m] = run;
  }
  __syncthreads();
  const int ntiles = tstart[m];
  const uint16_t* Qh = a.Q + (size_t)bh * N * 64;
  const uint16_t* Kh = a.K + (size_t)bh * N * 64;
  const uint16_t* Vh = a.V + (size_t)bh * N * 64;
  const int32_t* permh = a.perm + (size_t)bh * N;
  float* outh = a.out + (size_t)bh * N * 64;

  for (int t = part; t < ntiles; t += a.parts) {
    // expert of tile t: the last e with tstart[e] <= t (binary search)
    int lo = 0, hi = m - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tstart[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int q0 = offs[e] + (t - tstart[e]) * TQ;
    const int len = min(TQ, offs[e + 1] - q0);
    const int32_t* keys_e = a.idx + ((size_t)bh * m + e) * k;
    // this lane's query (column c16 of wave w's 16)
    const int qi = 16 * w + c16;
    const bool live = qi < len;
    const bool wave_has = 16 * w < len;
    const int n = live ? permh[q0 + qi] : 0;
    const u32x4 bq0 = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 8 * g);
    const u32x4 bq1 = *reinterpret_cast<const u32x4*>(Qh + (size_t)n * 64 + 32 + 8 * g);
    float mx = -INFINITY;
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
    f32x4 lsum = zero4();

    // ---- shared entries: landmarks, 32 at a time
    if (wave_has) {
      for (int c = 0; c < L.mp / 32; ++c) {
        float x[8];
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
          for (int r = 0; r < 4; ++r)
            x[4 * h + r] = (32 * c + 16 * h + 4 * g + r) < m ? s[r] * cs : -INFINITY;
        }
        u32x4 av[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const char* vr = sm + L.off_vlt + (16 * ct + c16) * L.vlt_stride;
          const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + (32 * c + 4 * g) * 2);
          const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + (32 * c + 16 + 4 * g) * 2);
          av[ct] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        }
        chunk_update(x, av, mx, acc, lsum);
      }
    }
    // ---- routed entries: the expert's keys, gathered 64 slots at a time
    for (int s0 = 0; s0 < k; s0 += EC) {
      __syncthreads();  // the previous chunk's readers are done
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int id = tid + 256 * i, sl = id >> 3, c = id & 7;
        const bool ok = s0 + sl < k;
        const int key = ok ? keys_e[s0 + sl] : 0;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm + L.off_ke + rc(sl, c)) =
            ok ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * 64 + 8 * c) : z;
      }
      {
        const int p = tid & 31, c = tid >> 5;  // slot pair (2p, 2p+1), 8-channel chunk
        const bool ok0 = s0 + 2 * p < k, ok1 = s0 + 2 * p + 1 < k;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 v0 = ok0 ? *reinterpret_cast<const u32x4*>(Vh + (size_t)keys_e[s0 + 2 * p] * 64 + 8 * c) : z;
        const u32x4 v1 = ok1 ? *reinterpret_cast<const u32x4*>(Vh + (size_t)keys_e[s0 + 2 * p + 1] * 64 + 8 * c) : z;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t x0 = (v0[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
          const uint32_t x1 = (v1[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
          *reinterpret_cast<uint32_t*>(sm + L.off_vet + (8 * c + q) * EVT_STRIDE + 4 * p) =
              pk_f16(bf16_bits_to_f32(x0), bf16_bits_to_f32(x1));
        }
      }
      __syncthreads();
      if (wave_has) {
        for (int hs = 0; hs < 2 && s0 + 32 * hs < k; ++hs) {
          float x[8];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = 32 * hs + 16 * h + c16;
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(sm + L.off_ke + rc(row, g));
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(sm + L.off_ke + rc(row, 4 + g));
            f32x4 s = zero4();
            s = mfma_bf16(a0, bq0, s);
            s = mfma_bf16(a1, bq1, s);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              x[4 * h + r] = (s0 + 32 * hs + 16 * h + 4 * g + r) < k ? s[r] * cs : -INFINITY;
          }
          u32x4 av[4];
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const char* vr = sm + L.off_vet + (16 * ct + c16) * EVT_STRIDE;
            const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vr + (32 * hs + 4 * g) * 2);
            const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vr + (32 * hs + 16 + 4 * g) * 2);
            av[ct] = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          }
          chunk_update(x, av, mx, acc, lsum);
        }
      }
    }
    if (live) {
      const float inv = 1.0f / lsum[0];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        *reinterpret_cast<float4*>(outh + (size_t)n * 64 + 16 * ct + 4 * g) =
            make_float4(acc[ct][0] * inv, acc[ct][1] * inv, acc[ct][2] * inv, acc[ct][3] * inv);
    }
  }
}

}  // namespace att

bool attend_bf16_supported(const Shape& s) { return s.bf16 && s.m <= att::MAXM; }

hipError_t launch_attend_bf16(const void* Q, const void* K, const void* V, const float* ql,
                              const float* vl, const int32_t* idx, const int32_t* offsets,
                              const int32_t* perm, float* out, const Shape& s, hipStream_t st) {
  const att::Lay L(s.m);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)att::attend_bf16_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr = true;
  }
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  // about six workgroups per CU in total (several resident per CU keep more
  // gathers in flight), at least one per head
  int parts = (6 * ncu + s.BH - 1) / s.BH;
  if (parts < 1) parts = 1;
  att::Args a{(const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, ql, vl, idx, offsets,
              perm, out, s.BH, s.N, s.m, s.k, parts};
  const int grid = ((s.BH + 7) / 8) * 8 * parts;
  att::attend_bf16_kernel<<<grid, 256, L.bytes, st>>>(a);
  return hipGetLastError();
}

}  // namespace mita
