// Exact top-k selection inside a 16-lane group (one row per group), for
// values held in registers: lane t holds entries e = t + 16u, u < NV.
//
// Order: larger value first; equal values go to the smaller key id.  The
// routine narrows the candidate set with 256-bin histograms over the
// candidates' current value range (linear bins are monotone in the value, so
// every bin above the one holding the need-th candidate is taken whole);
// when every remaining candidate has the same value, it selects the smallest
// key ids the same way on -key.  Each pass drops at least the range's
// minimum or maximum, so the loop ends.
#pragma once

#include "common.h"
#include "mfma.h"

namespace mita {

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
// quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror: after these four
// steps every lane of a 16-lane row holds the row's reduction.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// row_shl:n gives lane t the value of lane t+n of its row (zero past the end)
constexpr int kDppShl1 = 0x101, kDppShl2 = 0x102, kDppShl4 = 0x104, kDppShl8 = 0x108;

__device__ __forceinline__ float g16_maxf(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float g16_minf(float v) {
  v = fminf(v, dpp_f<kDppXor1>(v));
  v = fminf(v, dpp_f<kDppXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  return fminf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ int g16_addi(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  return v + dpp_i<kDppMirror>(v);
}
// inclusive suffix sum over the row: lane t gets sum over t' >= t
__device__ __forceinline__ int g16_suffix(int v) {
  v += dpp_i<kDppShl1>(v);
  v += dpp_i<kDppShl2>(v);
  v += dpp_i<kDppShl4>(v);
  return v + dpp_i<kDppShl8>(v);
}
__device__ __forceinline__ uint32_t g16_ballot(bool p, int g) {
  return (uint32_t)(__ballot(p) >> (16 * g)) & 0xFFFFu;
}

// Selects the `need` best of the candidate entries (bit u of `cand` marks
// entry t + 16u) and returns them as a mask.  `x` is scratch (overwritten),
// initialised by the caller to the values; `key` are the entries' key ids
// (distinct, < 2^24).  `hist` is 512 bytes of this group's LDS.  Every lane
// of the wave must call this together (groups may differ in their work, but
// all 16 lanes of a group always take the same branches).
template <int NV>
__device__ uint32_t group_topk(float (&x)[NV], const int (&key)[NV], uint32_t cand, int need,
                               char* hist, int t, int g) {
  uint32_t take = 0;
  // `done` must be the same on all 16 lanes of the group: the DPP reductions
  // below read every lane of the row, and a lane outside the active mask
  // would contribute 0 instead of its value
  bool done = need <= 0 || g16_addi(__popc(cand)) == 0;
  bool keymode = false;
  const uint32_t below = (1u << t) - 1u;
  auto range = [&](float& lo, float& hi) {
    float a = INFINITY, b = -INFINITY;
#pragma unroll
    for (int u = 0; u < NV; ++u)
      if (cand >> u & 1u) { a = fminf(a, x[u]); b = fmaxf(b, x[u]); }
    lo = g16_minf(a);
    hi = g16_maxf(b);
  };
  float lo, hi;
  range(lo, hi);
  for (int pass = 0; pass < 200; ++pass) {
    const int cc = g16_addi(__popc(cand));
    if (!done) {
      if (need >= cc) {
        take |= cand;
        cand = 0u;
        done = true;
      } else if (!(hi > lo) && !keymode) {
        // every candidate has the same value: keep the smallest key ids
        keymode = true;
#pragma unroll
        for (int u = 0; u < NV; ++u)
          if (cand >> u & 1u) x[u] = -(float)key[u];
      }
    }
    if (__ballot(!done) == 0) break;
    if (!done) {
      if (keymode) {
        // recompute the range on the key values (lanes of other groups idle)
        float a = INFINITY, b = -INFINITY;
#pragma unroll
        for (int u = 0; u < NV; ++u)
          if (cand >> u & 1u) { a = fminf(a, x[u]); b = fmaxf(b, x[u]); }
        lo = g16_minf(a);
        hi = g16_maxf(b);
      }
      const float scale = 256.0f / (hi - lo);
      *reinterpret_cast<u32x4*>(hist + 32 * t) = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(hist + 32 * t + 16) = u32x4{0u, 0u, 0u, 0u};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (cand >> u & 1u) {
          const int b = min(255, (int)((x[u] - lo) * scale));
          atomicAdd(reinterpret_cast<uint32_t*>(hist + (b >> 1) * 4), 1u << (16 * (b & 1)));
        }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const u32x4 d0 = *reinterpret_cast<const u32x4*>(hist + 32 * t);
      const u32x4 d1 = *reinterpret_cast<const u32x4*>(hist + 32 * t + 16);
      int local = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        local += (int)((d0[q] & 0xFFFFu) + (d0[q] >> 16) + (d1[q] & 0xFFFFu) + (d1[q] >> 16));
      const int suf = g16_suffix(local);
      const int above = suf - local;
      const bool mine = above < need && need <= suf;
      int bstar = 0, abv = 0;
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
              bstar = 16 * t + q;
              abv = acc;
            } else {
              acc += cq;
            }
          }
        }
      }
      // one lane of the group holds the answer: a masked sum broadcasts it
      bstar = g16_addi(mine ? bstar : 0);
      abv = g16_addi(mine ? abv : 0);
      uint32_t nc = 0u;
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (cand >> u & 1u) {
          const int b = min(255, (int)((x[u] - lo) * scale));
          if (b > bstar) take |= 1u << u;
          if (b == bstar) nc |= 1u << u;
        }
      need -= abv;
      cand = nc;
      float a = INFINITY, b = -INFINITY;
#pragma unroll
      for (int u = 0; u < NV; ++u)
        if (cand >> u & 1u) { a = fminf(a, x[u]); b = fmaxf(b, x[u]); }
      lo = g16_minf(a);
      hi = g16_maxf(b);
    }
  }
  (void)below;
  return take;
}

// One histogram pass: keeps every candidate whose value falls in or above the
// bin holding the need-th best (so at least `need` are kept, each at least as
// large as every dropped one).  Used to shrink a candidate buffer without an
// exact selection; returns all candidates when their values are all equal.
template <int NV>
__device__ uint32_t group_keep_top(const float (&x)[NV], uint32_t cand, int need, char* hist,
                                   int t, int g) {
  float a = INFINITY, b = -INFINITY;
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (cand >> u & 1u) { a = fminf(a, x[u]); b = fmaxf(b, x[u]); }
  const float lo = g16_minf(a), hi = g16_maxf(b);
  const int cc = g16_addi(__popc(cand));
  const bool work = cand != 0u || cc > 0;
  if (!(hi > lo) || need >= cc || !work) return cand;
  const float scale = 256.0f / (hi - lo);
  *reinterpret_cast<u32x4*>(hist + 32 * t) = u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(hist + 32 * t + 16) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (cand >> u & 1u) {
      const int bb = min(255, (int)((x[u] - lo) * scale));
      atomicAdd(reinterpret_cast<uint32_t*>(hist + (bb >> 1) * 4), 1u << (16 * (bb & 1)));
    }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const u32x4 d0 = *reinterpret_cast<const u32x4*>(hist + 32 * t);
  const u32x4 d1 = *reinterpret_cast<const u32x4*>(hist + 32 * t + 16);
  int local = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    local += (int)((d0[q] & 0xFFFFu) + (d0[q] >> 16) + (d1[q] & 0xFFFFu) + (d1[q] >> 16));
  const int suf = g16_suffix(local);
  const int above = suf - local;
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
          bstar = 16 * t + q;
        } else {
          acc += cq;
        }
      }
    }
  }
  bstar = g16_addi(mine ? bstar : 0);
  uint32_t keep = 0u;
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (cand >> u & 1u) {
      const int bb = min(255, (int)((x[u] - lo) * scale));
      if (bb >= bstar) keep |= 1u << u;
    }
  return keep;
}

}  // namespace mita
