// C ABI of libmita.so: argument validation, workspace layout and the launch
// sequence of the MiTA forward pass.  No allocation, no host copies, no
// synchronisation: everything is enqueued on the caller's stream.
#include <initializer_list>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/mita.h"
#include "internal.h"

// Device scratch of mita_forward_noalloc: the staged schedule's workspace for
// callers that cannot allocate.  Each GPU the library runs on holds its own
// copy until the process ends.  In host code this name is only a stand-in:
// kernels and copies get the address hipGetSymbolAddress returns for the
// current device (scratch_address below), never the name itself.
static __device__ __align__(256) char scratch[MITA_NOALLOC_SCRATCH_BYTES];


using mita::Shape;
using mita::align_up;

namespace {

thread_local std::string g_error;

mita_status fail(mita_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

mita_status ok() {
  g_error.clear();
  return MITA_OK;
}

mita_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MITA_OK;
  return fail(MITA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Records the caller's timing events around the kernels of one call.
struct Marker {
  void* const* ev = nullptr;
  int n = 0, i = 0;
  void mark(hipStream_t st) {
    if (ev && i < n && ev[i]) hipEventRecord((hipEvent_t)ev[i], st);
    ++i;
  }
  // records event j out of turn (a kernel enqueued before those listed ahead of it)
  void mark_at(int j, hipStream_t st) {
    if (ev && j < n && ev[j]) hipEventRecord((hipEvent_t)ev[j], st);
  }
};

// Shape checks common to every entry point.  Returns MITA_OK and fills *s.
mita_status make_shape(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                       mita_dtype dt, Shape* s) {
  if (B < 1 || H < 1) return fail(MITA_ERR_INVALID_ARG, "B=%d and H=%d must be >= 1", B, H);
  if (grid_h < 1 || grid_w < 1)
    return fail(MITA_ERR_INVALID_ARG, "grid %dx%d must be at least 1x1", grid_h, grid_w);
  if (m_h < 1 || m_w < 1 || m_h > grid_h || m_w > grid_w)
    return fail(MITA_ERR_INVALID_ARG, "landmark grid %dx%d must lie within 1x1..%dx%d", m_h, m_w,
                grid_h, grid_w);
  if (dt != MITA_F32 && dt != MITA_BF16)
    return fail(MITA_ERR_INVALID_ARG, "unknown input dtype %d", (int)dt);
  const long long N = (long long)grid_h * grid_w;
  const long long m = (long long)m_h * m_w;
  if (k < 1 || k > N) return fail(MITA_ERR_INVALID_ARG, "k=%d must lie in [1, N=%lld]", k, N);
  if (d != MITA_HEAD_DIM)
    return fail(MITA_ERR_UNSUPPORTED, "head dim d=%d: only %d is implemented", d, MITA_HEAD_DIM);
  if (N > MITA_MAX_N) return fail(MITA_ERR_UNSUPPORTED, "N=%lld exceeds %d", N, MITA_MAX_N);
  if (m > MITA_MAX_M) return fail(MITA_ERR_UNSUPPORTED, "m=%lld exceeds %d", m, MITA_MAX_M);
  if (k > MITA_MAX_K) return fail(MITA_ERR_UNSUPPORTED, "k=%d exceeds %d", k, MITA_MAX_K);
  const long long BH = (long long)B * H;
  if (BH > 65535) return fail(MITA_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", BH);
  s->B = B; s->H = H; s->grid_h = grid_h; s->grid_w = grid_w; s->d = d;
  s->m_h = m_h; s->m_w = m_w; s->k = k;
  s->N = (int)N; s->m = (int)m; s->BH = (int)BH;
  s->bf16 = (dt == MITA_BF16);
  return MITA_OK;
}

// The method variant carried by the extras (s experts per query, shared
// branch or route-only); NULL extras or zeros mean the plain pass.
mita_status set_variant(const mita_extras* ex, Shape* s) {
  const int sv = ex && ex->s ? ex->s : 1;
  const int ro = ex ? ex->route_only : 0;
  if (sv < 1 || sv > MITA_MAX_S || sv > s->m)
    return fail(MITA_ERR_INVALID_ARG, "s=%d must lie in [1, min(m=%d, %d)]", sv, s->m, MITA_MAX_S);
  if (ro != 0 && ro != 1) return fail(MITA_ERR_INVALID_ARG, "route_only must be 0 or 1");
  s->s = sv;
  s->shared = ro == 0;
  return MITA_OK;
}

int path_of(const mita_extras* ex) { return ex ? ex->path : MITA_PATH_AUTO; }

mita_status check_path(int path, const Shape& s) {
  if (path != MITA_PATH_AUTO && path != MITA_PATH_STAGED && path != MITA_PATH_FUSED)
    return fail(MITA_ERR_INVALID_ARG, "unknown path %d", path);
  if (path == MITA_PATH_FUSED && !mita::fused_supported(s))
    return fail(MITA_ERR_UNSUPPORTED,
                "fused schedule needs bf16 inputs, N <= 208, m <= 32, k <= 32 and the plain "
                "variant (s = 1, shared expert)");
  return MITA_OK;
}

bool runs_fused(int path, const Shape& s) {
  return mita::fused_supported(s) && path != MITA_PATH_STAGED;
}

// Which kernels each staged step uses: the MFMA kernels for bf16 inputs
// within their limits, the scalar kernels otherwise (fp32 inputs).
bool pool_mfma(const Shape& s) { return s.bf16; }
bool landmark_mfma(const Shape& s) { return mita::landmark_bf16_supported(s); }
bool route_mfma(const Shape& s) { return mita::route_bf16_supported(s); }
bool attend_mfma(const Shape& s) { return mita::attend_bf16_supported(s); }

size_t landmark_scratch(const Shape& s) {
  return landmark_mfma(s) ? mita::landmark_bf16_scratch_bytes(s) : mita::landmark_scratch_bytes(s);
}
size_t route_scratch(const Shape& s) { return route_mfma(s) ? mita::route_chist_bytes(s) : 0; }

mita_status run_pool(const void* Q, float* ql, const Shape& s, hipStream_t st,
                     Marker* mk = nullptr) {
  const mita_status r = hip_status(pool_mfma(s) ? mita::launch_pool_bf16(Q, ql, s, st)
                                                : mita::launch_pool(Q, ql, s, st),
                                   "pool launch");
  if (mk) mk->mark(st);
  return r;
}
mita_status run_landmark(const float* ql, const void* K, const void* V, int32_t* idx, float* vl,
                         void* scratch, const Shape& s, hipStream_t st, Marker* mk = nullptr,
                         float4* stats = nullptr) {
  const mita_status r =
      hip_status(landmark_mfma(s) ? mita::launch_landmark_bf16(ql, K, V, idx, vl, scratch, s, st, stats)
                                  : mita::launch_landmark(ql, K, V, idx, vl, scratch, s, st),
                 "landmark launch");
  if (mk) mk->mark(st);
  return r;
}
mita_status run_route(const void* Q, const float* ql, int32_t* route, int32_t* counts,
                      int32_t* offsets, int32_t* perm, void* scratch, const Shape& s,
                      hipStream_t st, Marker* mk = nullptr) {
  const bool mfma = route_mfma(s);
  mita_status r = hip_status(mfma ? mita::launch_route_bf16(Q, ql, route, (int32_t*)scratch, s, st)
                                  : mita::launch_route(Q, ql, route, s, st),
                             "route launch");
  if (mk) mk->mark(st);
  if (r != MITA_OK) return r;
  r = hip_status(mfma ? mita::launch_group_bf16(route, (int32_t*)scratch, counts, offsets,
                                                perm, s, st)
                      : mita::launch_group(route, counts, offsets, perm, s, st),
                 "group launch");
  if (mk) mk->mark(st);
  return r;
}
// s > 1 on the matrix-core attention kernel: per-item partials, then a merge
bool merges(const Shape& s) { return s.s > 1 && attend_mfma(s); }

mita_status run_attend(const void* Q, const void* K, const void* V, const float* ql,
                       const float* vl, const int32_t* idx, const int32_t* route,
                       const int32_t* offsets, const int32_t* perm, float* out, void* partial,
                       const Shape& s, hipStream_t st, Marker* mk = nullptr) {
  mita_status r = hip_status(
      attend_mfma(s)
          ? mita::launch_attend_bf16(Q, K, V, ql, vl, idx, offsets, perm, out, partial, s, st)
          : mita::launch_attend(Q, K, V, ql, vl, idx, route, offsets, perm, out, s, st),
      "attend launch");
  if (mk) mk->mark(st);
  if (r != MITA_OK || !merges(s)) return r;
  r = hip_status(mita::launch_merge(partial, out, s, st), "merge launch");
  if (mk) mk->mark(st);
  return r;
}
// Workspace of the staged schedule: every intermediate the caller did not
// supply, then the landmark and route steps' scratch.
struct Layout {
  size_t ql, vl, idx, route, counts, offsets, perm, scratch, rscratch, partial, total;
};

Layout layout_of(const Shape& s, bool with_partial = true) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes, 256); return at; };
  L.ql = take((size_t)s.BH * s.m * s.d * 4);
  L.vl = take((size_t)s.BH * s.m * s.d * 4);
  L.idx = take((size_t)s.BH * s.m * s.k * 4);
  L.route = take((size_t)s.BH * s.N * s.s * 4);
  L.counts = take((size_t)s.BH * s.m * 4);
  L.offsets = take((size_t)s.BH * (s.m + 1) * 4);
  L.perm = take((size_t)s.BH * s.N * s.s * 4);
  L.scratch = take(landmark_scratch(s));
  L.rscratch = take(route_scratch(s));
  L.partial = take(with_partial && merges(s) ? mita::attend_partial_bytes(s) : 0);
  L.total = off;
  return L;
}

template <typename P>
P* pick(P* user, void* ws, size_t off) {
  return user ? user : (P*)((char*)ws + off);
}

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mita_status scratch_address(void** ptr) {
  int dev = -1;
  if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MITA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
      return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MITA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MITA_OK;
}

}  // namespace

extern "C" {

const char* mita_status_string(mita_status s) {
  switch (s) {
    case MITA_OK: return "MITA_OK";
    case MITA_ERR_INVALID_ARG: return "MITA_ERR_INVALID_ARG";
    case MITA_ERR_UNSUPPORTED: return "MITA_ERR_UNSUPPORTED";
    case MITA_ERR_WORKSPACE: return "MITA_ERR_WORKSPACE";
    case MITA_ERR_HIP: return "MITA_ERR_HIP";
  }
  return "MITA_ERR_UNKNOWN";
}

const char* mita_last_error(void) { return g_error.c_str(); }

const char* mita_version(void) { return "mita-gfx950 0.2"; }

// Tensors are read and written 16 bytes per lane.
static bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p) & 15) return false;
  return true;
}

mita_status mita_sync_event_create(void** event) {
  if (!event) return fail(MITA_ERR_INVALID_ARG, "event is required");
  hipEvent_t e = nullptr;
  const mita_status st =
      hip_status(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence),
                 "sync event");
  if (st != MITA_OK) return st;
  *event = e;
  return ok();
}

size_t mita_workspace_bytes_ex(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w,
                               int k, mita_dtype in_dtype, const mita_extras* extras) {
  Shape s;
  if (make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s) != MITA_OK) return 0;
  if (set_variant(extras, &s) != MITA_OK) return 0;
  const int path = path_of(extras);
  if (check_path(path, s) != MITA_OK) return 0;
  return runs_fused(path, s) ? 0 : layout_of(s).total;
}

size_t mita_workspace_bytes(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                            mita_dtype in_dtype) {
  return mita_workspace_bytes_ex(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, nullptr);
}

int mita_schedule(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                  mita_dtype in_dtype) {
  Shape s;
  if (make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s) != MITA_OK) return -1;
  return mita::fused_supported(s) ? MITA_PATH_FUSED : MITA_PATH_STAGED;
}

mita_status mita_forward_ex(const void* Q, const void* K, const void* V, int B, int H, int grid_h,
                            int grid_w, int d, int m_h, int m_w, int k, mita_dtype in_dtype,
                            float* out, int32_t* idx, int32_t* route, const mita_extras* extras,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s);
  if (st != MITA_OK) return st;
  if ((st = set_variant(extras, &s)) != MITA_OK) return st;
  if (!Q || !K || !V || !out) return fail(MITA_ERR_INVALID_ARG, "Q, K, V and out are required");
  if (!aligned16({Q, K, V, out, extras ? extras->ql : nullptr, extras ? extras->vl : nullptr}))
    return fail(MITA_ERR_INVALID_ARG, "Q, K, V, out, ql and vl must be 16-byte aligned");
  const int path = path_of(extras);
  if ((st = check_path(path, s)) != MITA_OK) return st;
  const bool fused = runs_fused(path, s);
  const Layout L = layout_of(s);
  const size_t need = fused ? 0 : L.total;
  if (need && !workspace) return fail(MITA_ERR_INVALID_ARG, "workspace is required");
  if (workspace_bytes < need)
    return fail(MITA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace) & 255) return fail(MITA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  const bool side = extras && (extras->side_stream || extras->fork_event || extras->join_event);
  if (side && !(extras->side_stream && extras->fork_event && extras->join_event))
    return fail(MITA_ERR_INVALID_ARG, "side_stream, fork_event and join_event go together");
  Marker mk;
  if (extras && extras->events && extras->n_events > 0) {
    mk.ev = extras->events;
    mk.n = extras->n_events;
  }
  mk.mark(stream);
  if (fused) {
    st = hip_status(mita::launch_fused(Q, K, V, out, idx, route, extras ? extras->ql : nullptr,
                                       extras ? extras->vl : nullptr,
                                       extras ? extras->counts : nullptr,
                                       extras ? extras->offsets : nullptr,
                                       extras ? extras->perm : nullptr, s, stream),
                    "fused launch");
    mk.mark(stream);
    return st != MITA_OK ? st : ok();
  }

  float* ql = pick(extras ? extras->ql : nullptr, workspace, L.ql);
  // route-only computes no landmark values for the caller: its V_L goes to
  // the workspace, and a caller's vl is left untouched
  float* vl = pick(extras && s.shared ? extras->vl : nullptr, workspace, L.vl);
  int32_t* counts = pick(extras ? extras->counts : nullptr, workspace, L.counts);
  int32_t* offsets = pick(extras ? extras->offsets : nullptr, workspace, L.offsets);
  int32_t* perm = pick(extras ? extras->perm : nullptr, workspace, L.perm);
  int32_t* idx_p = pick(idx, workspace, L.idx);
  int32_t* route_p = pick(route, workspace, L.route);
  void* scratch = (char*)workspace + L.scratch;
  void* rscratch = (char*)workspace + L.rscratch;
  void* partial = (char*)workspace + L.partial;

  if ((st = run_pool(Q, ql, s, stream, &mk)) != MITA_OK) return st;
  {
    // routing and grouping need only Q and Q_L: with a caller-given side stream
    // they run there, beside the landmark pass, and join before attention
    const bool fork = side;
    hipStream_t rs = fork ? (hipStream_t)extras->side_stream : stream;
    hipEvent_t ef = fork ? (hipEvent_t)extras->fork_event : nullptr;
    hipEvent_t ej = fork ? (hipEvent_t)extras->join_event : nullptr;
    if (fork) {
      if ((st = hip_status(hipEventRecord(ef, stream), "fork")) != MITA_OK) return st;
      if ((st = hip_status(hipStreamWaitEvent(rs, ef, 0), "fork")) != MITA_OK) return st;
      // the landmark pass, the longer branch, is enqueued first so that its
      // workgroups reach the CUs first and routing fills the rest; its end
      // event keeps its place after routing's and grouping's in the list
      if ((st = run_landmark(ql, K, V, idx_p, vl, scratch, s, stream)) != MITA_OK) return st;
      mk.mark_at(mk.i + 2, stream);
      if ((st = run_route(Q, ql, route_p, counts, offsets, perm, rscratch, s, rs, &mk)) != MITA_OK)
        return st;
      ++mk.i;  // (the landmark event, recorded above)
      if ((st = hip_status(hipEventRecord(ej, rs), "join")) != MITA_OK) return st;
      if ((st = hip_status(hipStreamWaitEvent(stream, ej, 0), "join")) != MITA_OK) return st;
    } else {
      if ((st = run_route(Q, ql, route_p, counts, offsets, perm, rscratch, s, rs, &mk)) != MITA_OK)
        return st;
      if ((st = run_landmark(ql, K, V, idx_p, vl, scratch, s, stream, &mk)) != MITA_OK) return st;
    }
  }
  if ((st = run_attend(Q, K, V, ql, vl, idx_p, route_p, offsets, perm, out, partial, s, stream,
                       &mk)) != MITA_OK)
    return st;
  return ok();
}

int mita_kernel_names(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                      mita_dtype in_dtype, const mita_extras* extras, const char** names,
                      int* starts, int capacity) {
  Shape s;
  mita_status st = make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s);
  if (st != MITA_OK) return -(int)st;
  if ((st = set_variant(extras, &s)) != MITA_OK) return -(int)st;
  const int path = path_of(extras);
  if ((st = check_path(path, s)) != MITA_OK) return -(int)st;
  const bool forked = extras && extras->side_stream;
  static const char* const kFused[] = {"fused"};
  static const int kFusedStart[] = {0};
  static const char* const kStaged[] = {"pool", "route", "group", "landmark", "attend", "merge"};
  static const int kStagedStart[] = {0, 1, 2, 3, 4, 5};
  static const int kForkedStart[] = {0, 1, 2, 1, 4, 5};
  const bool fused = runs_fused(path, s);
  const char* const* list = fused ? kFused : kStaged;
  const int* start = fused ? kFusedStart : forked ? kForkedStart : kStagedStart;
  const int n = fused ? 1 : merges(s) ? 6 : 5;
  for (int i = 0; i < n && i < capacity; ++i) {
    if (names) names[i] = list[i];
    if (starts) starts[i] = start[i];
  }
  ok();
  return n;
}

mita_status mita_forward(const void* Q, const void* K, const void* V, int B, int H, int grid_h,
                         int grid_w, int d, int m_h, int m_w, int k, mita_dtype in_dtype,
                         float* out, int32_t* idx, int32_t* route, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return mita_forward_ex(Q, K, V, B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, out, idx, route,
                         nullptr, workspace, workspace_bytes, stream);
}

mita_status mita_forward_noalloc(const void* Q, const void* K, const void* V, int B, int H,
                                int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                                mita_dtype in_dtype, float* out, int32_t* idx, int32_t* route,
                                hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s);
  if (st != MITA_OK) return st;
  const size_t need = runs_fused(MITA_PATH_AUTO, s) ? 0 : layout_of(s).total;
  if (need > (size_t)MITA_NOALLOC_SCRATCH_BYTES)
    return fail(MITA_ERR_WORKSPACE,
                "this shape needs %zu bytes of scratch; the static scratch holds %zu "
                "(use mita_forward with a workspace)",
                need, (size_t)MITA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_address(&ws)) != MITA_OK) return st;
  return mita_forward_ex(Q, K, V, B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, out, idx, route,
                         nullptr, ws, need, stream);
}

// The backward's workspace: the forward's intermediates (recomputed, the
// same kernels and so the same choices), then the backward's own buffers.
size_t backward_layout(const Shape& s, Layout* L) {
  *L = layout_of(s, false);
  return L->total + mita::backward_scratch_bytes(s);
}

size_t mita_backward_workspace_bytes(int B, int H, int grid_h, int grid_w, int d, int m_h,
                                     int m_w, int k, mita_dtype in_dtype,
                                     const mita_extras* extras) {
  Shape s;
  if (make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s) != MITA_OK) return 0;
  if (set_variant(extras, &s) != MITA_OK) return 0;
  Layout L;
  return backward_layout(s, &L);
}

mita_status mita_backward(const void* Q, const void* K, const void* V, const float* dout, int B,
                          int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                          mita_dtype in_dtype, float* dQ, float* dK, float* dV,
                          const mita_extras* extras, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, grid_h, grid_w, d, m_h, m_w, k, in_dtype, &s);
  if (st != MITA_OK) return st;
  if ((st = set_variant(extras, &s)) != MITA_OK) return st;
  if (!Q || !K || !V || !dout || !dQ || !dK || !dV)
    return fail(MITA_ERR_INVALID_ARG, "Q, K, V, dOut, dQ, dK and dV are required");
  if (!aligned16({Q, K, V, dout, dQ, dK, dV}))
    return fail(MITA_ERR_INVALID_ARG, "Q, K, V, dOut, dQ, dK and dV must be 16-byte aligned");
  Layout L;
  const size_t need = backward_layout(s, &L);
  if (!workspace) return fail(MITA_ERR_INVALID_ARG, "workspace is required");
  if (workspace_bytes < need)
    return fail(MITA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace) & 255) return fail(MITA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  char* ws = (char*)workspace;
  float* ql = (float*)(ws + L.ql);
  float* vl = (float*)(ws + L.vl);
  int32_t* idx = (int32_t*)(ws + L.idx);
  int32_t* route = (int32_t*)(ws + L.route);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* perm = (int32_t*)(ws + L.perm);
  if ((st = run_pool(Q, ql, s, stream)) != MITA_OK) return st;
  // the MFMA landmark pass also leaves its rows' softmax statistics, which
  // the backward's landmark step reuses
  const bool stats_ready = s.shared && landmark_mfma(s);
  if ((st = run_landmark(ql, K, V, idx, vl, ws + L.scratch, s, stream, nullptr,
                         stats_ready ? mita::backward_stats(ws + L.total, s) : nullptr)) != MITA_OK)
    return st;
  if ((st = run_route(Q, ql, route, counts, offsets, perm, ws + L.rscratch, s, stream)) != MITA_OK)
    return st;
  if ((st = hip_status(mita::launch_backward(Q, K, V, dout, ql, vl, idx, route, offsets, perm, dQ,
                                             dK, dV, ws + L.total, s, stream, stats_ready),
                       "backward launch")) != MITA_OK)
    return st;
  return ok();
}

mita_status mita_pool(const void* Q, int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w,
                      mita_dtype in_dtype, float* ql, hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, grid_h, grid_w, d, m_h, m_w, 1, in_dtype, &s);
  if (st != MITA_OK) return st;
  if (!Q || !ql) return fail(MITA_ERR_INVALID_ARG, "Q and ql are required");
  if (!aligned16({Q, ql})) return fail(MITA_ERR_INVALID_ARG, "Q and ql must be 16-byte aligned");
  if ((st = run_pool(Q, ql, s, stream)) != MITA_OK) return st;
  return ok();
}

size_t mita_landmark_workspace_bytes(int B, int H, int N, int d, int m, int k,
                                     mita_dtype in_dtype) {
  Shape s;
  if (make_shape(B, H, N, 1, d, m, 1, k, in_dtype, &s) != MITA_OK) return 0;
  return landmark_scratch(s);
}

mita_status mita_landmark(const float* ql, const void* K, const void* V, int B, int H, int N, int d,
                          int m, int k, mita_dtype in_dtype, int32_t* idx, float* vl,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, N, 1, d, m, 1, k, in_dtype, &s);
  if (st != MITA_OK) return st;
  if (!ql || !K || !V || !idx || !vl)
    return fail(MITA_ERR_INVALID_ARG, "ql, K, V, idx and vl are required");
  if (!aligned16({ql, K, V, vl}))
    return fail(MITA_ERR_INVALID_ARG, "ql, K, V and vl must be 16-byte aligned");
  const size_t need = landmark_scratch(s);
  if (need && !workspace) return fail(MITA_ERR_INVALID_ARG, "workspace is required");
  if (workspace_bytes < need)
    return fail(MITA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if ((st = run_landmark(ql, K, V, idx, vl, workspace, s, stream)) != MITA_OK) return st;
  return ok();
}

size_t mita_route_workspace_bytes(int B, int H, int N, int d, int m, mita_dtype in_dtype) {
  Shape s;
  if (make_shape(B, H, N, 1, d, m, 1, 1, in_dtype, &s) != MITA_OK) return 0;
  return route_scratch(s);
}

mita_status mita_route(const void* Q, const float* ql, int B, int H, int N, int d, int m,
                       mita_dtype in_dtype, int32_t* route, int32_t* counts, int32_t* offsets,
                       int32_t* perm, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, N, 1, d, m, 1, 1, in_dtype, &s);
  if (st != MITA_OK) return st;
  if (!Q || !ql || !route || !counts || !offsets || !perm)
    return fail(MITA_ERR_INVALID_ARG, "Q, ql, route, counts, offsets and perm are required");
  if (!aligned16({Q, ql})) return fail(MITA_ERR_INVALID_ARG, "Q and ql must be 16-byte aligned");
  const size_t need = route_scratch(s);
  if (need && !workspace) return fail(MITA_ERR_INVALID_ARG, "workspace is required");
  if (workspace_bytes < need)
    return fail(MITA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if ((st = run_route(Q, ql, route, counts, offsets, perm, workspace, s, stream)) != MITA_OK)
    return st;
  return ok();
}

mita_status mita_attend(const void* Q, const void* K, const void* V, const float* ql,
                        const float* vl, const int32_t* idx, const int32_t* route,
                        const int32_t* offsets, const int32_t* perm, int B, int H, int N, int d,
                        int m, int k, mita_dtype in_dtype, float* out, hipStream_t stream) {
  Shape s;
  mita_status st = make_shape(B, H, N, 1, d, m, 1, k, in_dtype, &s);
  if (st != MITA_OK) return st;
  if (!Q || !K || !V || !ql || !vl || !idx || !route || !offsets || !perm || !out)
    return fail(MITA_ERR_INVALID_ARG, "every tensor argument of mita_attend is required");
  if (!aligned16({Q, K, V, ql, vl, out}))
    return fail(MITA_ERR_INVALID_ARG, "Q, K, V, ql, vl and out must be 16-byte aligned");
  if ((st = run_attend(Q, K, V, ql, vl, idx, route, offsets, perm, out, nullptr, s, stream)) !=
      MITA_OK)
    return st;
  return ok();
}

}  // extern "C"
