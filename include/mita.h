/*
 * mita.h -- C ABI of the MiTA (Mixture-of-Top-k Attention) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the attention layer described on the page
 * "NeurIPS'26：注意力也是FFN？从快权重出发，重新理解高效注意力" (新智元/36氪),
 * section "用少量地标查询，同时构造全局概括与细节专家" and its Algorithm 1
 * (English version: "NeurIPS'26: Is Attention Also FFN? ...", section
 * "Construct global generalization and detail experts at the same time with
 * a small number of landmark queries"); cited below as [ZH].  Per (batch b,
 * head h), with
 * N = grid_h*grid_w tokens in row-major order, m = m_h*m_w landmarks and
 * tau = 1/sqrt(d):
 *   Q_L     = 2-D adaptive average pooling of Q over the token grid  (m x d)
 *   S       = tau * Q_L K^T                                           (m x N)
 *   idx_i   = top-k keys of S[i,:], ties to the lowest key index      (m x k)
 *   V_L     = softmax_row(S) V                                        (m x d)
 *   route_n = argmax_i q_n . Q_L[i], ties to the lowest landmark      (N)
 *   out_n   = softmax(tau*[q_n Q_L^T, q_n K[idx_e]^T]) [V_L; V[idx_e]],
 *             e = route_n                                              (N x d)
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees, copies to the host or synchronises; it
 *     enqueues kernels on `stream` and returns (asynchronous).
 *   - Q, K, V, out are contiguous [B, H, N, d] row-major (token n = y*grid_w+x),
 *     16-byte aligned, like ql and vl where an entry point takes them (a
 *     misaligned one is MITA_ERR_INVALID_ARG).  Q, K, V are fp32 or bf16
 *     (`in_dtype`); out is always fp32 (no output-type argument: a bf16
 *     output would round values near 5 by more than 1e-2).
 *   - Precondition on bf16 inputs: every |V| < 65504, and every |Q| < 65504.
 *     The value products run on f16 matrix cores (V, V_L and the softmax
 *     weights are staged as f16), and for large m and k (when keeping all of
 *     an expert's k rows in LDS needs the room) the shared logits q . Q_L run
 *     on f16 matrix cores too (q and Q_L as f16), so larger values would
 *     become inf.  Nothing checks this (it would cost a pass over Q and V);
 *     the seeded workloads stay below 40.  fp32 inputs have no such bound.
 *   - Index outputs are int32.  idx rows list key ids in ascending order.
 *   - d must be 64 (MITA_ERR_UNSUPPORTED otherwise).
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK status nothing was launched.  MITA_ERR_HIP reports a failed
 *     launch.  mita_last_error() gives a thread-local description.
 *   - The same inputs give bitwise-identical outputs on every call.
 */
#ifndef MITA_H
#define MITA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MITA_OK = 0,
  MITA_ERR_INVALID_ARG = 1,  /* null pointer, bad size or range            */
  MITA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (d != 64, ...)    */
  MITA_ERR_WORKSPACE = 3,    /* workspace too small                         */
  MITA_ERR_HIP = 4           /* a HIP call or kernel launch failed          */
} mita_status;

typedef enum { MITA_F32 = 0, MITA_BF16 = 1 } mita_dtype;

/* Implementation limits (checked, MITA_ERR_UNSUPPORTED beyond them). */
#define MITA_HEAD_DIM 64
#define MITA_MAX_M 1024
#define MITA_MAX_K 1024
#define MITA_MAX_N (1 << 22)

/* Which kernel schedule mita_forward_ex runs. AUTO picks by shape. */
typedef enum { MITA_PATH_AUTO = 0, MITA_PATH_FUSED = 1, MITA_PATH_STAGED = 2 } mita_path;

/* Human-readable name of a status code (static storage). */
const char* mita_status_string(mita_status s);

/* Description of the last failure on the calling thread ("" if none). */
const char* mita_last_error(void);

/* Library version string (static storage). */
const char* mita_version(void);

/*
 * Bytes of device workspace mita_forward needs for this shape (the "device
 * memory query"): the caller allocates it (e.g. through PyTorch) and passes it
 * in.  0 when the schedule mita_forward runs for the shape needs none (the
 * fused one): the workspace pointer may then be NULL.  Also 0 for an invalid
 * shape (mita_forward then reports why).  The layout inside is private.
 */
size_t mita_workspace_bytes(int B, int H, int grid_h, int grid_w, int d,
                            int m_h, int m_w, int k, mita_dtype in_dtype);

/*
 * The schedule mita_forward runs for this shape with MITA_PATH_AUTO:
 * MITA_PATH_FUSED (one persistent kernel per call; bf16, N <= 208, m <= 32,
 * k <= 32) or MITA_PATH_STAGED (one kernel per step).  -1 for an invalid shape.
 */
int mita_schedule(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                  mita_dtype in_dtype);

/*
 * The whole forward pass (all steps above) on `stream`.
 *   out   [B,H,N,d] fp32, required.
 *   idx   [B,H,m,k] int32 or NULL: each landmark's expert (ascending key ids).
 *   route [B,H,N]   int32 or NULL: each query's landmark id in [0, m).
 *   workspace: at least mita_workspace_bytes(...) bytes of device memory,
 *   256-byte aligned (NULL allowed when that is 0); contents on entry are
 *   ignored.
 */
mita_status mita_forward(const void* Q, const void* K, const void* V,
                         int B, int H, int grid_h, int grid_w, int d,
                         int m_h, int m_w, int k, mita_dtype in_dtype,
                         float* out, int32_t* idx, int32_t* route,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mita_forward without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and plain pass (s = 1, shared
 * expert, automatic schedule, every kernel on `stream`) as mita_forward; the
 * staged schedule's intermediates go to a static device array of
 * MITA_NOALLOC_SCRATCH_BYTES inside the library instead (one per GPU, held
 * until the process ends; the fused schedule needs none).  The call
 * allocates and frees nothing.  A shape whose workspace
 * (mita_workspace_bytes) exceeds the array is MITA_ERR_WORKSPACE, nothing
 * launched.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind; the kernels write every byte they read within a call, so
 * nothing needs clearing, but calls that overlap on one GPU (two streams, two
 * host threads) race on it and must be serialised by the caller.
 */
#define MITA_NOALLOC_SCRATCH_BYTES (32u << 20)
mita_status mita_forward_noalloc(const void* Q, const void* K, const void* V,
                                 int B, int H, int grid_h, int grid_w, int d,
                                 int m_h, int m_w, int k, mita_dtype in_dtype,
                                 float* out, int32_t* idx, int32_t* route, hipStream_t stream);

/*
 * Optional extra outputs of mita_forward_ex (any member may be NULL), the
 * schedule to run, the method variant, and optional per-kernel timing
 * events.  Zero-initialised it asks for the plain pass.  Used to check every
 * intermediate of the pass, to time its kernels, and to run the variants.
 *   ql      [B,H,m,d] fp32  landmark queries
 *   vl      [B,H,m,d] fp32  landmark values (shared expert values)
 *   counts  [B,H,m]   int32 queries routed to each landmark
 *   offsets [B,H,m+1] int32 exclusive prefix sum of counts
 *   perm    [B,H,N]   int32 query ids grouped by route, ascending within a group
 *   events  NULL, or n_events caller-created hipEvent_t handles: the call
 *           records events[0] on `stream` before its first kernel and
 *           events[i] right after the i-th kernel mita_kernel_names lists,
 *           for i < n_events; kernel i runs between events[starts[i]] and
 *           events[i + 1] (starts as mita_kernel_names returns them).
 *   side_stream, fork_event, join_event
 *           NULL, or all three: a caller-owned hipStream_t on the same device
 *           and two caller-owned hipEvent_t.  The staged schedule then runs
 *           routing and grouping (which need only Q and Q_L) on side_stream,
 *           forked from `stream` after pooling (fork_event) and joined back
 *           before attention (join_event), so that they overlap the landmark
 *           pass.  The fused schedule ignores them.  Two calls in flight at
 *           once must not share them.  Without them every kernel goes on
 *           `stream`.  Either way the call is asynchronous with respect to
 *           the host, and work queued on `stream` after it sees every output.
 *           Events from mita_sync_event_create make the fork and the join
 *           cheapest.
 *   s       experts per query (0 means 1).  With s > 1 each query is routed
 *           to its s best landmarks (q . Q_L descending, ties to the lower
 *           landmark) and takes ONE softmax over its m shared entries and the
 *           s*k entries of those experts, concatenated without removing keys
 *           that two experts share (page [ZH], landmark-query section: the
 *           output is given there for one routed expert per query, s = 1;
 *           this is the plain extension to s).  route is then [B,H,N,s]
 *           (best first) and counts/offsets/perm group the N*s (query,
 *           rank) items t = n*s + j by expert.  1 <= s <= min(m, MITA_MAX_S).
 *   route_only
 *           nonzero: the ablation without the shared (compressed) branch
 *           (page [ZH], long-sequence section, the ablation with the same
 *           number of entries per query): each query's softmax covers only
 *           its routed experts' s*k entries; V_L is not computed (vl, if
 *           given, is left untouched).  Pass k = m + k_mita to give every
 *           query the same number of entries as the full method.
 */
typedef struct {
  float* ql;
  float* vl;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int path; /* mita_path */
  void* const* events;
  int n_events;
  void* side_stream; /* hipStream_t */
  void* fork_event;  /* hipEvent_t */
  void* join_event;  /* hipEvent_t */
  int s;
  int route_only;
} mita_extras;

#define MITA_MAX_S 8

/*
 * Bytes of device workspace mita_forward_ex needs with these extras (its
 * path, variant and supplied outputs; NULL means none): 0 when the schedule
 * it runs needs none.  0 also for an invalid shape or variant.
 */
size_t mita_workspace_bytes_ex(int B, int H, int grid_h, int grid_w, int d,
                               int m_h, int m_w, int k, mita_dtype in_dtype,
                               const mita_extras* extras);

mita_status mita_forward_ex(const void* Q, const void* K, const void* V,
                            int B, int H, int grid_h, int grid_w, int d,
                            int m_h, int m_w, int k, mita_dtype in_dtype,
                            float* out, int32_t* idx, int32_t* route,
                            const mita_extras* extras,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Creates a hipEvent_t, on the current device, for mita_extras.fork_event or
 * join_event: no timing, and a device-scope release when recorded instead of
 * the default system-scope fence.  Two streams of one device need no more,
 * and the default fence's cache write-back and invalidation put idle time
 * between the kernels on either side of each fork and join.  The event
 * cannot order work with the host or other devices.  Writes the handle to
 * *event; the caller owns it (hipEventDestroy).  Returns
 * MITA_ERR_INVALID_ARG for a NULL `event` and MITA_ERR_HIP when the runtime
 * cannot create the event.
 */
mita_status mita_sync_event_create(void** event);

/*
 * The kernels mita_forward_ex launches for this configuration and these
 * extras (path, variant; NULL means the plain pass), in the order of its
 * timing events: "fused" for the fused schedule; "pool", "route", "group",
 * "landmark", "attend" for the staged one, and "merge" after them when
 * s > 1.  Writes up to `capacity` static strings to names and, to starts,
 * the index of the event each kernel's interval opens with: i when the
 * kernel follows the previous one on the same stream; when the extras carry
 * a side stream, landmark opens with pooling's end event, like route.  names
 * and starts may be NULL.  Returns the kernel count, or a negative
 * mita_status for invalid sizes or an unsupported path.  Host only: the
 * extras' pointers are not dereferenced.
 */
int mita_kernel_names(int B, int H, int grid_h, int grid_w, int d, int m_h, int m_w, int k,
                      mita_dtype in_dtype, const mita_extras* extras, const char** names,
                      int* starts, int capacity);

/*
 * Gradients of the pass (training; page [ZH], long-sequence section, Table 5:
 * the training times with this attention): dQ, dK, dV [B,H,N,d] fp32 of
 * sum(dOut * out) for dOut [B,H,N,d] fp32, with the top-k sets and routes of
 * the forward held fixed (discrete choices: no gradient flows through them).
 * The call recomputes the forward's intermediates with the staged kernels
 * (the same kernels, so the same choices) and differentiates the one softmax
 * of the output, the landmark values' softmax and the pooling exactly.
 * extras: only s and route_only are read (NULL: the plain pass).  Needs
 * mita_backward_workspace_bytes(...) of workspace, 256-byte aligned.
 * dQ, dK, dV are overwritten.
 */
size_t mita_backward_workspace_bytes(int B, int H, int grid_h, int grid_w, int d,
                                     int m_h, int m_w, int k, mita_dtype in_dtype,
                                     const mita_extras* extras);
mita_status mita_backward(const void* Q, const void* K, const void* V, const float* dout,
                          int B, int H, int grid_h, int grid_w, int d,
                          int m_h, int m_w, int k, mita_dtype in_dtype,
                          float* dQ, float* dK, float* dV, const mita_extras* extras,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The steps one at a time (same kernels as the staged schedule, plain pass,
 * s = 1).  Each takes its inputs from device memory and writes its outputs
 * there, so a caller can run, time or check one step in isolation.
 * ------------------------------------------------------------------------- */

/*
 * Landmark pooling: Q [B,H,N,d] -> ql [B,H,m,d] fp32 (window mean, fp32 sums).
 * Page [ZH], landmark-query section (m landmark queries by local average
 * pooling of the queries); windows are those of 2-D adaptive average
 * pooling, rows [floor(r*gh/mh), ceil((r+1)*gh/mh)), columns likewise.
 */
mita_status mita_pool(const void* Q, int B, int H, int grid_h, int grid_w, int d,
                      int m_h, int m_w, mita_dtype in_dtype, float* ql, hipStream_t stream);

/*
 * Landmark pass: scores of ql [B,H,m,d] fp32 against K [B,H,N,d], each row's
 * top-k keys -> idx [B,H,m,k] (ascending), and the row softmax applied to V
 * -> vl [B,H,m,d] fp32.  Page [ZH], landmark-query section: each landmark
 * query scores every key and its k best form a routed expert; the same
 * scores, softmax-normalised over all keys, give the landmark values (the
 * shared expert's values, "top-k selection and the global summary share the
 * landmark scores").  Needs mita_landmark_workspace_bytes(...) of scratch
 * (0 when the bf16 MFMA kernel serves the shape -- bf16 inputs, k <= 400;
 * workspace may then be NULL).
 */
size_t mita_landmark_workspace_bytes(int B, int H, int N, int d, int m, int k,
                                     mita_dtype in_dtype);
mita_status mita_landmark(const float* ql, const void* K, const void* V,
                          int B, int H, int N, int d, int m, int k, mita_dtype in_dtype,
                          int32_t* idx, float* vl,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Routing and grouping: route [B,H,N] = argmax_i q_n . ql[i] (lowest i on
 * ties), then a stable counting sort of each head's queries by route:
 * counts [B,H,m], offsets [B,H,m+1], perm [B,H,N].  Page [ZH],
 * landmark-query section (each query picks the expert of the landmark it
 * matches best; the query-landmark scores are the ones the shared branch
 * reuses) and Algorithm 1 (queries grouped by route).  Needs
 * mita_route_workspace_bytes(...) of scratch (may be 0; workspace may then be
 * NULL).
 */
size_t mita_route_workspace_bytes(int B, int H, int N, int d, int m, mita_dtype in_dtype);
mita_status mita_route(const void* Q, const float* ql, int B, int H, int N, int d, int m,
                       mita_dtype in_dtype, int32_t* route, int32_t* counts,
                       int32_t* offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Grouped expert attention: for every query, one softmax over its m shared
 * logits and the k logits of its routed expert (idx row route_n), applied to
 * [vl; V[idx]] -> out [B,H,N,d] fp32.  Page [ZH], landmark-query section
 * (the s = 1 output: the two sets of key-value pairs are concatenated under
 * one softmax) and Algorithm 1 (queries grouped by route, partial results
 * merged by online softmax).  offsets/perm must be the grouping of `route`
 * produced by mita_route.
 */
mita_status mita_attend(const void* Q, const void* K, const void* V,
                        const float* ql, const float* vl, const int32_t* idx,
                        const int32_t* route, const int32_t* offsets, const int32_t* perm,
                        int B, int H, int N, int d, int m, int k, mita_dtype in_dtype,
                        float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MITA_H */
