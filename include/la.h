/*
 * la.h -- C ABI of the MI355X (gfx950) kernelized linear-attention library
 * (liblaphi.so).
 *
 * The method (nx_f32_linear_attention.nx source, header comment and
 * functions la_phi / nx_f32_linear_attention): with the positive feature
 * map phi(x) = relu(x) + 1,
 *     S = sum_j phi(K_j) (x) V_j   (d x d),   z = sum_j phi(K_j)   (d),
 *     out_i = (phi(Q_i) S) / (phi(Q_i) . z).
 * The order of the products is reassociated so that the n x n attention
 * matrix is never formed (LinearTile README, "How It Works": compute K^T V
 * first).  Three forms plus a decode step are exported:
 *   la_forward             non-causal: every query sees every key;
 *   la_causal_forward      causal: query i sees keys 0..i (a prefix mask
 *                          m = arange(n), trim-transformer 0.1.0, "Masking");
 *   la_prefix_mask_forward unnormalised Attn = Q K^T V with no feature map,
 *                          query i sees keys 0..m_i (trim-transformer 0.1.0,
 *                          "Masking");
 *   la_decode_step         one recurrent step on a cached (S, z) state
 *                          (trim-transformer 0.1.0, "Key-value caching").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Per head, tokens are rows and features are contiguous
 *   ([n_tokens, head_dim] row-major, as on the nx page); batches of heads are
 *   contiguous [B][H][n][d] ("BHND").  q and out are [B][Hq][n][d]; k and v
 *   are [B][Hkv][n][d].  Query head h reads key/value head h / (Hq / Hkv).
 * Pointers.  q, k, v, out, m, S, z, ws are DEVICE pointers on the current
 *   HIP device.  The caller owns every buffer; the library keeps no pointer
 *   after a call returns.  Base pointers must be 16-byte aligned.  out must
 *   not overlap q, k or v.
 * dtype.  LA_F32 or LA_BF16 for q, k, v and out (out has the input dtype,
 *   rounded to nearest-even from fp32).  Accumulation and the recurrent
 *   state (S, z) are always fp32.  S is stored [a][b] row-major per head
 *   (S[a*d + b] = sum_j phi(K_j)[a] V_j[b]), z as [a].
 * Limits.  1 <= d <= 128; n >= 1; B, H >= 1; Hq a multiple of Hkv.
 * stream.  A hipStream_t passed as void*; NULL is the default stream.  Every
 *   call only enqueues work on that stream and returns: no host
 *   synchronisation, no device allocation.
 * Workspace.  Forward calls take a device workspace of at least
 *   la_workspace_bytes(...) bytes, owned by the caller.  Its first 256 bytes
 *   are a control block that must hold zeros before the first call that
 *   uses the workspace (la_workspace_init, or any zero-fill of the buffer);
 *   calls keep it valid from then on.  The rest may hold anything before a
 *   call: every word a call reads there it wrote first, and the flags that
 *   order a call's workgroups carry an epoch that the control block makes
 *   new for every call -- also for every replay of a call captured into a
 *   HIP graph.  One workspace may serve calls of every kind and shape in turn
 *   (with the bytes the largest of them needs); calls that may overlap in time
 *   (on different streams) must not share a workspace.
 * Errors.  Every argument check runs on the host before anything is
 *   enqueued; on failure nothing is launched and a nonzero la_status is
 *   returned (0 means success, as the nx page's functions return 0).
 *   A launch failure returns LA_ERR_LAUNCH.  What only the device can see --
 *   a bounded wait between workgroups that gave up (the outputs of that call
 *   are then wrong), a prefix-mask value outside [0, n - 1] -- is recorded in
 *   the workspace's control block and returned by la_workspace_status.
 * Graphs.  Every call only launches kernels (no allocation, no memset, no
 *   host synchronisation), so it may be captured into a HIP graph; replays
 *   then run on the workspace captured with it, in stream order.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t la_status;
enum {
  LA_OK = 0,
  LA_ERR_NULL = 1,        /* a required pointer is NULL */
  LA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  LA_ERR_DTYPE = 3,       /* unknown dtype code */
  LA_ERR_UNSUPPORTED = 4, /* valid request this build does not offer (chunk) */
  LA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  LA_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
  LA_ERR_ALIAS = 7,       /* out overlaps an input */
  LA_ERR_LAUNCH = 8,      /* the HIP runtime rejected a launch */
  LA_ERR_TIMEOUT = 9,     /* (la_workspace_status) a bounded wait gave up */
  LA_ERR_RANGE = 10,      /* (la_workspace_status) a mask value out of range */
  LA_ERR_DEVICE = 11      /* (la_workspace_status) a HIP copy or sync failed */
};

typedef int32_t la_dtype;
enum { LA_F32 = 0, LA_BF16 = 1 };

/* Feature map phi of the normalised forms.  LA_PHI_RELU1: phi(x) = relu(x)
 * + 1 (nx_f32_linear_attention.nx, function la_phi), what la_forward,
 * la_causal_forward and la_decode_step use.  LA_PHI_ELU1: phi(x) = ELU(x) +
 * 1 with alpha = 1, i.e. x + 1 for x > 0 and e^x otherwise (LinearTile
 * 1.0.1, "How It Works").  LA_PHI_FEATURES: a feature map of the caller's
 * choice (LinearTile 1.0.1, "Features": phi replaceable at will), applied by
 * the caller: q and k (and the decode step's q and k) already hold phi(Q)
 * and phi(K), which must be positive (every denominator phi(Q_i) . z_i must
 * be > 0; nothing checks this), and the library computes
 * out_i = phi(Q_i) S_i / (phi(Q_i) . z_i) with S, z summed over phi(K) as
 * given.  Taken by the *_phi entry points below; any other value gives
 * LA_ERR_UNSUPPORTED. */
typedef int32_t la_phi;
enum { LA_PHI_RELU1 = 0, LA_PHI_ELU1 = 1, LA_PHI_FEATURES = 2 };

/* Operation codes for la_workspace_bytes. */
enum { LA_OP_FORWARD = 0, LA_OP_CAUSAL = 1, LA_OP_PREFIX_MASK = 2, LA_OP_PREFIX_MASK_BATCHED = 3,
       LA_OP_SEQS = 4, LA_OP_CAUSAL_BACKWARD = 5 };

/* Human-readable name of a status code (static string, never NULL). */
const char* la_status_str(la_status s);

/* Workspace bytes needed by la_forward (op LA_OP_FORWARD), la_causal_forward
 * (LA_OP_CAUSAL), la_prefix_mask_forward (LA_OP_PREFIX_MASK, pass Hq = Hkv
 * = H) or la_prefix_mask_forward_batched (LA_OP_PREFIX_MASK_BATCHED, the
 * same) for these sizes.  Returns 0 if the arguments are invalid. */
size_t la_workspace_bytes(int32_t op, int64_t B, int64_t Hq, int64_t Hkv,
                          int64_t n, int64_t d, la_dtype dtype, int32_t chunk);

/* Control block of a workspace (its first 256 bytes).
 * la_workspace_init: enqueue on `stream` a kernel that zeroes it (needed
 *   once for a new workspace that was not zero-filled).
 * la_workspace_status: wait for `stream` to finish (host synchronisation),
 *   then return the errors recorded since the last status call and clear
 *   them: LA_ERR_TIMEOUT if a bounded wait between workgroups gave up in some
 *   call (its outputs are wrong), else LA_ERR_RANGE if a prefix-mask value
 *   lay outside [0, n - 1], else LA_OK.  LA_ERR_DEVICE if the HIP runtime
 *   failed to synchronise or copy.
 * la_workspace_set_wait: diagnostics for testing failure handling.  limit is
 *   the number of polls after which a wait gives up (0: the default, about
 *   2^22 polls); skew is added to the epoch the waits expect, so with skew
 *   != 0 no wait can succeed and every one gives up after `limit` polls,
 *   while every kernel still runs to its end.  (0, 0) restores the default.
 * Each returns LA_ERR_NULL, LA_ERR_WORKSPACE (ws_bytes < 256) or LA_ERR_ALIGN
 * for a bad workspace and launches nothing then. */
la_status la_workspace_init(void* ws, size_t ws_bytes, void* stream);
la_status la_workspace_status(void* ws, size_t ws_bytes, void* stream);
la_status la_workspace_set_wait(void* ws, size_t ws_bytes, uint32_t limit, uint32_t skew, void* stream);

/* Non-causal normalised linear attention (nx_f32_linear_attention.nx: S, z
 * over all keys, then every query's normalised read).
 *   q [B][Hq][n][d], k, v [B][Hkv][n][d] -> out [B][Hq][n][d]. */
la_status la_forward(const void* q, const void* k, const void* v, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t n, int64_t d,
                     la_dtype dtype, void* out, void* ws, size_t ws_bytes,
                     void* stream);

/* Causal normalised linear attention: out_i uses S_i = sum_{j<=i}
 * phi(K_j) (x) V_j and z_i = sum_{j<=i} phi(K_j) (query i sees its own key).
 * Computed chunk by chunk: within a chunk of `chunk` tokens a masked
 * phi(Q) phi(K)^T V term, across chunks an exclusive prefix of the chunk
 * states.  chunk: 32, 64 or 128 where the tiles fit in LDS, or 0 for the
 * default (64, or 32 where that lets two workgroups share a compute unit:
 * bf16 with d > 64, fp32 with d > 32, except fp32 with d = 64 and Hq = Hkv,
 * which takes 64); the result does not depend on it beyond rounding.
 * S_final [B][Hkv][d][d] and z_final [B][Hkv][d] (fp32, device; either may
 * be NULL) receive the state after the last token -- the hand-off to
 * la_decode_step.  q and out may both be NULL for a state-only pass (then
 * Hq is still validated and S_final or z_final must be non-NULL). */
la_status la_causal_forward(const void* q, const void* k, const void* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                            int64_t d, la_dtype dtype, int32_t chunk,
                            void* out, float* S_final, float* z_final,
                            void* ws, size_t ws_bytes, void* stream);

/* la_causal_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same results
 * (the same kernels).  Its workspace is a static 64 MiB device array per GPU,
 * held until the process ends; sizes whose la_workspace_bytes(LA_OP_CAUSAL,
 * ...) exceed it return LA_ERR_WORKSPACE and launch nothing (the causal
 * workload B8 H8 n2048 d64 needs about 4.3 MB).  It calls no allocator.
 * Every call on a GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (on different streams) race on it.  The errors that
 * la_workspace_status reports for a caller's workspace are recorded in the
 * array and cannot be read back. */
la_status la_causal_forward_noalloc(const void* q, const void* k, const void* v,
                                    int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t n, int64_t d, la_dtype dtype,
                                    int32_t chunk, void* out, float* S_final,
                                    float* z_final, void* stream);

/* Unnormalised prefix-mask form Attn(Q,K,V) = Q K^T V (trim-transformer
 * 0.1.0): out_i = sum_{j <= m_i} (Q_i . K_j) V_j, no feature map, no
 * normaliser, no scale.  m is a device int64 array [n] shared by every batch
 * and head, any order, duplicates allowed; every m_i must lie in [0, n-1].
 * A value outside that range is a contract violation: the device clamps it
 * into range (so that no access leaves the buffers; the outputs of such rows
 * are then not the form's) and records it in the workspace's control block,
 * which la_workspace_status reports as LA_ERR_RANGE (the Python binding
 * checks this after every call when LA_DEBUG_CHECKS=1).
 * q, k, v, out [B][H][n][d].  chunk as for la_causal_forward, except that
 * the default for fp32 with d = 64 is 64. */
la_status la_prefix_mask_forward(const void* q, const void* k, const void* v,
                                 const int64_t* m, int64_t B, int64_t H,
                                 int64_t n, int64_t d, la_dtype dtype,
                                 int32_t chunk, void* out, void* ws,
                                 size_t ws_bytes, void* stream);

/* The same form with one mask per batch: m is a device int64 array [B][n]
 * and query i of batch b (every head) sees keys 0..m[b][i] (the masks of
 * the trim-transformer page, "Masking", one per sequence).  Each row has the
 * contract of la_prefix_mask_forward's m; the workspace is
 * la_workspace_bytes(LA_OP_PREFIX_MASK_BATCHED, ...) (a bucket sort per
 * batch).  Everything else as la_prefix_mask_forward. */
la_status la_prefix_mask_forward_batched(const void* q, const void* k,
                                         const void* v, const int64_t* m,
                                         int64_t B, int64_t H, int64_t n,
                                         int64_t d, la_dtype dtype,
                                         int32_t chunk, void* out, void* ws,
                                         size_t ws_bytes, void* stream);

/* Sliding-window causal normalised linear attention (LinearTile 1.0.1,
 * "Features": sliding-window attention, local context): query i sees the
 * `window` keys j with i - window < j <= i (keys 0..i while i < window):
 *     out_i = phi(Q_i) (S_i - S_{i-window}) / (phi(Q_i) . (z_i - z_{i-window})),
 * S_t, z_t the causal sums over keys 0..t (zero for t < 0).  window >= 1
 * (LA_ERR_SHAPE otherwise); window >= n is the causal form.  phi as for
 * la_causal_forward_phi.  q, out [B][Hq][n][d]; k, v [B][Hkv][n][d].  Needs
 * no workspace.  Offered where the kernel's tiles fit in LDS: bf16 with any
 * d <= 128, fp32 with d <= 64 (LA_ERR_UNSUPPORTED for fp32 with d > 64). */
la_status la_window_forward(const void* q, const void* k, const void* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                            int64_t d, la_dtype dtype, la_phi phi,
                            int64_t window, void* out, void* stream);

/* The causal (window = 0) or sliding-window (window >= 1) normalised form
 * over a table of sequences of any layout (LinearTile 1.0.1, "Features":
 * variable sequence length with no padding waste; the [batch, seq, dim]
 * inputs of trim-transformer 0.1.0's quickstart).  Sequence s, key/value head
 * g, query head h, token t of that sequence:
 *   K, V row at k + s*kv_strides[0] + (start(s) + t)*kv_strides[2] + g*kv_strides[1]
 *   Q, out row at q + s*q_strides[0] + (start(s) + t)*q_strides[2] + h*q_strides[1]
 * (strides in elements; the d features of a row are contiguous), where
 *   - cu_seqlens == NULL: nseq sequences of max_len tokens each, start(s) = 0
 *     (e.g. [B, n, H, d] with strides {n*H*d, d, H*d}; [B, H, n, d] with
 *     {H*n*d, n*d, d});
 *   - cu_seqlens != NULL: a DEVICE int64 array [nseq + 1], cu[0] = 0,
 *     nondecreasing, cu[nseq] <= total: sequence s is the packed token rows
 *     cu[s] .. cu[s+1] - 1 (start(s) = cu[s]) of buffers holding `total` rows
 *     (e.g. [total, H, d] with strides {0, d, H*d}); strides[0] must be 0 and
 *     every length at most max_len.  An inconsistent table is checked on
 *     the device: a sequence s with cu[s - 1] > cu[s] (s > 0), cu[s] > cu[s+1],
 *     cu[0] < 0, cu[s+1] > total or a length above max_len is left untouched
 *     (its out rows keep their contents) and LA_ERR_RANGE is recorded for
 *     la_workspace_status.
 * Query head h reads key/value head h / (Hq / Hkv).  phi as
 * la_causal_forward_phi.  window = 0: the causal form; S_final
 * [nseq][Hkv][d][d] and z_final [nseq][Hkv][d] (either may be NULL) receive
 * each sequence's final state (q = out = NULL: state only).  window >= 1:
 * query t sees keys t - window < j <= t of its sequence (S_final, z_final
 * must be NULL).  ws: la_workspace_bytes(LA_OP_SEQS, nseq, Hq, Hkv, max_len,
 * d, dtype, 0) bytes (covers both forms).  Offered where the kernels' tiles
 * fit in LDS: the causal form for every d <= 128, the window form for bf16
 * and for fp32 with d <= 64 (LA_ERR_UNSUPPORTED otherwise).  Errors as
 * elsewhere; LA_ERR_SHAPE for negative strides, heads of a row that overlap,
 * or a nonzero strides[0] with cu_seqlens. */
la_status la_causal_forward_strided(const void* q, const void* k, const void* v,
                                    const int64_t* cu_seqlens, int64_t nseq,
                                    int64_t max_len, int64_t total, int64_t Hq,
                                    int64_t Hkv, int64_t d,
                                    const int64_t* q_strides,
                                    const int64_t* kv_strides, la_dtype dtype,
                                    la_phi phi, int64_t window, void* out,
                                    float* S_final, float* z_final, void* ws,
                                    size_t ws_bytes, void* stream);

/* Gradients of the causal normalised form (LinearTile 1.0.1, "Project
 * Structure" and "Run Tests": the backward kernel of the training step) for
 * the loss L = sum_i dout_i . out_i, out as la_causal_forward_phi computes
 * it from q, k, v (recomputed here: nothing of the forward pass is kept):
 *   dq = dL/dq [B][Hq][n][d], dk = dL/dk and dv = dL/dv [B][Hkv][n][d], in
 *   dtype (dk and dv summed over the query heads of each key/value head).
 * With g_i = dout_i / den_i and beta_i = -(dout_i . out_i) / den_i:
 *   dphi(Q_i) = S_i g_i + beta_i z_i, dphi(K_j) = U_j V_j + u_j,
 *   dV_j = U_j^T phi(K_j), U_j = sum_{i>=j} phi(Q_i) g_i^T, u_j = sum_{i>=j}
 *   beta_i phi(Q_i); dq = dphi(Q) * phi'(q), dk = dphi(K) * phi'(k), with
 *   phi'(x) = 1 for x > 0 and 0 (relu + 1) or e^x (ELU + 1) otherwise, and
 *   1 for LA_PHI_FEATURES (gradients with respect to the features given).
 * phi is the map of the forward; ws: la_workspace_bytes(
 * LA_OP_CAUSAL_BACKWARD, B, Hq, Hkv, n, d, dtype, 0) bytes.  Offered for
 * d <= 64 (LA_ERR_UNSUPPORTED otherwise).  The gradient buffers must not
 * overlap each other or the inputs. */
la_status la_causal_backward(const void* q, const void* k, const void* v,
                             const void* dout, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t n, int64_t d,
                             la_dtype dtype, la_phi phi, void* dq, void* dk,
                             void* dv, void* ws, size_t ws_bytes,
                             void* stream);

/* One recurrent decode step (trim-transformer 0.1.0, "Key-value caching":
 * use and update the cache in one call).  For every (b, kv head g):
 *   S[b][g] += phi(k[b][g]) (x) v[b][g];  z[b][g] += phi(k[b][g]);
 * then for every query head h of g:
 *   out[b][h] = phi(q[b][h]) S[b][g] / (phi(q[b][h]) . z[b][g]).
 * q [B][Hq][d], k, v [B][Hkv][d], out [B][Hq][d] in dtype; S [B][Hkv][d][d]
 * and z [B][Hkv][d] fp32, updated in place.  Needs no workspace. */
la_status la_decode_step(const void* q, const void* k, const void* v,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                         la_dtype dtype, float* S, float* z, void* out,
                         void* stream);

/* The three normalised entry points with the feature map as an argument
 * (la_phi above); with LA_PHI_RELU1 each is exactly its plain counterpart.
 * Arguments, layouts, workspace and errors are as there: la_workspace_bytes
 * for the plain call's op and sizes covers either map.  A state built with
 * one map must be continued (la_decode_step_phi) with the same map.  With
 * LA_PHI_ELU1, phi(K) and phi(Q) are rounded to the input dtype before the
 * products (bf16 inputs: relative error about 2^-9 per weight). */
la_status la_forward_phi(const void* q, const void* k, const void* v,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                         int64_t d, la_dtype dtype, la_phi phi, void* out,
                         void* ws, size_t ws_bytes, void* stream);
la_status la_causal_forward_phi(const void* q, const void* k, const void* v,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                                int64_t d, la_dtype dtype, la_phi phi,
                                int32_t chunk, void* out, float* S_final,
                                float* z_final, void* ws, size_t ws_bytes,
                                void* stream);
la_status la_decode_step_phi(const void* q, const void* k, const void* v,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                             la_dtype dtype, la_phi phi, float* S, float* z,
                             void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LA_H */
