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
 *   la_workspace_bytes(...) bytes, owned by the caller.  Its contents before
 *   a call do not matter (no zero-fill is needed): every word a call reads
 *   there it wrote first, and the flags that order its workgroups must equal
 *   a value new to that call.  One workspace may serve calls of every kind
 *   and shape in turn (the library's workspace bytes for that shape at
 *   least); two calls that run concurrently must not share a workspace.
 * Errors.  Every argument check runs on the host before anything is
 *   enqueued; on failure nothing is launched and a nonzero la_status is
 *   returned (0 means success, as the nx page's functions return 0).
 *   A launch failure returns LA_ERR_LAUNCH.
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
  LA_ERR_LAUNCH = 8       /* the HIP runtime rejected a launch */
};

typedef int32_t la_dtype;
enum { LA_F32 = 0, LA_BF16 = 1 };

/* Feature map phi of the normalised forms.  LA_PHI_RELU1: phi(x) = relu(x)
 * + 1 (nx_f32_linear_attention.nx, function la_phi), what la_forward,
 * la_causal_forward and la_decode_step use.  LA_PHI_ELU1: phi(x) = ELU(x) +
 * 1 with alpha = 1, i.e. x + 1 for x > 0 and e^x otherwise (LinearTile
 * 1.0.1, "How It Works"), taken by the *_phi entry points below; any other
 * value gives LA_ERR_UNSUPPORTED. */
typedef int32_t la_phi;
enum { LA_PHI_RELU1 = 0, LA_PHI_ELU1 = 1 };

/* Operation codes for la_workspace_bytes. */
enum { LA_OP_FORWARD = 0, LA_OP_CAUSAL = 1, LA_OP_PREFIX_MASK = 2, LA_OP_PREFIX_MASK_BATCHED = 3 };

/* Human-readable name of a status code (static string, never NULL). */
const char* la_status_str(la_status s);

/* Workspace bytes needed by la_forward (op LA_OP_FORWARD), la_causal_forward
 * (LA_OP_CAUSAL), la_prefix_mask_forward (LA_OP_PREFIX_MASK, pass Hq = Hkv
 * = H) or la_prefix_mask_forward_batched (LA_OP_PREFIX_MASK_BATCHED, the
 * same) for these sizes.  Returns 0 if the arguments are invalid. */
size_t la_workspace_bytes(int32_t op, int64_t B, int64_t Hq, int64_t Hkv,
                          int64_t n, int64_t d, la_dtype dtype, int32_t chunk);

/* Non-causal normalised linear attention (nx_f32_linear_attention.nx: the
 * KV-summary loop over all keys, then the per-query read and division).
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

/* Unnormalised prefix-mask form Attn(Q,K,V) = Q K^T V (trim-transformer
 * 0.1.0): out_i = sum_{j <= m_i} (Q_i . K_j) V_j, no feature map, no
 * normaliser, no scale.  m is a device int64 array [n] shared by every batch
 * and head, any order, duplicates allowed; every m_i must lie in [0, n-1]
 * (not checked on the device: out-of-range values are a contract violation).
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
