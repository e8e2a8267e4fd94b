/*
 * la_oracle.h -- fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this library: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no header, helper or constant with the
 * HIP library.
 *
 * What it computes (plain definitions, fp64 accumulation):
 *   phi(x) = max(x, 0) + 1                       (nx_f32_linear_attention.nx,
 *                                                 function la_phi), or
 *   phi(x) = ELU(x) + 1 (alpha = 1)              (LinearTile 1.0.1,
 *                                                 "How It Works"), or
 *   any positive phi the caller gives             (LinearTile 1.0.1,
 *                                                 "Features": phi replaceable)
 *   S = sum_j phi(K_j) (x) V_j,  z = sum_j phi(K_j)
 *   out_i = (phi(Q_i) S) / (phi(Q_i) . z)          (same page, header comment)
 * in the non-causal form (all keys), the causal form (keys 0..i), the
 * unnormalised prefix-mask form out_i = Q_i . sum_{j<=m_i} K_j (x) V_j
 * (trim-transformer 0.1.0, "Masking"), and one recurrent decode step
 * (trim-transformer 0.1.0, "Key-value caching").
 *
 * Layouts: q [B][Hq][n][d], k and v [B][Hkv][n][d], row-major, d fastest.
 * Query head h reads key/value head h / (Hq / Hkv).  Inputs are fp32
 * (dtype LAO_F32), raw bf16 bit patterns (LAO_BF16), widened exactly, or
 * fp64 (LAO_F64).
 *
 * Row selection: `rows` (ascending, each in [0, n)) picks which query rows
 * are produced; out is then [B][Hq][nrows][d].  rows == NULL means all rows
 * (nrows is ignored and out is [B][Hq][n][d]).
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LAO_F32 = 0, LAO_BF16 = 1, LAO_F64 = 2 };
/* phik: the feature map.  LAO_PHI_FEATURES: the identity on q and k (they
 * hold a positive map applied beforehand -- by a caller, or by the Python
 * wrapper, which evaluates a test's own map in fp64 and passes the results
 * as LAO_F64 inputs). */
enum { LAO_PHI_RELU1 = 0, LAO_PHI_ELU1 = 1, LAO_PHI_FEATURES = 2 };

/* Number of OpenMP threads the oracle uses. */
int lao_num_threads(void);

/* Non-causal normalised form: every query sees every key. */
void lao_forward(const void* q, const void* k, const void* v, int dtype,
                 int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                 int64_t d, const int64_t* rows, int64_t nrows, double* out);

/* Causal normalised form: query i sees keys 0..i.  q/out may be NULL (state
 * only).  S_final [B][Hkv][d][d] and z_final [B][Hkv][d] (either may be NULL)
 * receive the state after the last token. */
void lao_causal(const void* q, const void* k, const void* v, int dtype,
                int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                int64_t d, const int64_t* rows, int64_t nrows, double* out,
                double* S_final, double* z_final);

/* Sliding-window normalised form: query i sees keys max(0, i - window + 1)
 * .. i (window >= 1).  Written as the pairwise weights themselves:
 * out_i = sum_j (phi(Q_i) . phi(K_j)) V_j / sum_j phi(Q_i) . phi(K_j) over
 * those keys (no state). */
void lao_window(const void* q, const void* k, const void* v, int dtype,
                int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                int64_t d, int64_t window, const int64_t* rows, int64_t nrows,
                double* out);

/* Gradients of the causal normalised form (the training step's backward;
 * LinearTile 1.0.1, "Project Structure" / "Run Tests": a backward kernel and
 * its test) for the loss L = sum_i dout_i . out_i: with weights
 * w_ij = phi(Q_i) . phi(K_j) and D_i = sum_{j<=i} w_ij,
 *   dV_j      = sum_{i>=j} w_ij dout_i / D_i
 *   dL/dw_ij  = dout_i . (V_j - out_i) / D_i                 (j <= i)
 *   dQ_i      = phi'(Q_i) * sum_{j<=i} dL/dw_ij phi(K_j)
 *   dK_j      = phi'(K_j) * sum_{i>=j} dL/dw_ij phi(Q_i)
 * summed over the query heads of a key/value head for dK, dV.  phi' of
 * relu + 1 is 1 for x > 0 and 0 otherwise (0 at x = 0); of ELU + 1 it is 1 for
 * x > 0 and e^x otherwise; with LAO_PHI_FEATURES the gradients are with
 * respect to the features themselves.  Pairwise O(n^2 d) sums: the
 * definition differentiated term by term, no state.  dq [B][Hq][n][d], dk,
 * dv [B][Hkv][n][d]; any may be NULL. */
void lao_causal_backward(const void* q, const void* k, const void* v,
                         const void* dout, int dtype, int phik, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t n, int64_t d,
                         double* dq, double* dk, double* dv);

/* Unnormalised prefix-mask form, identity feature map: query i of batch b
 * sees keys 0..m[b * m_bstride + i], each in [0, n); m_bstride = 0 shares one
 * mask [n] among the batches, m_bstride = n gives each its own ([B][n]).
 * Every head of a batch uses that batch's mask. */
void lao_prefix_mask(const void* q, const void* k, const void* v, int dtype,
                     const int64_t* m, int64_t m_bstride, int64_t B, int64_t H,
                     int64_t n, int64_t d, const int64_t* rows, int64_t nrows,
                     double* out);

/* One recurrent decode step.  S [B][Hkv][d][d] and z [B][Hkv][d] are
 * updated in place with the new token's key and value, then every query
 * head reads the updated state.  q [B][Hq][d], k and v [B][Hkv][d],
 * out [B][Hq][d]. */
void lao_decode_step(const void* q, const void* k, const void* v, int dtype,
                     int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                     double* S, double* z, double* out);

#ifdef __cplusplus
}
#endif
#endif
