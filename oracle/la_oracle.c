/*
 * la_oracle.c -- fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
 * benchmark).  Plain loops in fp64; no blocking, chunking or reordering
 * beyond the definitions below.  It shares no code with the HIP library.
 *
 * Sources (web pages this follows):
 *  - "nx_f32_linear_attention.nx source" (nishifamily.com), its header
 *    comment: the feature map phi(x) = relu(x) + 1, the key/value summary
 *    S = sum_j phi(K_j) (x) V_j (d x d) and z = sum_j phi(K_j), and the read
 *    out_i = phi(Q_i) S / (phi(Q_i) . z).  Each entry of S and z below is its
 *    own sum over the keys, written as the definition states it.
 *  - "LinearTile 1.0.1" (files.pythonhosted.org), section "How It Works":
 *    the same O = phi(Q) (phi(K)^T V) with phi(x) = ELU(x) + 1, the second
 *    feature map offered here (ELU with alpha = 1, the page naming no other:
 *    phi(x) = x + 1 for x > 0, exp(x) otherwise); section "Features": phi
 *    may be replaced at will -- any positive map, applied to q and k
 *    beforehand (LAO_PHI_FEATURES; the Python wrapper evaluates a test's map
 *    in fp64 and passes the results as fp64 inputs).
 *  - "trim-transformer 0.1.0" (pypi.org), section "Masking": query i attends
 *    to keys 0..m_i; a causal mask is m = arange(n).  Its kernel is
 *    Attn(Q,K,V) = Q K^T V with no feature map and no normaliser.
 *  - same page, section "Key-value caching": generation reuses and updates a
 *    cache token by token, linear in the number of generated tokens.
 *  - "LinearTile 1.0.1", section "Features": sliding-window attention (local
 *    context): query i sees only the last `window` keys, i - window < j <= i.
 *  - "LinearTile 1.0.1", sections "Project Structure" and "Run Tests": a
 *    backward kernel (core/kernels/backward.py) and its test: the gradients
 *    of the causal form, differentiated here term by term from the pairwise
 *    weights.
 *
 * Readings where the pages leave a step open:
 *  - no epsilon in the normaliser (relu + 1 >= 1 keeps the denominator >= 1;
 *    ELU + 1 > 0 keeps it positive);
 *  - causal queries see their own key (m_i = i is inclusive);
 *  - query head h uses key/value head h / (Hq / Hkv) (contiguous groups);
 *  - the decode step adds the new token to the state before reading it.
 *
 * Parity pins for every function here live in tests/test_oracle.py; none is
 * "parity unpinned".
 */
#include "la_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int lao_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Read element idx of an input array, widening fp32 or bf16 bits to fp64. */
static double rd(const void* p, int dtype, int64_t idx) {
  if (dtype == LAO_F32) return (double)((const float*)p)[idx];
  if (dtype == LAO_F64) return ((const double*)p)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* phi(x) = relu(x) + 1 (-0 and every negative value map to 1), or
 * phi(x) = ELU(x) + 1 = x + 1 for x > 0, exp(x) otherwise, or the identity
 * (features mapped beforehand). */
static double phi(double x, int kind) {
  if (kind == LAO_PHI_ELU1) return x > 0.0 ? x + 1.0 : exp(x);
  if (kind == LAO_PHI_FEATURES) return x;
  return (x > 0.0 ? x : 0.0) + 1.0;
}

/* Offset of row i of head h in a [B][H][n][d] tensor. */
static int64_t off4(int64_t b, int64_t h, int64_t i, int64_t H, int64_t n,
                    int64_t d) {
  return ((b * H + h) * n + i) * d;
}

/* out_row = phi(q_row) S / (phi(q_row) . z), with q_row read from q at off. */
static void normalised_read(const void* q, int dtype, int phik, int64_t off,
                            int64_t d, const double* S, const double* z,
                            double* pq, double* out_row) {
  double den = 0.0;
  for (int64_t a = 0; a < d; ++a) {
    pq[a] = phi(rd(q, dtype, off + a), phik);
    den += pq[a] * z[a];
  }
  for (int64_t c = 0; c < d; ++c) {
    double num = 0.0;
    for (int64_t a = 0; a < d; ++a) num += pq[a] * S[a * d + c];
    out_row[c] = num / den;
  }
}

void lao_forward(const void* q, const void* k, const void* v, int dtype,
                 int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                 int64_t d, const int64_t* rows, int64_t nrows, double* out) {
  const int64_t R = Hq / Hkv;
  const int64_t nr = rows ? nrows : n;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / R;
      double* S = (double*)malloc((size_t)(d * d) * sizeof(double));
      double* z = (double*)malloc((size_t)d * sizeof(double));
      double* pq = (double*)malloc((size_t)d * sizeof(double));
      double* pk = (double*)malloc((size_t)(n * d) * sizeof(double));
      const int64_t o = off4(b, g, 0, Hkv, n, d); /* key/value row 0 */
      for (int64_t e = 0; e < n * d; ++e) pk[e] = phi(rd(k, dtype, o + e), phik);
      /* z[a] = sum over all n keys of phi(K_j[a]);
       * S[a][c] = sum over all n keys of phi(K_j[a]) * V_j[c]. */
      for (int64_t a = 0; a < d; ++a) {
        double za = 0.0;
        for (int64_t j = 0; j < n; ++j) za += pk[j * d + a];
        z[a] = za;
        for (int64_t c = 0; c < d; ++c) {
          double sac = 0.0;
          for (int64_t j = 0; j < n; ++j) sac += pk[j * d + a] * rd(v, dtype, o + j * d + c);
          S[a * d + c] = sac;
        }
      }
      for (int64_t r = 0; r < nr; ++r) {
        const int64_t i = rows ? rows[r] : r;
        normalised_read(q, dtype, phik, off4(b, h, i, Hq, n, d), d, S, z, pq,
                        out + off4(b, h, r, Hq, nr, d));
      }
      free(S);
      free(z);
      free(pq);
      free(pk);
    }
  }
}

void lao_causal(const void* q, const void* k, const void* v, int dtype,
                int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                int64_t d, const int64_t* rows, int64_t nrows, double* out,
                double* S_final, double* z_final) {
  const int64_t R = Hq / Hkv;
  const int64_t nr = rows ? nrows : n;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t g = 0; g < Hkv; ++g) {
      double* S = (double*)calloc((size_t)(d * d), sizeof(double));
      double* z = (double*)calloc((size_t)d, sizeof(double));
      double* pk = (double*)malloc((size_t)d * sizeof(double));
      int64_t r = 0; /* next selected row */
      for (int64_t i = 0; i < n; ++i) {
        /* Add key/value i to the running state, then let query i read it. */
        const int64_t o = off4(b, g, i, Hkv, n, d);
        for (int64_t a = 0; a < d; ++a) {
          pk[a] = phi(rd(k, dtype, o + a), phik);
          z[a] += pk[a];
        }
        for (int64_t a = 0; a < d; ++a)
          for (int64_t c = 0; c < d; ++c)
            S[a * d + c] += pk[a] * rd(v, dtype, o + c);
        if (!q || !out || r >= nr) continue;
        if (rows && rows[r] != i) continue;
        for (int64_t h = g * R; h < (g + 1) * R; ++h)
          normalised_read(q, dtype, phik, off4(b, h, i, Hq, n, d), d, S, z,
                          pk, out + off4(b, h, r, Hq, nr, d));
        ++r;
      }
      if (S_final) memcpy(S_final + (b * Hkv + g) * d * d, S, (size_t)(d * d) * sizeof(double));
      if (z_final) memcpy(z_final + (b * Hkv + g) * d, z, (size_t)d * sizeof(double));
      free(S);
      free(z);
      free(pk);
    }
  }
}

void lao_window(const void* q, const void* k, const void* v, int dtype,
                int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                int64_t d, int64_t window, const int64_t* rows, int64_t nrows,
                double* out) {
  const int64_t R = Hq / Hkv;
  const int64_t nr = rows ? nrows : n;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t g = h / R;
      double* pq = (double*)malloc((size_t)d * sizeof(double));
      double* pk = (double*)malloc((size_t)(n * d) * sizeof(double));
      for (int64_t e = 0; e < n * d; ++e) pk[e] = phi(rd(k, dtype, off4(b, g, 0, Hkv, n, d) + e), phik);
      for (int64_t r = 0; r < nr; ++r) {
        const int64_t i = rows ? rows[r] : r;
        const int64_t lo = i - window + 1 > 0 ? i - window + 1 : 0;
        const int64_t oq = off4(b, h, i, Hq, n, d);
        for (int64_t a = 0; a < d; ++a) pq[a] = phi(rd(q, dtype, oq + a), phik);
        double* dst = out + off4(b, h, r, Hq, nr, d);
        for (int64_t c = 0; c < d; ++c) dst[c] = 0.0;
        double den = 0.0;
        /* the weight of key j is phi(Q_i) . phi(K_j); keys lo..i only */
        for (int64_t j = lo; j <= i; ++j) {
          const int64_t ok = off4(b, g, j, Hkv, n, d);
          double wij = 0.0;
          for (int64_t a = 0; a < d; ++a) wij += pq[a] * pk[j * d + a];
          den += wij;
          for (int64_t c = 0; c < d; ++c) dst[c] += wij * rd(v, dtype, ok + c);
        }
        for (int64_t c = 0; c < d; ++c) dst[c] /= den;
      }
      free(pq);
      free(pk);
    }
  }
}

/* phi'(x): relu + 1 -> 1 for x > 0 else 0; ELU + 1 -> 1 for x > 0 else e^x;
 * features given directly -> 1. */
static double dphi(double x, int kind) {
  if (kind == LAO_PHI_FEATURES) return 1.0;
  if (kind == LAO_PHI_ELU1) return x > 0.0 ? 1.0 : exp(x);
  return x > 0.0 ? 1.0 : 0.0;
}

void lao_causal_backward(const void* q, const void* k, const void* v,
                         const void* dout, int dtype, int phik, int64_t B,
                         int64_t Hq, int64_t Hkv, int64_t n, int64_t d,
                         double* dq, double* dk, double* dv) {
  const int64_t R = Hq / Hkv;
  if (dk) memset(dk, 0, (size_t)(B * Hkv * n * d) * sizeof(double));
  if (dv) memset(dv, 0, (size_t)(B * Hkv * n * d) * sizeof(double));
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t g = 0; g < Hkv; ++g) {
      double* pk = (double*)malloc((size_t)(n * d) * sizeof(double));
      double* pq = (double*)malloc((size_t)(n * d) * sizeof(double));
      double* D = (double*)malloc((size_t)n * sizeof(double));
      double* o = (double*)malloc((size_t)(n * d) * sizeof(double));
      double* gw = (double*)malloc((size_t)n * sizeof(double)); /* dL/dw_ij for one i */
      const int64_t okv = off4(b, g, 0, Hkv, n, d);
      for (int64_t e = 0; e < n * d; ++e) pk[e] = phi(rd(k, dtype, okv + e), phik);
      for (int64_t h = g * R; h < (g + 1) * R; ++h) {
        const int64_t oq = off4(b, h, 0, Hq, n, d);
        for (int64_t e = 0; e < n * d; ++e) pq[e] = phi(rd(q, dtype, oq + e), phik);
        /* the forward: D_i and out_i from the pairwise weights */
        for (int64_t i = 0; i < n; ++i) {
          double Di = 0.0;
          for (int64_t c = 0; c < d; ++c) o[i * d + c] = 0.0;
          for (int64_t j = 0; j <= i; ++j) {
            double w = 0.0;
            for (int64_t a = 0; a < d; ++a) w += pq[i * d + a] * pk[j * d + a];
            Di += w;
            for (int64_t c = 0; c < d; ++c) o[i * d + c] += w * rd(v, dtype, okv + j * d + c);
          }
          D[i] = Di;
          for (int64_t c = 0; c < d; ++c) o[i * d + c] /= Di;
        }
        /* the gradients, query by query */
        for (int64_t i = 0; i < n; ++i) {
          double* dqi = dq ? dq + oq + i * d : NULL;
          if (dqi)
            for (int64_t a = 0; a < d; ++a) dqi[a] = 0.0;
          for (int64_t j = 0; j <= i; ++j) {
            double w = 0.0, gv = 0.0;
            for (int64_t a = 0; a < d; ++a) w += pq[i * d + a] * pk[j * d + a];
            for (int64_t c = 0; c < d; ++c)
              gv += rd(dout, dtype, oq + i * d + c) * (rd(v, dtype, okv + j * d + c) - o[i * d + c]);
            gw[j] = gv / D[i];
            if (dqi)
              for (int64_t a = 0; a < d; ++a) dqi[a] += gw[j] * pk[j * d + a];
            if (dk)
              for (int64_t a = 0; a < d; ++a) dk[okv + j * d + a] += gw[j] * pq[i * d + a];
            if (dv)
              for (int64_t c = 0; c < d; ++c) dv[okv + j * d + c] += w * rd(dout, dtype, oq + i * d + c) / D[i];
          }
          if (dqi)
            for (int64_t a = 0; a < d; ++a) dqi[a] *= dphi(rd(q, dtype, oq + i * d + a), phik);
        }
      }
      if (dk)
        for (int64_t e = 0; e < n * d; ++e) dk[okv + e] *= dphi(rd(k, dtype, okv + e), phik);
      free(pk);
      free(pq);
      free(D);
      free(o);
      free(gw);
    }
  }
}

void lao_prefix_mask(const void* q, const void* k, const void* v, int dtype,
                     const int64_t* m, int64_t m_bstride, int64_t B, int64_t H,
                     int64_t n, int64_t d, const int64_t* rows, int64_t nrows,
                     double* out) {
  const int64_t nr = rows ? nrows : n;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      const int64_t* mb = m + b * m_bstride; /* this batch's mask */
      /* Lists L_t = {selected rows r : mb[row r] == t}, as a counting sort. */
      int64_t* start = (int64_t*)calloc((size_t)(n + 1), sizeof(int64_t));
      int64_t* list = (int64_t*)malloc((size_t)(nr > 0 ? nr : 1) * sizeof(int64_t));
      int64_t* fill = (int64_t*)malloc((size_t)(n + 1) * sizeof(int64_t));
      for (int64_t r = 0; r < nr; ++r) start[mb[rows ? rows[r] : r] + 1] += 1;
      for (int64_t t = 0; t < n; ++t) start[t + 1] += start[t];
      memcpy(fill, start, (size_t)(n + 1) * sizeof(int64_t));
      for (int64_t r = 0; r < nr; ++r) list[fill[mb[rows ? rows[r] : r]]++] = r;
      double* P = (double*)calloc((size_t)(d * d), sizeof(double));
      double* kt = (double*)malloc((size_t)d * sizeof(double));
      for (int64_t t = 0; t < n; ++t) {
        /* P = sum_{j <= t} K_j (x) V_j */
        const int64_t o = off4(b, h, t, H, n, d);
        for (int64_t a = 0; a < d; ++a) kt[a] = rd(k, dtype, o + a);
        for (int64_t a = 0; a < d; ++a)
          for (int64_t c = 0; c < d; ++c)
            P[a * d + c] += kt[a] * rd(v, dtype, o + c);
        /* every query whose mask ends at t reads Q_i . P */
        for (int64_t e = start[t]; e < start[t + 1]; ++e) {
          const int64_t r = list[e];
          const int64_t i = rows ? rows[r] : r;
          const int64_t oq = off4(b, h, i, H, n, d);
          double* dst = out + off4(b, h, r, H, nr, d);
          for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t a = 0; a < d; ++a)
              acc += rd(q, dtype, oq + a) * P[a * d + c];
            dst[c] = acc;
          }
        }
      }
      free(P);
      free(kt);
      free(start);
      free(list);
      free(fill);
    }
  }
}

void lao_decode_step(const void* q, const void* k, const void* v, int dtype,
                     int phik, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                     double* S, double* z, double* out) {
  const int64_t R = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t g = 0; g < Hkv; ++g) {
      double* Sg = S + (b * Hkv + g) * d * d;
      double* zg = z + (b * Hkv + g) * d;
      double* pk = (double*)malloc((size_t)d * sizeof(double));
      const int64_t o = (b * Hkv + g) * d;
      /* The new token joins the state first; then its queries read it. */
      for (int64_t a = 0; a < d; ++a) {
        pk[a] = phi(rd(k, dtype, o + a), phik);
        zg[a] += pk[a];
      }
      for (int64_t a = 0; a < d; ++a)
        for (int64_t c = 0; c < d; ++c)
          Sg[a * d + c] += pk[a] * rd(v, dtype, o + c);
      for (int64_t h = g * R; h < (g + 1) * R; ++h)
        normalised_read(q, dtype, phik, (b * Hq + h) * d, d, Sg, zg, pk,
                        out + (b * Hq + h) * d);
      free(pk);
    }
  }
}
