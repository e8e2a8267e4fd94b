// la_backward.hip -- gradients of the causal normalised form (gfx950).
//
// LinearTile 1.0.1 ("Project Structure", "Run Tests") pairs its forward with
// a backward kernel.  For the loss L = sum_i dO_i . o_i of the causal form
// (o_i = phi(Q_i) S_i / (phi(Q_i) . z_i), S_i and z_i over keys 0..i, as in
// nx_f32_linear_attention.nx), with g_i = dO_i / den_i and
// beta_i = -(dO_i . o_i) / den_i (den_i = phi(Q_i) . z_i):
//   dphi(Q_i) = S_i g_i + beta_i z_i
//   dphi(K_j) = U_j V_j + u_j,   dV_j = U_j^T phi(K_j),
// where U_j = sum_{i >= j} phi(Q_i) g_i^T (d x d) and u_j = sum_{i >= j}
// beta_i phi(Q_i) -- a scan from the end, the mirror of S and z -- and
// dQ = dphi(Q) * phi'(Q), dK = dphi(K) * phi'(K).  Chunked (C rows, the mask
// M keeps j <= i), for chunk c with the states S_pre(c), z_pre(c) of the
// chunks before it and U_after(c), u_after(c) of the chunks after it:
//   P = M * (phi(Q_c) phi(K_c)^T), o = (phi(Q_c) S_pre + P V_c) / den,
//   A = M * (G V_c^T + beta 1^T)
//   dphi(Q_c) = G S_pre^T + beta z_pre^T + A phi(K_c)
//   dphi(K_c) = V_c U_after^T + 1 u_after^T + A^T phi(Q_c)
//   dV_c      = phi(K_c) U_after + P^T G.
// Passes (one launch each): the forward's segment states and their exclusive
// prefix (la_window.hip, k_wstate + k_scan); k_bwd<MODE_U>, per segment,
// walks its chunks recomputing o, G and beta and sums phi(Q)^T G and
// phi(Q)^T beta into the segment's U aggregate; k_rscan turns those into
// suffix sums (every segment from s on); k_bwd<MODE_GRAD> walks each segment
// again with S_pre carried forward from its prefix and U_after carried from
// its suffix (each chunk's phi(Q)^T G leaves it), writing dQ, dK and dV.
// Nothing is written per chunk to memory but the gradients.  Every product
// is on fp32 MFMA: the d x d states S and U in 32 x 32 blocks
// (v_mfma_f32_32x32x2_f32, la_device.h conventions), everything shaped like
// the chunk's rows (the masked scores P and A, the numerator, dQ, dK, dV) in
// 16 x 16 sub-blocks (v_mfma_f32_16x16x4f32) dealt out evenly to the four
// waves; the feature map without the relu + 1 split; bf16 rows widened exactly as
// they are staged: with relu + 1 every weight phi(Q_i) . phi(K_j) is close
// to d, so out_i is close to the mean of V and dphi(Q) = S g + beta z is a
// small difference of two large terms -- operands rounded to bf16 would
// leave errors of several percent of it.  phi'(x) is
// taken from the input rows re-read at the store (x > 0: 1; else 0 for
// relu + 1, e^x for ELU + 1; 1 for caller-applied features).  Query heads of
// a key/value head run one after the other; dK and dV collect them in
// registers.  Contiguous [B, H, n, d], d <= 64.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;

enum { MODE_U = 0, MODE_GRAD = 1 };

struct BwdArgs {
  const void* q; const void* k; const void* v; const void* dout;
  void* dq; void* dk; void* dv;
  int64_t n;
  int d, R;
  int64_t G, nseg;       // segments of G chunks per key/value head
  bool vec;
  const float* fstates;  // forward: exclusive prefix slots, (nseg + 1) per KV head
  float* ustates;        // U aggregates (MODE_U writes), then suffix sums (MODE_GRAD reads)
};

// phi'(x) of the feature map
template <int PM> __device__ __forceinline__ float dphi(float x) {
  if (PM == PM_FEAT) return 1.0f;
  if (PM == PM_ELU1) return x > 0.0f ? 1.0f : __expf(x);
  return x > 0.0f ? 1.0f : 0.0f;
}

// LDS bytes of k_bwd<T, DP, C, .., MODE_GRAD> (the larger mode).
constexpr size_t bwd_lds(int eb, int DP, int C) {
  const size_t LQ = DP + PAD, LC = C + PAD;
  return (size_t)eb * (4 * C * LQ + 4 * DP * LC + 4 * DP * LQ + 3 * C * LC) +
         4 * (size_t)(2 * DP + 2 * C + (DP / 16) * C);
}

// Copy a C x DP tile staged in LDS (row stride LQ) to rows t0 .. t0 + nv - 1
// of a head (row stride d), multiplying by phi'(x) of the same rows of src
// when src is given.
template <typename T, typename TT, int DP, int PM>
__device__ __forceinline__ void rows_out(const TT* tile, int LQ, int nv, int d, bool vec, T* dst, const T* src,
                                         int64_t t0, int tid) {
  if (vec) {
    constexpr int EPP = 4;  // four elements per piece (8 bytes of bf16, 16 of fp32)
    constexpr int PPR = DP / EPP;
    for (int idx = tid; idx < nv * PPR; idx += NT) {
      const int r = idx / PPR, col = EPP * (idx % PPR);
      float x[EPP];
#pragma unroll
      for (int e = 0; e < EPP; ++e) x[e] = to_f(tile[r * LQ + col + e]);
      if (src) {
#pragma unroll
        for (int e = 0; e < EPP; ++e) x[e] *= dphi<PM>(to_f(src[(t0 + r) * d + col + e]));
      }
#pragma unroll
      for (int e = 0; e < EPP; ++e) dst[(t0 + r) * d + col + e] = cvt<T>(x[e]);
    }
  } else {
    for (int idx = tid; idx < nv * d; idx += NT) {
      const int r = idx / d, col = idx % d;
      float x = to_f(tile[r * LQ + col]);
      if (src) x *= dphi<PM>(to_f(src[(t0 + r) * d + col]));
      dst[(t0 + r) * d + col] = cvt<T>(x);
    }
  }
}

// acc += sum_k X[r][k] Y[c][k] over the 16-wide k-blocks kb0 .. kb1 - 1 on
// v_mfma_f32_16x16x4f32 (contraction index k = lane / 16, the other index
// lane % 16), X and Y pointing at the first of 16 rows each (row strides ldx,
// ldy): accumulator entry rr of lane l is X-row 4 (l / 16) + rr, Y-row
// l % 16.  A lane reads the four entries 16 f + 4 (l / 16) .. + 3 of its rows
// with one 16-byte read and feeds them to four k-steps (entry
// 16 f + 4 (l / 16) + jj is the k index l / 16 of step (f, jj) in both
// operands).
__device__ __forceinline__ void mm16(f32x4& acc, const float* X, int ldx, const float* Y, int ldy, int kb0, int kb1,
                                     int lane) {
  const int m = lane & 15, kq = lane >> 4;
  const float* px = X + m * ldx + 4 * kq;
  const float* py = Y + m * ldy + 4 * kq;
  for (int f = kb0; f < kb1; ++f) {
    const f32x4 xa = *reinterpret_cast<const f32x4*>(px + 16 * f);
    const f32x4 yb = *reinterpret_cast<const f32x4*>(py + 16 * f);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[jj], yb[jj], acc, 0, 0, 0);
  }
}

// Masked C x C scores, one 16 x 16 sub-block (key block kj, query block qi)
// per wave in turn, so that all four waves share the work:
//   acc[j][i] = sum_a X[j][a] Y[i][a] + add_i  for j <= i, else 0,
// stored to Z[i][j] (a 16-byte store per lane) and, with ZT, to ZT[j][i].
// X and Y are token-major (row stride LQ, DP features), Z and ZT have row
// stride LC.  Sub-blocks above the diagonal are only written where the
// 32-wide products read them (inside a diagonal 32 x 32 block), as zeros.
template <int DP, int C>
__device__ __forceinline__ void scores16(const float* X, const float* Y, int LQ, const float* add, float* Z,
                                         float* ZT, int LC, int w, int lane) {
  constexpr int NB16 = C / 16;
  const int m = lane & 15, kq = lane >> 4;
  int e = 0;
#pragma unroll
  for (int qi = 0; qi < NB16; ++qi)
#pragma unroll
    for (int kj = 0; kj < NB16; ++kj) {
      if (kj > qi && (kj >> 1) != (qi >> 1)) continue;  // never read
      if ((e++ % NW) != w) continue;
      f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (kj <= qi) {
        mm16(acc, X + 16 * kj * LQ, LQ, Y + 16 * qi * LQ, LQ, 0, DP / 16, lane);
        const int iq = 16 * qi + m;
        const float ad = add ? add[iq] : 0.0f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[rr] = 16 * kj + 4 * kq + rr > iq ? 0.0f : acc[rr] + ad;
      }
      *reinterpret_cast<f32x4*>(Z + (16 * qi + m) * LC + 16 * kj + 4 * kq) = acc;
      if (ZT) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) ZT[(16 * kj + 4 * kq + rr) * LC + 16 * qi + m] = acc[rr];
      }
    }
}

template <typename TI, int DP, int C, int PM, int MODE>
__global__ __launch_bounds__(NT) void k_bwd(BwdArgs A) {
  using T = float;  // every tile and product in fp32, whatever the input type (see above)
  constexpr int LQ = DP + PAD, LC = C + PAD;
  constexpr int PX = q_xform<PM>();
  constexpr bool GRAD = MODE == MODE_GRAD;
  static_assert(PM != PM_ID, "normalised form");
  // token-major: phi(Q), phi(K), V, dO then G; feature-major: the same four
  __shared__ __attribute__((aligned(16))) T sQ[C * LQ];
  __shared__ __attribute__((aligned(16))) T sK[C * LQ];
  __shared__ __attribute__((aligned(16))) T sV[GRAD ? C * LQ : 8];  // token-major V: the gradients only
  __shared__ __attribute__((aligned(16))) T sG[C * LQ];
  __shared__ __attribute__((aligned(16))) T sQT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sKT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sVT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sGT[DP * LC];
  // S^T (rows b, k = a) and, for the gradients, S, U (rows a, k = b) and U^T
  __shared__ __attribute__((aligned(16))) T sST[DP * LQ];
  __shared__ __attribute__((aligned(16))) T sS[GRAD ? DP * LQ : 1];
  __shared__ __attribute__((aligned(16))) T sU[GRAD ? DP * LQ : 1];
  __shared__ __attribute__((aligned(16))) T sUT[GRAD ? DP * LQ : 1];
  // P[i][j], then A[i][j]; P^T and A^T ([j][i]).  The U pass keeps P over
  // G^T's tile (P is read before G^T is written, and a barrier separates
  // them), so that its LDS leaves room for two workgroups per CU.
  constexpr bool P_OVER_GT = !GRAD && C <= DP;  // P fits G^T's tile
  __shared__ __attribute__((aligned(16))) T sPg[P_OVER_GT ? 1 : C * LC];
  __shared__ __attribute__((aligned(16))) T sPT[GRAD ? C * LC : 1];
  __shared__ __attribute__((aligned(16))) T sAT[GRAD ? C * LC : 1];
  __shared__ __attribute__((aligned(16))) float sz[DP];
  __shared__ __attribute__((aligned(16))) float su[DP];
  __shared__ float sinv[C], sbeta[C], spart[DP / 16][C];
  T* const sP = P_OVER_GT ? sGT : sPg;
  using SB = StateBlocks<DP>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t u = blockIdx.x / A.nseg, seg = blockIdx.x % A.nseg;
  const int64_t n = A.n, nchunks = (n + C - 1) / C;
  const int64_t c0 = seg * A.G, c1 = (c0 + A.G < nchunks) ? c0 + A.G : nchunks;
  const int d = A.d, R = A.R;
  const bool vec = A.vec;
  const TI* kb = reinterpret_cast<const TI*>(A.k) + u * n * d;
  const TI* vb = reinterpret_cast<const TI*>(A.v) + u * n * d;

  // S (the forward state before chunk c0) and U (MODE_U: this segment's sum,
  // from 0; MODE_GRAD: the sum over chunks >= c0) in accumulators, z and u
  // for thread tid < DP
  f32x16 accS[SB::PER_WAVE], accU[SB::PER_WAVE];
  float zrun = 0.0f, urun[1] = {0.0f};
  {
    const float* fs = A.fstates + (u * (A.nseg + 1) + seg) * slot_elems(DP);
    const float* us = A.ustates + (u * (A.nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      accS[s] = f32x16{};
      accU[s] = f32x16{};
      if (e < SB::TOTAL) {
        ld_state_block<DP>(accS[s], fs, e / SB::NB, e % SB::NB, lane);
        if (GRAD) ld_state_block<DP>(accU[s], us, e / SB::NB, e % SB::NB, lane);
      }
    }
    if (tid < DP) {
      zrun = fs[DP * DP + tid];
      if (GRAD) urun[0] = us[DP * DP + tid];
    }
  }

  // The output-shaped products go in 16 x 16 sub-blocks (query or key block
  // qb of 16 rows, feature block fb of 16), NSB per wave: sub-block
  // e = w + NW s is (e / NFB, e % NFB), so that each wave keeps one feature
  // block and the waves' shares of every product are equal.
  constexpr int NQB = C / 16, NFB = DP / 16, NSB = NQB * NFB / NW;
  static_assert(NQB * NFB % NW == 0, "whole sub-blocks per wave");
  const int m16 = lane & 15, kq = lane >> 4;

  // Rows are requested one step ahead: the next chunk's K and V while this
  // chunk's are in use, the next query head's (or the next chunk's first)
  // Q and dO rows while this head's are.
  StageRegs<TI, DP, C> rK, rV, rQ, rO;
  auto load_q = [&](int64_t c, int r) {
    const int64_t hq = u * R + r;
    const int nvl = chunk_rows(c, C, n);
    stage_load<TI, DP, C>(rQ, reinterpret_cast<const TI*>(A.q) + hq * n * d, d, c * C, nvl, vec, tid);
    stage_load<TI, DP, C>(rO, reinterpret_cast<const TI*>(A.dout) + hq * n * d, d, c * C, nvl, vec, tid);
  };
  stage_load<TI, DP, C>(rK, kb, d, c0 * C, chunk_rows(c0, C, n), vec, tid);
  stage_load<TI, DP, C>(rV, vb, d, c0 * C, chunk_rows(c0, C, n), vec, tid);
  load_q(c0, 0);

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = chunk_rows(c, C, n);
    __syncthreads();  // the previous chunk is done with every tile
    stage_put<TI, T, DP, C, PX, PX>(rK, kb, d, t0, nv, d, vec, sK, LQ, sKT, LC, tid);
    stage_put<TI, T, DP, C, GRAD ? XF_ID : XF_NONE, XF_ID>(rV, vb, d, t0, nv, d, vec, GRAD ? sV : nullptr, LQ,
                                                        sVT, LC, tid);
    if (c + 1 < c1) {
      stage_load<TI, DP, C>(rK, kb, d, (c + 1) * C, chunk_rows(c + 1, C, n), vec, tid);
      stage_load<TI, DP, C>(rV, vb, d, (c + 1) * C, chunk_rows(c + 1, C, n), vec, tid);
    }
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        st_accT(sST + nb * 32 * LQ + ma * 32, LQ, accS[s], lane);  // sST[b][a] = S[a][b]
        if (GRAD) st_acc(sS + ma * 32 * LQ + nb * 32, LQ, accS[s], lane);
      }
    }
    if (tid < DP) sz[tid] = zrun;
    // dphi(K)^T[a][j] and dV^T[b][j] sub-blocks (key block e / NFB, feature
    // block e % NFB), summed over the query heads
    f32x4 accK[NSB], accV[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      accK[sb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      accV[sb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    for (int r = 0; r < R; ++r) {
      const int64_t hq = u * R + r;
      const TI* qh = reinterpret_cast<const TI*>(A.q) + hq * n * d;
      const TI* oh = reinterpret_cast<const TI*>(A.dout) + hq * n * d;
      __syncthreads();  // the previous head is done with sQ, sG, sP and the rest
      stage_put<TI, T, DP, C, PX, PX>(rQ, qh, d, t0, nv, d, vec, sQ, LQ, sQT, LC, tid);
      stage_put<TI, T, DP, C, XF_ID, XF_NONE>(rO, oh, d, t0, nv, d, vec, sG, LQ, nullptr, 0, tid);
      if (r + 1 < R)
        load_q(c, r + 1);
      else if (c + 1 < c1)
        load_q(c + 1, 0);
      __syncthreads();

      // ---- P = M * (phi(Q) phi(K)^T): sP[i][j] (and sPT[j][i])
      scores16<DP, C>(sK, sQ, LQ, nullptr, sP, GRAD ? sPT : nullptr, LC, w, lane);
      __syncthreads();

      // ---- 1 / den_i with den_i = phi(Q_i) . z_pre + sum_j P[i][j] (TPQ
      // threads per query, each summing a share of the features and of the
      // keys of the written 32-blocks of P's row), and the numerator blocks
      // o^T[b][i] = sum_a S^T[b][a] phi(Q)[i][a] + sum_j V^T[b][j] P[i][j]
      // (keys j < 16 (qb + 1): P is 0 past the diagonal) with their partial
      // dots dO . o per feature block (scaled by 1 / den_i^2 in beta)
      {
        constexpr int TPQ = NT / C, FPT = DP / TPQ, KPT = C / TPQ;
        static_assert(FPT % 4 == 0 && KPT % 4 == 0, "16-byte shares");
        const int qi = tid / TPQ, pp = tid % TPQ, jlim = 32 * (qi / 32 + 1);
        float dd = 0.0f;
#pragma unroll
        for (int a = pp * FPT; a < (pp + 1) * FPT; a += 4) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(sQ + qi * LQ + a);
          const f32x4 zv = *reinterpret_cast<const f32x4*>(sz + a);
          dd += qv[0] * zv[0] + qv[1] * zv[1] + qv[2] * zv[2] + qv[3] * zv[3];
        }
#pragma unroll
        for (int jj = pp * KPT; jj < (pp + 1) * KPT; jj += 4) {
          if (jj < jlim) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(sP + qi * LC + jj);
            dd += pv[0] + pv[1] + pv[2] + pv[3];
          }
        }
#pragma unroll
        for (int off = 1; off < TPQ; off <<= 1) dd += __shfl_xor(dd, off);
        if (pp == 0) sinv[qi] = qi < nv ? 1.0f / dd : 0.0f;  // rows past the end: no gradient
      }
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int e = w + NW * sb, qb = e / NFB, fb = e % NFB;
        f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mm16(o, sST + 16 * fb * LQ, LQ, sQ + 16 * qb * LQ, LQ, 0, NFB, lane);
        mm16(o, sVT + 16 * fb * LC, LC, sP + 16 * qb * LC, LC, 0, qb + 1, lane);
        const int qi = 16 * qb + m16;  // o[rr]: feature 16 fb + 4 kq + rr of query qi
        const f32x4 g = *reinterpret_cast<const f32x4*>(sG + qi * LQ + 16 * fb + 4 * kq);
        float part = g[0] * o[0] + g[1] * o[1] + g[2] * o[2] + g[3] * o[3];
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (kq == 0) spart[fb][qi] = part;
      }
      __syncthreads();
      // beta_i = -inv_i (dO_i . o_i) = -inv_i^2 (dO_i . num_i); G = dO * inv
      // (token- and feature-major)
      if (tid < C) {
        float dot = 0.0f;
#pragma unroll
        for (int fb = 0; fb < NFB; ++fb) dot += spart[fb][tid];
        const float iv = sinv[tid];
        sbeta[tid] = -(iv * iv) * dot;
      }
      for (int idx = tid; idx < C * DP; idx += NT) {
        const int qi = idx / DP, b = idx % DP;
        const T gq = cvt<T>(to_f(sG[qi * LQ + b]) * sinv[qi]);
        sG[qi * LQ + b] = gq;
        sGT[b * LC + qi] = gq;
      }
      __syncthreads();

      if (!GRAD) {
        // ---- U += phi(Q)^T G, u += phi(Q)^T beta
#pragma unroll
        for (int s = 0; s < SB::PER_WAVE; ++s) {
          const int e = w + NW * s;
          if (e < SB::TOTAL)
            gemm_acc<T, C / 16>(accU[s], sQT + (e / SB::NB) * 32 * LC, LC, sGT + (e % SB::NB) * 32 * LC, LC, lane);
        }
        if (tid < DP) {
          float acc = 0.0f;
          for (int t = 0; t < C; ++t) acc += sbeta[t] * to_f(sQT[tid * LC + t]);
          urun[0] += acc;
        }
        continue;
      }

      // ---- A = M * (G V^T + beta 1^T): sP[i][j] (P is no longer needed
      // there) and sAT[j][i]
      scores16<DP, C>(sV, sG, LQ, sbeta, sP, sAT, LC, w, lane);
      __syncthreads();

      // ---- dphi(Q)^T[a][i] = sum_b S[a][b] G[i][b] + sum_j K^T[a][j] A[i][j]
      // (+ z_a beta_i, then staged in sQ: nothing reads phi(Q) token-major
      // any more), dphi(K)^T[a][j] += sum_i Q^T[a][i] A^T[j][i] and
      // dV^T[b][j] += sum_i G^T[b][i] P^T[j][i] over the queries i >= 16 jb
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int e = w + NW * sb, qb = e / NFB, fb = e % NFB;
        f32x4 aq = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mm16(aq, sS + 16 * fb * LQ, LQ, sG + 16 * qb * LQ, LQ, 0, NFB, lane);
        mm16(aq, sKT + 16 * fb * LC, LC, sP + 16 * qb * LC, LC, 0, qb + 1, lane);
        mm16(accK[sb], sQT + 16 * fb * LC, LC, sAT + 16 * qb * LC, LC, qb, NQB, lane);
        mm16(accV[sb], sGT + 16 * fb * LC, LC, sPT + 16 * qb * LC, LC, qb, NQB, lane);
        const int qi = 16 * qb + m16, a0 = 16 * fb + 4 * kq;
        const float bq = sbeta[qi];
        const f32x4 zv = *reinterpret_cast<const f32x4*>(sz + a0);
        *reinterpret_cast<f32x4*>(sQ + qi * LQ + a0) = aq + zv * bq;
      }
      // ---- U -= phi(Q)^T G, u -= phi(Q)^T beta: the states after chunk c
#pragma unroll
      for (int s = 0; s < SB::PER_WAVE; ++s) {
        const int e = w + NW * s;
        if (e < SB::TOTAL) {
          f32x16 t = f32x16{};
          gemm_acc<T, C / 16>(t, sQT + (e / SB::NB) * 32 * LC, LC, sGT + (e % SB::NB) * 32 * LC, LC, lane);
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) accU[s][rr] -= t[rr];
        }
      }
      if (tid < DP) {
        float acc = 0.0f;
        for (int t = 0; t < C; ++t) acc += sbeta[t] * to_f(sQT[tid * LC + t]);
        urun[0] -= acc;
      }
      __syncthreads();
      rows_out<TI, T, DP, PM>(sQ, LQ, nv, d, vec, reinterpret_cast<TI*>(A.dq) + hq * n * d, qh, t0, tid);
    }

    if (GRAD) {
      // ---- the state terms: dphi(K)^T += U V^T + u 1^T, dV^T += U^T phi(K)^T
#pragma unroll
      for (int s = 0; s < SB::PER_WAVE; ++s) {
        const int e = w + NW * s;
        if (e < SB::TOTAL) {
          const int ma = e / SB::NB, nb = e % SB::NB;
          st_acc(sU + ma * 32 * LQ + nb * 32, LQ, accU[s], lane);
          st_accT(sUT + nb * 32 * LQ + ma * 32, LQ, accU[s], lane);
        }
      }
      if (tid < DP) su[tid] = urun[0];
      __syncthreads();
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int e = w + NW * sb, jb = e / NFB, fb = e % NFB;
        mm16(accK[sb], sU + 16 * fb * LQ, LQ, sV + 16 * jb * LQ, LQ, 0, NFB, lane);
        mm16(accV[sb], sUT + 16 * fb * LQ, LQ, sK + 16 * jb * LQ, LQ, 0, NFB, lane);
      }
      __syncthreads();  // sQ and sG are free: dK and dV rows go out through them
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int e = w + NW * sb, jb = e / NFB, fb = e % NFB;
        const int kj = 16 * jb + m16, a0 = 16 * fb + 4 * kq;
        const f32x4 uv = *reinterpret_cast<const f32x4*>(su + a0);
        *reinterpret_cast<f32x4*>(sQ + kj * LQ + a0) = accK[sb] + uv;
        *reinterpret_cast<f32x4*>(sG + kj * LQ + a0) = accV[sb];
      }
      __syncthreads();
      rows_out<TI, T, DP, PM>(sQ, LQ, nv, d, vec, reinterpret_cast<TI*>(A.dk) + u * n * d, kb, t0, tid);
      rows_out<TI, T, DP, PM>(sG, LQ, nv, d, vec, reinterpret_cast<TI*>(A.dv) + u * n * d, nullptr, t0, tid);
    }

    // ---- S += phi(K_c)^T V_c, z += column sums of phi(K_c)
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        gemm_acc<T, C / 16>(accS[s], sKT + ma * 32 * LC, LC, sVT + nb * 32 * LC, LC, lane);
      }
    }
    if (tid < DP) zrun += row_sum<T, C>(sKT, tid);
  }

  if (!GRAD) {  // this segment's U aggregate (row-major [a][b], then u)
    float* dst = A.ustates + (u * (A.nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) st_state_block<DP>(dst, accU[s], e / SB::NB, e % SB::NB, lane);
    }
    if (tid < DP) dst[DP * DP + tid] = urun[0];
  }
}

// Suffix sums of the U aggregates: slot s <- sum of slots s .. nseg - 1, in a
// fixed order (one thread per slot element).
__global__ __launch_bounds__(NT) void k_rscan(float* __restrict__ ws, int64_t nseg, int64_t E) {
  const int64_t u = blockIdx.x;
  const int64_t e = (int64_t)blockIdx.y * NT + threadIdx.x;
  if (e >= E) return;
  float* base = ws + u * (nseg + 1) * E + e;
  float run = 0.0f;
  for (int64_t s = nseg - 1; s >= 0; --s) {
    run += base[s * E];
    base[s * E] = run;
  }
}

template <typename T, int DP, int C, int MODE>
void launch_bwd(const BwdArgs& A, int phi, dim3 grid, hipStream_t st) {
  if (phi == 1)
    k_bwd<T, DP, C, PM_ELU1, MODE><<<grid, NT, 0, st>>>(A);
  else if (phi == 2)
    k_bwd<T, DP, C, PM_FEAT, MODE><<<grid, NT, 0, st>>>(A);
  else
    k_bwd<T, DP, C, PM_RELU1, MODE><<<grid, NT, 0, st>>>(A);
}

template <typename T, int DP, int C>
int run_backward(const la_internal::BwdCall& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const la_internal::SeqCall sc = la_internal::backward_seqcall(a);
  const la_internal::Plan p = la_internal::seq_plan(sc, C);
  const int64_t units = a.B * a.Hkv;
  // forward prefix slots at a.ws: bf16 with relu + 1 or caller-applied
  // features on the bf16-MFMA state pass (exact products), otherwise on fp32
  // tiles
  int e = a.dtype != 0 ? la_internal::launch_state_bf16_exact(a.k, a.v, units, a.n, (int)a.d, a.phi, C, p.nchunks,
                                                               p.G, p.nseg, reinterpret_cast<float*>(a.ws), a.stream)
                       : -1;
  if (e == -1)
    e = la_internal::launch_seq_prefix(sc, C);
  else if (e == 0)
    e = la_internal::launch_scan(reinterpret_cast<float*>(a.ws), units, p.nseg, DP, (int)a.d, nullptr, nullptr,
                                 a.stream);
  if (e != 0) return e;
  float* fstates = reinterpret_cast<float*>(a.ws);
  float* ustates = fstates + units * (p.nseg + 1) * slot_elems(DP);
  BwdArgs A{a.q, a.k, a.v, a.dout, a.dq, a.dk, a.dv, a.n, (int)a.d, (int)(a.Hq / a.Hkv), p.G, p.nseg, sc.vec,
            fstates, ustates};
  const dim3 grid((unsigned)(units * p.nseg));
  launch_bwd<T, DP, C, MODE_U>(A, a.phi, grid, st);
  const int64_t E = slot_elems(DP);
  k_rscan<<<dim3((unsigned)units, (unsigned)((E + NT - 1) / NT)), NT, 0, st>>>(ustates, p.nseg, E);
  launch_bwd<T, DP, C, MODE_GRAD>(A, a.phi, grid, st);
  return (int)hipGetLastError();
}

}  // namespace

namespace la_internal {

int backward_chunk(int elem_bytes, int DP) {
  (void)elem_bytes;  // fp32 tiles for either input type
  if (DP > 64) return 0;
  for (int c : {64, 32})
    if (bwd_lds(4, DP, c) <= kLdsLimit) return c;
  return 0;
}

SeqCall backward_seqcall(const BwdCall& a) {
  SeqCall s{};
  s.q = a.q; s.k = a.k; s.v = a.v; s.out = nullptr;
  const int64_t n = a.n, d = a.d;
  s.S = Seqs{a.Hq * n * d, n * d, d, a.Hkv * n * d, n * d, d, nullptr, n, a.B * n};
  s.nseq = a.B; s.Hq = a.Hq; s.Hkv = a.Hkv; s.d = d;
  s.dtype = a.dtype; s.phi = a.phi; s.window = 0;
  s.vec = d == padded_dim(d);
  s.ws = a.ws; s.ctl = nullptr; s.stream = a.stream;
  return s;
}

size_t backward_ws_bytes(const BwdCall& a) {
  const int C = backward_chunk(a.dtype == 0 ? 4 : 2, padded_dim(a.d));
  if (C == 0) return 0;
  return 2 * state_bytes(seq_plan(backward_seqcall(a), C), a.B, a.Hkv);  // forward prefixes, then U sums
}

int launch_backward(const BwdCall& a) {
  const int DP = padded_dim(a.d);
  const int C = backward_chunk(a.dtype == 0 ? 4 : 2, DP);
#define LA_BWD(TT, DD, CC) \
  if (DP == DD && C == CC) return run_backward<TT, DD, CC>(a);
  if (a.dtype == 0) {
    LA_BWD(float, 32, 64)
    LA_BWD(float, 64, 32)
  } else {
    LA_BWD(bf16, 32, 64)
    LA_BWD(bf16, 64, 32)
  }
#undef LA_BWD
  return (int)hipErrorInvalidValue;
}

}  // namespace la_internal
