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
// is on fp32 MFMA (v_mfma_f32_32x32x2_f32 with la_device.h conventions, the
// masked scores P and A on v_mfma_f32_16x16x4f32 over all four waves; the
// feature map without the relu + 1 split), bf16 rows widened exactly as
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
         4 * (size_t)(2 * DP + 2 * C + (DP / 32) * C);
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

// Masked C x C scores on v_mfma_f32_16x16x4f32 (contraction index k = lane
// / 16, the other index lane % 16; accumulator entry rr of lane l is row
// 4 (l / 16) + rr, column l % 16), one 16 x 16 sub-block (key block kj,
// query block qi) per wave in turn, so that all four waves share the work:
//   acc[j][i] = sum_a X[j][a] Y[i][a] + add_i  for j <= i, else 0,
// stored to Z[i][j] (a 16-byte store per lane) and, with ZT, to ZT[j][i].
// X and Y are token-major (row stride LQ, DP features), Z and ZT have row
// stride LC.  A lane reads the four features 16 f + 4 (l / 16) .. + 3 of its
// rows with one 16-byte read and feeds them to four k-steps (feature
// 16 f + 4 (l / 16) + jj is the k index l / 16 of step (f, jj) in both
// operands).  Sub-blocks above the diagonal are only written where the
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
#pragma unroll
        for (int f = 0; f < DP / 16; ++f) {
          const f32x4 xa = *reinterpret_cast<const f32x4*>(X + (16 * kj + m) * LQ + 16 * f + 4 * kq);
          const f32x4 yb = *reinterpret_cast<const f32x4*>(Y + (16 * qi + m) * LQ + 16 * f + 4 * kq);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[jj], yb[jj], acc, 0, 0, 0);
        }
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
  constexpr int NIB = C / 32, NBB = DP / 32;
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
  __shared__ float su[DP], sinv[C], sbeta[C], spart[NBB][C];
  T* const sP = P_OVER_GT ? sGT : sPg;
  using SB = StateBlocks<DP>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
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

  const int ib = w % NIB, nb0 = w / NIB;
  constexpr int NB_STEP = NW / NIB;
  constexpr int NPW = (NBB + NB_STEP - 1) / NB_STEP;  // output blocks per wave
  const bool has_out = nb0 < NBB;
  // With one 32-row block per chunk and two 32-feature blocks (d = 64,
  // C = 32) the output blocks occupy two of the four waves; the gradient
  // pass then gives dphi(K) and dV to the other two (wave 2 + nb owns
  // feature block nb), so that all four work after A is formed.
  constexpr bool SPLIT_KV = GRAD && NIB == 1 && NBB == 2 && NW == 4;
  const bool kv_out = SPLIT_KV ? w >= 2 : has_out;  // this wave holds dphi(K) and dV blocks
  const int kv_nb0 = SPLIT_KV ? w - 2 : nb0;
  const int i = ib * 32 + (lane & 31);  // this lane's query row (num, dQ) or key row (dK, dV)

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
    f32x16 accK[NPW], accV[NPW];  // dphi(K)^T [a][j] and dV^T [b][j] blocks (key block ib)
#pragma unroll
    for (int uu = 0; uu < NPW; ++uu) {
      accK[uu] = f32x16{};
      accV[uu] = f32x16{};
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

      // ---- o^T = (S^T phi(Q)^T + V^T P^T) / den; partial dots dO . o for beta
      if (has_out) {
        // den_i = phi(Q_i) . z_pre + sum_j P[i][j] (P is 0 past the diagonal):
        // each half of the wave sums half of the features and keys
        float dpart = 0.0f;
#pragma unroll
        for (int a = 0; a < DP / 2; a += 4) {
          const f32x4 qv = *reinterpret_cast<const f32x4*>(sQ + i * LQ + h * (DP / 2) + a);
          const f32x4 zv = *reinterpret_cast<const f32x4*>(sz + h * (DP / 2) + a);
          dpart += qv[0] * zv[0] + qv[1] * zv[1] + qv[2] * zv[2] + qv[3] * zv[3];
        }
        for (int jb = 0; jb <= ib; ++jb) {
#pragma unroll
          for (int t = 0; t < 16; t += 4) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(sP + i * LC + jb * 32 + 16 * h + t);
            dpart += pv[0] + pv[1] + pv[2] + pv[3];
          }
        }
        const float den = dpart + __shfl_xor(dpart, 32);
        const float inv = i < nv ? 1.0f / den : 0.0f;  // rows past the end: no gradient
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = nb0 + uu * NB_STEP;
          if (nb < NBB) {
            f32x16 o = f32x16{};
            gemm_acc<T, DP / 16>(o, sST + nb * 32 * LQ, LQ, sQ + ib * 32 * LQ, LQ, lane);
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb)
              gemm_acc<T, 2>(o, sVT + nb * 32 * LC + jb * 32, LC, sP + ib * 32 * LC + jb * 32, LC, lane);
            float part = 0.0f;  // sum over this lane's 16 features b of dO[i][b] o[b][i]
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
              part += to_f(sG[i * LQ + nb * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3)]) * o[rr] * inv;
            part += __shfl_xor(part, 32);
            if (h == 0) spart[nb][i] = part;
          }
        }
        if (nb0 == 0 && h == 0) sinv[i] = inv;
      }
      __syncthreads();
      // beta_i = -inv_i (dO_i . o_i); G = dO * inv (token- and feature-major)
      if (tid < C) {
        float dot = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NBB; ++nb) dot += spart[nb][tid];
        sbeta[tid] = -sinv[tid] * dot;
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

      // ---- dphi(Q)^T [a][i] = S G^T + phi(K)^T A^T + z beta^T (staged in sQ),
      // dphi(K)^T += phi(Q)^T A, dV^T += G^T P (key block ib)
      f32x16 accQ[NPW];
      if (has_out) {
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = nb0 + uu * NB_STEP;
          accQ[uu] = f32x16{};
          if (nb < NBB) {
            gemm_acc<T, DP / 16>(accQ[uu], sS + nb * 32 * LQ, LQ, sG + ib * 32 * LQ, LQ, lane);
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb)
              gemm_acc<T, 2>(accQ[uu], sKT + nb * 32 * LC + jb * 32, LC, sP + ib * 32 * LC + jb * 32, LC, lane);
          }
        }
      }
      if (kv_out) {
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = kv_nb0 + uu * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int ib2 = ib; ib2 < NIB; ++ib2) {
              gemm_acc<T, 2>(accK[uu], sQT + nb * 32 * LC + ib2 * 32, LC, sAT + ib * 32 * LC + ib2 * 32, LC, lane);
              gemm_acc<T, 2>(accV[uu], sGT + nb * 32 * LC + ib2 * 32, LC, sPT + ib * 32 * LC + ib2 * 32, LC, lane);
            }
          }
        }
      }
      __syncthreads();  // sQ is free: dQ rows go out through it
      if (has_out) {
        const float bq = sbeta[i];
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = nb0 + uu * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int a = nb * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
              sQ[i * LQ + a] = cvt<T>(accQ[uu][rr] + sz[a] * bq);
            }
          }
        }
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
      if (kv_out) {
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = kv_nb0 + uu * NB_STEP;
          if (nb < NBB) {
            gemm_acc<T, DP / 16>(accK[uu], sU + nb * 32 * LQ, LQ, sV + ib * 32 * LQ, LQ, lane);
            gemm_acc<T, DP / 16>(accV[uu], sUT + nb * 32 * LQ, LQ, sK + ib * 32 * LQ, LQ, lane);
          }
        }
      }
      __syncthreads();  // sQ and sG are free: dK and dV rows go out through them
      if (kv_out) {
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = kv_nb0 + uu * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int a = nb * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
              sQ[i * LQ + a] = cvt<T>(accK[uu][rr] + su[a]);
              sG[i * LQ + a] = cvt<T>(accV[uu][rr]);
            }
          }
        }
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
  int e = la_internal::launch_seq_prefix(sc, C);  // forward prefix slots at a.ws
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
