// la_window.hip -- sliding-window causal normalised linear attention (gfx950).
//
// LinearTile 1.0.1, "Features" (sliding-window attention, local context),
// with the normalised read of nx_f32_linear_attention.nx (header comment):
// query i sees the w keys j with i - w < j <= i (keys 0..i while i < w), so
//     out_i = phi(Q_i) (S_i - S_{i-w}) / (phi(Q_i) . (z_i - z_{i-w})),
// S_t and z_t the sums over keys 0..t (zero for t < 0).
//
// Chunked form, every term a sum of positive weights (no long difference is
// formed, so nothing cancels).  For query chunk c (rows cC .. cC + C - 1)
// let nfull = max(floor(w / C) - 1, 0) and e = c - nfull: the chunks e .. c - 1
// lie inside the window of every query of chunk c.  With the window state
// W(c) = the sum of the chunk states (S and z, fp32) of those chunks,
//     num_i = phi(Q_i) W(c) + sum_{j in chunk c, i - w < j <= i} P_ij V_j
//                           + sum_{j in chunks e - 2, e - 1, j > i - w} P_ij V_j,
// P_ij = phi(Q_i) . phi(K_j), and den_i likewise with V_j replaced by 1 (the
// rest of the window, i - w < j < eC, always lies in the two chunks before
// e: the "trailing" tile).  With key offset t from (e - 2) C and query offset
// u from cC, a trailing key counts iff t >= u + delta, delta = (nfull + 2) C -
// w + 1.  From chunk to chunk W gains the leading chunk's state and loses
// chunk e - 1's (the second half of the next trailing tile), in fp32.
// Chunks with a negative index hold no keys.
//
// Work decomposition: one 256-thread workgroup per (key/value head, segment
// of G chunks); it first sums the states of chunks c0 - nfull - 1 .. c0 - 1
// into W (the warm-up, so G >= nfull keeps it about as long as the
// segment), then walks its chunks: per chunk the leading tiles (phi(K)
// token- and feature-major, V feature-major), the trailing tile of 2C keys,
// W minus the trailing tile's second half, and for each of the R query
// heads of the group the masked scores, num and den on MFMA (la_device.h
// conventions), division in the epilogue, rows staged through LDS.  No
// workspace: the state never leaves the workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;

// Copy ROWS rows x DP features of one head (row stride d, row0 first) into
// LDS: tm[row * ldt + col] transformed by TMX and/or fm[col * ldf + row]
// transformed by FMX.  Rows at or past nvalid and features at or past d are
// stored as 0 (not phi(0)).  vec: d == DP, 16-byte pieces.
template <typename T, int DP, int ROWS, int TMX, int FMX>
__device__ __forceinline__ void stage(const T* __restrict__ base, int64_t row0, int nvalid, int d, bool vec, T* tm,
                                      int ldt, T* fm, int ldf, int tid) {
  if (vec) {
    constexpr int EPP = 16 / (int)sizeof(T);
    constexpr int PPR = DP / EPP;
    constexpr int NP = ROWS * PPR;
    constexpr int PER = (NP + NT - 1) / NT;
    union V { uint4 u; T e[EPP]; };
    V raw[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {  // every load first
      const int p = tid + k * NT;
      const int row = p / PPR, col = (p % PPR) * EPP;
      raw[k].u = make_uint4(0, 0, 0, 0);
      if (p < NP && row < nvalid) raw[k].u = *reinterpret_cast<const uint4*>(base + (row0 + row) * DP + col);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int p = tid + k * NT;
      if (p >= NP) break;
      const int row = p / PPR, col = (p % PPR) * EPP;
      V a, b;
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const float x = to_f(raw[k].e[e]);
        a.e[e] = row < nvalid ? cvt<T>(xform<TMX>(x)) : cvt<T>(0.0f);
        b.e[e] = row < nvalid ? cvt<T>(xform<FMX>(x)) : cvt<T>(0.0f);
      }
      if (TMX != XF_NONE) {
        T* dst = tm + row * ldt + col;  // rows of ldt elements are 8-byte aligned
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(a.u.x, a.u.y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(a.u.z, a.u.w);
      }
      if (FMX != XF_NONE) {
#pragma unroll
        for (int e = 0; e < EPP; ++e) fm[(col + e) * ldf + row] = b.e[e];
      }
    }
  } else {
    for (int idx = tid; idx < ROWS * DP; idx += NT) {
      const int row = idx / DP, col = idx % DP;
      const bool ok = row < nvalid && col < d;
      const float x = ok ? to_f(base[(row0 + row) * d + col]) : 0.0f;
      if (TMX != XF_NONE) tm[row * ldt + col] = cvt<T>(ok ? xform<TMX>(x) : 0.0f);
      if (FMX != XF_NONE) fm[col * ldf + row] = cvt<T>(ok ? xform<FMX>(x) : 0.0f);
    }
  }
}

// Rows of chunk x of a sequence of n tokens (0 for x < 0 or past the end).
__device__ __forceinline__ int chunk_rows(int64_t x, int C, int64_t n) {
  if (x < 0) return 0;
  const int64_t r = n - x * C;
  return r <= 0 ? 0 : (r < C ? (int)r : C);
}

template <typename T, int DP, int C, int PM>
__global__ __launch_bounds__(NT) void k_window(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, T* __restrict__ out, int64_t n, int d, int R,
                                               int64_t nchunks, int64_t G, int64_t nseg, int64_t nfull, int wlen,
                                               int delta) {
  constexpr int LQ = DP + PAD;      // token-major rows (Q, K, trailing K, W^T)
  constexpr int LC = C + PAD;       // feature-major rows of the leading chunk, scores
  constexpr int LC2 = 2 * C + PAD;  // feature-major rows of the trailing tile, its scores
  constexpr int NIB = C / 32;       // 32-row query / key blocks of a chunk
  constexpr int NTB = 2 * NIB;      // key blocks of the trailing tile
  constexpr int NBB = DP / 32;
  constexpr int PX = q_xform<PM>();  // phi on Q and on every K tile (no relu split here)
  static_assert(PM != PM_ID, "normalised form");
  __shared__ __attribute__((aligned(16))) T sQ[C * LQ];
  __shared__ __attribute__((aligned(16))) T sK[C * LQ];
  __shared__ __attribute__((aligned(16))) T sKT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sVT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sKtr[2 * C * LQ];
  __shared__ __attribute__((aligned(16))) T sKTtr[DP * LC2];
  __shared__ __attribute__((aligned(16))) T sVTtr[DP * LC2];
  __shared__ __attribute__((aligned(16))) T sST[DP * LQ];
  __shared__ __attribute__((aligned(16))) T sP[C * LC];
  __shared__ __attribute__((aligned(16))) T sPtr[C * LC2];
  // z of the window as a high part and the remainder in T, a zero row and a
  // ones row: the A operand rows of the denominator products
  __shared__ __attribute__((aligned(16))) T szh[DP + 16];
  __shared__ __attribute__((aligned(16))) T szl[DP + 16];
  __shared__ __attribute__((aligned(16))) T szero[DP + 16];
  __shared__ __attribute__((aligned(16))) T sones[16];
  using SB = StateBlocks<DP>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const bool vec = d == DP;
  const T* kb = k + bh * n * d;
  const T* vb = v + bh * n * d;
  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;

  f32x16 accW[SB::PER_WAVE];
#pragma unroll
  for (int s = 0; s < SB::PER_WAVE; ++s) accW[s] = f32x16{};
  float zW = 0.0f;  // z of the window, feature tid (tid < DP)
  auto add_state = [&](const T* KT, int ldk, const T* VT, int ldv, bool sub) {
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        if (sub) {
          f32x16 t = f32x16{};
          gemm_acc<T, C / 16>(t, KT + ma * 32 * ldk, ldk, VT + nb * 32 * ldv, ldv, lane);
#pragma unroll
          for (int r = 0; r < 16; ++r) accW[s][r] -= t[r];
        } else {
          gemm_acc<T, C / 16>(accW[s], KT + ma * 32 * ldk, ldk, VT + nb * 32 * ldv, ldv, lane);
        }
      }
    }
    if (tid < DP) {
      float zs = 0.0f;
      for (int t = 0; t < C; ++t) zs += to_f(KT[tid * ldk + t]);
      zW += sub ? -zs : zs;
    }
  };

  // ---- warm-up: W = states of chunks c0 - nfull - 1 .. c0 - 1 (the first
  // step subtracts chunk c0 - nfull - 1 again); none while nfull = 0
  for (int64_t x = (c0 - nfull - 1 > 0 ? c0 - nfull - 1 : 0); nfull > 0 && x < c0; ++x) {
    const int nvx = chunk_rows(x, C, n);
    stage<T, DP, C, XF_NONE, PX>(kb, x * C, nvx, d, vec, nullptr, 0, sKT, LC, tid);
    stage<T, DP, C, XF_NONE, XF_ID>(vb, x * C, nvx, d, vec, nullptr, 0, sVT, LC, tid);
    __syncthreads();
    add_state(sKT, LC, sVT, LC, false);
    __syncthreads();
  }
  if (tid < 16) {
    sones[tid] = cvt<T>(1.0f);
    szero[DP + tid] = cvt<T>(0.0f);
    szh[DP + tid] = cvt<T>(0.0f);
    szl[DP + tid] = cvt<T>(0.0f);
  }

  const int ib = w % NIB, nb0 = w / NIB;
  constexpr int NB_STEP = NW / NIB;
  constexpr int NPW = (NBB + NB_STEP - 1) / NB_STEP;  // output blocks per wave
  const bool has_out = nb0 < NBB;

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C, ce = c - nfull;  // the first chunk inside every window
    const int nv = chunk_rows(c, C, n);
    // leading chunk: phi(K) token- and feature-major, V feature-major;
    // trailing tile: chunks e - 2 and e - 1 (phi(K) both ways, V feature-major)
    stage<T, DP, C, PX, PX>(kb, t0, nv, d, vec, sK, LQ, sKT, LC, tid);
    stage<T, DP, C, XF_NONE, XF_ID>(vb, t0, nv, d, vec, nullptr, 0, sVT, LC, tid);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t x = ce - 2 + half;
      const int nvx = chunk_rows(x, C, n);
      const int64_t r0 = x < 0 ? 0 : x * C;
      stage<T, DP, C, PX, PX>(kb, r0, nvx, d, vec, sKtr + half * C * LQ, LQ, sKTtr + half * C, LC2, tid);
      stage<T, DP, C, XF_NONE, XF_ID>(vb, r0, nvx, d, vec, nullptr, 0, sVTtr + half * C, LC2, tid);
    }
    if (nfull > 0) {  // W loses chunk e - 1, which has left the chunks inside every window
      __syncthreads();
      add_state(sKTtr + C, LC2, sVTtr + C, LC2, true);
    }
    // W^T (sST[b][a] = W[a][b]) and z of the window in T
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) st_accT(sST + (e % SB::NB) * 32 * LQ + (e / SB::NB) * 32, LQ, accW[s], lane);
    }
    if (tid < DP) {
      const T zh = cvt<T>(zW);
      szh[tid] = zh;
      szl[tid] = cvt<T>(zW - to_f(zh));
      szero[tid] = cvt<T>(0.0f);
    }

    for (int r = 0; r < R; ++r) {
      const T* qh = q + (bh * R + r) * n * d;
      __syncthreads();  // the tiles above are written; the previous head is done with sQ, sP, sPtr
      stage<T, DP, C, PX, XF_NONE>(qh, t0, nv, d, vec, sQ, LQ, nullptr, 0, tid);
      __syncthreads();

      // ---- scores: chunk c (keys i - w < j <= i) into sP[i][j]; the trailing
      // tile (keys t >= u + delta) into sPtr[u][t]
      {
        int e = 0;
#pragma unroll
        for (int ib2 = 0; ib2 < NIB; ++ib2) {
#pragma unroll
          for (int jb = 0; jb < NIB + NTB; ++jb) {
            const bool lead = jb < NIB;
            if (lead && jb > ib2) continue;
            if ((e++ % NW) != w) continue;
            f32x16 acc = f32x16{};
            const int kb2 = lead ? jb : jb - NIB;
            gemm_acc<T, DP / 16>(acc, (lead ? sK : sKtr) + kb2 * 32 * LQ, LQ, sQ + ib2 * 32 * LQ, LQ, lane);
            const int i = ib2 * 32 + (lane & 31);
            const int lo = lead ? i - wlen + 1 : i + delta, hi = lead ? i : 2 * C;  // kept key offsets
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
              const int j = kb2 * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
              if (j < lo || j > hi) acc[rr] = 0.0f;
            }
            if (lead)
              st_accT(sP + ib2 * 32 * LC + kb2 * 32, LC, acc, lane);
            else
              st_accT(sPtr + ib2 * 32 * LC2 + kb2 * 32, LC2, acc, lane);
          }
        }
      }
      __syncthreads();

      // ---- out^T[b][i] = W^T phi(Q)^T + V_c^T P^T + V_tr^T P_tr^T, divided
      // by den_i = sum_j P_ij + sum_t (P_tr)_it + phi(Q_i) . z_W
      f32x16 accO[NPW];
      float inv = 1.0f;
      const int i = ib * 32 + (lane & 31);
      if (has_out) {
        const int mrow = lane & 31;
        Frag<T> e0;
        ld_frag(e0, mrow == 0 ? sones : szero);
        f32x16 dacc = f32x16{};
#pragma unroll
        for (int jb = 0; jb <= ib; ++jb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            Frag<T> fb;
            ld_frag(fb, sP + i * LC + jb * 32 + 16 * kk + 4 * h);
            mma(dacc, e0, fb);
          }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            Frag<T> fb;
            ld_frag(fb, sPtr + i * LC2 + tb * 32 + 16 * kk + 4 * h);
            mma(dacc, e0, fb);
          }
        const T* zrow = (mrow == 0) ? szh : (mrow == 16) ? szl : szero;
#pragma unroll
        for (int kk = 0; kk < DP / 16; ++kk) {
          Frag<T> fa, fb;
          ld_frag(fa, zrow + 16 * kk + 4 * h);
          ld_frag(fb, sQ + i * LQ + 16 * kk + 4 * h);
          mma(dacc, fa, fb);
        }
        inv = 1.0f / __shfl(dacc[0] + dacc[8], lane & 31);
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int nb = nb0 + u * NB_STEP;
          accO[u] = f32x16{};
          if (nb < NBB) {
            gemm_acc<T, DP / 16>(accO[u], sST + nb * 32 * LQ, LQ, sQ + ib * 32 * LQ, LQ, lane);
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb)
              gemm_acc<T, 2>(accO[u], sVT + nb * 32 * LC + jb * 32, LC, sP + ib * 32 * LC + jb * 32, LC, lane);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
              gemm_acc<T, 2>(accO[u], sVTtr + nb * 32 * LC2 + tb * 32, LC2, sPtr + ib * 32 * LC2 + tb * 32, LC2,
                             lane);
          }
        }
      }
      __syncthreads();  // every wave is past its reads of sQ: the rows go out through it
      if (has_out) {
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int nb = nb0 + u * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              sQ[i * LQ + nb * 32 + 8 * (e >> 2) + 4 * h + (e & 3)] = cvt<T>(accO[u][e] * inv);
          }
        }
      }
      __syncthreads();
      T* ob = out + (bh * R + r) * n * d;
      if (vec) {
        constexpr int EPP = 8 / (int)sizeof(T);  // 8-byte pieces (LDS rows are 8-byte aligned)
        constexpr int PPR = DP / EPP;
        typedef uint32_t U __attribute__((ext_vector_type(2)));
        for (int idx = tid; idx < nv * PPR; idx += NT) {
          const int rr = idx / PPR, col = EPP * (idx % PPR);
          __builtin_nontemporal_store(*reinterpret_cast<const U*>(sQ + rr * LQ + col),
                                      reinterpret_cast<U*>(ob + (t0 + rr) * d + col));
        }
      } else {
        for (int idx = tid; idx < nv * d; idx += NT) {
          const int rr = idx / d, col = idx % d;
          ob[(t0 + rr) * d + col] = sQ[rr * LQ + col];
        }
      }
    }

    // ---- W += dS(c)
    if (nfull > 0) add_state(sKT, LC, sVT, LC, false);
    __syncthreads();
  }
}

// LDS bytes of k_window<T, DP, C>: must fit one CU's 160 KiB.
constexpr size_t window_lds(int eb, int DP, int C) {
  const size_t LQ = DP + PAD, LC = C + PAD, LC2 = 2 * C + PAD;
  return (size_t)eb * (2 * C * LQ + 2 * DP * LC + 2 * C * LQ + 2 * DP * LC2 + DP * LQ + C * LC + C * LC2 +
                       3 * (DP + 16) + 16);
}

template <typename T, int DP, int C>
int run_window(const la_internal::Fwd& a, int64_t window) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int64_t nbh = a.B * a.Hkv, nchunks = (a.n + C - 1) / C;
  const int64_t nfull = window / C > 1 ? window / C - 1 : 0;
  const int delta = (int)((nfull + 2) * C - window + 1);
  // segments of at least nfull chunks (the warm-up is then about as long as
  // the walk), about 512 workgroups where the sequence allows more
  int64_t G = (nbh * nchunks + 511) / 512;
  if (G < nfull) G = nfull;
  if (G < 1) G = 1;
  if (G > nchunks) G = nchunks;
  const int64_t nseg = (nchunks + G - 1) / G;
  const int R = (int)(a.Hq / a.Hkv);
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* out = reinterpret_cast<T*>(a.out);
  const dim3 grid((unsigned)(nbh * nseg));
  if (a.phi == 1)
    k_window<T, DP, C, PM_ELU1><<<grid, NT, 0, st>>>(q, k, v, out, a.n, (int)a.d, R, nchunks, G, nseg, nfull, (int)window, delta);
  else if (a.phi == 2)
    k_window<T, DP, C, PM_FEAT><<<grid, NT, 0, st>>>(q, k, v, out, a.n, (int)a.d, R, nchunks, G, nseg, nfull, (int)window, delta);
  else
    k_window<T, DP, C, PM_RELU1><<<grid, NT, 0, st>>>(q, k, v, out, a.n, (int)a.d, R, nchunks, G, nseg, nfull, (int)window, delta);
  return (int)hipGetLastError();
}

}  // namespace

namespace la_internal {

int window_chunk(int elem_bytes, int DP) {
  for (int c : {64, 32})
    if (window_lds(elem_bytes, DP, c) <= kLdsLimit) return c;
  return 0;
}

int launch_window(const Fwd& a, int64_t window) {
  const int DP = padded_dim(a.d);
  const int C = window_chunk(a.dtype == 0 ? 4 : 2, DP);
#define LA_WIN(TT, DD, CC)                                                                  \
  if (DP == DD && C == CC) {                                                                \
    if constexpr (window_lds((int)sizeof(TT), DD, CC) <= kLdsLimit) return run_window<TT, DD, CC>(a, window); \
  }
  if (a.dtype == 0) {
    LA_WIN(float, 32, 64)
    LA_WIN(float, 64, 32)
  } else {
    LA_WIN(bf16, 32, 64)
    LA_WIN(bf16, 64, 64)
    LA_WIN(bf16, 128, 32)
  }
#undef LA_WIN
  return (int)hipErrorInvalidValue;
}

}  // namespace la_internal
