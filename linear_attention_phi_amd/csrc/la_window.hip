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
//
// The same kernel with WIN = false is the causal form (w covers every
// earlier key): W starts from the exclusive prefix of the segment's first
// chunk (k_wstate's segment states, scanned by k_scan), there is no trailing
// tile, and W gains each chunk's state.  Both take their rows through a
// sequence table (Seqs): per sequence s, key/value head g and query head h,
// row t of K and V at k + s kb + start(s) kt + g kh + t kt and of Q and out at
// q + s qb + start(s) qt + h qh + t qt, where start(s) = cu[s] for packed
// sequences of different lengths (varlen: cu[s] .. cu[s + 1] - 1 are the
// tokens of sequence s, nothing padded) and 0 for a fixed length n.  Contiguous
// [B, H, n, d] (BHND), [B, n, H, d] (BNHD, as trim-transformer's
// [batch, seq, dim] quickstart) and packed [tokens, H, d] are all strides of
// this table.  A sequence whose entries of cu fall outside [0, total] or
// decrease (cu[s - 1] <= cu[s] <= cu[s + 1] must hold), or whose length
// exceeds the maximum the call states, is left empty and the fault is
// recorded in the control block (la_workspace_status: LA_ERR_RANGE).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_ctl.h"
#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;
using la_internal::Seqs;

// Sequence s of the table: its first token and its length (0, with the
// error recorded, if the table is inconsistent).
struct SeqSpan {
  int64_t start, len;
};
__device__ __forceinline__ SeqSpan seq_span(const Seqs& S, int64_t s, la_internal::Ctl* ctl, bool report) {
  if (!S.cu) return {0, S.n};
  const int64_t a = S.cu[s], b = S.cu[s + 1], prev = s > 0 ? S.cu[s - 1] : 0;
  if (a < prev || b < a || b > S.total || b - a > S.n) {  // (cu[0] itself must be >= 0)
    if (report) la_ctl::ctl_fail(ctl, la_internal::kErrRange);
    return {0, 0};
  }
  return {a, b - a};
}

struct WinArgs {
  const void* q; const void* k; const void* v; void* out;
  Seqs S;
  int d, R;
  int64_t Hkv, G, nseg;  // segments of G chunks; nseg per (sequence, KV head) in the grid
  int64_t nfull;         // window form: chunks inside every window of a query chunk (see above)
  int wlen, delta;       // window form: w, and the trailing tile's mask offset
  bool vec;              // 16-byte row pieces
  float* states;         // causal form: (nseg + 1) slots per (sequence, KV head), scanned
  la_internal::Ctl* ctl;
};

// The window state W (fp32 accumulators of the la_device.h layout, plus z of
// thread tid < DP) and its updates from feature-major phi(K) and V tiles.
template <typename T, int DP, int C>
struct WinState {
  using SB = StateBlocks<DP>;
  f32x16 acc[SB::PER_WAVE];
  float z = 0.0f;
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) acc[s] = f32x16{};
    z = 0.0f;
  }
  __device__ __forceinline__ void add(const T* KT, int ldk, const T* VT, int ldv, bool sub, int w, int lane, int tid) {
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        if (sub) {
          f32x16 t = f32x16{};
          gemm_acc<T, C / 16>(t, KT + ma * 32 * ldk, ldk, VT + nb * 32 * ldv, ldv, lane);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[s][r] -= t[r];
        } else {
          gemm_acc<T, C / 16>(acc[s], KT + ma * 32 * ldk, ldk, VT + nb * 32 * ldv, ldv, lane);
        }
      }
    }
    if (tid < DP) {
      float zs = 0.0f;
      for (int t = 0; t < C; ++t) zs += to_f(KT[tid * ldk + t]);
      z += sub ? -zs : zs;
    }
  }
};

// ------------------------------------------------------------------ k_wstate
// Causal form's state pass: the segment's chunk states summed (S row-major,
// then z: the slot layout of k_scan), zeros for segments past a sequence's
// end.
// TT: the tile type (T, or fp32 for the backward's fp32 prefixes of bf16 rows).
template <typename T, int DP, int C, int PM, typename TT = T>
__global__ __launch_bounds__(NT) void k_wstate(WinArgs A) {
  constexpr int LC = C + PAD;
  constexpr int PX = q_xform<PM>();
  __shared__ __attribute__((aligned(16))) TT sKT[DP * LC];
  __shared__ __attribute__((aligned(16))) TT sVT[DP * LC];
  using SB = StateBlocks<DP>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t u = blockIdx.x / A.nseg, seg = blockIdx.x % A.nseg;
  const int64_t sq = u / A.Hkv, g = u % A.Hkv;
  const SeqSpan sp = seq_span(A.S, sq, A.ctl, seg == 0 && tid == 0);
  const T* kb = reinterpret_cast<const T*>(A.k) + sq * A.S.kb + sp.start * A.S.kt + g * A.S.kh;
  const T* vb = reinterpret_cast<const T*>(A.v) + sq * A.S.kb + sp.start * A.S.kt + g * A.S.kh;
  const int64_t nch = (sp.len + C - 1) / C;
  const int64_t c0 = seg * A.G, c1 = (c0 + A.G < nch) ? c0 + A.G : nch;
  WinState<TT, DP, C> W;
  W.clear();
  // chunk c + 1's rows are requested before chunk c's state is added
  StageRegs<T, DP, C> rK, rV;
  if (c0 < c1) {
    stage_load<T, DP, C>(rK, kb, A.S.kt, c0 * C, chunk_rows(c0, C, sp.len), A.vec, tid);
    stage_load<T, DP, C>(rV, vb, A.S.kt, c0 * C, chunk_rows(c0, C, sp.len), A.vec, tid);
  }
  for (int64_t c = c0; c < c1; ++c) {
    const int nv = chunk_rows(c, C, sp.len);
    stage_put<T, TT, DP, C, XF_NONE, PX>(rK, kb, A.S.kt, c * C, nv, A.d, A.vec, nullptr, 0, sKT, LC, tid);
    stage_put<T, TT, DP, C, XF_NONE, XF_ID>(rV, vb, A.S.kt, c * C, nv, A.d, A.vec, nullptr, 0, sVT, LC, tid);
    if (c + 1 < c1) {
      const int nn = chunk_rows(c + 1, C, sp.len);
      stage_load<T, DP, C>(rK, kb, A.S.kt, (c + 1) * C, nn, A.vec, tid);
      stage_load<T, DP, C>(rV, vb, A.S.kt, (c + 1) * C, nn, A.vec, tid);
    }
    __syncthreads();
    W.add(sKT, LC, sVT, LC, false, w, lane, tid);
    __syncthreads();
  }
  float* dst = A.states + (u * (A.nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
  for (int s = 0; s < SB::PER_WAVE; ++s) {
    const int e = w + NW * s;
    if (e < SB::TOTAL) st_state_block<DP>(dst, W.acc[s], e / SB::NB, e % SB::NB, lane);
  }
  if (tid < DP) dst[DP * DP + tid] = W.z;
}

// ------------------------------------------------------------------ k_window
template <typename T, int DP, int C, int PM, bool WIN>
__global__ __launch_bounds__(NT) void k_window(WinArgs A) {
  constexpr int LQ = DP + PAD;      // token-major rows (Q, K, trailing K, W^T)
  constexpr int LC = C + PAD;       // feature-major rows of the leading chunk, scores
  constexpr int LC2 = 2 * C + PAD;  // feature-major rows of the trailing tile, its scores
  constexpr int NIB = C / 32;       // 32-row query / key blocks of a chunk
  constexpr int NTB = WIN ? 2 * NIB : 0;  // key blocks of the trailing tile
  constexpr int NBB = DP / 32;
  constexpr int PX = q_xform<PM>();  // phi on Q and on every K tile (no relu split here)
  static_assert(PM != PM_ID, "normalised form");
  // the trailing tile exists in the window form only
  constexpr int TR_K = WIN ? 2 * C * LQ : 8, TR_T = WIN ? DP * LC2 : 8, TR_P = WIN ? C * LC2 : 8;
  __shared__ __attribute__((aligned(16))) T sQ[C * LQ];
  __shared__ __attribute__((aligned(16))) T sK[C * LQ];
  __shared__ __attribute__((aligned(16))) T sKT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sVT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sKtr[TR_K];
  __shared__ __attribute__((aligned(16))) T sKTtr[TR_T];
  __shared__ __attribute__((aligned(16))) T sVTtr[TR_T];
  __shared__ __attribute__((aligned(16))) T sST[DP * LQ];
  __shared__ __attribute__((aligned(16))) T sP[C * LC];
  __shared__ __attribute__((aligned(16))) T sPtr[TR_P];
  // z of the window as a high part and the remainder in T, a zero row and a
  // ones row: the A operand rows of the denominator products
  __shared__ __attribute__((aligned(16))) T szh[DP + 16];
  __shared__ __attribute__((aligned(16))) T szl[DP + 16];
  __shared__ __attribute__((aligned(16))) T szero[DP + 16];
  __shared__ __attribute__((aligned(16))) T sones[16];
  using SB = StateBlocks<DP>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int64_t u = blockIdx.x / A.nseg, seg = blockIdx.x % A.nseg;
  const int64_t sq = u / A.Hkv, g = u % A.Hkv;
  const SeqSpan sp = seq_span(A.S, sq, A.ctl, seg == 0 && tid == 0);
  const int64_t n = sp.len, nchunks = (n + C - 1) / C;
  const int64_t c0 = seg * A.G, c1 = (c0 + A.G < nchunks) ? c0 + A.G : nchunks;
  if (c0 >= c1) return;  // past this sequence's end: nothing to do, and no barrier below is skipped by half the group
  const int d = A.d, R = A.R;
  const bool vec = A.vec;
  const int64_t kt = A.S.kt, qt = A.S.qt;
  const T* kb = reinterpret_cast<const T*>(A.k) + sq * A.S.kb + sp.start * kt + g * A.S.kh;
  const T* vb = reinterpret_cast<const T*>(A.v) + sq * A.S.kb + sp.start * kt + g * A.S.kh;
  const int64_t nfull = A.nfull;

  // Rows are requested one step ahead: while a step works from LDS, the
  // next step's leading chunk, trailing tile and first query head (or the
  // step's next query head) are in flight in registers.
  using RT = StageRegs<T, DP, C>;
  RT rK, rV, rKt[2], rVt[2], rQ;
  const T* qbase = reinterpret_cast<const T*>(A.q) + sq * A.S.qb + sp.start * qt;
  auto load_step = [&](int64_t c) {
    const int nvl = chunk_rows(c, C, n);
    stage_load<T, DP, C>(rK, kb, kt, c * C, nvl, vec, tid);
    stage_load<T, DP, C>(rV, vb, kt, c * C, nvl, vec, tid);
    if (WIN) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int64_t x = c - nfull - 2 + half;
        const int nvx = chunk_rows(x, C, n);
        const int64_t r0 = x < 0 ? 0 : x * C;
        stage_load<T, DP, C>(rKt[half], kb, kt, r0, nvx, vec, tid);
        stage_load<T, DP, C>(rVt[half], vb, kt, r0, nvx, vec, tid);
      }
    }
  };
  auto load_q = [&](int64_t c, int r) {
    stage_load<T, DP, C>(rQ, qbase + (g * R + r) * A.S.qh, qt, c * C, chunk_rows(c, C, n), vec, tid);
  };

  WinState<T, DP, C> W;
  if (WIN) {
    // warm-up: W = states of chunks c0 - nfull - 1 .. c0 - 1 (the first step
    // subtracts chunk c0 - nfull - 1 again); none while nfull = 0
    W.clear();
    const int64_t x0 = c0 - nfull - 1 > 0 ? c0 - nfull - 1 : 0;
    if (nfull > 0 && x0 < c0) {
      stage_load<T, DP, C>(rK, kb, kt, x0 * C, chunk_rows(x0, C, n), vec, tid);
      stage_load<T, DP, C>(rV, vb, kt, x0 * C, chunk_rows(x0, C, n), vec, tid);
    }
    for (int64_t x = x0; nfull > 0 && x < c0; ++x) {
      const int nvx = chunk_rows(x, C, n);
      stage_put<T, T, DP, C, XF_NONE, PX>(rK, kb, kt, x * C, nvx, d, vec, nullptr, 0, sKT, LC, tid);
      stage_put<T, T, DP, C, XF_NONE, XF_ID>(rV, vb, kt, x * C, nvx, d, vec, nullptr, 0, sVT, LC, tid);
      if (x + 1 < c0) {
        stage_load<T, DP, C>(rK, kb, kt, (x + 1) * C, chunk_rows(x + 1, C, n), vec, tid);
        stage_load<T, DP, C>(rV, vb, kt, (x + 1) * C, chunk_rows(x + 1, C, n), vec, tid);
      } else {
        load_step(c0);
        load_q(c0, 0);
      }
      __syncthreads();
      W.add(sKT, LC, sVT, LC, false, w, lane, tid);
      __syncthreads();
    }
    if (!(nfull > 0 && x0 < c0)) {
      load_step(c0);
      load_q(c0, 0);
    }
  } else {
    load_step(c0);
    load_q(c0, 0);
    // the exclusive prefix before chunk c0 (the scanned segment state)
    const float* src = A.states + (u * (A.nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) ld_state_block<DP>(W.acc[s], src, e / SB::NB, e % SB::NB, lane);
      else W.acc[s] = f32x16{};
    }
    W.z = tid < DP ? src[DP * DP + tid] : 0.0f;
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
    const int64_t t0 = c * C, ce = c - nfull;  // window form: the first chunk inside every window
    const int nv = chunk_rows(c, C, n);
    // leading chunk: phi(K) token- and feature-major, V feature-major;
    // trailing tile: chunks ce - 2 and ce - 1 (phi(K) both ways, V feature-major)
    stage_put<T, T, DP, C, PX, PX>(rK, kb, kt, t0, nv, d, vec, sK, LQ, sKT, LC, tid);
    stage_put<T, T, DP, C, XF_NONE, XF_ID>(rV, vb, kt, t0, nv, d, vec, nullptr, 0, sVT, LC, tid);
    if (WIN) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int64_t x = ce - 2 + half;
        const int nvx = chunk_rows(x, C, n);
        const int64_t r0 = x < 0 ? 0 : x * C;
        stage_put<T, T, DP, C, PX, PX>(rKt[half], kb, kt, r0, nvx, d, vec, sKtr + half * C * LQ, LQ,
                                       sKTtr + half * C, LC2, tid);
        stage_put<T, T, DP, C, XF_NONE, XF_ID>(rVt[half], vb, kt, r0, nvx, d, vec, nullptr, 0, sVTtr + half * C,
                                               LC2, tid);
      }
    }
    if (c + 1 < c1) load_step(c + 1);
    if (WIN) {
      if (nfull > 0) {  // W loses chunk ce - 1, which has left the chunks inside every window
        __syncthreads();
        W.add(sKTtr + C, LC2, sVTtr + C, LC2, true, w, lane, tid);
      }
    }
    // W^T (sST[b][a] = W[a][b]) and z of the window in T
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) st_accT(sST + (e % SB::NB) * 32 * LQ + (e / SB::NB) * 32, LQ, W.acc[s], lane);
    }
    if (tid < DP) {
      const T zh = cvt<T>(W.z);
      szh[tid] = zh;
      szl[tid] = cvt<T>(W.z - to_f(zh));
      szero[tid] = cvt<T>(0.0f);
    }

    for (int r = 0; r < R; ++r) {
      const int64_t hq = g * R + r;
      const T* qh = qbase + hq * A.S.qh;
      __syncthreads();  // the tiles above are written; the previous head is done with sQ, sP, sPtr
      stage_put<T, T, DP, C, PX, XF_NONE>(rQ, qh, qt, t0, nv, d, vec, sQ, LQ, nullptr, 0, tid);
      if (r + 1 < R)
        load_q(c, r + 1);
      else if (c + 1 < c1)
        load_q(c + 1, 0);
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
            const int lo = lead ? (WIN ? i - A.wlen + 1 : 0) : i + A.delta;  // kept key offsets: lo .. hi
            const int hi = lead ? i : 2 * C;
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
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = nb0 + uu * NB_STEP;
          accO[uu] = f32x16{};
          if (nb < NBB) {
            gemm_acc<T, DP / 16>(accO[uu], sST + nb * 32 * LQ, LQ, sQ + ib * 32 * LQ, LQ, lane);
#pragma unroll
            for (int jb = 0; jb <= ib; ++jb)
              gemm_acc<T, 2>(accO[uu], sVT + nb * 32 * LC + jb * 32, LC, sP + ib * 32 * LC + jb * 32, LC, lane);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
              gemm_acc<T, 2>(accO[uu], sVTtr + nb * 32 * LC2 + tb * 32, LC2, sPtr + ib * 32 * LC2 + tb * 32, LC2,
                             lane);
          }
        }
      }
      __syncthreads();  // every wave is past its reads of sQ: the rows go out through it
      if (has_out) {
#pragma unroll
        for (int uu = 0; uu < NPW; ++uu) {
          const int nb = nb0 + uu * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              sQ[i * LQ + nb * 32 + 8 * (e >> 2) + 4 * h + (e & 3)] = cvt<T>(accO[uu][e] * inv);
          }
        }
      }
      __syncthreads();
      T* ob = reinterpret_cast<T*>(A.out) + sq * A.S.qb + sp.start * qt + hq * A.S.qh;
      if (vec) {
        constexpr int EPP = 8 / (int)sizeof(T);  // 8-byte pieces (LDS rows are 8-byte aligned)
        constexpr int PPR = DP / EPP;
        typedef uint32_t U __attribute__((ext_vector_type(2)));
        for (int idx = tid; idx < nv * PPR; idx += NT) {
          const int rr = idx / PPR, col = EPP * (idx % PPR);
          __builtin_nontemporal_store(*reinterpret_cast<const U*>(sQ + rr * LQ + col),
                                      reinterpret_cast<U*>(ob + (t0 + rr) * qt + col));
        }
      } else {
        for (int idx = tid; idx < nv * d; idx += NT) {
          const int rr = idx / d, col = idx % d;
          ob[(t0 + rr) * qt + col] = sQ[rr * LQ + col];
        }
      }
    }

    // ---- W += dS(c) (the causal form always; the window form once chunks
    // lie inside every window)
    if (!WIN || nfull > 0) W.add(sKT, LC, sVT, LC, false, w, lane, tid);
    __syncthreads();
  }
}

// LDS bytes of k_window<T, DP, C, .., WIN>: must fit one CU's 160 KiB.
constexpr size_t window_lds(int eb, int DP, int C, bool win) {
  const size_t LQ = DP + PAD, LC = C + PAD, LC2 = 2 * C + PAD;
  const size_t tr = win ? 2 * C * LQ + 2 * DP * LC2 + C * LC2 : 24;
  return (size_t)eb * (2 * C * LQ + 2 * DP * LC + tr + DP * LQ + C * LC + 3 * (DP + 16) + 16);
}

template <typename T, int DP, int C, bool WIN>
int run_window(const la_internal::SeqCall& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const la_internal::Plan p = la_internal::seq_plan(a, C);
  WinArgs A{a.q, a.k, a.v, a.out, a.S, (int)a.d, (int)(a.Hq / a.Hkv), a.Hkv, p.G, p.nseg, 0, 0, 0,
            a.vec, reinterpret_cast<float*>(a.ws), a.ctl};
  if (WIN) {
    A.nfull = a.window / C > 1 ? a.window / C - 1 : 0;
    A.wlen = (int)a.window;
    A.delta = (int)((A.nfull + 2) * C - a.window + 1);
  }
  const dim3 grid((unsigned)(a.nseq * a.Hkv * p.nseg));
  if (!WIN) {  // the causal form: segment states, their exclusive prefix, then the walk
    if (a.phi == 1)
      k_wstate<T, DP, C, PM_ELU1><<<grid, NT, 0, st>>>(A);
    else if (a.phi == 2)
      k_wstate<T, DP, C, PM_FEAT><<<grid, NT, 0, st>>>(A);
    else
      k_wstate<T, DP, C, PM_RELU1><<<grid, NT, 0, st>>>(A);
    const int e = la_internal::launch_scan(A.states, a.nseq * a.Hkv, p.nseg, DP, (int)a.d, a.S_final, a.z_final,
                                           a.stream);
    if (e != 0) return e;
    if (!a.out) return (int)hipGetLastError();
  }
  if (a.phi == 1)
    k_window<T, DP, C, PM_ELU1, WIN><<<grid, NT, 0, st>>>(A);
  else if (a.phi == 2)
    k_window<T, DP, C, PM_FEAT, WIN><<<grid, NT, 0, st>>>(A);
  else
    k_window<T, DP, C, PM_RELU1, WIN><<<grid, NT, 0, st>>>(A);
  return (int)hipGetLastError();
}

}  // namespace

namespace la_internal {

int seq_chunk(int elem_bytes, int DP, bool window) {
  for (int c : {64, 32})
    if (window_lds(elem_bytes, DP, c, window) <= kLdsLimit) return c;
  return 0;
}

Plan seq_plan(const SeqCall& a, int C) {
  Plan p;
  p.DP = padded_dim(a.d);
  p.C = C;
  p.nchunks = (a.S.n + C - 1) / C;  // of the longest sequence
  const int64_t nfull = a.window > 0 && a.window / C > 1 ? a.window / C - 1 : 0;
  // about 512 workgroups; in the window form segments of at least nfull
  // chunks (the warm-up is then about as long as the walk)
  int64_t G = (a.nseq * a.Hkv * p.nchunks + 511) / 512;
  if (G < nfull) G = nfull;
  if (G < 1) G = 1;
  if (G > p.nchunks) G = p.nchunks;
  p.G = G;
  p.nseg = (p.nchunks + G - 1) / G;
  return p;
}

// The causal state pass and scan alone for chunk C (the backward's first
// pass, on fp32 tiles whatever the input type): a.ws receives the exclusive
// prefix slots of seq_plan(a, C).
template <typename T, int DP, int C>
int run_seq_prefix(const SeqCall& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const Plan p = seq_plan(a, C);
  WinArgs A{a.q, a.k, a.v, a.out, a.S, (int)a.d, (int)(a.Hq / a.Hkv), a.Hkv, p.G, p.nseg, 0, 0, 0,
            a.vec, reinterpret_cast<float*>(a.ws), a.ctl};
  const dim3 grid((unsigned)(a.nseq * a.Hkv * p.nseg));
  if (a.phi == 1)
    k_wstate<T, DP, C, PM_ELU1, float><<<grid, NT, 0, st>>>(A);
  else if (a.phi == 2)
    k_wstate<T, DP, C, PM_FEAT, float><<<grid, NT, 0, st>>>(A);
  else
    k_wstate<T, DP, C, PM_RELU1, float><<<grid, NT, 0, st>>>(A);
  return launch_scan(A.states, a.nseq * a.Hkv, p.nseg, DP, (int)a.d, nullptr, nullptr, a.stream);
}

int launch_seq_prefix(const SeqCall& a, int C) {
  const int DP = padded_dim(a.d);
#define LA_PFX(TT, DD, CC) \
  if (DP == DD && C == CC) return run_seq_prefix<TT, DD, CC>(a);
  if (a.dtype == 0) {
    LA_PFX(float, 32, 64)
    LA_PFX(float, 64, 32)
  } else {
    LA_PFX(bf16, 32, 64)
    LA_PFX(bf16, 64, 32)
  }
#undef LA_PFX
  return (int)hipErrorInvalidValue;
}

int launch_seq(const SeqCall& a) {
  const int DP = padded_dim(a.d);
  const bool win = a.window > 0;
  const int C = seq_chunk(a.dtype == 0 ? 4 : 2, DP, win);
#define LA_SEQ(TT, DD, CC, WW)                                                                     \
  if (DP == DD && C == CC && win == WW) {                                                         \
    if constexpr (window_lds((int)sizeof(TT), DD, CC, WW) <= kLdsLimit) return run_window<TT, DD, CC, WW>(a); \
  }
  if (a.dtype == 0) {
    LA_SEQ(float, 32, 64, true)
    LA_SEQ(float, 64, 32, true)
    LA_SEQ(float, 32, 64, false)
    LA_SEQ(float, 64, 64, false)
    LA_SEQ(float, 64, 32, false)
    LA_SEQ(float, 128, 32, false)
  } else {
    LA_SEQ(bf16, 32, 64, true)
    LA_SEQ(bf16, 64, 64, true)
    LA_SEQ(bf16, 128, 32, true)
    LA_SEQ(bf16, 32, 64, false)
    LA_SEQ(bf16, 64, 64, false)
    LA_SEQ(bf16, 128, 64, false)
    LA_SEQ(bf16, 128, 32, false)
  }
#undef LA_SEQ
  return (int)hipErrorInvalidValue;
}

}  // namespace la_internal
