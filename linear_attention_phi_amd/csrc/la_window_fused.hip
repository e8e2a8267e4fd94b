// la_window_fused.hip -- single-launch sliding-window kernel for bf16 inputs,
// d = 64, chunk 64, up to eight query heads per key/value head, windows
// w < 576 (gfx950).
//
// LinearTile 1.0.1, "Features" (sliding-window attention, local context),
// with the normalised read of nx_f32_linear_attention.nx: query i sees the
// keys i - w < j <= i.  The decomposition is that of la_window.hip: for query
// chunk c, nfull = max(floor(w / 64) - 1, 0), e = c - nfull,
//     num_i = phi(Q_i) W(c) + [keys of chunk c with i - w < j <= i]
//                           + [keys of chunks e - 2, e - 1 with t >= u + delta]
// where W(c) is the sum of the chunk states (S and z) of chunks e .. c - 1,
// t the key offset from (e - 2) 64, u the query offset from c 64 and delta =
// (nfull + 2) 64 - w + 1 (den likewise, with V replaced by 1).
//
// Work decomposition, no workspace and no waits between workgroups: a
// workgroup of eight waves owns a segment of eight query chunks (wave l:
// chunk c = 8 s + l).  W(c) is split at the segment's start:
//  - the segment's own chunks e .. c - 1 (clamped at the segment start):
//    from the eight own chunk states (fp32 tiles in LDS), as a difference of
//    the segment's exclusive prefixes, in fp32;
//  - the halo, chunks e .. 8 s - 1 before the segment (when nfull > l): wave
//    m = 1 .. nfull loads chunk 8 s + m - nfull - 1 -- which is also its own
//    query chunk's trailing chunk e - 1 -- and forms its state; the halo part
//    of W(8 s + l) is the suffix sum of those states from m = l + 1 on.
// Each part goes to the output separately (rounded to bf16 operands once,
// its products accumulated in fp32), as the causal kernel does with the
// segment and look-back parts of its prefix state.  Every term is a sum of
// chunk states inside one segment or its halo, so nothing long cancels.
//
// Phases (barriers between them): own chunk (its state, the leading tile's
// scores and numerator in registers), the own part's scan and products, the
// trailing chunks (e - 2 when w is not a multiple of 64 minus one, then e - 1
// with the halo state), the halo part's scan and products, output rows
// through LDS.  MFMA operand conventions are those of la_fused.hip.
//
// Rows come through a sequence table when SEQ (strides and cu_seqlens, as in
// la_fused.hip); a sequence whose cu entries are inconsistent is left empty
// and reported through the control block when one is given.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_bf16.h"
#include "la_ctl.h"
#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;
using namespace la_bf16;

constexpr int FD = 64;                    // head dim
constexpr int FC = 64;                    // chunk
constexpr int SEGC = 8;                   // chunks per segment = waves per workgroup
constexpr int FNT = 64 * SEGC;            // threads per workgroup
constexpr int RS = FD + 8;                // row stride (bf16) of the token-major tiles
constexpr int RSF = FD + 4;               // row stride (fp32) of the state tiles
constexpr int TILE_B = FC * RS * 2;       // bytes of one token-major bf16 tile
constexpr int REGION_B = 2 * TILE_B;      // one wave's LDS region
constexpr int kMaxNfull = SEGC - 1;       // halo chunks a segment can hold

// Heads: as in la_fused.hip, query head u = s H + h (H query heads per
// sequence) reads key/value head h / R; with R > 1 each query head
// recomputes its group's chunk states, and the group's heads are dispatched
// eight apart (xcd) so that they share K and V through one XCD's L2.
struct WfArgs {
  const bf16* q; const bf16* k; const bf16* v; bf16* out;
  int64_t n, nseg, NH;  // n, nseg: of the longest sequence; NH = sequences x query heads
  int64_t H, qb, qh, qt, kb, kh, kt;
  int R, xcd;
  const int64_t* cu; int64_t total;  // cu NULL: every sequence holds n tokens
  int nfull, delta, wlen;            // the window's decomposition (header)
  la_internal::Ctl* ctl;             // NULL: nothing to report
};

// LDS: one region per wave, reused phase by phase (K and V tiles, then a
// fp32 chunk state over them, then a window-part tile in bf16 in its first
// half and the output rows in its second).
struct WfLds {
  uint8_t reg[SEGC][REGION_B];
  float zloc[SEGC][FD];        // z of each wave's chunk (own, then halo)
  uint32_t zh[SEGC][FD / 2];   // a window part's z for each query chunk: bf16 (high, low) pairs
  uint32_t zl[SEGC][FD / 2];
  bf16 zero[FD];               // zeros: the rows of the z operand other than 0 and 16
};
static_assert(32 * RSF * 4 <= TILE_B, "state half-tile must fit a token-major tile");

__device__ __forceinline__ float* state_row(WfLds& L, int c, int b) {
  return reinterpret_cast<float*>(L.reg[c] + (b < 32 ? TILE_B : 0)) + (b & 31) * RSF;
}

template <int PM, bool SEQ, bool GQA>
__global__ __launch_bounds__(FNT, 1) void k_window_fused(WfArgs A) {
  constexpr bool SPLIT = PM == PM_RELU1;
  __shared__ __attribute__((aligned(16))) WfLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  const int64_t seg = blockIdx.y;
  uint32_t head32 = blockIdx.x;
  if (GQA && A.xcd) {  // dispatch index -> (group, member): groups of eight take 8 R consecutive indices
    const uint32_t blk = blockIdx.x / (8u * A.R), rem = blockIdx.x - blk * 8u * A.R;
    head32 = (blk * 8u + (rem & 7u)) * A.R + (rem >> 3);
  }
  const int64_t head = head32;
  const int64_t kvhead = GQA ? head32 / (uint32_t)A.R : head32;
  int64_t start = 0, len = A.n;
  if (SEQ && A.cu) {
    const int64_t sq = head32 / (uint32_t)A.H;
    const int64_t a = A.cu[sq], b = A.cu[sq + 1], prev = sq > 0 ? A.cu[sq - 1] : 0;
    if (a < prev || b < a || b > A.total || b - a > A.n) {
      if (seg == 0 && tid == 0 && A.ctl) la_ctl::ctl_fail(A.ctl, la_internal::kErrRange);
      len = 0;
    } else {
      start = a;
      len = b - a;
    }
  }
  const int64_t nch = (len + FC - 1) / FC;
  if (SEQ && seg * SEGC >= nch) return;  // past this sequence's end (the grid covers the longest)
  int qbytes = (int)(A.n * FD * 2), kbytes = qbytes;
  int64_t qoff = head * A.n * FD, koff = kvhead * A.n * FD;
  int qs = FD * 2, ks = FD * 2;  // row strides in bytes
  if (SEQ) {
    const uint32_t sq32 = head32 / (uint32_t)A.H;
    const int64_t sq = sq32, hh = head32 - sq32 * (uint32_t)A.H;
    qbytes = (int)(((len - 1) * A.qt + FD) * 2);
    kbytes = (int)(((len - 1) * A.kt + FD) * 2);
    qoff = sq * A.qb + start * A.qt + hh * A.qh;
    koff = sq * A.kb + start * A.kt + (GQA ? hh / A.R : hh) * A.kh;
    qs = (int)A.qt * 2;
    ks = (int)A.kt * 2;
  }
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.q + qoff), 0, qbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.k + koff), 0, kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.v + koff), 0, kbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(A.out + qoff, 0, qbytes, 0x00020000);

  const int64_t c_begin = seg * SEGC;
  const int ncl = (int)((nch - c_begin) < SEGC ? (nch - c_begin) : SEGC);  // query chunks of the segment
  const bool mine = w < ncl;
  const int64_t c = c_begin + w;
  const int t0 = (int)(c * FC);
  const int nv = mine ? (int)((len - t0) < FC ? (len - t0) : FC) : 0;
  const int nfull = A.nfull, delta = A.delta, wlen = A.wlen;
  // the trailing tile: x1 = e - 1 (the only trailing chunk with keys when
  // delta > 63), x2 = e - 2; both lie before c, so they are whole chunks
  const int64_t x1 = c - nfull - 1, x2 = x1 - 1;
  const bool use_x1 = mine && x1 >= 0 && 32 + 31 >= delta - FC;       // some key of x1 is kept
  const bool use_x2 = mine && x2 >= 0 && 32 + 31 >= delta;            // some key of x2 is kept
  const bool halo = w >= 1 && w <= nfull && x1 >= 0;                  // x1 is halo chunk m = w
  bf16* tK = reinterpret_cast<bf16*>(L.reg[w]);
  bf16* tV = reinterpret_cast<bf16*>(L.reg[w] + TILE_B);
  if (tid < FD) L.zero[tid] = (bf16)0.0f;

  const int prow = lane >> 3, pcol = 8 * (lane & 7);
  auto load_kv = [&](int64_t x, u32x4 (&kr)[8], u32x4 (&vr)[8]) {
    const int r0 = (int)(x * FC);
#pragma unroll
    for (int u = 0; u < 8; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (r0 + prow + 8 * u) * ks + pcol * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (r0 + prow + 8 * u) * ks + pcol * 2, 0, 0);
  };
  // relu(K) (the split map) or phi(K) with rows past nvalid as 0, and V, into
  // this wave's token-major tiles
  auto put_kv = [&](const u32x4 (&kr)[8], const u32x4 (&vr)[8], int nvalid) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      u32x4 x = kr[u];
      const bool real = prow + 8 * u < nvalid;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = SPLIT ? relu2(x[j]) : (real ? map2<PM>(x[j]) : 0u);
      *reinterpret_cast<u32x4*>(tK + (prow + 8 * u) * RS + pcol) = x;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<u32x4*>(tV + (prow + 8 * u) * RS + pcol) = vr[u];
    wave_lds_sync();
  };
  // V^T (feature block nb, token block kt) and relu(K)^T fragments, transposed reads
  auto frags_vt = [&](Frag<bf16> (&vt)[2][4]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) vt[nb][kt] = ld_tr<RS>(tV, 16 * kt, 32 * nb, lane);
  };
  auto frags_kt = [&](Frag<bf16> (&ktt)[2][4]) {
#pragma unroll
    for (int ab = 0; ab < 2; ++ab)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ktt[ab][kt] = ld_tr<RS>(tK, 16 * kt, 32 * ab, lane);
  };
  auto frags_k = [&](Frag<bf16> (&kf)[2][4]) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[jb][kb] = ld16(tK + (32 * jb + r) * RS + 16 * kb + 8 * h);
  };
  // the staged chunk's state dS = relu(K)^T V + ones^T V (fp32) into this
  // wave's state tile (transposed, rows b), and its z into zloc[w]; the
  // fragments have been read, so the tile may overwrite the K and V tiles
  auto chunk_state = [&](const Frag<bf16> (&ktt)[2][4], const Frag<bf16> (&vt)[2][4], int nvalid) {
    float cs[2] = {0.0f, 0.0f};
    if (SPLIT) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int p = 0; p < 4; ++p) cs[nb] = dot2(pair(vt[nb][kt], p), ONE2, cs[nb]);
        cs[nb] += __shfl_xor(cs[nb], 32);
      }
    }
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) {
      float zp = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int p = 0; p < 4; ++p) zp = dot2(pair(ktt[ab][kt], p), ONE2, zp);
      zp += __shfl_xor(zp, 32);
      if (h == 0) L.zloc[w][32 * ab + r] = zp + (SPLIT ? (float)nvalid : 0.0f);
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mma(acc, ktt[ab][kt], vt[bb][kt]);
        float* row = state_row(L, w, 32 * bb + r) + 32 * ab + 4 * h;
        const float cv = cs[bb];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4v*>(row + 8 * q) =
              f32x4v{acc[4 * q] + cv, acc[4 * q + 1] + cv, acc[4 * q + 2] + cv, acc[4 * q + 3] + cv};
      }
    }
  };

  f32x16 O[2][2];       // numerator blocks (feature block nb, query block ib)
  Frag<bf16> qf[2][4];  // phi(Q) fragments (query block ib, feature block kb)
  float qsum[2] = {0.0f, 0.0f};  // sum_a phi(Q_i)[a] (the split map's ones part of each score)
  float den[2] = {0.0f, 0.0f}, dz[2] = {0.0f, 0.0f};
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) O[nb][ib] = f32x16{};
  // P^T blocks of the staged keys (key block jb) against this wave's queries
  // (block ib), keeping the pairs whose offset j - i (local key and query
  // indices) lies in [lo, hi]; then V^T P^T into O and the rounded weights'
  // row sums into den.  A block with no such pair (the same for every lane)
  // is skipped.  Element e of a lane holds key 32 jb + 8 (e >> 2) + 4 h +
  // (e & 3) and query 32 ib + r: the offset is a compile-time constant plus
  // 4 h - r, so each test compares an immediate with one of two registers.
  auto scores_pv = [&](const Frag<bf16> (&kf)[2][4], const Frag<bf16> (&vt)[2][4], int lo, int hi) {
    const int dl = 4 * h - r, tlo = lo - dl, thi = hi - dl;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      float ds = 0.0f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int base = 32 * (jb - ib);
        if (base - 31 > hi || base + 31 < lo) continue;
        f32x16 pacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) pacc[e] = qsum[ib];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(pacc, kf[jb][kb], qf[ib][kb]);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int ce = base + 8 * (e >> 2) + (e & 3);
          pacc[e] = (ce >= tlo && ce <= thi) ? pacc[e] : 0.0f;
        }
        const Frag<bf16> p0 = acc_frag(pacc, 0), p1 = acc_frag(pacc, 1);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          mma(O[nb][ib], vt[nb][2 * jb], p0);
          mma(O[nb][ib], vt[nb][2 * jb + 1], p1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) ds = dot2(pair(p1, j), ONE2, dot2(pair(p0, j), ONE2, ds));
      }
      den[ib] += ds + __shfl_xor(ds, 32);
    }
  };
  // num += phi(Q) S (S^T [b][a] bf16 rows of RS), den_i += phi(Q_i) . z via
  // rows 0 and 16 of the z operand (high and low parts)
  auto state_products = [&](const bf16* tS, const uint32_t* zh, const uint32_t* zl) {
    const bf16* zbase = (r == 0) ? reinterpret_cast<const bf16*>(zh)
                                 : (r == 16) ? reinterpret_cast<const bf16*>(zl) : L.zero;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(O[nb][ib], ld16(tS + (32 * nb + r) * RS + 16 * kb + 8 * h), qf[ib][kb]);
      f32x16 zacc = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(zacc, ld16(zbase + 16 * kb + 8 * h), qf[ib][kb]);
      dz[ib] += zacc[0] + zacc[8];
    }
  };
  // scan slice of this thread: state rows b = sb, features sa .. sa + 7
  const int sb = 8 * w + (lane >> 3), sa = 8 * (lane & 7);
  auto read_slice = [&](int m, float (&x)[8]) {
    const float* src = state_row(L, m, sb) + sa;
    const f32x4v x0 = *reinterpret_cast<const f32x4v*>(src);
    const f32x4v x1v = *reinterpret_cast<const f32x4v*>(src + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = e < 4 ? x0[e] : x1v[e - 4];
  };
  auto write_part = [&](int m, const float (&x)[8]) {
    uint32_t y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = pack2(x[2 * j], x[2 * j + 1]);
    *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(L.reg[m]) + sb * RS + sa) = u32x4{y[0], y[1], y[2], y[3]};
  };

  // ------------------------------------------------------------------ own chunk
  if (mine) {
    u32x4 kr[8], vr[8], qr[2][4];
    load_kv(c, kr, vr);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        qr[ib][kb] = __builtin_amdgcn_raw_buffer_load_b128(rq, (t0 + 32 * ib + r) * qs + (16 * kb + 8 * h) * 2, 0, 0);
    put_kv(kr, vr, nv);
    Frag<bf16> vt[2][4], kf[2][4];
    {
      Frag<bf16> ktt[2][4];
      frags_vt(vt);
      frags_kt(ktt);
      frags_k(kf);
      wave_lds_sync();
      chunk_state(ktt, vt, nv);
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 x = qr[ib][kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = SPLIT ? phi2(x[j]) : map2<PM>(x[j]);
        qf[ib][kb].v = __builtin_bit_cast(bf16x8, x);
      }
      if (SPLIT) {
        float s = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int p = 0; p < 4; ++p) s = dot2(pair(qf[ib][kb], p), ONE2, s);
        qsum[ib] = s + __shfl_xor(s, 32);
      }
    }
    // the leading tile: keys of chunk c with i - w < j <= i
    scores_pv(kf, vt, 1 - wlen, 0);
  }
  __syncthreads();
  // The first trailing chunk's rows (e - 2 when some key of it can be kept,
  // else e - 1, which is also the halo chunk) are requested once the own
  // part's scan no longer needs the registers, to arrive during its products.
  const bool x2_pass = delta <= FC - 1;
  u32x4 kr[8], vr[8];  // a trailing chunk's rows in flight
  auto issue_trailing = [&]() {
    if (x2_pass) {
      if (use_x2) load_kv(x2, kr, vr);
    } else if (use_x1 || halo) {
      load_kv(x1, kr, vr);
    }
  };

  // ------------------------------------------------------------------ own part
  // W_own(l) = sum of this segment's chunk states max(0, l - nfull) .. l - 1,
  // the difference of two exclusive prefixes of the segment (fp32)
  if (nfull > 0) {
    float pre[SEGC][8];
    float zpre[SEGC];
    float run[8], zrun = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) run[e] = 0.0f;
#pragma unroll
    for (int m = 0; m < SEGC; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pre[m][e] = run[e];
      zpre[m] = zrun;
      if (m < ncl) {
        float x[8];
        read_slice(m, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] += x[e];
        if (w == 0) zrun += L.zloc[m][lane];
      }
    }
    __syncthreads();  // every state tile has been read
#pragma unroll
    for (int m = 1; m < SEGC; ++m) {
      if (m < ncl) {
        const int lo = m - nfull > 0 ? m - nfull : 0;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // the compile-time index keeps pre in registers
          float base = 0.0f;
#pragma unroll
          for (int mm = 0; mm < SEGC; ++mm) base = mm == lo ? pre[mm][e] : base;
          x[e] = pre[m][e] - base;
        }
        write_part(m, x);
        if (w == 0) {
          float zb = 0.0f;
#pragma unroll
          for (int mm = 0; mm < SEGC; ++mm) zb = mm == lo ? zpre[mm] : zb;
          store_z_pairs(L.zh[m], L.zl[m], zpre[m] - zb, lane);
        }
      }
    }
    issue_trailing();
    __syncthreads();
    if (mine && w > 0) state_products(reinterpret_cast<const bf16*>(L.reg[w]), L.zh[w], L.zl[w]);
  } else {
    issue_trailing();
  }
  __syncthreads();  // every wave is done with its region's window-part tile

  // ------------------------------------------------------------------ trailing and halo
  if (x2_pass) {
    if (use_x2) {  // keys of chunk e - 2 with t >= u + delta (t = j)
      put_kv(kr, vr, FC);
      Frag<bf16> vt[2][4], kf[2][4];
      frags_vt(vt);
      frags_k(kf);
      wave_lds_sync();  // read before the tiles are written again below
      scores_pv(kf, vt, delta, FC);
    }
    __builtin_amdgcn_sched_barrier(0);  // x1's requests after x2's products (registers)
    if (use_x1 || halo) load_kv(x1, kr, vr);
  }
  if (use_x1 || halo) {
    put_kv(kr, vr, FC);
    Frag<bf16> vt[2][4];
    frags_vt(vt);
    if (use_x1) {  // keys of chunk e - 1 with t >= u + delta (t = j + 64)
      Frag<bf16> kf[2][4];
      frags_k(kf);
      scores_pv(kf, vt, delta - FC, FC);
    }
    if (halo) {  // halo chunk m = w: its state (over this wave's tiles)
      Frag<bf16> ktt[2][4];
      frags_kt(ktt);
      wave_lds_sync();
      chunk_state(ktt, vt, FC);
    }
  }
  __syncthreads();

  // ------------------------------------------------------------------ halo part
  // H(l) = sum of the halo states m = l + 1 .. nfull (chunk 8 s + m - nfull - 1),
  // for the query chunks l < nfull
  if (nfull > 0 && seg > 0) {
    float hs[SEGC][8];
    float zh_[SEGC];
    float acc[8], zacc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int m = kMaxNfull; m >= 1; --m) {
      if (m <= nfull && c_begin + m - nfull - 1 >= 0) {
        float x[8];
        read_slice(m, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += x[e];
        if (w == 0) zacc += L.zloc[m][lane];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) hs[m - 1][e] = acc[e];
      zh_[m - 1] = zacc;
    }
    __syncthreads();  // every halo state tile has been read
#pragma unroll
    for (int l = 0; l < kMaxNfull; ++l) {
      if (l < nfull && l < ncl) {
        write_part(l, hs[l]);
        if (w == 0) store_z_pairs(L.zh[l], L.zl[l], zh_[l], lane);
      }
    }
    __syncthreads();
    if (mine && w < nfull) state_products(reinterpret_cast<const bf16*>(L.reg[w]), L.zh[w], L.zl[w]);
  }

  // ------------------------------------------------------------------ output
  if (mine) {
    float inv[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) inv[ib] = __builtin_amdgcn_rcpf(__shfl(den[ib] + dz[ib], r));  // from the lane with h == 0
    bf16* tO = reinterpret_cast<bf16*>(L.reg[w] + TILE_B);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const f32x16& o = O[nb][ib];
        uint2* dst = reinterpret_cast<uint2*>(tO + (32 * ib + r) * RS + 32 * nb + 4 * h);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[2 * q] = make_uint2(pack2(o[4 * q] * inv[ib], o[4 * q + 1] * inv[ib]),
                                  pack2(o[4 * q + 2] * inv[ib], o[4 * q + 3] * inv[ib]));
      }
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(tO + (prow + 8 * u) * RS + pcol), ro,
                                             (t0 + prow + 8 * u) * qs + pcol * 2, 0, CPOL_NT);
  }
}

template <bool SEQ, bool GQA>
void launch_pm(const WfArgs& A, int phi, hipStream_t st) {
  const dim3 grid((unsigned)A.NH, (unsigned)A.nseg);
  if (phi == 2)
    k_window_fused<PM_FEAT, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
  else if (phi == 1)
    k_window_fused<PM_ELU1, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
  else
    k_window_fused<PM_RELU1, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
}

template <bool SEQ>
int launch(WfArgs& A, int phi, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (A.R > 1)
    launch_pm<SEQ, true>(A, phi, st);
  else
    launch_pm<SEQ, false>(A, phi, st);
  return (int)hipGetLastError();
}

void decompose(WfArgs& A, int64_t window) {
  A.nfull = (int)(window / FC > 1 ? window / FC - 1 : 0);
  A.delta = (int)((A.nfull + 2) * FC - window + 1);
  A.wlen = (int)window;
}

}  // namespace

namespace la_internal {

bool window_fused_applies(const SeqCall& a) {
  const int64_t rs = a.S.qt > a.S.kt ? a.S.qt : a.S.kt;
  const int64_t nfull = a.window / FC > 1 ? a.window / FC - 1 : 0;
  return a.q && a.window >= 1 && nfull <= kMaxNfull && a.dtype == 1 && a.d == FD && a.Hq % a.Hkv == 0 &&
         a.Hq / a.Hkv <= kFusedMaxR && a.vec &&
         a.S.qt >= FD && a.S.kt >= FD && (a.S.n + FC) * rs * 2 < ((int64_t)1 << 31);
}

int launch_window_fused(const SeqCall& a, bool table) {
  const int64_t nchunks = (a.S.n + FC - 1) / FC;
  const int R = (int)(a.Hq / a.Hkv);
  WfArgs A{reinterpret_cast<const bf16*>(a.q), reinterpret_cast<const bf16*>(a.k),
           reinterpret_cast<const bf16*>(a.v), reinterpret_cast<bf16*>(a.out), a.S.n, (nchunks + SEGC - 1) / SEGC,
           a.nseq * a.Hq, a.Hq, a.S.qb, a.S.qh, a.S.qt, a.S.kb, a.S.kh, a.S.kt, R,
           R > 1 && (a.nseq * a.Hkv) % 8 == 0, a.S.cu, a.S.total, 0, 0, 0, a.ctl};
  decompose(A, a.window);
  return table ? launch<true>(A, a.phi, a.stream) : launch<false>(A, a.phi, a.stream);
}

}  // namespace la_internal
