// la_fused.hip -- single-launch causal kernel for bf16 inputs, d = 64,
// chunk 64, up to kFusedMaxR query heads per key/value head (gfx950).
//
// Same mathematics as the three-launch path in la_kernels.hip (causal form:
// out_i = phi(Q_i) S_i / (phi(Q_i) . z_i) with S_i, z_i over keys 0..i;
// nx_f32_linear_attention.nx for phi, S, z and the read; trim-transformer
// 0.1.0 "Masking" for the causal prefix), organised so that every input
// byte is read from HBM once and every output byte written once, with all
// of a workgroup's loads in flight from its start:
//
//  A  a workgroup owns a segment of eight chunks; wave w owns chunk w.  It
//     loads the chunk's Q, K and V at once and forms the chunk's state
//     dS = relu(K)^T V + ones^T V (fp32, written to LDS) and z (these need K
//     and V only), then, in registers, the chunk-local numerator
//     tril(phi(Q) phi(K)^T) V and denominator;
//  B  the eight waves scan the states of the segment (each wave a slice of
//     rows, over the eight chunks): exclusive prefixes S_loc(c), z_loc(c) and
//     the segment aggregate, which is published; the aggregates of all
//     earlier segments of the head are summed (waiting on their flags):
//     S_prev, z_prev; S_pre(c) = S_prev + S_loc(c) goes to LDS as bf16;
//  C  every wave adds phi(Q) S_pre(c) and phi(Q) . z_pre(c), normalises and
//     writes its chunk's rows.
//
// MFMA operands (v_mfma_f32_32x32x16_bf16): products over the feature index
// read 16 contiguous bytes per lane (k = 16 kb + 8 h + {0..7}); products
// over the token index take the accumulator-derived order of la_device.h
// (k = 16 kt + 4 h + {0..3}, 16 kt + 8 + 4 h + {0..3}), so P^T's accumulator
// feeds the V^T P^T product directly, and the transposed V and relu(K)
// operands are read from the token-major LDS tiles with ds_read_b64_tr_b16
// (la_bf16.h).  phi(K)^T V is formed as
// relu(K)^T V + 1 (x) sum_t V_t (exact products; see la_kernels.hip).
//
// Segments are numbered segment-major (grid x = head, y = segment; x varies
// fastest in dispatch order), so a workgroup only ever waits for workgroups
// dispatched before it.  Aggregates
// go through memory with device-scope stores and loads (the XCDs' L2 caches
// are not coherent with each other).  Flags are 64-bit words holding the
// call's epoch, taken from the workspace's control block (la_ctl.h), so that
// replays of a captured launch are ordered as well.  Spins are bounded;
// exhausting the bound records an error bit in the control block (read by
// la_workspace_status) instead of hanging.
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
constexpr int RS = FD + 8;                // row stride (bf16) of the token-major tiles: 144 bytes
constexpr int RSF = FD + 4;               // row stride (fp32) of the state tiles: 272 bytes
constexpr int AGG_FLOATS = FD * FD + FD;  // published segment aggregate: S^T [b][a], then z
constexpr int TILE_B = FC * RS * 2;       // bytes of one token-major bf16 tile
constexpr int REGION_B = 2 * TILE_B;      // one wave's LDS region

// Rows come through a sequence table: row t of query head h of sequence s at
// q + s qb + start(s) qt + h qh + t qt, of its key/value head h / R at
// k + s kb + start(s) kt + (h / R) kh + t kt (out with the q strides),
// start(s) = cu[s] for packed sequences of different lengths and 0 for one
// length n.  "head" below is the query head u = s H + h.  With R > 1 query
// heads per key/value head every query head runs as a head of its own (its
// own segment states, aggregates and flags, the key/value head's rows read
// by each); xcd: the R heads of a group are dispatched eight apart, so that
// they run on one XCD (workgroups go to the eight XCDs in turn) and read
// their K and V rows through its L2.
struct FusedArgs {
  const bf16* q; const bf16* k; const bf16* v; bf16* out;
  int64_t n, nchunks, nseg, NH;  // n, nchunks, nseg: of the longest sequence; NH = sequences x query heads
  int64_t H, qb, qh, qt, kb, kh, kt;  // H: query heads per sequence
  int R, xcd;                          // query heads per key/value head; dispatch order (above)
  const int64_t* cu; int64_t total;  // cu NULL: every sequence holds n tokens
  float* agg; uint64_t* flags;
  float* S_final; float* z_final; la_internal::Ctl* ctl;
  uint64_t host_epoch;  // the call's epoch, or 0: take it from the control block
};

// LDS: one region per wave, reused phase by phase:
//   A: relu(K) at [0, TILE_B), V at [TILE_B, 2 TILE_B), token-major rows of
//      RS; then the chunk's state dS^T [b][a] in fp32 rows of RSF, rows
//      b < 32 over the V tile and b >= 32 over the K tile;
//   C: S_pre^T [b][a] in bf16 at [0, TILE_B), the output rows at
//      [TILE_B, 2 TILE_B).
struct CpLds {
  uint8_t reg[SEGC][REGION_B];
  float zloc[SEGC][FD];        // z of each chunk
  uint32_t zh[SEGC][FD / 2];   // z_pre of each chunk as bf16 (high, low) pairs
  uint32_t zl[SEGC][FD / 2];
  bf16 zero[FD];               // zeros: the rows of the z operand other than 0 and 16
  bf16 sprev[FC * RS];         // S_prev^T [b][a] in bf16: the earlier segments' total
  uint32_t zhp[FD / 2];        // z_prev as bf16 (high, low) pairs
  uint32_t zlp[FD / 2];
  uint64_t epoch, expect;      // the call's epoch; what the waits compare flags with
  uint32_t limit;              // polls before a wait gives up
};
static_assert(32 * RSF * 4 <= TILE_B, "state half-tile must fit a token-major tile");

__device__ __forceinline__ float* state_row(CpLds& L, int c, int b) {
  return reinterpret_cast<float*>(L.reg[c] + (b < 32 ? TILE_B : 0)) + (b & 31) * RSF;
}

// PM: the feature map.  relu + 1 is split as relu(K) (exact in bf16) and the
// ones part (column sums of V, the key count in z, sum_a phi(Q_i)[a] at the
// start of each score); ELU + 1 has no such split: phi(K) and phi(Q) are
// rounded to bf16 in the tiles and fragments, and rows past the sequence end
// are stored as 0, not phi(0) = 1.  Caller-applied features (PM_FEAT) go
// through the same path with the identity.
//
// SEQ: rows through the sequence table (runtime strides, cu); without it the
// rows are contiguous [B, H, n, d] (compile-time strides: the address
// arithmetic of the loads and stores folds into immediate offsets).
// GQA: several query heads per key/value head (R > 1, the dispatch order
// above); without it every head is its own key/value head.
template <int PM, bool SEQ, bool GQA>
__global__ __launch_bounds__(FNT, 1) void k_causal_fused(FusedArgs A) {
  constexpr bool SPLIT = PM == PM_RELU1;
  __shared__ __attribute__((aligned(16))) CpLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  // grid (heads of every sequence, segments): x varies fastest, so the
  // dispatch order is segment-major
  const int64_t seg = blockIdx.y;
  uint32_t head32 = blockIdx.x;
  if (GQA && A.xcd) {  // dispatch index -> (group, member): groups of eight take 8 R consecutive indices
    const uint32_t blk = blockIdx.x / (8u * A.R), rem = blockIdx.x - blk * 8u * A.R;
    head32 = (blk * 8u + (rem & 7u)) * A.R + (rem >> 3);
  }
  const int64_t head = head32;                        // the query head
  const uint32_t member = GQA ? head32 % (uint32_t)A.R : 0u;
  const int64_t kvhead = GQA ? head32 / (uint32_t)A.R : head32;
  // the control words are requested first; wave 0 uses them after its loads
  la_ctl::CtlView cv{};
  if (w == 0) cv = la_ctl::ctl_load(A.ctl);
  // this sequence's rows: start and length (an inconsistent table entry
  // leaves the sequence empty and is recorded once, by its first segment)
  int64_t start = 0, len = A.n;
  if (SEQ && A.cu) {
    const int64_t sq = head32 / (uint32_t)A.H;
    const int64_t a = A.cu[sq], b = A.cu[sq + 1], prev = sq > 0 ? A.cu[sq - 1] : 0;
    if (a < prev || b < a || b > A.total || b - a > A.n) {
      if (seg == 0 && tid == 0) la_ctl::ctl_fail(A.ctl, la_internal::kErrRange);
      start = 0;
      len = 0;
    } else {
      start = a;
      len = b - a;
    }
  }
  const int64_t nch = (len + FC - 1) / FC, nseg_s = (nch + SEGC - 1) / SEGC;
  if (SEQ && seg >= nseg_s) {  // past this sequence's end (the grid covers the longest)
    if (seg == 0 && len == 0 && member == 0) {  // an empty sequence's final state is zero
      if (A.S_final)
        for (int e = tid; e < FD * FD; e += FNT) A.S_final[kvhead * FD * FD + e] = 0.0f;
      if (A.z_final && tid < FD) A.z_final[kvhead * FD + tid] = 0.0f;
    }
    if (tid == 0 && !A.host_epoch) {
      const uint32_t arrived = la_ctl::ctl_arrive(A.ctl, cv);
      la_ctl::ctl_leave(A.ctl, arrived, la_ctl::epoch_of(cv.gen));
    }
    return;
  }
  // buffer resources bounded to the sequence's rows of this head (rows past
  // its end read as zero and are not written; the caller keeps row strides
  // >= 64 elements and every offset below 2^31 bytes)
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
  const int64_t rem = nch - c_begin;
  const int ncl = (int)(rem < SEGC ? rem : SEGC);  // chunks of this segment (>= 1)
  const bool mine = w < ncl;                       // this wave owns a chunk
  const int t0 = (int)((c_begin + w) * FC);        // its first row
  const int nv = mine ? (int)((len - t0) < FC ? (len - t0) : FC) : 0;
  bf16* tK = reinterpret_cast<bf16*>(L.reg[w]);
  bf16* tV = reinterpret_cast<bf16*>(L.reg[w] + TILE_B);
  if (tid < FD) L.zero[tid] = (bf16)0.0f;

  // ------------------------------------------------------------------ A
  // Loads: K and V as 16-byte row pieces (rows lane / 8 + 8 u), Q directly
  // as operand fragments (query row 32 ib + r, features 16 kb + 8 h ..).
  // Rows past the sequence end read as zero.
  f32x16 O[2][2];     // numerator blocks (feature block nb, query block ib): rows b, column i
  Frag<bf16> qf[2][4];  // phi(Q) fragments (query block ib, feature block kb)
  float den[2] = {0.0f, 0.0f};  // chunk-local normaliser of query 32 ib + r
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) O[nb][ib] = f32x16{};
  if (mine) {
    u32x4 kr[8], vr[8], qr[2][4];
    const int prow = lane >> 3, pcol = 8 * (lane & 7);
#pragma unroll
    for (int u = 0; u < 8; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (t0 + prow + 8 * u) * ks + pcol * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (t0 + prow + 8 * u) * ks + pcol * 2, 0, 0);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        qr[ib][kb] = __builtin_amdgcn_raw_buffer_load_b128(rq, (t0 + 32 * ib + r) * qs + (16 * kb + 8 * h) * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      u32x4 x = kr[u];
      const bool real = prow + 8 * u < nv;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = SPLIT ? relu2(x[j]) : (real ? map2<PM>(x[j]) : 0u);
      *reinterpret_cast<u32x4*>(tK + (prow + 8 * u) * RS + pcol) = x;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<u32x4*>(tV + (prow + 8 * u) * RS + pcol) = vr[u];
    wave_lds_sync();

    // Fragments: V^T (feature block nb, token block kt): A operand of V^T P^T
    // and B operand of relu(K)^T V; relu(K)^T (feature block ab, token block
    // kt): A operand of relu(K)^T V; relu(K) token-major (key block jb,
    // feature block kb): A operand of P^T.  The chunk's state comes first: it
    // needs K and V only, so it runs while Q may still be arriving; the state
    // tile then overwrites the K and V tiles (rows b < 32 the V tile, rows
    // b >= 32 the K tile).
    Frag<bf16> vt[2][4], kt_[2][4], kf[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) vt[nb][kt] = ld_tr<RS>(tV, 16 * kt, 32 * nb, lane);
#pragma unroll
    for (int ab = 0; ab < 2; ++ab)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kt_[ab][kt] = ld_tr<RS>(tK, 16 * kt, 32 * ab, lane);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[jb][kb] = ld16(tK + (32 * jb + r) * RS + 16 * kb + 8 * h);
    wave_lds_sync();
    // column sums of V (b = 32 nb + r): the ones^T V part of the chunk's
    // state (phi(K) = relu(K) + 1), added to every row a below
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
    // z of the chunk: sum_t relu(K_t)[a] + nv, for a = 32 ab + r
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) {
      float zp = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int p = 0; p < 4; ++p) zp = dot2(pair(kt_[ab][kt], p), ONE2, zp);
      zp += __shfl_xor(zp, 32);
      if (h == 0) L.zloc[w][32 * ab + r] = zp + (SPLIT ? (float)nv : 0.0f);
    }
    // dS = relu(K)^T V + ones^T V, block (ab, bb): rows a, columns b; written
    // transposed (row b, four contiguous a per q) into the state tile
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mma(acc, kt_[ab][kt], vt[bb][kt]);
        float* row = state_row(L, w, 32 * bb + r) + 32 * ab + 4 * h;
        const float c = cs[bb];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4v*>(row + 8 * q) =
              f32x4v{acc[4 * q] + c, acc[4 * q + 1] + c, acc[4 * q + 2] + c, acc[4 * q + 3] + c};
      }
    }

#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 x = qr[ib][kb];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = SPLIT ? phi2(x[j]) : map2<PM>(x[j]);
        qf[ib][kb].v = __builtin_bit_cast(bf16x8, x);
      }
    // P^T blocks (key block jb, query block ib), jb <= ib (with ELU + 1 the
    // tile holds phi(K) and the accumulators start at 0):
    //   P_ij = phi(Q_i) . relu(K_j) + sum_a phi(Q_i)[a]
    // (the second term, the same for every key, is the accumulators' start
    // value: this lane's column is query r, whose features the lane pair
    // (h = 0, 1) holds between them); only the diagonal block is masked:
    // element e holds key row 8 (e >> 2) + 4 h + (e & 3) of query r.
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      float qs = 0.0f;
      if (SPLIT) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int p = 0; p < 4; ++p) qs = dot2(pair(qf[ib][kb], p), ONE2, qs);
        qs += __shfl_xor(qs, 32);
      }
      float ds = 0.0f;
#pragma unroll
      for (int jb = 0; jb <= ib; ++jb) {
        f32x16 pacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) pacc[e] = qs;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(pacc, kf[jb][kb], qf[ib][kb]);
        if (jb == ib) {
#pragma unroll
          for (int e = 0; e < 16; ++e) pacc[e] = (8 * (e >> 2) + 4 * h + (e & 3) <= r) ? pacc[e] : 0.0f;
        }
        const Frag<bf16> p0 = acc_frag(pacc, 0), p1 = acc_frag(pacc, 1);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          mma(O[nb][ib], vt[nb][2 * jb], p0);
          mma(O[nb][ib], vt[nb][2 * jb + 1], p1);
        }
        // den_i = sum_j P_ij over the rounded weights the numerator uses: this
        // lane's 16 rows j of column i
#pragma unroll
        for (int j = 0; j < 4; ++j) ds = dot2(pair(p1, j), ONE2, dot2(pair(p0, j), ONE2, ds));
      }
      den[ib] = ds + __shfl_xor(ds, 32);
    }
  }
  // the call's epoch, and this workgroup counted in (its loads are all in)
  uint32_t arrived = 0;
  if (tid == 0) {
    L.epoch = A.host_epoch ? A.host_epoch : la_ctl::epoch_of(cv.gen);
    L.expect = L.epoch + cv.skew;
    L.limit = la_ctl::wait_limit(cv);
    if (!A.host_epoch) arrived = la_ctl::ctl_arrive(A.ctl, cv);
  }
  __syncthreads();

  // ------------------------------------------------------------------ B
  // Scan: wave w owns state rows b = 8 w + lane / 8, features a0 .. a0 + 7.
  const int sb = 8 * w + (lane >> 3), sa = 8 * (lane & 7);
  float pre[SEGC][8];  // exclusive prefix over the segment's chunks
  float run[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) run[e] = 0.0f;
  float zpre[SEGC];
  float zrun = 0.0f;
#pragma unroll
  for (int c = 0; c < SEGC; ++c) {
    if (c < ncl) {
      const float* src = state_row(L, c, sb) + sa;
      const f32x4v x0 = *reinterpret_cast<const f32x4v*>(src);
      const f32x4v x1 = *reinterpret_cast<const f32x4v*>(src + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pre[c][e] = run[e];
        run[e] += e < 4 ? x0[e] : x1[e - 4];
      }
      if (w == 0) {
        zpre[c] = zrun;
        zrun += L.zloc[c][lane];
      }
    }
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(A.agg + head * A.nseg * AGG_FLOATS, 0, (int)(A.nseg * AGG_FLOATS * 4), 0x00020000);
  // A lane's slice of an aggregate (rows sb, features sa .. sa + 7) is kept as
  // two 16-byte halves 1 KB apart, so that each of a wave's store and load
  // instructions covers 1 KB contiguously
  const int soff = (w * 128 + lane) * 16;  // byte offset of this lane's first half in an aggregate
  const int zoff = FD * FD * 4;          // byte offset of z in an aggregate
  const bool publish = seg + 1 < nseg_s;  // the last segment has no successor
  uint64_t* flag = A.flags + head * A.nseg;
  if (publish) {
    const int base = (int)(seg * AGG_FLOATS * 4);
    st_buf<CPOL_SC1>(rs, base + soff, f32x4v{run[0], run[1], run[2], run[3]});
    st_buf<CPOL_SC1>(rs, base + soff + 1024, f32x4v{run[4], run[5], run[6], run[7]});
    if (w == 0) st_buf1<CPOL_SC1>(rs, base + zoff + lane * 4, zrun);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's aggregate stores have completed
  }
  __syncthreads();  // also: every state tile has been read
  if (publish && tid == 0) __hip_atomic_store(flag + seg, L.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // S_loc(c) (this segment's chunks before c) in bf16, [b][a] rows of RS,
  // over region c, and z_loc(c) as pairs; their products with phi(Q) run
  // while the earlier segments' aggregates are awaited.  S_loc(0) = 0.
#pragma unroll
  for (int c = 1; c < SEGC; ++c) {
    if (c < ncl) {
      uint32_t y[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = pack2(pre[c][2 * j], pre[c][2 * j + 1]);
      *reinterpret_cast<u32x4*>(reinterpret_cast<bf16*>(L.reg[c]) + sb * RS + sa) = u32x4{y[0], y[1], y[2], y[3]};
      if (w == 0) store_z_pairs(L.zh[c], L.zl[c], zpre[c], lane);
    }
  }
  __syncthreads();
  // num += phi(Q) S_loc (A operand S^T, rows b, over features); den_i +=
  // phi(Q_i) . z via rows 0 and 16 of the z operand (high and low parts)
  float dz[2] = {0.0f, 0.0f};  // phi(Q_i) . z terms (lanes with h == 0)
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
  if (mine && w > 0) state_products(reinterpret_cast<const bf16*>(L.reg[w]), L.zh[w], L.zl[w]);

  if (seg > 0) {
    if (w == 0) {
      const uint64_t expect = L.expect;
      const uint32_t limit = L.limit;
      for (int64_t p = lane; p < seg; p += 64) {
        uint32_t spins = 0;
        while (__hip_atomic_load(flag + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != expect) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins >= limit) {
            la_ctl::ctl_fail(A.ctl, la_internal::kErrWait);
            break;
          }
        }
      }
    }
    __syncthreads();
  }
  // S_prev and z_prev (this lane's slice), summed over earlier segments in
  // order, up to four segments' loads in flight
  float sp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sp[e] = 0.0f;
  float zprev = 0.0f;
  for (int64_t p = 0; p < seg; p += 4) {
    f32x4v x[4][2];
    float zx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (p + u < seg) {
        const int base = (int)((p + u) * AGG_FLOATS * 4);
        x[u][0] = ld_buf<CPOL_SC1>(rs, base + soff);
        x[u][1] = ld_buf<CPOL_SC1>(rs, base + soff + 1024);
        zx[u] = w == 0 ? ld_buf1<CPOL_SC1>(rs, base + zoff + lane * 4) : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (p + u < seg) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sp[e] += x[u][0][e];
          sp[e + 4] += x[u][1][e];
        }
        zprev += zx[u];
      }
    }
  }
  // S_prev in bf16 into the shared tile, z_prev as pairs
  if (seg > 0) {
    uint32_t y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = pack2(sp[2 * j], sp[2 * j + 1]);
    *reinterpret_cast<u32x4*>(L.sprev + sb * RS + sa) = u32x4{y[0], y[1], y[2], y[3]};
    if (w == 0) store_z_pairs(L.zhp, L.zlp, zprev, lane);
  }
  if (seg == nseg_s - 1 && member == 0) {  // the group's first member writes the final state
    if (A.S_final) {
      float* Sf = A.S_final + kvhead * FD * FD;
#pragma unroll
      for (int e = 0; e < 8; ++e) Sf[(sa + e) * FD + sb] = sp[e] + run[e];
    }
    if (A.z_final && w == 0) A.z_final[kvhead * FD + lane] = zprev + zrun;
  }
  __syncthreads();

  // ------------------------------------------------------------------ C
  if (mine) {
    if (seg > 0) state_products(L.sprev, L.zhp, L.zlp);
    float inv[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) inv[ib] = __builtin_amdgcn_rcpf(__shfl(den[ib] + dz[ib], r));  // from the lane with h == 0
    // the output rows go through LDS so that global stores cover whole
    // 128-byte rows, 16 bytes per lane; the stores are non-temporal, so that
    // they do not sit in L2 as dirty lines to be written back when the
    // kernel ends
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
    const int prow = lane >> 3, pcol = 8 * (lane & 7);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(tO + (prow + 8 * u) * RS + pcol), ro,
                                             (t0 + prow + 8 * u) * qs + pcol * 2, 0, CPOL_NT);
  }
  if (tid == 0 && !A.host_epoch) la_ctl::ctl_leave(A.ctl, arrived, L.epoch);
}

}  // namespace

namespace la_internal {

bool fused_causal_applies(int64_t Hq, int64_t Hkv, int64_t n, int64_t d, int dtype, int chunk) {
  // n bound: every segment sums the aggregates of all earlier segments of its
  // head, so the look-back grows with n; longer sequences take the
  // three-launch path, whose scan is linear in the number of segments.  With
  // grouped query heads each query head runs its own look-back, so the bound
  // is lower (B1 Hq32 Hkv8 d64, interleaved timing: 58.0 against 81.2 us at
  // n = 16384, 147 against 141 us at B2 Hq16 Hkv4 n = 32768, 375 against
  // 260 us at B1 Hq32 Hkv8 n = 65536, single launch against three).  R
  // bound: each query head reads its key/value head's rows again.
  const int64_t nmax = Hq == Hkv ? kFusedMaxN : kFusedMaxNGqa;
  return dtype == 1 && d == FD && Hq % Hkv == 0 && Hq / Hkv <= kFusedMaxR && chunk == FC && n <= nmax;
}

size_t fused_causal_ws_bytes(int64_t NH, int64_t nseg) {
  return (size_t)NH * nseg * (AGG_FLOATS * sizeof(float) + sizeof(uint64_t));
}

bool fused_seq_applies(const SeqCall& a) {
  const int64_t rs = a.S.qt > a.S.kt ? a.S.qt : a.S.kt;
  return a.q && a.window == 0 && a.vec && a.S.qt >= FD && a.S.kt >= FD &&
         fused_causal_applies(a.Hq, a.Hkv, a.S.n, a.d, a.dtype, FC) && (a.S.n + FC) * rs * 2 < ((int64_t)1 << 31);
}

template <bool SEQ, bool GQA>
static void launch_fused_pm(const FusedArgs& A, int phi, hipStream_t st) {
  const dim3 grid((unsigned)A.NH, (unsigned)A.nseg);
  if (phi == 2)
    k_causal_fused<PM_FEAT, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
  else if (phi == 1)
    k_causal_fused<PM_ELU1, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
  else
    k_causal_fused<PM_RELU1, SEQ, GQA><<<grid, FNT, 0, st>>>(A);
}

template <bool SEQ>
static int launch_fused(FusedArgs& A, int phi, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  static_assert(kFusedG == SEGC, "segment length");
  A.flags = reinterpret_cast<uint64_t*>(A.agg + A.NH * A.nseg * AGG_FLOATS);
  A.host_epoch = launch_epoch(stream);
  // the GQA instantiation only where needed: the kernel's schedule is
  // sensitive to the extra index arithmetic (0.8 us on the B8 H8 n2048 call)
  if (A.R > 1)
    launch_fused_pm<SEQ, true>(A, phi, st);
  else
    launch_fused_pm<SEQ, false>(A, phi, st);
  return (int)hipGetLastError();
}

// The XCD-aware dispatch order needs whole blocks of eight groups.
static int xcd_order(int64_t groups, int R) { return R > 1 && groups % 8 == 0; }

int launch_causal_fused(const Fwd& a, const Plan& p) {
  const int64_t n = a.n;
  const int R = (int)(a.Hq / a.Hkv);
  FusedArgs A{reinterpret_cast<const bf16*>(a.q), reinterpret_cast<const bf16*>(a.k),
              reinterpret_cast<const bf16*>(a.v), reinterpret_cast<bf16*>(a.out), n, p.nchunks, p.nseg,
              a.B * a.Hq, a.Hq, a.Hq * n * FD, n * FD, FD, a.Hkv * n * FD, n * FD, FD, R, xcd_order(a.B * a.Hkv, R),
              nullptr, a.B * n, reinterpret_cast<float*>(a.ws), nullptr, a.S_final, a.z_final, a.ctl, 0};
  return launch_fused<false>(A, a.phi, a.stream);
}

int launch_causal_fused_seq(const SeqCall& a) {
  const int64_t nchunks = (a.S.n + FC - 1) / FC;
  const int R = (int)(a.Hq / a.Hkv);
  FusedArgs A{reinterpret_cast<const bf16*>(a.q), reinterpret_cast<const bf16*>(a.k),
              reinterpret_cast<const bf16*>(a.v), reinterpret_cast<bf16*>(a.out), a.S.n, nchunks,
              (nchunks + SEGC - 1) / SEGC, a.nseq * a.Hq, a.Hq, a.S.qb, a.S.qh, a.S.qt, a.S.kb, a.S.kh, a.S.kt,
              R, xcd_order(a.nseq * a.Hkv, R), a.S.cu, a.S.total, reinterpret_cast<float*>(a.ws), nullptr,
              a.S_final, a.z_final, a.ctl, 0};
  return launch_fused<true>(A, a.phi, a.stream);
}

size_t fused_seq_ws_bytes(const SeqCall& a) {
  const int64_t nchunks = (a.S.n + FC - 1) / FC;
  return fused_causal_ws_bytes(a.nseq * a.Hq, (nchunks + SEGC - 1) / SEGC);
}

}  // namespace la_internal
