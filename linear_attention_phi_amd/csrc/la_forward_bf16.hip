// la_forward_bf16.hip -- non-causal pass for bf16 inputs with d = 64 (gfx950).
//
// out_i = phi(Q_i) S / (phi(Q_i) . z) with S = sum_j phi(K_j) (x) V_j and
// z = sum_j phi(K_j) over all n keys of the query's key/value head
// (nx_f32_linear_attention.nx source, header comment: S and z over all
// keys, then each query's normalised read; LinearTile 1.0.1, "How It Works": K^T V once, then Q).  One launch
// whose workgroups take one of three roles by their index, streaming the
// data once with one wave per 64-token chunk:
//
//  state    (the first NKV * nseg workgroups) a workgroup of four waves owns
//           four chunks of one key/value head; each wave forms its chunk's
//           relu(K)^T V on MFMA (fp32, transposed operands from LDS with
//           ds_read_b64_tr_b16), the column sums of V and z; the workgroup
//           sums its four chunks in LDS and publishes one partial (S^T [b][a]
//           fp32, then z);
//  reduce   (the next NKV * RED_BLOCKS) once a head's partials are all
//           published, sums them in segment order (one lane slot per
//           thread, so the result does not depend on timing) and publishes
//           S^T as bf16 in MFMA operand order and z as bf16 (high, low) pairs;
//  output   (the rest) one wave per two chunks of queries, so that at the
//           common shapes the whole grid is resident at once (two
//           workgroups per CU): its Q fragments are requested straight from
//           HBM at once, so they stream while the state is formed; once the
//           head's total is published, per chunk: num =
//           phi(Q) S and phi(Q) . z on MFMA, division, rows staged through
//           LDS and stored whole with non-temporal stores.
//
// A workgroup only waits for workgroups of lower index, which are
// dispatched before it.  Published data goes through memory with
// device-scope (sc1) stores and loads, and each publication is announced
// by a 64-bit flag set to the call's epoch (taken from the workspace's
// control block, la_ctl.h: a NaN pattern that no value the workspace held
// before can equal, new for every call and every replay of a captured
// launch) once the data stores have completed.  Spins are bounded;
// exhausting the bound records an error bit in the control block instead of
// hanging.
//
// phi(K)^T V is formed as relu(K)^T V + 1 (x) sum_t V_t and z as
// sum_t relu(K_t) + (number of keys), exactly as in the causal kernels; with
// ELU + 1 (template PM) phi(K) and phi(Q) are rounded to bf16 in the tiles
// and fragments instead, and key rows past the end are 0, not phi(0).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_bf16.h"
#include "la_ctl.h"
#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;
using namespace la_bf16;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int FD = 64;                     // head dim
constexpr int FC = 64;                     // chunk
constexpr int W = la_internal::kFwdSegChunks;  // chunks per state workgroup = waves
constexpr int OC = 2;                      // chunks per output wave
constexpr int WNT = 64 * W;                // threads per workgroup
constexpr int RS = FD + 8;                 // row stride (bf16) of the token-major tiles: 144 bytes
constexpr int RSF = FD + 4;                // row stride (fp32) of the state tiles: 272 bytes
constexpr int TILE_B = FC * RS * 2;        // bytes of one token-major bf16 tile
constexpr int REGION_B = 2 * TILE_B;       // one wave's LDS region (state kernel)
// S^T is published in MFMA operand order: fragment (nb, kb) -- rows b = 32 nb
// + 0..31, features a = 16 kb + 0..15 -- is a block of 64 lane slots, lane
// r + 32 h holding b = 32 nb + r, a = 16 kb + 8 h .. + 7.  A partial keeps
// each slot's 8 floats as two 16-byte halves in separate 1 KB blocks
// ((fragment, half) blocks of 64 lanes), the total keeps 8 bf16 per slot; so
// every store and load instruction of a wave covers 1 KB contiguously.
constexpr int PART_FLOATS = FD * FD + FD;  // one partial: S^T slots, then z
constexpr int TOT_BYTES = FD * FD * 2 + FD * 4;  // one total: S^T bf16 slots, then z high and low pairs
constexpr int RED_THREADS = 256;
constexpr int RED_S_BLOCKS = FD * FD / 8 / RED_THREADS;  // reduce workgroups per head for S^T (a slot each)
constexpr int RED_BLOCKS = RED_S_BLOCKS + 1;               // and one for z
constexpr int RED_BATCH = 16;                              // segments' loads in flight per reduce step

struct FwdArgs {
  const bf16* q; const bf16* k; const bf16* v; bf16* out;
  int64_t n, nchunks, nseg, NKV, NQ, R;  // nseg: state workgroups per head
  float* part;      // [NKV][nseg][PART_FLOATS]
  uint8_t* tot;     // [NKV][TOT_BYTES]
  uint64_t* sflag;  // [NKV][nseg]: the segment's partial is published
  uint64_t* rflag;  // [NKV][RED_BLOCKS]: the slice of the head's total is published
  la_internal::Ctl* ctl;
  uint64_t host_epoch;  // the call's epoch, or 0: take it from the control block
};

// The call's epoch as the workgroup sees it (in LDS, written by thread 0).
struct EpochLds {
  uint64_t epoch, expect;  // flags are set to epoch; waits compare with expect
  uint32_t limit;          // polls before a wait gives up
};

// Thread 0 takes the call's epoch from the control words it loaded and counts
// the workgroup in; returns the counter's old value (for ctl_leave).
__device__ __forceinline__ uint32_t take_epoch(const FwdArgs& A, const la_ctl::CtlView& cv, EpochLds& E) {
  E.epoch = A.host_epoch ? A.host_epoch : la_ctl::epoch_of(cv.gen);
  E.expect = E.epoch + cv.skew;
  E.limit = la_ctl::wait_limit(cv);
  return A.host_epoch ? 0u : la_ctl::ctl_arrive(A.ctl, cv);
}
// The thread that took the epoch, after its last use of it.
__device__ __forceinline__ void leave_epoch(const FwdArgs& A, uint32_t arrived, const EpochLds& E) {
  if (!A.host_epoch) la_ctl::ctl_leave(A.ctl, arrived, E.epoch);
}

// Every lane of the calling wave spins until flags[0 .. cnt) all hold the
// call's epoch, then orders its later loads after the flags.
__device__ __forceinline__ void wait_epoch(const uint64_t* flags, int64_t cnt, const FwdArgs& A, const EpochLds& E,
                                           int lane) {
  const uint64_t expect = E.expect;
  const uint32_t limit = E.limit;
  for (int64_t p = lane; p < cnt; p += 64) {
    uint32_t spins = 0;
    while (__hip_atomic_load(flags + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != expect) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins >= limit) {
        la_ctl::ctl_fail(A.ctl, la_internal::kErrWait);
        break;
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

struct StateLds {
  uint8_t reg[W][REGION_B];  // relu(K), V tiles; then the chunk's state dS^T [b][a] in fp32
  float zloc[W][FD];         // z of each chunk
  float vsum[W][FD];         // sum_t V_t of each chunk, by column b
};
static_assert(32 * RSF * 4 <= TILE_B, "state half-tile must fit a token-major tile");

__device__ __forceinline__ float* state_row(StateLds& L, int c, int b) {
  return reinterpret_cast<float*>(L.reg[c] + (b < 32 ? TILE_B : 0)) + (b & 31) * RSF;
}

template <int PM>
__device__ __forceinline__ void fwd_state(const FwdArgs& A, int64_t bid, StateLds& L, EpochLds& E) {
  constexpr bool SPLIT = PM == PM_RELU1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  la_ctl::CtlView cv{};
  if (w == 0) cv = la_ctl::ctl_load(A.ctl);  // used once this wave's loads are in
  const int64_t seg = bid / A.NKV, head = bid % A.NKV;
  const int hbytes = (int)(A.n * FD * 2);  // one head's rows (n <= 2^24)
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.k + head * A.n * FD), 0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.v + head * A.n * FD), 0, hbytes, 0x00020000);
  const int64_t c_begin = seg * W;
  const int64_t rem = A.nchunks - c_begin;
  const int ncl = (int)(rem < W ? rem : W);  // chunks of this segment (>= 1)
  const bool mine = w < ncl;
  const int t0 = (int)((c_begin + w) * FC);
  const int nv = mine ? (int)((A.n - t0) < FC ? (A.n - t0) : FC) : 0;

  if (mine) {
    bf16* tK = reinterpret_cast<bf16*>(L.reg[w]);
    bf16* tV = reinterpret_cast<bf16*>(L.reg[w] + TILE_B);
    u32x4 kr[8], vr[8];
    const int prow = lane >> 3, pcol = 8 * (lane & 7);
#pragma unroll
    for (int u = 0; u < 8; ++u) kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((t0 + prow + 8 * u) * FD + pcol) * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((t0 + prow + 8 * u) * FD + pcol) * 2, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      u32x4 x = kr[u];
      const bool real = prow + 8 * u < nv;  // ELU + 1: rows past the end hold 0, not phi(0)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = SPLIT ? relu2(x[j]) : (real ? map2<PM>(x[j]) : 0u);
      *reinterpret_cast<u32x4*>(tK + (prow + 8 * u) * RS + pcol) = x;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<u32x4*>(tV + (prow + 8 * u) * RS + pcol) = vr[u];
    wave_lds_sync();
    // V^T (feature block nb, token block kt) and relu(K)^T (feature block ab,
    // token block kt) fragments; then the state tile overwrites the tiles
    Frag<bf16> vt[2][4], kt_[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) vt[nb][kt] = ld_tr<RS>(tV, 16 * kt, 32 * nb, lane);
#pragma unroll
    for (int ab = 0; ab < 2; ++ab)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kt_[ab][kt] = ld_tr<RS>(tK, 16 * kt, 32 * ab, lane);
    wave_lds_sync();
    // column sums of V (b = 32 nb + r) and z (a = 32 ab + r)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float cs = 0.0f;  // (the ones part of relu + 1 only)
      if (SPLIT) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int p = 0; p < 4; ++p) cs = dot2(pair(vt[nb][kt], p), ONE2, cs);
        cs += __shfl_xor(cs, 32);
      }
      if (h == 0) L.vsum[w][32 * nb + r] = cs;
    }
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
    // dS = relu(K)^T V, block (ab, bb): rows a, columns b; written transposed
    // (row b, four contiguous a per q)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int ab = 0; ab < 2; ++ab) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mma(acc, kt_[ab][kt], vt[bb][kt]);
        float* row = state_row(L, w, 32 * bb + r) + 32 * ab + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<f32x4v*>(row + 8 * q) = f32x4v{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      }
    }
  }
  uint32_t arrived = 0;
  if (tid == 0) arrived = take_epoch(A, cv, E);
  __syncthreads();

  // The segment's partial: thread (w, lane) sums the lane slots of
  // fragments w and w + 4 -- rows b = 32 i + r (i = 0, 1), features a = 16 w
  // + 8 h .. + 7 -- over its chunks (plus the ones^T V part), wave 0 also z.
  float run[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) run[i][e] = 0.0f;
  float zrun = 0.0f;
#pragma unroll
  for (int c = 0; c < W; ++c) {
    if (c < ncl) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4v* src = reinterpret_cast<const f32x4v*>(state_row(L, c, 32 * i + r) + 16 * w + 8 * h);
        const float cs = L.vsum[c][32 * i + r];
        const f32x4v x0 = src[0], x1 = src[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          run[i][e] += x0[e] + cs;
          run[i][4 + e] += x1[e] + cs;
        }
      }
      zrun += L.zloc[c][lane];
    }
  }
  // publish: device-scope stores, completed before the barrier, then the flag
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      A.part + (head * A.nseg + seg) * PART_FLOATS, 0, PART_FLOATS * 4, 0x00020000);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      st_buf<CPOL_SC1>(rp, (((w + 4 * i) * 2 + hf) * 64 + lane) * 16,
                       f32x4v{run[i][4 * hf], run[i][4 * hf + 1], run[i][4 * hf + 2], run[i][4 * hf + 3]});
  if (w == 0) st_buf1<CPOL_SC1>(rp, (FD * FD + lane) * 4, zrun);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_store(A.sflag + head * A.nseg + seg, E.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    leave_epoch(A, arrived, E);
  }
}

// Thread t of a head's RED_BLOCKS * RED_THREADS handles floats 4 t .. 4 t + 3
// of a partial (S^T [b][a] for 4 t < FD * FD, else z).
__device__ __forceinline__ void fwd_reduce(const FwdArgs& A, int64_t bid, EpochLds& E) {
  const int64_t head = bid / RED_BLOCKS, slice = bid % RED_BLOCKS;
  uint32_t arrived = 0;
  if (threadIdx.x == 0) arrived = take_epoch(A, la_ctl::ctl_load(A.ctl), E);
  __syncthreads();
  wait_epoch(A.sflag + head * A.nseg, A.nseg, A, E, threadIdx.x & 63);
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      A.part + head * A.nseg * PART_FLOATS, 0, (int)(A.nseg * PART_FLOATS * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(A.tot + head * TOT_BYTES, 0, TOT_BYTES, 0x00020000);
  // past every head's partials (nseg * PART_FLOATS * 4 < 2^30 bytes): reads
  // as zero, and adding a slot's offset cannot overflow
  constexpr int OOB = 1 << 30;
  static_assert((la_internal::kFwdMaxN / (FC * W) + 1) * PART_FLOATS * 4 < (1 << 30), "partials below 2^30 bytes");
  if (slice < RED_S_BLOCKS) {
    // lane slot t of S^T: fragment t / 64, lane t % 64; its two halves
    const int t = (int)slice * RED_THREADS + threadIdx.x;
    const int o0 = ((t >> 6) * 2 * 64 + (t & 63)) * 16, o1 = o0 + 64 * 16;
    // up to RED_BATCH segments' loads in flight, summed in segment order
    f32x4v s0 = f32x4v{0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
    for (int64_t p = 0; p < A.nseg; p += RED_BATCH) {
      f32x4v x[RED_BATCH][2];
#pragma unroll
      for (int u = 0; u < RED_BATCH; ++u) {
        const int base = p + u < A.nseg ? (int)((p + u) * PART_FLOATS * 4) : OOB;
        x[u][0] = ld_buf<CPOL_SC1>(rp, base + o0);
        x[u][1] = ld_buf<CPOL_SC1>(rp, base + o1);
      }
#pragma unroll
      for (int u = 0; u < RED_BATCH; ++u) {
        s0 += x[u][0];
        s1 += x[u][1];
      }
    }
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{pack2(s0[0], s0[1]), pack2(s0[2], s0[3]), pack2(s1[0], s1[1]), pack2(s1[2], s1[3])}, rt, t * 16, 0,
        CPOL_SC1);
  } else if (threadIdx.x < FD / 4) {
    // z as (high, low) bf16 pairs: z = high + low to about 2^-17
    const int a = 4 * (int)threadIdx.x;
    f32x4v zs = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t p = 0; p < A.nseg; p += RED_BATCH) {
      f32x4v x[RED_BATCH];
#pragma unroll
      for (int u = 0; u < RED_BATCH; ++u)
        x[u] = ld_buf<CPOL_SC1>(rp, p + u < A.nseg ? (int)(((p + u) * PART_FLOATS + FD * FD + a) * 4) : OOB);
#pragma unroll
      for (int u = 0; u < RED_BATCH; ++u) zs += x[u];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t hi = pack2(zs[2 * j], zs[2 * j + 1]);
      const uint32_t lo = pack2(zs[2 * j] - lo_f(hi), zs[2 * j + 1] - hi_f(hi));
      __builtin_amdgcn_raw_buffer_store_b32(hi, rt, FD * FD * 2 + (a / 2 + j) * 4, 0, CPOL_SC1);
      __builtin_amdgcn_raw_buffer_store_b32(lo, rt, FD * FD * 2 + FD * 2 + (a / 2 + j) * 4, 0, CPOL_SC1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(A.rflag + head * RED_BLOCKS + slice, E.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    leave_epoch(A, arrived, E);
  }
}

template <int PM>
__device__ __forceinline__ void fwd_out(const FwdArgs& A, int64_t bid, uint8_t (&Lout)[W][TILE_B], EpochLds& E) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  const int64_t seg = bid / A.NQ, qh = bid % A.NQ, kvh = qh / A.R;
  const int64_t c0 = (seg * W + w) * OC;  // this wave's first chunk (wave 0 always has one)
  la_ctl::CtlView cv{};
  if (w == 0) cv = la_ctl::ctl_load(A.ctl);
  if (c0 >= A.nchunks) {  // a wave without a chunk leaves after the epoch barrier
    __syncthreads();
    return;
  }
  const int hbytes = (int)(A.n * FD * 2);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.q + qh * A.n * FD), 0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(A.out + qh * A.n * FD, 0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(A.tot + kvh * TOT_BYTES, 0, TOT_BYTES, 0x00020000);
  constexpr int OOB = 0x7FFFFFF0;  // past num_records: reads as zero
  // phi(Q) (chunk j, query block ib, feature block kb), S^T (feature block
  // nb, kb) and the z operand (row 0: high parts, row 16: low parts, other
  // rows zero).  Q of both chunks is requested first, before the wait for
  // the head's total (rows past the sequence end read as zero); the total's
  // loads are all issued before phi is applied to Q (left to itself the
  // compiler waits for each fragment before issuing the next)
  u32x4 qraw[OC][2][4];
#pragma unroll
  for (int j = 0; j < OC; ++j)
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        qraw[j][ib][kb] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (((int)(c0 + j) * FC + 32 * ib + r) * FD + 16 * kb + 8 * h) * 2, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t arrived = 0;
  if (tid == 0) arrived = take_epoch(A, cv, E);
  __syncthreads();
  wait_epoch(A.rflag + kvh * RED_BLOCKS, RED_BLOCKS, A, E, lane);
  Frag<bf16> sf[2][4], zf[4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sf[nb][kb].v = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rt, ((nb * 4 + kb) * 64 + lane) * 16, 0, CPOL_SC1));
  const int zrow = r == 0 ? FD * FD * 2 : (r == 16 ? FD * FD * 2 + FD * 2 : -1);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    zf[kb].v = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rt, zrow < 0 ? OOB : zrow + (16 * kb + 8 * h) * 2, 0, CPOL_SC1));
  __builtin_amdgcn_sched_barrier(0);

  bf16* tO = reinterpret_cast<bf16*>(Lout[w]);
  const int prow = lane >> 3, pcol = 8 * (lane & 7);
#pragma unroll
  for (int j = 0; j < OC; ++j) {
    const int t0 = (int)(c0 + j) * FC;
    Frag<bf16> qf[2][4];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 x = qraw[j][ib][kb];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = PM == PM_RELU1 ? phi2(x[e]) : map2<PM>(x[e]);
        qf[ib][kb].v = __builtin_bit_cast(bf16x8, x);
      }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      f32x16 zacc = f32x16{};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(zacc, zf[kb], qf[ib][kb]);
      const float inv = __builtin_amdgcn_rcpf(__shfl(zacc[0] + zacc[8], r));  // from the lane with h == 0
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x16 o = f32x16{};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(o, sf[nb][kb], qf[ib][kb]);
        uint2* dst = reinterpret_cast<uint2*>(tO + (32 * ib + r) * RS + 32 * nb + 4 * h);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dst[2 * q] = make_uint2(pack2(o[4 * q] * inv, o[4 * q + 1] * inv), pack2(o[4 * q + 2] * inv, o[4 * q + 3] * inv));
      }
    }
    wave_lds_sync();
    // whole 128-byte rows, 16 bytes per lane; rows past the sequence end fall
    // outside the bounded resource and are dropped (the wave's LDS accesses
    // run in order, so the next chunk's tile writes follow these reads)
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(tO + (prow + 8 * u) * RS + pcol), ro,
                                             ((t0 + prow + 8 * u) * FD + pcol) * 2, 0, CPOL_NT);
  }
  if (tid == 0) leave_epoch(A, arrived, E);
}

union FwdLds {
  StateLds state;
  uint8_t out[W][TILE_B];
};

template <int PM>
__global__ __launch_bounds__(WNT) void k_fwd_one(FwdArgs A) {
  __shared__ __attribute__((aligned(16))) FwdLds L;
  __shared__ EpochLds E;
  const int64_t nS = A.NKV * A.nseg, nR = A.NKV * RED_BLOCKS, b = blockIdx.x;
  if (b < nS)
    fwd_state<PM>(A, b, L.state, E);
  else if (b < nS + nR)
    fwd_reduce(A, b - nS, E);
  else
    fwd_out<PM>(A, b - nS - nR, L.out, E);
}

}  // namespace

namespace la_internal {

bool forward_bf16_applies(int64_t n, int64_t d, int dtype) {
  return dtype == 1 && d == FD && n <= kFwdMaxN;
}

int64_t forward_bf16_nseg(int64_t n) { return ((n + FC - 1) / FC + W - 1) / W; }

int64_t forward_bf16_grid(int64_t NKV, int64_t NQ, int64_t n) {
  const int64_t nchunks = (n + FC - 1) / FC;
  return NKV * forward_bf16_nseg(n) + NKV * RED_BLOCKS + NQ * ((nchunks + W * OC - 1) / (W * OC));
}

size_t forward_bf16_ws_bytes(int64_t NKV, int64_t nseg) {
  return (size_t)NKV * nseg * PART_FLOATS * sizeof(float) + (size_t)NKV * TOT_BYTES +
         (size_t)NKV * (nseg + RED_BLOCKS) * sizeof(uint64_t);
}

int launch_forward_bf16(const Fwd& a) {
  static_assert(RED_THREADS == WNT, "one block size for every role");
  static_assert(RED_S_BLOCKS * RED_THREADS * 8 == FD * FD && FD / 4 <= RED_THREADS, "reduce slices");
  static_assert(TOT_BYTES % 16 == 0 && (PART_FLOATS * 4) % 16 == 0, "workspace alignment");
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int64_t NKV = a.B * a.Hkv, NQ = a.B * a.Hq;
  const int64_t nchunks = (a.n + FC - 1) / FC, nseg = forward_bf16_nseg(a.n);
  float* part = reinterpret_cast<float*>(a.ws);
  uint8_t* tot = reinterpret_cast<uint8_t*>(part + NKV * nseg * PART_FLOATS);
  uint64_t* sflag = reinterpret_cast<uint64_t*>(tot + NKV * TOT_BYTES);
  uint64_t* rflag = sflag + NKV * nseg;
  FwdArgs A{reinterpret_cast<const bf16*>(a.q), reinterpret_cast<const bf16*>(a.k),
            reinterpret_cast<const bf16*>(a.v), reinterpret_cast<bf16*>(a.out), a.n, nchunks, nseg, NKV, NQ,
            a.Hq / a.Hkv, part, tot, sflag, rflag, a.ctl, launch_epoch(a.stream)};
  if (a.phi == 2)
    k_fwd_one<PM_FEAT><<<dim3((unsigned)forward_bf16_grid(NKV, NQ, a.n)), WNT, 0, st>>>(A);
  else if (a.phi == 1)
    k_fwd_one<PM_ELU1><<<dim3((unsigned)forward_bf16_grid(NKV, NQ, a.n)), WNT, 0, st>>>(A);
  else
    k_fwd_one<PM_RELU1><<<dim3((unsigned)forward_bf16_grid(NKV, NQ, a.n)), WNT, 0, st>>>(A);
  return (int)hipGetLastError();
}

}  // namespace la_internal
