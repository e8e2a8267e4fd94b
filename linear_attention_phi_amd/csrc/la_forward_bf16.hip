// la_forward_bf16.hip -- non-causal pass for bf16 inputs with d = 64 (gfx950).
//
// out_i = phi(Q_i) S / (phi(Q_i) . z) with S = sum_j phi(K_j) (x) V_j and
// z = sum_j phi(K_j) over all n keys of the query's key/value head
// (nx_f32_linear_attention.nx: "accumulate KV-summary" and "per-query"
// loops; LinearTile 1.0.1, "How It Works": K^T V once, then Q).  Three
// launches, each streaming its data once with one wave per 64-token chunk:
//
//  k_fwd_state   a workgroup of four waves owns four chunks of one key/value
//                head; each wave forms its chunk's relu(K)^T V on MFMA (fp32,
//                transposed operands from LDS with ds_read_b64_tr_b16), the
//                column sums of V and z; the workgroup sums its four chunks
//                in LDS and writes one partial (S^T [b][a] fp32, then z);
//  k_fwd_reduce  sums each head's partials in segment order (one 16-byte
//                slice per thread, so the result does not depend on timing)
//                and stores S^T as bf16 in MFMA operand order and z as bf16
//                (high, low) pairs;
//  k_fwd_out     one wave per chunk of queries: phi(Q) fragments straight
//                from HBM, num = phi(Q) S and phi(Q) . z on MFMA, division,
//                rows staged through LDS and stored whole with non-temporal
//                stores.
//
// phi(K)^T V is formed as relu(K)^T V + 1 (x) sum_t V_t and z as
// sum_t relu(K_t) + (number of keys), exactly as in the causal kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_bf16.h"
#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;
using namespace la_bf16;

constexpr int FD = 64;                     // head dim
constexpr int FC = 64;                     // chunk
constexpr int W = la_internal::kFwdSegChunks;  // chunks per state workgroup = waves
constexpr int WNT = 64 * W;                // threads per workgroup
constexpr int RS = FD + 8;                 // row stride (bf16) of the token-major tiles: 144 bytes
constexpr int RSF = FD + 4;                // row stride (fp32) of the state tiles: 272 bytes
constexpr int TILE_B = FC * RS * 2;        // bytes of one token-major bf16 tile
constexpr int REGION_B = 2 * TILE_B;       // one wave's LDS region (state kernel)
constexpr int PART_FLOATS = FD * FD + FD;  // one partial: S^T [b][a], then z
constexpr int TOT_BYTES = FD * FD * 2 + FD * 4;  // one total: S^T bf16, then z high and low pairs
constexpr int RED_THREADS = 256;
constexpr int RED_BLOCKS = (PART_FLOATS / 4 + RED_THREADS - 1) / RED_THREADS;  // blocks per head

struct FwdArgs {
  const bf16* q; const bf16* k; const bf16* v; bf16* out;
  int64_t n, nchunks, nseg, NKV, NQ, R;
  float* part;    // [NKV][nseg][PART_FLOATS]
  uint8_t* tot;   // [NKV][TOT_BYTES]
};

struct StateLds {
  uint8_t reg[W][REGION_B];  // relu(K), V tiles; then the chunk's state dS^T [b][a] in fp32
  float zloc[W][FD];         // z of each chunk
  float vsum[W][FD];         // sum_t V_t of each chunk, by column b
};
static_assert(32 * RSF * 4 <= TILE_B, "state half-tile must fit a token-major tile");

__device__ __forceinline__ float* state_row(StateLds& L, int c, int b) {
  return reinterpret_cast<float*>(L.reg[c] + (b < 32 ? TILE_B : 0)) + (b & 31) * RSF;
}

__global__ __launch_bounds__(WNT) void k_fwd_state(FwdArgs A) {
  __shared__ __attribute__((aligned(16))) StateLds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  const int64_t seg = blockIdx.x / A.NKV, head = blockIdx.x % A.NKV;
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
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = relu2(x[j]);
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
      float cs = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int p = 0; p < 4; ++p) cs = dot2(pair(vt[nb][kt], p), ONE2, cs);
      cs += __shfl_xor(cs, 32);
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
      if (h == 0) L.zloc[w][32 * ab + r] = zp + (float)nv;
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
  __syncthreads();

  // The segment's partial: wave w sums rows b = 16 w + lane / 4, features
  // a0 .. a0 + 15 over its chunks (plus the ones^T V part), wave 0 also z.
  const int sb = 16 * w + (lane >> 2), sa = 16 * (lane & 3);
  float run[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) run[e] = 0.0f;
  float zrun = 0.0f;
#pragma unroll
  for (int c = 0; c < W; ++c) {
    if (c < ncl) {
      const f32x4v* src = reinterpret_cast<const f32x4v*>(state_row(L, c, sb) + sa);
      const float cs = L.vsum[c][sb];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4v x = src[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) run[4 * j + e] += x[e] + cs;
      }
      zrun += L.zloc[c][lane];
    }
  }
  // non-temporal: the partials are read once, by the next launch, and would
  // otherwise wait in L2 as dirty lines for the write-back at the kernel's end
  float* dst = A.part + (head * A.nseg + seg) * PART_FLOATS;
  f32x4v* d4 = reinterpret_cast<f32x4v*>(dst + sb * FD + sa);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    __builtin_nontemporal_store(f32x4v{run[4 * j], run[4 * j + 1], run[4 * j + 2], run[4 * j + 3]}, d4 + j);
  if (w == 0) __builtin_nontemporal_store(zrun, dst + FD * FD + lane);
}

// Thread t of a head's RED_BLOCKS * RED_THREADS handles floats 4 t .. 4 t + 3
// of a partial (S^T [b][a] for 4 t < FD * FD, else z).
__global__ __launch_bounds__(RED_THREADS) void k_fwd_reduce(FwdArgs A) {
  const int64_t head = blockIdx.x / RED_BLOCKS;
  const int t = (int)(blockIdx.x % RED_BLOCKS) * RED_THREADS + threadIdx.x;
  if (4 * t >= PART_FLOATS) return;
  const float* src = A.part + head * A.nseg * PART_FLOATS + 4 * t;
  f32x4v s = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  int64_t p = 0;
  for (; p + 8 <= A.nseg; p += 8) {
    f32x4v x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const f32x4v*>(src + (p + u) * PART_FLOATS);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += x[u];
  }
  for (; p < A.nseg; ++p) s += *reinterpret_cast<const f32x4v*>(src + p * PART_FLOATS);
  uint8_t* tot = A.tot + head * TOT_BYTES;
  if (4 * t < FD * FD) {
    *reinterpret_cast<uint2*>(tot + 8 * t) = make_uint2(pack2(s[0], s[1]), pack2(s[2], s[3]));
  } else {
    // z as (high, low) bf16 pairs: z = high + low to about 2^-17
    const int a = 4 * t - FD * FD;
    uint32_t* zh = reinterpret_cast<uint32_t*>(tot + FD * FD * 2);
    uint32_t* zl = zh + FD / 2;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t hi = pack2(s[2 * j], s[2 * j + 1]);
      zh[a / 2 + j] = hi;
      zl[a / 2 + j] = pack2(s[2 * j] - lo_f(hi), s[2 * j + 1] - hi_f(hi));
    }
  }
}

__global__ __launch_bounds__(WNT) void k_fwd_out(FwdArgs A) {
  __shared__ __attribute__((aligned(16))) uint8_t Lout[W][TILE_B];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  const int64_t seg = blockIdx.x / A.NQ, qh = blockIdx.x % A.NQ, kvh = qh / A.R;
  const int64_t c = seg * W + w;
  if (c >= A.nchunks) return;  // no barrier below: a wave without a chunk leaves
  const int t0 = (int)(c * FC);
  const int hbytes = (int)(A.n * FD * 2);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(A.q + qh * A.n * FD), 0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(A.out + qh * A.n * FD, 0, hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(A.tot + kvh * TOT_BYTES, 0, TOT_BYTES, 0x00020000);
  constexpr int OOB = 0x7FFFFFF0;  // past num_records: reads as zero
  // phi(Q) (query block ib, feature block kb), S^T (feature block nb, kb) and
  // the z operand (row 0: high parts, row 16: low parts, other rows zero)
  // every load is issued before phi is applied to Q (left to itself the
  // compiler waits for each Q fragment before issuing the next)
  u32x4 qraw[2][4];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      qraw[ib][kb] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((t0 + 32 * ib + r) * FD + 16 * kb + 8 * h) * 2, 0, 0);
  Frag<bf16> qf[2][4], sf[2][4], zf[4];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      sf[nb][kb].v = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rt, ((32 * nb + r) * FD + 16 * kb + 8 * h) * 2, 0, 0));
  const int zrow = r == 0 ? FD * FD * 2 : (r == 16 ? FD * FD * 2 + FD * 2 : -1);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    zf[kb].v = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rt, zrow < 0 ? OOB : zrow + (16 * kb + 8 * h) * 2, 0, 0));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4 x = qraw[ib][kb];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = phi2(x[j]);
      qf[ib][kb].v = __builtin_bit_cast(bf16x8, x);
    }

  bf16* tO = reinterpret_cast<bf16*>(Lout[w]);
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
  // outside the bounded resource and are dropped
  const int prow = lane >> 3, pcol = 8 * (lane & 7);
#pragma unroll
  for (int u = 0; u < 8; ++u)
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(tO + (prow + 8 * u) * RS + pcol), ro,
                                           ((t0 + prow + 8 * u) * FD + pcol) * 2, 0, CPOL_NT);
}

}  // namespace

namespace la_internal {

bool forward_bf16_applies(int64_t n, int64_t d, int dtype) {
  return dtype == 1 && d == FD && n <= kFwdMaxN;
}

int64_t forward_bf16_nseg(int64_t n) { return ((n + FC - 1) / FC + W - 1) / W; }

size_t forward_bf16_ws_bytes(int64_t NKV, int64_t nseg) {
  return (size_t)NKV * nseg * PART_FLOATS * sizeof(float) + (size_t)NKV * TOT_BYTES + 256;
}

int launch_forward_bf16(const Fwd& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int64_t NKV = a.B * a.Hkv, NQ = a.B * a.Hq;
  const int64_t nchunks = (a.n + FC - 1) / FC, nseg = forward_bf16_nseg(a.n);
  float* part = reinterpret_cast<float*>(a.ws);
  uint8_t* tot = reinterpret_cast<uint8_t*>(part + NKV * nseg * PART_FLOATS);
  FwdArgs A{reinterpret_cast<const bf16*>(a.q), reinterpret_cast<const bf16*>(a.k),
            reinterpret_cast<const bf16*>(a.v), reinterpret_cast<bf16*>(a.out), a.n, nchunks, nseg, NKV, NQ,
            a.Hq / a.Hkv, part, tot};
  k_fwd_state<<<dim3((unsigned)(NKV * nseg)), WNT, 0, st>>>(A);
  k_fwd_reduce<<<dim3((unsigned)(NKV * RED_BLOCKS)), RED_THREADS, 0, st>>>(A);
  k_fwd_out<<<dim3((unsigned)(NQ * nseg)), WNT, 0, st>>>(A);
  return (int)hipGetLastError();
}

}  // namespace la_internal
