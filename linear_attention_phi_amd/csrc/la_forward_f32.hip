// la_forward_f32.hip -- non-causal pass for fp32 inputs with d = 64 (gfx950).
//
// out_i = phi(Q_i) S / (phi(Q_i) . z) with S = sum_j phi(K_j) (x) V_j and
// z = sum_j phi(K_j) over all n keys of the query's key/value head
// (nx_f32_linear_attention.nx source, header comment: S and z over all
// keys, then each query's normalised read; LinearTile 1.0.1, "How It Works": K^T V once, then Q).
//
// The products run on v_mfma_f32_16x16x4_f32, whose operands put the
// contraction index k on lane / 16 and the other index on lane % 16.  A
// lane that loads 16 bytes of a token-major row holds four consecutive
// features of one token, so:
//   - for S (a contraction over tokens) a wave instruction loads four whole
//     rows (1 KiB) and each of the four loaded features feeds its own MFMA:
//     component j of lane (m, kq) is the operand for feature 4 m + j of token
//     kq; the sixteen (j, j') pairs of K and V components give the 16 x 16
//     tiles of S[4 i + j][4 n + j'];
//   - for the output (a contraction over features) the product is taken
//     transposed, out^T = S^T phi(Q)^T, so that the accumulator of a lane
//     holds four consecutive output features of one query (16 bytes).  Its
//     operands and results run along the rows in 64-byte pieces, so Q rows
//     come in and output rows go out whole (1 KiB per wave instruction)
//     through a small LDS tile per wave, which measured about 2 us faster
//     at B2 H8 n4096 than the 64-byte pieces straight from and to HBM.
// Three launches:
//
//  k_fwd32_state   eight waves per 256 keys of a key/value head, 32 keys per
//                  wave: phi(K)^T V and z, the eight wave results summed in
//                  LDS in wave order into one partial per workgroup;
//  k_fwd32_reduce  sums each head's partials in segment order (the result
//                  does not depend on timing) and writes S in the output
//                  kernel's operand order, then z;
//  k_fwd32_out     eight waves per 256 queries, 32 queries per wave: Q rows
//                  through LDS into operand order, out^T on MFMA, phi(Q) . z
//                  on the VALU, division, output rows through LDS and out
//                  with non-temporal stores.
//
// phi(K) = relu(K) + 1 is formed in fp32; padded keys (past n) read as zero,
// so their phi(K) = 1 meets V = 0 in S, and z counts only the n real keys.
// With ELU + 1 (template ELU) phi(K) of a padded key is set to 0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_bf16.h"
#include "la_internal.h"

namespace {

using la_bf16::CPOL_NT;
using la_bf16::u32x4;
typedef la_bf16::f32x4v f32x4;

constexpr int FD = 64;                 // head dim
constexpr int TW = 32;                 // keys (state) or queries (output) per wave
constexpr int NW = 8;                  // waves per workgroup
constexpr int WNT = 64 * NW;           // threads per workgroup
constexpr int SEG = TW * NW;           // keys or queries per workgroup
constexpr int PART_F = FD * FD + FD;   // one partial or total: S (4096 floats), then z (64)
constexpr int RED_THREADS = 256;
constexpr int RED_BLOCKS = (PART_F / 4 + RED_THREADS - 1) / RED_THREADS;  // blocks per head
constexpr int RQ = FD + 4;             // row stride (floats) of the output kernel's LDS tiles

static_assert(SEG == la_internal::kFwd32SegTokens, "segment length");

struct Fwd32Args {
  const float* q; const float* k; const float* v; float* out;
  int64_t n, nseg, NKV, NQ, R;
  float* part;  // [NKV][nseg][PART_F]: S in accumulator order, then z
  float* tot;   // [NKV][PART_F]: S in operand order, then z
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 ld4(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)byte_off, 0, 0));
}

// Accumulator order: entry (blk = 4 j + j', lane l) holds, in its four
// floats rr = 0..3, S[16 (l / 16) + 4 rr + j][4 (l % 16) + j'].
struct St32Lds {
  f32x4 acc[NW][16][64];  // each wave's 64 x 64 result
  f32x4 z[NW][16];        // each wave's z[4 m .. 4 m + 3]
};

// ELU selects phi = ELU + 1 (alpha = 1: x + 1 for x > 0, e^x otherwise)
// instead of relu + 1; keys past the end then count as 0, not phi(0) = 1.
__device__ __forceinline__ float elu1(float x) { return x > 0.0f ? x + 1.0f : expf(x); }

template <bool ELU>
__global__ __launch_bounds__(WNT) void k_fwd32_state(Fwd32Args A) {
  __shared__ St32Lds L;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, kq = lane >> 4;
  const int64_t seg = blockIdx.x / A.NKV, head = blockIdx.x % A.NKV;
  const uint32_t hbytes = (uint32_t)(A.n * FD * 4);  // one head's rows (n <= kFwd32MaxN)
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.k + head * A.n * FD), 0, (int)hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.v + head * A.n * FD), 0, (int)hbytes, 0x00020000);
  const int64_t t0 = seg * SEG + w * TW;  // this wave's first key
  const int nv = (int)(A.n - t0 < 0 ? 0 : (A.n - t0 < TW ? A.n - t0 : TW));

  // step s: keys t0 + 4 s + kq, features 4 m .. 4 m + 3 (past n: zero).
  // All loads are issued before the arithmetic, step by step and kept in
  // that order (the scheduling barriers), so that with loads returning in
  // order step s waits only for its own K and V: the MFMAs of the early
  // steps run while the later rows are still arriving.
  f32x4 kr[TW / 4], vr[TW / 4];
#pragma unroll
  for (int s = 0; s < TW / 4; ++s) {
    kr[s] = ld4(rk, (uint32_t)((t0 + 4 * s + kq) * FD + 4 * m) * 4u);
    vr[s] = ld4(rv, (uint32_t)((t0 + 4 * s + kq) * FD + 4 * m) * 4u);
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) acc[j][jp] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 zr = f32x4{0.0f, 0.0f, 0.0f, 0.0f};  // sum of relu(K) (ELU: of phi(K)) over this lane's keys
#pragma unroll
  for (int s = 0; s < TW / 4; ++s) {
    f32x4 pk;
    const bool real = 4 * s + kq < nv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (ELU) {
        pk[j] = real ? elu1(kr[s][j]) : 0.0f;
        zr[j] += pk[j];
      } else {
        const float x = fmaxf(kr[s][j], 0.0f);
        zr[j] += x;
        pk[j] = x + 1.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) acc[j][jp] = mfma4(pk[j], vr[s][jp], acc[j][jp]);
    __builtin_amdgcn_sched_barrier(0);  // step by step, as the loads arrive
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    zr[j] += __shfl_xor(zr[j], 16);
    zr[j] += __shfl_xor(zr[j], 32);
    if (!ELU) zr[j] += (float)nv;  // the ones of phi(K) = relu(K) + 1, real keys only
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) L.acc[w][4 * j + jp][lane] = acc[j][jp];
  if (kq == 0) L.z[w][m] = zr;
  __syncthreads();

  // the workgroup's partial: the waves' results summed in wave order;
  // non-temporal, since only the next launch reads it
  float* dst = A.part + (head * A.nseg + seg) * PART_F;
  const f32x4* la = &L.acc[0][0][0];
  for (int e = tid; e < 16 * 64; e += WNT) {
    f32x4 s = la[e];
#pragma unroll
    for (int u = 1; u < NW; ++u) s += la[u * 16 * 64 + e];
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(dst) + e);
  }
  if (tid < 16) {
    f32x4 s = L.z[0][tid];
#pragma unroll
    for (int u = 1; u < NW; ++u) s += L.z[u][tid];
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(dst + FD * FD) + tid);
  }
}

// Thread t of a head's RED_BLOCKS * RED_THREADS sums float4 t of the
// partials.  Operand order of the total: entry (bb, tt, lane L) holds, in
// its four floats jj = 0..3, S[16 tt + 4 (L / 16) + jj][16 bb + L % 16] (the
// A operand of out^T for output features 16 bb .., features 16 tt ..).
__global__ __launch_bounds__(RED_THREADS) void k_fwd32_reduce(Fwd32Args A) {
  const int64_t head = blockIdx.x / RED_BLOCKS;
  const int t = (int)(blockIdx.x % RED_BLOCKS) * RED_THREADS + threadIdx.x;
  if (t >= PART_F / 4) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(A.part + head * A.nseg * PART_F) + t;
  constexpr int STRIDE = PART_F / 4;
  // sixteen segments' loads in flight, summed in segment order
  f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int64_t p = 0;
  for (; p + 16 <= A.nseg; p += 16) {
    f32x4 x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = src[(p + u) * STRIDE];
#pragma unroll
    for (int u = 0; u < 16; ++u) s += x[u];
  }
  for (; p < A.nseg; ++p) s += src[p * STRIDE];
  float* tot = A.tot + head * PART_F;
  if (t < 16 * 64) {
    // accumulator entry (4 j + j', l): S[16 kq + 4 rr + j][4 m + j'] ->
    // operand entry (bb = m / 4, tt = kq, L = 16 rr + 4 (m % 4) + j'), float j
    const int blk = t >> 6, l = t & 63, j = blk >> 2, jp = blk & 3, mm = l & 15, kk = l >> 4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      tot[(((mm >> 2) * 4 + kk) * 64 + 16 * rr + 4 * (mm & 3) + jp) * 4 + j] = s[rr];
  } else {
    *reinterpret_cast<f32x4*>(tot + FD * FD + 4 * (t - 16 * 64)) = s;
  }
}

template <bool ELU>
__global__ __launch_bounds__(WNT) void k_fwd32_out(Fwd32Args A) {
  __shared__ __attribute__((aligned(16))) float tiles[NW][TW * RQ];  // each wave's Q rows, then its output rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, kq = lane >> 4;
  const int64_t seg = blockIdx.x / A.NQ, qh = blockIdx.x % A.NQ, kvh = qh / A.R;
  const int64_t q0 = seg * SEG + w * TW;  // this wave's first query
  if (q0 >= A.n) return;                  // no barrier in this kernel
  const uint32_t hbytes = (uint32_t)(A.n * FD * 4);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(A.q + qh * A.n * FD), 0, (int)hbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(A.out + qh * A.n * FD, 0, (int)hbytes, 0x00020000);
  const float* tot = A.tot + kvh * PART_F;

  // S and z (read from L2 by every wave of the head), then the wave's Q rows
  // whole: load u covers rows q0 + 4 u .. + 3 (past n: zero, and those rows
  // are never stored)
  f32x4 so[4][4], zo[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) so[bb][tt] = reinterpret_cast<const f32x4*>(tot)[(bb * 4 + tt) * 64 + lane];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) zo[tt] = *reinterpret_cast<const f32x4*>(tot + FD * FD + 16 * tt + 4 * kq);
  const int prow = lane >> 4, pcol = 4 * (lane & 15);
  f32x4 qraw[TW / 4];
#pragma unroll
  for (int u = 0; u < TW / 4; ++u) qraw[u] = ld4(rq, (uint32_t)((q0 + 4 * u + prow) * FD + pcol) * 4u);

  // Q rows into the wave's tile, then the B operands: component jj of
  // (query block qb, feature block tt) is phi(Q)[q0 + 16 qb + m][16 tt + 4 kq + jj]
  float* tile = tiles[w];
#pragma unroll
  for (int u = 0; u < TW / 4; ++u) *reinterpret_cast<f32x4*>(tile + (4 * u + prow) * RQ + pcol) = qraw[u];
  la_bf16::wave_lds_sync();
  f32x4 qr[TW / 16][4];
#pragma unroll
  for (int qb = 0; qb < TW / 16; ++qb)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) qr[qb][tt] = *reinterpret_cast<const f32x4*>(tile + (16 * qb + m) * RQ + 16 * tt + 4 * kq);
  la_bf16::wave_lds_sync();  // every lane's reads are done before the tile is rewritten

#pragma unroll
  for (int qb = 0; qb < TW / 16; ++qb) {
    float den = 0.0f;
    f32x4 o[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) o[bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float x = ELU ? elu1(qr[qb][tt][jj]) : fmaxf(qr[qb][tt][jj], 0.0f) + 1.0f;
        den = fmaf(x, zo[tt][jj], den);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) o[bb] = mfma4(so[bb][tt][jj], x, o[bb]);
      }
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    const float inv = 1.0f / den;
    // lane (m, kq): output features 16 bb + 4 kq .. + 3 of query 16 qb + m
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) *reinterpret_cast<f32x4*>(tile + (16 * qb + m) * RQ + 16 * bb + 4 * kq) = o[bb] * inv;
    la_bf16::wave_lds_sync();
    // the block's 16 rows out whole, non-temporal; rows past n fall outside
    // the resource
#pragma unroll
    for (int u = 4 * qb; u < 4 * qb + 4; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(tile + (4 * u + prow) * RQ + pcol), ro,
                                             (int)((uint32_t)((q0 + 4 * u + prow) * FD + pcol) * 4u), 0, CPOL_NT);
  }
}

}  // namespace

namespace la_internal {

bool forward_f32_applies(int64_t n, int64_t d, int dtype) { return dtype == 0 && d == FD && n <= kFwd32MaxN; }

int64_t forward_f32_nseg(int64_t n) { return (n + SEG - 1) / SEG; }

size_t forward_f32_ws_bytes(int64_t NKV, int64_t nseg) {
  return (size_t)NKV * (nseg + 1) * PART_F * sizeof(float) + 256;
}

int launch_forward_f32(const Fwd& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const int64_t NKV = a.B * a.Hkv, NQ = a.B * a.Hq, nseg = forward_f32_nseg(a.n);
  float* part = reinterpret_cast<float*>(a.ws);
  float* tot = part + NKV * nseg * PART_F;
  Fwd32Args A{reinterpret_cast<const float*>(a.q), reinterpret_cast<const float*>(a.k),
              reinterpret_cast<const float*>(a.v), reinterpret_cast<float*>(a.out), a.n, nseg, NKV, NQ,
              a.Hq / a.Hkv, part, tot};
  const bool elu = a.phi == 1;
  if (elu)
    k_fwd32_state<true><<<dim3((unsigned)(NKV * nseg)), WNT, 0, st>>>(A);
  else
    k_fwd32_state<false><<<dim3((unsigned)(NKV * nseg)), WNT, 0, st>>>(A);
  k_fwd32_reduce<<<dim3((unsigned)(NKV * RED_BLOCKS)), RED_THREADS, 0, st>>>(A);
  if (elu)
    k_fwd32_out<true><<<dim3((unsigned)(NQ * nseg)), WNT, 0, st>>>(A);
  else
    k_fwd32_out<false><<<dim3((unsigned)(NQ * nseg)), WNT, 0, st>>>(A);
  return (int)hipGetLastError();
}

}  // namespace la_internal
