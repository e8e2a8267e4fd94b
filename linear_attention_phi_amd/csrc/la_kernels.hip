// la_kernels.hip -- gfx950 (MI355X) kernels for kernelized linear attention.
//
// Method (nx_f32_linear_attention.nx source, header comment: the feature
// map, the key/value summary and the normalised read): with
// phi(x) = relu(x) + 1,  S = sum_j phi(K_j) (x) V_j,  z = sum_j phi(K_j),
// out_i = phi(Q_i) S / (phi(Q_i) . z).  The causal and prefix-mask forms
// (trim-transformer 0.1.0, "Masking") restrict query i to keys 0..m_i.
//
// Work decomposition (per batch x key/value head, "bh"):
//   tokens are cut into chunks of C rows; G consecutive chunks form a segment,
//   and one 256-thread workgroup owns one segment of one head.
//   k_state : per segment, Delta S = sum_c phi(K_c)^T V_c and Delta z on MFMA
//             -> fp32 segment aggregate in the workspace.
//   k_scan  : per head, exclusive prefix over the segment aggregates (fixed
//             sequential order, so results are bit-reproducible), plus the
//             total (non-causal S, and the causal final state).
//   k_out   : per segment, walks its chunks in order carrying S in MFMA
//             accumulators: out_c = phi(Q_c) S_prev + tril(phi(Q_c) phi(K_c)^T) V_c,
//             den_c likewise, division fused in the epilogue; then
//             S += phi(K_c)^T V_c.  The prefix form gathers the queries whose
//             mask ends inside chunk c (a counting sort by floor(m_i / C)).
//   k_out_nc: non-causal output: phi(Q) S_total / (phi(Q) . z_total).
//   k_decode: one recurrent step, S += phi(k) (x) v, then out per query head.
//
// MFMA operand / accumulator conventions: see la_device.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "la_bf16.h"
#include "la_ctl.h"
#include "la_device.h"
#include "la_internal.h"

namespace {

using namespace la_dev;

// Copy the first nrows rows of a tile held in LDS (row stride LQ elements) to
// global rows of d elements: tile row r goes to row gidx[r] when gidx is
// given, else to row row0 + r.  With d == DP (vec) every lane moves four
// elements at once, so a wave writes whole rows.
template <typename T, int DP, int LQ>
__device__ __forceinline__ void copy_rows_out(const T* tile, int nrows, int d, bool vec, T* base,
                                              const int* gidx, int64_t row0, int tid) {
  // non-temporal stores: the output is not read again here, and dirty L2
  // lines would otherwise be written back when the kernel ends
  if (vec) {
    constexpr int PPR = DP / 4;
    typedef uint32_t U __attribute__((ext_vector_type(sizeof(T))));  // 4 elements
    for (int idx = tid; idx < nrows * PPR; idx += NT) {
      const int r = idx / PPR, col = 4 * (idx % PPR);
      const int64_t g = gidx ? (int64_t)gidx[r] : row0 + r;
      __builtin_nontemporal_store(*reinterpret_cast<const U*>(tile + r * LQ + col), reinterpret_cast<U*>(base + g * d + col));
    }
  } else {
    for (int idx = tid; idx < nrows * d; idx += NT) {
      const int r = idx / d, col = idx % d;
      const int64_t g = gidx ? (int64_t)gidx[r] : row0 + r;
      __builtin_nontemporal_store(tile[r * LQ + col], base + g * d + col);
    }
  }
}


// ------------------------------------------------------------------ k_state
// PM is the feature map of K.  With relu + 1 the state is built as
// phi(K)^T V = relu(K)^T V + 1 (x) sum_t V_t and z = sum_t relu(K_t) +
// (number of keys): relu of an input value is exact in the input type, so
// the MFMA products are exact and the state is exact up to fp32 summation
// (rounding phi(K) to bf16 would not be).  ELU + 1 has no such split: the
// tile holds phi(K) in the input type.  The identity (prefix form) builds
// K^T V and no z.
template <typename T, int DP, int C, int PM>
__global__ __launch_bounds__(NT) void k_state(const T* __restrict__ k, const T* __restrict__ v, int64_t n, int d,
                                              bool vec, int64_t nchunks, int64_t G, int64_t nseg,
                                              float* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) T sKT[DP * (C + PAD)];
  __shared__ __attribute__((aligned(16))) T sVT[DP * (C + PAD)];
  __shared__ float svs[DP];
  using SB = StateBlocks<DP>;
  constexpr int KX = k_xform<PM>();
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const T* kb = k + bh * n * d;
  const T* vb = v + bh * n * d;
  f32x16 accS[SB::PER_WAVE];
#pragma unroll
  for (int s = 0; s < SB::PER_WAVE; ++s) accS[s] = f32x16{};
  float zrun = 0.0f, vrun = 0.0f;
  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;
  // with d == DP the next chunk's K and V tiles load while this one is used
  TileRaw<T, DP, C> rK, rV;
  auto fetch = [&](int64_t c) {
    const int64_t tc = c * C;
    const int nvc = (int)((n - tc) < C ? (n - tc) : C);
    tile_fetch<T, DP, C>(rK, kb, tc, nullptr, nvc, tid);
    tile_fetch<T, DP, C>(rV, vb, tc, nullptr, nvc, tid);
  };
  if (vec && c0 < c1) fetch(c0);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)((n - t0) < C ? (n - t0) : C);
    if (vec) {
      tile_store<T, DP, C, XF_NONE, KX>(rK, nv, nullptr, sKT, tid);
      tile_store<T, DP, C, XF_NONE, XF_ID>(rV, nv, nullptr, sVT, tid);
      if (c + 1 < c1) fetch(c + 1);
    } else {
      load_tile<T, DP, C, XF_NONE, KX>(kb, t0, nullptr, nv, d, vec, nullptr, sKT, tid);
      load_tile<T, DP, C, XF_NONE, XF_ID>(vb, t0, nullptr, nv, d, vec, nullptr, sVT, tid);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        gemm_acc<T, C / 16>(accS[s], sKT + ma * 32 * (C + PAD), C + PAD, sVT + nb * 32 * (C + PAD), C + PAD, lane);
      }
    }
    if (PM != PM_ID && tid < DP) {
      zrun += row_sum<T, C>(sKT, tid) + (PM == PM_RELU1 && tid < d ? (float)nv : 0.0f);
      if (PM == PM_RELU1) vrun += row_sum<T, C>(sVT, tid);
    }
    __syncthreads();
  }
  if (PM == PM_RELU1) {
    if (tid < DP) svs[tid] = vrun;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) add_col(accS[s], svs[(e % SB::NB) * 32 + (lane & 31)], e / SB::NB, d, lane);
    }
  }
  float* dst = ws + (bh * (nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
  for (int s = 0; s < SB::PER_WAVE; ++s) {
    const int e = w + NW * s;
    if (e < SB::TOTAL) st_state_block<DP>(dst, accS[s], e / SB::NB, e % SB::NB, lane);
  }
  if (tid < DP) dst[DP * DP + tid] = zrun;
}

// --------------------------------------------------------------- k_state_tr
// k_state for bf16 with d = 128 and chunk 32 (the causal shape with four or
// two query heads per key/value head): the K and V tiles stay token-major in
// LDS (16-byte writes, two buffers, one barrier per chunk), and the operands
// over the token index come from transposed reads (ds_read_b64_tr_b16), so
// no feature-major copies are written.  Wave w owns state column block w
// (all four row blocks): the column sums of V its blocks need and z of rows
// 32 w .. are dot2 sums over fragments it reads anyway.
// Tile row stride (bf16): 80 dwords, so that the four rows and two 16-column
// halves a half-wave of ds_read_b64_tr_b16 touches fall in eight distinct
// 8-bank groups (rows 16 banks apart).  At 72 dwords (rows 8 banks apart) a
// row's second half shares banks with the next row's first: an LDS probe
// of the read measured 4.0 cycles per instruction against 2.0.
constexpr int STR_RS = 128 + 32;
// PM: relu + 1 (relu(K) in the tiles, the ones part added at the end) or
// ELU + 1 (phi(K) in the tiles, rows past the end 0).
template <int PM>
__global__ __launch_bounds__(NT) void k_state_tr(const bf16* __restrict__ k, const bf16* __restrict__ v, int64_t n,
                                                 int64_t nchunks, int64_t G, int64_t nseg, float* __restrict__ ws) {
  constexpr int DP = 128, C = 32, RS = STR_RS;
  constexpr bool SPLIT = PM == PM_RELU1;
  static_assert(NT == 256 && DP / 32 == NT / 64, "one column block per wave");
  __shared__ __attribute__((aligned(16))) bf16 sK[2][C * RS];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][C * RS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 31, h = lane >> 5;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const bf16* kb = k + bh * n * DP;
  const bf16* vb = v + bh * n * DP;
  f32x16 acc[DP / 32];  // row blocks ab of column block w
#pragma unroll
  for (int ab = 0; ab < DP / 32; ++ab) acc[ab] = f32x16{};
  float zrun = 0.0f, vrun = 0.0f;  // z[32 w + r] and sum_t V[t][32 w + r] (both halves)
  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;
  // piece u of a tile: row (tid + NT u) / 16, eight features from 8 ((tid + NT u) % 16)
  constexpr int PIECES = C * DP / 8 / NT;
  uint4 kr[PIECES], vr[PIECES];
  auto fetch = [&](int64_t c) {
    const int64_t t0 = c * C;
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pc = tid + NT * u, row = pc >> 4, col = 8 * (pc & 15);
      const bool ok = t0 + row < n;
      kr[u] = ok ? *reinterpret_cast<const uint4*>(kb + (t0 + row) * DP + col) : make_uint4(0, 0, 0, 0);
      vr[u] = ok ? *reinterpret_cast<const uint4*>(vb + (t0 + row) * DP + col) : make_uint4(0, 0, 0, 0);
    }
  };
  if (c0 < c1) fetch(c0);
  int buf = 0;
  for (int64_t c = c0; c < c1; ++c, buf ^= 1) {
    const int nv = (int)((n - c * C) < C ? (n - c * C) : C);
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
      const int pc = tid + NT * u, row = pc >> 4, col = 8 * (pc & 15);
      const uint4 x = kr[u];
      auto fk = [&](uint32_t y) { return SPLIT ? la_bf16::relu2(y) : (row < nv ? la_bf16::map2<PM>(y) : 0u); };
      *reinterpret_cast<uint4*>(sK[buf] + row * RS + col) = make_uint4(fk(x.x), fk(x.y), fk(x.z), fk(x.w));
      *reinterpret_cast<uint4*>(sV[buf] + row * RS + col) = vr[u];
    }
    if (c + 1 < c1) fetch(c + 1);
    // the other buffer was last read before this barrier's predecessor, so
    // one barrier per chunk suffices
    __syncthreads();
    Frag<bf16> vt[C / 16], kz[C / 16];
#pragma unroll
    for (int kt = 0; kt < C / 16; ++kt) {
      vt[kt] = la_bf16::ld_tr<RS>(sV[buf], 16 * kt, 32 * w, lane);
      kz[kt] = la_bf16::ld_tr<RS>(sK[buf], 16 * kt, 32 * w, lane);
    }
#pragma unroll
    for (int ab = 0; ab < DP / 32; ++ab)
#pragma unroll
      for (int kt = 0; kt < C / 16; ++kt) mma(acc[ab], la_bf16::ld_tr<RS>(sK[buf], 16 * kt, 32 * ab, lane), vt[kt]);
    float zs = 0.0f, vs = 0.0f;
#pragma unroll
    for (int kt = 0; kt < C / 16; ++kt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        zs = la_bf16::dot2(la_bf16::pair(kz[kt], q), la_bf16::ONE2, zs);
        vs = la_bf16::dot2(la_bf16::pair(vt[kt], q), la_bf16::ONE2, vs);
      }
    zrun += zs + __shfl_xor(zs, 32) + (SPLIT ? (float)nv : 0.0f);  // relu + 1: the ones over the nv keys
    vrun += vs + __shfl_xor(vs, 32);
  }
  // relu + 1: phi(K)^T V = relu(K)^T V + 1 (x) sum_t V_t
  if (SPLIT) {
#pragma unroll
    for (int ab = 0; ab < DP / 32; ++ab) add_col(acc[ab], vrun, ab, DP, lane);
  }
  float* dst = ws + (bh * (nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
  for (int ab = 0; ab < DP / 32; ++ab) st_state_block<DP>(dst, acc[ab], ab, w, lane);
  if (h == 0) dst[DP * DP + 32 * w + r] = zrun;
}

// ------------------------------------------------------------------- k_scan
// One thread per state element of one head: exclusive prefix over segments
// in place, total into slot nseg, and the caller's final state if asked.
// Only the prefixes of segments s with s % F == 0 are stored (the output
// launch that follows starts a workgroup at every F-th segment); the total
// always is.
// V consecutive state elements per thread (V = 1 or 4; with 4, 16-byte loads
// and stores: a quarter of the threads and instructions; the slot size
// DP (DP + 1) is a multiple of four and the workspace and its slots are
// 16-byte aligned).  Each element is summed in segment order either way.
template <int V>
__global__ __launch_bounds__(NT) void k_scan(float* __restrict__ ws, int64_t nseg, int DP, int d,
                                             float* __restrict__ S_final, float* __restrict__ z_final, int64_t F) {
  using vec = typename std::conditional<V == 4, f32x4, float>::type;
  const int64_t E = slot_elems(DP), EV = E / V;
  const int64_t bh = blockIdx.x;
  const int64_t ev = (int64_t)blockIdx.y * NT + threadIdx.x;
  if (ev >= EV) return;
  vec* base = reinterpret_cast<vec*>(ws + bh * (nseg + 1) * E) + ev;
  vec run = vec{};
  // segments in blocks of 16: all loads of a block are issued before its
  // stores (which the compiler could not move past them), in a fixed order
  constexpr int BLK = 16;
  for (int64_t s0 = 0; s0 < nseg; s0 += BLK) {
    vec x[BLK];
#pragma unroll
    for (int u = 0; u < BLK; ++u) x[u] = (s0 + u < nseg) ? base[(s0 + u) * EV] : vec{};
#pragma unroll
    for (int u = 0; u < BLK; ++u) {
      if (s0 + u < nseg) {
        if ((s0 + u) % F == 0) base[(s0 + u) * EV] = run;
        run += x[u];
      }
    }
  }
  base[nseg * EV] = run;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t e = V * ev + j;
    float r;
    if constexpr (V == 4) r = run[j];
    else r = run;
    if (e < (int64_t)DP * DP) {
      const int a = (int)(e / DP), b = (int)(e % DP);
      if (S_final && a < d && b < d) S_final[bh * d * d + (int64_t)a * d + b] = r;
    } else {
      const int a = (int)(e - (int64_t)DP * DP);
      if (z_final && a < d) z_final[bh * d + a] = r;
    }
  }
}

// k_scan over nunits units: four elements per thread when that still gives
// at least 64K threads (four waves per CU); with fewer units one element per
// thread, whose four times as many waves cover the serial chain's round trips
// (d128 B8 H8 n2048: 77.0 -> 68.6 us per call with four; the long-context GQA
// shape, eight units, and the fp32 prefix form, 32, measured slower with four)
void launch_k_scan(float* ws, int64_t nunits, int64_t nseg, int DP, int d, float* S_final, float* z_final,
                   int64_t F, hipStream_t st) {
  const int64_t E = slot_elems(DP);
  if (nunits * (E / 4) >= 65536) {
    k_scan<4><<<dim3((unsigned)nunits, (unsigned)((E / 4 + NT - 1) / NT)), NT, 0, st>>>(ws, nseg, DP, d, S_final,
                                                                                       z_final, F);
  } else {
    k_scan<1><<<dim3((unsigned)nunits, (unsigned)((E + NT - 1) / NT)), NT, 0, st>>>(ws, nseg, DP, d, S_final, z_final,
                                                                                   F);
  }
}

// ----------------------------------------------------------- k_out_prefix32
// Prefix form for fp32 with d = 64 and chunk 64 on v_mfma_f32_16x16x4_f32,
// with no LDS transposes:
//   out^T(bucket c) = S_prev(c)^T Q^T + V_c^T P^T,   P^T = mask(K_c Q^T),
// where S_prev(c) is the state before chunk c (the segment's exclusive prefix
// plus the segment's earlier chunks) and the mask keeps key j for query i iff
// j <= m_i.  The queries of bucket c go in groups of 16 NWV, one 16-query
// block per wave (in a group of fewer blocks than waves the waves share each
// block instead: one key block's scores and one block of output features
// each), their rows gathered through perm and staged in LDS.  Operands
// (the contraction index k is lane / 16, the other index lane % 16):
//   S^T  from LDS in operand order: entry (bb, tt, lane) is the float4 over
//        jj of S[16 tt + 4 (lane / 16) + jj][16 bb + lane % 16], kept in
//        slot lane ^ (4 bb + tt) of block 4 bb + tt (one 16-byte read per
//        lane, 1 KB per wave, no bank conflicts);
//   Q^T  the float4 of query row lane % 16 at features 16 tt + 4 (lane / 16);
//   K    the float4 of key row 16 kb + lane % 16 at the same features;
//   P^T  the score accumulator itself: its register rr holds key
//        16 kb + 4 (lane / 16) + rr of query lane % 16, which is the B operand
//        of the k-step over keys {16 kb + 4 k + rr};
//   V^T  for that k-step, V[16 kb + 4 (lane / 16) + rr][16 bb + lane % 16],
//        one float per lane from the V tile.
// A lane's output accumulator holds features 16 bb + 4 (lane / 16) .. + 3 of
// query lane % 16.  The last four waves keep the state: the w-th of them
// holds the blocks (tt, bb) = (w, 0..3) with entry rr of lane l =
// S[16 w + 4 (l / 16) + rr][16 bb + l % 16] -- exactly the readers' float4 of
// block (bb, tt), so it goes to LDS with one 16-byte store per block at the
// chunk's start -- and adds K_c^T V_c during the chunk's first query group
// (A = K^T with rows a, B = V with columns b, one float of each per lane and
// k-step, key 16 (st / 4) + 4 (l / 16) + st % 4 at step st).
// The state's operand-order stores are whole float4s (with the state held
// the other way round they were 16 scalar stores per wave and chunk, 8-way
// bank-conflicted on gfx950: 147.7 / 177.1 against 150.0 / 178.2 us per call
// at B4 H8 n8192, m = arange / uniform); the state update's scalar reads
// (rows four apart) and the V reads are conflict-free at the 68-float row
// stride.  (A 72-float stride for the K and Q tiles, whose 16-byte operand
// reads it makes conflict-free, measured no faster: 150.4 / 177.5 us.)
// With CS (the causal normalised form, feature map PM) the buckets are the
// chunks themselves (query i of chunk c = row c C + i, m_i = i, no sort), Q
// rows and K tiles take phi as they are staged (key rows past n stay 0), and
// z rides along with S: wave 0 keeps z_prev(c) (from the prefix slot, plus
// the column sums of the segment's earlier phi(K) tiles) and publishes it in
// LDS beside S; the denominator phi(Q_i) . z_prev + the masked score row sum
// divides each output row.
constexpr int PX_RS = 64 + 4;  // row stride (floats) of the LDS tiles
// NWV waves per workgroup, queries per group QG = 16 NWV (one 16-query block
// per wave); the state is owned by waves NWV - 4 .. NWV - 1, four tiles each.
// Four waves (69.4 KB of LDS, 77.3 KB with the prefix form's shared score
// buffers, so that two workgroups share a CU and cover each other's
// barriers) measured 146.9 / 179.3 us at B4 H8 n8192 (m = arange
// / uniform) against 162.7 / 190.9 us for eight.
constexpr int PX_NWV = 4;
// Workgroups of the GQA output launch (one per CU): each walks the chunks of
// several state segments.
#ifndef LA_GQA_OUT_GROUPS
#define LA_GQA_OUT_GROUPS 256
#endif
constexpr int64_t kGqaOutGroups = LA_GQA_OUT_GROUPS;
// Workgroups of the fp32 prefix-form output launch (two per CU).
#ifndef LA_PREFIX_OUT_GROUPS
#define LA_PREFIX_OUT_GROUPS 512
#endif
constexpr int64_t kPrefixOutGroups = LA_PREFIX_OUT_GROUPS;
template <int NWV, bool CS = false, int PM = PM_ID>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2))) void k_out_prefix32(const float* __restrict__ q, const float* __restrict__ k,
                                                      const float* __restrict__ v, float* __restrict__ out, int64_t n,
                                                      int64_t nchunks, int64_t G, int64_t nseg, int64_t F,
                                                      int64_t nseg_ws, const float* __restrict__ ws,
                                                      const int* __restrict__ perm,
                                                      const int* __restrict__ boff, const int64_t* __restrict__ m,
                                                      int64_t H, int64_t nmask) {
  constexpr int FD = 64, C = 64, QG = 16 * NWV, NT_ = 64 * NWV;
  constexpr int KVP = C * FD / 4 / NT_;  // 16-byte pieces of a K or V tile per thread
  static_assert(NWV == 4 || NWV == 8, "four or eight waves");
  constexpr int RK = PX_RS, RV = PX_RS;
  __shared__ __attribute__((aligned(16))) float sK[C * RK];
  __shared__ __attribute__((aligned(16))) float sV[C * RV];
  __shared__ __attribute__((aligned(16))) float sQ[QG * RK];
  __shared__ __attribute__((aligned(16))) float sS[16 * 64 * 4];  // S in operand order
  __shared__ __attribute__((aligned(16))) float sz[FD];            // z_prev (CS)
  __shared__ int sI[QG];  // the group's query rows
  __shared__ int sM[QG];  // and their mask values, clamped into [0, n - 1]
  __shared__ __attribute__((aligned(16))) float sP[2 * 4 * 64 * 4];  // shared score blocks (partial groups)
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, mm = lane & 15, kq = lane >> 4;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  if constexpr (!CS) {  // this batch's mask, buckets and permutation (one per batch, or one shared)
    const int64_t mb = nmask > 1 ? bh / H : 0;
    perm += mb * n;
    boff += mb * (nchunks + 1);
    m += mb * n;
  }
  // bucket c's first position, and the query row at a position
  // (boff is read through the constant address space: the same value for
  // every lane, so it comes in by scalar loads, which wait on a counter of
  // their own instead of on every vector load and store in flight)
  auto bo = [&](int64_t c) -> int64_t {
    if constexpr (CS) return c * C < n ? c * C : n;
    else return ((const __attribute__((address_space(4))) int*)boff)[c];
  };
  auto qrow = [&](int64_t i) -> int64_t {
    if constexpr (CS) return i;
    else return perm[i];
  };
  auto phi4 = [&](f32x4 x) -> f32x4 {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = phi_m<PM>(x[j]);
    return x;
  };
  const float* qh = q + bh * n * FD;
  const float* kh = k + bh * n * FD;
  const float* vh = v + bh * n * FD;
  float* oh = out + bh * n * FD;

  // the last four waves: state blocks (tt, bb) = (sj, 0..3), from the
  // segment's exclusive prefix (row-major)
  const bool owner = w >= NWV - 4;
  const int sj = w & 3;
  f32x4 accS[4];
  {
    const float* src = ws + (bh * (nseg_ws + 1) + F * seg) * slot_elems(FD);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) accS[bb][rr] = owner ? src[(16 * sj + 4 * kq + rr) * FD + 16 * bb + mm] : 0.0f;
  }
  float zacc = 0.0f;  // CS: z_prev of feature tid (wave 0)
  if (CS && tid < FD) zacc = ws[(bh * (nseg_ws + 1) + F * seg) * slot_elems(FD) + FD * FD + tid];
  auto state_update = [&]() {  // S += K_c^T V_c on this wave's blocks
#pragma unroll
    for (int st = 0; st < C / 4; ++st) {
      const int key = 16 * (st >> 2) + 4 * kq + (st & 3);
      const float ka = sK[key * RK + 16 * sj + mm];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        accS[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, sV[key * RV + 16 * bb + mm], accS[bb], 0, 0, 0);
    }
  };
  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;

  // next chunk's K and V rows (piece u: row (tid + NT_ u) / 16, features
  // 4 ((tid + NT_ u) % 16)), and the next query group's rows with their
  // query indexes and mask values
  f32x4 kr[KVP], vr[KVP], qraw[4];
  int qix[4];       // query row of piece u's group row
  int64_t mraw[4];  // its mask value (prefix form)
  int pn[4];        // perm entries of the group after the one being fetched
  int qok = 0;      // bit u: piece u's row is a query of the fetched group
  auto fetch_kv = [&](int64_t c) {
#pragma unroll
    for (int u = 0; u < KVP; ++u) {
      const int pc = tid + NT_ * u, row = pc >> 4, col = 4 * (pc & 15);
      const int64_t t = c * C + row;
      kr[u] = t < n ? *reinterpret_cast<const f32x4*>(kh + t * FD + col) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      vr[u] = t < n ? *reinterpret_cast<const f32x4*>(vh + t * FD + col) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  auto groups_of = [&](int64_t c) -> int { return (int)((bo(c + 1) - bo(c) + QG - 1) / QG); };
  auto after = [&](int64_t& cc, int& gg) {  // the query group after (cc, gg); cc == c1 past the last
    ++gg;
    while (cc < c1 && gg >= groups_of(cc)) {
      ++cc;
      gg = 0;
    }
  };
  // perm entries of group (cc, gg)'s rows.  They are requested one group
  // ahead of the rows they index: a gather that waited for its own perm
  // entries would wait for every load and store in flight (loads and
  // stores share one counter on this GPU), and with them for the next
  // chunk's K and V tiles (measured: 148 / 185 against 136 / 164 us per
  // call at fp32 B4 H8 n8192, m = arange / uniform, with no perm reads).
  // Rows past the group's end take its last entry (a group holds at least
  // one query): an unconditional load, whose value nothing reads before the
  // next wait (a choice between the loaded value and a constant would be
  // made, and waited for, at once); those rows are masked where used.
  // Past the walk's last group the loads take entry 0 (never used), so
  // that the registers are loaded on every path: a path without the loads
  // would have the compiler move the loaded values at the join, and wait.
  auto fetch_perm = [&](int64_t cc, int gg) {
    int64_t s0 = 0, e0 = 1;
    if (cc < c1) {
      s0 = bo(cc) + (int64_t)QG * gg;
      e0 = bo(cc + 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid + NT_ * u) >> 4;
      pn[u] = (int)qrow(s0 + row < e0 ? s0 + row : e0 - 1);
    }
  };
  auto fetch_q_after = [&](int64_t c, int grp) {  // rows of the query group after (c, grp), if any
    int64_t cc = c;
    int gg = grp;
    after(cc, gg);
    int64_t s0 = 0, e0 = 0;  // past the last group every row is masked (the same code path, as above)
    if (cc < c1) {
      s0 = bo(cc) + (int64_t)QG * gg;
      e0 = bo(cc + 1);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = tid + NT_ * u, row = pc >> 4, col = 4 * (pc & 15);
      const bool ok = s0 + row < e0;
      qix[u] = pn[u];
      qraw[u] = ok ? *reinterpret_cast<const f32x4*>(qh + (int64_t)pn[u] * FD + col) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      qok = ok ? (qok | (1 << u)) : (qok & ~(1 << u));
      if constexpr (!CS) mraw[u] = ok ? m[pn[u]] : 0;
    }
    after(cc, gg);
    fetch_perm(cc, gg);
  };
  if (c0 < c1) {
    fetch_kv(c0);
    int64_t cc = c0;
    int gg = -1;
    after(cc, gg);
    fetch_perm(cc, gg);
    fetch_q_after(c0, -1);
  }
  // Everything requested so far has arrived before the walk starts.  Left
  // out, the state registers' first loads would still count as pending at
  // every chunk's S store, whose wait would then also take in the next
  // chunk's K and V rows requested just before it.
  __builtin_amdgcn_s_waitcnt(0);

  // the fetched query group's rows into sQ, their query rows and mask
  // values into sI and sM
  auto stage_q = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = tid + NT_ * u, row = pc >> 4, col = 4 * (pc & 15);
      // (phi is applied here, not as the rows arrive: using a loaded value
      // waits for it)
      *reinterpret_cast<f32x4*>(sQ + row * RK + col) = (CS && ((qok >> u) & 1)) ? phi4(qraw[u]) : qraw[u];
      if (col == 0) {
        sI[row] = qix[u];
        int64_t mi = qix[u];
        if constexpr (!CS) {
          mi = mraw[u];
          mi = mi < 0 ? 0 : (mi >= n ? n - 1 : mi);  // same clamp as the bucket sort
        }
        sM[row] = (int)mi;
      }
    }
  };

  // Every wait for fetched data (staging into LDS) is a wait for all loads
  // and stores in flight, so each chunk and query group stages what it needs
  // before it requests the next one's rows: the chunk's K and V tiles and
  // its first group's queries together, then the next chunk's tiles and the
  // next group's rows go out.
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int ngroups = groups_of(c);
#pragma unroll
    for (int u = 0; u < KVP; ++u) {
      const int pc = tid + NT_ * u, row = pc >> 4, col = 4 * (pc & 15);
      f32x4 kk = kr[u];
      if (CS) kk = t0 + row < n ? phi4(kk) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      *reinterpret_cast<f32x4*>(sK + row * RK + col) = kk;
      *reinterpret_cast<f32x4*>(sV + row * RV + col) = vr[u];
    }
    if (CS && tid < FD) sz[tid] = zacc;
    if (c + 1 < c1) fetch_kv(c + 1);
    // S_prev(c) in operand order: block (bb, tt = sj) entry lane is accS[bb]
    if (owner) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int blk = bb * 4 + sj;
        *reinterpret_cast<f32x4*>(sS + (blk * 64 + (lane ^ blk)) * 4) = accS[bb];
      }
    }
    __syncthreads();  // tiles, S and the first group's rows visible
    if (ngroups == 0 && owner) state_update();

    for (int grp = 0; grp < ngroups; ++grp) {
      {
        stage_q();
        fetch_q_after(c, grp);
        __syncthreads();  // the group's query rows visible
      }
      if (grp == 0 && owner) state_update();
      const int64_t g0 = bo(c) + (int64_t)QG * grp;  // the group's first position in perm
      const int64_t i0 = g0 + 16 * w;                 // this wave's first query
      const int64_t e0 = bo(c + 1);
      // the group's 16-query blocks; fewer than one per wave (the last group
      // of a bucket, as a rule) and the waves share the blocks instead
      const int nbk = (int)(((e0 - g0 < QG ? e0 - g0 : QG) + 15) / 16);
      if (!CS && nbk < NWV) {
        // Block by block: wave w forms the masked scores of key block w
        // and leaves them in sP (its accumulator as the lane's float4), then
        // forms output features 16 w .. 16 w + 15 of the block's queries
        // from S and all four key blocks' scores: 48 MFMAs per wave and
        // block instead of 192 on one wave while the others wait.  sP has
        // two buffers: a wave writes block qb + 2's scores only after every
        // wave has passed block qb + 1's barrier, that is, after its reads
        // of block qb's.
        static_assert(NWV == 4, "one key block and one feature block per wave");
        for (int qb = 0; qb < nbk; ++qb) {
          const int row = 16 * qb + mm;
          const bool valid = g0 + row < e0;
          const int limit = valid ? (int)(sM[row] - t0) : -1;
          f32x4 qo[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) qo[tt] = *reinterpret_cast<const f32x4*>(sQ + row * RK + 16 * tt + 4 * kq);
          f32x4 sc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const f32x4 ko = *reinterpret_cast<const f32x4*>(sK + (16 * w + mm) * RK + 16 * tt + 4 * kq);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sc = __builtin_amdgcn_mfma_f32_16x16x4f32(ko[jj], qo[tt][jj], sc, 0, 0, 0);
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sc[rr] = (16 * w + 4 * kq + rr <= limit) ? sc[rr] : 0.0f;
          f32x4* pb = reinterpret_cast<f32x4*>(sP) + (qb & 1) * 4 * 64;
          pb[w * 64 + lane] = sc;
          f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {  // S^T Q^T for this wave's features
            const int blk = w * 4 + tt;
            const f32x4 so = *reinterpret_cast<const f32x4*>(sS + (blk * 64 + (lane ^ blk)) * 4);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o = __builtin_amdgcn_mfma_f32_16x16x4f32(so[jj], qo[tt][jj], o, 0, 0, 0);
          }
          __syncthreads();  // the block's four score blocks in sP
#pragma unroll
          for (int kb = 0; kb < C / 16; ++kb) {  // V^T P^T over the chunk's keys
            const f32x4 p = pb[kb * 64 + lane];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              o = __builtin_amdgcn_mfma_f32_16x16x4f32(sV[(16 * kb + 4 * kq + rr) * RV + 16 * w + mm], p[rr], o, 0, 0, 0);
          }
          if (valid)
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(oh + (int64_t)sI[row] * FD + 16 * w + 4 * kq));
        }
      } else if (i0 < e0) {
        const bool valid = i0 + mm < e0;
        const int qi = valid ? sI[16 * w + mm] : 0;
        const int64_t mi = valid ? sM[16 * w + mm] : 0;
        const int limit = (int)(mi - t0);
        f32x4 qo[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) qo[tt] = *reinterpret_cast<const f32x4*>(sQ + (16 * w + mm) * RK + 16 * tt + 4 * kq);
        f32x4 o[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) o[bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // S_prev^T Q^T
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 so[4];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) so[bb] = *reinterpret_cast<const f32x4*>(sS + ((bb * 4 + tt) * 64 + (lane ^ (bb * 4 + tt))) * 4);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) o[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(so[bb][jj], qo[tt][jj], o[bb], 0, 0, 0);
        }
        // the four key blocks' scores (independent chains), masked, then
        // V^T P^T over their keys
        f32x4 sc[C / 16];
#pragma unroll
        for (int kb = 0; kb < C / 16; ++kb) sc[kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 ko[C / 16];
#pragma unroll
          for (int kb = 0; kb < C / 16; ++kb) ko[kb] = *reinterpret_cast<const f32x4*>(sK + (16 * kb + mm) * RK + 16 * tt + 4 * kq);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int kb = 0; kb < C / 16; ++kb) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ko[kb][jj], qo[tt][jj], sc[kb], 0, 0, 0);
        }
#pragma unroll
        for (int kb = 0; kb < C / 16; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) sc[kb][rr] = (16 * kb + 4 * kq + rr <= limit) ? sc[kb][rr] : 0.0f;
#pragma unroll
        for (int kb = 0; kb < C / 16; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
              o[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(sV[(16 * kb + 4 * kq + rr) * RV + 16 * bb + mm], sc[kb][rr], o[bb], 0, 0, 0);
        if constexpr (CS) {  // denominator of query mm: phi(Q) . z_prev + its masked scores
          float dn = 0.0f;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const f32x4 zz = *reinterpret_cast<const f32x4*>(sz + 16 * tt + 4 * kq);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dn += qo[tt][jj] * zz[jj];
          }
#pragma unroll
          for (int kb = 0; kb < C / 16; ++kb)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) dn += sc[kb][rr];
          dn += __shfl_xor(dn, 16);
          dn += __shfl_xor(dn, 32);
          const float rd = 1.0f / dn;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) o[bb][jj] *= rd;
        }
        if (valid) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
            __builtin_nontemporal_store(o[bb], reinterpret_cast<f32x4*>(oh + (int64_t)qi * FD + 16 * bb + 4 * kq));
        }
      }
      // the group's rows are no longer read (after a chunk's last group the
      // barrier at the chunk's end serves)
      if (grp + 1 < ngroups) __syncthreads();
    }
    if (CS && tid < FD) {  // z_prev(c + 1): add this chunk's phi(K) column sums (rows past n are 0)
#pragma unroll 8
      for (int r = 0; r < C; ++r) zacc += sK[r * RK + tid];
    }
    __syncthreads();  // tiles and S are rewritten by the next chunk
  }
}

// -------------------------------------------------------------------- k_out
// Causal (FORM = CAUSAL: phi, normalised; the queries of chunk c are its own
// rows, for each of the R query heads of this key/value head) or prefix
// (FORM = PREFIX: identity feature map, no normaliser, R = 1; the queries of
// chunk c are the bucket perm[boff[c] .. boff[c+1]) in tiles of C).
// Waves per SIMD that k_out is compiled for: two where its tiles leave room for
// two workgroups per CU (then the registers must fit that occupancy), else one.
template <typename T, int DP, int C>
constexpr int k_out_waves() {
  return la_internal::chunk_lds_bytes((int)sizeof(T), DP, C) <= la_internal::kLdsLimit / 2 ? 2 : 1;
}

template <typename T, int DP, int C, int FORM, int PM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(k_out_waves<T, DP, C>()))) void k_out(const T* __restrict__ q, const T* __restrict__ k,
                                            const T* __restrict__ v, T* __restrict__ out, int64_t n, int d,
                                            int R, bool vec, int64_t nchunks, int64_t G, int64_t nseg,
                                            const float* __restrict__ ws, const int* __restrict__ perm,
                                            const int* __restrict__ boff, const int64_t* __restrict__ m,
                                            int64_t H, int64_t nmask) {
  constexpr int LQ = DP + PAD;  // row stride of sQ, sK, sST
  constexpr int LC = C + PAD;   // row stride of sKT, sVT, sP
  constexpr int NIB = C / 32;   // 32-row query / key blocks per chunk
  constexpr int NBB = DP / 32;  // 32-wide feature blocks
  constexpr bool NORM = (FORM == CAUSAL);
  static_assert(NORM == (PM != PM_ID), "the causal form takes a feature map, the prefix form none");
  // tiles of phi(Q) and phi(K) (scores), of the keys the state update takes
  // (relu(K) with the relu + 1 split, below), and whether S and z carry that
  // split (S = accS + 1 (x) sum of V, z counts the keys)
  constexpr int QX = q_xform<PM>();
  constexpr int KTX = k_xform<PM>();
  constexpr bool SPLIT = PM == PM_RELU1;
  __shared__ __attribute__((aligned(16))) T sQ[C * LQ];
  __shared__ __attribute__((aligned(16))) T sK[C * LQ];
  __shared__ __attribute__((aligned(16))) T sKT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sVT[DP * LC];
  __shared__ __attribute__((aligned(16))) T sST[DP * LQ];
  __shared__ __attribute__((aligned(16))) T sP[C * LC];
  __shared__ float sz[DP];
  __shared__ float svc[DP];  // sum of V over the chunks done so far (see k_state)
  // z in the input type as a high part and the remainder (z = high + low to
  // about 2^-17 in bf16; exact high and zero low in fp32), and a zero row:
  // the rows of the A operand of the phi(Q) . z products
  __shared__ __attribute__((aligned(16))) T szh[DP + 16];
  __shared__ __attribute__((aligned(16))) T szl[DP + 16];
  __shared__ __attribute__((aligned(16))) T szero[DP + 16];
  __shared__ __attribute__((aligned(16))) T sones[16];
  using SB = StateBlocks<DP>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  if (FORM == PREFIX) {  // this batch's mask, buckets and permutation (one per batch, or one shared)
    const int64_t mb = nmask > 1 ? bh / H : 0;
    perm += mb * n;
    boff += mb * (nchunks + 1);
    m += mb * n;
  }
  const T* kb = k + bh * n * d;
  const T* vb = v + bh * n * d;

  // This wave's output blocks: fixed query block ib, feature blocks nb.
  const int ib = w % NIB;
  const int nb0 = w / NIB;
  constexpr int NB_STEP = NW / NIB;  // NIB divides NW
  const bool has_out = nb0 < NBB;

  f32x16 accS[SB::PER_WAVE];
  {
    const float* src = ws + (bh * (nseg + 1) + seg) * slot_elems(DP);
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) ld_state_block<DP>(accS[s], src, e / SB::NB, e % SB::NB, lane);
      else accS[s] = f32x16{};
    }
  }
  // The accumulators hold relu(K)^T V terms on top of the exclusive prefix;
  // S = accS + 1 (x) vrun over the rows a < d (vrun: sum of V since the
  // segment start).  z is carried exactly in zrun.
  float zrun = 0.0f, vrun = 0.0f;
  if (NORM && tid < DP) zrun = ws[(bh * (nseg + 1) + seg) * slot_elems(DP) + DP * DP + tid];
  if (NORM && tid < 16) sones[tid] = cvt<T>(1.0f);
  if (NORM && tid < 16) {
    szero[DP + tid] = cvt<T>(0.0f);
    szh[DP + tid] = cvt<T>(0.0f);
    szl[DP + tid] = cvt<T>(0.0f);
  }
  if (NORM && tid < DP) svc[tid] = 0.0f;
  if (NORM) __syncthreads();

  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;
  // Query groups of chunk c: R heads (causal) or bucket tiles (prefix).
  auto groups_of = [&](int64_t c) -> int {
    if (FORM == CAUSAL) return R;
    return (int)((boff[c + 1] - boff[c] + C - 1) / C);
  };
  // Query tile of group grp of chunk c: base, gather indices, rows
  struct QTile {
    const T* base;
    const int* gidx;
    int rows;
  };
  auto qtile = [&](int64_t c, int grp) -> QTile {
    const int64_t tc = c * C;
    if (FORM == CAUSAL) return {q + (bh * R + grp) * n * d, nullptr, (int)((n - tc) < C ? (n - tc) : C)};
    const int64_t s0 = boff[c] + (int64_t)grp * C;
    const int64_t rem = boff[c + 1] - s0;
    return {q + bh * n * d, perm + s0, (int)(rem < C ? rem : C)};
  };
  // With d == DP the tiles are prefetched one step ahead: the next query tile
  // while the current group runs, and K and V of the next chunk while the
  // current chunk's groups run (the kernel is compiled for two waves per
  // SIMD, so that two workgroups share a CU where LDS allows).
  constexpr bool PF_KV = true;
  TileRaw<T, DP, C> rK, rV, rQ;
  int64_t kv_c = -1, q_c = -1;  // which chunk / (chunk, group) the registers hold
  int q_g = 0;
  auto fetch_kv = [&](int64_t c) {
    const int64_t tc = c * C;
    const int nvc = (int)((n - tc) < C ? (n - tc) : C);
    tile_fetch<T, DP, C>(rK, kb, tc, nullptr, nvc, tid);
    tile_fetch<T, DP, C>(rV, vb, tc, nullptr, nvc, tid);
    kv_c = c;
  };
  auto fetch_q_after = [&](int64_t c, int grp) {  // the group after (c, grp), if any
    int64_t cc = c;
    int gg = grp + 1;
    while (cc < c1 && gg >= groups_of(cc)) {
      ++cc;
      gg = 0;
    }
    if (cc < c1) {
      const QTile qt = qtile(cc, gg);
      tile_fetch<T, DP, C>(rQ, qt.base, cc * C, qt.gidx, qt.rows, tid);
      q_c = cc;
      q_g = gg;
    } else {
      q_c = -1;
    }
  };
  if (vec && c0 < c1) {
    if (PF_KV) fetch_kv(c0);
    fetch_q_after(c0, -1);
  }
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)((n - t0) < C ? (n - t0) : C);
    const int ngroups = groups_of(c);

    if (PF_KV && vec && kv_c == c) {
      tile_store<T, DP, C, QX, KTX>(rK, nv, sK, sKT, tid);
      tile_store<T, DP, C, XF_NONE, XF_ID>(rV, nv, nullptr, sVT, tid);
      if (c + 1 < c1) fetch_kv(c + 1);
    } else {
      load_tile<T, DP, C, QX, KTX>(kb, t0, nullptr, nv, d, vec, sK, sKT, tid);
      load_tile<T, DP, C, XF_NONE, XF_ID>(vb, t0, nullptr, nv, d, vec, nullptr, sVT, tid);
    }
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        f32x16 cur = accS[s];
        if (SPLIT) add_col(cur, svc[nb * 32 + (lane & 31)], ma, d, lane);
        st_accT(sST + nb * 32 * LQ + ma * 32, LQ, cur, lane);  // sST[b][a] = S[a][b]
      }
    }
    if (NORM && tid < DP) {
      sz[tid] = zrun;
      const T zh = cvt<T>(zrun);
      szh[tid] = zh;
      szl[tid] = cvt<T>(zrun - to_f(zh));
      szero[tid] = cvt<T>(0.0f);
    }

    for (int grp = 0; grp < ngroups; ++grp) {
      // ---- query tile of this group
      const QTile qt = qtile(c, grp);
      const int* gidx = qt.gidx;
      const int qcount = qt.rows;
      if (grp > 0) __syncthreads();  // previous group is done with sQ / sP
      if (vec && q_c == c && q_g == grp) {
        tile_store<T, DP, C, QX, XF_NONE>(rQ, qcount, sQ, nullptr, tid);
        fetch_q_after(c, grp);
      } else {
        load_tile<T, DP, C, QX, XF_NONE>(qt.base, t0, gidx, qcount, d, vec, sQ, nullptr, tid);
      }
      __syncthreads();

      // ---- P^T blocks (key block jb, query block ib2), masked, -> sP[i][j]
      {
        int e = 0;
#pragma unroll
        for (int ib2 = 0; ib2 < NIB; ++ib2) {
#pragma unroll
          for (int jb = 0; jb < NIB; ++jb) {
            if (FORM == CAUSAL && jb > ib2) continue;
            if ((e++ % NW) != w) continue;
            f32x16 acc = f32x16{};
            gemm_acc<T, DP / 16>(acc, sK + jb * 32 * LQ, LQ, sQ + ib2 * 32 * LQ, LQ, lane);
            const int i = ib2 * 32 + (lane & 31);
            int limit;
            if (FORM == CAUSAL) {
              limit = i;
            } else {
              limit = -1;
              if (i < qcount) {
                int64_t mi = m[gidx[i]];
                mi = mi < 0 ? 0 : (mi >= n ? n - 1 : mi);  // same clamp as k_bucket
                limit = (int)(mi - t0);
              }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = jb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              if (j > limit) acc[r] = 0.0f;
            }
            st_accT(sP + ib2 * 32 * LC + jb * 32, LC, acc, lane);
          }
        }
      }
      __syncthreads();

      // ---- outputs of this wave: out^T[b][i] = S^T phi(Q)^T + V^T P^T
      constexpr int NPW = (NBB + NB_STEP - 1) / NB_STEP;  // output blocks per wave
      f32x16 accO[NPW];
      float inv = 1.0f;
      const int i = ib * 32 + (lane & 31);
      if (has_out) {
        if (NORM) {
          // den_i = sum_j P_ij + phi(Q_i) . z on MFMA: A operand rows 0 (ones
          // over the keys, then z high over the features) and 16 (z low);
          // the results land in registers 0 and 8 of the lanes with h == 0
          const int m = lane & 31;
          Frag<T> e0;
          ld_frag(e0, m == 0 ? sones : szero);
          f32x16 dacc = f32x16{};
#pragma unroll
          for (int jb = 0; jb < NIB; ++jb) {
            if (FORM == CAUSAL && jb > ib) continue;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              Frag<T> fb;
              ld_frag(fb, sP + i * LC + jb * 32 + 16 * kb + 4 * h);
              mma(dacc, e0, fb);
            }
          }
          const T* zrow = (m == 0) ? szh : (m == 16) ? szl : szero;
#pragma unroll
          for (int kb = 0; kb < DP / 16; ++kb) {
            Frag<T> fa, fb;
            ld_frag(fa, zrow + 16 * kb + 4 * h);
            ld_frag(fb, sQ + i * LQ + 16 * kb + 4 * h);
            mma(dacc, fa, fb);
          }
          inv = 1.0f / __shfl(dacc[0] + dacc[8], lane & 31);
        }
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int nb = nb0 + u * NB_STEP;
          accO[u] = f32x16{};
          if (nb < NBB) {
            gemm_acc<T, DP / 16>(accO[u], sST + nb * 32 * LQ, LQ, sQ + ib * 32 * LQ, LQ, lane);
#pragma unroll
            for (int jb = 0; jb < NIB; ++jb) {
              if (FORM == CAUSAL && jb > ib) continue;
              gemm_acc<T, 2>(accO[u], sVT + nb * 32 * LC + jb * 32, LC, sP + ib * 32 * LC + jb * 32, LC, lane);
            }
          }
        }
      }
      // the tile goes out through sQ (free once every wave is past this
      // barrier) so that global stores cover whole rows
      __syncthreads();
      if (has_out) {
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int nb = nb0 + u * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              sQ[i * LQ + nb * 32 + 8 * (e >> 2) + 4 * h + (e & 3)] = cvt<T>(NORM ? accO[u][e] * inv : accO[u][e]);
          }
        }
      }
      __syncthreads();
      if (FORM == CAUSAL)
        copy_rows_out<T, DP, LQ>(sQ, qcount, d, vec, out + (bh * R + grp) * n * d, nullptr, t0, tid);
      else
        copy_rows_out<T, DP, LQ>(sQ, qcount, d, vec, out + bh * n * d, gidx, 0, tid);
    }

    // ---- S += phi(K_c)^T V_c ;  z += column sums of phi(K_c)
#pragma unroll
    for (int s = 0; s < SB::PER_WAVE; ++s) {
      const int e = w + NW * s;
      if (e < SB::TOTAL) {
        const int ma = e / SB::NB, nb = e % SB::NB;
        gemm_acc<T, C / 16>(accS[s], sKT + ma * 32 * LC, LC, sVT + nb * 32 * LC, LC, lane);
      }
    }
    if (NORM && tid < DP) {
      zrun += row_sum<T, C>(sKT, tid) + (SPLIT && tid < d ? (float)nv : 0.0f);
      if (SPLIT) {
        vrun += row_sum<T, C>(sVT, tid);
        svc[tid] = vrun;  // read at the next chunk's start, after the barrier below
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------- k_out_gqa
// Causal output for bf16 with d = 128, chunk 32 and R = 1, 2, 4 or 8 query
// heads per key/value head: the R query heads of a chunk are worked on at
// once (NWV = 8 waves for R >= 2, four for R = 1; head g = w / (NWV / R),
// each of its NWV / R waves 4 / (NWV / R) of the four 32-wide output feature
// blocks), so that a chunk costs two barriers whatever R is (three at R = 8,
// whose output tiles reuse the query tiles: each head has one wave, which
// forms all its output blocks before writing them over its phi(Q) tile),
// against four per query head in k_out.  Each wave forms its
// head's score block P^T = phi(K) phi(Q)^T itself, in registers (its
// accumulator is the B operand of V^T P^T; la_device.h), and the row sums of
// the rounded P for the normaliser.  The state is carried as in k_out: two of
// the 16 32 x 32 state blocks per wave in MFMA accumulators (four with four
// waves), relu(K)^T V on top of the segment's exclusive prefix, plus
// 1 (x) (sum of V).  relu(K) and V stay token-major in LDS; their operands
// over the token index (V^T for V^T P^T, both operands of relu(K)^T V) are
// transposed reads, and z and the sums of V are dot2 sums over those
// fragments (eight waves: waves 0-3 z of rows 32 w .., waves 4-7 sums of V of
// columns 32 (w - 4) ..; four waves: wave w both, for 32 w ..).
// A workgroup walks F state segments (G chunks of the state pass each) and
// starts from the exclusive prefix in slot F * seg of the workspace, whose
// per-head stride is nseg_ws + 1 slots.
template <int R> constexpr int gqa_waves() { return R == 1 ? 4 : 8; }
template <int R, int PM>
// (two waves per SIMD: one eight-wave workgroup or two four-wave ones per CU)
__global__ __launch_bounds__(64 * gqa_waves<R>()) __attribute__((amdgpu_waves_per_eu(2))) void k_out_gqa(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                 const bf16* __restrict__ v, bf16* __restrict__ out, int64_t n,
                                                 int64_t nchunks, int64_t G, int64_t nseg, int64_t F,
                                                 int64_t nseg_ws, const float* __restrict__ ws) {
  constexpr int DP = 128, C = 32;
  constexpr int LQ = DP + PAD;  // row stride of sK, sQ, sO, sST
  constexpr int RS = STR_RS;    // row stride of sKr, sV (conflict-free transposed reads)
  constexpr int NWV = gqa_waves<R>(), NT_ = 64 * NWV;
  constexpr int NPH = NWV / R;   // waves per query head
  constexpr int NBW = 4 / NPH;   // 32-wide output feature blocks per wave
  constexpr int NH = NWV / 4;    // 256-thread halves sharing the tile loads
  constexpr int NSW = 16 / NWV;  // state blocks per wave
  static_assert(R == 1 || R == 2 || R == 4 || R == 8, "one, two, four or eight query heads per key/value head");
  constexpr bool OQ = R == 8;  // output tiles over the query tiles
  // relu + 1 split as in k_state_tr; ELU + 1: phi(K), phi(Q) in the tiles
  constexpr bool SPLIT = PM == PM_RELU1;
  __shared__ __attribute__((aligned(16))) bf16 sK[C * LQ];       // phi(K), token-major
  __shared__ __attribute__((aligned(16))) bf16 sKr[C * RS];     // relu(K), token-major
  __shared__ __attribute__((aligned(16))) bf16 sV[C * RS];      // V, token-major
  __shared__ __attribute__((aligned(16))) bf16 sST[DP * LQ];     // S^T in bf16
  __shared__ __attribute__((aligned(16))) bf16 sQ[R][C * LQ];    // phi(Q) of each query head
  __shared__ __attribute__((aligned(16))) bf16 sO[OQ ? 1 : R][C * LQ];  // outputs on their way out (R = 8: in sQ)
  __shared__ __attribute__((aligned(16))) bf16 szh[DP];          // z as bf16 high part,
  __shared__ __attribute__((aligned(16))) bf16 szl[DP];          // the remainder,
  __shared__ __attribute__((aligned(16))) bf16 szero[DP];        // and zeros: the z operand's rows
  __shared__ float svc[DP];  // sum of V over the chunks done so far

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, r = lane & 31;
  const int half = tid >> 8, ht = tid & 255;  // the 256-thread halves share the tile loads
  const int g = w / NPH, hf = w % NPH;
  const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
  const bf16* kb = k + bh * n * DP;
  const bf16* vb = v + bh * n * DP;
  const float* slot = ws + (bh * (nseg_ws + 1) + F * seg) * slot_elems(DP);

  // state blocks e = w + NWV s: (row block ma, column block nb) = (e / 4, e % 4)
  f32x16 accS[NSW];
#pragma unroll
  for (int s = 0; s < NSW; ++s) ld_state_block<DP>(accS[s], slot, (w + NWV * s) / 4, (w + NWV * s) % 4, lane);
  // waves 0-3: z[32 w + r]; the sum of V[., 32 (w - 4) + r] on waves 4-7 (8
  // waves), of V[., 32 w + r] beside z (4 waves)
  float zrun = 0.0f, vrun = 0.0f;
  if (w < 4) zrun = slot[DP * DP + 32 * w + r];
  if (tid < DP) {
    svc[tid] = 0.0f;
    szero[tid] = (bf16)0.0f;
  }

  // Tiles of a chunk: half 0 loads K, half 1 V (one half: both), two adjacent
  // rows x 8 features per thread; query tile g goes to half g % NH.
  constexpr int QPH = R / NH;  // query tiles per half
  TileRaw<bf16, DP, C> raw[QPH];
  la_bf16::u32x4 kv2[2], vv2[2];
  const int pr0 = 2 * (ht >> 4), pc0 = 8 * (ht & 15);
  const int64_t c0 = seg * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;
  auto fetch = [&](int64_t c) {
    const int64_t tc = c * C;
    const int nvc = (int)((n - tc) < C ? (n - tc) : C);
    const bf16* src = half == 0 ? kb : vb;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      kv2[rr] = pr0 + rr < nvc ? *reinterpret_cast<const la_bf16::u32x4*>(src + (tc + pr0 + rr) * DP + pc0)
                               : la_bf16::u32x4{0u, 0u, 0u, 0u};
    if constexpr (NH == 1) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        vv2[rr] = pr0 + rr < nvc ? *reinterpret_cast<const la_bf16::u32x4*>(vb + (tc + pr0 + rr) * DP + pc0)
                                 : la_bf16::u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < QPH; ++u)
      tile_fetch<bf16, DP, C>(raw[u], q + (bh * R + NH * u + half) * n * DP, tc, nullptr, nvc, ht);
  };
  if (c0 < c1) fetch(c0);
  __syncthreads();

  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)((n - t0) < C ? (n - t0) : C);
    {
      // K: relu(K) and phi(K) token-major (phi(K) zero past the sequence
      // end; relu(K) and V are zero there as loaded); V: token-major
      bf16* tm = half == 0 ? sKr : sV;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        la_bf16::u32x4 x = kv2[rr];
        if (half == 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            x[j] = SPLIT ? la_bf16::relu2(x[j]) : (pr0 + rr < nv ? la_bf16::map2<PM>(x[j]) : 0u);
        }
        *reinterpret_cast<la_bf16::u32x4*>(tm + (pr0 + rr) * RS + pc0) = x;
        if constexpr (NH == 1) *reinterpret_cast<la_bf16::u32x4*>(sV + (pr0 + rr) * RS + pc0) = vv2[rr];
      }
      if (half == 0) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          uint32_t y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[j] = pr0 + rr < nv ? (SPLIT ? la_bf16::phi2(kv2[rr][j]) : la_bf16::map2<PM>(kv2[rr][j])) : 0u;
          uint2* dst = reinterpret_cast<uint2*>(sK + (pr0 + rr) * LQ + pc0);
          dst[0] = make_uint2(y[0], y[1]);
          dst[1] = make_uint2(y[2], y[3]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < QPH; ++u)
      tile_store<bf16, DP, C, q_xform<PM>(), XF_NONE>(raw[u], nv, sQ[NH * u + half], nullptr, ht);
    if (c + 1 < c1) fetch(c + 1);
#pragma unroll
    for (int s = 0; s < NSW; ++s) {
      const int e = w + NWV * s, ma = e / 4, nb = e % 4;
      f32x16 cur = accS[s];
      if (SPLIT) add_col(cur, svc[nb * 32 + r], ma, DP, lane);
      st_accT(sST + nb * 32 * LQ + ma * 32, LQ, cur, lane);  // sST[b][a] = S[a][b]
    }
    if (w < 4 && h == 0) {
      const bf16 zh = (bf16)zrun;
      szh[32 * w + r] = zh;
      szl[32 * w + r] = (bf16)(zrun - (float)zh);
    }
    __syncthreads();

    // ---- head g: P^T (keys j, queries i), masked; its row sums; phi(Q) . z
    const bf16* qg = sQ[g];
    f32x16 pacc = f32x16{};
    gemm_acc<bf16, DP / 16>(pacc, sK, LQ, qg, LQ, lane);
#pragma unroll
    for (int e = 0; e < 16; ++e) pacc[e] = (8 * (e >> 2) + 4 * h + (e & 3) <= r) ? pacc[e] : 0.0f;
    const Frag<bf16> p0 = la_bf16::acc_frag(pacc, 0), p1 = la_bf16::acc_frag(pacc, 1);
    float ds = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      ds = la_bf16::dot2(la_bf16::pair(p1, j), la_bf16::ONE2, la_bf16::dot2(la_bf16::pair(p0, j), la_bf16::ONE2, ds));
    ds += __shfl_xor(ds, 32);
    f32x16 zacc = f32x16{};
    {
      const bf16* zrow = (r == 0) ? szh : (r == 16) ? szl : szero;
      gemm_acc<bf16, DP / 16>(zacc, zrow - r * LQ, LQ, qg, LQ, lane);
    }
    const float inv = 1.0f / __shfl(ds + zacc[0] + zacc[8], r);  // from the lane with h == 0
    // ---- this wave's output blocks: out^T[b][i] = S^T phi(Q)^T + V^T P^T
    // (at R = 8 all four are formed before any is written over phi(Q))
    if constexpr (OQ) {
      f32x16 o[NBW];
#pragma unroll
      for (int u = 0; u < NBW; ++u) {
        const int nb = hf * NBW + u;
        o[u] = f32x16{};
        gemm_acc<bf16, DP / 16>(o[u], sST + nb * 32 * LQ, LQ, qg, LQ, lane);
        mma(o[u], la_bf16::ld_tr<RS>(sV, 0, nb * 32, lane), p0);
        mma(o[u], la_bf16::ld_tr<RS>(sV, 16, nb * 32, lane), p1);
      }
#pragma unroll
      for (int u = 0; u < NBW; ++u) {
        const int nb = hf * NBW + u;
        uint2* dst = reinterpret_cast<uint2*>(sQ[g] + r * LQ + nb * 32 + 4 * h);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          dst[2 * qq] = make_uint2(la_bf16::pack2(o[u][4 * qq] * inv, o[u][4 * qq + 1] * inv),
                                   la_bf16::pack2(o[u][4 * qq + 2] * inv, o[u][4 * qq + 3] * inv));
      }
    } else {
#pragma unroll
      for (int u = 0; u < NBW; ++u) {
        const int nb = hf * NBW + u;
        f32x16 o = f32x16{};
        gemm_acc<bf16, DP / 16>(o, sST + nb * 32 * LQ, LQ, qg, LQ, lane);
        mma(o, la_bf16::ld_tr<RS>(sV, 0, nb * 32, lane), p0);
        mma(o, la_bf16::ld_tr<RS>(sV, 16, nb * 32, lane), p1);
        uint2* dst = reinterpret_cast<uint2*>(sO[g] + r * LQ + nb * 32 + 4 * h);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          dst[2 * qq] = make_uint2(la_bf16::pack2(o[4 * qq] * inv, o[4 * qq + 1] * inv),
                                   la_bf16::pack2(o[4 * qq + 2] * inv, o[4 * qq + 3] * inv));
      }
    }

    // ---- the R output tiles (R < 8): whole 256-byte rows, non-temporal
    // stores, issued before the state update so that they have its time to
    // complete before the next chunk's wait for its rows (which also waits
    // for every store before it): one barrier more per chunk, 384.5 -> 378.2
    // us at the long-context GQA shape (interleaved timing)
    constexpr int PIECES = C * (DP / 8);  // 16-byte pieces per tile
    if constexpr (!OQ) {
      __syncthreads();  // every wave's output blocks in sO
#pragma unroll
      for (int gg = 0; gg < R; ++gg) {
#pragma unroll
        for (int pp = tid; pp < PIECES; pp += NT_) {
          const int row = pp / (DP / 8), col = 8 * (pp % (DP / 8));
          if (row < nv)
            __builtin_nontemporal_store(*reinterpret_cast<const la_bf16::u32x4*>(sO[gg] + row * LQ + col),
                                        reinterpret_cast<la_bf16::u32x4*>(out + ((bh * R + gg) * n + t0 + row) * DP + col));
        }
      }
    }
    // ---- S += relu(K_c)^T V_c (two blocks per wave); z and the sum of V
    {
      Frag<bf16> vt[C / 16];
#pragma unroll
      for (int kt = 0; kt < C / 16; ++kt) vt[kt] = la_bf16::ld_tr<RS>(sV, 16 * kt, (w % 4) * 32, lane);
#pragma unroll
      for (int s = 0; s < NSW; ++s) {
        const int ma = (w + NWV * s) / 4;  // column block w % 4
#pragma unroll
        for (int kt = 0; kt < C / 16; ++kt) mma(accS[s], la_bf16::ld_tr<RS>(sKr, 16 * kt, ma * 32, lane), vt[kt]);
      }
      // waves 0-3: z of rows 32 w ..; the sums of V of columns 32 (w - 4) ..
      // on waves 4-7, of columns 32 w .. beside z with four waves
      float cs = 0.0f, csv = 0.0f;
#pragma unroll
      for (int kt = 0; kt < C / 16; ++kt) {
        const Frag<bf16> f = w < 4 ? la_bf16::ld_tr<RS>(sKr, 16 * kt, w * 32, lane) : vt[kt];
#pragma unroll
        for (int j = 0; j < 4; ++j) cs = la_bf16::dot2(la_bf16::pair(f, j), la_bf16::ONE2, cs);
        if constexpr (NWV == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) csv = la_bf16::dot2(la_bf16::pair(vt[kt], j), la_bf16::ONE2, csv);
        }
      }
      cs += __shfl_xor(cs, 32);
      if constexpr (NWV == 4) {
        csv += __shfl_xor(csv, 32);
        zrun += cs + (SPLIT ? (float)nv : 0.0f);
        vrun += csv;
        if (h == 0) svc[32 * w + r] = vrun;  // read at the next chunk's start (this chunk read it before the barrier above)
      } else if (w < 4) {
        zrun += cs + (SPLIT ? (float)nv : 0.0f);
      } else {
        vrun += cs;
        if (h == 0) svc[32 * (w - 4) + r] = vrun;  // read at the next chunk's start (this chunk read it before the barrier above)
      }
    }
    __syncthreads();

    // ---- R = 8: the output tiles, from the query tiles
    if constexpr (OQ) {
#pragma unroll
      for (int gg = 0; gg < R; ++gg) {
#pragma unroll
        for (int pp = tid; pp < PIECES; pp += NT_) {
          const int row = pp / (DP / 8), col = 8 * (pp % (DP / 8));
          if (row < nv)
            __builtin_nontemporal_store(*reinterpret_cast<const la_bf16::u32x4*>(sQ[gg] + row * LQ + col),
                                        reinterpret_cast<la_bf16::u32x4*>(out + ((bh * R + gg) * n + t0 + row) * DP + col));
        }
      }
      __syncthreads();  // the output tiles are read before the next chunk's query tiles overwrite them
    }
  }
}

// ----------------------------------------------------------------- k_out_nc
// Non-causal output: out_i = phi(Q_i) S / (phi(Q_i) . z) with the total state
// (slot nseg of the head).  One workgroup per (head, run of G chunks of
// queries), for each of the R query heads.
template <typename T, int DP, int C, int PM>
__global__ __launch_bounds__(NT) void k_out_nc(const T* __restrict__ q, T* __restrict__ out, int64_t n, int d, int R,
                                               bool vec, int64_t nchunks, int64_t G, int64_t nqseg, int64_t nseg,
                                               const float* __restrict__ ws) {
  constexpr int LQ = DP + PAD;
  constexpr int NIB = C / 32;
  constexpr int NBB = DP / 32;
  __shared__ __attribute__((aligned(16))) T sQ[C * LQ];
  __shared__ __attribute__((aligned(16))) T sST[DP * LQ];
  __shared__ float sz[DP];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5;
  const int64_t bh = blockIdx.x / nqseg, qs = blockIdx.x % nqseg;
  const float* tot = ws + (bh * (nseg + 1) + nseg) * slot_elems(DP);
  for (int idx = tid; idx < DP * DP; idx += NT) {
    const int a = idx / DP, b = idx % DP;
    sST[b * LQ + a] = cvt<T>(tot[idx]);
  }
  if (tid < DP) sz[tid] = tot[DP * DP + tid];
  const int ib = w % NIB;
  const int nb0 = w / NIB;
  constexpr int NB_STEP = NW / NIB;
  constexpr int NPW = (NBB + NB_STEP - 1) / NB_STEP;  // output blocks per wave
  const bool has_out = nb0 < NBB;
  const int64_t c0 = qs * G, c1 = (c0 + G < nchunks) ? c0 + G : nchunks;
  // with d == DP the next (chunk, head) query tile loads while this one is used
  TileRaw<T, DP, C> rQ;
  auto fetch = [&](int64_t c, int r) {
    const int64_t tc = c * C;
    tile_fetch<T, DP, C>(rQ, q + (bh * R + r) * n * d, tc, nullptr, (int)((n - tc) < C ? (n - tc) : C), tid);
  };
  if (vec && c0 < c1) fetch(c0, 0);
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t t0 = c * C;
    const int nv = (int)((n - t0) < C ? (n - t0) : C);
    for (int r = 0; r < R; ++r) {
      __syncthreads();  // sQ free (and sST / sz visible on the first pass)
      if (vec) {
        tile_store<T, DP, C, q_xform<PM>(), XF_NONE>(rQ, nv, sQ, nullptr, tid);
        if (r + 1 < R) fetch(c, r + 1);
        else if (c + 1 < c1) fetch(c + 1, 0);
      } else {
        load_tile<T, DP, C, q_xform<PM>(), XF_NONE>(q + (bh * R + r) * n * d, t0, nullptr, nv, d, vec, sQ,
                                                                  nullptr, tid);
      }
      __syncthreads();
      const int i = ib * 32 + (lane & 31);
      f32x16 acc[NPW];
      float inv = 0.0f;
      if (has_out) {
        float part = 0.0f;
        const T* qrow = sQ + i * LQ + h * (DP / 2);
        const float* zz = sz + h * (DP / 2);
        for (int a = 0; a < DP / 2; ++a) part += to_f(qrow[a]) * zz[a];
        inv = 1.0f / (part + __shfl_xor(part, 32));
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          acc[u] = f32x16{};
          const int nb = nb0 + u * NB_STEP;
          if (nb < NBB) gemm_acc<T, DP / 16>(acc[u], sST + nb * 32 * LQ, LQ, sQ + ib * 32 * LQ, LQ, lane);
        }
      }
      // the tile goes out through sQ so that global stores cover whole rows
      __syncthreads();
      if (has_out) {
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          const int nb = nb0 + u * NB_STEP;
          if (nb < NBB) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sQ[i * LQ + nb * 32 + 8 * (e >> 2) + 4 * h + (e & 3)] = cvt<T>(acc[u][e] * inv);
          }
        }
      }
      __syncthreads();
      copy_rows_out<T, DP, LQ>(sQ, nv, d, vec, out + (bh * R + r) * n * d, nullptr, t0, tid);
    }
  }
}

// ----------------------------------------------------------------- k_bucket
// Counting sort of the queries by the chunk their mask ends in,
// c(i) = floor(m_i / C): boff[c] is the first slot of bucket c in perm,
// boff[nchunks] = n.  One workgroup; the histogram and the fill cursors live
// in LDS (nchunks <= kMaxBuckets).  The order inside a bucket is arbitrary,
// which changes no output: each query's row is computed on its own.
// m_i outside [0, n-1] is clamped into that range.
// Add 1 for each valid lane to cnt[b] and return the counter's value before
// this lane's unit.  When every valid lane of the wave has the same b (as
// when m is sorted), one lane adds the wave's count and each lane takes its
// rank among the valid lanes; otherwise each lane adds its own unit.
__device__ __forceinline__ int bucket_take(int* cnt, int b, bool valid, int lane) {
  const uint64_t act = __ballot(valid);
  if (act == 0) return 0;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const int b0 = __shfl(b, leader);
  if (__ballot(valid && b == b0) == act) {
    int base = 0;
    if (lane == leader) base = atomicAdd(&cnt[b0], __popcll(act));
    base = __shfl(base, leader);
    return base + __popcll(act & ((1ull << lane) - 1ull));
  }
  return valid ? atomicAdd(&cnt[b], 1) : 0;
}

// The sort, for one workgroup of up to 1024 threads; cnt holds nchunks + 1
// ints and part one int per thread, both in LDS.  A mask value outside
// [0, n - 1] breaks the form's contract: it is clamped into range (so that
// every access stays inside the buffers) and recorded in the control
// block's error word, which la_workspace_status reports.
template <int PER>
__device__ __forceinline__ void bucket_sort(const int64_t* __restrict__ m, int64_t n, int C, int64_t nchunks, int* __restrict__ boff,
                            int* __restrict__ perm, int* cnt, int* part, la_internal::Ctl* ctl) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  bool bad = false;
  const int len = (int)nchunks + 1;
  for (int c = tid; c < len; c += nt) cnt[c] = 0;
  __syncthreads();
  // queries in blocks of PER per thread: all of a block's mask values are
  // requested before its counters are touched.  When one block covers the
  // whole mask (n <= PER x threads) the bucket of each query stays in
  // registers for the scatter pass, so the mask is read once.
  const int64_t step = (int64_t)nt * PER;
  const bool one_block = n <= step;
  int bk[PER];
  auto buckets = [&](int64_t base, bool count) {
    int64_t mv[PER];  // every load of the block first (left to itself the
                      // compiler waits for each before issuing the next)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int64_t i = base + tid + (int64_t)k * nt;
      mv[k] = i < n ? m[i] : -1;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int64_t i = base + tid + (int64_t)k * nt;
      bk[k] = -1;
      if (i < n) {
        int64_t mi = mv[k];
        if (count) bad |= mi < 0 || mi >= n;
        mi = mi < 0 ? 0 : (mi >= n ? n - 1 : mi);
        bk[k] = (int)(mi / C);
      }
    }
  };
  for (int64_t base = 0; base < n; base += step) {
    buckets(base, true);
#pragma unroll
    for (int k = 0; k < PER; ++k) bucket_take(cnt, bk[k] + 1, bk[k] >= 0, lane);
  }
  if (__ballot(bad) != 0 && lane == 0) la_ctl::ctl_fail(ctl, la_internal::kErrRange);
  __syncthreads();
  // inclusive scan of cnt[0..nchunks] (cnt[0] == 0): contiguous per-thread
  // ranges, then a scan of the per-thread sums
  const int per = (len + nt - 1) / nt;
  const int lo = tid * per, hi = (lo + per < len) ? lo + per : len;
  int sum = 0;
  for (int c = lo; c < hi; ++c) sum += cnt[c];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int c = lo; c < hi; ++c) {
    run += cnt[c];
    cnt[c] = run;
    boff[c] = run;
  }
  __syncthreads();
  // cnt[c] is now bucket c's fill cursor
  for (int64_t base = 0; base < n; base += step) {
    if (!one_block) buckets(base, false);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int pos = bucket_take(cnt, bk[k], bk[k] >= 0, lane);
      if (bk[k] >= 0) perm[pos] = (int)(base + tid + (int64_t)k * nt);
    }
  }
}

// Workgroup b sorts mask b (m [nmask][n] into boff [nmask][nchunks + 1] and
// perm [nmask][n]).
__global__ __launch_bounds__(1024) void k_bucket(const int64_t* __restrict__ m, int64_t n, int C, int64_t nchunks,
                                                 int* __restrict__ boff, int* __restrict__ perm,
                                                 la_internal::Ctl* ctl) {
  m += blockIdx.x * n;
  boff += blockIdx.x * (nchunks + 1);
  perm += blockIdx.x * n;
  __shared__ int cnt[la_internal::kMaxBuckets + 1];
  __shared__ int part[1024];
  bucket_sort<8>(m, n, C, nchunks, boff, perm, cnt, part, ctl);  // 1024 threads
}

// ---------------------------------------------------------------- k_state32
// k_state for fp32 with d = 64, on v_mfma_f32_16x16x4_f32 straight from
// token-major rows (no LDS transposes; the scheme of la_forward_f32.hip): a
// lane that loads 16 bytes of a row holds four consecutive features of one
// key, and each of them is the operand of its own MFMA.  The segment's keys
// go in 32-key blocks to the eight waves in turn; the buffer resources end
// at the segment's last key, so rows past it read as zero.  The wave
// results are summed in LDS in wave order and written to the segment's slot
// (S row-major, then z).  With bucket arguments (the prefix form), block 0
// of the same launch does k_bucket's sort (dispatched first, so that its
// serial passes overlap the state work).  n <= kFwd32MaxN, so
// that a head's rows stay below 2^31 bytes (the resources' record count).
union State32Lds {
  struct {
    f32x4 acc[4][16][64];  // entry (4 j + j', lane l), float rr: S[16 (l / 16) + 4 rr + j][4 (l % 16) + j']
    f32x4 z[8][16];        // z[4 m .. 4 m + 3] of each wave
  } s;
  struct {
    int cnt[la_internal::kMaxBuckets + 1];
    int part[512];
  } b;
};

// PM: the identity (prefix form), relu + 1 (split) or ELU + 1 (keys past the
// segment contribute 0, not phi(0) = 1).
template <int PM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_state32(const float* __restrict__ k, const float* __restrict__ v, int64_t n,
                                                 int64_t nchunks, int C, int64_t G, int64_t nseg,
                                                 float* __restrict__ ws, const int64_t* __restrict__ m,
                                                 int* __restrict__ boff, int* __restrict__ perm, int64_t nmask,
                                                 la_internal::Ctl* ctl) {
  constexpr int FD = 64, TW = 16, NW8 = 8;
  __shared__ State32Lds L;
  int64_t sb = blockIdx.x;  // state block
  if (m) {
    if (sb < nmask) {  // blocks 0 .. nmask - 1 sort the masks
      bucket_sort<16>(m + sb * n, n, C, nchunks, boff + sb * (nchunks + 1), perm + sb * n, L.b.cnt, L.b.part, ctl);
      return;
    }
    sb -= nmask;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, mm = lane & 15, kq = lane >> 4;
  const int64_t bh = sb / nseg, seg = sb % nseg;
  const int64_t k0 = seg * G * C, k1r = (seg + 1) * G * C, k1 = k1r < n ? k1r : n;
  // resources over this head's rows [0, k1): keys past the segment read as zero
  const int ebytes = (int)(k1 * FD * 4);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(k + bh * n * FD), 0, ebytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(v + bh * n * FD), 0, ebytes, 0x00020000);
  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int jp = 0; jp < 4; ++jp) acc[j][jp] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 zr = f32x4{0.0f, 0.0f, 0.0f, 0.0f};  // sum of relu(K) over this lane's keys
  int nkeys = 0;                               // keys this wave has taken
  const int64_t nblk = (k1 - k0 + TW - 1) / TW;
  for (int64_t blk = w; blk < nblk; blk += NW8) {
    const int64_t t0 = k0 + blk * TW;
    nkeys += (int)((k1 - t0) < TW ? (k1 - t0) : TW);
    // step s: keys t0 + 4 s + kq, features 4 mm ..; loads first, in step
    // order, then the steps (pinned so that step s waits for its own rows)
    f32x4 kr[TW / 4], vr[TW / 4];
#pragma unroll
    for (int s = 0; s < TW / 4; ++s) {
      const uint32_t off = (uint32_t)((t0 + 4 * s + kq) * FD + 4 * mm) * 4u;
      kr[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0, 0));
      vr[s] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, 0));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 0; s < TW / 4; ++s) {
      f32x4 pk;
      const bool real = t0 + 4 * s + kq < k1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (PM == PM_RELU1) {
          const float x = fmaxf(kr[s][j], 0.0f);
          zr[j] += x;
          pk[j] = x + 1.0f;  // keys past the segment: 1, against V = 0
        } else if (PM == PM_ELU1 || PM == PM_FEAT) {  // phi(K) as it is, 0 past the segment
          pk[j] = real ? (PM == PM_ELU1 ? elu1_f(kr[s][j]) : kr[s][j]) : 0.0f;
          zr[j] += pk[j];
        } else {
          pk[j] = kr[s][j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int jp = 0; jp < 4; ++jp)
          acc[j][jp] = __builtin_amdgcn_mfma_f32_16x16x4f32(pk[j], vr[s][jp], acc[j][jp], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    zr[j] += __shfl_xor(zr[j], 16);
    zr[j] += __shfl_xor(zr[j], 32);
    zr[j] += PM == PM_RELU1 ? (float)nkeys : 0.0f;  // the ones of phi(K), real keys only
  }
  // the segment's aggregate: waves 4-7 hand their results to waves 0-3
  // (w + 4 into w), whose sums are then added in wave order, and taken from
  // accumulator order to S row-major (64 KB of LDS, so that two workgroups
  // share a CU)
  if (w >= 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) L.s.acc[w - 4][4 * j + jp][lane] = acc[j][jp];
  }
  if (kq == 0) L.s.z[w][mm] = zr;
  __syncthreads();
  if (w < 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) acc[j][jp] += L.s.acc[w][4 * j + jp][lane];
  }
  __syncthreads();
  if (w < 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) L.s.acc[w][4 * j + jp][lane] = acc[j][jp];
  }
  __syncthreads();
  float* dst = ws + (bh * (nseg + 1) + seg) * slot_elems(FD);
  const f32x4* la = &L.s.acc[0][0][0];
  for (int e = tid; e < 16 * 64; e += 512) {
    f32x4 sm = la[e];
#pragma unroll
    for (int u = 1; u < 4; ++u) sm += la[u * 16 * 64 + e];
    const int b = e >> 6, l = e & 63, j = b >> 2, jp = b & 3, m4 = l & 15, kk = l >> 4;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) dst[(16 * kk + 4 * rr + j) * FD + 4 * m4 + jp] = sm[rr];
  }
  if (tid < 16) {
    f32x4 sm = L.s.z[0][tid];
#pragma unroll
    for (int u = 1; u < NW8; ++u) sm += L.s.z[u][tid];
    *reinterpret_cast<f32x4*>(dst + FD * FD + 4 * tid) = sm;
  }
}

// ----------------------------------------------------------------- k_decode
// One workgroup per (batch, key/value head): S += phi(k) (x) v, z += phi(k),
// then out_h = phi(q_h) S / (phi(q_h) . z) for the R query heads of the group.
// Thread t owns column b = t % 128 of rows a = t / 128 + 2u (u < 64) and keeps
// them in registers between the update and the reads.  The state goes
// through buffer instructions bounded to this head's d x d floats: entries
// outside the d x d square get an offset past the end, so their loads return
// zero and their stores are dropped, and the update runs without branches
// (a branch per element would make every store wait for the previous one).
template <typename T, int PM>
__global__ __launch_bounds__(NT) void k_decode(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, int d, int R, float* __restrict__ S,
                                               float* __restrict__ z, T* __restrict__ out) {
  constexpr int MD = la_internal::kMaxD;
  __shared__ float pk[MD], vv[MD], zn[MD];
  __shared__ float pq[MD];
  __shared__ float red[2][MD];
  __shared__ float sden;
  const int tid = threadIdx.x;
  const int64_t bg = blockIdx.x;  // b * Hkv + g
  float* Sg = S + bg * d * d;
  float* zg = z + bg * d;
  if (tid < MD) {
    // entries past d are zero so that padded rows and columns add nothing
    float pkv = 0.0f, vvv = 0.0f, znew = 0.0f;
    if (tid < d) {
      pkv = phi_m<PM>(to_f(k[bg * d + tid]));
      vvv = to_f(v[bg * d + tid]);
      znew = zg[tid] + pkv;
      zg[tid] = znew;
    }
    pk[tid] = pkv;
    vv[tid] = vvv;
    zn[tid] = znew;
  }
  __syncthreads();
  const int b = tid & 127, half = tid >> 7;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(Sg, 0, d * d * 4, 0x00020000);
  constexpr int OOB = 0x7FFFFFF0;  // past num_records for every d <= 128
  float s[64];
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const int a = half + 2 * u;
    const int off = (a < d && b < d) ? (a * d + b) * 4 : OOB;
    s[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
  const float vb = vv[b];
#pragma unroll
  for (int u = 0; u < 64; ++u) {
    const int a = half + 2 * u;
    const int off = (a < d && b < d) ? (a * d + b) * 4 : OOB;
    s[u] += pk[a] * vb;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s[u]), rs, off, 0, 0);
  }
  for (int r = 0; r < R; ++r) {
    const int64_t qh = bg * R + r;  // (b * Hkv + g) * R + r = b * Hq + g * R + r
    __syncthreads();                // previous head's reads of pq / red are done
    if (tid < MD) pq[tid] = tid < d ? phi_m<PM>(to_f(q[qh * d + tid])) : 0.0f;
    __syncthreads();
    if (tid < 64) {  // wave 0: den = phi(q) . z
      float p = pq[tid] * zn[tid] + pq[tid + 64] * zn[tid + 64];
      for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
      if (tid == 0) sden = p;
    }
    float num = 0.0f;
#pragma unroll
    for (int u = 0; u < 64; ++u) num += pq[half + 2 * u] * s[u];
    red[half][b] = num;
    __syncthreads();
    if (tid < d) out[qh * d + tid] = cvt<T>((red[0][tid] + red[1][tid]) / sden);
  }
}

// Same step for a power-of-two head dim D, with 16-byte state accesses:
// thread t owns columns 4 (t % (D/4)) .. +3 of rows t / (D/4) + (NT / (D/4)) j
// (bounded buffer instructions again, so rows past D need no branch); the
// per-head column sums are reduced across the threads that share columns
// through LDS.
template <typename T, int D, int PM>
__global__ __launch_bounds__(NT) void k_decode4(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, int R, float* __restrict__ S,
                                                float* __restrict__ z, T* __restrict__ out) {
  constexpr int CG = D / 4;                   // 4-column groups per row
  constexpr int RSTEP = NT / CG;              // row step between a thread's groups
  constexpr int NV = (D * CG + NT - 1) / NT;  // groups per thread
  __shared__ float pk[D], vv[D], zn[D], pq[D];
  __shared__ __attribute__((aligned(16))) float red[RSTEP][D];
  __shared__ float sden;
  const int tid = threadIdx.x;
  const int64_t bg = blockIdx.x;  // b * Hkv + g
  float* Sg = S + bg * D * D;
  float* zg = z + bg * D;
  if (tid < D) {
    const float pkv = phi_m<PM>(to_f(k[bg * D + tid]));
    pk[tid] = pkv;
    vv[tid] = to_f(v[bg * D + tid]);
    const float znew = zg[tid] + pkv;
    zg[tid] = znew;
    zn[tid] = znew;
  }
  __syncthreads();
  const int cg = tid % CG, r0 = tid / CG;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(Sg, 0, D * D * 4, 0x00020000);
  constexpr int OOB = 0x7FFFFFF0;  // past num_records: loads give zero, stores are dropped
  f32x4 s4[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int a = r0 + RSTEP * j;
    const int off = a < D ? (a * D + 4 * cg) * 4 : OOB;
    s4[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  const f32x4 vb = {vv[4 * cg], vv[4 * cg + 1], vv[4 * cg + 2], vv[4 * cg + 3]};
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int a = r0 + RSTEP * j;
    const float pa = a < D ? pk[a] : 0.0f;
    const int off = a < D ? (a * D + 4 * cg) * 4 : OOB;
    s4[j] += pa * vb;
    typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_, s4[j]), rs, off, 0, 0);
  }
  for (int r = 0; r < R; ++r) {
    const int64_t qh = bg * R + r;  // (b * Hkv + g) * R + r = b * Hq + g * R + r
    __syncthreads();                // previous head's reads of pq / red are done
    if (tid < D) pq[tid] = phi_m<PM>(to_f(q[qh * D + tid]));
    __syncthreads();
    if (tid < 64) {  // wave 0: den = phi(q) . z
      float p = (tid < D ? pq[tid] * zn[tid] : 0.0f) + (tid + 64 < D ? pq[tid + 64] * zn[tid + 64] : 0.0f);
      for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
      if (tid == 0) sden = p;
    }
    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int a = r0 + RSTEP * j;
      num += (a < D ? pq[a] : 0.0f) * s4[j];
    }
    *reinterpret_cast<f32x4*>(&red[r0][4 * cg]) = num;
    __syncthreads();
    if (tid < D) {
      float acc = 0.0f;
#pragma unroll 8
      for (int kk = 0; kk < RSTEP; ++kk) acc += red[kk][tid];
      out[qh * D + tid] = cvt<T>(acc / sden);
    }
  }
}

// The same step for D = 128 without LDS: wave w owns columns 32 w .. 32 w +
// 31 of the head's state (lane l: columns 32 w + 4 (l % 8) .. + 3 of rows
// l / 8 + 8 j, j < 16; a wave instruction covers eight whole 128-byte row
// pieces), so phi(q) S for those columns and the normaliser reduce within
// the wave by lane shuffles: no barrier per query head.  phi(q) of all R
// query heads of the group is staged in LDS (R * 512 bytes, dynamic) while
// the state loads are in flight, so no query load waits at the end.  One
// barrier only: it publishes phi(q), and every wave has read the old z
// before wave 0 writes the new one.
template <typename T, int PM>
__global__ __launch_bounds__(256) void k_decode128(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, int R, float* __restrict__ S,
                                                   float* __restrict__ z, T* __restrict__ out) {
  constexpr int D = 128, NJ = 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, cg = lane & 7, r0 = lane >> 3;
  const int64_t bg = blockIdx.x;  // b * Hkv + g
  const int col0 = 32 * w + 4 * cg;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(S + bg * D * D, 0, D * D * 4, 0x00020000);
  f32x4 s4[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    s4[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, ((r0 + 8 * j) * D + col0) * 4, 0, 0));
  float pk[NJ], zn[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    pk[j] = phi_m<PM>(to_f(k[bg * D + r0 + 8 * j]));
    zn[j] = z[bg * D + r0 + 8 * j] + pk[j];  // z after this step's key
  }
  const f32x4 vb = {to_f(v[bg * D + col0]), to_f(v[bg * D + col0 + 1]), to_f(v[bg * D + col0 + 2]),
                    to_f(v[bg * D + col0 + 3])};
  extern __shared__ float pqs[];  // [R][D]: phi(q) of the group's query heads
  const T* qg = q + bg * R * D;   // heads (b * Hkv + g) * R + r are contiguous
#pragma unroll 4
  for (int i = tid; i < R * D; i += 256) pqs[i] = phi_m<PM>(to_f(qg[i]));
  __syncthreads();  // phi(q) staged; every wave has read the old z
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (cg == 0) z[bg * D + r0 + 8 * j] = zn[j];
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    s4[j] += pk[j] * vb;
    typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_, s4[j]), rs, ((r0 + 8 * j) * D + col0) * 4, 0, 0);
  }
  for (int r = 0; r < R; ++r) {
    const int64_t qh = bg * R + r;  // (b * Hkv + g) * R + r = b * Hq + g * R + r
    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float pq = pqs[r * D + r0 + 8 * j];
      num += pq * s4[j];
      den = fmaf(pq, zn[j], den);
    }
    // sum over the eight row groups (lane bits 3..5)
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] += __shfl_xor(num[e], off);
      den += __shfl_xor(den, off);
    }
    if (r0 == 0) {
      const float inv = 1.0f / den;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[qh * D + col0 + e] = cvt<T>(num[e] * inv);
    }
  }
}

// ------------------------------------------------------------------ dispatch
// The causal form on the general kernels, for feature map PM: the state pass
// (k_state_tr for bf16 d = 128 chunk 32, k_state32 for fp32 d = 64, else
// k_state), the scan, then the output pass (k_out_gqa for two or four query
// heads per key/value head at bf16 d = 128 chunk 32; k_out_prefix32 with
// the chunks as buckets for fp32 d = 64 chunk 64 and one query head per
// key/value head; else k_out).  The specialised kernels walk F state
// segments per workgroup, so that about kGqaOutGroups / kPrefixOutGroups
// workgroups (one / two per CU) each walk a longer run of chunks.
template <typename T, int DP, int C, int PM>
int run_causal(const la_internal::Fwd& a, const la_internal::Plan& p) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const bool vec = (a.d == DP);
  const int64_t nbh = a.B * a.Hkv;
  float* states = reinterpret_cast<float*>(a.ws);
  const int R = (int)(a.Hq / a.Hkv);
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* out = reinterpret_cast<T*>(a.out);
  bool tr = false, s32 = false, px = false;
  if constexpr (std::is_same<T, bf16>::value && DP == 128 && C == 32) tr = vec;
  if constexpr (std::is_same<T, float>::value && DP == 64) s32 = vec && a.n <= la_internal::kFwd32MaxN;
  if constexpr (std::is_same<T, float>::value && DP == 64 && C == 64) px = vec && q && out && R == 1;
  const bool gq = tr && q && out && (R == 1 || R == 2 || R == 4 || R == 8);
  if (tr) {
    if constexpr (std::is_same<T, bf16>::value && DP == 128 && C == 32)
      k_state_tr<PM><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, p.nchunks, p.G, p.nseg, states);
  } else if (s32) {
    if constexpr (std::is_same<T, float>::value && DP == 64)
      k_state32<PM><<<dim3((unsigned)(nbh * p.nseg)), 512, 0, st>>>(k, v, a.n, p.nchunks, C, p.G, p.nseg, states,
                                                                    nullptr, nullptr, nullptr, 1, nullptr);
  } else {
    k_state<T, DP, C, PM><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, (int)a.d, vec, p.nchunks, p.G,
                                                                         p.nseg, states);
  }
  // output workgroups per CU: one of the eight-wave GQA kernel, two of the
  // four-wave one (R = 1) and of the prefix-form kernel
  int64_t F = gq ? nbh * p.nseg / (R == 1 ? 2 * kGqaOutGroups : kGqaOutGroups)
                 : px ? nbh * p.nseg / kPrefixOutGroups : 1;
  if (F < 1) F = 1;
  launch_k_scan(states, nbh, p.nseg, DP, (int)a.d, a.S_final, a.z_final, F, st);
  if (!(q && out)) return (int)hipGetLastError();
  const int64_t GO = p.G * F, nseg_o = (p.nchunks + GO - 1) / GO;
  if constexpr (std::is_same<T, bf16>::value && DP == 128 && C == 32) {
    if (gq) {
      const bf16* qq = reinterpret_cast<const bf16*>(q);
      if (R == 1)
        k_out_gqa<1, PM><<<dim3((unsigned)(nbh * nseg_o)), 256, 0, st>>>(qq, k, v, out, a.n, p.nchunks, GO, nseg_o,
                                                                         F, p.nseg, states);
      else if (R == 2)
        k_out_gqa<2, PM><<<dim3((unsigned)(nbh * nseg_o)), 512, 0, st>>>(qq, k, v, out, a.n, p.nchunks, GO, nseg_o,
                                                                         F, p.nseg, states);
      else if (R == 4)
        k_out_gqa<4, PM><<<dim3((unsigned)(nbh * nseg_o)), 512, 0, st>>>(qq, k, v, out, a.n, p.nchunks, GO, nseg_o,
                                                                         F, p.nseg, states);
      else
        k_out_gqa<8, PM><<<dim3((unsigned)(nbh * nseg_o)), 512, 0, st>>>(qq, k, v, out, a.n, p.nchunks, GO, nseg_o,
                                                                         F, p.nseg, states);
      return (int)hipGetLastError();
    }
  }
  if constexpr (std::is_same<T, float>::value && DP == 64 && C == 64) {
    if (px) {
      k_out_prefix32<PX_NWV, true, PM><<<dim3((unsigned)(nbh * nseg_o)), 64 * PX_NWV, 0, st>>>(
          q, k, v, out, a.n, p.nchunks, GO, nseg_o, F, p.nseg, states, nullptr, nullptr, nullptr, a.Hq, 1);
      return (int)hipGetLastError();
    }
  }
  k_out<T, DP, C, CAUSAL, PM><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(
      q, k, v, out, a.n, (int)a.d, R, vec, p.nchunks, p.G, p.nseg, states, nullptr, nullptr, nullptr, a.Hq, 1);
  return (int)hipGetLastError();
}

// The prefix-mask form (no feature map): the bucket sort (for fp32 d = 64 as
// extra workgroups of the k_state32 launch), the state pass, the scan, then
// k_out_prefix32 (fp32 d = 64 chunk 64) or k_out.
template <typename T, int DP, int C>
int run_prefix(const la_internal::Fwd& a, const la_internal::Plan& p) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const bool vec = (a.d == DP);
  const int64_t nbh = a.B * a.Hkv;
  float* states = reinterpret_cast<float*>(a.ws);
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* out = reinterpret_cast<T*>(a.out);
  char* bw = reinterpret_cast<char*>(a.ws) + la_internal::state_bytes(p, a.B, a.Hkv);
  int* boff = reinterpret_cast<int*>(bw);   // [nmask][nchunks + 1]
  int* perm = boff + a.nmask * (p.nchunks + 1);  // [nmask][n]
  bool state_done = false;
  if constexpr (std::is_same<T, float>::value && DP == 64) {
    if (vec && a.n <= la_internal::kFwd32MaxN) {  // the sort as one more workgroup of the state launch
      k_state32<PM_ID><<<dim3((unsigned)(nbh * p.nseg + a.nmask)), 512, 0, st>>>(k, v, a.n, p.nchunks, C, p.G,
                                                                                  p.nseg, states, a.m, boff, perm,
                                                                                  a.nmask, a.ctl);
      state_done = true;
    }
  }
  if (!state_done) {
    k_bucket<<<dim3((unsigned)a.nmask), 1024, 0, st>>>(a.m, a.n, C, p.nchunks, boff, perm, a.ctl);
    k_state<T, DP, C, PM_ID><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, (int)a.d, vec, p.nchunks,
                                                                            p.G, p.nseg, states);
  }
  bool px = false;
  if constexpr (std::is_same<T, float>::value && DP == 64 && C == 64) px = vec;
  int64_t F = px ? nbh * p.nseg / kPrefixOutGroups : 1;
  if (F < 1) F = 1;
  const int64_t GO = p.G * F, nseg_o = (p.nchunks + GO - 1) / GO;
  launch_k_scan(states, nbh, p.nseg, DP, (int)a.d, nullptr, nullptr, F, st);
  if constexpr (std::is_same<T, float>::value && DP == 64 && C == 64) {
    if (px) {
      k_out_prefix32<PX_NWV><<<dim3((unsigned)(nbh * nseg_o)), 64 * PX_NWV, 0, st>>>(
          q, k, v, out, a.n, p.nchunks, GO, nseg_o, F, p.nseg, states, perm, boff, a.m, a.Hq, a.nmask);
      return (int)hipGetLastError();
    }
  }
  k_out<T, DP, C, PREFIX, PM_ID><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(
      q, k, v, out, a.n, (int)a.d, 1, vec, p.nchunks, p.G, p.nseg, states, perm, boff, a.m, a.Hq, a.nmask);
  return (int)hipGetLastError();
}

template <typename T, int DP, int C>
int run_causal_or_prefix(const la_internal::Fwd& a, const la_internal::Plan& p, int form) {
  if (form == PREFIX) return run_prefix<T, DP, C>(a, p);
  if (a.phi == 2) return run_causal<T, DP, C, PM_FEAT>(a, p);
  if (a.phi == 1) return run_causal<T, DP, C, PM_ELU1>(a, p);
  return run_causal<T, DP, C, PM_RELU1>(a, p);
}

template <typename T, int DP, int C>
int run_forward(const la_internal::Fwd& a, const la_internal::Plan& p) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const bool vec = (a.d == DP);
  const int64_t nbh = a.B * a.Hkv;
  float* states = reinterpret_cast<float*>(a.ws);
  const int R = (int)(a.Hq / a.Hkv);
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  T* out = reinterpret_cast<T*>(a.out);
  const bool elu = a.phi == 1, feat = a.phi == 2;
  if (feat)
    k_state<T, DP, C, PM_FEAT><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, (int)a.d, vec, p.nchunks, p.G,
                                                                             p.nseg, states);
  else if (elu)
    k_state<T, DP, C, PM_ELU1><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, (int)a.d, vec, p.nchunks, p.G,
                                                                             p.nseg, states);
  else
    k_state<T, DP, C, PM_RELU1><<<dim3((unsigned)(nbh * p.nseg)), NT, 0, st>>>(k, v, a.n, (int)a.d, vec, p.nchunks, p.G,
                                                                              p.nseg, states);
  launch_k_scan(states, nbh, p.nseg, DP, (int)a.d, nullptr, nullptr, 1, st);
  // query runs: about 1024 workgroups in total for 2-byte inputs (several per
  // CU keep more query tiles in flight), about 256 for 4-byte inputs (longer
  // runs, each loading its next, twice as large, tile while it computes)
  const int64_t target = sizeof(T) == 2 ? 1024 : 256;
  int64_t Gq = (nbh * p.nchunks + target - 1) / target;
  if (Gq < 1) Gq = 1;
  const int64_t nqseg = (p.nchunks + Gq - 1) / Gq;
  if (feat)
    k_out_nc<T, DP, C, PM_FEAT><<<dim3((unsigned)(nbh * nqseg)), NT, 0, st>>>(q, out, a.n, (int)a.d, R, vec, p.nchunks,
                                                                             Gq, nqseg, p.nseg, states);
  else if (elu)
    k_out_nc<T, DP, C, PM_ELU1><<<dim3((unsigned)(nbh * nqseg)), NT, 0, st>>>(q, out, a.n, (int)a.d, R, vec, p.nchunks,
                                                                             Gq, nqseg, p.nseg, states);
  else
    k_out_nc<T, DP, C, PM_RELU1><<<dim3((unsigned)(nbh * nqseg)), NT, 0, st>>>(q, out, a.n, (int)a.d, R, vec, p.nchunks,
                                                                              Gq, nqseg, p.nseg, states);
  return (int)hipGetLastError();
}

// Instantiate for a (T, DP) pair and every chunk that fits in LDS.
template <typename T, int DP>
int dispatch_chunk(const la_internal::Fwd& a, const la_internal::Plan& p, int op) {
  switch (p.C) {
#define LA_CASE(CC)                                                                            \
  case CC:                                                                                     \
    if constexpr (la_internal::chunk_fits((int)sizeof(T), DP, CC)) {                           \
      if (op == 0) return run_forward<T, DP, CC>(a, p);                                        \
      return run_causal_or_prefix<T, DP, CC>(a, p, op == 1 ? CAUSAL : PREFIX);                  \
    }                                                                                          \
    break;
    LA_CASE(32)
    LA_CASE(64)
    LA_CASE(128)
#undef LA_CASE
  }
  return (int)hipErrorInvalidValue;
}

template <int DP>
int dispatch_dtype(const la_internal::Fwd& a, const la_internal::Plan& p, int op) {
  if (a.dtype == 0) return dispatch_chunk<float, DP>(a, p, op);
  return dispatch_chunk<bf16, DP>(a, p, op);
}

int dispatch(const la_internal::Fwd& a, const la_internal::Plan& p, int op) {
  switch (p.DP) {
    case 32: return dispatch_dtype<32>(a, p, op);
    case 64: return dispatch_dtype<64>(a, p, op);
    case 128: return dispatch_dtype<128>(a, p, op);
  }
  return (int)hipErrorInvalidValue;
}

// One decode step with feature map PM, dispatched on d and the dtype.
template <int PM>
int launch_decode_pm(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                     int dtype, float* S, float* z, void* out, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int R = (int)(Hq / Hkv);
  const dim3 grid((unsigned)(B * Hkv));
#define LA_DEC4_LAUNCH(DD)                                                                                    \
    if (dtype == 0)                                                                                           \
      k_decode4<float, DD, PM><<<grid, NT, 0, st>>>(reinterpret_cast<const float*>(q),                        \
                                                    reinterpret_cast<const float*>(k),                        \
                                                    reinterpret_cast<const float*>(v), R, S, z,               \
                                                    reinterpret_cast<float*>(out));                           \
    else                                                                                                      \
      k_decode4<bf16, DD, PM><<<grid, NT, 0, st>>>(reinterpret_cast<const bf16*>(q),                          \
                                                   reinterpret_cast<const bf16*>(k),                          \
                                                   reinterpret_cast<const bf16*>(v), R, S, z,                 \
                                                   reinterpret_cast<bf16*>(out));                             \
    return (int)hipGetLastError();
#define LA_DEC4(DD) \
  case DD:          \
    LA_DEC4_LAUNCH(DD)
  constexpr int kDec128MaxR = 64;  // phi(q) staging of at most 32 KB of LDS
  switch (d) {
    LA_DEC4(4)
    LA_DEC4(8)
    LA_DEC4(16)
    LA_DEC4(32)
    LA_DEC4(64)
  case 128:
    if (R > kDec128MaxR) {
      LA_DEC4_LAUNCH(128)
    }
    if (dtype == 0)
      k_decode128<float, PM><<<grid, 256, R * 128 * 4, st>>>(reinterpret_cast<const float*>(q),
                                                             reinterpret_cast<const float*>(k),
                                                             reinterpret_cast<const float*>(v), R, S, z,
                                                             reinterpret_cast<float*>(out));
    else
      k_decode128<bf16, PM><<<grid, 256, R * 128 * 4, st>>>(reinterpret_cast<const bf16*>(q),
                                                            reinterpret_cast<const bf16*>(k),
                                                            reinterpret_cast<const bf16*>(v), R, S, z,
                                                            reinterpret_cast<bf16*>(out));
    return (int)hipGetLastError();
    default:
      break;
  }
#undef LA_DEC4
#undef LA_DEC4_LAUNCH
  if (dtype == 0)
    k_decode<float, PM><<<grid, NT, 0, st>>>(reinterpret_cast<const float*>(q), reinterpret_cast<const float*>(k),
                                             reinterpret_cast<const float*>(v), (int)d, R, S, z,
                                             reinterpret_cast<float*>(out));
  else
    k_decode<bf16, PM><<<grid, NT, 0, st>>>(reinterpret_cast<const bf16*>(q), reinterpret_cast<const bf16*>(k),
                                            reinterpret_cast<const bf16*>(v), (int)d, R, S, z,
                                            reinterpret_cast<bf16*>(out));
  return (int)hipGetLastError();
}

}  // namespace

namespace la_internal {

int launch_forward(const Fwd& a, const Plan& p) { return dispatch(a, p, 0); }
int launch_causal(const Fwd& a, const Plan& p) { return dispatch(a, p, 1); }
int launch_prefix(const Fwd& a, const Plan& p) { return dispatch(a, p, 2); }

int launch_scan(float* ws, int64_t nunits, int64_t nseg, int DP, int d, float* S_final, float* z_final,
                void* stream) {
  launch_k_scan(ws, nunits, nseg, DP, d, S_final, z_final, 1, reinterpret_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

int launch_state_bf16_exact(const void* k, const void* v, int64_t units, int64_t n, int d, int phi, int C,
                            int64_t nchunks, int64_t G, int64_t nseg, float* ws, void* stream) {
  if (d != 64 || C != 32 || phi == 1) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bf16* kk = reinterpret_cast<const bf16*>(k);
  const bf16* vv = reinterpret_cast<const bf16*>(v);
  const dim3 grid((unsigned)(units * nseg));
  if (phi == 2)
    k_state<bf16, 64, 32, PM_FEAT><<<grid, NT, 0, st>>>(kk, vv, n, d, true, nchunks, G, nseg, ws);
  else
    k_state<bf16, 64, 32, PM_RELU1><<<grid, NT, 0, st>>>(kk, vv, n, d, true, nchunks, G, nseg, ws);
  return (int)hipGetLastError();
}

int launch_decode(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                  int dtype, int phi, float* S, float* z, void* out, void* stream) {
  if (phi == 2) return launch_decode_pm<PM_FEAT>(q, k, v, B, Hq, Hkv, d, dtype, S, z, out, stream);
  return phi == 1 ? launch_decode_pm<PM_ELU1>(q, k, v, B, Hq, Hkv, d, dtype, S, z, out, stream)
                  : launch_decode_pm<PM_RELU1>(q, k, v, B, Hq, Hkv, d, dtype, S, z, out, stream);
}

}  // namespace la_internal
