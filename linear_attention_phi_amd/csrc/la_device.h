// la_device.h -- device-side building blocks shared by the gfx950 kernels:
// element conversions, the feature map, MFMA fragments and tile loads.
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16 for bf16, v_mfma_f32_32x32x2_f32
// for fp32).  Every operand matrix lives in LDS row-major with the
// *non-contracted* index as the row and the contracted index k contiguous.
// For a 32x32 product block and a 16-wide k block kb, lane l (row r = l % 32,
// half h = l / 32) reads the 8 values at k = 16kb + 4h + {0..3} and
// 16kb + 8 + 4h + {0..3}.  A and B use this same k assignment, which is all a
// contraction needs.  The accumulator of a block with rows m and columns n
// holds, in lane l, column n = l % 32 and rows m = 8q + 4h + s in register
// 4q + s.  So registers 8kb .. 8kb+7 of an accumulator are exactly the
// operand fragment, for k block kb, of the matrix whose k index is m: an
// accumulator can feed the next product without leaving registers, and
// written back "transposed" (row n, four contiguous m per q) it is readable
// from LDS as such an operand.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la_dev {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NT = 256;  // threads per workgroup
constexpr int NW = 4;    // waves per workgroup
constexpr int PAD = 4;   // LDS row padding (elements): 8-byte (bf16) / 16-byte
                         // (fp32) fragment reads of 32 rows hit distinct banks

enum Form { CAUSAL = 0, PREFIX = 1 };

__device__ __forceinline__ float phi_f(float x) { return fmaxf(x, 0.0f) + 1.0f; }
// The feature maps a call can take: the identity (the prefix form),
// relu(x) + 1 (nx_f32_linear_attention.nx, function la_phi), ELU(x) + 1
// with alpha = 1 (LinearTile 1.0.1, "How It Works"): x + 1 for x > 0, e^x
// otherwise, and caller-applied features (PM_FEAT: Q and K already hold
// phi(Q) and phi(K) for a positive map of the caller's choice, LinearTile
// 1.0.1, "Features": a replaceable phi): the normalised forms with the
// identity on Q and K, z summed over K as given.
enum PhiMode { PM_ID = 0, PM_RELU1 = 1, PM_ELU1 = 2, PM_FEAT = 3 };
// e^x as the hardware exp2 of x log2(e): a few fp32 ulp for the arguments
// here (x <= 0), far inside every tolerance, and several times cheaper than
// the correctly rounded expf in the tile transforms
__device__ __forceinline__ float elu1_f(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }
template <int PM> __device__ __forceinline__ float phi_m(float x) {
  return PM == PM_ELU1 ? elu1_f(x) : PM == PM_FEAT ? x : phi_f(x);
}
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T cvt(float x);
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 cvt<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------- fragments
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void ld_frag(Frag<bf16>& f, const bf16* p) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void ld_frag(Frag<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 8);
}
__device__ __forceinline__ void mma(f32x16& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[u], b.lo[u], acc, 0, 0, 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[u], b.hi[u], acc, 0, 0, 0);
}

// acc[m][n] += sum_k A[m][k] B[n][k] over NKB k-blocks of 16, with A and B
// pointing at row 0 / column k0 of their 32-row blocks in LDS.
template <typename T, int NKB>
__device__ __forceinline__ void gemm_acc(f32x16& acc, const T* A, int lda, const T* B, int ldb, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const T* pa = A + r * lda + 4 * h;
  const T* pb = B + r * ldb + 4 * h;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    Frag<T> fa, fb;
    ld_frag(fa, pa + 16 * kb);
    ld_frag(fb, pb + 16 * kb);
    mma(acc, fa, fb);
  }
}

// Write an accumulator block (rows m, columns n) to X[n][m] in LDS, rounded to T.
__device__ __forceinline__ void st_accT(bf16* X, int ldx, const f32x16& acc, int lane) {
  const int n = lane & 31, h = lane >> 5;
  bf16* p = X + n * ldx + 4 * h;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bf16x4 t = {(bf16)acc[4 * q], (bf16)acc[4 * q + 1], (bf16)acc[4 * q + 2], (bf16)acc[4 * q + 3]};
    *reinterpret_cast<bf16x4*>(p + 8 * q) = t;
  }
}
__device__ __forceinline__ void st_accT(float* X, int ldx, const f32x16& acc, int lane) {
  const int n = lane & 31, h = lane >> 5;
  float* p = X + n * ldx + 4 * h;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 t = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    *reinterpret_cast<f32x4*>(p + 8 * q) = t;
  }
}

// ---------------------------------------------------------------- tile loads
// What a tile copy holds: not written, the raw value, phi(x) = relu(x) + 1,
// relu(x), or ELU(x) + 1.
enum Xf { XF_NONE = 0, XF_ID = 1, XF_PHI = 2, XF_RELU = 3, XF_ELU1 = 4 };

// The tile transforms of a feature map: on Q (phi), and on the keys of the
// state (relu(K) with the relu + 1 split, phi(K) otherwise)
template <int PM> constexpr int q_xform() {
  return PM == PM_RELU1 ? XF_PHI : PM == PM_ELU1 ? XF_ELU1 : XF_ID;
}
template <int PM> constexpr int k_xform() {
  return PM == PM_RELU1 ? XF_RELU : PM == PM_ELU1 ? XF_ELU1 : XF_ID;
}

template <int X> __device__ __forceinline__ float xform(float x) {
  if (X == XF_PHI) return phi_f(x);
  if (X == XF_RELU) return fmaxf(x, 0.0f);
  if (X == XF_ELU1) return elu1_f(x);
  return x;
}

// Load C rows x DP features of one head (base = row 0 of the head, row stride
// d) into LDS: tm[row][col] (token-major, stride DP+PAD) transformed by TMX,
// and/or fm[col][row] (feature-major, stride C+PAD) transformed by FMX.  Row r
// of the tile is global row (gidx ? gidx[r] : row0 + r) and exists for
// r < nvalid.  Missing rows and the padding features col >= d are stored as
// 0 -- NOT phi(0) = 1 -- so that they add nothing to any sum.
// vec: d == DP, 16-byte pieces (base and row stride are 16-byte aligned).
template <typename T, int DP, int C, int TMX, int FMX>
__device__ __forceinline__ void load_tile(const T* __restrict__ base, int64_t row0, const int* __restrict__ gidx,
                                          int nvalid, int d, bool vec, T* tm, T* fm, int tid) {
  if (vec) {
    // every piece this thread owns is requested before any is used
    constexpr int EPP = 16 / (int)sizeof(T);
    constexpr int PPR = DP / EPP;
    constexpr int NP = C * PPR;
    constexpr int PER = (NP + NT - 1) / NT;
    union V { uint4 u; T e[EPP]; };
    V raw[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int p = tid + k * NT;
      raw[k].u = make_uint4(0, 0, 0, 0);
      const int row = p / PPR, col = (p % PPR) * EPP;
      if (p < NP && row < nvalid) {
        const int64_t grow = gidx ? (int64_t)gidx[row] : row0 + row;
        raw[k].u = *reinterpret_cast<const uint4*>(base + grow * DP + col);
      }
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
        T* dst = tm + row * (DP + PAD) + col;
        if (sizeof(T) == 4) {
          *reinterpret_cast<uint4*>(dst) = a.u;
        } else {  // rows of DP+PAD bf16 are only 8-byte aligned
          reinterpret_cast<uint2*>(dst)[0] = make_uint2(a.u.x, a.u.y);
          reinterpret_cast<uint2*>(dst)[1] = make_uint2(a.u.z, a.u.w);
        }
      }
      if (FMX != XF_NONE) {
#pragma unroll
        for (int e = 0; e < EPP; ++e) fm[(col + e) * (C + PAD) + row] = b.e[e];
      }
    }
  } else {
    for (int idx = tid; idx < C * DP; idx += NT) {
      const int row = idx / DP, col = idx % DP;
      float x = 0.0f;
      const bool ok = row < nvalid && col < d;
      if (ok) {
        const int64_t grow = gidx ? (int64_t)gidx[row] : row0 + row;
        x = to_f(base[grow * d + col]);
      }
      if (TMX != XF_NONE) tm[row * (DP + PAD) + col] = cvt<T>(ok ? xform<TMX>(x) : 0.0f);
      if (FMX != XF_NONE) fm[col * (C + PAD) + row] = cvt<T>(ok ? xform<FMX>(x) : 0.0f);
    }
  }
}

// A tile's raw 16-byte pieces held in registers between their global loads
// (tile_fetch) and their transform into LDS (tile_store), so that the loads
// of the next tile can be in flight while the current one is used.  Only for
// d == DP (whole 16-byte pieces); rows at or past nvalid are zero.
template <typename T, int DP, int C>
struct TileRaw {
  static constexpr int EPP = 16 / (int)sizeof(T);
  static constexpr int PPR = DP / EPP;
  static constexpr int NP = C * PPR;
  static constexpr int PER = (NP + NT - 1) / NT;
  uint4 u[PER];
};

template <typename T, int DP, int C>
__device__ __forceinline__ void tile_fetch(TileRaw<T, DP, C>& t, const T* __restrict__ base, int64_t row0,
                                           const int* __restrict__ gidx, int nvalid, int tid) {
  using TR = TileRaw<T, DP, C>;
#pragma unroll
  for (int k = 0; k < TR::PER; ++k) {
    const int p = tid + k * NT;
    const int row = p / TR::PPR, col = (p % TR::PPR) * TR::EPP;
    t.u[k] = make_uint4(0, 0, 0, 0);
    if (p < TR::NP && row < nvalid) {
      const int64_t grow = gidx ? (int64_t)gidx[row] : row0 + row;
      t.u[k] = *reinterpret_cast<const uint4*>(base + grow * DP + col);
    }
  }
}

template <typename T, int DP, int C, int TMX, int FMX>
__device__ __forceinline__ void tile_store(const TileRaw<T, DP, C>& t, int nvalid, T* tm, T* fm, int tid) {
  using TR = TileRaw<T, DP, C>;
#pragma unroll
  for (int k = 0; k < TR::PER; ++k) {
    const int p = tid + k * NT;
    if (p >= TR::NP) break;
    const int row = p / TR::PPR, col = (p % TR::PPR) * TR::EPP;
    union V { uint4 u; T e[TR::EPP]; };
    V raw, a, b;
    raw.u = t.u[k];
#pragma unroll
    for (int e = 0; e < TR::EPP; ++e) {
      const float x = to_f(raw.e[e]);
      a.e[e] = row < nvalid ? cvt<T>(xform<TMX>(x)) : cvt<T>(0.0f);
      b.e[e] = row < nvalid ? cvt<T>(xform<FMX>(x)) : cvt<T>(0.0f);
    }
    if (TMX != XF_NONE) {
      T* dst = tm + row * (DP + PAD) + col;
      if (sizeof(T) == 4) {
        *reinterpret_cast<uint4*>(dst) = a.u;
      } else {  // rows of DP+PAD bf16 are only 8-byte aligned
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(a.u.x, a.u.y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(a.u.z, a.u.w);
      }
    }
    if (FMX != XF_NONE) {
#pragma unroll
      for (int e = 0; e < TR::EPP; ++e) fm[(col + e) * (C + PAD) + row] = b.e[e];
    }
  }
}

// The 16-byte row pieces of one ROWS x DP tile that thread tid owns, held
// in registers between stage_load (the requests) and stage_put (the LDS
// writes), so that a walk can request the next chunk's rows before it works
// on the current one.
template <typename T, int DP, int ROWS>
struct StageRegs {
  static constexpr int EPP = 16 / (int)sizeof(T);
  static constexpr int PPR = DP / EPP;
  static constexpr int NP = ROWS * PPR;
  static constexpr int PER = (NP + NT - 1) / NT;
  uint4 u[PER];
};

// Request the tile's rows row0 .. row0 + nvalid - 1 (16-byte pieces; rows
// past nvalid read as zero).  Without vec nothing is requested here: the
// element path of stage_put loads as it writes.
template <typename T, int DP, int ROWS>
__device__ __forceinline__ void stage_load(StageRegs<T, DP, ROWS>& R, const T* __restrict__ base, int64_t ld,
                                           int64_t row0, int nvalid, bool vec, int tid) {
  using SR = StageRegs<T, DP, ROWS>;
  if (!vec) return;
#pragma unroll
  for (int k = 0; k < SR::PER; ++k) {
    const int p = tid + k * NT;
    const int row = p / SR::PPR, col = (p % SR::PPR) * SR::EPP;
    R.u[k] = make_uint4(0, 0, 0, 0);
    if (p < SR::NP && row < nvalid) R.u[k] = *reinterpret_cast<const uint4*>(base + (row0 + row) * ld + col);
  }
}

// Write the tile requested by stage_load (same arguments) into LDS, as stage
// (below) describes.
template <typename T, typename TT, int DP, int ROWS, int TMX, int FMX>
__device__ __forceinline__ void stage_put(const StageRegs<T, DP, ROWS>& R, const T* __restrict__ base, int64_t ld,
                                          int64_t row0, int nvalid, int d, bool vec, TT* tm, int ldt, TT* fm,
                                          int ldf, int tid) {
  using SR = StageRegs<T, DP, ROWS>;
  if (vec) {
    constexpr int EPP = SR::EPP, PPR = SR::PPR, NP = SR::NP;
    constexpr int PIECES = EPP * (int)sizeof(TT) / 8;  // 8-byte stores per row piece of the tile
    union V { uint4 u; T e[EPP]; };
    union W { uint2 u[PIECES]; TT e[EPP]; };
#pragma unroll
    for (int k = 0; k < SR::PER; ++k) {
      const int p = tid + k * NT;
      if (p >= NP) break;
      const int row = p / PPR, col = (p % PPR) * EPP;
      V raw;
      raw.u = R.u[k];
      W a, b;
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const float x = to_f(raw.e[e]);
        a.e[e] = row < nvalid ? cvt<TT>(xform<TMX>(x)) : cvt<TT>(0.0f);
        b.e[e] = row < nvalid ? cvt<TT>(xform<FMX>(x)) : cvt<TT>(0.0f);
      }
      if (TMX != XF_NONE) {
        uint2* dst = reinterpret_cast<uint2*>(tm + row * ldt + col);  // rows of ldt elements are 8-byte aligned
#pragma unroll
        for (int q = 0; q < PIECES; ++q) dst[q] = a.u[q];
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
      const float x = ok ? to_f(base[(row0 + row) * ld + col]) : 0.0f;
      if (TMX != XF_NONE) tm[row * ldt + col] = cvt<TT>(ok ? xform<TMX>(x) : 0.0f);
      if (FMX != XF_NONE) fm[col * ldf + row] = cvt<TT>(ok ? xform<FMX>(x) : 0.0f);
    }
  }
}

// Copy ROWS rows x DP features of T (row stride ld elements, row0 first)
// into LDS tiles of TT: tm[row * ldt + col] transformed by TMX and/or
// fm[col * ldf + row] transformed by FMX.  Rows at or past nvalid and
// features at or past d are stored as 0 (not phi(0)).  vec: d == DP and
// 16-byte rows, 16-byte pieces.  TT may be wider than T (bf16 rows widened
// exactly into fp32 tiles).
template <typename T, typename TT, int DP, int ROWS, int TMX, int FMX>
__device__ __forceinline__ void stage(const T* __restrict__ base, int64_t ld, int64_t row0, int nvalid, int d,
                                      bool vec, TT* tm, int ldt, TT* fm, int ldf, int tid) {
  StageRegs<T, DP, ROWS> R;
  stage_load<T, DP, ROWS>(R, base, ld, row0, nvalid, vec, tid);
  stage_put<T, TT, DP, ROWS, TMX, FMX>(R, base, ld, row0, nvalid, d, vec, tm, ldt, fm, ldf, tid);
}

// Rows of chunk x of a sequence of n tokens (0 for x < 0 or past the end).
__device__ __forceinline__ int chunk_rows(int64_t x, int C, int64_t n) {
  if (x < 0) return 0;
  const int64_t r = n - x * C;
  return r <= 0 ? 0 : (r < C ? (int)r : C);
}

// Write an accumulator block (rows m, columns n) to X[m][n] in LDS, rounded
// to T (not transposed: 16 element stores per lane).
template <typename T>
__device__ __forceinline__ void st_acc(T* X, int ldx, const f32x16& acc, int lane) {
  const int n = lane & 31, h = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) X[(8 * (r >> 2) + 4 * h + (r & 3)) * ldx + n] = cvt<T>(acc[r]);
}

// Sum of the C entries of LDS row r (stride C+PAD), in order.
template <typename T, int C>
__device__ __forceinline__ float row_sum(const T* X, int r) {
  float sum = 0.0f;
  for (int t = 0; t < C; ++t) sum += to_f(X[r * (C + PAD) + t]);
  return sum;
}

// Number of 32x32 state blocks (a-block, b-block) each wave owns.
template <int DP> struct StateBlocks {
  static constexpr int NB = DP / 32;
  static constexpr int TOTAL = NB * NB;
  static constexpr int PER_WAVE = (TOTAL + NW - 1) / NW;
};

// Accumulator block <-> fp32 [DP][DP] row-major state in global memory.
template <int DP>
__device__ __forceinline__ void ld_state_block(f32x16& acc, const float* __restrict__ S, int ma, int nb, int lane) {
  const int b = nb * 32 + (lane & 31), h = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = S[(ma * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * DP + b];
}
template <int DP>
__device__ __forceinline__ void st_state_block(float* __restrict__ S, const f32x16& acc, int ma, int nb, int lane) {
  const int b = nb * 32 + (lane & 31), h = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) S[(ma * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * DP + b] = acc[r];
}

// acc[a][b] += add (lane's column b) for the rows a < d of block row ma.
__device__ __forceinline__ void add_col(f32x16& acc, float add, int ma, int d, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (ma * 32 + 8 * (r >> 2) + 4 * h + (r & 3) < d) acc[r] += add;
}

// Per-head slot layout of the state workspace: (nseg + 1) slots of
// DP*DP + DP floats (S row-major [a][b], then z[a]); slot s < nseg holds the
// aggregate of segment s (after k_scan: the exclusive prefix before segment
// s); slot nseg holds the total.
__host__ __device__ __forceinline__ int64_t slot_elems(int DP) { return (int64_t)DP * DP + DP; }


}  // namespace la_dev
