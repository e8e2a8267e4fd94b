// la_bf16.h -- device helpers of the bf16, d = 64 kernels (la_fused.hip,
// la_forward_bf16.hip): packed bf16 arithmetic, MFMA operand fragments read
// from LDS (16-byte reads over the feature index; ds_read_b64_tr_b16
// transposed reads over the token index), and buffer accesses with explicit
// cache policies.
//
// ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane k reads 4
// elements at its address; lane i receives element e of lane 4 e + i / 4's
// read, at position i % 4.  With lane k addressing row r0 + k / 4, column
// c0 + 4 (k % 4) of a row-major tile, lane i gets rows r0 .. r0 + 3 of
// column c0 + i (checked on the GPU with an in-bounds probe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_device.h"

namespace la_bf16 {

using namespace la_dev;

typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const bf16x2 t = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, t);
}
__device__ __forceinline__ float lo_f(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_f(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }
// relu of two packed bf16 values: as 16-bit integers, max(x, 0) keeps every
// value whose sign bit is clear and sends the others (including -0) to +0
__device__ __forceinline__ uint32_t relu2(uint32_t x) {
  const s16x2 z = {0, 0};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, x), z));
}
// phi = relu + 1 of two packed bf16 values, rounded to nearest-even bf16
__device__ __forceinline__ uint32_t phi2(uint32_t x) {
  const uint32_t r = relu2(x);
  return pack2(lo_f(r) + 1.0f, hi_f(r) + 1.0f);
}
// phi = ELU + 1 (alpha = 1) of two packed bf16 values: x + 1 for x > 0, e^x
// otherwise, rounded to nearest-even bf16 (e^x by the hardware exp2 of
// x log2(e), a few ulp of fp32 below the bf16 rounding)
__device__ __forceinline__ float elu1f(float x) { return x > 0.0f ? x + 1.0f : __expf(x); }
__device__ __forceinline__ uint32_t elu2(uint32_t x) { return pack2(elu1f(lo_f(x)), elu1f(hi_f(x))); }
// The non-split feature map of two packed bf16 values: ELU + 1, or the
// identity for caller-applied features
template <int PM> __device__ __forceinline__ uint32_t map2(uint32_t x) { return PM == PM_FEAT ? x : elu2(x); }
// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs, accumulated in fp32
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ uint32_t pair(const Frag<bf16>& f, int p) {
  return __builtin_bit_cast(u32x4, f.v)[p];
}
constexpr uint32_t ONE2 = 0x3F803F80u;  // two bf16 ones

// 16 contiguous bf16 bytes: an operand fragment over the feature index.
__device__ __forceinline__ Frag<bf16> ld16(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
// Operand fragment over the token index from a token-major tile: lane l
// (row index r = l % 32, half h = l / 32) gets column c0 + r of rows
// t0 + 4 h + {0..3} and t0 + 8 + 4 h + {0..3}, where c0 is the 32-column
// block; two transposed reads.  RS: the tile's row stride in elements.
template <int RS>
__device__ __forceinline__ Frag<bf16> ld_tr(const bf16* tile, int t0, int c0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const bf16* p = tile + (t0 + 4 * (g >> 1) + (i >> 2)) * RS + c0 + 16 * (g & 1) + 4 * (i & 3);
  const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
  const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 8 * RS));
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
// Accumulator registers 8 half .. 8 half + 7 as an operand fragment over the
// accumulator's row index (token order of ld_tr).
__device__ __forceinline__ Frag<bf16> acc_frag(const f32x16& acc, int half) {
  u32x4 u;
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = pack2(acc[8 * half + 2 * j], acc[8 * half + 2 * j + 1]);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}
// Waits for this wave's LDS operations, so that lanes read what other lanes
// of the wave wrote (a wave's LDS accesses complete in order).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Cross-workgroup data (segment aggregates) is written and read with
// device-scope (sc1) buffer accesses, which gfx950 performs at the device
// coherence point, so no L2 writeback or invalidate is needed.  Order: each
// wave waits for its aggregate stores to complete (s_waitcnt vmcnt(0)) before
// the workgroup barrier; only then does one thread store the flag (an
// agent-scope atomic).  A reader observes the flag, passes a barrier, and only
// then issues its sc1 aggregate loads.
constexpr int CPOL_SC1 = 16;  // cache-policy bit of buffer instructions: device scope (memory)
constexpr int CPOL_NT = 2;    // cache-policy bit: non-temporal (streamed through the caches)

template <int CPOL>
__device__ __forceinline__ void st_buf(__amdgpu_buffer_rsrc_t rs, int byte_off, f32x4v x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, byte_off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ void st_buf1(__amdgpu_buffer_rsrc_t rs, int byte_off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rs, byte_off, 0, CPOL);
}
template <int CPOL>
__device__ __forceinline__ f32x4v ld_buf(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(f32x4v, __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off, 0, CPOL));
}
template <int CPOL>
__device__ __forceinline__ float ld_buf1(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, CPOL));
}
// Write z values held one per lane (feature a = lane) into (high, low) bf16
// pair arrays: even lanes pair with their right neighbour.  All 64 lanes call.
__device__ __forceinline__ void store_z_pairs(uint32_t* zh, uint32_t* zl, float z, int a) {
  const float zn = __shfl_down(z, 1);
  if ((a & 1) == 0) {
    const uint32_t hi = pack2(z, zn);
    zh[a >> 1] = hi;
    zl[a >> 1] = pack2(z - lo_f(hi), zn - hi_f(hi));
  }
}

}  // namespace la_bf16
