// la_internal.h -- interface between the host-only API layer (la_api.cpp:
// argument checks, workspace sizing) and the HIP launchers (la_kernels.hip).
// No HIP type appears here, so the API layer builds without HIP headers.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace la_internal {

constexpr int kMaxD = 128;

// Feature dimension padded to the 32-wide MFMA tile.
inline int padded_dim(int64_t d) { return d <= 32 ? 32 : (d <= 64 ? 64 : 128); }

// Static LDS bytes of the chunk kernel (k_out) for (element bytes, padded
// dim, chunk): sQ and sK [C][DP+4], sKT and sVT [DP][C+4], sST [DP][DP+4],
// sP [C][C+4] in the element type, plus two [DP] fp32 vectors.  A (dtype,
// chunk) pair is offered only when this fits in one CU's 160 KiB of LDS.
constexpr size_t chunk_lds_bytes(int eb, int DP, int C) {
  return (size_t)eb * (2 * C * (DP + 4) + 2 * DP * (C + 4) + DP * (DP + 4) + C * (C + 4) + 3 * (DP + 16) + 16) +
         8 * (size_t)DP;
}
constexpr size_t kLdsLimit = 160 * 1024;
constexpr bool chunk_fits(int eb, int DP, int C) { return chunk_lds_bytes(eb, DP, C) <= kLdsLimit; }
int default_chunk(int elem_bytes, int DP);

// The prefix form sorts queries into ceil(n / C) buckets held in LDS.
constexpr int64_t kMaxBuckets = 16383;

// How a causal / prefix / non-causal pass splits each head's chunks into
// segments (one workgroup per segment and head).
struct Plan {
  int DP;        // padded feature dim
  int C;         // chunk length
  int64_t nchunks;
  int64_t G;     // chunks per segment
  int64_t nseg;  // segments per head
};
Plan make_plan(int op, int64_t B, int64_t Hkv, int64_t n, int64_t d, int elem_bytes, int chunk);

// Workspace layout (bytes) for a plan.
size_t state_bytes(const Plan& p, int64_t B, int64_t Hkv);  // fp32 segment states
size_t bucket_bytes(int64_t n, int C);                        // prefix-mask bucketing

struct Fwd {
  const void* q; const void* k; const void* v; void* out;
  int64_t B, Hq, Hkv, n, d;
  int dtype;
  const int64_t* m;      // prefix form only
  float* S_final; float* z_final;
  void* ws;
  void* stream;
  int phi = 0;           // feature map of the normalised forms: 0 relu + 1, 1 ELU + 1
  int64_t nmask = 1;     // prefix form: masks in m (1: shared [n]; B: one per batch, [B][n])
};

// Each returns 0 on success, else a nonzero HIP error code.
int launch_forward(const Fwd& a, const Plan& p);
int launch_causal(const Fwd& a, const Plan& p);
int launch_prefix(const Fwd& a, const Plan& p);
// Single-launch causal kernel (la_fused.hip): bf16, d = 64, chunk 64,
// Hq == Hkv, outputs requested.  Segments hold kFusedG chunks.
constexpr int kFusedG = 8;
constexpr int64_t kFusedMaxN = 131072;  // up to 256 segments per head
bool fused_causal_applies(int64_t Hq, int64_t Hkv, int64_t n, int64_t d, int dtype, int chunk);
size_t fused_causal_ws_bytes(int64_t NH, int64_t nseg);
int launch_causal_fused(const Fwd& a, const Plan& p, uint64_t epoch);

// Non-causal path for bf16, d = 64 (la_forward_bf16.hip): one launch; state
// partials per segment of kFwdSegChunks chunks, a reduce, then the output
// pass, ordered by flags that carry the call's epoch.
constexpr int kFwdSegChunks = 4;
// n bound: one head's rows, padded to a whole segment, stay below 2^31 bytes
// (the range of a buffer resource's record count and offsets).
constexpr int64_t kFwdMaxN = (int64_t)1 << 23;
bool forward_bf16_applies(int64_t n, int64_t d, int dtype);
int64_t forward_bf16_nseg(int64_t n);
size_t forward_bf16_ws_bytes(int64_t NKV, int64_t nseg);
int64_t forward_bf16_grid(int64_t NKV, int64_t NQ, int64_t n);
int launch_forward_bf16(const Fwd& a, uint64_t epoch);

// Non-causal path for fp32, d = 64 (la_forward_f32.hip): state partials per
// segment of kFwd32SegTokens keys, a reduce, then the output pass.
constexpr int kFwd32SegTokens = 256;
constexpr int64_t kFwd32MaxN = (int64_t)1 << 22;  // as kFwdMaxN, for 4-byte elements
bool forward_f32_applies(int64_t n, int64_t d, int dtype);
int64_t forward_f32_nseg(int64_t n);
size_t forward_f32_ws_bytes(int64_t NKV, int64_t nseg);
int launch_forward_f32(const Fwd& a);

int launch_decode(const void* q, const void* k, const void* v, int64_t B,
                  int64_t Hq, int64_t Hkv, int64_t d, int dtype, int phi,
                  float* S, float* z, void* out, void* stream);

}  // namespace la_internal
