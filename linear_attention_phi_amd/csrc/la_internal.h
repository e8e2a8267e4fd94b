// la_internal.h -- interface between the host-only API layer (la_api.cpp:
// argument checks, workspace sizing) and the HIP launchers (la_kernels.hip).
// No HIP type appears here, so the API layer builds without HIP headers.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace la_internal {

constexpr int kMaxD = 128;

// Control block: the first kCtlBytes of every workspace (the data regions
// follow it).  It must hold zeros before the first call that uses the
// workspace; every call leaves it valid for the next one on the same stream.
//   gen         epoch of the last call whose workgroups were ordered by
//               flags; a call's flags carry the next epoch, so that flags a
//               previous call (or a replay of the same captured launch) left
//               behind never match
//   arrive      workgroups of the running call that have taken their epoch;
//               the last one stores the new gen and resets it to 0
//   err         sticky error bits, read and cleared by la_workspace_status
//   wait_limit  polls before a bounded wait gives up (0: kDefaultWaitLimit)
//   wait_skew   added to the epoch that waits expect: 0, except when a test
//               makes every wait give up on purpose
constexpr size_t kCtlBytes = 256;
struct Ctl {
  uint64_t gen;
  uint32_t arrive;
  uint32_t err;
  uint32_t wait_limit;
  uint32_t wait_skew;
};
constexpr uint32_t kErrWait = 1;   // a bounded wait gave up
constexpr uint32_t kErrRange = 2;  // a prefix-mask value lay outside [0, n - 1]
constexpr uint32_t kDefaultWaitLimit = 1u << 22;
// The epoch a launch on this stream passes to its kernel: a new host epoch
// (top bits 0xFFF8) if the stream is not capturing, 0 if it is (the kernel
// then takes its epoch from the control block; la_ctl.h).
uint64_t launch_epoch(void* stream);

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
  Ctl* ctl = nullptr;    // the workspace's control block (ws points past it)
};

// Each returns 0 on success, else a nonzero HIP error code.
int launch_forward(const Fwd& a, const Plan& p);
int launch_causal(const Fwd& a, const Plan& p);
int launch_prefix(const Fwd& a, const Plan& p);
// Single-launch causal kernel (la_fused.hip): bf16, d = 64, chunk 64,
// Hq == Hkv, outputs requested.  Segments hold kFusedG chunks.
constexpr int kFusedG = 8;
constexpr int64_t kFusedMaxN = 131072;  // up to 256 segments per head
constexpr int64_t kFusedMaxR = 8;       // query heads per key/value head
constexpr int64_t kFusedMaxNGqa = 16384;  // n bound with grouped query heads (each runs its own look-back)
bool fused_causal_applies(int64_t Hq, int64_t Hkv, int64_t n, int64_t d, int dtype, int chunk);
size_t fused_causal_ws_bytes(int64_t NH, int64_t nseg);
int launch_causal_fused(const Fwd& a, const Plan& p);

// Non-causal path for bf16, d = 64 (la_forward_bf16.hip): one launch; state
// partials per segment of kFwdSegChunks chunks, a reduce, then the output
// pass, ordered by flags that carry the call's epoch (from the control block).
constexpr int kFwdSegChunks = 4;
// n bound: one head's rows, padded to a whole segment, stay below 2^31 bytes
// (the range of a buffer resource's record count and offsets).
constexpr int64_t kFwdMaxN = (int64_t)1 << 23;
bool forward_bf16_applies(int64_t n, int64_t d, int dtype);
int64_t forward_bf16_nseg(int64_t n);
size_t forward_bf16_ws_bytes(int64_t NKV, int64_t nseg);
int64_t forward_bf16_grid(int64_t NKV, int64_t NQ, int64_t n);
int launch_forward_bf16(const Fwd& a);

// Non-causal path for fp32, d = 64 (la_forward_f32.hip): state partials per
// segment of kFwd32SegTokens keys, a reduce, then the output pass.
constexpr int kFwd32SegTokens = 256;
constexpr int64_t kFwd32MaxN = (int64_t)1 << 22;  // as kFwdMaxN, for 4-byte elements
bool forward_f32_applies(int64_t n, int64_t d, int dtype);
int64_t forward_f32_nseg(int64_t n);
size_t forward_f32_ws_bytes(int64_t NKV, int64_t nseg);
int launch_forward_f32(const Fwd& a);

// A table of sequences (la_window.hip): per sequence s, key/value head g and
// query head h, row t of K and V at k + s kb + start(s) kt + g kh + t kt and
// of Q and out at q + s qb + start(s) qt + h qh + t qt (element strides);
// start(s) = cu[s] for packed sequences (cu [nseq + 1] on the device, every
// length at most n, every token below total), else 0 with every length n.
struct Seqs {
  int64_t qb, qh, qt, kb, kh, kt;
  const int64_t* cu;
  int64_t n, total;
};
// The causal (window = 0) or sliding-window (window >= 1) form over such a
// table: k_wstate + k_scan + k_window, or k_window alone.
struct SeqCall {
  const void* q; const void* k; const void* v; void* out;  // q, out NULL: state only (causal)
  Seqs S;
  int64_t nseq, Hq, Hkv, d;
  int dtype, phi;
  int64_t window;
  bool vec;              // 16-byte rows: d a power of two >= 8, strides and bases 16-byte aligned
  float* S_final; float* z_final;
  void* ws;              // causal form: (nseg + 1) state slots per (sequence, KV head)
  Ctl* ctl;              // may be NULL (no packed table to check)
  void* stream;
};
// The chunk of the sequence kernels for (element bytes, padded dim, form), 0
// if their tiles do not fit in LDS; the segment plan of a call.
int seq_chunk(int elem_bytes, int DP, bool window);
Plan seq_plan(const SeqCall& a, int C);
int launch_seq(const SeqCall& a);
// The causal form's state pass and scan alone, for chunk C (bf16 or fp32,
// d <= 64): a.ws receives the exclusive prefix slots of seq_plan(a, C).
int launch_seq_prefix(const SeqCall& a, int C);
// The causal form over a sequence table on the single-launch kernel
// (la_fused.hip): bf16, d = 64, Hq == Hkv, outputs requested, 16-byte rows
// with row strides of at least 64 elements, offsets below 2^31 bytes.  Its
// workspace (past the control block): the fused kernel's aggregates and flags.
bool fused_seq_applies(const SeqCall& a);
size_t fused_seq_ws_bytes(const SeqCall& a);
int launch_causal_fused_seq(const SeqCall& a);
// The sliding-window form on the single-launch kernel (la_window_fused.hip):
// bf16, d = 64, up to kFusedMaxR query heads per key/value head, windows
// shorter than 576 tokens, the row
// conditions of fused_seq_applies; no workspace (a.ctl may be NULL).  table:
// rows through the sequence table, else contiguous [B, H, n, d].
bool window_fused_applies(const SeqCall& a);
int launch_window_fused(const SeqCall& a, bool table);
// Gradients of the causal form (la_backward.hip): contiguous [B, H, n, d],
// d <= 64.  backward_chunk is 0 where the tiles do not fit in LDS.
struct BwdCall {
  const void* q; const void* k; const void* v; const void* dout;
  void* dq; void* dk; void* dv;
  int64_t B, Hq, Hkv, n, d;
  int dtype, phi;
  void* ws;  // the data regions past the control block
  void* stream;
};
int backward_chunk(int elem_bytes, int DP);
SeqCall backward_seqcall(const BwdCall& a);
size_t backward_ws_bytes(const BwdCall& a);
int launch_backward(const BwdCall& a);
// k_scan over (nseg + 1) slots per unit, F = 1 (la_kernels.hip).
int launch_scan(float* ws, int64_t nunits, int64_t nseg, int DP, int d, float* S_final, float* z_final,
                void* stream);
// The causal form's segment states on bf16 MFMA (k_state, la_kernels.hip)
// for contiguous bf16 [units, n, d] rows with d = 64 and chunk 32, where they
// are exact up to fp32 summation (relu + 1 through its split, or
// caller-applied features): ws receives one slot per segment of G chunks.
// Returns -1 (nothing launched) for any other case.
int launch_state_bf16_exact(const void* k, const void* v, int64_t units, int64_t n, int d, int phi, int C,
                            int64_t nchunks, int64_t G, int64_t nseg, float* ws, void* stream);

int launch_decode(const void* q, const void* k, const void* v, int64_t B,
                  int64_t Hq, int64_t Hkv, int64_t d, int dtype, int phi,
                  float* S, float* z, void* out, void* stream);

}  // namespace la_internal
