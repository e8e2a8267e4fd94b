// la_api.cpp -- the C ABI declared in include/la.h: argument checks,
// workspace sizing and the choice of chunk / segment sizes.  Host-only C++:
// every check runs before anything is enqueued, and no HIP call is made on an
// error path (so the checks also run on a machine without a GPU).
#include "la.h"

#include <stdint.h>

#include "la_internal.h"

namespace la_internal {

// The default chunk is the larger of 64 and 32 whose tiles leave room for two
// workgroups per CU (the general kernels hide load latency with the second
// workgroup), else the larger one that fits at all.
int default_chunk(int elem_bytes, int DP) {
  for (int c : {64, 32})
    if (chunk_lds_bytes(elem_bytes, DP, c) <= kLdsLimit / 2) return c;
  return chunk_fits(elem_bytes, DP, 64) ? 64 : 32;
}
// The non-causal form's kernels hold at most two tiles per chunk: the larger
// chunk that fits.
static int forward_chunk(int elem_bytes, int DP) { return chunk_fits(elem_bytes, DP, 64) ? 64 : 32; }

// Segments: about kTargetGroups workgroups per state pass, so that the 256
// CUs each get two, while each workgroup still walks a run of chunks and the
// scan has few segment states to read (the output launches of the GQA and
// prefix kernels group several segments per workgroup again).  The
// non-causal form needs only the total state, so it takes longer segments
// (about one workgroup per CU): fewer partial states to write and sum.
static constexpr int64_t kTargetGroups = 512;
static constexpr int64_t kTargetGroupsForward = 256;

Plan make_plan(int op, int64_t B, int64_t Hkv, int64_t n, int64_t d, int elem_bytes, int chunk) {
  Plan p;
  p.DP = padded_dim(d);
  p.C = chunk;
  p.nchunks = (n + chunk - 1) / chunk;
  const int64_t units = B * Hkv * p.nchunks;
  const int64_t target = op == LA_OP_FORWARD ? kTargetGroupsForward : kTargetGroups;
  int64_t G = (units + target - 1) / target;
  if (G < 1) G = 1;
  if (G > p.nchunks) G = p.nchunks;
  p.G = G;
  p.nseg = (p.nchunks + G - 1) / G;
  (void)elem_bytes;
  return p;
}

Plan make_fused_plan(int64_t n) {
  Plan p;
  p.DP = 64;
  p.C = 64;
  p.nchunks = (n + 63) / 64;
  p.G = kFusedG;
  p.nseg = (p.nchunks + kFusedG - 1) / kFusedG;
  return p;
}

size_t state_bytes(const Plan& p, int64_t B, int64_t Hkv) {
  const size_t slot = ((size_t)p.DP * p.DP + p.DP) * sizeof(float);
  return (size_t)B * Hkv * (size_t)(p.nseg + 1) * slot;
}

size_t bucket_bytes(int64_t n, int C) {
  const int64_t nchunks = (n + C - 1) / C;
  return (size_t)(nchunks + 1 + n) * sizeof(int);
}

}  // namespace la_internal

using namespace la_internal;

namespace {

constexpr int64_t kMaxGrid = (int64_t)1 << 31;

int elem_bytes(la_dtype dt) { return dt == LA_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Sizes shared by the three forward forms.  Returns LA_OK or an error.
la_status check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t d, la_dtype dt) {
  if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || n < 1 || d < 1 || d > kMaxD) return LA_ERR_SHAPE;
  if (Hq % Hkv != 0) return LA_ERR_SHAPE;
  if (n >= ((int64_t)1 << 31)) return LA_ERR_SHAPE;
  // element counts must stay well inside int64 (and byte counts inside size_t)
  const int64_t lim = (int64_t)1 << 40;
  if (B > lim / Hq || B * Hq > lim / n || B * Hq * n > lim / d) return LA_ERR_SHAPE;
  return LA_OK;
}

la_status resolve_chunk(int32_t chunk, la_dtype dt, int64_t d, int* C) {
  const int DP = padded_dim(d);
  const int eb = elem_bytes(dt);
  int c = chunk == 0 ? default_chunk(eb, DP) : chunk;
  if (c != 32 && c != 64 && c != 128) return LA_ERR_UNSUPPORTED;
  if (!chunk_fits(eb, DP, c)) return LA_ERR_UNSUPPORTED;
  *C = c;
  return LA_OK;
}

size_t required_ws(int32_t op, int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t d, la_dtype dt, int C,
                   Plan* out_plan) {
  (void)Hq;
  const Plan p = make_plan(op, B, Hkv, n, d, elem_bytes(dt), C);
  if (out_plan) *out_plan = p;
  size_t bytes = state_bytes(p, B, Hkv);
  if (op == LA_OP_PREFIX_MASK) bytes += bucket_bytes(n, C);
  if (op == LA_OP_PREFIX_MASK_BATCHED) bytes += (size_t)B * bucket_bytes(n, C);  // one sort per batch
  if (op == LA_OP_CAUSAL && fused_causal_applies(Hq, Hkv, n, d, (int)dt, C)) {
    const size_t f = fused_causal_ws_bytes(B * Hq, make_fused_plan(n).nseg);  // one set per query head
    if (f > bytes) bytes = f;
  }
  if (op == LA_OP_FORWARD && forward_bf16_applies(n, d, (int)dt)) {
    const size_t f = forward_bf16_ws_bytes(B * Hkv, forward_bf16_nseg(n));
    if (f > bytes) bytes = f;
  }
  if (op == LA_OP_FORWARD && forward_f32_applies(n, d, (int)dt)) {
    const size_t f = forward_f32_ws_bytes(B * Hkv, forward_f32_nseg(n));
    if (f > bytes) bytes = f;
  }
  return kCtlBytes + bytes;  // the control block, then the data regions
}

// The launchers see the data regions (past the control block) and the block.
void attach_ws(Fwd& a, void* ws) {
  a.ctl = reinterpret_cast<Ctl*>(ws);
  a.ws = reinterpret_cast<char*>(ws) + kCtlBytes;
}

la_status check_grid(const Plan& p, int64_t B, int64_t Hkv) {
  if (B * Hkv * p.nseg >= kMaxGrid) return LA_ERR_SHAPE;
  return LA_OK;
}

la_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return LA_OK;
  if (!ws || ws_bytes < need) return LA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LA_ERR_ALIGN;
  return LA_OK;
}

}  // namespace

extern "C" {

const char* la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE: a size is out of range or inconsistent";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE: unknown dtype code";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: chunk size not offered for this dtype / head dim";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: an output overlaps an input";
    case LA_ERR_LAUNCH: return "LA_ERR_LAUNCH: the HIP runtime rejected a launch";
    case LA_ERR_TIMEOUT: return "LA_ERR_TIMEOUT: a bounded wait between workgroups gave up (outputs are wrong)";
    case LA_ERR_RANGE: return "LA_ERR_RANGE: a prefix-mask value lay outside [0, n - 1]";
    case LA_ERR_DEVICE: return "LA_ERR_DEVICE: a HIP call failed while reading or writing the control block";
    default: return "unknown la_status";
  }
}

// The prefix form, and the causal form with one query head per key/value
// head, default to chunk 64 for fp32 with d = 64: their state and output
// kernels (16x16x4 fp32 MFMA, no LDS transposes) exist for that chunk.
static int32_t prefix_chunk(bool take, int32_t chunk, la_dtype dtype, int64_t d) {
  return take && chunk == 0 && dtype == LA_F32 && d == 64 ? 64 : chunk;
}

size_t la_workspace_bytes(int32_t op, int64_t B, int64_t Hq, int64_t Hkv, int64_t n, int64_t d, la_dtype dtype,
                          int32_t chunk) {
  if (op == LA_OP_CAUSAL_BACKWARD) {
    if (check_sizes(B, Hq, Hkv, n, d, dtype) != LA_OK) return 0;
    BwdCall a{};
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.n = n; a.d = d; a.dtype = (int)dtype;
    const size_t b = backward_ws_bytes(a);
    return b ? kCtlBytes + b : 0;
  }
  if (op == LA_OP_SEQS) {  // la_causal_forward_strided: B sequences of length at most n
    if (check_sizes(B, Hq, Hkv, n, d, dtype) != LA_OK) return 0;
    const int C = seq_chunk(elem_bytes(dtype), padded_dim(d), false);
    if (C == 0) return 0;
    SeqCall a{};
    a.S.n = n;
    a.nseq = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.d = d;
    // the general kernels' segment states, or the single-launch kernel's
    // aggregates where the strides may let it run
    const size_t general = state_bytes(seq_plan(a, C), B, Hkv);
    const size_t fused = dtype == LA_BF16 && fused_causal_applies(Hq, Hkv, n, d, (int)dtype, 64)
                             ? fused_seq_ws_bytes(a)
                             : 0;
    return kCtlBytes + (general > fused ? general : fused);
  }
  if (op != LA_OP_FORWARD && op != LA_OP_CAUSAL && op != LA_OP_PREFIX_MASK && op != LA_OP_PREFIX_MASK_BATCHED)
    return 0;
  const bool prefix = op == LA_OP_PREFIX_MASK || op == LA_OP_PREFIX_MASK_BATCHED;
  if (check_sizes(B, Hq, Hkv, n, d, dtype) != LA_OK) return 0;
  int C = 0;
  if (op == LA_OP_FORWARD) {
    C = forward_chunk(elem_bytes(dtype), padded_dim(d));
  } else if (resolve_chunk(prefix_chunk(prefix || Hq == Hkv, chunk, dtype, d), dtype, d, &C) != LA_OK) {
    return 0;
  }
  if (prefix && (Hq != Hkv || (n + C - 1) / C > kMaxBuckets)) return 0;
  return required_ws(op, B, Hq, Hkv, n, d, dtype, C, nullptr);
}

la_status la_forward_phi(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                         int64_t d, la_dtype dtype, la_phi phi, void* out, void* ws, size_t ws_bytes, void* stream) {
  la_status st = check_sizes(B, Hq, Hkv, n, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * Hq * n * d) * eb, kvb = (size_t)(B * Hkv * n * d) * eb;
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb)) return LA_ERR_ALIAS;
  const int C = forward_chunk((int)eb, padded_dim(d));
  Plan p;
  const size_t need = required_ws(LA_OP_FORWARD, B, Hq, Hkv, n, d, dtype, C, &p);
  if ((st = check_grid(p, B, Hkv)) != LA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, need)) != LA_OK) return st;
  if (overlaps(ws, need, out, qb) || overlaps(ws, need, q, qb) || overlaps(ws, need, k, kvb) ||
      overlaps(ws, need, v, kvb))
    return LA_ERR_ALIAS;
  Fwd a{q, k, v, out, B, Hq, Hkv, n, d, (int)dtype, nullptr, nullptr, nullptr, ws, stream, (int)phi};
  attach_ws(a, ws);
  if (forward_bf16_applies(n, d, (int)dtype)) {  // every feature map
    if (forward_bf16_grid(B * Hkv, B * Hq, n) >= kMaxGrid) return LA_ERR_SHAPE;
    return launch_forward_bf16(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
  }
  if (phi != LA_PHI_FEATURES && forward_f32_applies(n, d, (int)dtype)) {  // relu + 1 or ELU + 1
    if (B * Hq * forward_f32_nseg(n) >= kMaxGrid) return LA_ERR_SHAPE;
    return launch_forward_f32(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
  }
  return launch_forward(a, p) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_forward(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t n,
                     int64_t d, la_dtype dtype, void* out, void* ws, size_t ws_bytes, void* stream) {
  return la_forward_phi(q, k, v, B, Hq, Hkv, n, d, dtype, LA_PHI_RELU1, out, ws, ws_bytes, stream);
}

la_status la_causal_forward_phi(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t n, int64_t d, la_dtype dtype, la_phi phi, int32_t chunk, void* out,
                                float* S_final, float* z_final, void* ws, size_t ws_bytes, void* stream) {
  la_status st = check_sizes(B, Hq, Hkv, n, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (!k || !v) return LA_ERR_NULL;
  if ((q == nullptr) != (out == nullptr)) return LA_ERR_NULL;
  if (!q && !S_final && !z_final) return LA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || (q && !aligned16(q)) || (out && !aligned16(out)) ||
      (S_final && !aligned16(S_final)) || (z_final && !aligned16(z_final)))
    return LA_ERR_ALIGN;
  int C = 0;
  if ((st = resolve_chunk(prefix_chunk(Hq == Hkv, chunk, dtype, d), dtype, d, &C)) != LA_OK) return st;
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * Hq * n * d) * eb, kvb = (size_t)(B * Hkv * n * d) * eb;
  const size_t sb = (size_t)(B * Hkv * d * d) * sizeof(float), zb = (size_t)(B * Hkv * d) * sizeof(float);
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb)) return LA_ERR_ALIAS;
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {qb, kvb, kvb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(S_final, sb, ins[i], inb[i]) || overlaps(z_final, zb, ins[i], inb[i])) return LA_ERR_ALIAS;
  if (overlaps(S_final, sb, out, qb) || overlaps(z_final, zb, out, qb) || overlaps(S_final, sb, z_final, zb))
    return LA_ERR_ALIAS;
  Plan p;
  const size_t need = required_ws(LA_OP_CAUSAL, B, Hq, Hkv, n, d, dtype, C, &p);
  if ((st = check_grid(p, B, Hkv)) != LA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, need)) != LA_OK) return st;
  for (int i = 0; i < 3; ++i)
    if (overlaps(ws, need, ins[i], inb[i])) return LA_ERR_ALIAS;
  if (overlaps(ws, need, out, qb) || overlaps(ws, need, S_final, sb) || overlaps(ws, need, z_final, zb))
    return LA_ERR_ALIAS;
  Fwd a{q, k, v, out, B, Hq, Hkv, n, d, (int)dtype, nullptr, S_final, z_final, ws, stream, (int)phi};
  attach_ws(a, ws);
  if (q && fused_causal_applies(Hq, Hkv, n, d, (int)dtype, C)) {  // every feature map
    const Plan fp = make_fused_plan(n);
    if (B * Hq * fp.nseg >= kMaxGrid) return LA_ERR_SHAPE;
    return launch_causal_fused(a, fp) == 0 ? LA_OK : LA_ERR_LAUNCH;
  }
  return launch_causal(a, p) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_causal_forward(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t n, int64_t d, la_dtype dtype, int32_t chunk, void* out, float* S_final,
                            float* z_final, void* ws, size_t ws_bytes, void* stream) {
  return la_causal_forward_phi(q, k, v, B, Hq, Hkv, n, d, dtype, LA_PHI_RELU1, chunk, out, S_final, z_final, ws,
                               ws_bytes, stream);
}

// The prefix form with one shared mask (batched = false: m [n]) or one mask
// per batch (batched: m [B][n]).
static la_status prefix_impl(const void* q, const void* k, const void* v, const int64_t* m, bool batched,
                             int64_t B, int64_t H, int64_t n, int64_t d, la_dtype dtype, int32_t chunk, void* out,
                             void* ws, size_t ws_bytes, void* stream) {
  la_status st = check_sizes(B, H, H, n, d, dtype);
  if (st != LA_OK) return st;
  if (!q || !k || !v || !m || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(m) || !aligned16(out)) return LA_ERR_ALIGN;
  int C = 0;
  if ((st = resolve_chunk(prefix_chunk(true, chunk, dtype, d), dtype, d, &C)) != LA_OK) return st;
  if ((n + C - 1) / C > kMaxBuckets) return LA_ERR_UNSUPPORTED;
  const size_t eb = elem_bytes(dtype);
  const size_t tb = (size_t)(B * H * n * d) * eb, mb = (size_t)(batched ? B : 1) * n * sizeof(int64_t);
  if (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) || overlaps(out, tb, m, mb))
    return LA_ERR_ALIAS;
  Plan p;
  const size_t need = required_ws(batched ? LA_OP_PREFIX_MASK_BATCHED : LA_OP_PREFIX_MASK, B, H, H, n, d, dtype, C, &p);
  if ((st = check_grid(p, B, H)) != LA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, need)) != LA_OK) return st;
  if (overlaps(ws, need, q, tb) || overlaps(ws, need, k, tb) || overlaps(ws, need, v, tb) ||
      overlaps(ws, need, m, mb) || overlaps(ws, need, out, tb))
    return LA_ERR_ALIAS;
  Fwd a{q, k, v, out, B, H, H, n, d, (int)dtype, m, nullptr, nullptr, ws, stream, 0, batched ? B : 1};
  attach_ws(a, ws);
  return launch_prefix(a, p) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_prefix_mask_forward(const void* q, const void* k, const void* v, const int64_t* m, int64_t B,
                                 int64_t H, int64_t n, int64_t d, la_dtype dtype, int32_t chunk, void* out,
                                 void* ws, size_t ws_bytes, void* stream) {
  return prefix_impl(q, k, v, m, false, B, H, n, d, dtype, chunk, out, ws, ws_bytes, stream);
}

la_status la_prefix_mask_forward_batched(const void* q, const void* k, const void* v, const int64_t* m, int64_t B,
                                         int64_t H, int64_t n, int64_t d, la_dtype dtype, int32_t chunk, void* out,
                                         void* ws, size_t ws_bytes, void* stream) {
  return prefix_impl(q, k, v, m, true, B, H, n, d, dtype, chunk, out, ws, ws_bytes, stream);
}

la_status la_window_forward(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t n, int64_t d, la_dtype dtype, la_phi phi, int64_t window, void* out,
                            void* stream) {
  la_status st = check_sizes(B, Hq, Hkv, n, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (window < 1) return LA_ERR_SHAPE;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  const size_t eb = elem_bytes(dtype);
  const int C = seq_chunk((int)eb, padded_dim(d), true);
  if (C == 0) return LA_ERR_UNSUPPORTED;
  const size_t qb = (size_t)(B * Hq * n * d) * eb, kvb = (size_t)(B * Hkv * n * d) * eb;
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kvb) || overlaps(out, qb, v, kvb)) return LA_ERR_ALIAS;
  if (window > n) window = n;  // the whole causal prefix
  // contiguous [B, H, n, d] as a table of B sequences of length n
  SeqCall a{q, k, v, out, Seqs{Hq * n * d, n * d, d, Hkv * n * d, n * d, d, nullptr, n, B * n},
            B, Hq, Hkv, d, (int)dtype, (int)phi, window, d == padded_dim(d) && d * (int64_t)eb >= 16,
            nullptr, nullptr, nullptr, nullptr, stream};
  if (window_fused_applies(a)) return launch_window_fused(a, false) == 0 ? LA_OK : LA_ERR_LAUNCH;
  const Plan p = seq_plan(a, C);
  if (B * Hkv * p.nseg >= kMaxGrid) return LA_ERR_SHAPE;
  return launch_seq(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

// Bytes spanned by one tensor of a sequence table: the largest element offset
// plus one row (0 if a stride is negative or the span overflows).
static size_t table_span(int64_t nseq, int64_t H, int64_t n, int64_t d, const int64_t* st, bool packed,
                         int64_t total, size_t eb) {
  if (st[0] < 0 || st[1] < 0 || st[2] < 0) return 0;
  const int64_t lim = (int64_t)1 << 50;
  if (st[0] > lim / (nseq + 1) || st[1] > lim / (H + 1) || st[2] > lim / (total + n + 1)) return 0;
  const int64_t rows = packed ? total : n;
  if (rows == 0) return 0;
  const int64_t last = (packed ? 0 : (nseq - 1) * st[0]) + (H - 1) * st[1] + (rows - 1) * st[2];
  return (size_t)(last + d) * eb;
}

la_status la_causal_forward_strided(const void* q, const void* k, const void* v, const int64_t* cu_seqlens,
                                    int64_t nseq, int64_t max_len, int64_t total, int64_t Hq, int64_t Hkv, int64_t d,
                                    const int64_t* q_strides, const int64_t* kv_strides, la_dtype dtype, la_phi phi,
                                    int64_t window, void* out, float* S_final, float* z_final, void* ws,
                                    size_t ws_bytes, void* stream) {
  const bool packed = cu_seqlens != nullptr;
  la_status st = check_sizes(nseq, Hq, Hkv, max_len, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (!q_strides || !kv_strides) return LA_ERR_NULL;
  if (window < 0) return LA_ERR_SHAPE;
  if (packed && (total < 0 || total >= ((int64_t)1 << 40) || q_strides[0] != 0 || kv_strides[0] != 0))
    return LA_ERR_SHAPE;
  if (!packed) total = nseq * max_len;
  if (window > max_len) window = max_len;  // the whole causal prefix of the longest sequence
  if (!k || !v) return LA_ERR_NULL;
  if ((q == nullptr) != (out == nullptr)) return LA_ERR_NULL;
  if (!q && (window > 0 || (!S_final && !z_final))) return LA_ERR_NULL;
  if (window > 0 && (S_final || z_final)) return LA_ERR_UNSUPPORTED;  // a window has no running state to hand on
  if (!aligned16(k) || !aligned16(v) || (q && !aligned16(q)) || (out && !aligned16(out)) ||
      (S_final && !aligned16(S_final)) || (z_final && !aligned16(z_final)) || (packed && !aligned16(cu_seqlens)))
    return LA_ERR_ALIGN;
  const size_t eb = elem_bytes(dtype);
  const int DP = padded_dim(d);
  const int C = seq_chunk((int)eb, DP, window > 0);
  if (C == 0) return LA_ERR_UNSUPPORTED;
  const size_t qspan = table_span(nseq, Hq, max_len, d, q_strides, packed, total, eb);
  const size_t kvspan = table_span(nseq, Hkv, max_len, d, kv_strides, packed, total, eb);
  if (kvspan == 0 || (q && qspan == 0)) return LA_ERR_SHAPE;
  if (q_strides[1] < d && Hq > 1) return LA_ERR_SHAPE;   // heads of one row must not overlap
  if (kv_strides[1] < d && Hkv > 1) return LA_ERR_SHAPE;
  const size_t sb = (size_t)(nseq * Hkv * d * d) * sizeof(float), zb = (size_t)(nseq * Hkv * d) * sizeof(float);
  if (overlaps(out, qspan, q, qspan) || overlaps(out, qspan, k, kvspan) || overlaps(out, qspan, v, kvspan))
    return LA_ERR_ALIAS;
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {qspan, kvspan, kvspan};
  for (int i = 0; i < 3; ++i)
    if (overlaps(S_final, sb, ins[i], inb[i]) || overlaps(z_final, zb, ins[i], inb[i])) return LA_ERR_ALIAS;
  if (overlaps(S_final, sb, out, qspan) || overlaps(z_final, zb, out, qspan) || overlaps(S_final, sb, z_final, zb))
    return LA_ERR_ALIAS;
  // 16-byte row pieces when every row and every row start is 16-byte aligned
  const int64_t align_el = 16 / (int64_t)eb;
  bool vec = d == DP && d >= align_el;
  for (int i = 0; i < 3; ++i) vec = vec && q_strides[i] % align_el == 0 && kv_strides[i] % align_el == 0;
  SeqCall a{q, k, v, out,
            Seqs{q_strides[0], q_strides[1], q_strides[2], kv_strides[0], kv_strides[1], kv_strides[2], cu_seqlens,
                 max_len, total},
            nseq, Hq, Hkv, d, (int)dtype, (int)phi, window, vec, S_final, z_final, nullptr, nullptr, stream};
  const Plan p = seq_plan(a, C);
  if (nseq * Hkv * p.nseg >= kMaxGrid) return LA_ERR_SHAPE;
  const bool fused = fused_seq_applies(a);
  if (fused && nseq * Hq * ((max_len + kFusedG * 64 - 1) / (kFusedG * 64)) >= kMaxGrid) return LA_ERR_SHAPE;
  const size_t need = kCtlBytes + (fused ? fused_seq_ws_bytes(a) : window > 0 ? 0 : state_bytes(p, nseq, Hkv));
  if ((st = check_ws(ws, ws_bytes, need)) != LA_OK) return st;
  for (int i = 0; i < 3; ++i)
    if (overlaps(ws, need, ins[i], inb[i])) return LA_ERR_ALIAS;
  if (overlaps(ws, need, out, qspan) || overlaps(ws, need, S_final, sb) || overlaps(ws, need, z_final, zb) ||
      overlaps(ws, need, cu_seqlens, (size_t)(nseq + 1) * sizeof(int64_t)))
    return LA_ERR_ALIAS;
  a.ctl = reinterpret_cast<Ctl*>(ws);
  a.ws = reinterpret_cast<char*>(ws) + kCtlBytes;
  if (fused) return launch_causal_fused_seq(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
  if (window_fused_applies(a)) return launch_window_fused(a, true) == 0 ? LA_OK : LA_ERR_LAUNCH;
  return launch_seq(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_causal_backward(const void* q, const void* k, const void* v, const void* dout, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t n, int64_t d, la_dtype dtype, la_phi phi, void* dq, void* dk,
                             void* dv, void* ws, size_t ws_bytes, void* stream) {
  la_status st = check_sizes(B, Hq, Hkv, n, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv))
    return LA_ERR_ALIGN;
  const size_t eb = elem_bytes(dtype);
  if (backward_chunk((int)eb, padded_dim(d)) == 0) return LA_ERR_UNSUPPORTED;
  const size_t qb = (size_t)(B * Hq * n * d) * eb, kvb = (size_t)(B * Hkv * n * d) * eb;
  const void* ins[4] = {q, k, v, dout};
  const size_t inb[4] = {qb, kvb, kvb, qb};
  const void* outs[3] = {dq, dk, dv};
  const size_t outb[3] = {qb, kvb, kvb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], outb[o], ins[i], inb[i])) return LA_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], outb[o], outs[o2], outb[o2])) return LA_ERR_ALIAS;
  }
  BwdCall a{q, k, v, dout, dq, dk, dv, B, Hq, Hkv, n, d, (int)dtype, (int)phi, nullptr, stream};
  const size_t need = kCtlBytes + backward_ws_bytes(a);
  const int C = backward_chunk((int)eb, padded_dim(d));
  if (B * Hkv * seq_plan(backward_seqcall(a), C).nseg >= kMaxGrid) return LA_ERR_SHAPE;
  if ((st = check_ws(ws, ws_bytes, need)) != LA_OK) return st;
  for (int i = 0; i < 4; ++i)
    if (overlaps(ws, need, ins[i], inb[i])) return LA_ERR_ALIAS;
  for (int o = 0; o < 3; ++o)
    if (overlaps(ws, need, outs[o], outb[o])) return LA_ERR_ALIAS;
  a.ws = reinterpret_cast<char*>(ws) + kCtlBytes;
  return launch_backward(a) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_decode_step_phi(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv,
                             int64_t d, la_dtype dtype, la_phi phi, float* S, float* z, void* out, void* stream) {
  la_status st = check_sizes(B, Hq, Hkv, 1, d, dtype);
  if (st != LA_OK) return st;
  if (phi != LA_PHI_RELU1 && phi != LA_PHI_ELU1 && phi != LA_PHI_FEATURES) return LA_ERR_UNSUPPORTED;
  if (B * Hkv >= kMaxGrid) return LA_ERR_SHAPE;
  if (!q || !k || !v || !S || !z || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(z) || !aligned16(out))
    return LA_ERR_ALIGN;
  const size_t eb = elem_bytes(dtype);
  const size_t qb = (size_t)(B * Hq * d) * eb, kvb = (size_t)(B * Hkv * d) * eb;
  const size_t sb = (size_t)(B * Hkv * d * d) * sizeof(float), zb = (size_t)(B * Hkv * d) * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t inb[3] = {qb, kvb, kvb};
  for (int i = 0; i < 3; ++i)
    if (overlaps(out, qb, ins[i], inb[i]) || overlaps(S, sb, ins[i], inb[i]) || overlaps(z, zb, ins[i], inb[i]))
      return LA_ERR_ALIAS;
  if (overlaps(out, qb, S, sb) || overlaps(out, qb, z, zb) || overlaps(S, sb, z, zb)) return LA_ERR_ALIAS;
  return launch_decode(q, k, v, B, Hq, Hkv, d, (int)dtype, (int)phi, S, z, out, stream) == 0 ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_decode_step(const void* q, const void* k, const void* v, int64_t B, int64_t Hq, int64_t Hkv,
                         int64_t d, la_dtype dtype, float* S, float* z, void* out, void* stream) {
  return la_decode_step_phi(q, k, v, B, Hq, Hkv, d, dtype, LA_PHI_RELU1, S, z, out, stream);
}

}  // extern "C"
