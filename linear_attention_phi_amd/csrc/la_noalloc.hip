// la_noalloc.hip -- la_causal_forward_noalloc: la_causal_forward for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).  Its workspace is a
// file-scope device array of kScratchBytes, one per GPU the library runs on,
// held until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address: the address comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the entry point's first call there, and only
// that address is ever passed on.  The array is zero when the code object is
// loaded, so its control block (the first 256 bytes) starts valid, and every
// call leaves it valid for the next one.  Every call on a GPU shares that
// GPU's array: calls that may overlap in time on one GPU (on different
// streams) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "la.h"
#include "la_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per GPU
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];

// The device address of this GPU's array, or nullptr if the runtime fails.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) g_ptr[dev] = p;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" la_status la_causal_forward_noalloc(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                                               int64_t Hkv, int64_t n, int64_t d, la_dtype dtype, int32_t chunk,
                                               void* out, float* S_final, float* z_final, void* stream) {
  // every argument check of la_causal_forward, which reaches its workspace
  // check (and launches nothing) only if all the others pass
  const la_status pre =
      la_causal_forward(q, k, v, B, Hq, Hkv, n, d, dtype, chunk, out, S_final, z_final, nullptr, 0, stream);
  if (pre != LA_ERR_WORKSPACE) return pre;
  if (la_workspace_bytes(LA_OP_CAUSAL, B, Hq, Hkv, n, d, dtype, chunk) > kScratchBytes) return LA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return LA_ERR_DEVICE;
  return la_causal_forward(q, k, v, B, Hq, Hkv, n, d, dtype, chunk, out, S_final, z_final, ws, kScratchBytes,
                           stream);
}
