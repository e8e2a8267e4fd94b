// la_control.hip -- the workspace control block calls of the C ABI
// (la_workspace_init, la_workspace_status, la_workspace_set_wait): the
// block's layout and meaning are in la_internal.h (struct Ctl), its use by the
// kernels in la_ctl.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "la.h"
#include "la_internal.h"

using la_internal::Ctl;
using la_internal::kCtlBytes;

namespace {

// Zero the control block (a kernel rather than a memset, so that the call
// may also be captured into a graph).
__global__ void k_ctl_zero(uint32_t* c) {
  if (threadIdx.x < kCtlBytes / 4) c[threadIdx.x] = 0u;
}

__global__ void k_ctl_set_wait(Ctl* c, uint32_t limit, uint32_t skew) {
  if (threadIdx.x == 0) {
    c->wait_limit = limit;
    c->wait_skew = skew;
  }
}

la_status check_ctl(const void* ws, size_t ws_bytes) {
  if (!ws) return LA_ERR_NULL;
  if (ws_bytes < kCtlBytes) return LA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 15u) != 0) return LA_ERR_ALIGN;
  return LA_OK;
}

std::atomic<uint64_t> g_host_epoch{0};

}  // namespace

namespace la_internal {

uint64_t launch_epoch(void* stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(reinterpret_cast<hipStream_t>(stream), &cs);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // a stream that cannot be asked is treated as capturing
    return 0;
  }
  if (cs != hipStreamCaptureStatusNone) return 0;
  return 0xFFF8000000000000ull | ((g_host_epoch.fetch_add(1, std::memory_order_relaxed) + 1) & 0x0000FFFFFFFFFFFFull);
}

}  // namespace la_internal

extern "C" {

la_status la_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  const la_status st = check_ctl(ws, ws_bytes);
  if (st != LA_OK) return st;
  k_ctl_zero<<<1, 64, 0, reinterpret_cast<hipStream_t>(stream)>>>(reinterpret_cast<uint32_t*>(ws));
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_workspace_set_wait(void* ws, size_t ws_bytes, uint32_t limit, uint32_t skew, void* stream) {
  const la_status st = check_ctl(ws, ws_bytes);
  if (st != LA_OK) return st;
  k_ctl_set_wait<<<1, 64, 0, reinterpret_cast<hipStream_t>(stream)>>>(reinterpret_cast<Ctl*>(ws), limit, skew);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_workspace_status(void* ws, size_t ws_bytes, void* stream) {
  const la_status st = check_ctl(ws, ws_bytes);
  if (st != LA_OK) return st;
  if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return LA_ERR_DEVICE;
  Ctl c;
  if (hipMemcpy(&c, ws, sizeof c, hipMemcpyDeviceToHost) != hipSuccess) return LA_ERR_DEVICE;
  if (c.err == 0) return LA_OK;
  const uint32_t zero = 0;
  if (hipMemcpy(reinterpret_cast<char*>(ws) + offsetof(Ctl, err), &zero, sizeof zero, hipMemcpyHostToDevice) !=
      hipSuccess)
    return LA_ERR_DEVICE;
  return (c.err & la_internal::kErrWait) ? LA_ERR_TIMEOUT : LA_ERR_RANGE;
}

}  // extern "C"
