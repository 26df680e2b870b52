// Row top-k for callers that cannot allocate device memory.
//
// pw_topk takes its workspace from the caller. Code under HIP graph capture,
// tight serving loops and harnesses that forbid allocation cannot provide
// one, so pw_topk_noalloc runs the same planner and kernels with the
// workspace in a file-scope device array of kScratchBytes. Each GPU the
// library runs on holds its own copy of the array until the process ends;
// its device address is resolved once per device with hipGetSymbolAddress
// (the array's name in host code is only a host-side stand-in).
//
// The array is shared by every call on a GPU and keeps the last call's
// contents: the top-k path writes every workspace byte it later reads
// (column norms, epilogue vectors, split partials), so nothing needs
// clearing. Calls that overlap on one GPU (two streams, two host threads)
// race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pw.h"

namespace {

constexpr size_t kScratchBytes = PW_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's address of `scratch`, resolved on first use.
int scratch_address(void **out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PW_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PW_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PW_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PW_OK;
}

}  // namespace

extern "C" int pw_topk_noalloc(const pw_expr *e, int k, int largest, void *values, int64_t *indices, void *stream) {
  if (!e) return PW_ERR_INVALID;
  size_t need = 0;
  int rc = pw_workspace_size(e, PW_C_TOPK, 0, k, &need);
  if (rc != PW_OK) return rc;
  if (need > kScratchBytes) return PW_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    rc = scratch_address(&ws);
    if (rc != PW_OK) return rc;
  }
  return pw_topk(e, k, largest, values, indices, ws, need > 0 ? kScratchBytes : 0, stream);
}
