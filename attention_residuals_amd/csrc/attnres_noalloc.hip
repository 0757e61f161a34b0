// attnres_noalloc.hip -- attnres_bwd_noalloc: the single-query backward with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array's name is a host-side stand-in in host code, not a device address: its address on a
// device comes from hipGetSymbolAddress, taken once per device with that device current and kept
// per device (every GPU holds its own copy of the array at its own address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "attnres_internal.hpp"

namespace {

constexpr size_t kScratchBytes = attnres::kNoAllocScratchBytes;
constexpr int kMaxDevices = 64;

// The backward's counters (first 256 bytes) and partial rows; zero-initialised when the code object
// is loaded on a device, and held by that device until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {nullptr};

// Device address of `scratch` on the current device.
attnres_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return attnres::report_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return attnres::report(ATTNRES_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return attnres::report_hip(e, "hipGetSymbolAddress(scratch)");
    if (!p) return attnres::report(ATTNRES_ERR_HIP, "hipGetSymbolAddress returned NULL");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return ATTNRES_OK;
}

}  // namespace

extern "C" attnres_status attnres_bwd_noalloc(const attnres_desc* desc,
                                              const attnres_sources* values, const void* query,
                                              const void* norm_w, const void* out_w,
                                              const float* lse, const float* out_rstd,
                                              const float* o32, const void* dout,
                                              int64_t dout_row_stride,
                                              const attnres_sources* dvalues, void* dq, void* dw,
                                              void* dow, void* stream) {
  void* ws = nullptr;
  attnres_status st = scratch_ptr(&ws);
  if (st != ATTNRES_OK) return st;
  // the counter words start at zero on every call (a kernel clears them first on the stream);
  // the partial rows are planned to fit the array
  return attnres::bwd_call(desc, values, query, norm_w, out_w, lse, out_rstd, o32, dout,
                           dout_row_stride, dvalues, dq, dw, dow, ws, kScratchBytes,
                           kScratchBytes, true, stream);
}
