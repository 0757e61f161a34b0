// Instantiations of bwd_stream_kernel and finalize_kernel, and the counter reset kernels.
#include "attnres_kernels.hpp"
#include "attnres_internal.hpp"

namespace attnres {

#define ATTNRES_CASE(BF, ACC, CH, SB) \
  case SB: return full ? (const void*)&bwd_stream_kernel<BF, CH, SB, true, ACC> \
                       : (const void*)&bwd_stream_kernel<BF, CH, SB, false, ACC>;

template <bool BF, bool ACC>
static const void* stream_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_STREAM(ATTNRES_CASE, BF, ACC, 1) default: break; } break;
    case 2: switch (sb) { ATTNRES_SB_STREAM(ATTNRES_CASE, BF, ACC, 2) default: break; } break;
    case 4: switch (sb) { ATTNRES_SB_STREAM(ATTNRES_CASE, BF, ACC, 4) default: break; } break;
    default: break;
  }
  return nullptr;
}

const void* bwd_stream_kernel_ptr(bool bf16, int ch, int sb, bool full, bool acc) {
  if (acc) return bf16 ? stream_ptr<true, true>(ch, sb, full) : stream_ptr<false, true>(ch, sb, full);
  return bf16 ? stream_ptr<true, false>(ch, sb, full) : stream_ptr<false, false>(ch, sb, full);
}

// Zeroes the counter words of a workspace's first 256 bytes on the launch stream (kernel stores:
// no memset node, so the call stays capturable into a HIP graph). Every word a kernel counts with
// is among them; the selected-query forward's id flag (word kCtrIdFlag) is left as it is.
__global__ __launch_bounds__(64) void ticket_reset_kernel(uint32_t* ctr) {
  if (threadIdx.x < kCtrIdFlag) ctr[threadIdx.x] = 0u;  // not the sticky id flag
}

const void* ticket_reset_kernel_ptr() { return (const void*)&ticket_reset_kernel; }

const void* finalize_kernel_ptr(bool bf16) {
  return bf16 ? (const void*)&finalize_kernel<true> : (const void*)&finalize_kernel<false>;
}

const void* finalize_rows_kernel_ptr(bool bf16) {
  return bf16 ? (const void*)&finalize_rows_kernel<true> : (const void*)&finalize_rows_kernel<false>;
}

}  // namespace attnres
