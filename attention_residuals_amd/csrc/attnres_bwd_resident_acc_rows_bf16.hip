// Instantiations of bwd_resident_kernel for bf16 storage, accumulating into dvalues, with FP32
// gradient rows (no exact bins).
#include "attnres_kernels.hpp"
#include "attnres_internal.hpp"

namespace attnres {

#define ATTNRES_CASE(CH, SB) \
  case SB: return full ? (const void*)&bwd_resident_kernel<true, CH, SB, true, true, false> \
                       : (const void*)&bwd_resident_kernel<true, CH, SB, false, true, false>;

const void* bwd_resident_acc_rows_kernel_ptr_bf16(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, 1) default: break; } break;
    case 2: switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, 2) default: break; } break;
    case 4: switch (sb) { ATTNRES_SB_CH4(ATTNRES_CASE, 4) default: break; } break;
    default: break;
  }
  return nullptr;
}

}  // namespace attnres
