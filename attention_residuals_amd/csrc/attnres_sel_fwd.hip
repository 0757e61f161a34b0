// Instantiations of the selected-query forward (multi_fwd_kernel with per-token queries): groups of
// two queries, one or two chunks per thread, bf16 and f32 storage.
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(BF, CH, SB) \
  case SB: return full ? (const void*)&multi_fwd_kernel<BF, CH, SB, true, 2, true> \
                       : (const void*)&multi_fwd_kernel<BF, CH, SB, false, 2, true>;

template <bool BF>
static const void* fwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, BF, 1) default: break; } break;
    case 2: switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, BF, 2) default: break; } break;
    default: break;
  }
  return nullptr;
}

const void* sel_fwd_kernel_ptr(bool bf16, int ch, int sb, bool full) {
  return bf16 ? fwd_ptr<true>(ch, sb, full) : fwd_ptr<false>(ch, sb, full);
}

}  // namespace attnres
