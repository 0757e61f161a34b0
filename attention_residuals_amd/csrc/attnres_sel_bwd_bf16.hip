// Instantiations of the selected-query backward (multi_bwd_kernel with per-token queries and
// partial bank rows) for bf16 storage: groups of two queries, one or two chunks per thread.
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(ACC, CH, SB) \
  case SB: return full ? (const void*)&multi_bwd_kernel<true, CH, SB, true, 2, ACC, true> \
                       : (const void*)&multi_bwd_kernel<true, CH, SB, false, 2, ACC, true>;

template <bool ACC>
static const void* bwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, ACC, 1) default: break; } break;
    case 2: switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, ACC, 2) default: break; } break;
    default: break;
  }
  return nullptr;
}

const void* sel_bwd_kernel_ptr_bf16(int ch, int sb, bool full, bool acc) {
  return acc ? bwd_ptr<true>(ch, sb, full) : bwd_ptr<false>(ch, sb, full);
}

}  // namespace attnres
