// Instantiations of multi_bwd_kernel (bf16 storage).
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(MQ, CH, SB) \
  case SB: return full ? (const void*)&multi_bwd_kernel<true, CH, SB, true, MQ, false, false> \
                       : (const void*)&multi_bwd_kernel<true, CH, SB, false, MQ, false, false>;

template <int MQ>
static const void* bwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, MQ, 1) default: break; } break;
    case 2:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, MQ, 2) default: break; }
      }
      break;
    case 4:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH4(ATTNRES_CASE, MQ, 4) default: break; }
      }
      break;
    default: break;
  }
  return nullptr;
}

const void* multi_bwd_kernel_ptr_bf16(int ch, int sb, bool full, int mq) {
  if (mq == 2) return bwd_ptr<2>(ch, sb, full);
  if (mq == 3) return bwd_ptr<3>(ch, sb, full);
  if (mq == 4) return bwd_ptr<4>(ch, sb, full);
  return nullptr;
}

}  // namespace attnres
