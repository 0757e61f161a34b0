// Instantiations of multi_fwd_kernel (bf16 and f32 storage). Groups of three and four queries are
// built for one chunk per thread only (wider rows would spill registers).
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(BF, MQ, CH, SB) \
  case SB: return full ? (const void*)&multi_fwd_kernel<BF, CH, SB, true, MQ, false> \
                       : (const void*)&multi_fwd_kernel<BF, CH, SB, false, MQ, false>;

template <bool BF, int MQ>
static const void* fwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, BF, MQ, 1) default: break; } break;
    case 2:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, BF, MQ, 2) default: break; }
      }
      break;
    case 4:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH4(ATTNRES_CASE, BF, MQ, 4) default: break; }
      }
      break;
    default: break;
  }
  return nullptr;
}

const void* multi_fwd_kernel_ptr(bool bf16, int ch, int sb, bool full, int mq) {
  if (mq == 2) return bf16 ? fwd_ptr<true, 2>(ch, sb, full) : fwd_ptr<false, 2>(ch, sb, full);
  if (mq == 3) return bf16 ? fwd_ptr<true, 3>(ch, sb, full) : fwd_ptr<false, 3>(ch, sb, full);
  if (mq == 4) return bf16 ? fwd_ptr<true, 4>(ch, sb, full) : fwd_ptr<false, 4>(ch, sb, full);
  return nullptr;
}

}  // namespace attnres
