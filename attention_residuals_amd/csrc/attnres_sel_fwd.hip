// Instantiations of the selected-query forward (multi_fwd_kernel with per-token queries), bf16 and
// f32 storage: groups of two queries with one or two chunks per thread, and groups of three and
// four with one chunk per thread (wider rows would spill registers).
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(BF, MQ, CH, SB) \
  case SB: return full ? (const void*)&multi_fwd_kernel<BF, CH, SB, true, MQ, true> \
                       : (const void*)&multi_fwd_kernel<BF, CH, SB, false, MQ, true>;

template <bool BF, int MQ>
static const void* fwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1: switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, BF, MQ, 1) default: break; } break;
    case 2:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, BF, MQ, 2) default: break; }
      }
      break;
    default: break;
  }
  return nullptr;
}

const void* sel_fwd_kernel_ptr(bool bf16, int ch, int sb, bool full, int mq) {
  switch (mq) {
    case 2: return bf16 ? fwd_ptr<true, 2>(ch, sb, full) : fwd_ptr<false, 2>(ch, sb, full);
    case 3: return bf16 ? fwd_ptr<true, 3>(ch, sb, full) : fwd_ptr<false, 3>(ch, sb, full);
    case 4: return bf16 ? fwd_ptr<true, 4>(ch, sb, full) : fwd_ptr<false, 4>(ch, sb, full);
    default: return nullptr;
  }
}

}  // namespace attnres
