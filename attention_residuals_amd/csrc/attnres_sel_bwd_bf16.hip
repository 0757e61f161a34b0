// Instantiations of the selected-query backward (multi_bwd_kernel with per-token queries and
// partial bank rows) for bf16 storage: groups of two queries with one or two chunks per thread, and
// groups of three and four with one chunk per thread (four: blocks of at most 10 sources).
#include "attnres_internal.hpp"
#include "attnres_multi_kernels.hpp"

namespace attnres {

#define ATTNRES_CASE(ACC, MQ, CH, SB) \
  case SB: return full ? (const void*)&multi_bwd_kernel<true, CH, SB, true, MQ, ACC, true> \
                       : (const void*)&multi_bwd_kernel<true, CH, SB, false, MQ, ACC, true>;

template <bool ACC, int MQ>
static const void* bwd_ptr(int ch, int sb, bool full) {
  switch (ch) {
    case 1:
      if constexpr (MQ == 4) {
        switch (sb) { ATTNRES_SB_CH1_LE10(ATTNRES_CASE, ACC, MQ, 1) default: break; }
      } else {
        switch (sb) { ATTNRES_SB_CH1(ATTNRES_CASE, ACC, MQ, 1) default: break; }
      }
      break;
    case 2:
      if constexpr (MQ <= 2) {
        switch (sb) { ATTNRES_SB_CH2(ATTNRES_CASE, ACC, MQ, 2) default: break; }
      }
      break;
    default: break;
  }
  return nullptr;
}

const void* sel_bwd_kernel_ptr_bf16(int ch, int sb, bool full, bool acc, int mq) {
  if (mq == 2) return acc ? bwd_ptr<true, 2>(ch, sb, full) : bwd_ptr<false, 2>(ch, sb, full);
  if (mq == 3) return acc ? bwd_ptr<true, 3>(ch, sb, full) : bwd_ptr<false, 3>(ch, sb, full);
  if (mq == 4) return acc ? bwd_ptr<true, 4>(ch, sb, full) : bwd_ptr<false, 4>(ch, sb, full);
  return nullptr;
}

}  // namespace attnres
