// attnres_internal.hpp -- host-side tables shared by the dispatcher and the instantiation files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attnres.h"

namespace attnres {

// Source-block sizes instantiated per chunks-per-thread CH. A token's rows are kept on chip when
// S <= the largest bucket of its CH (the register budget: SB * CH 16-byte chunks per thread). A
// source count between buckets runs the next bucket up with empty slots; exact blocks of 3 and 5
// measured faster than padding to 4 and 8 (S = 6, 7, 9, 11 ran as fast or faster padded).
#define ATTNRES_SB_CH1(M, ...) M(__VA_ARGS__, 1) M(__VA_ARGS__, 2) M(__VA_ARGS__, 3) \
  M(__VA_ARGS__, 4) M(__VA_ARGS__, 5) M(__VA_ARGS__, 8) M(__VA_ARGS__, 10)          \
  M(__VA_ARGS__, 12) M(__VA_ARGS__, 16) M(__VA_ARGS__, 24)
// Blocks of at most 10 sources with one chunk per thread (the four-slot selected backward).
#define ATTNRES_SB_CH1_LE10(M, ...) M(__VA_ARGS__, 1) M(__VA_ARGS__, 2) M(__VA_ARGS__, 3) \
  M(__VA_ARGS__, 4) M(__VA_ARGS__, 5) M(__VA_ARGS__, 8) M(__VA_ARGS__, 10)
#define ATTNRES_SB_CH2(M, ...) M(__VA_ARGS__, 1) M(__VA_ARGS__, 2) M(__VA_ARGS__, 3) \
  M(__VA_ARGS__, 4) M(__VA_ARGS__, 5) M(__VA_ARGS__, 8) M(__VA_ARGS__, 10)          \
  M(__VA_ARGS__, 12)
#define ATTNRES_SB_CH4(M, ...) M(__VA_ARGS__, 1) M(__VA_ARGS__, 2) M(__VA_ARGS__, 3) \
  M(__VA_ARGS__, 4)
// Streaming backward source blocks.
#define ATTNRES_SB_STREAM(M, ...) M(__VA_ARGS__, 1) M(__VA_ARGS__, 2) M(__VA_ARGS__, 4) \
  M(__VA_ARGS__, 8)

inline constexpr int kSbCh1[] = {1, 2, 3, 4, 5, 8, 10, 12, 16, 24};
inline constexpr int kSbCh2[] = {1, 2, 3, 4, 5, 8, 10, 12};
inline constexpr int kSbCh4[] = {1, 2, 3, 4};
inline constexpr int kSbStream[] = {1, 2, 4, 8};

// Largest workgroup any kernel is launched with (matches the kernels' launch bounds).
inline constexpr int kMaxThreads = 512;

// Forward workspace: one token counter, padded to the 256-byte alignment the ABI asks for.
inline constexpr size_t kFwdWorkspaceBytes = 256;

// Token counters are 32-bit and a call takes at most N + 2 * grid tickets from them: larger
// token counts use the static split.
inline constexpr int64_t kMaxTicketTokens = int64_t(1) << 31;


// Kernel entry points by configuration; nullptr when that configuration is not built.
const void* fwd_kernel_ptr_bf16(int ch, int sb, bool full, bool one_block);
const void* fwd_kernel_ptr_f32(int ch, int sb, bool full, bool one_block);
const void* bwd_resident_kernel_ptr_bf16(int ch, int sb, bool full);
const void* bwd_resident_rows_kernel_ptr_bf16(int ch, int sb, bool full);  // FP32 rows, no bins
const void* bwd_resident_kernel_ptr_f32(int ch, int sb, bool full);
const void* bwd_resident_acc_kernel_ptr_bf16(int ch, int sb, bool full);
const void* bwd_resident_acc_rows_kernel_ptr_bf16(int ch, int sb, bool full);  // FP32 rows
const void* bwd_resident_acc_kernel_ptr_f32(int ch, int sb, bool full);
const void* bwd_stream_kernel_ptr(bool bf16, int ch, int sb, bool full, bool acc);
const void* finalize_kernel_ptr(bool bf16);
const void* finalize_rows_kernel_ptr(bool bf16);
const void* multi_fwd_kernel_ptr(bool bf16, int ch, int sb, bool full, int mq);
const void* multi_bwd_kernel_ptr_bf16(int ch, int sb, bool full, int mq);
const void* multi_bwd_kernel_ptr_f32(int ch, int sb, bool full, int mq);
const void* multi_bwd_kernel_ptr_acc_bf16(int ch, int sb, bool full, int mq);
const void* multi_bwd_kernel_ptr_acc_f32(int ch, int sb, bool full, int mq);
const void* sel_fwd_kernel_ptr(bool bf16, int ch, int sb, bool full, int mq);
// Multi-query forward through matrix cores: cgw = 128-column chunk groups per wave (8 waves),
// mq = queries the kernel is built for (4, 8 or 16), sel = the selected-query read (queries from a
// bank by per-token ids); LDS for qrows staged query rows (M, or E + 1 for the selected read).
inline constexpr int kMfmaWaves = 8;
const void* multi_fwd_mfma_kernel_ptr(int cgw, int mq, bool full, bool sel);
size_t multi_fwd_mfma_lds(int cgw, int mq, int qrows);
// Multi-query backward through matrix cores (8 waves): nt = 32-column tiles per wave (D = 256 nt),
// dqm = where dq is summed (1: in the kernel's LDS, M <= 4; 0: by the separate dq kernel); qm =
// query staging (0: four-row groups, 1: groups and full rows for M <= 8, 2: the selected-query read
// with M slots per token over E <= 16 bank rows).
const void* multi_bwd_mfma_kernel_ptr(int nt, int dqm, bool full, bool acc, int qm);
const void* multi_dq_mfma_kernel_ptr();
// Multi- and selected-query forward in the same operand layout (8 waves, D = 256 nt), two tokens
// in flight; LDS for `rows` staged rows (M queries or E bank rows).
const void* multi_fwd_tile_kernel_ptr(int nt, bool full, bool sel, int stg);
size_t multi_fwd_tile_lds(int nt, int rows, bool sel, int stg);
const void* stream_probe_kernel_ptr(int cpt);
size_t multi_bwd_mfma_lds(int nt, int dqm, int M, int qm, int E);
// The multi-query backward with the sources and dY rows in one 16-row tile (S + M <= 16).
const void* multi_bwd_compact_kernel_ptr(int nt, bool dq, bool full, bool acc, bool sel);
size_t multi_bwd_compact_lds(int nt, bool dq, int rows, int M);
const void* sel_bwd_kernel_ptr_bf16(int ch, int sb, bool full, bool acc, int mq);
const void* sel_bwd_kernel_ptr_f32(int ch, int sb, bool full, bool acc, int mq);
const void* ticket_reset_kernel_ptr();

// Bytes of the allocation-free backward's device array (attnres_bwd_noalloc).
inline constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;

// attnres_bwd with its workspace given explicitly: `budget` > 0 caps the planned workspace
// (ATTNRES_ERR_WORKSPACE when even a static split's partial rows do not fit), `clear_counters`
// first launches a kernel that zeroes the workspace's counter words on the stream.
attnres_status bwd_call(const attnres_desc* d, const attnres_sources* values, const void* query,
                        const void* norm_w, const void* out_w, const float* lse,
                        const float* out_rstd, const float* o32, const void* dout,
                        int64_t dout_row_stride, const attnres_sources* dvalues, void* dq, void* dw,
                        void* dow, void* workspace, size_t workspace_bytes, size_t budget,
                        bool clear_counters, void* stream);

// Record a failure for attnres_last_error (from other translation units of the library).
attnres_status report(attnres_status st, const char* what);
attnres_status report_hip(hipError_t e, const char* what);

}  // namespace attnres
