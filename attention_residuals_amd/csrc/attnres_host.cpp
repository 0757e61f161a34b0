// attnres_host.cpp -- C ABI of the AttnRes read library: argument checks, launch planning and
// kernel launches on the caller's stream. Declarations and contracts: include/attnres.h.
//
// Planning (everything derives from the descriptor and the current device):
//   * a row of D elements is cut into 16-byte chunks; a workgroup of W <= 8 waves covers it with
//     CH chunks per thread (CH = 1, 2 or 4, the smallest that keeps W <= 8);
//   * the backward keeps a token's S rows in VGPRs when S fits a source-block bucket of that CH
//     and no output norm is applied; otherwise it streams the sources and needs the forward's
//     FP32 mixture o (attnres_o32_elems);
//   * persistent grids: min(N, CUs x resident workgroups per CU from the occupancy calculator);
//   * the single-query backward's token-resident kernel sums every token's q/w gradient into
//     exact FP64 bins (one partial row per workgroup, tokens by ticket); the streaming kernel
//     writes FP32 rows of fixed token sets (a static head per workgroup, each ticketed tail batch
//     its own row); a finaliser sums each column's rows in a fixed order and zeroes the counter.
//     The multi- and selected-query backwards write one FP32 row per workgroup (tokens by ticket
//     unless deterministic) and the same kind of finaliser merges them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attnres.h"
#include "attnres_args.hpp"
#include "attnres_internal.hpp"

namespace {

using namespace attnres;

thread_local std::string g_err;

attnres_status fail(attnres_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

attnres_status hip_fail(hipError_t e, const char* what) {
  return fail(ATTNRES_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Optional tuning overrides read once from the environment: ATTNRES_CH forces chunks per thread
// (1, 2 or 4) when the resulting workgroup still fits; ATTNRES_WG_PER_CU caps workgroups per CU;
// ATTNRES_FWD_GRID_MULT / ATTNRES_BWD_GRID_MULT multiply the resident-workgroup grid.
int env_int(const char* name) {
  const char* v = std::getenv(name);
  return v ? std::atoi(v) : 0;
}

// ------------------------------------------------------------------ shape (descriptor only)

struct Shape {
  bool bf16;
  int vec, esz;
  int ch, W, threads;
  bool full;      // R == D
  bool resident;  // backward keeps every source row of a token on chip
  int sb_fwd, sb_bwd;
  bool fwd_one;   // forward holds all S sources in one block
};

int bucket_at_least(int S, const int* b, int nb) {
  for (int i = 0; i < nb; ++i)
    if (b[i] >= S) return b[i];
  return 0;
}

attnres_status check_desc(const attnres_desc* d) {
  if (!d) return fail(ATTNRES_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != ATTNRES_F32 && d->dtype != ATTNRES_BF16)
    return fail(ATTNRES_ERR_INVALID_ARG, "dtype %d is neither ATTNRES_F32 nor ATTNRES_BF16",
                d->dtype);
  if (d->S < 1 || d->S > kMaxSources)
    return fail(ATTNRES_ERR_INVALID_ARG, "S=%d outside [1, %d]", d->S, kMaxSources);
  if (d->D < 1 || d->R < 1 || d->R > d->D)
    return fail(ATTNRES_ERR_INVALID_ARG, "need 1 <= R <= D (R=%d, D=%d)", d->R, d->D);
  if (d->N < 0) return fail(ATTNRES_ERR_INVALID_ARG, "N=%lld is negative", (long long)d->N);
  const int vec = d->dtype == ATTNRES_BF16 ? 8 : 4;
  if (d->D % vec != 0)
    return fail(ATTNRES_ERR_UNSUPPORTED, "D=%d must be a multiple of %d for this dtype", d->D, vec);
  const int dmax = d->dtype == ATTNRES_BF16 ? 16384 : 8192;
  if (d->D < 8 || d->D > dmax)
    return fail(ATTNRES_ERR_UNSUPPORTED, "D=%d outside [8, %d] for this dtype", d->D, dmax);
  if (!(d->eps >= 0.f) || d->eps > 3.0e38f)
    return fail(ATTNRES_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!(d->scale == d->scale) || d->scale > 3.0e38f || d->scale < -3.0e38f)
    return fail(ATTNRES_ERR_INVALID_ARG, "scale must be finite");
  if (d->has_out_weight && !d->out_norm)
    return fail(ATTNRES_ERR_INVALID_ARG, "has_out_weight requires out_norm");
  if (d->deterministic != 0 && d->deterministic != 1)
    return fail(ATTNRES_ERR_INVALID_ARG, "deterministic must be 0 or 1");
  if (d->accumulate_dvalues != 0 && d->accumulate_dvalues != 1)
    return fail(ATTNRES_ERR_INVALID_ARG, "accumulate_dvalues must be 0 or 1");
  return ATTNRES_OK;
}

attnres_status make_shape(const attnres_desc* d, Shape* sh) {
  attnres_status st = check_desc(d);
  if (st != ATTNRES_OK) return st;
  sh->bf16 = d->dtype == ATTNRES_BF16;
  sh->vec = sh->bf16 ? 8 : 4;
  sh->esz = sh->bf16 ? 2 : 4;
  const int chunks = d->D / sh->vec;
  static const int forced = env_int("ATTNRES_CH");
  int ch = 0;
  if ((forced == 1 || forced == 2 || forced == 4) && (chunks + 64 * forced - 1) / (64 * forced) <= 8)
    ch = forced;
  // Resident shapes: 4-wave workgroups (CH = ceil(chunks / 256)) measured best on MI355X; the
  // streaming path (output norm, or sources that do not fit a bucket) keeps CH <= 2 to leave
  // registers for the FP32 mixture and do rows, with up to 8 waves.
  auto fit_for = [&](int c) {
    const int* b = c == 1 ? kSbCh1 : c == 2 ? kSbCh2 : kSbCh4;
    const int nb = c == 1 ? (int)(sizeof kSbCh1 / sizeof(int))
                   : c == 2 ? (int)(sizeof kSbCh2 / sizeof(int))
                            : (int)(sizeof kSbCh4 / sizeof(int));
    return bucket_at_least(d->S, b, nb);
  };
  if (!ch && !d->out_norm) {
    const int c = std::min(4, std::max(1, (chunks + 255) / 256));
    const int cc = c == 3 ? 4 : c;
    if ((chunks + 64 * cc - 1) / (64 * cc) <= 8 && fit_for(cc) > 0) ch = cc;
  }
  if (!ch) {
    for (int c : {1, 2, 4})
      if ((chunks + 64 * c - 1) / (64 * c) <= 8) {
        ch = c;
        break;
      }
  }
  if (!ch) return fail(ATTNRES_ERR_UNSUPPORTED, "D=%d too wide", d->D);
  sh->ch = ch;
  sh->W = (chunks + 64 * ch - 1) / (64 * ch);
  sh->threads = 64 * sh->W;
  sh->full = d->R == d->D;
  const int fit = fit_for(ch);
  sh->resident = !d->out_norm && fit > 0;
  // forward: one block when the sources fit a bucket, else blocks of the stream size
  // Source blocks of the streaming kernels: the forward holds one block, the backward two (it
  // double-buffers them) and, accumulating into dvalues, their existing gradient rows too: the
  // largest blocks that stay in registers.
  const int fwd_stream_max = ch == 4 ? 4 : 8;
  const int bwd_stream_max = ch == 4 ? 2 : (d->accumulate_dvalues && ch == 2) ? 2 : 4;
  sh->sb_fwd = fit > 0 ? fit : fwd_stream_max;
  sh->fwd_one = fit > 0;
  if (sh->resident) {
    sh->sb_bwd = fit;
  } else {
    int s = bucket_at_least(d->S, kSbStream, (int)(sizeof kSbStream / sizeof(int)));
    sh->sb_bwd = (s > 0 && s <= bwd_stream_max) ? s : bwd_stream_max;
  }
  return ATTNRES_OK;
}

const void* fwd_ptr(const Shape& sh) {
  return sh.bf16 ? fwd_kernel_ptr_bf16(sh.ch, sh.sb_fwd, sh.full, sh.fwd_one)
                 : fwd_kernel_ptr_f32(sh.ch, sh.sb_fwd, sh.full, sh.fwd_one);
}

// binned: the token-resident kernel with exact FP64 bins (always for FP32 storage; the bf16
// kernels, overwriting or accumulating, also come with FP32 rows)
const void* bwd_ptr(const Shape& sh, bool acc, bool binned = true) {
  if (sh.resident) {
    if (acc) {
      if (!binned && sh.bf16)
        return bwd_resident_acc_rows_kernel_ptr_bf16(sh.ch, sh.sb_bwd, sh.full);
      return sh.bf16 ? bwd_resident_acc_kernel_ptr_bf16(sh.ch, sh.sb_bwd, sh.full)
                     : bwd_resident_acc_kernel_ptr_f32(sh.ch, sh.sb_bwd, sh.full);
    }
    if (!binned && sh.bf16) return bwd_resident_rows_kernel_ptr_bf16(sh.ch, sh.sb_bwd, sh.full);
    return sh.bf16 ? bwd_resident_kernel_ptr_bf16(sh.ch, sh.sb_bwd, sh.full)
                   : bwd_resident_kernel_ptr_f32(sh.ch, sh.sb_bwd, sh.full);
  }
  return bwd_stream_kernel_ptr(sh.bf16, sh.ch, sh.sb_bwd, sh.full, acc);
}

// LDS of every kernel: the per-thread parameter region (u = w*q as float4 slots, plus the
// three-term bf16 split for bf16), then two exchange buffers (and the backward's ticket slots).
size_t param_lds(const Shape& sh) {
  if (sh.ch > 2) return 0;  // CH == 4 keeps the parameter vectors in registers
  const size_t slots = sh.ch * sh.vec / 4 + (sh.bf16 ? 3 * sh.ch : 0);
  return slots * sh.threads * 16u;
}
size_t fwd_lds(const Shape& sh) {
  return param_lds(sh) + 2u * (2u * sh.sb_fwd) * (4u * sh.W) * sizeof(float) + 4 * sizeof(float);
}
size_t bwd_lds(const Shape& sh) {
  return param_lds(sh) + 2u * (3u * sh.sb_bwd) * (4u * sh.W) * sizeof(float) + 4 * sizeof(float);
}

// ------------------------------------------------------------------ device facts

struct DevFacts {
  int cus = 0;
  int lds_per_block = 0;  // bytes of LDS one workgroup may allocate
};

attnres_status device_facts(DevFacts* f) {
  static std::mutex mu;
  static int cached[64] = {0};
  static int cached_lds[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(ATTNRES_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    if (cus <= 0) return fail(ATTNRES_ERR_HIP, "device reports %d compute units", cus);
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock)");
    cached[dev] = cus;
    cached_lds[dev] = lds;
  }
  f->cus = cached[dev];
  f->lds_per_block = cached_lds[dev];
  return ATTNRES_OK;
}

// Workgroups per CU for a persistent grid: the occupancy limit, capped at `wave_cap` waves per
// CU when wave_cap > 0 (two 4-wave token workgroups per CU measured best for the streaming
// read/write mix on MI355X: more concurrent rows per CU lowered the achieved bandwidth).
attnres_status blocks_per_cu(const void* fn, int threads, size_t lds, int* out, int wave_cap = 0) {
  int nb = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (wave_cap > 0) nb = std::min(nb, std::max(1, wave_cap / (threads / 64)));
  static const int cap = env_int("ATTNRES_WG_PER_CU");
  if (cap > 0) nb = std::min(nb, cap);
  if (nb <= 0) return fail(ATTNRES_ERR_UNSUPPORTED, "kernel cannot be resident (occupancy 0)");
  *out = nb;
  return ATTNRES_OK;
}

// Tokens per ticket of the dynamic schedules (see the kernels). Two effects, measured on MI355X:
//  - the device-wide counter serves its atomics one at a time; near ~70 tickets/us the queue
//    stalls every workgroup, so a batch must keep the ticket rate below `max_rate` tickets per
//    microsecond (the token rate is estimated at 5.6 TB/s over the kernel's bytes per token);
//  - workgroups finish up to one batch apart, so every workgroup keeps at least `min_batches`
//    batches (the backward asks for 16: at N = 8192 it has 16 tokens per workgroup), and the
//    grid never shrinks below one batch per resident slot.
// The forward waits for its ticket behind one output row, the backward behind S gradient rows, so
// the backward's ticket costs more and its rate bound is lower.
int64_t tokens_per_ticket(int64_t N, int64_t grid, double bytes_per_token, double max_rate,
                          int64_t min_batches) {
  static const int forced = env_int("ATTNRES_TOKENS_PER_TICKET");
  if (forced > 0) return forced;
  const double rate = 5.6e6 / bytes_per_token;  // tokens per microsecond at 5.6 TB/s
  int64_t b = std::max<int64_t>(1, (int64_t)std::ceil(rate / max_rate));
  b = std::min(b, std::max<int64_t>(1, N / (grid * std::max<int64_t>(1, min_batches))));
  return b;
}

// ------------------------------------------------------------------ backward plan

struct BwdPlan {
  int P = 0;               // backward workgroups (0: nothing to read, N == 0)
  int64_t tpt = 1;         // tokens per batch
  int64_t nbatch = 0;      // ceil(N / tpt)
  int64_t hb_end = 0;      // first tail batch (== nbatch: static split, no ticket)
  int rows = 0;            // partial rows
  bool binned = false;     // rows of exact FP64 bins (token-resident kernel) or FP32 sums
  int64_t wc = 0;          // columns per partial row
  int cols = 0;            // finaliser columns: R (+ D with dow)
  size_t off_part = 0, bytes = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workgroups per CU from the occupancy calculator, capped like the resident grids.
attnres_status bwd_grid(const attnres_desc* d, const Shape& sh, bool binned, int64_t* cap) {
  const void* fn = bwd_ptr(sh, d->accumulate_dvalues != 0, binned);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no backward kernel for this shape");
  DevFacts f;
  attnres_status st = device_facts(&f);
  if (st != ATTNRES_OK) return st;
  int per_cu = 0;
  static const int env_waves = env_int("ATTNRES_BWD_WAVES_PER_CU");
  st = blocks_per_cu(fn, sh.threads, bwd_lds(sh), &per_cu,
                     sh.resident ? (env_waves > 0 ? env_waves : 8) : 0);
  if (st != ATTNRES_OK) return st;
  static const int mult = std::max(1, env_int("ATTNRES_BWD_GRID_MULT"));
  *cap = (int64_t)f.cus * per_cu * mult;
  return ATTNRES_OK;
}

// The backward's schedule (see BwdArgs) and its partial rows. `budget` > 0 caps the workspace
// bytes: the streaming kernel's ticketed tail shrinks (down to a static split) until its rows
// fit, and ATTNRES_ERR_WORKSPACE is returned when even one row per workgroup does not.
attnres_status plan_bwd(const attnres_desc* d, const Shape& sh, BwdPlan* pl, size_t budget = 0) {
  // The token-resident kernel sums the q/w gradients into exact bins when the result must not
  // depend on the schedule (deterministic; and always for FP32 storage, which has no row
  // variant); the default bf16 backward keeps FP32 rows, 1.6% faster at the headline shape
  // (backward 1.017 -> 1.002 ms) and without the bins' spills when accumulating into dvalues,
  // reproducible to FP32 rounding under tickets.
  const bool binned = sh.resident && (d->deterministic || !sh.bf16);
  int64_t cap = 0;
  attnres_status st = bwd_grid(d, sh, binned, &cap);
  if (st != ATTNRES_OK) return st;
  const int64_t N = d->N;
  const int64_t P0 = std::max<int64_t>(1, std::min<int64_t>(N, cap));
  // tokens go out by ticket in both modes: the binned sums and the streaming kernel's rows of fixed
  // token sets do not depend on which workgroup ran a batch
  const bool dyn = N >= 2 * P0 && N < kMaxTicketTokens;
  pl->tpt = 1;
  if (dyn) {
    const double row_bytes = (double)d->D * sh.esz;
    const double per_token =
        ((d->accumulate_dvalues ? 3 : 2) * d->S + 1) * row_bytes + (sh.resident ? 0 : 4.0 * d->D);
    pl->tpt = tokens_per_ticket(N, P0, per_token, 30.0, 16);
  }
  pl->nbatch = (N + pl->tpt - 1) / pl->tpt;
  pl->P = (int)std::min<int64_t>(pl->nbatch, P0);
  pl->binned = binned;
  pl->hb_end = pl->nbatch;
  if (dyn && sh.resident) {
    pl->hb_end = pl->P;  // one row per workgroup: every batch after its first goes by ticket
  } else if (dyn) {
    // FP32 rows of fixed token sets: a static head, then about a quarter of the batches (at
    // least two per workgroup) by ticket, each into its own row (ATTNRES_BWD_TAIL: batches per
    // workgroup); a row costs D or 2D floats against a batch's (2S+1) rows of sources
    // and gradients plus the FP32 mixture
    static const int env_tail = env_int("ATTNRES_BWD_TAIL");
    const int64_t tail = env_tail > 0 ? env_tail : std::max<int64_t>(2, pl->nbatch / pl->P / 4);
    const int64_t h = std::max<int64_t>(1, pl->nbatch / pl->P - tail);
    pl->hb_end = std::min<int64_t>(pl->nbatch, h * pl->P);
  }
  pl->wc = (int64_t)d->D * (d->has_out_weight ? 2 : 1);
  pl->cols = d->R + (d->has_out_weight ? d->D : 0);
  const size_t row_bytes = (size_t)pl->wc * (pl->binned ? 2 * sizeof(double) : sizeof(float));
  pl->off_part = kCtrWords * sizeof(uint32_t);
  auto bytes_for = [&](int64_t rows) { return align256(pl->off_part + (size_t)rows * row_bytes); };
  int64_t rows = sh.resident ? pl->P : pl->P + (pl->nbatch - pl->hb_end);
  if (budget > 0 && bytes_for(rows) > budget) {
    const int64_t fit = budget > pl->off_part ? (int64_t)((budget - pl->off_part) / row_bytes) : 0;
    if (fit < pl->P)
      return fail(ATTNRES_ERR_WORKSPACE, "the backward needs %zu bytes of scratch, %zu available",
                  bytes_for(pl->P), budget);
    pl->hb_end = pl->nbatch - (fit - pl->P);  // (streaming rows only: the resident kernel's are P)
    rows = fit;
  }
  pl->rows = (int)rows;
  pl->bytes = bytes_for(rows);
  return ATTNRES_OK;
}

// ------------------------------------------------------------------ pointer checks

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
  const char* what;
};

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Byte range of one [N, D] row block with the given row stride.
Range rows_range(const void* p, int64_t N, int64_t rs, int D, int esz, const char* what) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const uintptr_t len = N > 0 ? (uintptr_t)(((N - 1) * rs + D) * esz) : 0;
  return Range{lo, lo + len, what};
}

attnres_status check_sources(const attnres_desc* d, const Shape& sh, const attnres_sources* src,
                             const char* what, const void** out_ptrs) {
  if (!src) return fail(ATTNRES_ERR_INVALID_ARG, "%s is NULL", what);
  if ((src->packed == nullptr) == (src->list == nullptr))
    return fail(ATTNRES_ERR_INVALID_ARG, "%s: exactly one of packed / list must be set", what);
  if (src->row_stride < d->D)
    return fail(ATTNRES_ERR_INVALID_ARG, "%s: row_stride %lld < D %d", what,
                (long long)src->row_stride, d->D);
  if ((src->row_stride * sh.esz) % 16 != 0)
    return fail(ATTNRES_ERR_ALIGNMENT, "%s: row stride is not a multiple of 16 bytes", what);
  for (int s = 0; s < d->S; ++s) {
    const void* p;
    if (src->packed) {
      if ((src->src_stride * sh.esz) % 16 != 0)
        return fail(ATTNRES_ERR_ALIGNMENT, "%s: src_stride is not a multiple of 16 bytes", what);
      p = static_cast<const char*>(src->packed) + (int64_t)s * src->src_stride * sh.esz;
    } else {
      p = src->list[s];
    }
    if (!p) return fail(ATTNRES_ERR_INVALID_ARG, "%s: source %d is NULL", what, s);
    if (!aligned(p, 16)) return fail(ATTNRES_ERR_ALIGNMENT, "%s: source %d not 16-byte aligned", what, s);
    out_ptrs[s] = p;
  }
  return ATTNRES_OK;
}

attnres_status check_param(const void* p, bool want, int esz, const char* what) {
  if (want && !p) return fail(ATTNRES_ERR_INVALID_ARG, "%s is required", what);
  if (!want && p) return fail(ATTNRES_ERR_INVALID_ARG, "%s must be NULL for this descriptor", what);
  if (p && !aligned(p, esz)) return fail(ATTNRES_ERR_ALIGNMENT, "%s is misaligned", what);
  return ATTNRES_OK;
}

attnres_status check_disjoint(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j]))
        return fail(ATTNRES_ERR_INVALID_ARG, "output %s overlaps output %s", outs[i].what,
                    outs[j].what);
    for (const Range& r : ins)
      if (overlap(outs[i], r))
        return fail(ATTNRES_ERR_INVALID_ARG, "output %s overlaps input %s", outs[i].what, r.what);
  }
  return ATTNRES_OK;
}

attnres_status launch(const void* fn, unsigned grid_x, unsigned grid_y, int threads, size_t lds,
                      void* args, void* stream, const char* what) {
  void* kargs[] = {args};
  hipError_t e = hipLaunchKernel(fn, dim3(grid_x, grid_y, 1), dim3(threads, 1, 1), kargs, lds,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, what);
  return ATTNRES_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

const char* attnres_status_str(attnres_status s) {
  switch (s) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_ERR_INVALID_ARG: return "invalid argument";
    case ATTNRES_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTNRES_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case ATTNRES_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTNRES_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attnres_last_error(void) { return g_err.c_str(); }

attnres_status attnres_o32_elems(const attnres_desc* d, size_t* elems) {
  g_err.clear();
  if (!elems) return fail(ATTNRES_ERR_INVALID_ARG, "elems is NULL");
  Shape sh;
  attnres_status st = make_shape(d, &sh);
  if (st != ATTNRES_OK) return st;
  *elems = sh.resident ? 0 : (size_t)d->N * d->D;
  return ATTNRES_OK;
}

attnres_status attnres_workspace_bytes(const attnres_desc* d, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  Shape sh;
  attnres_status st = make_shape(d, &sh);
  if (st != ATTNRES_OK) return st;
  BwdPlan pl;
  st = plan_bwd(d, sh, &pl);
  if (st != ATTNRES_OK) return st;
  *bytes = pl.bytes;
  return ATTNRES_OK;
}

attnres_status attnres_fwd_workspace_bytes(const attnres_desc* d, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  Shape sh;
  attnres_status st = make_shape(d, &sh);
  if (st != ATTNRES_OK) return st;
  *bytes = kFwdWorkspaceBytes;
  return ATTNRES_OK;
}

attnres_status attnres_fwd(const attnres_desc* d, const attnres_sources* values,
                           const void* query, const void* norm_w, const void* out_w, void* out,
                           float* lse, float* out_rstd, float* o32, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_err.clear();
  Shape sh;
  attnres_status st = make_shape(d, &sh);
  if (st != ATTNRES_OK) return st;
  if (workspace && (workspace_bytes < kFwdWorkspaceBytes || !aligned(workspace, 256)))
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace: %zu bytes given, %zu (256-byte aligned) "
                "needed", workspace_bytes, kFwdWorkspaceBytes);
  if (!workspace && workspace_bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace is NULL but workspace_bytes = %zu",
                workspace_bytes);
  if ((st = check_param(query, true, sh.esz, "query")) != ATTNRES_OK) return st;
  if ((st = check_param(norm_w, d->has_norm_weight, sh.esz, "norm_w")) != ATTNRES_OK) return st;
  if ((st = check_param(out_w, d->has_out_weight, sh.esz, "out_w")) != ATTNRES_OK) return st;
  if (d->N == 0) return ATTNRES_OK;  // nothing to read or write
  FwdArgs a;
  std::memset(&a, 0, sizeof a);
  st = check_sources(d, sh, values, "values", a.src);
  if (st != ATTNRES_OK) return st;
  if (!out || !aligned(out, 16))
    return fail(out ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "out NULL or misaligned");
  if (!lse || !aligned(lse, 4))
    return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
  if ((st = check_param(out_rstd, d->out_norm, 4, "out_rstd")) != ATTNRES_OK) return st;
  const bool need_o32 = !sh.resident;
  if ((st = check_param(o32, need_o32, 16, "o32")) != ATTNRES_OK) return st;

  const int64_t N = d->N;
  std::vector<Range> ins, outs;
  for (int s = 0; s < d->S; ++s)
    ins.push_back(rows_range(a.src[s], N, values->row_stride, d->D, sh.esz, "values"));
  outs.push_back(rows_range(out, N, d->D, d->D, sh.esz, "out"));
  outs.push_back(rows_range(lse, N, 1, 1, 4, "lse"));
  if (out_rstd) outs.push_back(rows_range(out_rstd, N, 1, 1, 4, "out_rstd"));
  if (o32) outs.push_back(rows_range(o32, N, d->D, d->D, 4, "o32"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  const void* fn = fwd_ptr(sh);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no forward kernel for this shape");
  DevFacts f;
  if ((st = device_facts(&f)) != ATTNRES_OK) return st;
  int per_cu = 0;
  // waves per CU of the single-block forward's grid: 12 with one chunk per thread and at most 8
  // sources (short rows: more tokens in flight per CU; 4-6% faster at D = 2048, S = 8), else 8
  // (12 measured slower with two chunks per thread and with 24-source blocks)
  static const int env_waves = env_int("ATTNRES_FWD_WAVES_PER_CU");
  const int def_waves = (sh.ch == 1 && sh.sb_fwd <= 8) ? 12 : 8;
  const int wave_cap = sh.fwd_one ? (env_waves > 0 ? env_waves : def_waves) : 0;
  if ((st = blocks_per_cu(fn, sh.threads, fwd_lds(sh), &per_cu, wave_cap)) != ATTNRES_OK)
    return st;
  // With the token counter (single-block path and a workspace) the grid is one resident pass and
  // workgroups take tokens as they finish. Without it, 8x the resident grid lets the hardware
  // dispatcher balance workgroups over CUs (measured better than a one-pass static grid).
  // the counter pays off once every resident workgroup has at least two tokens
  const int64_t resident = (int64_t)f.cus * per_cu;
  const bool dyn = workspace != nullptr && sh.fwd_one && N >= 2 * resident && N < kMaxTicketTokens;
  static const int env_mult = env_int("ATTNRES_FWD_GRID_MULT");
  const int mult = env_mult > 0 ? env_mult : (dyn ? 1 : 8);
  const int64_t slots = resident * mult;
  a.tpt = dyn ? tokens_per_ticket(N, slots, (double)(d->S + 1) * d->D * sh.esz, 55.0, 1) : 1;
  const int grid = (int)std::min<int64_t>((N + a.tpt - 1) / a.tpt, slots);
  if (dyn) a.ticket = static_cast<uint32_t*>(workspace);  // counters zero at launch (contract)

  a.row_stride = values->row_stride;
  a.N = N;
  a.S = d->S;
  a.D = d->D;
  a.R = d->R;
  a.lo = d->D - d->R;
  a.eps = d->eps;
  a.scale = d->scale;
  a.inv_R = 1.0f / (float)d->R;
  a.inv_D = 1.0f / (float)d->D;
  a.query = query;
  a.norm_w = norm_w;
  a.out_w = out_w;
  a.y = out;
  a.lse = lse;
  a.o_rstd = out_rstd;
  a.o32 = o32;
  a.out_norm = d->out_norm ? 1 : 0;
  return launch(fn, grid, 1, sh.threads, fwd_lds(sh), &a, stream, "forward launch");
}

}  // extern "C"

namespace attnres {

attnres_status report(attnres_status st, const char* what) {
  g_err.clear();
  return fail(st, "%s", what);
}

attnres_status report_hip(hipError_t e, const char* what) {
  g_err.clear();
  return hip_fail(e, what);
}

attnres_status bwd_call(const attnres_desc* d, const attnres_sources* values, const void* query,
                        const void* norm_w, const void* out_w, const float* lse,
                        const float* out_rstd, const float* o32, const void* dout,
                        int64_t dout_row_stride, const attnres_sources* dvalues, void* dq, void* dw,
                        void* dow, void* workspace, size_t workspace_bytes, size_t budget,
                        bool clear_counters, void* stream) {
  g_err.clear();
  Shape sh;
  attnres_status st = make_shape(d, &sh);
  if (st != ATTNRES_OK) return st;
  BwdArgs a;
  std::memset(&a, 0, sizeof a);
  const void* dptr[kMaxSources] = {nullptr};
  const int64_t N = d->N;
  if ((st = check_param(query, true, sh.esz, "query")) != ATTNRES_OK) return st;
  if ((st = check_param(norm_w, d->has_norm_weight, sh.esz, "norm_w")) != ATTNRES_OK) return st;
  if ((st = check_param(out_w, d->has_out_weight, sh.esz, "out_w")) != ATTNRES_OK) return st;
  if (N > 0) {  // with N == 0 no per-token array is touched (they may be NULL)
    st = check_sources(d, sh, values, "values", a.src);
    if (st != ATTNRES_OK) return st;
    st = check_sources(d, sh, dvalues, "dvalues", dptr);
    if (st != ATTNRES_OK) return st;
    if (!lse || !aligned(lse, 4))
      return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
    if ((st = check_param(out_rstd, d->out_norm, 4, "out_rstd")) != ATTNRES_OK) return st;
    if ((st = check_param(o32, !sh.resident, 16, "o32")) != ATTNRES_OK) return st;
    if (!dout || !aligned(dout, 16))
      return fail(dout ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "dout NULL or misaligned");
    if (dout_row_stride < d->D || (dout_row_stride * sh.esz) % 16 != 0)
      return fail(ATTNRES_ERR_ALIGNMENT, "dout_row_stride must be >= D and a multiple of 16 bytes");
  }
  if ((st = check_param(dq, true, sh.esz, "dq")) != ATTNRES_OK) return st;
  if ((st = check_param(dw, d->has_norm_weight, sh.esz, "dw")) != ATTNRES_OK) return st;
  if ((st = check_param(dow, d->has_out_weight, sh.esz, "dow")) != ATTNRES_OK) return st;
  if (!workspace) return fail(ATTNRES_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(ATTNRES_ERR_ALIGNMENT, "workspace not 256-byte aligned");

  std::vector<Range> ins, outs;
  if (N > 0) {
    for (int s = 0; s < d->S; ++s)
      ins.push_back(rows_range(a.src[s], N, values->row_stride, d->D, sh.esz, "values"));
    ins.push_back(rows_range(dout, N, dout_row_stride, d->D, sh.esz, "dout"));
    ins.push_back(rows_range(lse, N, 1, 1, 4, "lse"));
    if (o32) ins.push_back(rows_range(o32, N, d->D, d->D, 4, "o32"));
    if (out_rstd) ins.push_back(rows_range(out_rstd, N, 1, 1, 4, "out_rstd"));
    for (int s = 0; s < d->S; ++s)
      outs.push_back(rows_range(dptr[s], N, dvalues->row_stride, d->D, sh.esz, "dvalues"));
  }
  outs.push_back(rows_range(dq, 1, d->R, d->R, sh.esz, "dq"));
  if (dw) outs.push_back(rows_range(dw, 1, d->R, d->R, sh.esz, "dw"));
  if (dow) outs.push_back(rows_range(dow, 1, d->D, d->D, sh.esz, "dow"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  BwdPlan pl;
  if ((st = plan_bwd(d, sh, &pl, budget)) != ATTNRES_OK) return st;
  if (workspace_bytes < pl.bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                pl.bytes);
  const void* fn = bwd_ptr(sh, d->accumulate_dvalues != 0, pl.binned);
  char* ws = static_cast<char*>(workspace);
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws);
  if (clear_counters) {
    void* carg = ctr;
    st = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &carg, stream, "counter clear launch");
    if (st != ATTNRES_OK) return st;
  }

  if (pl.P > 0) {
    for (int s = 0; s < d->S; ++s) a.dsrc[s] = const_cast<void*>(dptr[s]);
    a.row_stride = values->row_stride;
    a.drow_stride = dvalues->row_stride;
    a.dout_stride = dout_row_stride;
    a.N = N;
    a.S = d->S;
    a.D = d->D;
    a.R = d->R;
    a.lo = d->D - d->R;
    a.eps = d->eps;
    a.scale = d->scale;
    a.inv_R = 1.0f / (float)d->R;
    a.inv_D = 1.0f / (float)d->D;
    a.query = query;
    a.norm_w = norm_w;
    a.out_w = out_w;
    a.lse = lse;
    a.o_rstd = out_rstd;
    a.o32 = o32;
    a.dout = dout;
    a.out_norm = d->out_norm ? 1 : 0;
    a.part = ws + pl.off_part;
    a.wc = pl.wc;
    a.tpt = pl.tpt;
    a.nbatch = pl.nbatch;
    a.hb_end = pl.hb_end;
    a.ctr = ctr;
    st = launch(fn, pl.P, 1, sh.threads, bwd_lds(sh), &a, stream, "backward launch");
    if (st != ATTNRES_OK) return st;
  }

  FinRowsArgs fa;
  std::memset(&fa, 0, sizeof fa);
  fa.part = ws + pl.off_part;
  fa.wc = pl.wc;
  fa.rows = pl.rows;
  fa.binned = pl.binned ? 1 : 0;
  fa.lo = d->D - d->R;
  fa.D = d->D;
  fa.R = d->R;
  fa.cols = pl.cols;
  fa.query = query;
  fa.norm_w = norm_w;
  fa.dq = dq;
  fa.dw = dw;
  fa.dow = dow;
  fa.ctr = ctr;
  return launch(finalize_rows_kernel_ptr(sh.bf16), (pl.cols + kFinRowsCols - 1) / kFinRowsCols, 1,
                kFinRowsCols * kFinRowsPhases, 0, &fa, stream, "finalize launch");
}

}  // namespace attnres

extern "C" {

attnres_status attnres_bwd(const attnres_desc* d, const attnres_sources* values,
                           const void* query, const void* norm_w, const void* out_w,
                           const float* lse, const float* out_rstd, const float* o32,
                           const void* dout, int64_t dout_row_stride,
                           const attnres_sources* dvalues, void* dq, void* dw, void* dow,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return attnres::bwd_call(d, values, query, norm_w, out_w, lse, out_rstd, o32, dout,
                           dout_row_stride, dvalues, dq, dw, dow, workspace, workspace_bytes, 0,
                           false, stream);
}

}  // extern "C"

// ====================================================================== multi-query read

namespace {

constexpr int kMaxQueries = 16;

struct MultiShape {
  Shape base;     // dtype facts (bf16, esz, vec) for the shared argument checks
  int ch = 0, W = 0, threads = 0, sb = 0;
  bool full = false;
  int mq_max = 2;  // queries per launch group (see make_multi_shape)
};

struct Group {
  int m0, cnt, mq;  // queries m0 .. m0 + cnt - 1, served by the MQ = mq kernel
};

attnres_desc single_desc(const attnres_multi_desc* m) {
  attnres_desc d;
  std::memset(&d, 0, sizeof d);
  d.S = m->S;
  d.D = m->D;
  d.R = m->R;
  d.dtype = m->dtype;
  d.N = m->N;
  d.eps = m->eps;
  d.scale = m->scale;
  d.deterministic = m->deterministic;
  d.accumulate_dvalues = m->accumulate_dvalues;
  return d;
}

// The multi-query kernels keep a token's S rows in VGPRs. With M <= 2 the single-query read's
// 4-wave workgroups (CH = ceil(chunks / 256)) measured best when the sources fit their bucket; with
// more queries (and otherwise) the fewest chunks per thread with at most 8 waves, which leaves
// registers for four queries per launch.
attnres_status make_multi_shape(const attnres_multi_desc* m, MultiShape* ms,
                                bool fewest_chunks = false) {
  if (!m) return fail(ATTNRES_ERR_INVALID_ARG, "desc is NULL");
  const attnres_desc d = single_desc(m);
  attnres_status st = check_desc(&d);
  if (st != ATTNRES_OK) return st;
  if (m->M < 1 || m->M > kMaxQueries)
    return fail(ATTNRES_ERR_INVALID_ARG, "M=%d outside [1, %d]", m->M, kMaxQueries);
  if (m->layout != ATTNRES_QUERY_MAJOR && m->layout != ATTNRES_TOKEN_MAJOR)
    return fail(ATTNRES_ERR_INVALID_ARG, "layout %d is neither query- nor token-major", m->layout);
  ms->base.bf16 = d.dtype == ATTNRES_BF16;
  ms->base.vec = ms->base.bf16 ? 8 : 4;
  ms->base.esz = ms->base.bf16 ? 2 : 4;
  const int chunks = d.D / ms->base.vec;
  auto bucket = [&](int c) {
    const int* b = c == 1 ? kSbCh1 : c == 2 ? kSbCh2 : kSbCh4;
    const int nb = c == 1 ? (int)(sizeof kSbCh1 / sizeof(int))
                   : c == 2 ? (int)(sizeof kSbCh2 / sizeof(int))
                            : (int)(sizeof kSbCh4 / sizeof(int));
    return bucket_at_least(d.S, b, nb);
  };
  static const int forced = env_int("ATTNRES_MULTI_CH");
  if ((forced == 1 || forced == 2 || forced == 4) && (chunks + 64 * forced - 1) / (64 * forced) <= 8)
    ms->ch = forced;
  if (!ms->ch && m->M <= 2 && !fewest_chunks) {
    const int c = std::min(4, std::max(1, (chunks + 255) / 256));
    const int cc = c == 3 ? 4 : c;
    if ((chunks + 64 * cc - 1) / (64 * cc) <= 8 && bucket(cc) > 0) ms->ch = cc;
  }
  for (int c : {1, 2, 4})
    if (!ms->ch && (chunks + 64 * c - 1) / (64 * c) <= 8) {
      ms->ch = c;
      break;
    }
  if (!ms->ch) return fail(ATTNRES_ERR_UNSUPPORTED, "D=%d too wide", d.D);
  ms->W = (chunks + 64 * ms->ch - 1) / (64 * ms->ch);
  ms->threads = 64 * ms->W;
  ms->full = d.R == d.D;
  ms->sb = bucket(ms->ch);
  if (ms->sb <= 0)
    return fail(ATTNRES_ERR_UNSUPPORTED,
                "the multi-query read keeps a token's rows on chip: S=%d sources of D=%d is too "
                "many for %d chunks per thread", d.S, d.D, ms->ch);
  // Four queries share one launch with one chunk per thread and at most 12 sources (fewer passes
  // over the sources and, for M > 4, fewer intermediate roundings of dvalues); groups that also
  // hold the existing gradient rows spill a few registers there. Otherwise groups of two.
  ms->mq_max = (ms->ch == 1 && ms->sb <= 12) ? kMaxGroupQueries : 2;
  return ATTNRES_OK;
}

// The fewest launch groups of at most mq_max queries, sized as evenly as possible (larger ones
// first): the kernels are VALU-bound beyond two queries, so a padded slot costs time (M = 5 runs
// as 3 + 2, not 4 + 1 padded to 2).
std::vector<Group> plan_groups(const attnres_multi_desc* m, const MultiShape& ms) {
  std::vector<Group> g;
  const int n = (m->M + ms.mq_max - 1) / ms.mq_max;
  for (int i = 0, m0 = 0; i < n; ++i) {
    const int cnt = m->M / n + (i < m->M % n ? 1 : 0);
    g.push_back(Group{m0, cnt, cnt <= 2 ? 2 : cnt});
    m0 += cnt;
  }
  return g;
}

// The one-pass matrix-core forward of the multi-query read (ids == nullptr: M fixed queries) or
// of the selected-query read (M slots per token, queries = the [E, R] bank): bf16, 3 <= M <= 16,
// 2 <= S <= 16, D <= 4096, and the staged queries (M rows, or E + 1 with a zero row) within the
// workgroup's LDS; ATTNRES_MULTI_MFMA=0 turns it off. *used tells whether it was launched.
attnres_status try_mfma_fwd(int S, int D, int R, int M, float eps, float scale, bool bf16,
                            const void* const* src, int64_t row_stride, int64_t N,
                            const void* queries, const int64_t* ids, int E, void* y, int64_t y_sm,
                            int64_t y_sn, float* lse, int64_t l_sm, int64_t l_sn, void* workspace,
                            const DevFacts& f, void* stream, bool* used) {
  *used = false;
  const char* e = std::getenv("ATTNRES_MULTI_MFMA");
  if (e && e[0] == '0') return ATTNRES_OK;
  const bool sel = ids != nullptr;
  // rows of D = 256 nt columns, five or more queries (or the selected read): the forward in the
  // matrix-core backward's operand layout, two tokens in flight; with three or four queries the
  // kernel below is as fast (ATTNRES_MULTI_TILE_FWD=0 keeps it for every shape)
  {
    static const char* te = std::getenv("ATTNRES_MULTI_TILE_FWD");
    const int nt = D / 256;
    const int rows = sel ? E : M;
    // outputs staged through LDS and stored as whole lines: five to eight rows in the exchange
    // blocks, more in staging blocks of their own where they fit; fewer rows are stored from the
    // operand layout (forward at S = 10, N = 32768, D = 4096, direct / staged, ms: M = 6 0.887 /
    // 0.871, M = 8 0.943 / 0.924, selected K = 3 0.809 / 0.838, K = 4 0.828 / 0.852)
    int stg = M > 8 ? (sel ? 0 : 16) : (M >= 5 ? 8 : 0);
    if (stg == 16 && multi_fwd_tile_lds(nt, rows, sel, 16) > (size_t)f.lds_per_block) stg = 0;
    const size_t lds = multi_fwd_tile_lds(nt, rows, sel, stg);
    bool al = aligned(queries, 16) && aligned(y, 16) && y_sm % 8 == 0 && y_sn % 8 == 0;
    for (int s = 0; s < S && s < 16; ++s) al = al && aligned(src[s], 16);
    if (!(te && te[0] == '0') && al && bf16 && S >= 2 && S <= 16 && M >= (sel ? 3 : 5) &&
        M <= 16 &&
        D % 256 == 0 && (nt == 4 || nt == 8 || nt == 12 || nt == 16) && R % 8 == 0 &&
        row_stride % 8 == 0 && lds <= (size_t)f.lds_per_block) {
      const void* fn = multi_fwd_tile_kernel_ptr(nt, R == D, sel, stg);
      if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no tile multi-query forward kernel");
      int per_cu = 0;
      attnres_status st = blocks_per_cu(fn, 64 * kMfmaWaves, lds, &per_cu);
      if (st != ATTNRES_OK) return st;
      MfmaFwdArgs ta;
      std::memset(&ta, 0, sizeof ta);
      for (int s = 0; s < S; ++s) ta.src[s] = src[s];
      ta.row_stride = row_stride;
      ta.N = N;
      ta.S = S;
      ta.D = D;
      ta.R = R;
      ta.lo = D - R;
      ta.M = M;
      ta.eps = eps;
      ta.scale = scale;
      ta.inv_R = 1.0f / (float)R;
      ta.query = queries;
      ta.y = y;
      ta.y_sm = y_sm;
      ta.y_sn = y_sn;
      ta.lse = lse;
      ta.l_sm = l_sm;
      ta.l_sn = l_sn;
      ta.ids = ids;
      ta.E = E;
      ta.id_flag = (sel && workspace) ? static_cast<uint32_t*>(workspace) + kCtrIdFlag : nullptr;
      *used = true;
      const int grid = (int)std::min<int64_t>(N, (int64_t)f.cus * per_cu);
      return launch(fn, grid, 1, 64 * kMfmaWaves, lds, &ta, stream,
                    "tile multi-query forward launch");
    }
  }
  const int cgw = (D + 1023) / 1024;
  const int mq = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
  const size_t lds = multi_fwd_mfma_lds(cgw, mq, sel ? E + 1 : mq);
  if (!bf16 || S < 2 || S > 16 || M < 3 || M > 16 || cgw > 4 || lds > (size_t)f.lds_per_block)
    return ATTNRES_OK;
  const void* fn = multi_fwd_mfma_kernel_ptr(cgw, mq, R == D, sel);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no matrix-core multi-query forward kernel");
  int per_cu = 0;
  attnres_status st = blocks_per_cu(fn, 64 * kMfmaWaves, lds, &per_cu);
  if (st != ATTNRES_OK) return st;
  MfmaFwdArgs ma;
  std::memset(&ma, 0, sizeof ma);
  for (int s = 0; s < S; ++s) ma.src[s] = src[s];
  ma.row_stride = row_stride;
  ma.N = N;
  ma.S = S;
  ma.D = D;
  ma.R = R;
  ma.lo = D - R;
  ma.M = M;
  ma.eps = eps;
  ma.scale = scale;
  ma.inv_R = 1.0f / (float)R;
  ma.query = queries;
  ma.y = y;
  ma.y_sm = y_sm;
  ma.y_sn = y_sn;
  ma.lse = lse;
  ma.l_sm = l_sm;
  ma.l_sn = l_sn;
  ma.ids = ids;
  ma.E = E;
  ma.id_flag = (sel && workspace) ? static_cast<uint32_t*>(workspace) + kCtrIdFlag : nullptr;
  // sixteen slots, a workspace and at least two tokens per resident workgroup: tokens come in
  // batches from a counter in the workspace (reset by a kernel: no memset, so the call stays
  // capturable); the kernels of fewer slots keep the static stride
  const int64_t resident = (int64_t)f.cus * per_cu;
  const bool dyn = mq == 16 && workspace != nullptr && N >= 2 * resident && N < kMaxTicketTokens;
  ma.tpt = dyn ? tokens_per_ticket(N, resident, (double)(S + M) * D * 2, 55.0, 1) : 1;
  ma.ticket = nullptr;
  *used = true;
  if (dyn) {
    ma.ticket = static_cast<uint32_t*>(workspace);
    void* targ = ma.ticket;
    attnres_status rs = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &targ, stream,
                               "ticket reset launch");
    if (rs != ATTNRES_OK) return rs;
  }
  const int grid = (int)std::min<int64_t>((N + ma.tpt - 1) / ma.tpt, resident);
  return launch(fn, grid, 1, 64 * kMfmaWaves, lds, &ma, stream, "matrix-core forward launch");
}

// Exchange buffers and ticket slots; with fixed queries (not the selected read) and two or more
// chunks per thread also the group's query slices, 16 bytes per thread, query and chunk.
size_t multi_fwd_lds(const MultiShape& ms, int mq, bool fixed_queries) {
  return 2u * (size_t)(1 + mq) * ms.sb * (4u * ms.W) * sizeof(float) + 4 * sizeof(float) +
         (fixed_queries && ms.ch >= 2 ? (size_t)mq * ms.ch * ms.threads * 16u : 0u);
}
size_t multi_bwd_lds(const MultiShape& ms, int mq) {
  return 2u * (size_t)(1 + 2 * mq) * ms.sb * (4u * ms.W) * sizeof(float) + 4 * sizeof(float);
}

const void* multi_bwd_ptr(const MultiShape& ms, int mq, bool acc) {
  if (acc)
    return ms.base.bf16 ? multi_bwd_kernel_ptr_acc_bf16(ms.ch, ms.sb, ms.full, mq)
                        : multi_bwd_kernel_ptr_acc_f32(ms.ch, ms.sb, ms.full, mq);
  return ms.base.bf16 ? multi_bwd_kernel_ptr_bf16(ms.ch, ms.sb, ms.full, mq)
                      : multi_bwd_kernel_ptr_f32(ms.ch, ms.sb, ms.full, mq);
}

// Element strides of y / dout rows and of lse between queries and between tokens.
void multi_strides(const attnres_multi_desc* m, int64_t* row_sm, int64_t* row_sn, int64_t* l_sm,
                   int64_t* l_sn) {
  if (m->layout == ATTNRES_QUERY_MAJOR) {
    *row_sm = m->N * (int64_t)m->D;
    *row_sn = m->D;
    *l_sm = m->N;
    *l_sn = 1;
  } else {
    *row_sm = m->D;
    *row_sn = (int64_t)m->M * m->D;
    *l_sm = 1;
    *l_sn = m->M;
  }
}

// A single query is the single-query read without a key-norm weight: its resident kernels serve it.
bool single_query_fast_path(const attnres_multi_desc* m, attnres_desc* d) {
  if (m->M != 1) return false;
  *d = single_desc(m);
  Shape sh;
  if (make_shape(d, &sh) != ATTNRES_OK) return false;
  g_err.clear();
  return sh.resident;
}

struct MultiBwdPlan {
  int P = 0;
  size_t off_part = 256, bytes = 256;
  // one-pass matrix-core backward (bf16, 3 <= M <= 16, 2 <= S <= 16, D <= 4096)
  bool mfma = false;
  bool compact = false;  // sources and dY rows in one 16-row tile (S + M <= 16)
  int nt = 0, dqm = 0, qm = 0, grid = 0, tiles = 0, ranges = 0, chunk0 = 0;
  int64_t tpr = 0;
  size_t lds = 0, off_coef = 0;
};

// The one-pass matrix-core backward: every query's gradient in one pass over the sources, so
// dvalues are written (and rounded) once. One workgroup per CU over a static token stride, the
// queries staged in its LDS. With M <= 4 (the compact tile: M <= 8 where the sums fit its LDS) each
// workgroup also sums dq for its tokens in LDS and writes one [M * R] partial row; otherwise the
// per-token coefficients a_{m,s} go to the workspace
// ([N][16][16] FP32) and the dq kernel reads the key slice of the sources again over static token
// ranges (about two workgroups per CU). The finaliser adds the partial rows in a fixed order.
// Rows of D = 256 nt columns (nt = 4, 8, 12 or 16 tiles of 32 columns per wave), R and the row
// strides multiples of 8 elements. ATTNRES_MULTI_MFMA=0 turns it off.
// The plan of the per-token matrix-core backward for M queries (or slots) of rows D = 256 nt, the
// queries staged as M rows (sel: E bank rows, the dq kernel forming dbank). No plan (mfma false)
// when the shape or the LDS does not fit.
attnres_status plan_mfma_bwd(int S, int D, int R, int M, bool sel, int E, int64_t N, bool acc,
                             int64_t row_stride, int64_t drow_stride, MultiBwdPlan* pl) {
  pl->mfma = false;
  const char* e = std::getenv("ATTNRES_MULTI_MFMA");
  if (e && e[0] == '0') return ATTNRES_OK;
  const int nt = D / 256;
  if (S < 2 || S > 16 || M < 3 || M > 16 || D % 256 != 0 ||
      (nt != 4 && nt != 8 && nt != 12 && nt != 16) || R % 8 != 0 || row_stride % 8 != 0 ||
      drow_stride % 8 != 0 || (sel && (E < 1 || E > 16)))
    return ATTNRES_OK;
  int dqm = (!sel && M <= 4) ? 1 : 0;
  DevFacts f;
  attnres_status st = device_facts(&f);
  if (st != ATTNRES_OK) return st;
  // the separate tiles' staged queries (full rows where they fit, M <= 8: the score operand
  // without transposes); false when they do not fit the LDS
  int qm = 0;
  size_t lds = 0;
  auto separate_fits = [&](int* qm_out, size_t* lds_out) {
    int q = sel ? 2 : (M <= 8 ? 1 : 0);
    size_t b = multi_bwd_mfma_lds(nt, dqm, M, q, E);
    if (q == 1 && b > (size_t)f.lds_per_block && dqm == 0) {
      q = 0;
      b = multi_bwd_mfma_lds(nt, dqm, M, q, E);
    }
    *qm_out = q;
    *lds_out = b;
    return b <= (size_t)f.lds_per_block;
  };
  // sources and dY rows together in one 16-row tile when they fit (S + M <= 16): half the row
  // registers, two tokens in flight (ATTNRES_MULTI_COMPACT=0 turns it off). Up to four queries
  // (slots) the separate tiles are faster where they fit (backward call at S = 10, N = 32768,
  // D = 4096, M = 4: 1.32 ms against 1.60 ms for the compact tile, accumulating 2.01 against
  // 2.12 ms, both with dq in LDS; selected E = 8, K = 4: 1.85 against 1.90 ms)
  static const char* ce = std::getenv("ATTNRES_MULTI_COMPACT");
  bool compact = S + M <= 16 && !(ce && ce[0] == '0');
  if (compact && M <= 4 && separate_fits(&qm, &lds)) compact = false;
  if (compact) {
    // dq summed in the kernel's LDS for up to eight queries where the sums fit beside the staged
    // queries (backward call at S = 10, N = 32768, D = 4096: M = 6 1.99 ms with the dq pass over
    // the sources, 1.75 ms with the sums in LDS; M = 5 1.86 / 1.62 ms)
    const bool cdq =
        !sel && M <= 8 && multi_bwd_compact_lds(nt, true, M, M) <= (size_t)f.lds_per_block;
    lds = multi_bwd_compact_lds(nt, cdq, sel ? E : M, M);
    compact = lds <= (size_t)f.lds_per_block;
    if (compact) dqm = cdq ? 1 : 0;
  }
  if (!compact && !separate_fits(&qm, &lds)) return ATTNRES_OK;
  const void* fn = compact ? multi_bwd_compact_kernel_ptr(nt, dqm != 0, R == D, acc, sel)
                           : multi_bwd_mfma_kernel_ptr(nt, dqm, R == D, acc, qm);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no matrix-core multi-query backward kernel");
  int per_cu = 0;
  if ((st = blocks_per_cu(fn, 64 * kMfmaWaves, lds, &per_cu)) != ATTNRES_OK) return st;
  const int rows = sel ? E : M;  // rows of the reduced gradient (dq or dbank)
  pl->mfma = true;
  pl->compact = compact;
  pl->nt = nt;
  pl->dqm = dqm;
  pl->qm = qm;
  pl->lds = lds;
  pl->grid = (int)std::min<int64_t>(N, (int64_t)f.cus * per_cu);
  if (dqm != 0) {
    pl->P = pl->grid;
    pl->off_part = 256;
    pl->bytes = align256(pl->off_part + (size_t)pl->P * rows * R * sizeof(float));
    return ATTNRES_OK;
  }
  pl->chunk0 = (D - R) / 8;
  const int key_chunks = D / 8 - pl->chunk0;
  pl->tiles = (key_chunks + 16 * kMfmaWaves - 1) / (16 * kMfmaWaves);
  const int64_t want = std::max<int64_t>(1, (2 * (int64_t)f.cus + pl->tiles - 1) / pl->tiles);
  pl->tpr = N > 0 ? (N + std::min<int64_t>(N, want) - 1) / std::min<int64_t>(N, want) : 1;
  pl->ranges = N > 0 ? (int)((N + pl->tpr - 1) / pl->tpr) : 0;
  pl->P = pl->ranges;
  pl->off_coef = 256;
  pl->off_part = align256(pl->off_coef + (size_t)N * 256 * sizeof(float));
  pl->bytes = align256(pl->off_part + (size_t)pl->ranges * rows * R * sizeof(float));
  return ATTNRES_OK;
}

attnres_status plan_multi_bwd_mfma(const attnres_multi_desc* m, const MultiShape& ms,
                                   int64_t row_stride, int64_t drow_stride, MultiBwdPlan* pl) {
  pl->mfma = false;
  // accumulating into dvalues, up to three queries with S <= 12 are one launch of the query-group
  // kernel, which rounds dvalues once as well and measured faster there (M = 3 at S = 10,
  // N = 32768, D = 4096: 1.81 ms against 1.96 ms); overwriting, the separate-tile kernel is faster
  // (1.29 against 1.39 ms)
  if (!ms.base.bf16 || (m->accumulate_dvalues && m->M <= 3 && m->S <= 12)) return ATTNRES_OK;
  return plan_mfma_bwd(m->S, m->D, m->R, m->M, false, 0, m->N, m->accumulate_dvalues != 0,
                       row_stride, drow_stride, pl);
}

// Launches the per-token matrix-core backward and, when it does not sum dq itself, the dq kernel;
// `b` carries the call's rows, queries and gradients. The finaliser is the caller's.
attnres_status launch_mfma_bwd(const MultiBwdPlan& pl, MfmaBwdArgs& b, bool sel, bool acc,
                               char* ws, void* stream) {
  if (pl.dqm == 0) b.coef = reinterpret_cast<float*>(ws + pl.off_coef);
  else b.part = reinterpret_cast<float*>(ws + pl.off_part);
  const void* fn =
      pl.compact ? multi_bwd_compact_kernel_ptr(pl.nt, pl.dqm != 0, b.R == b.D, acc, sel)
                 : multi_bwd_mfma_kernel_ptr(pl.nt, pl.dqm, b.R == b.D, acc, pl.qm);
  attnres_status st = launch(fn, pl.grid, 1, 64 * kMfmaWaves, pl.lds, &b, stream,
                             "matrix-core multi-query backward launch");
  if (st != ATTNRES_OK || pl.dqm != 0) return st;
  MfmaDqArgs q;
  std::memset(&q, 0, sizeof q);
  for (int s = 0; s < b.S; ++s) q.src[s] = b.src[s];
  q.row_stride = b.row_stride;
  q.N = b.N;
  q.S = b.S;
  q.D = b.D;
  q.R = b.R;
  q.lo = b.lo;
  q.M = sel ? b.E : b.M;
  q.chunk0 = pl.chunk0;
  q.tpr = pl.tpr;
  q.coef = b.coef;
  q.part = reinterpret_cast<float*>(ws + pl.off_part);
  return launch(multi_dq_mfma_kernel_ptr(), pl.tiles, pl.ranges, 64 * kMfmaWaves, 0, &q, stream,
                "matrix-core multi-query dq launch");
}

// The backward's plan for rows with the given strides (in elements); mfma_ok = false (or rows
// the matrix-core kernel cannot take) plans the query-group kernels.
attnres_status plan_multi_bwd(const attnres_multi_desc* m, const MultiShape& ms,
                              int64_t row_stride, int64_t drow_stride, bool mfma_ok,
                              MultiBwdPlan* pl) {
  *pl = MultiBwdPlan();
  if (mfma_ok) {
    attnres_status st0 = plan_multi_bwd_mfma(m, ms, row_stride, drow_stride, pl);
    if (st0 != ATTNRES_OK || pl->mfma) return st0;
  }
  const std::vector<Group> groups = plan_groups(m, ms);
  const void* fn = multi_bwd_ptr(ms, groups[0].mq, m->accumulate_dvalues != 0);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no multi-query backward kernel for this shape");
  DevFacts f;
  attnres_status st = device_facts(&f);
  if (st != ATTNRES_OK) return st;
  int per_cu = 0;
  st = blocks_per_cu(fn, ms.threads, multi_bwd_lds(ms, groups[0].mq), &per_cu, 8);
  if (st != ATTNRES_OK) return st;
  pl->P = (int)std::min<int64_t>(m->N, (int64_t)f.cus * per_cu);
  pl->off_part = 256;
  pl->bytes = align256(pl->off_part + (size_t)pl->P * m->M * m->R * sizeof(float));
  return ATTNRES_OK;
}

}  // namespace

extern "C" {

attnres_status attnres_multi_fwd_workspace_bytes(const attnres_multi_desc* m, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  MultiShape ms;
  attnres_status st = make_multi_shape(m, &ms);
  if (st != ATTNRES_OK) return st;
  *bytes = kFwdWorkspaceBytes;
  return ATTNRES_OK;
}

attnres_status attnres_multi_workspace_bytes(const attnres_multi_desc* m, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  MultiShape ms;
  attnres_status st = make_multi_shape(m, &ms);
  if (st != ATTNRES_OK) return st;
  attnres_desc d;
  if (single_query_fast_path(m, &d)) return attnres_workspace_bytes(&d, bytes);
  // enough for either backward: the matrix-core one (when the rows are dense and aligned) and the
  // query-group one that serves other strides
  MultiBwdPlan pm, pv;
  if ((st = plan_multi_bwd(m, ms, m->D, m->D, true, &pm)) != ATTNRES_OK) return st;
  *bytes = pm.bytes;
  if (pm.mfma) {
    if (plan_multi_bwd(m, ms, m->D, m->D, false, &pv) == ATTNRES_OK)
      *bytes = std::max(pm.bytes, pv.bytes);
    g_err.clear();
  }
  return ATTNRES_OK;
}

attnres_status attnres_multi_fwd(const attnres_multi_desc* m, const attnres_sources* values,
                                 const void* queries, void* y, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err.clear();
  MultiShape ms;
  attnres_status st = make_multi_shape(m, &ms);
  if (st != ATTNRES_OK) return st;
  if (workspace && (workspace_bytes < kFwdWorkspaceBytes || !aligned(workspace, 256)))
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace: %zu bytes given, %zu (256-byte aligned) "
                "needed", workspace_bytes, kFwdWorkspaceBytes);
  if (!workspace && workspace_bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace is NULL but workspace_bytes = %zu",
                workspace_bytes);
  const attnres_desc d = single_desc(m);
  if ((st = check_param(queries, true, ms.base.esz, "queries")) != ATTNRES_OK) return st;
  if (m->N == 0) return ATTNRES_OK;
  MultiFwdArgs a;
  std::memset(&a, 0, sizeof a);
  if ((st = check_sources(&d, ms.base, values, "values", a.src)) != ATTNRES_OK) return st;
  if (!y || !aligned(y, 16))
    return fail(y ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "y NULL or misaligned");
  if (!lse || !aligned(lse, 4))
    return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
  const int64_t N = m->N, M = m->M;
  std::vector<Range> ins, outs;
  for (int s = 0; s < m->S; ++s)
    ins.push_back(rows_range(a.src[s], N, values->row_stride, m->D, ms.base.esz, "values"));
  ins.push_back(rows_range(queries, M, m->R, m->R, ms.base.esz, "queries"));
  outs.push_back(rows_range(y, M * N, m->D, m->D, ms.base.esz, "y"));
  outs.push_back(rows_range(lse, M * N, 1, 1, 4, "lse"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  attnres_desc d1;
  if (single_query_fast_path(m, &d1))
    return attnres_fwd(&d1, values, queries, nullptr, nullptr, y, lse, nullptr, nullptr, workspace,
                       workspace_bytes, stream);

  DevFacts f;
  if ((st = device_facts(&f)) != ATTNRES_OK) return st;
  int64_t y_sm, y_sn, l_sm, l_sn;
  multi_strides(m, &y_sm, &y_sn, &l_sm, &l_sn);

  // Three to sixteen bf16 queries: one pass through the matrix-core forward when it applies.
  {
    bool used = false;
    st = try_mfma_fwd(m->S, m->D, m->R, (int)M, m->eps, m->scale, ms.base.bf16, a.src,
                      values->row_stride, N, queries, nullptr, 0, y, y_sm, y_sn, lse, l_sm, l_sn,
                      workspace, f, stream, &used);
    if (st != ATTNRES_OK || used) return st;
  }
  a.row_stride = values->row_stride;
  a.N = N;
  a.S = m->S;
  a.D = m->D;
  a.R = m->R;
  a.lo = m->D - m->R;
  a.eps = m->eps;
  a.scale = m->scale;
  a.inv_R = 1.0f / (float)m->R;
  a.y_sm = y_sm;
  a.y_sn = y_sn;
  a.l_sm = l_sm;
  a.l_sn = l_sn;
  for (const Group& g : plan_groups(m, ms)) {
    const void* fn = multi_fwd_kernel_ptr(ms.base.bf16, ms.ch, ms.sb, ms.full, g.mq);
    if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no multi-query forward kernel for this shape");
    const size_t lds = multi_fwd_lds(ms, g.mq, true);
    int per_cu = 0;
    if ((st = blocks_per_cu(fn, ms.threads, lds, &per_cu, 8)) != ATTNRES_OK) return st;
    const int64_t resident = (int64_t)f.cus * per_cu;
    const bool dyn = workspace != nullptr && N >= 2 * resident && N < kMaxTicketTokens;
    const int64_t slots = resident * (dyn ? 1 : 8);
    a.tpt = dyn ? tokens_per_ticket(N, slots, (double)(m->S + g.mq) * m->D * ms.base.esz, 55.0, 1)
                : 1;
    a.ticket = nullptr;
    if (dyn) {
      a.ticket = static_cast<uint32_t*>(workspace);
      void* targ = a.ticket;
      st = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &targ, stream, "ticket reset launch");
      if (st != ATTNRES_OK) return st;
    }
    a.M = g.cnt;
    a.query = static_cast<const char*>(queries) + (int64_t)g.m0 * m->R * ms.base.esz;
    a.y = static_cast<char*>(y) + g.m0 * y_sm * ms.base.esz;
    a.lse = lse + g.m0 * l_sm;
    const int grid = (int)std::min<int64_t>((N + a.tpt - 1) / a.tpt, slots);
    st = launch(fn, grid, 1, ms.threads, lds, &a, stream, "multi-query forward launch");
    if (st != ATTNRES_OK) return st;
  }
  return ATTNRES_OK;
}

attnres_status attnres_multi_bwd(const attnres_multi_desc* m, const attnres_sources* values,
                                 const void* queries, const float* lse, const void* dout,
                                 const attnres_sources* dvalues, void* dq, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  g_err.clear();
  MultiShape ms;
  attnres_status st = make_multi_shape(m, &ms);
  if (st != ATTNRES_OK) return st;
  const attnres_desc d = single_desc(m);
  const int64_t N = m->N, M = m->M;
  MultiBwdArgs a;
  std::memset(&a, 0, sizeof a);
  const void* dptr[kMaxSources] = {nullptr};
  if ((st = check_param(queries, true, ms.base.esz, "queries")) != ATTNRES_OK) return st;
  if ((st = check_param(dq, true, ms.base.esz, "dq")) != ATTNRES_OK) return st;
  if (N > 0) {
    if ((st = check_sources(&d, ms.base, values, "values", a.src)) != ATTNRES_OK) return st;
    if ((st = check_sources(&d, ms.base, dvalues, "dvalues", dptr)) != ATTNRES_OK) return st;
    if (!lse || !aligned(lse, 4))
      return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
    if (!dout || !aligned(dout, 16))
      return fail(dout ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "dout NULL or misaligned");
  }
  if (!workspace) return fail(ATTNRES_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(ATTNRES_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  std::vector<Range> ins, outs;
  if (N > 0) {
    for (int s = 0; s < m->S; ++s)
      ins.push_back(rows_range(a.src[s], N, values->row_stride, m->D, ms.base.esz, "values"));
    ins.push_back(rows_range(dout, M * N, m->D, m->D, ms.base.esz, "dout"));
    ins.push_back(rows_range(lse, M * N, 1, 1, 4, "lse"));
    for (int s = 0; s < m->S; ++s)
      outs.push_back(rows_range(dptr[s], N, dvalues->row_stride, m->D, ms.base.esz, "dvalues"));
  }
  ins.push_back(rows_range(queries, M, m->R, m->R, ms.base.esz, "queries"));
  outs.push_back(rows_range(dq, M, m->R, m->R, ms.base.esz, "dq"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  attnres_desc d1;
  if (single_query_fast_path(m, &d1))
    return attnres_bwd(&d1, values, queries, nullptr, nullptr, lse, nullptr, nullptr, dout, m->D,
                       dvalues, dq, nullptr, nullptr, workspace, workspace_bytes, stream);

  MultiBwdPlan pl;
  if ((st = plan_multi_bwd(m, ms, values->row_stride, dvalues->row_stride, aligned(queries, 16),
                           &pl)) != ATTNRES_OK)
    return st;
  if (workspace_bytes < pl.bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                pl.bytes);
  char* ws = static_cast<char*>(workspace);
  if (pl.mfma && N > 0) {
    int64_t g_sm, g_sn, l_sm, l_sn;
    multi_strides(m, &g_sm, &g_sn, &l_sm, &l_sn);
    MfmaBwdArgs b;
    std::memset(&b, 0, sizeof b);
    for (int s = 0; s < m->S; ++s) {
      b.src[s] = a.src[s];
      b.dsrc[s] = const_cast<void*>(dptr[s]);
    }
    b.row_stride = values->row_stride;
    b.drow_stride = dvalues->row_stride;
    b.N = N;
    b.S = m->S;
    b.D = m->D;
    b.R = m->R;
    b.lo = m->D - m->R;
    b.M = m->M;
    b.eps = m->eps;
    b.scale = m->scale;
    b.inv_R = 1.0f / (float)m->R;
    b.query = queries;
    b.lse = lse;
    b.l_sm = l_sm;
    b.l_sn = l_sn;
    b.dout = dout;
    b.g_sm = g_sm;
    b.g_sn = g_sn;
    st = launch_mfma_bwd(pl, b, false, m->accumulate_dvalues != 0, ws, stream);
    if (st != ATTNRES_OK) return st;
  } else if (pl.P > 0 && !pl.mfma) {
    int64_t g_sm, g_sn, l_sm, l_sn;
    multi_strides(m, &g_sm, &g_sn, &l_sm, &l_sn);
    for (int s = 0; s < m->S; ++s) a.dsrc[s] = const_cast<void*>(dptr[s]);
    a.row_stride = values->row_stride;
    a.drow_stride = dvalues->row_stride;
    a.N = N;
    a.S = m->S;
    a.D = m->D;
    a.R = m->R;
    a.lo = m->D - m->R;
    a.eps = m->eps;
    a.scale = m->scale;
    a.inv_R = 1.0f / (float)m->R;
    a.l_sm = l_sm;
    a.l_sn = l_sn;
    a.g_sm = g_sm;
    a.g_sn = g_sn;
    a.part_stride = M * m->R;
    const std::vector<Group> groups = plan_groups(m, ms);
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group& g = groups[gi];
      // later groups add to the gradient rows the first group wrote
      const bool acc = m->accumulate_dvalues != 0 || gi > 0;
      const void* fn = multi_bwd_ptr(ms, g.mq, acc);
      if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no multi-query backward kernel for this shape");
      a.tpt = 1;
      a.ticket = nullptr;
      if (!m->deterministic && N >= 2 * (int64_t)pl.P && N < kMaxTicketTokens) {
        a.tpt = tokens_per_ticket(N, pl.P,
                                  (double)((acc ? 3 : 2) * m->S + g.mq) * m->D * ms.base.esz,
                                  30.0, 16);
        a.ticket = reinterpret_cast<uint32_t*>(ws);
        void* targ = a.ticket;
        st = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &targ, stream, "ticket reset launch");
        if (st != ATTNRES_OK) return st;
      }
      a.M = g.cnt;
      a.query = static_cast<const char*>(queries) + (int64_t)g.m0 * m->R * ms.base.esz;
      a.lse = lse + g.m0 * l_sm;
      a.dout = static_cast<const char*>(dout) + g.m0 * g_sm * ms.base.esz;
      a.part = reinterpret_cast<float*>(ws + pl.off_part) + (int64_t)g.m0 * m->R;
      st = launch(fn, pl.P, 1, ms.threads, multi_bwd_lds(ms, g.mq), &a, stream,
                  "multi-query backward launch");
      if (st != ATTNRES_OK) return st;
    }
  }
  // dq [M, R]: the partial rows are [P, M * R]; the finaliser sums them as one long row
  FinArgs fa;
  std::memset(&fa, 0, sizeof fa);
  fa.part_du = reinterpret_cast<const float*>(ws + pl.off_part);
  fa.P = pl.P;
  fa.R = (int)(M * m->R);
  fa.D = 0;
  fa.cols = (int)(M * m->R);
  fa.query = queries;
  fa.dq = dq;
  return launch(finalize_kernel_ptr(ms.base.bf16), (fa.cols + kFinCols - 1) / kFinCols, 1,
                kFinCols * kFinPhases, 0, &fa, stream, "finalize launch");
}

}  // extern "C"

// ====================================================================== selected-query read

namespace {

constexpr size_t kMaxSelPartialBytes = size_t(1) << 30;  // cap on the partial bank rows

attnres_multi_desc multi_of(const attnres_selected_desc* d) {
  attnres_multi_desc m;
  std::memset(&m, 0, sizeof m);
  m.S = d->S;
  m.D = d->D;
  m.R = d->R;
  m.M = d->K;
  m.dtype = d->dtype;
  m.N = d->N;
  m.eps = d->eps;
  m.scale = d->scale;
  m.layout = ATTNRES_TOKEN_MAJOR;
  m.deterministic = d->deterministic;
  m.accumulate_dvalues = d->accumulate_dvalues;
  return m;
}

// The selected-query kernels are the multi-query kernels with per-token queries, built for groups
// of two queries and one or two chunks per thread. The forward takes the two-query read's
// workgroup shape (four waves when the sources fit their bucket: most bytes in flight per CU). The
// backward takes eight waves with the fewest chunks per thread: its per-token bank update keeps
// the query gradients and their partial rows live beside the sources, which at two chunks per
// thread spills heavily (measured 2.9x slower at S = 10, D = 4096 bf16).
attnres_status make_sel_shape(const attnres_selected_desc* d, MultiShape* ms, bool backward) {
  if (!d) return fail(ATTNRES_ERR_INVALID_ARG, "desc is NULL");
  if (d->E < 1) return fail(ATTNRES_ERR_INVALID_ARG, "E=%d: the bank needs a row", d->E);
  // the kernels address a workgroup's partial bank rows with 32-bit signed byte offsets
  if (d->R >= 1 && (int64_t)d->E * d->R * 4 >= (int64_t(1) << 31))
    return fail(ATTNRES_ERR_UNSUPPORTED, "bank of %d x %d: 2 GiB or more of FP32 partial rows",
                d->E, d->R);
  const attnres_multi_desc m = multi_of(d);
  attnres_status st = make_multi_shape(&m, ms, backward);
  if (st == ATTNRES_OK && ms->ch > 2) {  // four-chunk rows: the eight-wave shape
    *ms = MultiShape();
    st = make_multi_shape(&m, ms, true);
  }
  if (st != ATTNRES_OK) return st;
  if (ms->ch > 2)
    return fail(ATTNRES_ERR_UNSUPPORTED, "selected-query read: D=%d is too wide", d->D);
  // the forward runs up to four slots per launch with one chunk per thread (as the multi-query
  // read); the backward also four with one chunk per thread and at most 10 sources, else two (its
  // per-token bank update needs the registers of two-chunk rows)
  if (!backward)
    ms->mq_max = (ms->ch == 1 && ms->sb <= 12) ? kMaxGroupQueries : 2;
  else
    ms->mq_max = (ms->ch == 1 && ms->sb <= 10) ? kMaxGroupQueries : 2;
  return ATTNRES_OK;
}

// The backward's partial bank rows: in LDS when the whole [E, R] FP32 bank fits beside the exchange
// buffers within one workgroup's LDS allocation, else per-workgroup global blocks. Either way the
// workspace holds P blocks of E * R floats for the finaliser. (The eight-wave backward holds one
// workgroup per CU for its registers, so a large LDS block costs no occupancy there; the host
// takes the occupancy with the LDS size into account either way.)
constexpr size_t kSelLdsCap = 160 * 1024;

struct SelBwdPlan {
  int P = 0;
  bool lds_bank = false;
  size_t bank_lds = 0;  // LDS bytes of the partial bank rows (0 with global blocks)
  size_t off_part = 256, bytes = 256;
};

const void* sel_bwd_ptr(const MultiShape& ms, bool acc, int mq) {
  return ms.base.bf16 ? sel_bwd_kernel_ptr_bf16(ms.ch, ms.sb, ms.full, acc, mq)
                      : sel_bwd_kernel_ptr_f32(ms.ch, ms.sb, ms.full, acc, mq);
}

attnres_status plan_sel_bwd(const attnres_selected_desc* d, const MultiShape& ms,
                            SelBwdPlan* pl) {
  // the first (largest) group's kernel and exchange size the bank placement and the grid
  const attnres_multi_desc m = multi_of(d);
  const int mq = plan_groups(&m, ms)[0].mq;
  const void* fn = sel_bwd_ptr(ms, d->accumulate_dvalues != 0, mq);
  if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no selected-query backward kernel for this shape");
  DevFacts f;
  attnres_status st = device_facts(&f);
  if (st != ATTNRES_OK) return st;
  const size_t row = (size_t)d->E * d->R * sizeof(float);
  const size_t base = multi_bwd_lds(ms, mq);
  pl->lds_bank = base + row <= std::min<size_t>(kSelLdsCap, (size_t)f.lds_per_block);
  pl->bank_lds = pl->lds_bank ? row : 0;
  int per_cu = 0;
  st = blocks_per_cu(fn, ms.threads, base + pl->bank_lds, &per_cu, 8);
  if (st != ATTNRES_OK) return st;
  const int64_t cap = std::max<int64_t>(1, (int64_t)(kMaxSelPartialBytes / row));
  pl->P = (int)std::min<int64_t>(std::min<int64_t>(d->N, (int64_t)f.cus * per_cu), cap);
  pl->off_part = 256;
  pl->bytes = align256(pl->off_part + (size_t)pl->P * row);
  return ATTNRES_OK;
}

attnres_status check_ids(const int64_t* ids, int64_t N) {
  if (N > 0 && (!ids || !aligned(ids, 8)))
    return fail(ids ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "ids NULL or misaligned");
  return ATTNRES_OK;
}

// Slot counts for which the selected backward tries the matrix-core kernels (see its dispatch).
bool sel_mfma_slots(const attnres_selected_desc* d, const MultiShape& ms) {
  return d->K > ms.mq_max || (d->K >= 4 && d->S + d->K <= 16);
}

}  // namespace

extern "C" {

attnres_status attnres_selected_fwd_workspace_bytes(const attnres_selected_desc* d,
                                                    size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  MultiShape ms;
  attnres_status st = make_sel_shape(d, &ms, false);
  if (st != ATTNRES_OK) return st;
  *bytes = kFwdWorkspaceBytes;
  return ATTNRES_OK;
}

attnres_status attnres_selected_workspace_bytes(const attnres_selected_desc* d, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(ATTNRES_ERR_INVALID_ARG, "bytes is NULL");
  MultiShape ms;
  attnres_status st = make_sel_shape(d, &ms, true);
  if (st != ATTNRES_OK) return st;
  SelBwdPlan pl;
  if ((st = plan_sel_bwd(d, ms, &pl)) != ATTNRES_OK) return st;
  *bytes = pl.bytes;
  // or the matrix-core backward's, when it may serve the call (dense rows assumed here)
  if (ms.base.bf16 && sel_mfma_slots(d, ms) && d->N > 0) {
    MultiBwdPlan mp;
    if (plan_mfma_bwd(d->S, d->D, d->R, d->K, true, d->E, d->N, d->accumulate_dvalues != 0, d->D,
                      d->D, &mp) == ATTNRES_OK &&
        mp.mfma)
      *bytes = std::max(*bytes, mp.bytes);
    g_err.clear();
  }
  return ATTNRES_OK;
}

attnres_status attnres_stream_probe(const void* const* in_rows, int32_t n_in,
                                    void* const* out_rows, int32_t n_out, int64_t n_rows,
                                    int64_t row_bytes, int32_t chunks_per_thread,
                                    int32_t blocks_per_cu, void* stream) {
  g_err.clear();
  if (!in_rows || !out_rows) return fail(ATTNRES_ERR_INVALID_ARG, "stream arrays are NULL");
  if (n_in < 1 || n_in > kProbeMaxStreams || n_out < 1 || n_out > kProbeMaxStreams)
    return fail(ATTNRES_ERR_INVALID_ARG, "n_in=%d, n_out=%d: 1 .. %d streams each", n_in, n_out,
                kProbeMaxStreams);
  const void* fn = stream_probe_kernel_ptr(chunks_per_thread);
  if (!fn || blocks_per_cu < 1 || blocks_per_cu > 64)
    return fail(ATTNRES_ERR_INVALID_ARG, "chunks_per_thread=%d (1, 2 or 4), blocks_per_cu=%d "
                "(1 .. 64)", chunks_per_thread, blocks_per_cu);
  if (n_rows < 0 || row_bytes < 16 || row_bytes % 16 != 0)
    return fail(ATTNRES_ERR_INVALID_ARG, "n_rows=%lld, row_bytes=%lld: rows of whole 16-byte "
                "chunks", (long long)n_rows, (long long)row_bytes);
  ProbeArgs a;
  std::memset(&a, 0, sizeof a);
  for (int j = 0; j < n_in; ++j) {
    if (!in_rows[j] || !aligned(in_rows[j], 16))
      return fail(ATTNRES_ERR_ALIGNMENT, "input stream %d NULL or not 16-byte aligned", j);
    a.in[j] = in_rows[j];
  }
  for (int j = 0; j < n_out; ++j) {
    if (!out_rows[j] || !aligned(out_rows[j], 16))
      return fail(ATTNRES_ERR_ALIGNMENT, "output stream %d NULL or not 16-byte aligned", j);
    a.out[j] = out_rows[j];
  }
  std::vector<Range> ins, outs;
  for (int j = 0; j < n_in; ++j)
    ins.push_back(rows_range(a.in[j], n_rows, row_bytes, (int)row_bytes, 1, "in"));
  for (int j = 0; j < n_out; ++j)
    outs.push_back(rows_range(a.out[j], n_rows, row_bytes, (int)row_bytes, 1, "out"));
  attnres_status st = check_disjoint(outs, ins);
  if (st != ATTNRES_OK) return st;
  if (n_rows == 0) return ATTNRES_OK;
  a.n_in = n_in;
  a.n_out = n_out;
  a.n_rows = n_rows;
  a.row_chunks = row_bytes / 16;
  DevFacts f;
  if ((st = device_facts(&f)) != ATTNRES_OK) return st;
  const int64_t chunks = n_rows * a.row_chunks;
  const int grid = (int)std::min<int64_t>((chunks + 255) / 256, (int64_t)f.cus * blocks_per_cu);
  return launch(fn, grid, 1, 256, 0, &a, stream, "stream probe launch");
}

attnres_status attnres_selected_ids_flag(const void* workspace, size_t workspace_bytes,
                                         int32_t clear, int32_t* flag, void* stream) {
  g_err.clear();
  if (!flag) return fail(ATTNRES_ERR_INVALID_ARG, "flag is NULL");
  if (!workspace || workspace_bytes < kFwdWorkspaceBytes || !aligned(workspace, 256))
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace NULL, smaller than %zu bytes or not "
                "256-byte aligned", kFwdWorkspaceBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t* word = static_cast<uint32_t*>(const_cast<void*>(workspace)) + kCtrIdFlag;
  uint32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, word, sizeof host, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess && clear) e = hipMemsetAsync(word, 0, sizeof host, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return report_hip(e, "reading the id flag");
  *flag = host != 0u;
  return ATTNRES_OK;
}

attnres_status attnres_selected_fwd(const attnres_selected_desc* d, const attnres_sources* values,
                                    const void* bank, const int64_t* ids, void* y, float* lse,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  MultiShape ms;
  attnres_status st = make_sel_shape(d, &ms, false);
  if (st != ATTNRES_OK) return st;
  if (workspace && (workspace_bytes < kFwdWorkspaceBytes || !aligned(workspace, 256)))
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace: %zu bytes given, %zu (256-byte aligned) "
                "needed", workspace_bytes, kFwdWorkspaceBytes);
  if (!workspace && workspace_bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "forward workspace is NULL but workspace_bytes = %zu",
                workspace_bytes);
  const attnres_multi_desc m = multi_of(d);
  const attnres_desc d1 = single_desc(&m);
  if ((st = check_param(bank, true, ms.base.esz, "bank")) != ATTNRES_OK) return st;
  if ((st = check_ids(ids, d->N)) != ATTNRES_OK) return st;
  if (d->N == 0) return ATTNRES_OK;
  MultiFwdArgs a;
  std::memset(&a, 0, sizeof a);
  if ((st = check_sources(&d1, ms.base, values, "values", a.src)) != ATTNRES_OK) return st;
  if (!y || !aligned(y, 16))
    return fail(y ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "y NULL or misaligned");
  if (!lse || !aligned(lse, 4))
    return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
  const int64_t N = d->N, K = d->K;
  std::vector<Range> ins, outs;
  for (int s = 0; s < d->S; ++s)
    ins.push_back(rows_range(a.src[s], N, values->row_stride, d->D, ms.base.esz, "values"));
  ins.push_back(rows_range(bank, d->E, d->R, d->R, ms.base.esz, "bank"));
  ins.push_back(rows_range(ids, N, K, (int)K, 8, "ids"));
  outs.push_back(rows_range(y, N * K, d->D, d->D, ms.base.esz, "y"));
  outs.push_back(rows_range(lse, N * K, 1, 1, 4, "lse"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  DevFacts f;
  if ((st = device_facts(&f)) != ATTNRES_OK) return st;

  // Three to sixteen bf16 slots, the bank staged in LDS: one pass through the matrix-core forward
  // when it applies.
  {
    bool used = false;
    st = try_mfma_fwd(d->S, d->D, d->R, (int)K, d->eps, d->scale, ms.base.bf16, a.src,
                      values->row_stride, N, bank, ids, d->E, y, d->D, K * d->D, lse, 1, K,
                      workspace, f, stream, &used);
    if (st != ATTNRES_OK || used) return st;
  }

  const std::vector<Group> groups = plan_groups(&m, ms);
  // occupancy of the largest group's kernel (the first) sizes the grid of every group
  const void* fn0 = sel_fwd_kernel_ptr(ms.base.bf16, ms.ch, ms.sb, ms.full, groups[0].mq);
  if (!fn0) return fail(ATTNRES_ERR_UNSUPPORTED, "no selected-query forward kernel for this shape");
  int per_cu = 0;
  st = blocks_per_cu(fn0, ms.threads, multi_fwd_lds(ms, groups[0].mq, false), &per_cu, 8);
  if (st != ATTNRES_OK) return st;
  const int64_t resident = (int64_t)f.cus * per_cu;
  const bool dyn = workspace != nullptr && N >= 2 * resident && N < kMaxTicketTokens;
  const int64_t slots = resident * (dyn ? 1 : 8);
  a.row_stride = values->row_stride;
  a.N = N;
  a.S = d->S;
  a.D = d->D;
  a.R = d->R;
  a.lo = d->D - d->R;
  a.eps = d->eps;
  a.scale = d->scale;
  a.inv_R = 1.0f / (float)d->R;
  a.y_sm = d->D;
  a.y_sn = K * d->D;
  a.l_sm = 1;
  a.l_sn = K;
  a.sel.bank = bank;
  a.sel.ids = ids;
  a.sel.E = d->E;
  a.sel.K = (int)K;
  a.sel.id_flag = workspace ? static_cast<uint32_t*>(workspace) + kCtrIdFlag : nullptr;
  for (const Group& g : groups) {
    const void* fn = sel_fwd_kernel_ptr(ms.base.bf16, ms.ch, ms.sb, ms.full, g.mq);
    if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no selected-query forward kernel for this shape");
    const size_t lds = multi_fwd_lds(ms, g.mq, false);
    a.tpt = dyn ? tokens_per_ticket(N, slots, (double)(d->S + g.cnt) * d->D * ms.base.esz, 55.0, 1)
                : 1;
    a.ticket = nullptr;
    if (dyn) {
      a.ticket = static_cast<uint32_t*>(workspace);
      void* targ = a.ticket;
      st = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &targ, stream, "ticket reset launch");
      if (st != ATTNRES_OK) return st;
    }
    a.M = g.cnt;
    a.sel.m0 = g.m0;
    a.y = static_cast<char*>(y) + (int64_t)g.m0 * d->D * ms.base.esz;
    a.lse = lse + g.m0;
    const int grid = (int)std::min<int64_t>((N + a.tpt - 1) / a.tpt, slots);
    st = launch(fn, grid, 1, ms.threads, lds, &a, stream, "selected-query forward launch");
    if (st != ATTNRES_OK) return st;
  }
  return ATTNRES_OK;
}

attnres_status attnres_selected_bwd(const attnres_selected_desc* d, const attnres_sources* values,
                                    const void* bank, const int64_t* ids, const float* lse,
                                    const void* dout, const attnres_sources* dvalues, void* dbank,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  MultiShape ms;
  attnres_status st = make_sel_shape(d, &ms, true);
  if (st != ATTNRES_OK) return st;
  const attnres_multi_desc m = multi_of(d);
  const attnres_desc d1 = single_desc(&m);
  const int64_t N = d->N, K = d->K;
  MultiBwdArgs a;
  std::memset(&a, 0, sizeof a);
  const void* dptr[kMaxSources] = {nullptr};
  if ((st = check_param(bank, true, ms.base.esz, "bank")) != ATTNRES_OK) return st;
  if ((st = check_param(dbank, true, ms.base.esz, "dbank")) != ATTNRES_OK) return st;
  if ((st = check_ids(ids, N)) != ATTNRES_OK) return st;
  if (N > 0) {
    if ((st = check_sources(&d1, ms.base, values, "values", a.src)) != ATTNRES_OK) return st;
    if ((st = check_sources(&d1, ms.base, dvalues, "dvalues", dptr)) != ATTNRES_OK) return st;
    if (!lse || !aligned(lse, 4))
      return fail(lse ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "lse NULL or misaligned");
    if (!dout || !aligned(dout, 16))
      return fail(dout ? ATTNRES_ERR_ALIGNMENT : ATTNRES_ERR_INVALID_ARG, "dout NULL or misaligned");
  }
  if (!workspace) return fail(ATTNRES_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, 256)) return fail(ATTNRES_ERR_ALIGNMENT, "workspace not 256-byte aligned");
  std::vector<Range> ins, outs;
  if (N > 0) {
    for (int s = 0; s < d->S; ++s)
      ins.push_back(rows_range(a.src[s], N, values->row_stride, d->D, ms.base.esz, "values"));
    ins.push_back(rows_range(dout, N * K, d->D, d->D, ms.base.esz, "dout"));
    ins.push_back(rows_range(lse, N * K, 1, 1, 4, "lse"));
    ins.push_back(rows_range(ids, N, K, (int)K, 8, "ids"));
    for (int s = 0; s < d->S; ++s)
      outs.push_back(rows_range(dptr[s], N, dvalues->row_stride, d->D, ms.base.esz, "dvalues"));
  }
  ins.push_back(rows_range(bank, d->E, d->R, d->R, ms.base.esz, "bank"));
  outs.push_back(rows_range(dbank, d->E, d->R, d->R, ms.base.esz, "dbank"));
  if ((st = check_disjoint(outs, ins)) != ATTNRES_OK) return st;

  char* ws = static_cast<char*>(workspace);
  // one pass on matrix cores (dvalues rounded once) for bf16 slots that the slot-group kernel
  // would take in two or more launches, and for four or more slots that fit the compact tile with
  // the sources (S + K <= 16), when the shape and the bank fit. Measured at S = 10, N = 32768,
  // D = 4096, E = 8 (backward ms, slot groups / compact tile): three slots 1.70 / 1.82, four 2.09 /
  // 1.87; six 1.95 compact against 2.21 for the separate-tile kernel
  MultiBwdPlan mp;
  if (N > 0 && ms.base.bf16 && sel_mfma_slots(d, ms) && aligned(bank, 16)) {
    st = plan_mfma_bwd(d->S, d->D, d->R, (int)K, true, d->E, N, d->accumulate_dvalues != 0,
                       values->row_stride, dvalues->row_stride, &mp);
    if (st != ATTNRES_OK) return st;
  }
  if (mp.mfma) {
    if (workspace_bytes < mp.bytes)
      return fail(ATTNRES_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  mp.bytes);
    MfmaBwdArgs b;
    std::memset(&b, 0, sizeof b);
    for (int s = 0; s < d->S; ++s) {
      b.src[s] = a.src[s];
      b.dsrc[s] = const_cast<void*>(dptr[s]);
    }
    b.row_stride = values->row_stride;
    b.drow_stride = dvalues->row_stride;
    b.N = N;
    b.S = d->S;
    b.D = d->D;
    b.R = d->R;
    b.lo = d->D - d->R;
    b.M = (int)K;
    b.eps = d->eps;
    b.scale = d->scale;
    b.inv_R = 1.0f / (float)d->R;
    b.query = bank;
    b.lse = lse;
    b.l_sm = 1;
    b.l_sn = K;
    b.dout = dout;
    b.g_sm = d->D;
    b.g_sn = K * d->D;
    b.ids = ids;
    b.E = d->E;
    if ((st = launch_mfma_bwd(mp, b, true, d->accumulate_dvalues != 0, ws, stream)) != ATTNRES_OK)
      return st;
    FinArgs fm;
    std::memset(&fm, 0, sizeof fm);
    fm.part_du = reinterpret_cast<const float*>(ws + mp.off_part);
    fm.P = mp.P;
    fm.R = d->E * d->R;
    fm.D = 0;
    fm.cols = d->E * d->R;
    fm.query = bank;
    fm.dq = dbank;
    return launch(finalize_kernel_ptr(true), (fm.cols + kFinCols - 1) / kFinCols, 1,
                  kFinCols * kFinPhases, 0, &fm, stream, "finalize launch");
  }

  SelBwdPlan pl;
  if ((st = plan_sel_bwd(d, ms, &pl)) != ATTNRES_OK) return st;
  if (workspace_bytes < pl.bytes)
    return fail(ATTNRES_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                pl.bytes);
  if (pl.P > 0) {
    for (int s = 0; s < d->S; ++s) a.dsrc[s] = const_cast<void*>(dptr[s]);
    a.row_stride = values->row_stride;
    a.drow_stride = dvalues->row_stride;
    a.N = N;
    a.S = d->S;
    a.D = d->D;
    a.R = d->R;
    a.lo = d->D - d->R;
    a.eps = d->eps;
    a.scale = d->scale;
    a.inv_R = 1.0f / (float)d->R;
    a.l_sm = 1;
    a.l_sn = K;
    a.g_sm = d->D;
    a.g_sn = K * d->D;
    a.part = reinterpret_cast<float*>(ws + pl.off_part);
    a.part_stride = (int64_t)d->E * d->R;
    a.sel.bank = bank;
    a.sel.ids = ids;
    a.sel.E = d->E;
    a.sel.K = (int)K;
    const std::vector<Group> groups = plan_groups(&m, ms);
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const Group& g = groups[gi];
      const bool acc = d->accumulate_dvalues != 0 || gi > 0;
      const void* fn = sel_bwd_ptr(ms, acc, g.mq);
      if (!fn) return fail(ATTNRES_ERR_UNSUPPORTED, "no selected-query backward kernel");
      a.tpt = 1;
      a.ticket = nullptr;
      if (!d->deterministic && N >= 2 * (int64_t)pl.P && N < kMaxTicketTokens) {
        a.tpt = tokens_per_ticket(N, pl.P, (double)((acc ? 3 : 2) * d->S + 2) * d->D * ms.base.esz,
                                  30.0, 16);
        a.ticket = reinterpret_cast<uint32_t*>(ws);
        void* targ = a.ticket;
        st = launch(ticket_reset_kernel_ptr(), 1, 1, 64, 0, &targ, stream, "ticket reset launch");
        if (st != ATTNRES_OK) return st;
      }
      a.M = g.cnt;
      a.sel.m0 = g.m0;
      a.sel.first = gi == 0 ? 1 : 0;
      a.sel.lds_bank = pl.lds_bank ? 1 : 0;
      a.lse = lse + g.m0;
      a.dout = static_cast<const char*>(dout) + (int64_t)g.m0 * d->D * ms.base.esz;
      st = launch(fn, pl.P, 1, ms.threads, multi_bwd_lds(ms, g.mq) + pl.bank_lds, &a, stream,
                  "selected-query backward launch");
      if (st != ATTNRES_OK) return st;
    }
  }
  FinArgs fa;
  std::memset(&fa, 0, sizeof fa);
  fa.part_du = reinterpret_cast<const float*>(ws + pl.off_part);
  fa.P = pl.P;
  fa.R = d->E * d->R;
  fa.D = 0;
  fa.cols = d->E * d->R;
  fa.query = bank;
  fa.dq = dbank;
  return launch(finalize_kernel_ptr(ms.base.bf16), (fa.cols + kFinCols - 1) / kFinCols, 1,
                kFinCols * kFinPhases, 0, &fa, stream, "finalize launch");
}

}  // extern "C"
