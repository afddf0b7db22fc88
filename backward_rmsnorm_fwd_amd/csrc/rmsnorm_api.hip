// C ABI of the RMSNorm library: argument checks, launch plans, dispatch.
//
// Contract (page "Check an AI model calculation before accelerating it",
// section "The memory contract is part of the computation"): inputs are
// checked before anything is written, and unsupported inputs are rejected
// rather than rerouted (section "Adapting the kernel and moving to
// production": no silent fallback).  The accepted domain is widened from the
// page's (fp32/fp16, N <= 4096, a 64 MiB scratch cap on an M x N partial
// array) to fp32/fp16/bf16 and N <= 2^24, because the M x N partial array is
// replaced by a [P, N] one (P = number of backward workgroups) and rows longer
// than 65536 elements take the split-row plan (rmsnorm_split.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "../../include/layernorm.h"
#include "../../include/rmsnorm.h"
#include "../../include/rmsnorm_add.h"
#include "../../include/rmsnorm_cast.h"
#include "rmsnorm_fast.hpp"
#include "rmsnorm_fast_table.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"

namespace {

using namespace rmsnorm_hip;

// The plan is a pure function of its arguments (no device queries), so the
// workspace size and the order of every reduction are reproducible.  It is
// sized for MI355X: 256 compute units.
constexpr int kCUs = 256;
constexpr int kMaxChunksPreferred = 16;  // register-resident chunks per thread
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int64_t kMaxRowN = 65536;  // longest row handled by one workgroup

int elem_bytes(int dtype) { return dtype == RMSNORM_F32 ? 4 : 2; }

int pow2_at_least(int64_t v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

int pow2_at_most(int64_t v) {
  int p = 1;
  while (2 * static_cast<int64_t>(p) <= v) p <<= 1;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Widest vector (elements) such that rows and every pointer stay aligned.
int pick_vec(int64_t N, int esize, int align_bytes) {
  int vb = 16;
  while (vb > esize && ((N * esize) % vb != 0 || (align_bytes % vb) != 0)) vb >>= 1;
  return vb / esize;
}

int pointer_alignment(std::initializer_list<const void*> ptrs) {
  int a = 16;
  for (const void* p : ptrs) {
    if (!p) continue;
    const uintptr_t v = reinterpret_cast<uintptr_t>(p);
    while (a > 1 && (v % a) != 0) a >>= 1;
  }
  return a;
}

// ---- full-width (16-byte vector) configurations ----------------------------
//
// Chosen by measurement on MI355X, timing the whole forward -> backward rows
// -> backward reduce sequence (the order a training step runs them in, which
// differs from timing each kernel alone because each kernel inherits the
// previous one's dirty cache lines), nontemporal accesses throughout:
//  forward   few chunks per thread and several wavefronts per row keep the
//            most rows' loads in flight: 4 wavefronts x 2 chunks at N=4096,
//            1 x 2 at N=1024 (fp16), 4 x 3 at N=5120.
//  backward  x arrives in LDS by DMA (no VGPRs while in flight), 1-2 chunks
//            per thread, P = 512 workgroups: 4 x 2 at N=4096 (1024-thread
//            workgroups: step 225.1 us vs 230.2 us for 1 wavefront x 8
//            chunks; now 512 threads, below), 2 x 1 at N=1024 fp16 (441.8 us vs 465.3 us), 8 x 2 at
//            N=5120 (592.8 us vs 616.6 us).  Staging dy in LDS as well was
//            slower everywhere.  Rows needing more than 3 chunks at 16
//            wavefronts keep only the dgamma accumulators in registers (x in
//            LDS, weight re-read from cache).
//  shapes at 4-8 KiB rows, measured in the same three scopes: the
//            pipelined forward with 4 wavefronts x 2 chunks per row (4 rows
//            per 1024-thread workgroup, 512 workgroups) and bwd_fast with
//            512-thread workgroups (2 rows each, P = 512): 201.0 / 210.7 /
//            230.7 us per bf16 32768 x 4096 step against 207.2 / 220.8 /
//            245.4 us for 2 wavefronts x 4 chunks and 1024 threads (same GPU,
//            same session).  Each half helps alone (forward: rotating and
//            cold -5 us; backward: -2 to -4 us in all three); 256
//            forward workgroups, 8-wavefront rows, P = 256 or 1024, and
//            256-thread backward workgroups all measured slower.
//  row order of bwd_fast_kernel: reverse cyclic (the grid sweeps the matrix
//            back to front, against the forward's sweep).  bf16 32768 x 4096,
//            three timing scopes (step over one buffer set / steps over three
//            buffer sets in turn / forward + backward each after a 1 GiB
//            read): 206.1 / 220.6 / 245.9 us against 208.7 / 221.7 / 257.3
//            us for contiguous row blocks and 207.9 / 221.0 / 244.9 us for
//            the front-to-back sweep.  With the data out of cache, P
//            scattered streams cost the HBM more than one moving window.
struct Cfg {
  bool ok;
  int wpr, ch, block, greg, xlds;
};

#define RMSNORM_IS_LISTED_FWD(W, C, B, GR) \
  if (c.wpr == W && c.ch == C && c.block == B && c.greg == GR) return true;
bool listed_fwd(const Cfg& c) {
  RMSNORM_FWD_FAST_LIST(RMSNORM_IS_LISTED_FWD)
  return false;
}
#undef RMSNORM_IS_LISTED_FWD

#define RMSNORM_IS_LISTED_BWD(W, C, B, GR, XL) \
  if (c.wpr == W && c.ch == C && c.block == B && c.greg == GR && c.xlds == XL) return true;
bool listed_bwd(const Cfg& c) {
  RMSNORM_BWD_FAST_LIST(RMSNORM_IS_LISTED_BWD)
  return false;
}
#undef RMSNORM_IS_LISTED_BWD

Cfg plan_fast_fwd(int64_t nvec) {
  Cfg c{true, 1, 1, 256, 1, 0};
  if (nvec == 640) {
    // Rows of 640 vectors (bf16 5120): 5 wavefronts x 2 chunks fill the row
    // exactly; 210.5 us against 215.9 us for 4 x 3 in the 65536 x 5120 step.
    c.wpr = 5;
    c.ch = 2;
    c.block = 640;
    c.ok = listed_fwd(c);
    return c;
  }
  c.wpr = std::min(8, pow2_at_most(std::max<int64_t>(1, nvec / 128)));
  c.ch = static_cast<int>(ceil_div(nvec, 64 * c.wpr));
  if (c.ch > 16) {
    c.wpr = 16;
    c.ch = static_cast<int>(ceil_div(nvec, 1024));
  }
  c.block = c.wpr <= 2 ? 256 : (c.wpr <= 8 ? 512 : 1024);
  c.greg = (c.block == 1024 && c.ch > 8) ? 0 : 1;
  c.ok = listed_fwd(c);
  return c;
}

Cfg plan_fast_bwd(int64_t nvec) {
  Cfg c{true, 1, 1, 512, 1, 1};
  if (nvec < 256) {
    c.wpr = pow2_at_least(ceil_div(nvec, 64));
  } else {
    c.wpr = std::min(16, pow2_at_least(ceil_div(nvec, 128)));
  }
  c.ch = static_cast<int>(ceil_div(nvec, 64 * c.wpr));
  if (c.ch >= 4) c.greg = 0;  // long rows: weight re-read, x in LDS
  c.ok = listed_bwd(c);
  return c;
}

int64_t fast_bwd_partials(int64_t M, const Cfg& c) {
  const int64_t groups = c.block / (64 * c.wpr);
  const int64_t cap = c.greg ? 512 : 256;
  return std::min<int64_t>(ceil_div(M, groups), cap);
}

int64_t fast_bwd_lds(const Cfg& c, int64_t N, int es) {
  const int64_t groups = c.block / (64 * c.wpr);
  const int64_t sweep = 64 * c.wpr * (16 / es);
  const int64_t stage = c.xlds ? groups * N * es : 0;
  const int64_t comb = groups > 1 ? groups * sweep * 4 : 0;
  return std::max(stage, comb);
}

// ---- software-pipelined full-width configurations --------------------------
//
// Measured the same way (whole step, same GPU, same session; step medians):
//  forward   rows of 4-8 KiB: x staged in LDS by DMA one row ahead, rows
//            interleaved across 512 workgroups of 1024 threads, 2 wavefronts
//            x 4 chunks per row: 207.8 us per bf16 32768x4096 step against
//            238.4 us with fwd_fast 4 x 2 (the backward unchanged); since
//            4 wavefronts x 2 chunks (see the full-width notes above).  Shorter
//            and longer rows (fp16 N=1024, bf16 N=5120) measured slower
//            pipelined than fwd_fast and keep it.
//  backward  rows up to 4 KiB: one chunk per thread, dy prefetched into
//            registers, x into LDS, 256 interleaving workgroups: 443.2 us per
//            fp16 262144x1024 step against 462.5 us with bwd_fast;
//            rows of 8-16 KiB: one chunk per thread over 16 wavefronts, x and
//            dy both prefetched into LDS: 542.0 us per bf16 65536x5120 step
//            against 602.0 us.  Rows of 4-8 KiB keep bwd_fast (the pipelined
//            variants measured 214-241 us against 207.8 us per step).
struct PipeCfg {
  bool ok;
  int wpr, ch, block, lds_flag;  // lds_flag: XL (forward) or DLDS (backward)
};

#define RMSNORM_IS_LISTED_PIPE(W, C, B, F) \
  if (c.wpr == W && c.ch == C && c.block == B && c.lds_flag == F) return true;
bool listed_pipe_fwd(const PipeCfg& c) {
  RMSNORM_FWD_PIPE_LIST(RMSNORM_IS_LISTED_PIPE)
  return false;
}
bool listed_pipe_bwd(const PipeCfg& c) {
  RMSNORM_BWD_PIPE_LIST(RMSNORM_IS_LISTED_PIPE)
  return false;
}
#undef RMSNORM_IS_LISTED_PIPE

constexpr int64_t kPipeFwdWorkgroups = 512;
constexpr int64_t kPipeBwdWorkgroups = 256;

PipeCfg plan_pipe_fwd(int64_t nvec) {
  PipeCfg c{false, 4, 1, 1024, 1};
  if (nvec <= 256 || nvec > 512) return c;
  c.ch = static_cast<int>(ceil_div(nvec, 64 * c.wpr));
  c.ok = listed_pipe_fwd(c);
  return c;
}

PipeCfg plan_pipe_bwd(int64_t nvec) {
  PipeCfg c{false, 1, 1, 1024, 0};
  if (nvec <= 256) {
    c.wpr = pow2_at_least(ceil_div(nvec, 64));
  } else if (nvec == 640) {
    // Rows of 640 vectors (bf16 5120): 10 wavefronts x 1 chunk in a
    // 640-thread workgroup fill the row exactly, where 16 wavefronts leave
    // 384 of 1024 lanes idle; 332.5 us against 362.5 us for stage 1 in the
    // 65536 x 5120 step (step 547.2 against 577.2 us).  512 workgroups
    // instead of 256 measured slower (394.5 us).
    c.wpr = 10;
    c.block = 640;
    c.lds_flag = 1;
  } else if (nvec > 512 && nvec <= 1024) {
    c.wpr = 16;
    c.lds_flag = 1;
  } else {
    return c;
  }
  c.ok = listed_pipe_bwd(c);
  return c;
}

int64_t pipe_groups(const PipeCfg& c) { return c.block / (64 * c.wpr); }

int64_t pipe_fwd_grid(int64_t M, const PipeCfg& c) {
  return std::min<int64_t>(ceil_div(M, pipe_groups(c)), kPipeFwdWorkgroups);
}

int64_t pipe_bwd_partials(int64_t M, const PipeCfg& c) {
  return std::min<int64_t>(ceil_div(M, pipe_groups(c)), kPipeBwdWorkgroups);
}

// Two stage buffers of G rows of x (and of dy with DLDS); the backward reuses
// the area for its [G][chunk sweep] float32 combine at the end.
int64_t pipe_lds(const PipeCfg& c, int64_t N, int es, bool backward) {
  const int64_t groups = pipe_groups(c);
  const int64_t sets = (backward && c.lds_flag) ? 2 : 1;
  const int64_t stage = (backward || c.lds_flag) ? 2 * sets * groups * N * es : 0;
  const int64_t comb = (backward && groups > 1) ? groups * 64 * c.wpr * (16 / es) * 4 : 0;
  return std::max(stage, comb);
}

// ---- long rows (16 KiB < row <= 128 KiB): bwd_longrow_kernel --------------
//
// One 512-thread workgroup per row keeps x (LDS), dy and the dgamma
// accumulators on chip for rows up to 128 KiB (8 KiB per chunk, <= 16
// chunks), P = min(M, 256) workgroups (one per compute unit: the row of x
// fills most of the LDS).  bf16 2048x65536: 187.9 us for stage 1 + stage 2
// against 410.1 us with the 1024-thread bwd_fast (which spilled).
constexpr int64_t kLongBwdWorkgroups = 256;

int plan_long_bwd(int64_t nvec) {
  if (nvec <= 1024 || nvec > 8192) return 0;
  const int ch = static_cast<int>(ceil_div(nvec, 512));
#define RMSNORM_IS_LISTED_LONG(C) if (ch == C) return ch;
  RMSNORM_BWD_LONG_LIST(RMSNORM_IS_LISTED_LONG)
#undef RMSNORM_IS_LISTED_LONG
  return 0;
}

// ---- generic (any alignment) configurations --------------------------------

struct Rows {
  int tpr;     // threads per row
  int chunks;  // vector accesses per thread
};

// Threads per row: one wavefront while the row fits in kMaxChunksPreferred
// chunks per lane, else the smallest power-of-two workgroup that does, up
// to 1024 threads (more chunks per thread beyond that).
Rows pick_rows(int64_t N, int vec) {
  const int64_t nvec = ceil_div(N, vec);
  for (int tpr = kWave; tpr <= 1024; tpr <<= 1) {
    const int64_t ch = ceil_div(nvec, tpr);
    if (ch <= kMaxChunksPreferred) return {tpr, static_cast<int>(ch)};
  }
  return {1024, static_cast<int>(ceil_div(nvec, 1024))};
}

int64_t generic_bwd_partials(int64_t M, int64_t N, int vec) {
  const Rows rw = pick_rows(N, vec);
  if (rw.tpr == kWave) {
    const int maxc = pow2_at_least(rw.chunks);
    const int groups = 8;  // wavefronts (rows) per workgroup
    const int per_cu = maxc <= 2 ? 4 : (maxc <= 4 ? 2 : 1);
    return std::min<int64_t>(ceil_div(M, groups), static_cast<int64_t>(kCUs) * per_cu);
  }
  const int per_cu = std::max(1, 1024 / rw.tpr);
  return std::min<int64_t>(M, static_cast<int64_t>(kCUs) * per_cu);
}

// ---- split rows (N > kMaxRowN): rmsnorm_split.hip ----------------------------
//
// Segments of 16 KiB; P row blocks.  The forward aims at 2048 workgroups.
// The backward keeps at least 16 rows per block where M allows (each block
// writes one float32 partial row, so fewer rows per block cost more partial
// traffic) and otherwise aims at 1024 workgroups.  The grid stays below 2^24
// workgroups of 256 threads.
constexpr int64_t kSplitFwdWorkgroups = 2048;
constexpr int64_t kSplitBwdWorkgroups = 1024;
constexpr int64_t kSplitBwdRowsPerBlock = 16;
constexpr int64_t kMaxSplitGrid = (int64_t(1) << 24) - 1;

bool split_rows(int64_t N) { return N > kMaxRowN; }

// Rows the generic kernels would otherwise take (no full-width kernel at
// this alignment: odd N, narrow alignment, or float32 rows over 128 KiB)
// run the split plan too once they are longer than kGenericSplitMinN.
// Measured per kernel on one MI355X (generic -> split, us): fp32
// 2048 x 65536 backward 906 -> 516; fp32 4096 x 40000 backward 836 -> 595;
// bf16 2048 x 65535 (2-byte accesses) forward 992 -> 416, backward
// 2802 -> 1040; fp16 8192 x 20001 backward 10865 -> 1313.  Full-width rows
// keep their kernels: bf16 2048 x 40000 forward 53 against 83, backward
// 109 against 142 split.
constexpr int64_t kGenericSplitMinN = 16384;

int64_t split_nseg(int64_t N, int es) { return ceil_div(N, split_segment_elems(es)); }

int64_t split_partials(int64_t M, int64_t N, int es, bool backward) {
  const int64_t nseg = split_nseg(N, es);
  int64_t P = backward ? std::max(ceil_div(M, kSplitBwdRowsPerBlock),
                                  ceil_div(kSplitBwdWorkgroups, nseg))
                       : ceil_div(kSplitFwdWorkgroups, nseg);
  P = std::min(P, kMaxSplitGrid / nseg);
  return std::max<int64_t>(1, std::min(P, M));
}

// Row blocks of a split pass that keeps no column sums (every forward pass,
// LayerNorm's backward stats pass, RMSNorm's backward apply pass): its
// blocking is free, and one row per block keeps the most rows in flight.
// Measured (us, blocks of the column-sum pass or of 2048 forward workgroups
// -> one row per block): LayerNorm stage 1 bf16 2048 x 65536 251.6 -> 230.0,
// bf16 1024 x 131072 261.0 -> 232.8, fp32 512 x 262144 494.0 -> 471.1;
// RMSNorm stage 1 bf16 1024 x 131072 240.9 -> 230.6, fp32 512 x 262144
// 516.2 -> 455.3, bf16 2048 x 65535 1050.6 -> 891.0; RMSNorm forward fp32
// 512 x 262144 289.1 -> 260.1, bf16 2048 x 65535 417.7 -> 189.6, fp16
// 8192 x 20001 579.4 -> 244.2.  Only with very few rows (fp16 8 x 2^24:
// forward 289.7 -> 309.6, stage 1 385.3 -> 402.3) does the extra weight
// traffic of the smaller blocks show.  LayerNorm's forward keeps its blocks
// (bf16 1024 x 131072 145.1 against 193.5 us one row per block).
int64_t split_free_partials(int64_t M, int64_t nseg) {
  return std::max<int64_t>(1, std::min(M, kMaxSplitGrid / nseg));
}

// Backward workspace of the split plan: part[P, N], then the per-(row,
// segment) dot partials [M, nseg], then the per-row coefficients [M], each
// starting on a 16-byte boundary.
struct SplitWorkspace {
  int64_t part_floats, dotp_offset, coef_offset, total_floats;
};

SplitWorkspace split_workspace_for(int64_t P, int64_t M, int64_t N, int es) {
  SplitWorkspace w;
  w.part_floats = P * N;
  w.dotp_offset = ceil_div(w.part_floats, 4) * 4;
  w.coef_offset = w.dotp_offset + ceil_div(M * split_nseg(N, es), 4) * 4;
  w.total_floats = w.coef_offset + ceil_div(M, 4) * 4;
  return w;
}

SplitWorkspace split_workspace(int64_t M, int64_t N, int es) {
  return split_workspace_for(split_partials(M, N, es, true), M, N, es);
}

// Whether a full-width kernel takes rows of N at access width vec.
bool full_width_plan(int64_t N, int es, int vec, bool backward) {
  if (vec * es != 16 || N > kMaxRowN) return false;
  const int64_t nvec = N / vec;
  if (backward) return plan_pipe_bwd(nvec).ok || plan_long_bwd(nvec) || plan_fast_bwd(nvec).ok;
  return plan_pipe_fwd(nvec).ok || plan_fast_fwd(nvec).ok;
}

bool use_split(int64_t N, int es, int vec, bool backward) {
  return split_rows(N) || (N > kGenericSplitMinN && !full_width_plan(N, es, vec, backward));
}

// Backward workgroup count P: a function of (M, N, dtype) only, computed
// with the vector width that N alone allows (pointer alignment can only
// change which kernel runs, never P; a layout narrower than that runs the
// split or generic kernels on the same P).
int64_t bwd_partials(int64_t M, int64_t N, int dtype) {
  if (M <= 0) return 0;
  const int es = elem_bytes(dtype);
  if (split_rows(N)) return split_partials(M, N, es, true);
  const int vec = pick_vec(N, es, 16);
  if (vec * es == 16) {
    const PipeCfg pc = plan_pipe_bwd(N / vec);
    if (pc.ok) return pipe_bwd_partials(M, pc);
    if (plan_long_bwd(N / vec)) return std::min<int64_t>(M, kLongBwdWorkgroups);
    const Cfg c = plan_fast_bwd(N / vec);
    if (c.ok) return fast_bwd_partials(M, c);
  }
  if (N > kGenericSplitMinN) return split_partials(M, N, es, true);
  return generic_bwd_partials(M, N, vec);
}

// Backward workspace: [P, N] partials, and past kGenericSplitMinN (where a
// layout may run the split kernels) the split plan's row sums after them.
int64_t bwd_workspace_floats(int64_t M, int64_t N, int dtype) {
  const int64_t P = bwd_partials(M, N, dtype);
  if (N > kGenericSplitMinN) return split_workspace_for(P, M, N, elem_bytes(dtype)).total_floats;
  return P * N;
}

// Stage 2 over a [P, N] block of partial column sums.
void fill_reduce_plan(int64_t P, int64_t N, rmsnorm_plan_t* p) {
  std::memset(p, 0, sizeof(*p));
  p->partials = P;
  p->vec = 1;
  if (N % 4 == 0 && N <= 8192) {
    p->kernel = RMSNORM_KERNEL_BWD_REDUCE16;
    p->block_threads = 256;
    p->grid = ceil_div(N, 16);
  } else if (N % 4 == 0) {
    // One wavefront slice per 4 partial rows, at most 16.
    p->kernel = RMSNORM_KERNEL_BWD_REDUCE_WIDE;
    p->block_threads = kWave * std::min(16, pow2_at_least(ceil_div(P, 4)));
    p->grid = ceil_div(N, 256);
  } else {
    p->kernel = RMSNORM_KERNEL_BWD_REDUCE;
    p->block_threads = 1024;
    p->grid = ceil_div(N, kWave);
  }
}

void fill_plan(int64_t M, int64_t N, int dtype, int pass, int align, rmsnorm_plan_t* p) {
  std::memset(p, 0, sizeof(*p));
  const int es = elem_bytes(dtype);
  const int vec = pick_vec(N, es, align);
  const bool full = vec * es == 16;
  if (pass == RMSNORM_PASS_BWD_REDUCE) {
    fill_reduce_plan(bwd_partials(M, N, dtype), N, p);
    return;
  }
  p->vec = vec;
  if (use_split(N, es, vec, pass == RMSNORM_PASS_BWD_ROWS)) {
    const bool bwd = pass == RMSNORM_PASS_BWD_ROWS;
    const int64_t nseg = split_nseg(N, es);
    p->kernel = bwd ? RMSNORM_KERNEL_BWD_SPLIT : RMSNORM_KERNEL_FWD_SPLIT;
    p->segments = static_cast<int32_t>(nseg);
    p->threads_per_row = static_cast<int32_t>(256 * nseg);
    p->chunks = split_chunks(vec, es);
    p->block_threads = 256;
    p->weight_in_regs = 1;
    const int64_t P = bwd ? bwd_partials(M, N, dtype) : split_free_partials(M, nseg);
    p->partials = bwd ? P : 0;
    p->grid = P * nseg;
    return;
  }
  if (pass == RMSNORM_PASS_FWD && full) {
    const PipeCfg pc = plan_pipe_fwd(N / vec);
    if (pc.ok) {
      p->kernel = RMSNORM_KERNEL_FWD_PIPE;
      p->threads_per_row = 64 * pc.wpr;
      p->chunks = pc.ch;
      p->block_threads = pc.block;
      p->weight_in_regs = 1;
      p->x_in_lds = pc.lds_flag;
      p->grid = pipe_fwd_grid(M, pc);
      p->lds_bytes = pipe_lds(pc, N, es, false);
      return;
    }
  }
  if (pass == RMSNORM_PASS_BWD_ROWS && full) {
    const PipeCfg pc = plan_pipe_bwd(N / vec);
    if (pc.ok) {
      p->kernel = RMSNORM_KERNEL_BWD_PIPE;
      p->threads_per_row = 64 * pc.wpr;
      p->chunks = pc.ch;
      p->block_threads = pc.block;
      p->weight_in_regs = 1;
      p->x_in_lds = 1;
      p->dy_in_lds = pc.lds_flag;
      p->partials = bwd_partials(M, N, dtype);
      p->grid = p->partials;
      p->lds_bytes = pipe_lds(pc, N, es, true);
      return;
    }
  }
  if (pass == RMSNORM_PASS_BWD_ROWS && full) {
    const int ch = plan_long_bwd(N / vec);
    if (ch) {
      p->kernel = RMSNORM_KERNEL_BWD_LONG;
      p->threads_per_row = 512;
      p->chunks = ch;
      p->block_threads = 512;
      p->x_in_lds = 1;
      p->partials = bwd_partials(M, N, dtype);
      p->grid = p->partials;
      p->lds_bytes = N * es;
      return;
    }
  }
  if (pass == RMSNORM_PASS_FWD && full) {
    const Cfg c = plan_fast_fwd(N / vec);
    if (c.ok) {
      p->kernel = RMSNORM_KERNEL_FWD_ROWS;
      p->threads_per_row = 64 * c.wpr;
      p->chunks = c.ch;
      p->block_threads = c.block;
      p->weight_in_regs = c.greg;
      const int64_t groups = c.block / (64 * c.wpr);
      p->grid = std::min<int64_t>(ceil_div(M, groups), int64_t(1) << 20);
      return;
    }
  }
  if (pass == RMSNORM_PASS_BWD_ROWS && full) {
    const Cfg c = plan_fast_bwd(N / vec);
    if (c.ok) {
      p->kernel = RMSNORM_KERNEL_BWD_ROWS;
      p->threads_per_row = 64 * c.wpr;
      p->chunks = c.ch;
      p->block_threads = c.block;
      p->weight_in_regs = c.greg;
      p->x_in_lds = c.xlds;
      p->partials = bwd_partials(M, N, dtype);
      p->grid = p->partials;
      p->lds_bytes = fast_bwd_lds(c, N, es);
      return;
    }
  }
  const Rows rw = pick_rows(N, vec);
  p->chunks = rw.chunks;
  p->threads_per_row = rw.tpr;
  if (pass == RMSNORM_PASS_FWD) {
    p->weight_in_regs = rw.tpr == kWave ? 1 : 0;
    if (rw.tpr == kWave) {
      p->kernel = RMSNORM_KERNEL_FWD_WAVE;
      p->block_threads = 256;
      const int64_t groups = p->block_threads / kWave;
      p->grid = std::min<int64_t>(ceil_div(M, groups), static_cast<int64_t>(kCUs) * 8);
    } else {
      p->kernel = RMSNORM_KERNEL_FWD_BLOCK;
      p->block_threads = rw.tpr;
      p->grid = std::min<int64_t>(M, static_cast<int64_t>(kCUs) * std::max(1, 2048 / rw.tpr));
    }
  } else {
    p->partials = bwd_partials(M, N, dtype);
    p->grid = p->partials;
    if (rw.tpr == kWave) {
      p->kernel = RMSNORM_KERNEL_BWD_WAVE;
      p->block_threads = 512;
      p->weight_in_regs = 1;
      p->lds_bytes = N * 4;
    } else {
      p->kernel = RMSNORM_KERNEL_BWD_BLOCK;
      p->block_threads = rw.tpr;
      const int64_t xbytes = N * es;
      p->x_in_lds = (xbytes + 1024 <= kMaxLdsBytes) ? 1 : 0;
      p->lds_bytes = p->x_in_lds ? xbytes : 0;
    }
  }
}

// Elements between the starts of consecutive rows of each matrix (N for a
// dense matrix).
struct RowStrides {
  int64_t x, y, dy, dx;
};

// ---- dispatch over the compile-time (dtype, vec, maxc) instantiations ----
// maxc (register chunk slots) is the next power of two >= chunks: up to 16
// for every vector width, and beyond that only where a 65536-wide row over
// 1024 threads needs it (32 for vec <= 2, 64 for vec = 1).

#define RMSNORM_MAXC_CASES(MACRO, DT, VEC) \
  case 1: MACRO(DT, VEC, 1); break;        \
  case 2: MACRO(DT, VEC, 2); break;        \
  case 4: MACRO(DT, VEC, 4); break;        \
  case 8: MACRO(DT, VEC, 8); break;        \
  case 16: MACRO(DT, VEC, 16); break;      \
  case 32: if constexpr (VEC <= 2) { MACRO(DT, VEC, 32); } break; \
  case 64: if constexpr (VEC <= 1) { MACRO(DT, VEC, 64); } break;

template <int DT, int VEC>
hipError_t fwd_dispatch(const rmsnorm_plan_t& p, const void* x, const void* g,
                        void* y, float* rstd, int64_t M, int N, float eps,
                        int offset, const RowStrides& ld, hipStream_t s) {
  hipError_t err = hipErrorInvalidValue;
  const int maxc = pow2_at_least(p.chunks);
#define FWD_LAUNCH(DT_, VEC_, MAXC_)                                              \
  err = (p.kernel == RMSNORM_KERNEL_FWD_WAVE)                                     \
            ? launch(fwd_wave_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads, 0, \
                     s, x, g, y, rstd, M, N, p.chunks, eps, offset, ld.x, ld.y)   \
            : launch(fwd_block_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads, 0, \
                     s, x, g, y, rstd, M, N, p.chunks, eps, offset, ld.x, ld.y)
  switch (maxc) { RMSNORM_MAXC_CASES(FWD_LAUNCH, DT, VEC) default: break; }
#undef FWD_LAUNCH
  return err;
}

template <int DT, int VEC>
hipError_t bwd_rows_dispatch(const rmsnorm_plan_t& p, const void* dy, const void* x,
                             const void* g, const float* rstd, void* dx, float* part,
                             int64_t M, int N, int offset, const RowStrides& ld,
                             hipStream_t s) {
  hipError_t err = hipErrorInvalidValue;
  const int maxc = pow2_at_least(p.chunks);
  const int64_t P = p.partials;
#define BWD_LAUNCH(DT_, VEC_, MAXC_)                                                   \
  if (p.kernel == RMSNORM_KERNEL_BWD_WAVE)                                             \
    err = launch(bwd_wave_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads,           \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P, ld.dy, ld.x, ld.dx);                             \
  else if (p.x_in_lds)                                                                 \
    err = launch(bwd_block_kernel<DT_, VEC_, MAXC_, true>, p.grid, p.block_threads,    \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P, ld.dy, ld.x, ld.dx);                             \
  else                                                                                 \
    err = launch(bwd_block_kernel<DT_, VEC_, MAXC_, false>, p.grid, p.block_threads,   \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P, ld.dy, ld.x, ld.dx)
  switch (maxc) { RMSNORM_MAXC_CASES(BWD_LAUNCH, DT, VEC) default: break; }
#undef BWD_LAUNCH
  return err;
}

template <int DT>
hipError_t fwd_by_vec(const rmsnorm_plan_t& p, const void* x, const void* g, void* y,
                      float* rstd, int64_t M, int N, float eps, int offset,
                      const RowStrides& ld, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  if (p.kernel == RMSNORM_KERNEL_FWD_ROWS || p.kernel == RMSNORM_KERNEL_FWD_PIPE) {
    const FastFwdArgs a{x, g, y, rstd, M, N, eps, offset, ld.x * es, ld.y * es};
    if (p.kernel == RMSNORM_KERNEL_FWD_ROWS)
      return fast_fwd_launch<DT>(p.threads_per_row / 64, p.chunks, p.block_threads,
                                 p.weight_in_regs, p.grid, a, s);
    return pipe_fwd_launch<DT>(p.threads_per_row / 64, p.chunks, p.block_threads, p.x_in_lds,
                               p.grid, p.lds_bytes, a, s);
  }
  switch (p.vec * es) {
    case 16: return fwd_dispatch<DT, 16 / es>(p, x, g, y, rstd, M, N, eps, offset, ld, s);
    case 8: return fwd_dispatch<DT, 8 / es>(p, x, g, y, rstd, M, N, eps, offset, ld, s);
    case 4: return fwd_dispatch<DT, 4 / es>(p, x, g, y, rstd, M, N, eps, offset, ld, s);
    case 2:
      if constexpr (es == 2) return fwd_dispatch<DT, 1>(p, x, g, y, rstd, M, N, eps, offset, ld, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t bwd_rows_by_vec(const rmsnorm_plan_t& p, const void* dy, const void* x,
                           const void* g, const float* rstd, void* dx, float* part,
                           int64_t M, int N, int offset, const RowStrides& ld, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  const FastBwdArgs a{dy, x, g, rstd, dx, part, M, N, offset, p.partials,
                      ld.dy * es, ld.x * es, ld.dx * es};
  switch (p.kernel) {
    case RMSNORM_KERNEL_BWD_ROWS:
      return fast_bwd_launch<DT>(p.threads_per_row / 64, p.chunks, p.block_threads,
                                 p.weight_in_regs, p.x_in_lds, p.lds_bytes, a, s);
    case RMSNORM_KERNEL_BWD_LONG:
      return long_bwd_launch<DT>(p.chunks, p.lds_bytes, a, s);
    case RMSNORM_KERNEL_BWD_PIPE:
      return pipe_bwd_launch<DT>(p.threads_per_row / 64, p.chunks, p.block_threads,
                                 p.dy_in_lds, p.lds_bytes, a, s);
    default: break;
  }
  switch (p.vec * es) {
    case 16: return bwd_rows_dispatch<DT, 16 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, ld, s);
    case 8: return bwd_rows_dispatch<DT, 8 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, ld, s);
    case 4: return bwd_rows_dispatch<DT, 4 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, ld, s);
    case 2:
      if constexpr (es == 2)
        return bwd_rows_dispatch<DT, 1>(p, dy, x, g, rstd, dx, part, M, N, offset, ld, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// ---- argument checks --------------------------------------------------------

int check_common(int64_t M, int64_t N, int dtype, uint32_t flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_F16 && dtype != RMSNORM_BF16)
    return RMSNORM_ERR_DTYPE;
  if (flags & ~(RMSNORM_FLAG_OFFSET | RMSNORM_FLAG_DGAMMA_IN_DTYPE)) return RMSNORM_ERR_FLAGS;
  if (N < 1 || N > RMSNORM_MAX_N || M < 0 || M > RMSNORM_MAX_M) return RMSNORM_ERR_SHAPE;
  // Keeps every row-block boundary p*M (p < 2^24 workgroups) inside int64.
  if (M > RMSNORM_MAX_ELEMENTS / N) return RMSNORM_ERR_SHAPE;
  return RMSNORM_OK;
}

// Bytes per dgamma element: float32, or the input dtype with
// RMSNORM_FLAG_DGAMMA_IN_DTYPE.
int dgamma_elem_bytes(int dtype, uint32_t flags) {
  return (flags & RMSNORM_FLAG_DGAMMA_IN_DTYPE) ? elem_bytes(dtype) : 4;
}

bool misaligned(const void* p, int bytes) {
  return p && (reinterpret_cast<uintptr_t>(p) % bytes) != 0;
}

// Largest power of two <= 16 dividing v (v > 0).
int alignment_of(int64_t v) {
  int a = 16;
  while (a > 1 && v % a) a >>= 1;
  return a;
}

// Memory touched by a matrix of `rows` rows of `width` bytes whose starts are
// `pitch` bytes apart (a vector is one row).
struct Region {
  int64_t base, pitch, rows, width;
};

Region matrix(const void* p, int64_t rows, int64_t pitch, int64_t width) {
  return {static_cast<int64_t>(reinterpret_cast<uintptr_t>(p)), pitch, rows, width};
}

Region vec(const void* p, int64_t bytes) { return matrix(p, bytes > 0 ? 1 : 0, bytes, bytes); }

// Spans are measured in 128-bit integers: with up to 2^40 rows of a pitch up
// to 2^40 elements, (rows - 1) * pitch alone can pass 2^63.
using wide_t = __int128;

// One past the last byte of a region (its base when it is empty).
wide_t region_end(const Region& r) {
  if (r.rows == 0 || r.width == 0) return r.base;
  return wide_t(r.base) + wide_t(r.rows - 1) * r.pitch + r.width;
}

// Every address a kernel forms is base + row * pitch + column, in 64-bit
// integers; a region that reaches past 2^57 bytes (beyond any virtual
// address space the GPU or the host maps) would make those sums meaningless.
constexpr int64_t kAddressLimit = int64_t(1) << 57;

bool region_fits(const Region& r) { return region_end(r) <= wide_t(kAddressLimit); }

// Whether two regions share a byte.  Extents are compared first; two matrices
// with one common pitch are then compared row against row, so interleaved
// layouts (say x in the first N columns of a buffer, y in the next N) are
// recognised as disjoint.  Other layouts with overlapping extents count as
// overlapping.  All products are formed in 128 bits.
bool overlaps(const Region& a, const Region& b) {
  if (a.base == 0 || b.base == 0 || a.rows == 0 || b.rows == 0 || a.width == 0 || b.width == 0)
    return false;
  const wide_t a_end = region_end(a), b_end = region_end(b);
  if (a_end <= b.base || b_end <= a.base) return false;
  if (a.pitch != b.pitch || a.rows == 1 || b.rows == 1) return true;
  // Row i of a meets row j of b iff -b.width < d + k*pitch < a.width with
  // d = a.base - b.base and k = i - j in [-(b.rows-1), a.rows-1]; the middle
  // term grows with k, so only the first k past -b.width needs a look.
  const wide_t d = wide_t(a.base) - b.base, p = a.pitch;
  const wide_t k_lo = -wide_t(b.rows - 1), k_hi = a.rows - 1;
  const wide_t num = -wide_t(b.width) - d;  // need k*p > num
  wide_t k = num >= 0 ? num / p + 1 : -((-num) / p);
  if (k * p <= num) ++k;
  if (k < k_lo) k = k_lo;
  if (k > k_hi) return false;
  return d + k * p < a.width;
}

// Status of a call's buffers: a region past the address limit is a stride
// error when its rows are padded (a shape error otherwise); any output that
// shares a byte with an input or with another output is an overlap.
int span_status(std::initializer_list<Region> outs, std::initializer_list<Region> ins) {
  for (std::initializer_list<Region> group : {outs, ins})
    for (const Region& r : group)
      if (!region_fits(r))
        return (r.rows > 1 && r.pitch != r.width) ? RMSNORM_ERR_STRIDE : RMSNORM_ERR_SHAPE;
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Region& i : ins)
      if (overlaps(*o, i)) return RMSNORM_ERR_OVERLAP;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlaps(*o, *o2)) return RMSNORM_ERR_OVERLAP;
  }
  return RMSNORM_OK;
}

bool bad_stride(int64_t ld, int64_t N) { return ld < N || ld > (int64_t(1) << 40); }

int check_fwd_args(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                   int64_t N, int dtype, uint32_t flags, const void* y, int64_t ldy,
                   const float* rstd) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_ERR_EPS;
  if (bad_stride(ldx, N) || bad_stride(ldy, N)) return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !y || !rstd) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(x, es) || misaligned(gamma, es) || misaligned(y, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(y, M, ldy * es, N * es), vec(rstd, M * 4)},
                  {matrix(x, M, ldx * es, N * es), vec(gamma, N * es)}))
    return sp;
  return RMSNORM_OK;
}

int check_bwd_rows_args(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                        const void* gamma, const float* rstd, int64_t M, int64_t N, int dtype,
                        uint32_t flags, const void* dx, int64_t lddx, const void* workspace,
                        size_t workspace_bytes, bool library_scratch = false) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (bad_stride(lddy, N) || bad_stride(ldx, N) || bad_stride(lddx, N)) return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!dy || !x || !gamma || !rstd || !dx) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(dy, es) || misaligned(x, es) || misaligned(gamma, es) ||
      misaligned(dx, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, static_cast<rmsnorm_dtype_t>(dtype), flags);
  // The library's own scratch is a separate device allocation, sized and
  // aligned by the library: only the caller's buffers are checked here.
  if (library_scratch) {
    if (need > RMSNORM_NOALLOC_SCRATCH_BYTES) return RMSNORM_ERR_WORKSPACE;
    workspace = nullptr;
  } else {
    if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
    if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  }
  if (const int sp = span_status({matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(x, M, ldx * es, N * es),
                   vec(gamma, N * es), vec(rstd, M * 4)}))
    return sp;
  return RMSNORM_OK;
}

int check_dgamma_args(const void* dgamma, int64_t N, int dtype, uint32_t flags) {
  if (!dgamma) return RMSNORM_ERR_NULL_POINTER;
  if (misaligned(dgamma, dgamma_elem_bytes(dtype, flags))) return RMSNORM_ERR_ALIGNMENT;
  return RMSNORM_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_LAUNCH; }

// Alignment the plan may assume: every pointer and every row pitch.
int layout_alignment(std::initializer_list<const void*> ptrs,
                     std::initializer_list<int64_t> pitches) {
  int a = pointer_alignment(ptrs);
  for (int64_t p : pitches) a = std::min(a, alignment_of(p));
  return a;
}

int fwd_impl(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M, int64_t N,
             rmsnorm_dtype_t dtype, uint32_t flags, void* y, int64_t ldy, float* rstd,
             hipStream_t stream) {
  int st = check_fwd_args(x, ldx, gamma, eps, M, N, dtype, flags, y, ldy, rstd);
  if (st != RMSNORM_OK || M == 0) return st;
  const int es = elem_bytes(dtype);
  rmsnorm_plan_t p;
  fill_plan(M, N, dtype, RMSNORM_PASS_FWD,
            layout_alignment({x, gamma, y}, {ldx * es, ldy * es}), &p);
  const int off = (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0;
  const int n = static_cast<int>(N);
  const RowStrides ld{ldx, ldy, 0, 0};
  hipError_t e;
  if (p.kernel == RMSNORM_KERNEL_FWD_SPLIT) {
    const FastFwdArgs a{x, gamma, y, rstd, M, n, eps, off, ldx * es, ldy * es};
    const SplitPlan sp{p.vec, p.segments, p.grid / p.segments};
    return status_of(split_fwd_launch(dtype, sp, a, stream));
  }
  switch (dtype) {
    case RMSNORM_F32: e = fwd_by_vec<kF32>(p, x, gamma, y, rstd, M, n, eps, off, ld, stream); break;
    case RMSNORM_F16: e = fwd_by_vec<kF16>(p, x, gamma, y, rstd, M, n, eps, off, ld, stream); break;
    default: e = fwd_by_vec<kBF16>(p, x, gamma, y, rstd, M, n, eps, off, ld, stream); break;
  }
  return status_of(e);
}

// Stage 1 after its arguments were checked.
int bwd_rows_launch(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
                    const float* rstd, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                    uint32_t flags, void* dx, int64_t lddx, void* workspace,
                    hipStream_t stream) {
  if (M == 0) return RMSNORM_OK;
  const int es = elem_bytes(dtype);
  rmsnorm_plan_t p;
  fill_plan(M, N, dtype, RMSNORM_PASS_BWD_ROWS,
            layout_alignment({dy, x, gamma, dx}, {lddy * es, ldx * es, lddx * es}), &p);
  const int off = (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0;
  const int n = static_cast<int>(N);
  float* part = static_cast<float*>(workspace);
  const RowStrides ld{ldx, 0, lddy, lddx};
  hipError_t e;
  if (p.kernel == RMSNORM_KERNEL_BWD_SPLIT) {
    const FastBwdArgs a{dy, x, gamma, rstd, dx, part, M, n, off, p.partials,
                        lddy * es, ldx * es, lddx * es};
    const SplitPlan sp{p.vec, p.segments, p.partials, split_free_partials(M, p.segments)};
    const SplitWorkspace w = split_workspace_for(p.partials, M, N, es);
    return status_of(split_bwd_launch(dtype, sp, a, part + w.dotp_offset, part + w.coef_offset,
                                      stream));
  }
  switch (dtype) {
    case RMSNORM_F32: e = bwd_rows_by_vec<kF32>(p, dy, x, gamma, rstd, dx, part, M, n, off, ld, stream); break;
    case RMSNORM_F16: e = bwd_rows_by_vec<kF16>(p, dy, x, gamma, rstd, dx, part, M, n, off, ld, stream); break;
    default: e = bwd_rows_by_vec<kBF16>(p, dy, x, gamma, rstd, dx, part, M, n, off, ld, stream); break;
  }
  return status_of(e);
}

// Column sums of a [P, N] float32 partial block into dst (float32, or the
// input dtype with RMSNORM_FLAG_DGAMMA_IN_DTYPE), with the stage-2 kernel
// fill_plan picks for (P, N).
int reduce_columns(const float* part, int64_t P, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                   void* dst, hipStream_t stream, const float* part_b = nullptr,
                   void* dst_b = nullptr);

// Stage 2 after its arguments were checked.
int bwd_reduce_launch(const void* workspace, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                      uint32_t flags, void* dgamma, hipStream_t stream) {
  return reduce_columns(static_cast<const float*>(workspace), bwd_partials(M, N, dtype), N, dtype,
                        flags, dgamma, stream);
}

// part_b / dst_b: a second [P, N] block reduced in the same launch (the
// grid doubles; its second half takes the second block).
int reduce_columns(const float* part, int64_t P, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                   void* dgamma, hipStream_t stream, const float* part_b, void* dst_b) {
  rmsnorm_plan_t p;
  fill_reduce_plan(P, N, &p);
  if (part_b) p.grid *= 2;
  const int n = static_cast<int>(N);
  const int out = (flags & RMSNORM_FLAG_DGAMMA_IN_DTYPE) ? static_cast<int>(dtype) : kOutF32;
#define RMSNORM_REDUCE(OUT)                                                                   \
  switch (p.kernel) {                                                                         \
    case RMSNORM_KERNEL_BWD_REDUCE16:                                                         \
      return status_of(launch(bwd_reduce16_kernel<OUT>, p.grid, p.block_threads, 0, stream,   \
                              part, dgamma, p.partials, n, part_b, dst_b));                   \
    case RMSNORM_KERNEL_BWD_REDUCE_WIDE:                                                      \
      return status_of(launch(bwd_reduce_wide_kernel<OUT>, p.grid, p.block_threads, 0, stream, \
                              part, dgamma, p.partials, n, part_b, dst_b));                   \
    default:                                                                                  \
      return status_of(launch(bwd_reduce_kernel<OUT>, p.grid, p.block_threads, 0, stream,     \
                              part, dgamma, p.partials, n, part_b, dst_b));                   \
  }
  switch (out) {
    case kF32: RMSNORM_REDUCE(kF32);
    case kF16: RMSNORM_REDUCE(kF16);
    case kBF16: RMSNORM_REDUCE(kBF16);
    default: RMSNORM_REDUCE(kOutF32);
  }
#undef RMSNORM_REDUCE
}

int bwd_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
             const float* rstd, int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
             void* dx, int64_t lddx, void* dgamma, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
  int st = check_bwd_rows_args(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, flags, dx, lddx,
                               workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  st = check_dgamma_args(dgamma, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  const int es = elem_bytes(dtype);
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, dtype, flags);
  if (const int sp = span_status({vec(dgamma, N * dgamma_elem_bytes(dtype, flags)),
                   matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(x, M, ldx * es, N * es),
                   vec(gamma, N * es), vec(rstd, M * 4)}))
    return sp;
  st = bwd_rows_launch(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, flags, dx, lddx, workspace,
                       stream);
  if (st != RMSNORM_OK) return st;
  return bwd_reduce_launch(workspace, M, N, dtype, flags, dgamma, stream);
}

// ---- LayerNorm (layernorm.hip) ----------------------------------------------
//
// Row-resident plan: the row over `wpr` wavefronts of a 1024-thread
// workgroup with at most 4 vectors (32 elements) per lane in the forward and
// 16 elements (8 vectors) in the backward, whose two float32 column
// accumulators per element are the register cost; rows of 16384 elements
// with 2-byte accesses (odd N or misaligned 16-bit data) need 16 vectors per
// lane over 16 wavefronts.  The backward's P (rows of each partial block) is a
// function of (M, N, dtype): it is computed with the vector width N alone
// allows, so pointer alignment changes only the kernel variant.
// Workgroups of 256 threads (64*wpr for rows over more than four
// wavefronts): several per compute unit, so one waiting at a row barrier
// does not idle the unit.  The forward gives each workgroup one row step
// (G row groups x R rows, R as the kernel takes it for the `matrices` row
// operands it reads): 89.4 against 94.3 us at bf16 32768 x 4096 with 4 steps
// per workgroup, 174.2 against 184.5 us at fp16 262144 x 1024.
constexpr int64_t kLnFwdWorkgroups = 65536;  // of 256 threads; fewer when larger
constexpr int64_t kLnBwdWorkgroups = 512;

LnPlan ln_plan(int64_t M, int64_t N, int es, bool backward, int align, int matrices = 1) {
  LnPlan p{};
  p.vec = pick_vec(N, es, align);
  const int64_t nvec = N / p.vec;
  const int target = backward ? std::max(1, std::min(8, 16 / p.vec))
                              : std::max(1, std::min(4, 32 / p.vec));
  p.wpr = std::min(16, pow2_at_least(ceil_div(nvec, int64_t(kWave) * target)));
  p.chunks = static_cast<int>(ceil_div(nvec, int64_t(kWave) * p.wpr));
  if (backward && p.wpr > 4 && nvec % kWave == 0 && int64_t(kWave) * p.wpr * p.chunks > nvec) {
    // Exact fit for rows over four wavefronts (one row per workgroup either
    // way): the fewest wavefronts, over four, that divide the row's 64-lane
    // sweeps within the chunk budget.  bf16 65536 x 5120 (640 vectors): 5 wavefronts x 2 chunks
    // against 8 x 2 with 384 of 1024 slots idle; stage 1 361.0 against
    // 434.3 us (LayerNorm) and 386.9 against 398.6 us (fused add).  The
    // forward measured slower with such shapes and keeps the plan above.
    const int64_t sweeps = nvec / kWave;
    for (int w = 5; w <= 16; ++w) {
      if (sweeps % w == 0 && sweeps / w <= target) {
        p.wpr = w;
        p.chunks = static_cast<int>(sweeps / w);
        break;
      }
    }
  }
  p.block = std::max(256, kWave * p.wpr);
  const int64_t G = p.block / (kWave * p.wpr);
  if (backward) {
    p.lds = G > 1 ? int64_t(p.block) * p.vec * 4 : 0;
    const LnPlan base = p.vec == pick_vec(N, es, 16) ? p : ln_plan(M, N, es, true, 16);
    const int64_t Gb = base.block / (kWave * base.wpr);
    p.grid = std::min(ceil_div(M, Gb), kLnBwdWorkgroups);
  } else {
    const int R = rowres::row_step_rows(p.vec * es, rowres::pow2_ceil(p.chunks), matrices,
                                        p.block == 256);
    p.grid = std::min(ceil_div(M, G * R), kLnFwdWorkgroups * 256 / p.block);
  }
  return p;
}

// LayerNorm rows longer than the row-resident kernels hold take the
// split-row plan (layernorm_split.hip) on RMSNorm's segments and row blocks:
// split_partials gives P, and the backward's workspace adds the per-(row,
// segment) sums and the per-row coefficients after the two [P, N] blocks.
bool ln_split_rows(int64_t N) { return N > LAYERNORM_RESIDENT_MAX_N; }

int64_t ln_partials(int64_t M, int64_t N, int es) {
  if (M <= 0) return 0;
  if (ln_split_rows(N)) return split_partials(M, N, es, true);
  return ln_plan(M, N, es, true, 16).grid;
}

// LayerNorm backward rows of 4-8 KiB (257 to 512 16-byte vectors) take
// layernorm_rows.hip's kernel, on RMSNorm's bwd_rows geometry: four
// wavefronts x two chunks per row, two rows per 512-thread workgroup, x in
// LDS, rows swept back to front, P = min(ceil(M/2), 512).  bf16 32768 x 4096
// in a forward -> stage 1 loop: stage 1 121 against 127 us for the
// row-resident kernel (the forward loading x cacheably in both).  A layout
// that is not 16-byte aligned runs the row-resident kernel on the same P.
constexpr int kLnRowsWpr = 4, kLnRowsChunks = 2, kLnRowsBlock = 512;
constexpr int64_t kLnRowsWorkgroups = 512;

bool ln_rows_fast(int64_t N, int es, int align) {
  if (ln_split_rows(N)) return false;
  const int vec = pick_vec(N, es, align);
  if (vec * es != 16) return false;
  const int64_t nvec = N / vec;
  return nvec > 256 && nvec <= 512;
}

int64_t ln_rows_lds(int64_t N, int es) {
  const int64_t groups = kLnRowsBlock / (kWave * kLnRowsWpr);
  const int64_t sweep = int64_t(kWave) * kLnRowsWpr * (16 / es);
  return std::max(groups * N * es, groups * sweep * 4);
}

// LayerNorm's P, a function of (M, N, dtype) only.
int64_t layernorm_partials(int64_t M, int64_t N, int es) {
  if (M > 0 && ln_rows_fast(N, es, 16)) {
    const int64_t groups = kLnRowsBlock / (kWave * kLnRowsWpr);
    return std::min(ceil_div(M, groups), kLnRowsWorkgroups);
  }
  return ln_partials(M, N, es);
}

struct LnSplitWorkspace {
  int64_t sums_offset, coef_offset, total_floats;  // in floats
};

// LayerNorm forward rows over 16384 elements that are full-width (16-byte
// vectors) and at most 8 chunks per lane over 16 wavefronts (bf16/fp16
// N <= 65536, fp32 N <= 32768) stay row-resident (ln_fwd_long_launch; the
// weights are read from cache, so the row fits in 128 VGPRs); other rows
// take the split plan.  bf16 2048 x 65536: forward 125.5 us resident
// against 148.8 us split (step 384.8 against 404.3 us).
bool ln_long_fwd(int64_t N, int es, int vec) {
  return ln_split_rows(N) && vec * es == 16 && N / vec <= 8192;
}

LnPlan ln_long_fwd_plan(int64_t M, int64_t N, int vec) {
  LnPlan p{};
  p.vec = vec;
  p.wpr = 16;
  p.chunks = static_cast<int>(ceil_div(N / vec, int64_t(1024)));
  p.block = 1024;
  p.grid = std::min<int64_t>(M, kLnFwdWorkgroups * 256 / 1024);
  return p;
}


LnSplitWorkspace ln_split_workspace(int64_t M, int64_t N, int es) {
  LnSplitWorkspace w;
  w.sums_offset = ceil_div(2 * split_partials(M, N, es, true) * N, 4) * 4;
  w.coef_offset = w.sums_offset + ceil_div(3 * M * split_nseg(N, es), 4) * 4;
  w.total_floats = w.coef_offset + ceil_div(3 * M, 4) * 4;
  return w;
}

int check_ln_common(int64_t M, int64_t N, int dtype, uint32_t flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_F16 && dtype != RMSNORM_BF16)
    return RMSNORM_ERR_DTYPE;
  if (flags & ~RMSNORM_FLAG_DGAMMA_IN_DTYPE) return RMSNORM_ERR_FLAGS;
  if (N < 1 || N > LAYERNORM_MAX_N || M < 0 || M > RMSNORM_MAX_M) return RMSNORM_ERR_SHAPE;
  if (M > RMSNORM_MAX_ELEMENTS / N) return RMSNORM_ERR_SHAPE;
  return RMSNORM_OK;
}

int ln_fwd_impl(const void* x, int64_t ldx, const void* gamma, const void* beta, float eps,
                int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* y, int64_t ldy,
                float* mean, float* rstd, hipStream_t stream) {
  int st = check_ln_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_ERR_EPS;
  if (bad_stride(ldx, N) || bad_stride(ldy, N)) return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !y || !mean || !rstd) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(x, es) || misaligned(gamma, es) || misaligned(beta, es) ||
      misaligned(y, es) || misaligned(mean, 4) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(y, M, ldy * es, N * es), vec(mean, M * 4), vec(rstd, M * 4)},
                  {matrix(x, M, ldx * es, N * es), vec(gamma, N * es),
                   vec(beta, beta ? N * es : 0)}))
    return sp;
  const int align = layout_alignment({x, gamma, beta, y}, {ldx * es, ldy * es});
  const LnFwdArgs a{x, gamma, beta, y, mean, rstd, M, static_cast<int>(N), eps, ldx * es,
                    ldy * es};
  const int vec = pick_vec(N, es, align);
  if (ln_long_fwd(N, es, vec)) {
    const LnPlan p = ln_long_fwd_plan(M, N, vec);
    if (p.chunks <= 4) return status_of(ln_fwd_launch(dtype, p, a, stream));
    return status_of(ln_fwd_long_launch(dtype, p, a, stream));
  }
  if (ln_split_rows(N)) {
    const SplitPlan sp{vec, static_cast<int>(split_nseg(N, es)), split_partials(M, N, es, false)};
    return status_of(ln_split_fwd_launch(dtype, sp, a, stream));
  }
  const LnPlan p = ln_plan(M, N, es, false, align);
  return status_of(ln_fwd_launch(dtype, p, a, stream));
}

size_t ln_workspace_bytes(int64_t M, int64_t N, int dtype) {
  if (M <= 0) return 0;
  const int es = elem_bytes(dtype);
  if (ln_split_rows(N)) return static_cast<size_t>(ln_split_workspace(M, N, es).total_floats * 4);
  return static_cast<size_t>(2 * layernorm_partials(M, N, es) * N * 4);
}

// Stage-1 argument checks (dy, x, gamma, mean, rstd, dx, workspace).
int check_ln_rows_args(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                       const void* gamma, const float* mean, const float* rstd, int64_t M,
                       int64_t N, int dtype, uint32_t flags, const void* dx, int64_t lddx,
                       const void* workspace, size_t workspace_bytes) {
  int st = check_ln_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (bad_stride(lddy, N) || bad_stride(ldx, N) || bad_stride(lddx, N)) return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!dy || !x || !gamma || !mean || !rstd || !dx) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(dy, es) || misaligned(x, es) || misaligned(gamma, es) || misaligned(dx, es) ||
      misaligned(mean, 4) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const size_t need = ln_workspace_bytes(M, N, dtype);
  if (workspace_bytes < need || !workspace) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(x, M, ldx * es, N * es),
                   vec(gamma, N * es), vec(mean, M * 4), vec(rstd, M * 4)}))
    return sp;
  return RMSNORM_OK;
}

int ln_rows_launch(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
                   const float* mean, const float* rstd, int64_t M, int64_t N,
                   rmsnorm_dtype_t dtype, void* dx, int64_t lddx, void* workspace,
                   hipStream_t stream) {
  if (M == 0) return RMSNORM_OK;
  const int es = elem_bytes(dtype);
  const int align = layout_alignment({dy, x, gamma, dx}, {lddy * es, ldx * es, lddx * es});
  float* part = static_cast<float*>(workspace);
  const LnBwdArgs a{dy, x, gamma, mean, rstd, dx, part, M, static_cast<int>(N), lddy * es,
                    ldx * es, lddx * es};
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, es);
    const SplitPlan sp{pick_vec(N, es, align), static_cast<int>(nseg),
                       split_partials(M, N, es, true), split_free_partials(M, nseg)};
    const LnSplitWorkspace w = ln_split_workspace(M, N, es);
    return status_of(ln_split_bwd_launch(dtype, sp, a, part + w.sums_offset,
                                         part + w.coef_offset, stream));
  }
  const int64_t P = layernorm_partials(M, N, es);
  if (ln_rows_fast(N, es, align))
    return status_of(ln_bwd_rows_launch(dtype, P, ln_rows_lds(N, es), a, stream));
  LnPlan p = ln_plan(M, N, es, true, align);
  p.grid = P;
  return status_of(ln_bwd_launch(dtype, p, a, stream));
}

int ln_reduce_launch(const void* workspace, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                     uint32_t flags, void* dgamma, void* dbeta, hipStream_t stream) {
  const int64_t P = layernorm_partials(M, N, elem_bytes(dtype));
  const float* part = static_cast<const float*>(workspace);
  // dgamma and dbeta in one launch
  if (dbeta && M > 0)
    return reduce_columns(part, P, N, dtype, flags, dgamma, stream, part + P * N, dbeta);
  int st = reduce_columns(part, P, N, dtype, flags, dgamma, stream);
  if (st != RMSNORM_OK || !dbeta) return st;
  return reduce_columns(part, P, N, dtype, flags, dbeta, stream);
}

int check_ln_reduce_args(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                         int dtype, uint32_t flags, const void* dgamma, const void* dbeta) {
  int st = check_ln_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!dgamma) return RMSNORM_ERR_NULL_POINTER;
  const int gb = dgamma_elem_bytes(dtype, flags);
  if (misaligned(dgamma, gb) || misaligned(dbeta, gb)) return RMSNORM_ERR_ALIGNMENT;
  const size_t need = ln_workspace_bytes(M, N, dtype);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({vec(dgamma, N * gb), vec(dbeta, dbeta ? N * gb : 0)},
                  {vec(workspace, static_cast<int64_t>(need))}))
    return sp;
  return RMSNORM_OK;
}

int ln_bwd_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
                const float* mean, const float* rstd, int64_t M, int64_t N,
                rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx, void* dgamma,
                void* dbeta, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_ln_rows_args(dy, lddy, x, ldx, gamma, mean, rstd, M, N, dtype, flags, dx, lddx,
                              workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  st = check_ln_reduce_args(workspace, workspace_bytes, M, N, dtype, flags, dgamma, dbeta);
  if (st != RMSNORM_OK) return st;
  const int es = elem_bytes(dtype);
  const int gb = dgamma_elem_bytes(dtype, flags);
  const size_t need = ln_workspace_bytes(M, N, dtype);
  if (const int sp = span_status({vec(dgamma, N * gb), vec(dbeta, dbeta ? N * gb : 0),
                   matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(x, M, ldx * es, N * es),
                   vec(gamma, N * es), vec(mean, M * 4), vec(rstd, M * 4)}))
    return sp;
  st = ln_rows_launch(dy, lddy, x, ldx, gamma, mean, rstd, M, N, dtype, dx, lddx, workspace,
                      stream);
  if (st != RMSNORM_OK) return st;
  return ln_reduce_launch(workspace, M, N, dtype, flags, dgamma, dbeta, stream);
}

void fill_ln_plan(int64_t M, int64_t N, int dtype, int pass, int align, rmsnorm_plan_t* out,
                  int matrices = 1, bool layernorm = false) {
  std::memset(out, 0, sizeof(*out));
  const int es = elem_bytes(dtype);
  if (pass == RMSNORM_PASS_BWD_REDUCE) {
    fill_reduce_plan(layernorm ? layernorm_partials(M, N, es) : ln_partials(M, N, es), N, out);
    return;
  }
  const bool bwd = pass == RMSNORM_PASS_BWD_ROWS;
  if (layernorm && bwd && ln_rows_fast(N, es, align)) {
    out->kernel = LAYERNORM_KERNEL_BWD_ROWS;
    out->vec = 16 / es;
    out->threads_per_row = kWave * kLnRowsWpr;
    out->block_threads = kLnRowsBlock;
    out->chunks = kLnRowsChunks;
    out->x_in_lds = 1;
    out->weight_in_regs = 1;
    out->partials = layernorm_partials(M, N, es);
    out->grid = out->partials;
    out->lds_bytes = ln_rows_lds(N, es);
    return;
  }
  if (layernorm && !bwd && ln_long_fwd(N, es, pick_vec(N, es, align))) {
    const LnPlan p = ln_long_fwd_plan(M, N, pick_vec(N, es, align));
    out->kernel = LAYERNORM_KERNEL_FWD;
    out->vec = p.vec;
    out->threads_per_row = kWave * p.wpr;
    out->block_threads = p.block;
    out->chunks = p.chunks;
    out->weight_in_regs = p.chunks <= 4 ? 1 : 0;
    out->grid = p.grid;
    return;
  }
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, es);
    const int vec = pick_vec(N, es, align);
    // LayerNorm's forward passes keep their row blocks (its float64 stats
    // pass measured slower one row per block); the RMSNorm kernels' forward
    // takes one row per block.
    const int64_t P = bwd ? split_partials(M, N, es, true)
                          : (layernorm ? split_partials(M, N, es, false)
                                       : split_free_partials(M, nseg));
    out->kernel = bwd ? LAYERNORM_KERNEL_BWD_SPLIT : LAYERNORM_KERNEL_FWD_SPLIT;
    out->vec = vec;
    out->segments = static_cast<int32_t>(nseg);
    out->threads_per_row = static_cast<int32_t>(256 * nseg);
    out->chunks = split_chunks(vec, es);
    out->block_threads = 256;
    out->weight_in_regs = 1;
    out->partials = bwd ? P : 0;
    out->grid = P * nseg;
    return;
  }
  const LnPlan p = ln_plan(M, N, es, bwd, align, matrices);
  out->kernel = bwd ? LAYERNORM_KERNEL_BWD : LAYERNORM_KERNEL_FWD;
  out->vec = p.vec;
  out->threads_per_row = kWave * p.wpr;
  out->block_threads = p.block;
  out->chunks = p.chunks;
  out->weight_in_regs = 1;
  out->grid = bwd && layernorm ? layernorm_partials(M, N, es) : p.grid;
  out->partials = bwd ? out->grid : 0;
  out->lds_bytes = bwd ? p.lds : 0;
}

// ---- RMSNorm with the residual add fused before it (fused_add.hip) ----------
//
// The row-resident plan of LayerNorm (same targets, workgroups and P); the
// backward's workspace is one [P, N] block.  The forward reads two row
// operands (x and res), which sets its rows per step.
constexpr int kAddFwdMatrices = 2;

int check_add_common(int64_t M, int64_t N, int dtype, uint32_t flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_F16 && dtype != RMSNORM_BF16)
    return RMSNORM_ERR_DTYPE;
  if (flags & ~(RMSNORM_FLAG_OFFSET | RMSNORM_FLAG_DGAMMA_IN_DTYPE)) return RMSNORM_ERR_FLAGS;
  if (N < 1 || N > RMSNORM_ADD_MAX_N || M < 0 || M > RMSNORM_MAX_M) return RMSNORM_ERR_SHAPE;
  if (M > RMSNORM_MAX_ELEMENTS / N) return RMSNORM_ERR_SHAPE;
  return RMSNORM_OK;
}

// Rows over 16384 elements: full-width rows of up to 128 KiB run on
// RMSNorm's long-row kernels (the forward's fwd_fast_kernel with the add,
// bwd_longrow_kernel on h with dh), one row per 512-thread workgroup at a
// time; other layouts take RMSNorm's split plan.  The split
// fused step at bf16 2048 x 65536 measured 568.8 us, slower than the
// unfused pair (torch's add around the long-row RMSNorm, 541.0 us).
// P is a function of (M, N, dtype): the long-row count wherever the
// full-width layout can take the long-row backward, so a misaligned call
// runs the split kernels on the same P, and the workspace always has the
// split layout ([P, N] partials, per-(row, segment) sums, per-row
// coefficients).
int add_long_fwd_ch(int64_t N, int es, int align) {
  if (!ln_split_rows(N)) return 0;
  const int vec = pick_vec(N, es, align);
  if (vec * es != 16) return 0;
  const Cfg c = plan_fast_fwd(N / vec);
  if (!c.ok || c.wpr != 8 || c.block != 512 || !c.greg || c.ch < 5 || c.ch > 16) return 0;
  return c.ch;
}

int add_long_bwd_ch(int64_t N, int es, int align) {
  if (!ln_split_rows(N)) return 0;
  const int vec = pick_vec(N, es, align);
  if (vec * es != 16) return 0;
  const int ch = plan_long_bwd(N / vec);
  return ch >= 5 ? ch : 0;
}

int64_t add_bwd_partials(int64_t M, int64_t N, int es) {
  if (M <= 0) return 0;
  if (!ln_split_rows(N)) return ln_partials(M, N, es);
  if (add_long_bwd_ch(N, es, 16)) return std::min<int64_t>(M, kLongBwdWorkgroups);
  return split_partials(M, N, es, true);
}

size_t add_workspace_bytes(int64_t M, int64_t N, int dtype) {
  if (M <= 0) return 0;
  const int es = elem_bytes(dtype);
  const int64_t P = add_bwd_partials(M, N, es);
  if (ln_split_rows(N)) return static_cast<size_t>(split_workspace_for(P, M, N, es).total_floats * 4);
  return static_cast<size_t>(P * N * 4);
}

hipError_t add_long_fwd(int dtype, int ch, int64_t grid, const AddFwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case RMSNORM_F32: return add_long_fwd_launch<kF32>(ch, grid, a, s);
    case RMSNORM_F16: return add_long_fwd_launch<kF16>(ch, grid, a, s);
    default: return add_long_fwd_launch<kBF16>(ch, grid, a, s);
  }
}

hipError_t add_long_bwd(int dtype, int ch, int64_t P, int64_t lds, const AddBwdArgs& a,
                        hipStream_t s) {
  switch (dtype) {
    case RMSNORM_F32: return add_long_bwd_launch<kF32>(ch, P, lds, a, s);
    case RMSNORM_F16: return add_long_bwd_launch<kF16>(ch, P, lds, a, s);
    default: return add_long_bwd_launch<kBF16>(ch, P, lds, a, s);
  }
}

// Forward grid of the long-row add: one row per workgroup at a time.
int64_t add_long_fwd_grid(int64_t M) { return std::min<int64_t>(M, int64_t(1) << 20); }

int add_fwd_impl(const void* x, int64_t ldx, const void* res, int64_t ldr, const void* gamma,
                 float eps, int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* y,
                 int64_t ldy, void* h, int64_t ldh, float* rstd, hipStream_t stream) {
  int st = check_add_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_ERR_EPS;
  if (bad_stride(ldx, N) || bad_stride(ldr, N) || bad_stride(ldy, N) || bad_stride(ldh, N))
    return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!x || !res || !gamma || !y || !h || !rstd) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(x, es) || misaligned(res, es) || misaligned(gamma, es) || misaligned(y, es) ||
      misaligned(h, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(y, M, ldy * es, N * es), matrix(h, M, ldh * es, N * es),
                   vec(rstd, M * 4)},
                  {matrix(x, M, ldx * es, N * es), matrix(res, M, ldr * es, N * es),
                   vec(gamma, N * es)}))
    return sp;
  const int align = layout_alignment({x, res, gamma, y, h},
                                     {ldx * es, ldr * es, ldy * es, ldh * es});
  const AddFwdArgs a{x, res, gamma, y, h, rstd, M, static_cast<int>(N), eps,
                     (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0, ldx * es, ldr * es, ldy * es,
                     ldh * es};
  if (const int ch = add_long_fwd_ch(N, es, align))
    return status_of(add_long_fwd(dtype, ch, add_long_fwd_grid(M), a, stream));
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, es);
    const SplitPlan sp{pick_vec(N, es, align), static_cast<int>(nseg), split_free_partials(M, nseg)};
    return status_of(add_split_fwd_launch(dtype, sp, a, stream));
  }
  const LnPlan p = ln_plan(M, N, es, false, align, kAddFwdMatrices);
  return status_of(add_fwd_launch(dtype, p, a, stream));
}

int check_add_rows_args(const void* dy, int64_t lddy, const void* dh, int64_t lddh,
                        const void* h, int64_t ldh, const void* gamma, const float* rstd,
                        int64_t M, int64_t N, int dtype, uint32_t flags, const void* dx,
                        int64_t lddx, const void* workspace, size_t workspace_bytes) {
  int st = check_add_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (bad_stride(lddy, N) || bad_stride(ldh, N) || bad_stride(lddx, N) ||
      (dh && bad_stride(lddh, N)))
    return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!dy || !h || !gamma || !rstd || !dx) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(dy, es) || misaligned(dh, es) || misaligned(h, es) || misaligned(gamma, es) ||
      misaligned(dx, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const size_t need = add_workspace_bytes(M, N, dtype);
  if (workspace_bytes < need || !workspace) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(dh, dh ? M : 0, lddh * es, N * es),
                   matrix(h, M, ldh * es, N * es), vec(gamma, N * es), vec(rstd, M * 4)}))
    return sp;
  return RMSNORM_OK;
}

int add_rows_launch(const void* dy, int64_t lddy, const void* dh, int64_t lddh, const void* h,
                    int64_t ldh, const void* gamma, const float* rstd, int64_t M, int64_t N,
                    rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx,
                    void* workspace, hipStream_t stream) {
  if (M == 0) return RMSNORM_OK;
  const int es = elem_bytes(dtype);
  const int align = layout_alignment({dy, dh, h, gamma, dx},
                                     {lddy * es, dh ? lddh * es : 16, ldh * es, lddx * es});
  float* part = static_cast<float*>(workspace);
  const AddBwdArgs a{dy, dh, h, gamma, rstd, dx, part, M, static_cast<int>(N),
                     (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0, lddy * es, lddh * es, ldh * es,
                     lddx * es};
  const int64_t P = add_bwd_partials(M, N, es);
  if (const int ch = add_long_bwd_ch(N, es, align))
    return status_of(add_long_bwd(dtype, ch, P, N * es, a, stream));
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, es);
    const SplitPlan sp{pick_vec(N, es, align), static_cast<int>(nseg), P,
                       split_free_partials(M, nseg)};
    const SplitWorkspace w = split_workspace_for(P, M, N, es);
    return status_of(add_split_bwd_launch(dtype, sp, a, part + w.dotp_offset,
                                          part + w.coef_offset, stream));
  }
  const LnPlan p = ln_plan(M, N, es, true, align);
  return status_of(add_bwd_launch(dtype, p, a, stream));
}

int check_add_reduce_args(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                          int dtype, uint32_t flags, const void* dgamma) {
  int st = check_add_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  st = check_dgamma_args(dgamma, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  const size_t need = add_workspace_bytes(M, N, dtype);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({vec(dgamma, N * dgamma_elem_bytes(dtype, flags))},
                  {vec(workspace, static_cast<int64_t>(need))}))
    return sp;
  return RMSNORM_OK;
}

int add_bwd_impl(const void* dy, int64_t lddy, const void* dh, int64_t lddh, const void* h,
                 int64_t ldh, const void* gamma, const float* rstd, int64_t M, int64_t N,
                 rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx, void* dgamma,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_add_rows_args(dy, lddy, dh, lddh, h, ldh, gamma, rstd, M, N, dtype, flags, dx,
                               lddx, workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  st = check_add_reduce_args(workspace, workspace_bytes, M, N, dtype, flags, dgamma);
  if (st != RMSNORM_OK) return st;
  const int es = elem_bytes(dtype);
  const size_t need = add_workspace_bytes(M, N, dtype);
  if (const int sp = span_status({vec(dgamma, N * dgamma_elem_bytes(dtype, flags)),
                   matrix(dx, M, lddx * es, N * es), vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * es, N * es), matrix(dh, dh ? M : 0, lddh * es, N * es),
                   matrix(h, M, ldh * es, N * es), vec(gamma, N * es), vec(rstd, M * 4)}))
    return sp;
  st = add_rows_launch(dy, lddy, dh, lddh, h, ldh, gamma, rstd, M, N, dtype, flags, dx, lddx,
                       workspace, stream);
  if (st != RMSNORM_OK) return st;
  return reduce_columns(static_cast<const float*>(workspace), add_bwd_partials(M, N, es), N, dtype,
                        flags, dgamma, stream);
}

void fill_add_plan(int64_t M, int64_t N, int dtype, int pass, int align, rmsnorm_plan_t* out) {
  const int es = elem_bytes(dtype);
  if (pass == RMSNORM_PASS_BWD_REDUCE) {
    std::memset(out, 0, sizeof(*out));
    fill_reduce_plan(add_bwd_partials(M, N, es), N, out);
    return;
  }
  fill_ln_plan(M, N, dtype, pass, align, out, kAddFwdMatrices);
  const bool bwd = pass == RMSNORM_PASS_BWD_ROWS;
  const int ch = bwd ? add_long_bwd_ch(N, es, align) : add_long_fwd_ch(N, es, align);
  if (ch) {
    std::memset(out, 0, sizeof(*out));
    out->kernel = bwd ? RMSNORM_KERNEL_ADD_BWD_LONG : RMSNORM_KERNEL_ADD_FWD_LONG;
    out->vec = 16 / es;
    out->threads_per_row = 512;
    out->chunks = ch;
    out->block_threads = 512;
    out->weight_in_regs = bwd ? 0 : 1;
    out->x_in_lds = bwd ? 1 : 0;
    out->partials = bwd ? add_bwd_partials(M, N, es) : 0;
    out->grid = bwd ? out->partials : add_long_fwd_grid(M);
    out->lds_bytes = bwd ? N * es : 0;
  } else if (ln_split_rows(N)) {
    out->kernel = bwd ? RMSNORM_KERNEL_ADD_BWD_SPLIT : RMSNORM_KERNEL_ADD_FWD_SPLIT;
    if (bwd) {
      out->partials = add_bwd_partials(M, N, es);
      out->grid = out->partials * out->segments;
    }
  } else {
    out->kernel = bwd ? RMSNORM_KERNEL_ADD_BWD : RMSNORM_KERNEL_ADD_FWD;
  }
}

// ---- RMSNorm with its output cast to a narrower dtype (fused_cast.hip) ------
//
// float32 x, gamma and dx; y and dy in the output dtype.  The row-resident
// plan of LayerNorm at float32 (same targets, workgroups and P); the
// backward's workspace is one [P, N] block.  Vector widths follow the common
// alignment of all operands, so the narrow operands are aligned for their
// half-width accesses too.
constexpr int kCastIn = 4;  // bytes per input element

int check_cast_common(int64_t M, int64_t N, int dtype, int out_dtype, uint32_t flags) {
  if (dtype != RMSNORM_F32 || (out_dtype != RMSNORM_BF16 && out_dtype != RMSNORM_F16))
    return RMSNORM_ERR_DTYPE;
  if (flags & ~(RMSNORM_FLAG_OFFSET | RMSNORM_FLAG_DGAMMA_IN_DTYPE)) return RMSNORM_ERR_FLAGS;
  if (N < 1 || N > RMSNORM_CAST_MAX_N || M < 0 || M > RMSNORM_MAX_M) return RMSNORM_ERR_SHAPE;
  if (M > RMSNORM_MAX_ELEMENTS / N) return RMSNORM_ERR_SHAPE;
  return RMSNORM_OK;
}

size_t cast_workspace_bytes(int64_t M, int64_t N) {
  if (M <= 0) return 0;
  if (ln_split_rows(N)) return static_cast<size_t>(split_workspace(M, N, kCastIn).total_floats * 4);
  return static_cast<size_t>(ln_partials(M, N, kCastIn) * N * 4);
}

int cast_fwd_impl(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                  int64_t N, rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype, uint32_t flags,
                  void* y, int64_t ldy, float* rstd, hipStream_t stream) {
  int st = check_cast_common(M, N, dtype, out_dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_ERR_EPS;
  if (bad_stride(ldx, N) || bad_stride(ldy, N)) return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !y || !rstd) return RMSNORM_ERR_NULL_POINTER;
  const int eo = elem_bytes(out_dtype);
  if (misaligned(x, kCastIn) || misaligned(gamma, kCastIn) || misaligned(y, eo) ||
      misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(y, M, ldy * eo, N * eo), vec(rstd, M * 4)},
                  {matrix(x, M, ldx * kCastIn, N * kCastIn), vec(gamma, N * kCastIn)}))
    return sp;
  const int align = layout_alignment({x, gamma, y}, {ldx * kCastIn, ldy * eo});
  const CastFwdArgs a{x, gamma, y, rstd, M, static_cast<int>(N), eps,
                      (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0, ldx * kCastIn, ldy * eo};
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, kCastIn);
    const SplitPlan sp{pick_vec(N, kCastIn, align), static_cast<int>(nseg),
                       split_free_partials(M, nseg)};
    return status_of(cast_split_fwd_launch(out_dtype, sp, a, stream));
  }
  const LnPlan p = ln_plan(M, N, kCastIn, false, align);
  return status_of(cast_fwd_launch(out_dtype, p, a, stream));
}

int check_cast_rows_args(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                         const void* gamma, const float* rstd, int64_t M, int64_t N, int dtype,
                         int out_dtype, uint32_t flags, const void* dx, int64_t lddx,
                         const void* workspace, size_t workspace_bytes) {
  int st = check_cast_common(M, N, dtype, out_dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (bad_stride(lddy, N) || bad_stride(ldx, N) || bad_stride(lddx, N))
    return RMSNORM_ERR_STRIDE;
  if (M == 0) return RMSNORM_OK;
  if (!dy || !x || !gamma || !rstd || !dx) return RMSNORM_ERR_NULL_POINTER;
  const int eo = elem_bytes(out_dtype);
  if (misaligned(dy, eo) || misaligned(x, kCastIn) || misaligned(gamma, kCastIn) ||
      misaligned(dx, kCastIn) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const size_t need = cast_workspace_bytes(M, N);
  if (workspace_bytes < need || !workspace) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({matrix(dx, M, lddx * kCastIn, N * kCastIn),
                   vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * eo, N * eo), matrix(x, M, ldx * kCastIn, N * kCastIn),
                   vec(gamma, N * kCastIn), vec(rstd, M * 4)}))
    return sp;
  return RMSNORM_OK;
}

int cast_rows_launch(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                     const void* gamma, const float* rstd, int64_t M, int64_t N,
                     rmsnorm_dtype_t out_dtype, uint32_t flags, void* dx, int64_t lddx,
                     void* workspace, hipStream_t stream) {
  if (M == 0) return RMSNORM_OK;
  const int eo = elem_bytes(out_dtype);
  const int align = layout_alignment({dy, x, gamma, dx},
                                     {lddy * eo, ldx * kCastIn, lddx * kCastIn});
  float* part = static_cast<float*>(workspace);
  const CastBwdArgs a{dy, x, gamma, rstd, dx, part, M, static_cast<int>(N),
                      (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0, lddy * eo, ldx * kCastIn,
                      lddx * kCastIn};
  if (ln_split_rows(N)) {
    const int64_t nseg = split_nseg(N, kCastIn);
    const SplitPlan sp{pick_vec(N, kCastIn, align), static_cast<int>(nseg),
                       split_partials(M, N, kCastIn, true), split_free_partials(M, nseg)};
    const SplitWorkspace w = split_workspace(M, N, kCastIn);
    return status_of(cast_split_bwd_launch(out_dtype, sp, a, part + w.dotp_offset,
                                           part + w.coef_offset, stream));
  }
  const LnPlan p = ln_plan(M, N, kCastIn, true, align);
  return status_of(cast_bwd_launch(out_dtype, p, a, stream));
}

int check_cast_reduce_args(const void* workspace, size_t workspace_bytes, int64_t M,
                           int64_t N, int dtype, int out_dtype, uint32_t flags,
                           const void* dgamma) {
  int st = check_cast_common(M, N, dtype, out_dtype, flags);
  if (st != RMSNORM_OK) return st;
  st = check_dgamma_args(dgamma, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  const size_t need = cast_workspace_bytes(M, N);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({vec(dgamma, N * 4)}, {vec(workspace, static_cast<int64_t>(need))}))
    return sp;
  return RMSNORM_OK;
}

int cast_bwd_impl(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
                  const float* rstd, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                  rmsnorm_dtype_t out_dtype, uint32_t flags, void* dx, int64_t lddx,
                  void* dgamma, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_cast_rows_args(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, out_dtype, flags, dx,
                                lddx, workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  st = check_cast_reduce_args(workspace, workspace_bytes, M, N, dtype, out_dtype, flags, dgamma);
  if (st != RMSNORM_OK) return st;
  const int eo = elem_bytes(out_dtype);
  const size_t need = cast_workspace_bytes(M, N);
  if (const int sp = span_status({vec(dgamma, N * 4), matrix(dx, M, lddx * kCastIn, N * kCastIn),
                   vec(workspace, static_cast<int64_t>(need))},
                  {matrix(dy, M, lddy * eo, N * eo), matrix(x, M, ldx * kCastIn, N * kCastIn),
                   vec(gamma, N * kCastIn), vec(rstd, M * 4)}))
    return sp;
  st = cast_rows_launch(dy, lddy, x, ldx, gamma, rstd, M, N, out_dtype, flags, dx, lddx,
                        workspace, stream);
  if (st != RMSNORM_OK) return st;
  return reduce_columns(static_cast<const float*>(workspace), ln_partials(M, N, kCastIn), N,
                        dtype, flags, dgamma, stream);
}

void fill_cast_plan(int64_t M, int64_t N, int pass, int align, rmsnorm_plan_t* out) {
  fill_ln_plan(M, N, RMSNORM_F32, pass, align, out);
  if (pass == RMSNORM_PASS_BWD_REDUCE) return;
  const bool bwd = pass == RMSNORM_PASS_BWD_ROWS;
  if (ln_split_rows(N))
    out->kernel = bwd ? RMSNORM_KERNEL_CAST_BWD_SPLIT : RMSNORM_KERNEL_CAST_FWD_SPLIT;
  else
    out->kernel = bwd ? RMSNORM_KERNEL_CAST_BWD : RMSNORM_KERNEL_CAST_FWD;
}

}  // namespace

// ---- the allocation-free backward's scratch --------------------------------
//
// rmsnorm_bwd_noalloc keeps its dgamma partial sums in this file-scope device
// array instead of a caller workspace.  Every device the library runs on
// holds its own copy, reserved when this file's code object is loaded there
// and held until the process ends.  Stage 1 writes every partial that stage 2
// reads, so nothing in it has to start at zero.
static __device__ __align__(256) float scratch[RMSNORM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each device's copy is looked up once, with that device
// current, and only that address is passed to kernels.
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RMSNORM_ERR_LAUNCH;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
        return RMSNORM_ERR_LAUNCH;
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RMSNORM_OK;
}

}  // namespace

extern "C" {

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RMSNORM_ERR_DTYPE: return "unsupported dtype (fp32, fp16 and bf16 are supported)";
    case RMSNORM_ERR_SHAPE:
      return "unsupported shape (need 0 <= M <= 2^40, 1 <= N <= 2^24 and M*N <= 2^46, for "
             "rmsnorm_*, layernorm_*, rmsnorm_add_* and rmsnorm_cast_* alike), or a buffer "
             "ending past byte address 2^57";
    case RMSNORM_ERR_EPS: return "eps must be finite and positive";
    case RMSNORM_ERR_FLAGS: return "unknown flag bits";
    case RMSNORM_ERR_WORKSPACE:
      return "workspace missing or smaller than the matching *_bwd_workspace_bytes(), or (for "
             "rmsnorm_bwd_noalloc) a need above RMSNORM_NOALLOC_SCRATCH_BYTES";
    case RMSNORM_ERR_ALIGNMENT: return "pointer not aligned to its element size (workspace: 16 bytes)";
    case RMSNORM_ERR_OVERLAP: return "an output buffer overlaps an input or another output";
    case RMSNORM_ERR_LAUNCH: return "kernel launch failed";
    case RMSNORM_ERR_ARGUMENT: return "invalid argument";
    case RMSNORM_ERR_STRIDE:
      return "a row stride is smaller than N or above 2^40, or a padded matrix ends past byte "
             "address 2^57";
    default: return "unknown status";
  }
}

int rmsnorm_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                       int pass, int align_bytes, rmsnorm_plan_t* plan) {
  const int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!plan) return RMSNORM_ERR_NULL_POINTER;
  if (pass < RMSNORM_PASS_FWD || pass > RMSNORM_PASS_BWD_REDUCE) return RMSNORM_ERR_ARGUMENT;
  if (align_bytes < 1 || align_bytes > 4096 || (align_bytes & (align_bytes - 1)))
    return RMSNORM_ERR_ARGUMENT;
  fill_plan(M, N, dtype, pass, std::min(align_bytes, 16), plan);
  return RMSNORM_OK;
}

size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                   uint32_t flags) {
  if (check_common(M, N, dtype, flags) != RMSNORM_OK || M == 0) return 0;
  return static_cast<size_t>(bwd_workspace_floats(M, N, dtype) * 4);
}

int rmsnorm_fwd(const void* x, const void* gamma, float eps, int64_t M, int64_t N,
                rmsnorm_dtype_t dtype, uint32_t flags, void* y, float* rstd,
                hipStream_t stream) {
  return fwd_impl(x, N, gamma, eps, M, N, dtype, flags, y, N, rstd, stream);
}

int rmsnorm_fwd_strided(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                        int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* y, int64_t ldy,
                        float* rstd, hipStream_t stream) {
  return fwd_impl(x, ldx, gamma, eps, M, N, dtype, flags, y, ldy, rstd, stream);
}

int rmsnorm_bwd_rows(const void* dy, const void* x, const void* gamma, const float* rstd,
                     int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bwd_rows_args(dy, N, x, N, gamma, rstd, M, N, dtype, flags, dx, N, workspace,
                               workspace_bytes);
  if (st != RMSNORM_OK) return st;
  return bwd_rows_launch(dy, N, x, N, gamma, rstd, M, N, dtype, flags, dx, N, workspace, stream);
}

int rmsnorm_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                       rmsnorm_dtype_t dtype, uint32_t flags, void* dgamma,
                       hipStream_t stream) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  st = check_dgamma_args(dgamma, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, dtype, flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (const int sp = span_status({vec(dgamma, N * dgamma_elem_bytes(dtype, flags))},
                  {vec(workspace, static_cast<int64_t>(need))}))
    return sp;
  return bwd_reduce_launch(workspace, M, N, dtype, flags, dgamma, stream);
}

int rmsnorm_bwd(const void* dy, const void* x, const void* gamma, const float* rstd,
                int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                void* dgamma, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(dy, N, x, N, gamma, rstd, M, N, dtype, flags, dx, N, dgamma, workspace,
                  workspace_bytes, stream);
}

int rmsnorm_bwd_noalloc(const void* dy, const void* x, const void* gamma, const float* rstd,
                        int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                        void* dgamma, hipStream_t stream) {
  // Every caller argument is checked before the scratch is looked up.
  int st = check_bwd_rows_args(dy, N, x, N, gamma, rstd, M, N, dtype, flags, dx, N, nullptr, 0,
                               /*library_scratch=*/true);
  if (st != RMSNORM_OK) return st;
  st = check_dgamma_args(dgamma, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  const int es = elem_bytes(dtype);
  if (const int sp = span_status({vec(dgamma, N * dgamma_elem_bytes(dtype, flags)),
                                  matrix(dx, M, N * es, N * es)},
                                 {matrix(dy, M, N * es, N * es), matrix(x, M, N * es, N * es),
                                  vec(gamma, N * es), vec(rstd, M * 4)}))
    return sp;
  float* part = nullptr;
  if (rmsnorm_bwd_workspace_bytes(M, N, dtype, flags) > 0) {
    st = scratch_on_current_device(&part);
    if (st != RMSNORM_OK) return st;
  }
  st = bwd_rows_launch(dy, N, x, N, gamma, rstd, M, N, dtype, flags, dx, N, part, stream);
  if (st != RMSNORM_OK) return st;
  return bwd_reduce_launch(part, M, N, dtype, flags, dgamma, stream);
}

int rmsnorm_bwd_strided(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                        const void* gamma, const float* rstd, int64_t M, int64_t N,
                        rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx,
                        void* dgamma, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return bwd_impl(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, flags, dx, lddx, dgamma,
                  workspace, workspace_bytes, stream);
}

int layernorm_fwd(const void* x, int64_t ldx, const void* gamma, const void* beta, float eps,
                  int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* y,
                  int64_t ldy, float* mean, float* rstd, hipStream_t stream) {
  return ln_fwd_impl(x, ldx, gamma, beta, eps, M, N, dtype, flags, y, ldy, mean, rstd, stream);
}

size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                     uint32_t flags) {
  if (check_ln_common(M, N, dtype, flags) != RMSNORM_OK || M == 0) return 0;
  return ln_workspace_bytes(M, N, dtype);
}

int layernorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx, const void* gamma,
                  const float* mean, const float* rstd, int64_t M, int64_t N,
                  rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx, void* dgamma,
                  void* dbeta, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ln_bwd_impl(dy, lddy, x, ldx, gamma, mean, rstd, M, N, dtype, flags, dx, lddx, dgamma,
                     dbeta, workspace, workspace_bytes, stream);
}

int layernorm_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                       const void* gamma, const float* mean, const float* rstd, int64_t M,
                       int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_ln_rows_args(dy, lddy, x, ldx, gamma, mean, rstd, M, N, dtype, flags, dx,
                                    lddx, workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  return ln_rows_launch(dy, lddy, x, ldx, gamma, mean, rstd, M, N, dtype, dx, lddx, workspace,
                        stream);
}

int layernorm_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                         rmsnorm_dtype_t dtype, uint32_t flags, void* dgamma, void* dbeta,
                         hipStream_t stream) {
  const int st = check_ln_reduce_args(workspace, workspace_bytes, M, N, dtype, flags, dgamma,
                                      dbeta);
  if (st != RMSNORM_OK) return st;
  return ln_reduce_launch(workspace, M, N, dtype, flags, dgamma, dbeta, stream);
}

int layernorm_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, int pass,
                         int align_bytes, rmsnorm_plan_t* plan) {
  const int st = check_ln_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!plan) return RMSNORM_ERR_NULL_POINTER;
  if (pass < RMSNORM_PASS_FWD || pass > RMSNORM_PASS_BWD_REDUCE) return RMSNORM_ERR_ARGUMENT;
  if (align_bytes < 1 || align_bytes > 4096 || (align_bytes & (align_bytes - 1)))
    return RMSNORM_ERR_ARGUMENT;
  fill_ln_plan(M, N, dtype, pass, std::min(align_bytes, 16), plan, 1, true);
  return RMSNORM_OK;
}

int rmsnorm_add_fwd(const void* x, int64_t ldx, const void* res, int64_t ldr, const void* gamma,
                    float eps, int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                    void* y, int64_t ldy, void* h, int64_t ldh, float* rstd,
                    hipStream_t stream) {
  return add_fwd_impl(x, ldx, res, ldr, gamma, eps, M, N, dtype, flags, y, ldy, h, ldh, rstd,
                      stream);
}

size_t rmsnorm_add_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                       uint32_t flags) {
  if (check_add_common(M, N, dtype, flags) != RMSNORM_OK || M == 0) return 0;
  return add_workspace_bytes(M, N, dtype);
}

int rmsnorm_add_bwd(const void* dy, int64_t lddy, const void* dh, int64_t lddh, const void* h,
                    int64_t ldh, const void* gamma, const float* rstd, int64_t M, int64_t N,
                    rmsnorm_dtype_t dtype, uint32_t flags, void* dx, int64_t lddx,
                    void* dgamma, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return add_bwd_impl(dy, lddy, dh, lddh, h, ldh, gamma, rstd, M, N, dtype, flags, dx, lddx,
                      dgamma, workspace, workspace_bytes, stream);
}

int rmsnorm_add_bwd_rows(const void* dy, int64_t lddy, const void* dh, int64_t lddh,
                         const void* h, int64_t ldh, const void* gamma, const float* rstd,
                         int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                         int64_t lddx, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  const int st = check_add_rows_args(dy, lddy, dh, lddh, h, ldh, gamma, rstd, M, N, dtype, flags,
                                     dx, lddx, workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  return add_rows_launch(dy, lddy, dh, lddh, h, ldh, gamma, rstd, M, N, dtype, flags, dx, lddx,
                         workspace, stream);
}

int rmsnorm_add_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                           rmsnorm_dtype_t dtype, uint32_t flags, void* dgamma,
                           hipStream_t stream) {
  const int st = check_add_reduce_args(workspace, workspace_bytes, M, N, dtype, flags, dgamma);
  if (st != RMSNORM_OK) return st;
  return reduce_columns(static_cast<const float*>(workspace),
                        add_bwd_partials(M, N, elem_bytes(dtype)), N, dtype, flags, dgamma,
                        stream);
}

int rmsnorm_add_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                           int pass, int align_bytes, rmsnorm_plan_t* plan) {
  const int st = check_add_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!plan) return RMSNORM_ERR_NULL_POINTER;
  if (pass < RMSNORM_PASS_FWD || pass > RMSNORM_PASS_BWD_REDUCE) return RMSNORM_ERR_ARGUMENT;
  if (align_bytes < 1 || align_bytes > 4096 || (align_bytes & (align_bytes - 1)))
    return RMSNORM_ERR_ARGUMENT;
  fill_add_plan(M, N, dtype, pass, std::min(align_bytes, 16), plan);
  return RMSNORM_OK;
}

int rmsnorm_cast_fwd(const void* x, int64_t ldx, const void* gamma, float eps, int64_t M,
                     int64_t N, rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype,
                     uint32_t flags, void* y, int64_t ldy, float* rstd, hipStream_t stream) {
  return cast_fwd_impl(x, ldx, gamma, eps, M, N, dtype, out_dtype, flags, y, ldy, rstd, stream);
}

size_t rmsnorm_cast_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                        rmsnorm_dtype_t out_dtype, uint32_t flags) {
  if (check_cast_common(M, N, dtype, out_dtype, flags) != RMSNORM_OK || M == 0) return 0;
  return cast_workspace_bytes(M, N);
}

int rmsnorm_cast_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                     const void* gamma, const float* rstd, int64_t M, int64_t N,
                     rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype, uint32_t flags,
                     void* dx, int64_t lddx, void* dgamma, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return cast_bwd_impl(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, out_dtype, flags, dx, lddx,
                       dgamma, workspace, workspace_bytes, stream);
}

int rmsnorm_cast_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                          const void* gamma, const float* rstd, int64_t M, int64_t N,
                          rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype, uint32_t flags,
                          void* dx, int64_t lddx, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const int st = check_cast_rows_args(dy, lddy, x, ldx, gamma, rstd, M, N, dtype, out_dtype,
                                      flags, dx, lddx, workspace, workspace_bytes);
  if (st != RMSNORM_OK) return st;
  return cast_rows_launch(dy, lddy, x, ldx, gamma, rstd, M, N, out_dtype, flags, dx, lddx,
                          workspace, stream);
}

int rmsnorm_cast_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M,
                            int64_t N, rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype,
                            uint32_t flags, void* dgamma, hipStream_t stream) {
  const int st = check_cast_reduce_args(workspace, workspace_bytes, M, N, dtype, out_dtype,
                                        flags, dgamma);
  if (st != RMSNORM_OK) return st;
  return reduce_columns(static_cast<const float*>(workspace), ln_partials(M, N, kCastIn), N,
                        dtype, flags, dgamma, stream);
}

int rmsnorm_cast_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                            rmsnorm_dtype_t out_dtype, uint32_t flags, int pass,
                            int align_bytes, rmsnorm_plan_t* plan) {
  const int st = check_cast_common(M, N, dtype, out_dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!plan) return RMSNORM_ERR_NULL_POINTER;
  if (pass < RMSNORM_PASS_FWD || pass > RMSNORM_PASS_BWD_REDUCE) return RMSNORM_ERR_ARGUMENT;
  if (align_bytes < 1 || align_bytes > 4096 || (align_bytes & (align_bytes - 1)))
    return RMSNORM_ERR_ARGUMENT;
  fill_cast_plan(M, N, pass, std::min(align_bytes, 16), plan);
  return RMSNORM_OK;
}

}  // extern "C"
