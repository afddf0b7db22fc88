// C ABI of the RMSNorm library: argument checks, launch plans, dispatch.
//
// Contract (page "Check an AI model calculation before accelerating it",
// section "The memory contract is part of the computation"): inputs are
// checked before anything is written, and unsupported inputs are rejected
// rather than rerouted (section "Adapting the kernel and moving to
// production": no silent fallback).  The accepted domain is widened from the
// page's (fp32/fp16, N <= 4096, a 64 MiB scratch cap on an M x N partial
// array) to fp32/fp16/bf16 and N <= 65536, because the M x N partial array is
// replaced by a [P, N] one (P = number of backward workgroups).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "../../include/rmsnorm.h"
#include "rmsnorm_kernels.hpp"

namespace {

using namespace rmsnorm_hip;

// The plan is a pure function of its arguments (no device queries), so the
// workspace size and the order of every reduction are reproducible.  It is
// sized for MI355X: 256 compute units.
constexpr int kCUs = 256;
constexpr int kMaxChunksPreferred = 16;  // register-resident chunks per thread
constexpr int kMaxLdsBytes = 160 * 1024;

int elem_bytes(int dtype) { return dtype == RMSNORM_F32 ? 4 : 2; }

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
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

// Backward workgroup count P: a function of (M, N, dtype) only, computed
// with the vector width that N alone allows.
int64_t bwd_partials(int64_t M, int64_t N, int dtype) {
  if (M <= 0) return 0;
  const int vec = pick_vec(N, elem_bytes(dtype), 16);
  const Rows rw = pick_rows(N, vec);
  if (rw.tpr == kWave) {
    const int maxc = pow2_at_least(rw.chunks);
    const int groups = 8;                     // wavefronts (rows) per workgroup
    const int per_cu = maxc <= 2 ? 4 : (maxc <= 4 ? 2 : 1);
    return std::min<int64_t>(ceil_div(M, groups), static_cast<int64_t>(kCUs) * per_cu);
  }
  const int per_cu = std::max(1, 1024 / rw.tpr);
  return std::min<int64_t>(M, static_cast<int64_t>(kCUs) * per_cu);
}

void fill_plan(int64_t M, int64_t N, int dtype, int pass, int align,
               rmsnorm_plan_t* p) {
  std::memset(p, 0, sizeof(*p));
  const int es = elem_bytes(dtype);
  const int vec = pick_vec(N, es, align);
  const Rows rw = pick_rows(N, vec);
  p->vec = vec;
  p->chunks = rw.chunks;
  p->threads_per_row = rw.tpr;
  if (pass == RMSNORM_PASS_FWD) {
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
  } else if (pass == RMSNORM_PASS_BWD_ROWS) {
    p->partials = bwd_partials(M, N, dtype);
    p->grid = p->partials;
    if (rw.tpr == kWave) {
      p->kernel = RMSNORM_KERNEL_BWD_WAVE;
      p->block_threads = 512;
      p->lds_bytes = N * 4;
    } else {
      p->kernel = RMSNORM_KERNEL_BWD_BLOCK;
      p->block_threads = rw.tpr;
      const int64_t xbytes = N * es;
      p->x_in_lds = (xbytes + 1024 <= kMaxLdsBytes) ? 1 : 0;
      p->lds_bytes = p->x_in_lds ? xbytes : 0;
    }
  } else {
    p->kernel = RMSNORM_KERNEL_BWD_REDUCE;
    p->partials = bwd_partials(M, N, dtype);
    p->block_threads = 1024;
    p->grid = ceil_div(N, kWave);
    p->threads_per_row = 0;
    p->chunks = 0;
    p->vec = 1;
  }
}

template <typename... KArgs>
hipError_t launch_exact(void (*kernel)(KArgs...), int64_t grid, int block,
                        size_t lds, hipStream_t stream, KArgs... args) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel),
                         dim3(static_cast<unsigned>(grid)), dim3(block), argv, lds,
                         stream);
}

// Converts each argument to the kernel's parameter type, then launches.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), int64_t grid, int block, size_t lds,
                  hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  return launch_exact(kernel, grid, block, lds, stream, static_cast<KArgs>(args)...);
}

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
                        int offset, hipStream_t s) {
  hipError_t err = hipErrorInvalidValue;
  const int maxc = pow2_at_least(p.chunks);
#define FWD_LAUNCH(DT_, VEC_, MAXC_)                                              \
  err = (p.kernel == RMSNORM_KERNEL_FWD_WAVE)                                     \
            ? launch(fwd_wave_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads, 0, \
                     s, x, g, y, rstd, M, N, p.chunks, eps, offset)               \
            : launch(fwd_block_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads, 0, \
                     s, x, g, y, rstd, M, N, p.chunks, eps, offset)
  switch (maxc) { RMSNORM_MAXC_CASES(FWD_LAUNCH, DT, VEC) default: break; }
#undef FWD_LAUNCH
  return err;
}

template <int DT, int VEC>
hipError_t bwd_rows_dispatch(const rmsnorm_plan_t& p, const void* dy, const void* x,
                             const void* g, const float* rstd, void* dx, float* part,
                             int64_t M, int N, int offset, hipStream_t s) {
  hipError_t err = hipErrorInvalidValue;
  const int maxc = pow2_at_least(p.chunks);
  const int64_t P = p.partials;
#define BWD_LAUNCH(DT_, VEC_, MAXC_)                                                   \
  if (p.kernel == RMSNORM_KERNEL_BWD_WAVE)                                             \
    err = launch(bwd_wave_kernel<DT_, VEC_, MAXC_>, p.grid, p.block_threads,           \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P);                                                 \
  else if (p.x_in_lds)                                                                 \
    err = launch(bwd_block_kernel<DT_, VEC_, MAXC_, true>, p.grid, p.block_threads,    \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P);                                                 \
  else                                                                                 \
    err = launch(bwd_block_kernel<DT_, VEC_, MAXC_, false>, p.grid, p.block_threads,   \
                 static_cast<size_t>(p.lds_bytes), s, dy, x, g, rstd, dx, part, M, N,  \
                 p.chunks, offset, P)
  switch (maxc) { RMSNORM_MAXC_CASES(BWD_LAUNCH, DT, VEC) default: break; }
#undef BWD_LAUNCH
  return err;
}

template <int DT>
hipError_t fwd_by_vec(const rmsnorm_plan_t& p, const void* x, const void* g, void* y,
                      float* rstd, int64_t M, int N, float eps, int offset,
                      hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (p.vec * es) {
    case 16: return fwd_dispatch<DT, 16 / es>(p, x, g, y, rstd, M, N, eps, offset, s);
    case 8: return fwd_dispatch<DT, 8 / es>(p, x, g, y, rstd, M, N, eps, offset, s);
    case 4: return fwd_dispatch<DT, 4 / es>(p, x, g, y, rstd, M, N, eps, offset, s);
    case 2:
      if constexpr (es == 2) return fwd_dispatch<DT, 1>(p, x, g, y, rstd, M, N, eps, offset, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t bwd_rows_by_vec(const rmsnorm_plan_t& p, const void* dy, const void* x,
                           const void* g, const float* rstd, void* dx, float* part,
                           int64_t M, int N, int offset, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (p.vec * es) {
    case 16: return bwd_rows_dispatch<DT, 16 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, s);
    case 8: return bwd_rows_dispatch<DT, 8 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, s);
    case 4: return bwd_rows_dispatch<DT, 4 / es>(p, dy, x, g, rstd, dx, part, M, N, offset, s);
    case 2:
      if constexpr (es == 2)
        return bwd_rows_dispatch<DT, 1>(p, dy, x, g, rstd, dx, part, M, N, offset, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// ---- argument checks --------------------------------------------------------

int check_common(int64_t M, int64_t N, int dtype, uint32_t flags) {
  if (dtype != RMSNORM_F32 && dtype != RMSNORM_F16 && dtype != RMSNORM_BF16)
    return RMSNORM_ERR_DTYPE;
  if (flags & ~RMSNORM_FLAG_OFFSET) return RMSNORM_ERR_FLAGS;
  if (N < 1 || N > RMSNORM_MAX_N || M < 0 || M > RMSNORM_MAX_M) return RMSNORM_ERR_SHAPE;
  return RMSNORM_OK;
}

bool misaligned(const void* p, int bytes) {
  return p && (reinterpret_cast<uintptr_t>(p) % bytes) != 0;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Span a, Span b) {
  if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Every output span must be disjoint from every input span and from every
// other output span.
bool any_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Span& i : ins)
      if (overlaps(*o, i)) return true;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlaps(*o, *o2)) return true;
  }
  return false;
}

int check_bwd_rows_args(const void* dy, const void* x, const void* gamma,
                        const float* rstd, int64_t M, int64_t N, int dtype,
                        uint32_t flags, const void* dx, const void* workspace,
                        size_t workspace_bytes) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (M == 0) return RMSNORM_OK;
  if (!dy || !x || !gamma || !rstd || !dx) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(dy, es) || misaligned(x, es) || misaligned(gamma, es) ||
      misaligned(dx, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, static_cast<rmsnorm_dtype_t>(dtype), flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  const int64_t mat = M * N * es;
  if (any_overlap({span(dx, mat), span(workspace, static_cast<int64_t>(need))},
                  {span(dy, mat), span(x, mat), span(gamma, N * es), span(rstd, M * 4)}))
    return RMSNORM_ERR_OVERLAP;
  return RMSNORM_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? RMSNORM_OK : RMSNORM_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* rmsnorm_status_string(int status) {
  switch (status) {
    case RMSNORM_OK: return "ok";
    case RMSNORM_ERR_NULL_POINTER: return "a required pointer is NULL";
    case RMSNORM_ERR_DTYPE: return "unsupported dtype (fp32, fp16 and bf16 are supported)";
    case RMSNORM_ERR_SHAPE: return "unsupported shape (need 1 <= N <= 65536 and 0 <= M <= 2^40)";
    case RMSNORM_ERR_EPS: return "eps must be finite and positive";
    case RMSNORM_ERR_FLAGS: return "unknown flag bits";
    case RMSNORM_ERR_WORKSPACE: return "workspace missing or smaller than rmsnorm_bwd_workspace_bytes()";
    case RMSNORM_ERR_ALIGNMENT: return "pointer not aligned to its element size (workspace: 16 bytes)";
    case RMSNORM_ERR_OVERLAP: return "an output buffer overlaps an input or another output";
    case RMSNORM_ERR_LAUNCH: return "kernel launch failed";
    case RMSNORM_ERR_ARGUMENT: return "invalid argument";
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
  if (check_common(M, N, dtype, flags) != RMSNORM_OK) return 0;
  return static_cast<size_t>(bwd_partials(M, N, dtype) * N * 4);
}

int rmsnorm_fwd(const void* x, const void* gamma, float eps, int64_t M, int64_t N,
                rmsnorm_dtype_t dtype, uint32_t flags, void* y, float* rstd,
                hipStream_t stream) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return RMSNORM_ERR_EPS;
  if (M == 0) return RMSNORM_OK;
  if (!x || !gamma || !y || !rstd) return RMSNORM_ERR_NULL_POINTER;
  const int es = elem_bytes(dtype);
  if (misaligned(x, es) || misaligned(gamma, es) || misaligned(y, es) || misaligned(rstd, 4))
    return RMSNORM_ERR_ALIGNMENT;
  const int64_t mat = M * N * es;
  if (any_overlap({span(y, mat), span(rstd, M * 4)}, {span(x, mat), span(gamma, N * es)}))
    return RMSNORM_ERR_OVERLAP;
  rmsnorm_plan_t p;
  fill_plan(M, N, dtype, RMSNORM_PASS_FWD, pointer_alignment({x, gamma, y}), &p);
  const int off = (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0;
  const int n = static_cast<int>(N);
  hipError_t e;
  switch (dtype) {
    case RMSNORM_F32: e = fwd_by_vec<kF32>(p, x, gamma, y, rstd, M, n, eps, off, stream); break;
    case RMSNORM_F16: e = fwd_by_vec<kF16>(p, x, gamma, y, rstd, M, n, eps, off, stream); break;
    default: e = fwd_by_vec<kBF16>(p, x, gamma, y, rstd, M, n, eps, off, stream); break;
  }
  return status_of(e);
}

int rmsnorm_bwd_rows(const void* dy, const void* x, const void* gamma, const float* rstd,
                     int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bwd_rows_args(dy, x, gamma, rstd, M, N, dtype, flags, dx, workspace,
                               workspace_bytes);
  if (st != RMSNORM_OK || M == 0) return st;
  rmsnorm_plan_t p;
  fill_plan(M, N, dtype, RMSNORM_PASS_BWD_ROWS, pointer_alignment({dy, x, gamma, dx}), &p);
  const int off = (flags & RMSNORM_FLAG_OFFSET) ? 1 : 0;
  const int n = static_cast<int>(N);
  float* part = static_cast<float*>(workspace);
  hipError_t e;
  switch (dtype) {
    case RMSNORM_F32: e = bwd_rows_by_vec<kF32>(p, dy, x, gamma, rstd, dx, part, M, n, off, stream); break;
    case RMSNORM_F16: e = bwd_rows_by_vec<kF16>(p, dy, x, gamma, rstd, dx, part, M, n, off, stream); break;
    default: e = bwd_rows_by_vec<kBF16>(p, dy, x, gamma, rstd, dx, part, M, n, off, stream); break;
  }
  return status_of(e);
}

int rmsnorm_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M, int64_t N,
                       rmsnorm_dtype_t dtype, uint32_t flags, float* dgamma,
                       hipStream_t stream) {
  int st = check_common(M, N, dtype, flags);
  if (st != RMSNORM_OK) return st;
  if (!dgamma) return RMSNORM_ERR_NULL_POINTER;
  if (misaligned(dgamma, 4)) return RMSNORM_ERR_ALIGNMENT;
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, dtype, flags);
  if (workspace_bytes < need || (need > 0 && !workspace)) return RMSNORM_ERR_WORKSPACE;
  if (misaligned(workspace, 16)) return RMSNORM_ERR_ALIGNMENT;
  if (any_overlap({span(dgamma, N * 4)}, {span(workspace, static_cast<int64_t>(need))}))
    return RMSNORM_ERR_OVERLAP;
  rmsnorm_plan_t p;
  fill_plan(M, N, dtype, RMSNORM_PASS_BWD_REDUCE, 16, &p);
  const float* part = static_cast<const float*>(workspace);
  const int n = static_cast<int>(N);
  return status_of(launch(bwd_reduce_kernel, p.grid, p.block_threads, 0, stream, part,
                          dgamma, p.partials, n));
}

int rmsnorm_bwd(const void* dy, const void* x, const void* gamma, const float* rstd,
                int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                float* dgamma, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_bwd_rows_args(dy, x, gamma, rstd, M, N, dtype, flags, dx, workspace,
                               workspace_bytes);
  if (st != RMSNORM_OK) return st;
  if (!dgamma) return RMSNORM_ERR_NULL_POINTER;
  if (misaligned(dgamma, 4)) return RMSNORM_ERR_ALIGNMENT;
  const int es = elem_bytes(dtype);
  const int64_t mat = M * N * es;
  const size_t need = rmsnorm_bwd_workspace_bytes(M, N, dtype, flags);
  if (any_overlap({span(dgamma, N * 4), span(dx, mat), span(workspace, static_cast<int64_t>(need))},
                  {span(dy, mat), span(x, mat), span(gamma, N * es), span(rstd, M * 4)}))
    return RMSNORM_ERR_OVERLAP;
  st = rmsnorm_bwd_rows(dy, x, gamma, rstd, M, N, dtype, flags, dx, workspace,
                        workspace_bytes, stream);
  if (st != RMSNORM_OK) return st;
  return rmsnorm_bwd_reduce(workspace, workspace_bytes, M, N, dtype, flags, dgamma, stream);
}

}  // extern "C"
