// Host-side launch helpers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace rmsnorm_hip {

template <typename... KArgs>
hipError_t launch_exact(void (*kernel)(KArgs...), int64_t grid, int block, size_t lds,
                        hipStream_t stream, KArgs... args) {
  // Dynamic LDS beyond the default limit (64 KiB including the kernel's
  // static LDS, at most a few KiB here) must be allowed explicitly.
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel),
                         dim3(static_cast<unsigned>(grid)), dim3(block), argv, lds, stream);
}

// Converts each argument to the kernel's parameter type, then launches.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), int64_t grid, int block, size_t lds,
                  hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  return launch_exact(kernel, grid, block, lds, stream, static_cast<KArgs>(args)...);
}

struct FastFwdArgs {
  const void* x;
  const void* gamma;
  void* y;
  float* rstd;
  int64_t M;
  int N;
  float eps;
  int offset;
  int64_t x_pitch;  // bytes between row starts
  int64_t y_pitch;
};

struct FastBwdArgs {
  const void* dy;
  const void* x;
  const void* gamma;
  const float* rstd;
  void* dx;
  float* part;
  int64_t M;
  int N;
  int offset;
  int64_t P;
  int64_t dy_pitch;  // bytes between row starts
  int64_t x_pitch;
  int64_t dx_pitch;
};

// Launch a listed full-width configuration (rmsnorm_fast_table.hpp) for
// dtype DT.  Returns hipErrorInvalidValue for a configuration not listed.
template <int DT>
hipError_t fast_fwd_launch(int wpr, int ch, int block, int greg, int64_t grid,
                           const FastFwdArgs& a, hipStream_t s);
template <int DT>
hipError_t fast_bwd_launch(int wpr, int ch, int block, int greg, int xlds, int64_t lds,
                           const FastBwdArgs& a, hipStream_t s);
template <int DT>
hipError_t pipe_fwd_launch(int wpr, int ch, int block, int xl, int64_t grid, int64_t lds,
                           const FastFwdArgs& a, hipStream_t s);
template <int DT>
hipError_t pipe_bwd_launch(int wpr, int ch, int block, int dlds, int64_t lds,
                           const FastBwdArgs& a, hipStream_t s);
template <int DT>
hipError_t long_bwd_launch(int ch, int64_t lds, const FastBwdArgs& a, hipStream_t s);

// Split-row plan (rows longer than 65536 elements): segments of
// split_segment_elems(elem_bytes) elements, P row blocks, workgroup
// p*nseg + s on segment s of block p.  `vec` is the access width in
// elements.
struct SplitPlan {
  int vec;
  int nseg;
  int64_t P;
  // Row blocks of the backward pass that keeps no column sums (LayerNorm's
  // stats pass, RMSNorm's apply pass); 0: P.
  int64_t P_free = 0;
};
int split_segment_elems(int elem_bytes);
int split_chunks(int vec, int elem_bytes);
// Forward: stats, finish and apply kernels (y rows hold the segment sums
// between the first two).
hipError_t split_fwd_launch(int dtype, const SplitPlan& sp, const FastFwdArgs& a,
                            hipStream_t s);
// Backward stage 1: stats (dot partials [M, nseg] and part[P, N]), finish
// (coef[M]) and apply (dx).
hipError_t split_bwd_launch(int dtype, const SplitPlan& sp, const FastBwdArgs& a, float* dotp,
                            float* coef, hipStream_t s);

// LayerNorm (layernorm.hip): row-resident kernels, `wpr` wavefronts per row,
// `chunks` vector accesses of `vec` elements per lane, `block` threads per
// workgroup.  Backward: grid = P row blocks, `lds` bytes for the combine.
struct LnPlan {
  int vec;
  int wpr;
  int chunks;
  int block;
  int64_t grid;
  int64_t lds;
};

struct LnFwdArgs {
  const void* x;
  const void* gamma;
  const void* beta;  // may be null: no bias
  void* y;
  float* mean;
  float* rstd;
  int64_t M;
  int N;
  float eps;
  int64_t x_pitch;  // bytes between row starts
  int64_t y_pitch;
};

struct LnBwdArgs {
  const void* dy;
  const void* x;
  const void* gamma;
  const float* mean;
  const float* rstd;
  void* dx;
  float* part;  // [2, P, N]: dgamma partials, then dbeta partials
  int64_t M;
  int N;
  int64_t dy_pitch;
  int64_t x_pitch;
  int64_t dx_pitch;
};

hipError_t ln_fwd_launch(int dtype, const LnPlan& p, const LnFwdArgs& a, hipStream_t s);
// The row-resident forward for full-width rows of up to 8 chunks per lane
// over 16 wavefronts, the weights read from cache (rows past the 16384
// elements of ln_fwd_launch's plans; bf16/fp16 N <= 65536, fp32 N <= 32768).
hipError_t ln_fwd_long_launch(int dtype, const LnPlan& p, const LnFwdArgs& a, hipStream_t s);

// LayerNorm split-row plan (layernorm_split.hip, rows over 16384 elements),
// on the RMSNorm split geometry.  Forward: stats, finish, apply and head
// kernels (y rows hold the segment statistics, then the mean's remainder,
// between them).  Backward stage 1: stats (sums[M, nseg, 3]), finish
// (coef[M, 3]) and apply (dx and part[2, P, N]).
hipError_t ln_split_fwd_launch(int dtype, const SplitPlan& sp, const LnFwdArgs& a,
                               hipStream_t s);
hipError_t ln_split_bwd_launch(int dtype, const SplitPlan& sp, const LnBwdArgs& a, float* sums,
                               float* coef, hipStream_t s);

// RMSNorm with the residual add fused before it (fused_add.hip), on the
// row-resident plan of LayerNorm.
struct AddFwdArgs {
  const void* x;
  const void* res;
  const void* gamma;
  void* y;
  void* h;  // x + res in the dtype
  float* rstd;
  int64_t M;
  int N;
  float eps;
  int offset;
  int64_t x_pitch;  // bytes between row starts
  int64_t res_pitch;
  int64_t y_pitch;
  int64_t h_pitch;
};

struct AddBwdArgs {
  const void* dy;
  const void* dh;  // may be null
  const void* h;
  const void* gamma;
  const float* rstd;
  void* dx;
  float* part;  // [P, N]
  int64_t M;
  int N;
  int offset;
  int64_t dy_pitch;
  int64_t dh_pitch;
  int64_t h_pitch;
  int64_t dx_pitch;
};

hipError_t add_fwd_launch(int dtype, const LnPlan& p, const AddFwdArgs& a, hipStream_t s);
hipError_t add_bwd_launch(int dtype, const LnPlan& p, const AddBwdArgs& a, hipStream_t s);

// The fused add on RMSNorm's long-row kernels (rmsnorm_fast.hpp, listed in
// RMSNORM_ADD_LONG_LIST), for full-width rows of 16 KiB to 128 KiB: the
// forward fwd_fast_kernel with ADD (grid workgroups of 512 threads, one row
// each at a time), the backward bwd_longrow_kernel on h with dh (P
// workgroups, `lds` bytes for a row of h).
template <int DT>
hipError_t add_long_fwd_launch(int ch, int64_t grid, const AddFwdArgs& a, hipStream_t s);
template <int DT>
hipError_t add_long_bwd_launch(int ch, int64_t P, int64_t lds, const AddBwdArgs& a,
                               hipStream_t s);
hipError_t ln_bwd_launch(int dtype, const LnPlan& p, const LnBwdArgs& a, hipStream_t s);
// Backward stage 1 for full-width rows of 4-8 KiB (layernorm_rows.hip):
// grid P, 512 threads, `lds` bytes of dynamic LDS.
hipError_t ln_bwd_rows_launch(int dtype, int64_t P, int64_t lds, const LnBwdArgs& a,
                              hipStream_t s);

// RMSNorm with its output cast to a narrower dtype (fused_cast.hip): float32
// x, gamma and dx; y and dy in the output dtype.  Row-resident plan of
// LayerNorm at float32.
struct CastFwdArgs {
  const void* x;
  const void* gamma;
  void* y;
  float* rstd;
  int64_t M;
  int N;
  float eps;
  int offset;
  int64_t x_pitch;  // bytes between row starts
  int64_t y_pitch;
};

struct CastBwdArgs {
  const void* dy;
  const void* x;
  const void* gamma;
  const float* rstd;
  void* dx;
  float* part;  // [P, N]
  int64_t M;
  int N;
  int offset;
  int64_t dy_pitch;
  int64_t x_pitch;
  int64_t dx_pitch;
};

hipError_t cast_fwd_launch(int out_dtype, const LnPlan& p, const CastFwdArgs& a,
                           hipStream_t s);
hipError_t cast_bwd_launch(int out_dtype, const LnPlan& p, const CastBwdArgs& a,
                           hipStream_t s);

// Split-row plans of the fused add and the fused cast (rmsnorm_split.hip,
// rows over 16384 elements): RMSNorm's split kernels, the add forming and
// writing h in the stats pass and adding dh in the backward apply, the cast
// with float32 x and dx and 16-bit y and dy.  Segments are 16 KiB of x.
hipError_t add_split_fwd_launch(int dtype, const SplitPlan& sp, const AddFwdArgs& a,
                                hipStream_t s);
hipError_t add_split_bwd_launch(int dtype, const SplitPlan& sp, const AddBwdArgs& a,
                                float* dotp, float* coef, hipStream_t s);
hipError_t cast_split_fwd_launch(int out_dtype, const SplitPlan& sp, const CastFwdArgs& a,
                                 hipStream_t s);
hipError_t cast_split_bwd_launch(int out_dtype, const SplitPlan& sp, const CastBwdArgs& a,
                                 float* dotp, float* coef, hipStream_t s);

}  // namespace rmsnorm_hip
