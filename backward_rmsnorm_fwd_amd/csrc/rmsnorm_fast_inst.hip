// Full-width kernel instantiations for one dtype, compiled once per dtype
// with -DRMSNORM_INST_DT=kF32, kF16 or kBF16: the build makes three objects
// of this file, so the library's translation units compile in parallel.
#ifndef RMSNORM_INST_DT
#error "compile with -DRMSNORM_INST_DT=kF32, kF16 or kBF16"
#endif
#include "rmsnorm_fast.hpp"
#include "rmsnorm_fast_table.hpp"
#include "rmsnorm_launch.hpp"

namespace rmsnorm_hip {

constexpr int kDT = RMSNORM_INST_DT;

template <>
hipError_t fast_fwd_launch<kDT>(int wpr, int ch, int block, int greg, int64_t grid,
                                const FastFwdArgs& a, hipStream_t s) {
#define RMSNORM_X(W, C, B, GR)                                                          \
  if (wpr == W && ch == C && block == B && greg == GR)                                  \
    return launch(fwd_fast_kernel<kDT, C, W, B, GR != 0, true>, grid, B, 0, s, a.x,     \
                  a.gamma, a.y, a.rstd, a.M, a.N, a.eps, a.offset, a.x_pitch,           \
                  a.y_pitch, nullptr, nullptr, int64_t(0), int64_t(0));
  RMSNORM_FWD_FAST_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t fast_bwd_launch<kDT>(int wpr, int ch, int block, int greg, int xlds, int64_t lds,
                                const FastBwdArgs& a, hipStream_t s) {
#define RMSNORM_X(W, C, B, GR, XL)                                                      \
  if (wpr == W && ch == C && block == B && greg == GR && xlds == XL)                    \
    return launch(bwd_fast_kernel<kDT, C, W, B, GR != 0, XL != 0, true, kRowsReverse>,  \
                  a.P, B, static_cast<size_t>(lds), s, a.dy, a.x, a.gamma, a.rstd,      \
                  a.dx, a.part, a.M, a.N, a.offset, a.P, a.dy_pitch, a.x_pitch,         \
                  a.dx_pitch);
  RMSNORM_BWD_FAST_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t pipe_fwd_launch<kDT>(int wpr, int ch, int block, int xl, int64_t grid, int64_t lds,
                                const FastFwdArgs& a, hipStream_t s) {
#define RMSNORM_X(W, C, B, XL)                                                          \
  if (wpr == W && ch == C && block == B && xl == XL)                                    \
    return launch(fwd_pipe_kernel<kDT, C, W, B, true, XL != 0, kRowsCyclic>, grid, B,   \
                  static_cast<size_t>(lds), s, a.x, a.gamma, a.y, a.rstd, a.M, a.N,     \
                  a.eps, a.offset, a.x_pitch, a.y_pitch);
  RMSNORM_FWD_PIPE_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t pipe_bwd_launch<kDT>(int wpr, int ch, int block, int dlds, int64_t lds,
                                const FastBwdArgs& a, hipStream_t s) {
#define RMSNORM_X(W, C, B, DL)                                                          \
  if (wpr == W && ch == C && block == B && dlds == DL)                                  \
    return launch(bwd_pipe_kernel<kDT, C, W, B, true, DL != 0, kRowsCyclic>, a.P, B,    \
                  static_cast<size_t>(lds), s, a.dy, a.x, a.gamma, a.rstd, a.dx,        \
                  a.part, a.M, a.N, a.offset, a.P, a.dy_pitch, a.x_pitch, a.dx_pitch);
  RMSNORM_BWD_PIPE_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t long_bwd_launch<kDT>(int ch, int64_t lds, const FastBwdArgs& a, hipStream_t s) {
#define RMSNORM_X(C)                                                                    \
  if (ch == C)                                                                          \
    return launch(bwd_longrow_kernel<kDT, C, true>, a.P, 512, static_cast<size_t>(lds), \
                  s, a.dy, a.x, a.gamma, a.rstd, a.dx, a.part, a.M, a.N, a.offset,      \
                  a.P, a.dy_pitch, a.x_pitch, a.dx_pitch, nullptr, int64_t(0));
  RMSNORM_BWD_LONG_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t add_long_fwd_launch<kDT>(int ch, int64_t grid, const AddFwdArgs& a, hipStream_t s) {
#define RMSNORM_X(C)                                                                    \
  if (ch == C)                                                                          \
    return launch(fwd_fast_kernel<kDT, C, 8, 512, true, true, 1, true>, grid, 512, 0,   \
                  s, a.x, a.gamma, a.y, a.rstd, a.M, a.N, a.eps, a.offset, a.x_pitch,   \
                  a.y_pitch, a.res, a.h, a.res_pitch, a.h_pitch);
  RMSNORM_ADD_LONG_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

template <>
hipError_t add_long_bwd_launch<kDT>(int ch, int64_t P, int64_t lds, const AddBwdArgs& a,
                                    hipStream_t s) {
#define RMSNORM_X(C)                                                                    \
  if (ch == C) {                                                                        \
    if (a.dh)                                                                           \
      return launch(bwd_longrow_kernel<kDT, C, true, true>, P, 512,                     \
                    static_cast<size_t>(lds), s, a.dy, a.h, a.gamma, a.rstd, a.dx,      \
                    a.part, a.M, a.N, a.offset, P, a.dy_pitch, a.h_pitch, a.dx_pitch,   \
                    a.dh, a.dh_pitch);                                                  \
    return launch(bwd_longrow_kernel<kDT, C, true, false>, P, 512,                      \
                  static_cast<size_t>(lds), s, a.dy, a.h, a.gamma, a.rstd, a.dx,        \
                  a.part, a.M, a.N, a.offset, P, a.dy_pitch, a.h_pitch, a.dx_pitch,     \
                  nullptr, int64_t(0));                                                 \
  }
  RMSNORM_ADD_LONG_LIST(RMSNORM_X)
#undef RMSNORM_X
  return hipErrorInvalidValue;
}

}  // namespace rmsnorm_hip
