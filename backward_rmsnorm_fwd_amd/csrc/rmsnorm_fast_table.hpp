// Instantiated full-width (16-byte vector) kernel configurations, shared by
// the host plan (which may only pick a listed configuration) and by the
// per-dtype objects of rmsnorm_fast_inst.hip that instantiate them.
//
// Forward entries:  X(WPR, CH, BLOCK, GREG)
// Backward entries: X(WPR, CH, BLOCK, GREG, XLDS)
// Pipelined forward entries:  X(WPR, CH, BLOCK, XL)
// Pipelined backward entries: X(WPR, CH, BLOCK, DLDS)
// Long-row backward entries: X(CH), 512 threads per row
// Fused-add long-row entries: X(CH), 8 wavefronts of a 512-thread workgroup
//   per row in both directions (the forward with the weight in registers),
//   for rows of 16 KiB to 128 KiB
//   WPR  wavefronts per row, CH 16-byte chunks per thread and row,
//   BLOCK threads per workgroup, GREG weight held in registers across rows,
//   XLDS / XL x staged in LDS by DMA, DLDS dy staged in LDS too.  The
//   pipelined kernels always keep the weight in registers.
// The choice rules live in rmsnorm_api.hip (plan_fast_fwd / plan_fast_bwd);
// the measurements behind them are summarised next to those rules.
#pragma once

#define RMSNORM_FWD_FAST_LIST(X)                                                  \
  X(5, 2, 640, 1)                                                                 \
  X(1, 1, 256, 1) X(1, 2, 256, 1) X(1, 3, 256, 1) X(1, 4, 256, 1)                 \
  X(2, 2, 256, 1) X(2, 3, 256, 1) X(2, 4, 256, 1)                                 \
  X(4, 2, 512, 1) X(4, 3, 512, 1) X(4, 4, 512, 1)                                 \
  X(8, 2, 512, 1) X(8, 3, 512, 1) X(8, 4, 512, 1) X(8, 5, 512, 1) X(8, 6, 512, 1) \
  X(8, 7, 512, 1) X(8, 8, 512, 1) X(8, 9, 512, 1) X(8, 10, 512, 1)                \
  X(8, 11, 512, 1) X(8, 12, 512, 1) X(8, 13, 512, 1) X(8, 14, 512, 1)             \
  X(8, 15, 512, 1) X(8, 16, 512, 1)                                               \
  X(16, 9, 1024, 0) X(16, 10, 1024, 0) X(16, 11, 1024, 0) X(16, 12, 1024, 0)      \
  X(16, 13, 1024, 0) X(16, 14, 1024, 0) X(16, 15, 1024, 0) X(16, 16, 1024, 0)

#define RMSNORM_BWD_FAST_LIST(X) X(4, 2, 512, 1, 1)

#define RMSNORM_FWD_PIPE_LIST(X) X(4, 2, 1024, 1)

#define RMSNORM_BWD_PIPE_LIST(X) \
  X(1, 1, 1024, 0) X(2, 1, 1024, 0) X(4, 1, 1024, 0) X(16, 1, 1024, 1) X(10, 1, 640, 1)

#define RMSNORM_BWD_LONG_LIST(X) \
  X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

#define RMSNORM_ADD_LONG_LIST(X) \
  X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
