/*
 * rmsnorm_cast.h -- RMSNorm with the cast of its output to a narrower dtype
 * fused after it, in the same MI355X (gfx950) library (librmsnorm.so).
 *
 * The page "PyTorch torch.compile ... LayerNorm and RMSNorm" (itsolotime,
 * introduction) argues that a normalisation kernel gains from fusing the
 * operations around it.  After the norm the usual neighbour is a dtype
 * conversion: a float32 residual stream is normalised and handed to a
 * bfloat16 or float16 consumer.  Fused, for every row i of an M x N matrix:
 *
 *   forward   r_i  = 1 / sqrt(sum_j x_ij^2 / N + eps),  g = gamma or 1 + w
 *             y_ij = T_out((x_ij * r_i) * g_j)   (float32 arithmetic as in
 *                                                rmsnorm_fwd, then one
 *                                                round-to-nearest-even cast)
 *   backward  dy arrives in T_out.  A dtype conversion passes its gradient
 *             through unchanged, so dy is widened (exactly) and the RMSNorm
 *             backward runs on it:
 *             u = dy*g,  dx = r*u - x*(r^3 * sum_j(u*x)/N)   (float32)
 *             dgamma_j = sum_i dy_ij * x_ij * r_i
 *
 * Types: x, gamma and dx are float32 (dtype must be RMSNORM_F32); y and dy
 * have out_dtype, RMSNORM_BF16 or RMSNORM_F16; rstd and dgamma are float32.
 * Any other pair is RMSNORM_ERR_DTYPE.
 *
 * Conventions are those of rmsnorm.h (device pointers on the current device,
 * caller-owned buffers, row pitches in elements >= N, work enqueued on
 * `stream`, host-side validation before anything is enqueued, no fallback,
 * no overlapping outputs, bitwise reproducible), with
 * 1 <= N <= RMSNORM_CAST_MAX_N (2^24) and M * N <= RMSNORM_MAX_ELEMENTS: rows
 * of up to RMSNORM_CAST_RESIDENT_MAX_N elements are held in registers,
 * longer rows take the split-row plan.  Flags: RMSNORM_FLAG_OFFSET;
 * RMSNORM_FLAG_DGAMMA_IN_DTYPE is accepted and changes nothing (the input
 * dtype is float32).
 */
#ifndef RMSNORM_CAST_H
#define RMSNORM_CAST_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define RMSNORM_CAST_MAX_N (((int64_t)1) << 24)
#define RMSNORM_CAST_RESIDENT_MAX_N 16384

#define RMSNORM_KERNEL_CAST_FWD 19 /* forward with the cast, rows in registers */
#define RMSNORM_KERNEL_CAST_BWD 20 /* backward stage 1 from the narrow dy */
/* Rows over RMSNORM_CAST_RESIDENT_MAX_N: RMSNorm's split-row plan on 16 KiB
 * segments of the float32 x, the per-segment sums parked in the narrow y. */
#define RMSNORM_KERNEL_CAST_FWD_SPLIT 25 /* forward, three kernels */
#define RMSNORM_KERNEL_CAST_BWD_SPLIT 26 /* backward stage 1, three kernels */

/*
 * Forward.
 *   x      [M, N] float32, read (row pitch ldx)
 *   gamma  [N] float32, read (w in offset mode)
 *   eps    finite and > 0
 *   y      [M, N] out_dtype, written (row pitch ldy)
 *   rstd   [M] float32, written
 * Errors: NULL_POINTER, DTYPE (see above), SHAPE (N outside
 * [1, RMSNORM_CAST_MAX_N], M outside [0, RMSNORM_MAX_M], M * N above
 * RMSNORM_MAX_ELEMENTS), EPS, FLAGS, STRIDE,
 * ALIGNMENT (a pointer not aligned to its element size), OVERLAP, LAUNCH.
 */
int rmsnorm_cast_fwd(const void* x, int64_t ldx, const void* gamma, float eps,
                     int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                     rmsnorm_dtype_t out_dtype, uint32_t flags, void* y, int64_t ldy,
                     float* rstd, hipStream_t stream);

/* Workspace bytes of rmsnorm_cast_bwd: float32 partial column sums [P, N],
 * P a fixed function of (M, N); split rows add one float32 sum per (row,
 * segment) and one coefficient per row, each part from a 16-byte boundary.
 * 0 for M = 0 or invalid arguments. */
size_t rmsnorm_cast_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                        rmsnorm_dtype_t out_dtype, uint32_t flags);

/*
 * Backward (stage 1 then the column sums, on `stream`).
 *   dy     [M, N] out_dtype, read (row pitch lddy)
 *   x      [M, N] float32, read (row pitch ldx): the forward's input
 *   gamma  [N] float32, read
 *   rstd   [M] float32, read: as written by rmsnorm_cast_fwd for this x, eps
 *   dx     [M, N] float32, written (row pitch lddx)
 *   dgamma [N] float32, written; zeros when M = 0
 *   workspace, workspace_bytes: at least rmsnorm_cast_bwd_workspace_bytes(...)
 *          bytes of device memory, 16-byte aligned, owned by the caller and
 *          not shared with a call that may run concurrently.
 * Errors: as rmsnorm_cast_fwd (no EPS), plus WORKSPACE.
 */
int rmsnorm_cast_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                     const void* gamma, const float* rstd, int64_t M, int64_t N,
                     rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype, uint32_t flags,
                     void* dx, int64_t lddx, void* dgamma, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Backward stage 1 alone (dx and the [P, N] partial column sums in the
 * workspace) and stage 2 alone (dgamma from them), as rmsnorm_bwd_rows and
 * rmsnorm_bwd_reduce. */
int rmsnorm_cast_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                          const void* gamma, const float* rstd, int64_t M, int64_t N,
                          rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype, uint32_t flags,
                          void* dx, int64_t lddx, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);
int rmsnorm_cast_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M,
                            int64_t N, rmsnorm_dtype_t dtype, rmsnorm_dtype_t out_dtype,
                            uint32_t flags, void* dgamma, hipStream_t stream);

/* The launch a pass would use (RMSNORM_PASS_*) when every pointer and row
 * pitch is `align_bytes`-aligned, as rmsnorm_query_plan.  No device work. */
int rmsnorm_cast_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                            rmsnorm_dtype_t out_dtype, uint32_t flags, int pass,
                            int align_bytes, rmsnorm_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_CAST_H */
