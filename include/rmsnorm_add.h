/*
 * rmsnorm_add.h -- RMSNorm with the residual add fused before it, in the
 * same MI355X (gfx950) library (librmsnorm.so).
 *
 * The page "PyTorch torch.compile ... LayerNorm and RMSNorm" (itsolotime,
 * introduction) argues that a normalisation kernel gains from fusing the
 * operations around it.  In a transformer block the sublayer output x is
 * added to the residual stream right before the norm; fused, for every row i
 * of M x N matrices:
 *
 *   forward   h_ij = T(x_ij + res_ij)   (the dtype's own add: the float32 sum
 *                                        of the widened operands, rounded to
 *                                        nearest even once; the new residual
 *                                        stream)
 *             y    = RMSNorm(h)          (exactly as rmsnorm_fwd, on h)
 *   backward  dx   = dRMSNorm/dh(dy) + dh
 *             where dh is the gradient arriving on h from the residual
 *             stream (NULL: none); dx is the gradient of both x and res.
 *             The sum is formed in float32 and rounded once.
 *             dgamma = RMSNorm's weight gradient at h (a sum over rows)
 *
 * Conventions are those of rmsnorm.h (device pointers on the current device,
 * caller-owned buffers, row pitches in elements >= N, host-side validation,
 * no fallback, no overlapping outputs, reproducible), with
 * 1 <= N <= RMSNORM_ADD_MAX_N (2^24) and M * N <= RMSNORM_MAX_ELEMENTS: rows
 * of up to RMSNORM_ADD_RESIDENT_MAX_N elements are held in registers, longer
 * rows take the split-row plan.  Flags: RMSNORM_FLAG_OFFSET and
 * RMSNORM_FLAG_DGAMMA_IN_DTYPE as in rmsnorm.h.
 */
#ifndef RMSNORM_ADD_H
#define RMSNORM_ADD_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define RMSNORM_ADD_MAX_N (((int64_t)1) << 24)
#define RMSNORM_ADD_RESIDENT_MAX_N 16384

#define RMSNORM_KERNEL_ADD_FWD 17 /* fused add + forward, rows in registers */
#define RMSNORM_KERNEL_ADD_BWD 18 /* backward stage 1 plus dh, same geometry */
/* Rows over RMSNORM_ADD_RESIDENT_MAX_N: RMSNorm's split-row plan (16 KiB
 * segments); the forward's stats kernel forms and writes h, its apply
 * kernel reads h back; the backward's apply kernel adds dh. */
#define RMSNORM_KERNEL_ADD_FWD_SPLIT 23 /* forward, three kernels */
#define RMSNORM_KERNEL_ADD_BWD_SPLIT 24 /* backward stage 1, three kernels */
/* Full-width rows of 16 to 128 KiB over RMSNORM_ADD_RESIDENT_MAX_N: one
 * 512-thread workgroup per row at a time, as RMSNorm's long rows; the
 * backward keeps a row of h in LDS. */
#define RMSNORM_KERNEL_ADD_FWD_LONG 27 /* forward, the row in registers */
#define RMSNORM_KERNEL_ADD_BWD_LONG 28 /* backward stage 1, h in LDS, dy in registers */

/*
 * Forward.
 *   x      [M, N] T, read (row pitch ldx): the sublayer output
 *   res    [M, N] T, read (row pitch ldr): the residual stream
 *   gamma  [N] T, read (w in offset mode)
 *   eps    finite and > 0
 *   y      [M, N] T, written (row pitch ldy)
 *   h      [M, N] T, written (row pitch ldh): x + res, kept for the residual
 *          stream and for the backward
 *   rstd   [M] float32, written
 * Errors: as rmsnorm_fwd_strided (SHAPE for N > RMSNORM_ADD_MAX_N or
 * M * N above RMSNORM_MAX_ELEMENTS).
 */
int rmsnorm_add_fwd(const void* x, int64_t ldx, const void* res, int64_t ldr,
                    const void* gamma, float eps, int64_t M, int64_t N,
                    rmsnorm_dtype_t dtype, uint32_t flags, void* y, int64_t ldy,
                    void* h, int64_t ldh, float* rstd, hipStream_t stream);

/* Workspace bytes of rmsnorm_add_bwd: float32 partial column sums [P, N],
 * P a fixed function of (M, N, dtype); split rows add one float32 sum per
 * (row, segment) and one coefficient per row, each part from a 16-byte
 * boundary.  0 for M = 0 or invalid arguments. */
size_t rmsnorm_add_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                       uint32_t flags);

/*
 * Backward (stage 1 then the column sums, on `stream`).
 *   dy     [M, N] T, read (row pitch lddy)
 *   dh     [M, N] T, read (row pitch lddh), or NULL when no gradient arrives
 *          on h from the residual stream
 *   h      [M, N] T, read (row pitch ldh): as written by rmsnorm_add_fwd
 *   gamma, rstd  as for rmsnorm_bwd (rstd from rmsnorm_add_fwd)
 *   dx     [M, N] T, written (row pitch lddx): the gradient of x and of res
 *   dgamma [N] float32 (T with RMSNORM_FLAG_DGAMMA_IN_DTYPE), written
 *   workspace, workspace_bytes  as for rmsnorm_bwd, with
 *          rmsnorm_add_bwd_workspace_bytes
 * Errors: as rmsnorm_bwd_strided.
 */
int rmsnorm_add_bwd(const void* dy, int64_t lddy, const void* dh, int64_t lddh,
                    const void* h, int64_t ldh, const void* gamma, const float* rstd,
                    int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                    void* dx, int64_t lddx, void* dgamma, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Backward stage 1 alone (dx and the [P, N] partial column sums in the
 * workspace) and stage 2 alone (dgamma from them), as rmsnorm_bwd_rows and
 * rmsnorm_bwd_reduce. */
int rmsnorm_add_bwd_rows(const void* dy, int64_t lddy, const void* dh, int64_t lddh,
                         const void* h, int64_t ldh, const void* gamma, const float* rstd,
                         int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                         void* dx, int64_t lddx, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);
int rmsnorm_add_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M,
                           int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                           void* dgamma, hipStream_t stream);

/* The launch a pass would use (RMSNORM_PASS_*), as rmsnorm_query_plan. */
int rmsnorm_add_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                           uint32_t flags, int pass, int align_bytes,
                           rmsnorm_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_ADD_H */
