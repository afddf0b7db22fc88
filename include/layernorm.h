/*
 * layernorm.h -- C ABI of the LayerNorm forward/backward kernels in the same
 * MI355X (gfx950) library as RMSNorm (librmsnorm.so).
 *
 * The operation (page "PyTorch torch.compile ... LayerNorm and RMSNorm",
 * itsolotime; section 1.1: each row normalised by its mean and variance,
 * scaled by a learned weight and shifted by a learned bias; section 2: the
 * backward yields the input, weight and bias gradients; section 1.4: the
 * forward keeps the row statistics for the backward), for every row i of an
 * M x N matrix:
 *
 *   forward   mu_i  = (1/N) sum_j x_ij
 *             var_i = (1/N) sum_j (x_ij - mu_i)^2      (biased variance)
 *             r_i   = 1 / sqrt(var_i + eps)
 *             y_ij  = (x_ij - mu_i) * r_i * gamma_j + beta_j
 *   backward  xhat_ij = (x_ij - mu_i) * r_i,  u_ij = dy_ij * gamma_j
 *             dx_ij   = r_i * (u_ij - mean_j(u_ij) - xhat_ij * mean_j(u_ij * xhat_ij))
 *             dgamma_j = sum_i dy_ij * xhat_ij,   dbeta_j = sum_i dy_ij
 *
 * Arithmetic: inputs widened to float32 on load; the row sum is taken in
 * float64; the variance is the mean of the squared deviations from the row
 * mean (from the row held in registers, or, for split rows, from per-segment
 * float64 statistics merged in segment order); the column sums add
 * per-workgroup float32 partials in float64 in a fixed order and round once.
 * Outputs of type T round to nearest even.
 *
 * Conventions are those of rmsnorm.h (device pointers on the current device,
 * caller-owned buffers, work enqueued on `stream`, host-side validation
 * before anything is enqueued, no fallback, no overlapping outputs, bitwise
 * reproducible for equal inputs, shape and alignment), with these
 * differences:
 *  - 1 <= N <= LAYERNORM_MAX_N (2^24) and M * N <= RMSNORM_MAX_ELEMENTS.
 *    Rows of up to LAYERNORM_RESIDENT_MAX_N elements are held in registers
 *    across up to 16 wavefronts of one workgroup; longer rows take the
 *    split-row plan (LAYERNORM_KERNEL_FWD_SPLIT / BWD_SPLIT);
 *  - flags: only RMSNORM_FLAG_DGAMMA_IN_DTYPE (it applies to dgamma and
 *    dbeta); RMSNORM_FLAG_OFFSET is RMSNORM_ERR_FLAGS;
 *  - beta may be NULL in the forward (no bias), dbeta may be NULL in the
 *    backward (the bias gradient is then not written).
 * Status codes and rmsnorm_status_string are shared with rmsnorm.h.
 */
#ifndef LAYERNORM_H
#define LAYERNORM_H

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

#define LAYERNORM_MAX_N (((int64_t)1) << 24)
#define LAYERNORM_RESIDENT_MAX_N 16384

/* Kernels (rmsnorm_plan_t.kernel). */
#define LAYERNORM_KERNEL_FWD 15 /* forward, rows resident in registers */
#define LAYERNORM_KERNEL_BWD 16 /* backward stage 1, same geometry */
/* Split-row plan for N > LAYERNORM_RESIDENT_MAX_N, on the segments of the
 * RMSNorm split plan (16 KiB, one 256-thread workgroup per (row block,
 * segment)).  Forward: a stats kernel writes each segment's float64 sum and
 * sum of squared deviations into the first bytes of the row of y, a finish
 * kernel merges them per row (segment order) into mean and rstd and leaves
 * the mean's float32 rounding remainder in the row's first 4 bytes, an apply
 * kernel writes y except those bytes, and a head kernel writes them.
 * Backward stage 1: stats, finish and apply kernels with the per-row sums in
 * the workspace. */
#define LAYERNORM_KERNEL_FWD_SPLIT 21 /* forward, four kernels */
#define LAYERNORM_KERNEL_BWD_SPLIT 22 /* backward stage 1, three kernels */
/* Backward stage 1 for rows of 257 to 512 16-byte vectors (bf16/fp16
 * 2048 < N <= 4096, float32 1024 < N <= 2048) when every pointer and row
 * pitch is 16-byte aligned: two rows per 512-thread workgroup, x staged in
 * LDS, P = min(ceil(M/2), 512).  Other layouts of the same N run
 * LAYERNORM_KERNEL_BWD on the same P. */
#define LAYERNORM_KERNEL_BWD_ROWS 29

/*
 * Forward.
 *   x      [M, N] T, read; row i starts at element i*ldx (ldx >= N)
 *   gamma  [N] T, read
 *   beta   [N] T, read, or NULL for no bias
 *   eps    added to the variance inside the square root; finite and > 0
 *   y      [M, N] T, written; row i at element i*ldy (ldy >= N)
 *   mean   [M] float32, written (mu_i)
 *   rstd   [M] float32, written (r_i)
 * Errors: NULL_POINTER (x, gamma, y, mean or rstd NULL with M > 0), DTYPE,
 * SHAPE (N outside [1, LAYERNORM_MAX_N], M outside [0, RMSNORM_MAX_M],
 * M * N above RMSNORM_MAX_ELEMENTS), EPS,
 * FLAGS, STRIDE, ALIGNMENT (a pointer not aligned to its element size),
 * OVERLAP (an output overlaps an input or another output), LAUNCH.
 */
int layernorm_fwd(const void* x, int64_t ldx, const void* gamma, const void* beta,
                  float eps, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                  uint32_t flags, void* y, int64_t ldy, float* mean, float* rstd,
                  hipStream_t stream);

/*
 * Bytes of device workspace layernorm_bwd needs: two float32 partial blocks
 * [P, N] (dgamma, then dbeta), P a fixed function of (M, N, dtype); split
 * rows add three float32 sums per (row, segment) and three coefficients per
 * row, each part starting on a 16-byte boundary.  Returns 0 for M = 0 and
 * for invalid arguments.
 */
size_t layernorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                     uint32_t flags);

/*
 * Backward: stage 1 (dx and the partial column sums) then stage 2 (the
 * column sums), both on `stream`.
 *   dy     [M, N] T, read (row pitch lddy)
 *   x      [M, N] T, read (row pitch ldx): the forward's input
 *   gamma  [N] T, read
 *   mean, rstd  [M] float32, read: as written by layernorm_fwd for this x, eps
 *   dx     [M, N] T, written (row pitch lddx)
 *   dgamma [N] float32 (T with RMSNORM_FLAG_DGAMMA_IN_DTYPE), written; zeros
 *          when M = 0
 *   dbeta  [N] like dgamma, written, or NULL to skip the bias gradient
 *   workspace, workspace_bytes: at least layernorm_bwd_workspace_bytes(...)
 *          bytes of device memory, 16-byte aligned, owned by the caller and
 *          not shared with a call that may run concurrently.
 * Errors: as layernorm_fwd (no EPS), plus WORKSPACE.
 */
int layernorm_bwd(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                  const void* gamma, const float* mean, const float* rstd,
                  int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                  void* dx, int64_t lddx, void* dgamma, void* dbeta,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward stage 1 alone: dx and the two [P, N] partial blocks in the
 * workspace.  Arguments as layernorm_bwd, without dgamma and dbeta.
 */
int layernorm_bwd_rows(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                       const void* gamma, const float* mean, const float* rstd,
                       int64_t M, int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                       void* dx, int64_t lddx, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * Backward stage 2 alone: dgamma (and dbeta unless NULL) from the partial
 * blocks layernorm_bwd_rows wrote for the same (M, N, dtype, flags).
 */
int layernorm_bwd_reduce(const void* workspace, size_t workspace_bytes, int64_t M,
                         int64_t N, rmsnorm_dtype_t dtype, uint32_t flags,
                         void* dgamma, void* dbeta, hipStream_t stream);

/*
 * The launch a pass would use (RMSNORM_PASS_FWD, RMSNORM_PASS_BWD_ROWS or
 * RMSNORM_PASS_BWD_REDUCE) for (M, N, dtype, flags) when every pointer and
 * row pitch is `align_bytes`-aligned.  threads_per_row is 64 * wavefronts per
 * row; chunks and vec as in rmsnorm.h.  No device work.
 */
int layernorm_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                         uint32_t flags, int pass, int align_bytes,
                         rmsnorm_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* LAYERNORM_H */
