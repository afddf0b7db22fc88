/*
 * rmsnorm.h -- C ABI of the MI355X (gfx950) RMSNorm forward/backward library.
 *
 * The operation (page "Check an AI model calculation before accelerating it",
 * partitech; sections "Problem and reference formula", "Input backward pass:
 * keep the right N", "Where does the cube of r come from?" and "A sum is not
 * an average"), for every row i of an M x N matrix:
 *
 *   forward   r_i  = 1 / sqrt( (1/N) * sum_j x_ij^2 + eps )
 *             y_ij = x_ij * r_i * g_j
 *   backward  u_ij = dy_ij * g_j
 *             c_i  = (1/N) * sum_j u_ij * x_ij
 *             dx_ij = r_i * u_ij - x_ij * r_i^3 * c_i
 *             dgamma_j = sum_i dy_ij * x_ij * r_i        (a sum over rows)
 *
 * where g_j = gamma_j, or g_j = 1 + w_j when RMSNORM_FLAG_OFFSET is set
 * (offset weight; torchtitan kernel-numerics-verifier page, section
 * "仓库实例 OffsetRMSNorm").  The 1 is added in float32 after the weight is
 * read.  dgamma has the same expression in both modes.
 *
 * Arithmetic: inputs are widened to float32 as they are loaded, before any
 * square or product (section "Why convert before reducing?"); all reductions
 * accumulate in float32 except the final column sum of dgamma, which adds the
 * per-workgroup partial sums in float64.  The mean divides by the logical N
 * (section "N and BLOCK: two sizes you must never confuse").  Outputs of type
 * T are rounded to nearest even.
 *
 * Conventions shared by every entry point:
 *  - x, gamma, dy, y and dx hold elements of one dtype T (rmsnorm_dtype_t);
 *    rstd is float32, dgamma float32 unless RMSNORM_FLAG_DGAMMA_IN_DTYPE
 *    asks for T (the page's reduce_gamma_gradient returns gamma's dtype).
 *  - Matrices are row-major: row i starts at element i*N (dense), or at
 *    element i*ld for the *_strided entry points, ld >= N given per matrix.
 *    Any leading dimensions are flattened into M by the caller.
 *  - All pointers are device pointers on the calling thread's current HIP
 *    device; the stream belongs to that device (0 = the null stream).
 *  - The caller owns and allocates every buffer.  The library allocates
 *    nothing, keeps no state between calls and never synchronizes the host:
 *    kernels are enqueued on `stream` and the call returns.  Calls on
 *    different streams are independent.  The one exception is
 *    rmsnorm_bwd_noalloc, which uses a fixed device buffer of the library's
 *    own (see there).
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call returns a negative status and writes nothing.  There is no
 *    fallback path: an unsupported input is an error.
 *  - Outputs must not overlap inputs or each other (RMSNORM_ERR_OVERLAP).
 *  - Every buffer must end below byte address 2^57 (base + (M-1)*pitch +
 *    row bytes, formed without overflow); a matrix past that limit is
 *    RMSNORM_ERR_STRIDE when its rows are padded (ld > N) and
 *    RMSNORM_ERR_SHAPE otherwise, so the kernels' 64-bit address sums
 *    cannot wrap.
 *  - Pointers must be aligned to their element size (RMSNORM_ERR_ALIGNMENT);
 *    the workspace to 16 bytes.  Wider alignment lets the kernels use wider
 *    (up to 16-byte) accesses.
 *  - Bitwise reproducibility: the same inputs and (M, N, dtype, flags, and
 *    pointer alignment modulo 16 bytes) give bitwise-identical outputs; no
 *    atomics are used and every reduction has a fixed order.
 *  - Limits: 1 <= N <= RMSNORM_MAX_N (2^24), 0 <= M <= RMSNORM_MAX_M and
 *    M * N <= RMSNORM_MAX_ELEMENTS.  M = 0 is a no-op for the row outputs;
 *    the backward then writes dgamma = 0.  Rows of more than 65536 elements
 *    take the split-row plan (RMSNORM_KERNEL_FWD_SPLIT / BWD_SPLIT).
 */
#ifndef RMSNORM_H
#define RMSNORM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RMSNORM_F32 = 0,
  RMSNORM_F16 = 1,
  RMSNORM_BF16 = 2,
  /* Not dtypes.  They widen the enum to every 32-bit value, so that any code
   * a C or foreign-function caller passes is a defined value of the type,
   * which the library then rejects with RMSNORM_ERR_DTYPE. */
  RMSNORM_DTYPE_ENUM_MIN_ = -2147483647 - 1,
  RMSNORM_DTYPE_ENUM_MAX_ = 2147483647
} rmsnorm_dtype_t;

/* flags */
#define RMSNORM_FLAG_OFFSET 1u /* apply the weight as (1 + w) */
/* Write dgamma in the input dtype T (rounded to nearest even from the
 * float32 value of the sum), as the weight's own dtype, instead of float32. */
#define RMSNORM_FLAG_DGAMMA_IN_DTYPE 2u

#define RMSNORM_MAX_N (((int64_t)1) << 24)
#define RMSNORM_MAX_M (((int64_t)1) << 40)
#define RMSNORM_MAX_ELEMENTS (((int64_t)1) << 46) /* M * N */

/* status codes */
#define RMSNORM_OK 0
#define RMSNORM_ERR_NULL_POINTER (-1)
#define RMSNORM_ERR_DTYPE (-2)
#define RMSNORM_ERR_SHAPE (-3)
#define RMSNORM_ERR_EPS (-4)
#define RMSNORM_ERR_FLAGS (-5)
#define RMSNORM_ERR_WORKSPACE (-6)
#define RMSNORM_ERR_ALIGNMENT (-7)
#define RMSNORM_ERR_OVERLAP (-8)
#define RMSNORM_ERR_LAUNCH (-9)
#define RMSNORM_ERR_ARGUMENT (-10)
#define RMSNORM_ERR_STRIDE (-11) /* a row stride below N or above 2^40, or a
                                   padded matrix ending past byte 2^57 */

/*
 * Forward: y = x * r * g per row, and rstd[i] = r_i (float32) kept for the
 * backward (the page keeps the inverse RMS between the passes).
 *   x     [M, N] T, read
 *   gamma [N] T (gamma, or w in offset mode), read
 *   eps   added to the mean square inside the square root; finite and > 0
 *   y     [M, N] T, written (every element).  For N > 65536 the first
 *         bytes of each row of y hold the per-segment partial sums between
 *         the forward's kernels; on return y holds only the result.
 *   rstd  [M] float32, written
 * Errors: NULL_POINTER (a needed pointer is NULL; pointers may be NULL only
 * when M = 0), DTYPE, SHAPE, EPS, FLAGS, ALIGNMENT, OVERLAP, LAUNCH (the
 * kernel launch failed; the HIP error is not cleared).
 */
int rmsnorm_fwd(const void* x, const void* gamma, float eps, int64_t M,
                int64_t N, rmsnorm_dtype_t dtype, uint32_t flags, void* y,
                float* rstd, hipStream_t stream);

/*
 * Bytes of device workspace the backward needs for (M, N, dtype, flags): the
 * per-workgroup float32 partial sums of dgamma, [P, N] with P a fixed
 * function of (M, N, dtype).  For N > 65536 it also holds, each from a
 * 16-byte boundary, the [M, segments] float32 partial row sums of dy*g*x and
 * the [M] per-row coefficients r^3*c.  Returns 0 for M = 0 and for invalid
 * arguments (which the backward then rejects).
 */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                                   uint32_t flags);

/*
 * Backward, both stages on `stream`, in order: rmsnorm_bwd_rows then
 * rmsnorm_bwd_reduce.
 *   dy     [M, N] T, read (gradient of the loss with respect to y)
 *   x      [M, N] T, read (the forward's input)
 *   gamma  [N] T, read (gamma, or w in offset mode)
 *   rstd   [M] float32, read (as written by rmsnorm_fwd for this x and eps)
 *   dx     [M, N] T, written
 *   dgamma [N] float32, written (sum over the M rows; zeros when M = 0); with
 *          RMSNORM_FLAG_DGAMMA_IN_DTYPE [N] T instead
 *   workspace, workspace_bytes: device scratch of at least
 *          rmsnorm_bwd_workspace_bytes(M, N, dtype, flags) bytes, 16-byte
 *          aligned, owned by the caller; its contents on entry do not matter
 *          and on return hold the partial sums.  It must not be shared with a
 *          call that may run concurrently.
 * Errors: as rmsnorm_fwd (no EPS: eps is already inside rstd), plus
 * WORKSPACE (too small, or NULL when a non-zero size is needed).
 */
int rmsnorm_bwd(const void* dy, const void* x, const void* gamma,
                const float* rstd, int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                uint32_t flags, void* dx, void* dgamma, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/*
 * Backward stage 1 alone (the page's per-row backward pass, section
 * "Input backward pass: keep the right N"): writes dx and the [P, N] float32
 * partial column sums of dy*x*r into the workspace, each workgroup summing a
 * fixed block of rows (section "Reducing dgamma without a write race": each
 * program writes its own area, a second pass adds them by column).
 * Arguments as rmsnorm_bwd, without dgamma.
 */
int rmsnorm_bwd_rows(const void* dy, const void* x, const void* gamma,
                     const float* rstd, int64_t M, int64_t N,
                     rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Backward stage 2 alone: dgamma[j] = sum over p = 0..P-1 of partial[p, j],
 * added in float64 in a fixed order and rounded once to float32 (then to T
 * with RMSNORM_FLAG_DGAMMA_IN_DTYPE).  The
 * workspace must hold what rmsnorm_bwd_rows wrote for the same
 * (M, N, dtype, flags).
 */
int rmsnorm_bwd_reduce(const void* workspace, size_t workspace_bytes,
                       int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                       uint32_t flags, void* dgamma, hipStream_t stream);

/*
 * Strided variants (the page's section "Adapting the kernel and moving to
 * production": other layouts need addressing through strides, and tests).
 * Identical to rmsnorm_fwd / rmsnorm_bwd except that row i of x, y, dy and dx
 * starts at element i*ldx, i*ldy, i*lddy, i*lddx of its matrix (each ld >= N;
 * elements between the end of one row and the start of the next are neither
 * read nor written).  The contiguous entry points are these with ld = N.
 * An output may share a buffer with an input when their rows interleave
 * without a common byte (same ld, column ranges disjoint); matrices with
 * different strides must have disjoint extents.
 * Errors: as rmsnorm_fwd / rmsnorm_bwd, plus STRIDE.
 */
int rmsnorm_fwd_strided(const void* x, int64_t ldx, const void* gamma, float eps,
                        int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                        uint32_t flags, void* y, int64_t ldy, float* rstd,
                        hipStream_t stream);

int rmsnorm_bwd_strided(const void* dy, int64_t lddy, const void* x,
                        int64_t ldx, const void* gamma, const float* rstd,
                        int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                        uint32_t flags, void* dx, int64_t lddx, void* dgamma,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Backward with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Arguments, results and errors are those
 * of rmsnorm_bwd, whose kernels and plan it uses (dx and dgamma are bitwise
 * identical to rmsnorm_bwd's), except that the dgamma partial sums go to a
 * buffer the library holds in device memory: RMSNORM_NOALLOC_SCRATCH_BYTES
 * (72 MiB) on each device the library runs on, reserved when the library's
 * code is loaded on that device and held until the process ends.  The call
 * allocates nothing; the first call with a device current looks up that
 * device's buffer.
 *   - Shapes needing more than RMSNORM_NOALLOC_SCRATCH_BYTES of partial sums
 *     (rmsnorm_bwd_workspace_bytes gives the need) are rejected with
 *     WORKSPACE before anything is enqueued.
 *   - All calls on one device share its buffer, which keeps the last call's
 *     partial sums (nothing in it needs to start at zero).  Calls on one
 *     stream are ordered and safe; calls that may overlap in time on one
 *     device (other streams, other threads without ordering) race and give
 *     wrong dgamma.
 * Errors: as rmsnorm_bwd (WORKSPACE as above), and LAUNCH when the buffer's
 * device address cannot be obtained.
 */
#define RMSNORM_NOALLOC_SCRATCH_BYTES (((size_t)72) << 20)
int rmsnorm_bwd_noalloc(const void* dy, const void* x, const void* gamma,
                        const float* rstd, int64_t M, int64_t N,
                        rmsnorm_dtype_t dtype, uint32_t flags, void* dx,
                        void* dgamma, hipStream_t stream);

/* Static text for a status code (never NULL). */
const char* rmsnorm_status_string(int status);

/* Launch plan, for inspection by tests and benchmarks. */
typedef struct {
  int32_t kernel;          /* RMSNORM_KERNEL_* */
  int32_t vec;             /* elements per vector access */
  int32_t threads_per_row; /* lanes that share one row */
  int32_t block_threads;   /* threads per workgroup */
  int32_t chunks;          /* vector accesses per thread per row */
  int32_t x_in_lds;        /* 1 when the row of x is staged in LDS */
  int32_t weight_in_regs;  /* 1 when the weight stays in registers across rows */
  int32_t dy_in_lds;       /* 1 when the row of dy is staged in LDS */
  int64_t grid;            /* workgroups launched */
  int64_t partials;        /* P: rows of the dgamma partial-sum workspace */
  int64_t lds_bytes;       /* dynamic LDS per workgroup */
  int32_t segments;        /* split-row plan: workgroups sharing one row */
  int32_t reserved;
} rmsnorm_plan_t;

/* Kernels.  The *_ROWS kernels use 16-byte accesses with the row geometry
 * fixed at compile time and are used whenever N*sizeof(T) and every pointer
 * are 16-byte aligned; the others take any alignment. */
#define RMSNORM_KERNEL_FWD_WAVE 1  /* forward, one wavefront per row */
#define RMSNORM_KERNEL_FWD_BLOCK 2 /* forward, one workgroup per row */
#define RMSNORM_KERNEL_BWD_WAVE 3  /* backward stage 1, one wavefront per row */
#define RMSNORM_KERNEL_BWD_BLOCK 4 /* backward stage 1, one workgroup per row */
#define RMSNORM_KERNEL_BWD_REDUCE 5
#define RMSNORM_KERNEL_FWD_ROWS 6  /* forward, full-width rows */
#define RMSNORM_KERNEL_BWD_ROWS 7  /* backward stage 1, full-width rows */
#define RMSNORM_KERNEL_BWD_REDUCE16 8 /* backward stage 2, 16-column tiles */
/* Software-pipelined full-width kernels: each workgroup loops over rows
 * interleaved with the other workgroups (row groups w, w+P, ...) and
 * prefetches the next row while it computes the current one. */
#define RMSNORM_KERNEL_FWD_PIPE 9  /* forward */
#define RMSNORM_KERNEL_BWD_PIPE 10 /* backward stage 1 */
/* Backward stage 1 for rows of 16-128 KiB: one 512-thread workgroup per
 * row, x staged in LDS and dy in registers for the whole row, the next
 * row's chunks loaded behind the current row's dx stores. */
#define RMSNORM_KERNEL_BWD_LONG 11
/* Split-row plan for N > 65536: each row is cut into `segments` segments of
 * 16 KiB, one 256-thread workgroup per (row block, segment).  A stats kernel
 * writes each segment's partial row sum, a finish kernel adds them per row
 * (float64, segment order) and an apply kernel writes the row outputs.  The
 * forward keeps the segment sums in the first bytes of each row of y
 * between its kernels; the backward keeps them in the workspace. */
#define RMSNORM_KERNEL_FWD_SPLIT 12 /* forward, three kernels */
#define RMSNORM_KERNEL_BWD_SPLIT 13 /* backward stage 1, three kernels */
/* Backward stage 2 for rows of more than 8192 elements (N % 4 == 0): 256
 * columns per workgroup with 16-byte loads, up to 16 slices of partial rows. */
#define RMSNORM_KERNEL_BWD_REDUCE_WIDE 14

#define RMSNORM_PASS_FWD 0
#define RMSNORM_PASS_BWD_ROWS 1
#define RMSNORM_PASS_BWD_REDUCE 2

/*
 * Fills *plan with the launch the given pass would use for (M, N, dtype,
 * flags) when every pointer is `align_bytes`-aligned (16 for typical
 * allocations).  Returns a status code; no device work.
 */
int rmsnorm_query_plan(int64_t M, int64_t N, rmsnorm_dtype_t dtype,
                       uint32_t flags, int pass, int align_bytes,
                       rmsnorm_plan_t* plan);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_H */
