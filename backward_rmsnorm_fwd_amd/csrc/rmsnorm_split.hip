// Split-row plan: rows longer than one workgroup keeps on chip (N > 65536).
//
// The operation is unchanged (page "Check an AI model calculation before
// accelerating it", sections "Problem and reference formula" and "Input
// backward pass: keep the right N"); only the row reduction is cut in two
// passes.  Row i is cut into `nseg` segments of 16 KiB (256 threads x 64
// bytes; the last segment may be shorter).  Workgroup
// w = p*nseg + s owns segment s of the rows of block p, [p*M/P, (p+1)*M/P),
// so the weight slice of a segment is read once per workgroup and the
// workgroup's dgamma partial covers fixed rows and columns.
//
// Forward:  stats   per (row, segment) float32 sum of x^2, parked in the
//                   leading bytes of the row's own y (y is written in full
//                   later, so it serves as the scratch between the passes)
//           finish  per row: the segment sums added in float64 in segment
//                   order, r = 1/sqrt(ss/N + eps) -> rstd
//           apply   y = (x*r)*g
// Backward: stats   per (row, segment) float32 sum of dy*g*x -> workspace;
//                   per-workgroup column sums of dy*x*r -> part[p, columns]
//           finish  per row: c = (segment sums in float64, segment order)/N,
//                   coefficient r^3*c -> workspace
//           apply   dx = r*u - x*(r^3*c)
// then the usual stage 2 adds part[P, N] by column.
//
// The stats passes read with ordinary loads so the apply passes may find
// the lines again in the caches; the apply passes stream (nontemporal).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "split_common.hpp"

namespace rmsnorm_hip {
namespace {

using namespace split;

// Segment s of a row of y holds its float32 partial sum between the passes:
// element s (float32 rows) or the two 16-bit elements 2s, 2s+1.
template <int DT>
__device__ __forceinline__ void put_slot(void* y, int64_t row_elem, int s, float v) {
  if constexpr (DT == kF32) {
    static_cast<float*>(y)[row_elem + s] = v;
  } else {
    const u32 b = __builtin_bit_cast(u32, v);
    u16* p = static_cast<u16*>(y) + row_elem + 2 * s;
    p[0] = static_cast<u16>(b & 0xffffu);
    p[1] = static_cast<u16>(b >> 16);
  }
}

template <int DT>
__device__ __forceinline__ float get_slot(const void* y, int64_t row_elem, int s) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(y)[row_elem + s];
  } else {
    const u16* p = static_cast<const u16*>(y) + row_elem + 2 * s;
    return __builtin_bit_cast(float, static_cast<u32>(p[0]) | (static_cast<u32>(p[1]) << 16));
  }
}

// ---- forward ---------------------------------------------------------------

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_fwd_stats_kernel(
    const void* __restrict__ x, void* __restrict__ y, int64_t M, int N, int nseg, int64_t P,
    int64_t ldx, int64_t ldy) {
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  __shared__ float slots[2][kSplitWaves][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  int parity = 0;
  // Two rows per step: both rows' loads are in flight before either sum.
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const char* xa = row_ptr<DT>(x, row, ldx);
    const char* xb = row_ptr<DT>(x, row + 1, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DT, VEC, false>(a[c], xa, e);
        if (two) load_at<DT, VEC, false>(b[c], xb, e);
      }
    }
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float fa = a[c].get(k), fb = b[c].get(k);
        sa = fmaf(fa, fa, sa);
        sb = fmaf(fb, fb, sb);
      }
    }
    block_sum2(sa, sb, slots, parity, wave, lane);
    if (threadIdx.x == 0) {
      put_slot<DT>(y, row * ldy, ix.s, sa);
      if (two) put_slot<DT>(y, (row + 1) * ldy, ix.s, sb);
    }
  }
}

template <int DT>
__global__ __launch_bounds__(256) void split_fwd_finish_kernel(
    const void* __restrict__ y, float* __restrict__ rstd, int64_t m0, int64_t m1, int N,
    int nseg, int64_t ldy, float eps) {
  const int64_t row = m0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= m1) return;
  double ss = 0.0;
  for (int s = 0; s < nseg; ++s) ss += static_cast<double>(get_slot<DT>(y, row * ldy, s));
  const float ssf = static_cast<float>(ss);
  rstd[row] = 1.0f / sqrtf(ssf / static_cast<float>(N) + eps);
}

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_fwd_apply_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ y, int64_t M, int N, int nseg, int64_t P, int offset,
    int64_t ldx, int64_t ldy) {
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  PK g[CH];
  load_weight<DT, VEC, CH>(g, gamma, ix.e0, N);
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const char* xa = row_ptr<DT>(x, row, ldx);
    const char* xb = row_ptr<DT>(x, row + 1, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DT, VEC, true>(a[c], xa, e);
        if (two) load_at<DT, VEC, true>(b[c], xb, e);
      }
    }
    const float ra = rstd[row];
    const float rb = two ? rstd[row + 1] : 0.f;
    const char* ya = row_ptr<DT>(y, row, ldy);
    const char* yb = row_ptr<DT>(y, row + 1, ldy);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = (a[c].get(k) * ra) * weight_of(g[c].get(k), offset);
        PK out;
        out.set(o);
        store_at<DT, VEC>(out, ya, e);
        if (two) {
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = (b[c].get(k) * rb) * weight_of(g[c].get(k), offset);
          out.set(o);
          store_at<DT, VEC>(out, yb, e);
        }
      }
    }
  }
}

// ---- backward --------------------------------------------------------------

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_bwd_stats_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ rstd, float* __restrict__ part, float* __restrict__ dotp,
    int64_t M, int N, int nseg, int64_t P, int offset, int64_t lddy, int64_t ldx) {
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  __shared__ float slots[2][kSplitWaves][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  int parity = 0;
  PK g[CH];
  load_weight<DT, VEC, CH>(g, gamma, ix.e0, N);
  float acc[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
  // One row per step (the column sums already hold CH*VEC registers); rows
  // in order, so each column sum adds its rows in row order.
  for (int64_t row = ix.r0; row < ix.r1; ++row) {
    const char* dyr = row_ptr<DT>(dy, row, lddy);
    const char* xr = row_ptr<DT>(x, row, ldx);
    PK dv[CH], xv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      dv[c].zero();
      xv[c].zero();
      if (e < N) {
        load_at<DT, VEC, false>(dv[c], dyr, e);
        load_at<DT, VEC, false>(xv[c], xr, e);
      }
    }
    const float r = rstd[row];
    float d = 0.f, unused = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float xf = xv[c].get(k), dyf = dv[c].get(k);
        d = fmaf(dyf * weight_of(g[c].get(k), offset), xf, d);
        acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
      }
    }
    block_sum2(d, unused, slots, parity, wave, lane);
    if (threadIdx.x == 0) dotp[row * nseg + ix.s] = d;
  }
  float* dst = part + static_cast<int64_t>(blockIdx.x / nseg) * N;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = chunk_elem<VEC>(ix.e0, c);
    if (e < N) store_f32<VEC>(dst + e, acc[c]);
  }
}

__global__ __launch_bounds__(256) void split_bwd_finish_kernel(
    const float* __restrict__ dotp, const float* __restrict__ rstd, float* __restrict__ coef,
    int64_t m0, int64_t m1, int N, int nseg) {
  const int64_t row = m0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= m1) return;
  double d = 0.0;
  for (int s = 0; s < nseg; ++s) d += static_cast<double>(dotp[row * nseg + s]);
  const float dot = static_cast<float>(d);
  const float r = rstd[row];
  coef[row] = ((r * r) * r) * (dot / static_cast<float>(N));
}

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_bwd_apply_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ rstd, const float* __restrict__ coef, void* __restrict__ dx,
    int64_t M, int N, int nseg, int64_t P, int offset, int64_t lddy, int64_t ldx,
    int64_t lddx) {
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  PK g[CH];
  load_weight<DT, VEC, CH>(g, gamma, ix.e0, N);
  for (int64_t row = ix.r0; row < ix.r1; ++row) {
    const char* dyr = row_ptr<DT>(dy, row, lddy);
    const char* xr = row_ptr<DT>(x, row, ldx);
    PK dv[CH], xv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      dv[c].zero();
      xv[c].zero();
      if (e < N) {
        load_at<DT, VEC, true>(dv[c], dyr, e);
        load_at<DT, VEC, true>(xv[c], xr, e);
      }
    }
    const float r = rstd[row], k3 = coef[row];
    const char* dxr = row_ptr<DT>(dx, row, lddx);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          o[k] = fmaf(-xv[c].get(k), k3, r * (dv[c].get(k) * weight_of(g[c].get(k), offset)));
        PK out;
        out.set(o);
        store_at<DT, VEC>(out, dxr, e);
      }
    }
  }
}

// ---- host side ---------------------------------------------------------------

// All row blocks in one launch per kernel.  Launching them in batches small
// enough for the 256 MB memory-side cache to keep a batch between its stats
// and apply kernels measured slower at every batch size tried (32-128 MiB):
// the apply kernels do not run faster and every batch adds three launches.
template <int DT, int VEC>
hipError_t split_fwd_vec(const SplitPlan& sp, const FastFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  const int64_t ldx = a.x_pitch / es, ldy = a.y_pitch / es;
  const int64_t grid = sp.P * sp.nseg;
  hipError_t e = launch(split_fwd_stats_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.x, a.y, a.M,
                        a.N, sp.nseg, sp.P, ldx, ldy);
  if (e != hipSuccess) return e;
  e = launch(split_fwd_finish_kernel<DT>, (a.M + 255) / 256, 256, 0, s, a.y, a.rstd, int64_t(0),
             a.M, a.N, sp.nseg, ldy, a.eps);
  if (e != hipSuccess) return e;
  return launch(split_fwd_apply_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.x, a.gamma, a.rstd,
                a.y, a.M, a.N, sp.nseg, sp.P, a.offset, ldx, ldy);
}

template <int DT, int VEC>
hipError_t split_bwd_vec(const SplitPlan& sp, const FastBwdArgs& a, float* dotp, float* coef,
                         hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  const int64_t lddy = a.dy_pitch / es, ldx = a.x_pitch / es, lddx = a.dx_pitch / es;
  const int64_t grid = sp.P * sp.nseg;
  hipError_t e = launch(split_bwd_stats_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.dy, a.x,
                        a.gamma, a.rstd, a.part, dotp, a.M, a.N, sp.nseg, sp.P, a.offset, lddy,
                        ldx);
  if (e != hipSuccess) return e;
  e = launch(split_bwd_finish_kernel, (a.M + 255) / 256, 256, 0, s, dotp, a.rstd, coef,
             int64_t(0), a.M, a.N, sp.nseg);
  if (e != hipSuccess) return e;
  return launch(split_bwd_apply_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.dy, a.x, a.gamma,
                a.rstd, coef, a.dx, a.M, a.N, sp.nseg, sp.P, a.offset, lddy, ldx, lddx);
}

template <int DT>
hipError_t split_fwd_dt(const SplitPlan& sp, const FastFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (sp.vec * es) {
    case 16: return split_fwd_vec<DT, 16 / es>(sp, a, s);
    case 8: return split_fwd_vec<DT, 8 / es>(sp, a, s);
    case 4: return split_fwd_vec<DT, 4 / es>(sp, a, s);
    case 2:
      if constexpr (es == 2) return split_fwd_vec<DT, 1>(sp, a, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t split_bwd_dt(const SplitPlan& sp, const FastBwdArgs& a, float* dotp, float* coef,
                        hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (sp.vec * es) {
    case 16: return split_bwd_vec<DT, 16 / es>(sp, a, dotp, coef, s);
    case 8: return split_bwd_vec<DT, 8 / es>(sp, a, dotp, coef, s);
    case 4: return split_bwd_vec<DT, 4 / es>(sp, a, dotp, coef, s);
    case 2:
      if constexpr (es == 2) return split_bwd_vec<DT, 1>(sp, a, dotp, coef, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

int split_segment_elems(int elem_bytes) { return kSplitBlock * kBytesPerThread / elem_bytes; }

int split_chunks(int vec, int elem_bytes) { return kBytesPerThread / (vec * elem_bytes); }

hipError_t split_fwd_launch(int dtype, const SplitPlan& sp, const FastFwdArgs& a,
                            hipStream_t s) {
  switch (dtype) {
    case kF32: return split_fwd_dt<kF32>(sp, a, s);
    case kF16: return split_fwd_dt<kF16>(sp, a, s);
    case kBF16: return split_fwd_dt<kBF16>(sp, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t split_bwd_launch(int dtype, const SplitPlan& sp, const FastBwdArgs& a, float* dotp,
                            float* coef, hipStream_t s) {
  switch (dtype) {
    case kF32: return split_bwd_dt<kF32>(sp, a, dotp, coef, s);
    case kF16: return split_bwd_dt<kF16>(sp, a, dotp, coef, s);
    case kBF16: return split_bwd_dt<kBF16>(sp, a, dotp, coef, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
