// Split-row plan: rows longer than one workgroup keeps on chip (RMSNorm
// rows over 65536 elements; rows over 16384 for the fused residual add and
// the fused output cast, whose row-resident kernels stop there).
//
// The operation is unchanged (page "Check an AI model calculation before
// accelerating it", sections "Problem and reference formula" and "Input
// backward pass: keep the right N"; the fused neighbours as in fused_add.hip
// and fused_cast.hip); only the row reduction is cut in two passes.  Row i
// is cut into `nseg` segments of 16 KiB of x (256 threads x 64 bytes; the
// last segment may be shorter).  Workgroup w = p*nseg + s owns segment s of
// the rows of block p, [p*M/P, (p+1)*M/P), so the weight slice of a segment
// is read once per workgroup and the workgroup's dgamma partial covers fixed
// rows and columns.
//
// Two dtypes: DX for x, gamma, dx (and the fused add's res, h and dh), DY for
// y and dy.  They differ only for the fused cast (float32 x, 16-bit y, dy).
//
// Forward:  stats   per (row, segment) float32 sum of x^2, parked in the
//                   leading bytes of the row's own y (y is written in full
//                   later, so it serves as the scratch between the passes);
//                   the fused add first forms h = DX(x + res), writes it and
//                   sums h^2
//           finish  per row: the segment sums added in float64 in segment
//                   order, r = 1/sqrt(ss/N + eps) -> rstd
//           apply   y = DY((x*r)*g), from h for the fused add
// Backward: stats   per (row, segment) float32 sum of dy*g*x -> workspace;
//                   per-workgroup column sums of dy*x*r -> part[p, columns]
//           finish  per row: c = (segment sums in float64, segment order)/N,
//                   coefficient r^3*c -> workspace
//           apply   dx = r*u - x*(r^3*c) (+ dh for the fused add, whose x
//                   is h)
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

template <int DX, int DY, int VEC, bool ADD>
__global__ __launch_bounds__(kSplitBlock) void split_fwd_stats_kernel(
    const void* __restrict__ x, const void* __restrict__ res, void* __restrict__ h,
    void* __restrict__ y, int64_t M, int N, int nseg, int64_t P, int64_t ldx, int64_t ldr,
    int64_t ldh, int64_t ldy) {
  using PK = Pack<DX, VEC>;
  constexpr int CH = SplitGeom<DX, VEC>::kCh;
  __shared__ float slots[2][kSplitWaves][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DX, VEC>(M, nseg, P);
  int parity = 0;
  // Two rows per step: both rows' loads are in flight before either sum.
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const char* xa = row_ptr<DX>(x, row, ldx);
    const char* xb = row_ptr<DX>(x, row + 1, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DX, VEC, false>(a[c], xa, e);
        if (two) load_at<DX, VEC, false>(b[c], xb, e);
      }
    }
    if constexpr (ADD) {
      // h = DX(x + res): the float32 sum of the widened operands, rounded
      // once on packing; the sums below use the rounded h.
      const char* rsa = row_ptr<DX>(res, row, ldr);
      const char* rsb = row_ptr<DX>(res, row + 1, ldr);
      PK qa[CH], qb[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int e = chunk_elem<VEC>(ix.e0, c);
        qa[c].zero();
        qb[c].zero();
        if (e < N) {
          load_at<DX, VEC, false>(qa[c], rsa, e);
          if (two) load_at<DX, VEC, false>(qb[c], rsb, e);
        }
      }
      const char* ha = row_ptr<DX>(h, row, ldh);
      const char* hb = row_ptr<DX>(h, row + 1, ldh);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        float fa[VEC], fb[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          fa[k] = a[c].get(k) + qa[c].get(k);
          fb[k] = b[c].get(k) + qb[c].get(k);
        }
        a[c].set(fa);
        b[c].set(fb);
        const int e = chunk_elem<VEC>(ix.e0, c);
        if (e < N) {
          store_at<DX, VEC>(a[c], ha, e);
          if (two) store_at<DX, VEC>(b[c], hb, e);
        }
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
      put_slot<DY>(y, row * ldy, ix.s, sa);
      if (two) put_slot<DY>(y, (row + 1) * ldy, ix.s, sb);
    }
  }
}

template <int DY>
__global__ __launch_bounds__(256) void split_fwd_finish_kernel(
    const void* __restrict__ y, float* __restrict__ rstd, int64_t m0, int64_t m1, int N,
    int nseg, int64_t ldy, float eps) {
  const int64_t row = m0 + static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= m1) return;
  double ss = 0.0;
  for (int s = 0; s < nseg; ++s) ss += static_cast<double>(get_slot<DY>(y, row * ldy, s));
  const float ssf = static_cast<float>(ss);
  rstd[row] = 1.0f / sqrtf(ssf / static_cast<float>(N) + eps);
}

template <int DX, int DY, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_fwd_apply_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ y, int64_t M, int N, int nseg, int64_t P, int offset,
    int64_t ldx, int64_t ldy) {
  using PK = Pack<DX, VEC>;
  using PO = Pack<DY, VEC>;
  constexpr int CH = SplitGeom<DX, VEC>::kCh;
  const SegIndex ix = seg_index<DX, VEC>(M, nseg, P);
  PK g[CH];
  load_weight<DX, VEC, CH>(g, gamma, ix.e0, N);
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const char* xa = row_ptr<DX>(x, row, ldx);
    const char* xb = row_ptr<DX>(x, row + 1, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DX, VEC, true>(a[c], xa, e);
        if (two) load_at<DX, VEC, true>(b[c], xb, e);
      }
    }
    const float ra = rstd[row];
    const float rb = two ? rstd[row + 1] : 0.f;
    const char* ya = row_ptr<DY>(y, row, ldy);
    const char* yb = row_ptr<DY>(y, row + 1, ldy);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = (a[c].get(k) * ra) * weight_of(g[c].get(k), offset);
        PO out;
        out.set(o);
        store_at<DY, VEC>(out, ya, e);
        if (two) {
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = (b[c].get(k) * rb) * weight_of(g[c].get(k), offset);
          out.set(o);
          store_at<DY, VEC>(out, yb, e);
        }
      }
    }
  }
}

// ---- backward --------------------------------------------------------------

template <int DX, int DY, int VEC>
__global__ __launch_bounds__(kSplitBlock) void split_bwd_stats_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ rstd, float* __restrict__ part, float* __restrict__ dotp,
    int64_t M, int N, int nseg, int64_t P, int offset, int64_t lddy, int64_t ldx) {
  using PK = Pack<DX, VEC>;
  using PD = Pack<DY, VEC>;
  constexpr int CH = SplitGeom<DX, VEC>::kCh;
  __shared__ float slots[2][kSplitWaves][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DX, VEC>(M, nseg, P);
  int parity = 0;
  PK g[CH];
  load_weight<DX, VEC, CH>(g, gamma, ix.e0, N);
  float acc[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
  // One row per step (the column sums already hold CH*VEC registers); rows
  // in order, so each column sum adds its rows in row order.
  for (int64_t row = ix.r0; row < ix.r1; ++row) {
    const char* dyr = row_ptr<DY>(dy, row, lddy);
    const char* xr = row_ptr<DX>(x, row, ldx);
    PD dv[CH];
    PK xv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      dv[c].zero();
      xv[c].zero();
      if (e < N) {
        load_at<DY, VEC, false>(dv[c], dyr, e);
        load_at<DX, VEC, false>(xv[c], xr, e);
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

template <int DX, int DY, int VEC, bool DH>
__global__ __launch_bounds__(kSplitBlock) void split_bwd_apply_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ rstd, const float* __restrict__ coef, const void* __restrict__ dh,
    void* __restrict__ dx, int64_t M, int N, int nseg, int64_t P, int offset, int64_t lddy,
    int64_t ldx, int64_t lddh, int64_t lddx) {
  using PK = Pack<DX, VEC>;
  using PD = Pack<DY, VEC>;
  constexpr int CH = SplitGeom<DX, VEC>::kCh;
  const SegIndex ix = seg_index<DX, VEC>(M, nseg, P);
  PK g[CH];
  load_weight<DX, VEC, CH>(g, gamma, ix.e0, N);
  for (int64_t row = ix.r0; row < ix.r1; ++row) {
    const char* dyr = row_ptr<DY>(dy, row, lddy);
    const char* xr = row_ptr<DX>(x, row, ldx);
    PD dv[CH];
    PK xv[CH], ev[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      dv[c].zero();
      xv[c].zero();
      ev[c].zero();
      if (e < N) {
        load_at<DY, VEC, true>(dv[c], dyr, e);
        load_at<DX, VEC, true>(xv[c], xr, e);
        if constexpr (DH) load_at<DX, VEC, true>(ev[c], row_ptr<DX>(dh, row, lddh), e);
      }
    }
    const float r = rstd[row], k3 = coef[row];
    const char* dxr = row_ptr<DX>(dx, row, lddx);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          o[k] = fmaf(-xv[c].get(k), k3, r * (dv[c].get(k) * weight_of(g[c].get(k), offset)));
          if constexpr (DH) o[k] = o[k] + ev[c].get(k);
        }
        PK out;
        out.set(o);
        store_at<DX, VEC>(out, dxr, e);
      }
    }
  }
}

// ---- host side ---------------------------------------------------------------

// One split call's operands, pitches in elements of their own dtype.
struct SplitFwdIO {
  const void* x;
  const void* res;  // fused add only
  void* h;          // fused add only
  const void* gamma;
  void* y;
  float* rstd;
  int64_t M;
  int N;
  float eps;
  int offset;
  int64_t ldx, ldr, ldh, ldy;
};

struct SplitBwdIO {
  const void* dy;
  const void* x;  // h for the fused add
  const void* gamma;
  const float* rstd;
  const void* dh;  // fused add, may be null
  void* dx;
  float* part;
  int64_t M;
  int N;
  int offset;
  int64_t lddy, ldx, lddh, lddx;
};

// All row blocks in one launch per kernel.  Launching them in batches small
// enough for the 256 MB memory-side cache to keep a batch between its stats
// and apply kernels measured slower at every batch size tried (32-128 MiB):
// the apply kernels do not run faster and every batch adds three launches.
template <int DX, int DY, int VEC, bool ADD>
hipError_t split_fwd_vec(const SplitPlan& sp, const SplitFwdIO& a, hipStream_t s) {
  const int64_t grid = sp.P * sp.nseg;
  hipError_t e = launch(split_fwd_stats_kernel<DX, DY, VEC, ADD>, grid, kSplitBlock, 0, s, a.x,
                        a.res, a.h, a.y, a.M, a.N, sp.nseg, sp.P, a.ldx, a.ldr, a.ldh, a.ldy);
  if (e != hipSuccess) return e;
  e = launch(split_fwd_finish_kernel<DY>, (a.M + 255) / 256, 256, 0, s, a.y, a.rstd, int64_t(0),
             a.M, a.N, sp.nseg, a.ldy, a.eps);
  if (e != hipSuccess) return e;
  return launch(split_fwd_apply_kernel<DX, DY, VEC>, grid, kSplitBlock, 0, s,
                ADD ? static_cast<const void*>(a.h) : a.x, a.gamma, a.rstd, a.y, a.M, a.N,
                sp.nseg, sp.P, a.offset, ADD ? a.ldh : a.ldx, a.ldy);
}

template <int DX, int DY, int VEC, bool DH>
hipError_t split_bwd_vec(const SplitPlan& sp, const SplitBwdIO& a, float* dotp, float* coef,
                         hipStream_t s) {
  const int64_t grid = sp.P * sp.nseg;
  hipError_t e = launch(split_bwd_stats_kernel<DX, DY, VEC>, grid, kSplitBlock, 0, s, a.dy, a.x,
                        a.gamma, a.rstd, a.part, dotp, a.M, a.N, sp.nseg, sp.P, a.offset, a.lddy,
                        a.ldx);
  if (e != hipSuccess) return e;
  e = launch(split_bwd_finish_kernel, (a.M + 255) / 256, 256, 0, s, dotp, a.rstd, coef,
             int64_t(0), a.M, a.N, sp.nseg);
  if (e != hipSuccess) return e;
  // The apply pass keeps no column sums, so it may cut the rows finer.
  const int64_t Pa = sp.P_free > 0 ? sp.P_free : sp.P;
  return launch(split_bwd_apply_kernel<DX, DY, VEC, DH>, Pa * sp.nseg, kSplitBlock, 0, s, a.dy,
                a.x, a.gamma, a.rstd, coef, a.dh, a.dx, a.M, a.N, sp.nseg, Pa, a.offset, a.lddy,
                a.ldx, a.lddh, a.lddx);
}

// The access width sp.vec (elements of DX) picks the instantiation.
template <int DX, int DY, bool ADD>
hipError_t split_fwd_dt(const SplitPlan& sp, const SplitFwdIO& a, hipStream_t s) {
  constexpr int es = ElemBytes<DX>::value;
  switch (sp.vec * es) {
    case 16: return split_fwd_vec<DX, DY, 16 / es, ADD>(sp, a, s);
    case 8: return split_fwd_vec<DX, DY, 8 / es, ADD>(sp, a, s);
    case 4: return split_fwd_vec<DX, DY, 4 / es, ADD>(sp, a, s);
    case 2:
      if constexpr (es == 2) return split_fwd_vec<DX, DY, 1, ADD>(sp, a, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DX, int DY, bool DH>
hipError_t split_bwd_dt(const SplitPlan& sp, const SplitBwdIO& a, float* dotp, float* coef,
                        hipStream_t s) {
  constexpr int es = ElemBytes<DX>::value;
  switch (sp.vec * es) {
    case 16: return split_bwd_vec<DX, DY, 16 / es, DH>(sp, a, dotp, coef, s);
    case 8: return split_bwd_vec<DX, DY, 8 / es, DH>(sp, a, dotp, coef, s);
    case 4: return split_bwd_vec<DX, DY, 4 / es, DH>(sp, a, dotp, coef, s);
    case 2:
      if constexpr (es == 2) return split_bwd_vec<DX, DY, 1, DH>(sp, a, dotp, coef, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

// One dtype for x and y (RMSNorm and the fused add).
template <bool ADD>
hipError_t split_fwd_same(int dtype, const SplitPlan& sp, const SplitFwdIO& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return split_fwd_dt<kF32, kF32, ADD>(sp, a, s);
    case kF16: return split_fwd_dt<kF16, kF16, ADD>(sp, a, s);
    case kBF16: return split_fwd_dt<kBF16, kBF16, ADD>(sp, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool DH>
hipError_t split_bwd_same(int dtype, const SplitPlan& sp, const SplitBwdIO& a, float* dotp,
                          float* coef, hipStream_t s) {
  switch (dtype) {
    case kF32: return split_bwd_dt<kF32, kF32, DH>(sp, a, dotp, coef, s);
    case kF16: return split_bwd_dt<kF16, kF16, DH>(sp, a, dotp, coef, s);
    case kBF16: return split_bwd_dt<kBF16, kBF16, DH>(sp, a, dotp, coef, s);
    default: return hipErrorInvalidValue;
  }
}

int elem_size(int dtype) { return dtype == kF32 ? 4 : 2; }

int64_t elems(int64_t pitch_bytes, int es) { return pitch_bytes / es; }

}  // namespace

int split_segment_elems(int elem_bytes) { return kSplitBlock * kBytesPerThread / elem_bytes; }

int split_chunks(int vec, int elem_bytes) { return kBytesPerThread / (vec * elem_bytes); }

hipError_t split_fwd_launch(int dtype, const SplitPlan& sp, const FastFwdArgs& a,
                            hipStream_t s) {
  const int es = elem_size(dtype);
  const SplitFwdIO io{a.x, nullptr, nullptr, a.gamma, a.y, a.rstd, a.M, a.N, a.eps, a.offset,
                      elems(a.x_pitch, es), 0, 0, elems(a.y_pitch, es)};
  return split_fwd_same<false>(dtype, sp, io, s);
}

hipError_t split_bwd_launch(int dtype, const SplitPlan& sp, const FastBwdArgs& a, float* dotp,
                            float* coef, hipStream_t s) {
  const int es = elem_size(dtype);
  const SplitBwdIO io{a.dy, a.x, a.gamma, a.rstd, nullptr, a.dx, a.part, a.M, a.N, a.offset,
                      elems(a.dy_pitch, es), elems(a.x_pitch, es), 0, elems(a.dx_pitch, es)};
  return split_bwd_same<false>(dtype, sp, io, dotp, coef, s);
}

hipError_t add_split_fwd_launch(int dtype, const SplitPlan& sp, const AddFwdArgs& a,
                                hipStream_t s) {
  const int es = elem_size(dtype);
  const SplitFwdIO io{a.x, a.res, a.h, a.gamma, a.y, a.rstd, a.M, a.N, a.eps, a.offset,
                      elems(a.x_pitch, es), elems(a.res_pitch, es), elems(a.h_pitch, es),
                      elems(a.y_pitch, es)};
  return split_fwd_same<true>(dtype, sp, io, s);
}

hipError_t add_split_bwd_launch(int dtype, const SplitPlan& sp, const AddBwdArgs& a,
                                float* dotp, float* coef, hipStream_t s) {
  const int es = elem_size(dtype);
  const SplitBwdIO io{a.dy, a.h, a.gamma, a.rstd, a.dh, a.dx, a.part, a.M, a.N, a.offset,
                      elems(a.dy_pitch, es), elems(a.h_pitch, es),
                      a.dh ? elems(a.dh_pitch, es) : 0, elems(a.dx_pitch, es)};
  return a.dh ? split_bwd_same<true>(dtype, sp, io, dotp, coef, s)
              : split_bwd_same<false>(dtype, sp, io, dotp, coef, s);
}

hipError_t cast_split_fwd_launch(int out_dtype, const SplitPlan& sp, const CastFwdArgs& a,
                                 hipStream_t s) {
  const SplitFwdIO io{a.x, nullptr, nullptr, a.gamma, a.y, a.rstd, a.M, a.N, a.eps, a.offset,
                      elems(a.x_pitch, 4), 0, 0, elems(a.y_pitch, elem_size(out_dtype))};
  switch (out_dtype) {
    case kF16: return split_fwd_dt<kF32, kF16, false>(sp, io, s);
    case kBF16: return split_fwd_dt<kF32, kBF16, false>(sp, io, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t cast_split_bwd_launch(int out_dtype, const SplitPlan& sp, const CastBwdArgs& a,
                                 float* dotp, float* coef, hipStream_t s) {
  const SplitBwdIO io{a.dy, a.x, a.gamma, a.rstd, nullptr, a.dx, a.part, a.M, a.N, a.offset,
                      elems(a.dy_pitch, elem_size(out_dtype)), elems(a.x_pitch, 4), 0,
                      elems(a.dx_pitch, 4)};
  switch (out_dtype) {
    case kF16: return split_bwd_dt<kF32, kF16, false>(sp, io, dotp, coef, s);
    case kBF16: return split_bwd_dt<kF32, kBF16, false>(sp, io, dotp, coef, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
