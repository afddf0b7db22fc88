// LayerNorm, split-row plan: rows longer than the row-resident kernels hold
// on chip (N > 16384 elements).
//
// The operation is unchanged (the page "PyTorch torch.compile ... LayerNorm
// and RMSNorm", sections 1.1 and 2: each row normalised by its own mean and
// variance, then scaled by gamma and shifted by beta; the backward yields
// dx, dgamma and dbeta); only the row reductions are cut into passes.  Rows
// are cut into 16 KiB segments and workgroup p*nseg + s owns segment s of
// the rows of block p (split_common.hpp).
//
// Forward:  stats   per (row, segment): S = sum(x) and M2 = sum((x - S/n)^2)
//                   over the segment's n elements, in float64 (the widened
//                   elements are exact there), parked as two doubles at
//                   byte 16*s of the row's own y (written in full later, so
//                   it serves as the scratch between passes)
//           finish  per row, segments in order, float64: mu = sum(S)/N and
//                   the squared deviations about the running mean merged
//                   segment by segment; r = 1/sqrt(M2/N + eps) -> mean (mu
//                   rounded to float32), rstd; the remainder c = mu - mean
//                   -> the row's first 4 bytes of y
//           apply   y = ((x - mean)*r - c*r)*gamma + beta, all but the
//                   leading elements that hold c
//           head    the same for those elements, one thread per row
// Backward: stats   per (row, segment), with d = x - mean and u = dy*gamma:
//                   sum(u), sum(u*d) and sum(d) in float32 -> workspace
//           finish  per row, segments in order, float64: c = sum(d)/N
//                   (what the stored float32 mean is off by), c1 = sum(u)/N,
//                   c2 = r*(sum(u*d) - c*sum(u))/N -> workspace
//           apply   xhat = (d - c)*r, dx = r*((u - c1) - xhat*c2), and the
//                   workgroup's column sums of dy*xhat and dy over its rows
//                   (row order) -> part[p, columns] and part[P + p, columns]
// then the LayerNorm stage 2 adds both [P, N] blocks by column.  These are
// the row-resident kernels' formulas (layernorm.hip) with the row sums taken
// in pieces; the forward's variance is taken in float64 throughout.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"
#include "split_common.hpp"

namespace rmsnorm_hip {
namespace {

using namespace split;

// Sums of K values over the workgroup, added in wavefront order, returned to
// every thread.  One barrier per call; `parity` alternates the slot set, so
// a set is only rewritten after every thread has passed a later barrier.
template <int K>
__device__ __forceinline__ void block_sum_all(double (&v)[K], double (*slots)[kSplitWaves][K],
                                              int& parity, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = rowres::wave_sum_f64(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) slots[parity][wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) t += slots[parity][w][k];
    v[k] = t;
  }
  parity ^= 1;
}

template <int K>
__device__ __forceinline__ void block_sum_all(float (&v)[K], float (*slots)[kSplitWaves][K],
                                              int& parity, int wave, int lane) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) slots[parity][wave][k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) t += slots[parity][w][k];
    v[k] = t;
  }
  parity ^= 1;
}

// The two doubles of segment s parked at byte 16*s of a row of y.  The row's
// start is only element-aligned, so they are moved in element-sized pieces.
template <int DT>
__device__ __forceinline__ void put_stats(void* yrow, int s, double a, double b) {
  const uint64_t w[2] = {__builtin_bit_cast(uint64_t, a), __builtin_bit_cast(uint64_t, b)};
  char* p = static_cast<char*>(yrow) + 16 * static_cast<int64_t>(s);
  if constexpr (ElemBytes<DT>::value == 4) {
    u32* q = reinterpret_cast<u32*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = static_cast<u32>(w[i / 2] >> (32 * (i % 2)));
  } else {
    u16* q = reinterpret_cast<u16*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = static_cast<u16>(w[i / 4] >> (16 * (i % 4)));
  }
}

template <int DT>
__device__ __forceinline__ void get_stats(const void* yrow, int s, double& a, double& b) {
  uint64_t w[2] = {0, 0};
  const char* p = static_cast<const char*>(yrow) + 16 * static_cast<int64_t>(s);
  if constexpr (ElemBytes<DT>::value == 4) {
    const u32* q = reinterpret_cast<const u32*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i / 2] |= static_cast<uint64_t>(q[i]) << (32 * (i % 2));
  } else {
    const u16* q = reinterpret_cast<const u16*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4] |= static_cast<uint64_t>(q[i]) << (16 * (i % 4));
  }
  a = __builtin_bit_cast(double, w[0]);
  b = __builtin_bit_cast(double, w[1]);
}

// Elements of segment s of a row of N.
template <int DT, int VEC>
__device__ __forceinline__ int seg_count(int s, int N) {
  const int seg = SplitGeom<DT, VEC>::kSeg;
  const int left = N - s * seg;
  return left < seg ? left : seg;
}

// ---- forward ---------------------------------------------------------------

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void ln_split_fwd_stats_kernel(
    const void* __restrict__ x, void* __restrict__ y, int64_t M, int N, int nseg, int64_t P,
    int64_t ldx, int64_t ldy) {
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  __shared__ double slots[2][kSplitWaves][2];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  const double n_s = static_cast<double>(seg_count<DT, VEC>(ix.s, N));
  int parity = 0;
  // Two rows per step: both rows' loads are in flight before either sum.
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const char* xa = row_ptr<DT>(x, row, ldx);
    const char* xb = row_ptr<DT>(x, two ? row + 1 : row, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DT, VEC, false>(a[c], xa, e);
        load_at<DT, VEC, false>(b[c], xb, e);
      }
    }
    double t[2] = {0.0, 0.0};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        t[0] += static_cast<double>(a[c].get(k));
        t[1] += static_cast<double>(b[c].get(k));
      }
    }
    block_sum_all<2>(t, slots, parity, wave, lane);
    const double sa = t[0], sb = t[1];
    const double ma = sa / n_s, mb = sb / n_s;
    double q[2] = {0.0, 0.0};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const double da = static_cast<double>(a[c].get(k)) - ma;
          const double db = static_cast<double>(b[c].get(k)) - mb;
          q[0] = fma(da, da, q[0]);
          q[1] = fma(db, db, q[1]);
        }
      }
    }
    block_sum_all<2>(q, slots, parity, wave, lane);
    if (threadIdx.x == 0) {
      put_stats<DT>(const_cast<char*>(row_ptr<DT>(y, row, ldy)), ix.s, sa, q[0]);
      if (two) put_stats<DT>(const_cast<char*>(row_ptr<DT>(y, row + 1, ldy)), ix.s, sb, q[1]);
    }
  }
}

// The float32 mean is the exact mean rounded; the remainder c = mu - mean
// is taken out of x - mean before scaling, as the row-resident kernel does.
// The finish kernel leaves c in the first 4 bytes of the row of y, which the
// apply kernel reads and does not write; the head kernel writes y there last.
template <int DT>
__device__ __forceinline__ void put_offset(void* yrow, float c) {
  const u32 w = __builtin_bit_cast(u32, c);
  if constexpr (ElemBytes<DT>::value == 4) {
    *static_cast<u32*>(yrow) = w;
  } else {
    u16* q = static_cast<u16*>(yrow);
    q[0] = static_cast<u16>(w & 0xffffu);
    q[1] = static_cast<u16>(w >> 16);
  }
}

template <int DT>
__device__ __forceinline__ float get_offset(const void* yrow) {
  if constexpr (ElemBytes<DT>::value == 4) {
    return __builtin_bit_cast(float, *static_cast<const u32*>(yrow));
  } else {
    const u16* q = static_cast<const u16*>(yrow);
    return __builtin_bit_cast(float, static_cast<u32>(q[0]) | (static_cast<u32>(q[1]) << 16));
  }
}

// Leading elements of a row that hold the offset during the apply pass:
// 4 bytes rounded up to whole accesses of VEC elements.
template <int DT, int VEC>
constexpr int head_elems() {
  constexpr int e = 4 / ElemBytes<DT>::value;
  return VEC > e ? VEC : e;
}

// One thread per row, segments in order.  The mean is the float64 sum of the
// segment sums over N; the squared deviations about it combine the
// segments' own (M2_s) with each segment's mean offset, merged one segment
// at a time (M2 += M2_s + delta^2 * n*n_s/(n + n_s), delta the difference
// of the segment mean and the running mean): one read of the parked values.
template <int DT>
__global__ __launch_bounds__(256) void ln_split_fwd_finish_kernel(
    void* __restrict__ y, float* __restrict__ mean, float* __restrict__ rstd, int64_t M, int N,
    int nseg, int seg, int64_t ldy, float eps) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= M) return;
  char* yrow = const_cast<char*>(row_ptr<DT>(y, row, ldy));
  double total = 0.0, n = 0.0, run_mean = 0.0, m2 = 0.0;
  for (int s = 0; s < nseg; ++s) {
    double S, Q;
    get_stats<DT>(yrow, s, S, Q);
    const int left = N - s * seg;
    const double ns = static_cast<double>(left < seg ? left : seg);
    const double ms = S / ns;
    total += S;
    if (s == 0) {
      run_mean = ms;
      m2 = Q;
    } else {
      const double nn = n + ns;
      const double delta = ms - run_mean;
      run_mean += delta * (ns / nn);
      m2 += Q + delta * delta * (n * ns / nn);
    }
    n += ns;
  }
  const double mu = total / static_cast<double>(N);
  const float mu32 = static_cast<float>(mu);
  const double var = m2 / static_cast<double>(N);
  mean[row] = mu32;
  rstd[row] = static_cast<float>(1.0 / sqrt(var + static_cast<double>(eps)));
  put_offset<DT>(yrow, static_cast<float>(mu - static_cast<double>(mu32)));
}

// y = (x - mean - c)*r*gamma + beta, the scaled deviation as one fma; the
// head kernel repeats the same operations for the leading elements.
__device__ __forceinline__ float ln_out(float x, float mu, float r, float ncr, float g,
                                        float b) {
  return fmaf(fmaf(x - mu, r, ncr), g, b);
}

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void ln_split_fwd_apply_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta,
    const float* __restrict__ mean, const float* __restrict__ rstd, void* __restrict__ y,
    int64_t M, int N, int nseg, int64_t P, int64_t ldx, int64_t ldy) {
#pragma clang fp contract(off)
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  constexpr int kHead = head_elems<DT, VEC>();
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  PK g[CH], bt[CH];
  load_weight<DT, VEC, CH>(g, gamma, ix.e0, N);
  if (beta) {
    load_weight<DT, VEC, CH>(bt, beta, ix.e0, N);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) bt[c].zero();
  }
  // Two rows per step: both rows' loads are in flight before either store.
  for (int64_t row = ix.r0; row < ix.r1; row += 2) {
    const bool two = row + 1 < ix.r1;
    const int64_t rb = two ? row + 1 : row;
    const char* xa = row_ptr<DT>(x, row, ldx);
    const char* xb = row_ptr<DT>(x, rb, ldx);
    PK a[CH], b[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = chunk_elem<VEC>(ix.e0, c);
      a[c].zero();
      b[c].zero();
      if (e < N) {
        load_at<DT, VEC, true>(a[c], xa, e);
        load_at<DT, VEC, true>(b[c], xb, e);
      }
    }
    const char* ya = row_ptr<DT>(y, row, ldy);
    const char* yb = row_ptr<DT>(y, rb, ldy);
    const float mu[2] = {mean[row], mean[rb]};
    const float r[2] = {rstd[row], rstd[rb]};
    const float ncr[2] = {-(get_offset<DT>(ya) * r[0]), -(get_offset<DT>(yb) * r[1])};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      bt[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N && e >= kHead) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          o[k] = ln_out(a[c].get(k), mu[0], r[0], ncr[0], g[c].get(k), bt[c].get(k));
        PK out;
        out.set(o);
        store_at<DT, VEC>(out, ya, e);
        if (two) {
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = ln_out(b[c].get(k), mu[1], r[1], ncr[1], g[c].get(k), bt[c].get(k));
          out.set(o);
          store_at<DT, VEC>(out, yb, e);
        }
      }
    }
  }
}

// The leading elements of each row, after the apply pass: the thread reads
// the row's offset before it overwrites it.
template <int DT, int HEAD>
__global__ __launch_bounds__(256) void ln_split_fwd_head_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta,
    const float* __restrict__ mean, const float* __restrict__ rstd, void* __restrict__ y,
    int64_t M, int64_t ldx, int64_t ldy) {
#pragma clang fp contract(off)
  using PK = Pack<DT, 1>;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= M) return;
  const char* yr = row_ptr<DT>(y, row, ldy);
  const char* xr = row_ptr<DT>(x, row, ldx);
  const float mu = mean[row], r = rstd[row];
  const float ncr = -(get_offset<DT>(yr) * r);
  PK out[HEAD];
#pragma unroll
  for (int e = 0; e < HEAD; ++e) {
    PK xv, gv, bv;
    load_at<DT, 1, false>(xv, xr, e);
    load_at<DT, 1, false>(gv, static_cast<const char*>(gamma), e);
    bv.zero();
    if (beta) load_at<DT, 1, false>(bv, static_cast<const char*>(beta), e);
    const float v[1] = {ln_out(xv.get(0), mu, r, ncr, gv.get(0), bv.get(0))};
    out[e].set(v);
  }
#pragma unroll
  for (int e = 0; e < HEAD; ++e) store_at<DT, 1>(out[e], yr, e);
}

// ---- backward --------------------------------------------------------------

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void ln_split_bwd_stats_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ mean, float* __restrict__ sums, int64_t M, int N, int nseg,
    int64_t P, int64_t lddy, int64_t ldx) {
#pragma clang fp contract(off)
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  __shared__ float slots[2][kSplitWaves][3];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  int parity = 0;
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
        load_at<DT, VEC, false>(dv[c], dyr, e);
        load_at<DT, VEC, false>(xv[c], xr, e);
      }
    }
    const float mu = mean[row];
    float t[3] = {0.f, 0.f, 0.f};  // sum(u), sum(u*d), sum(d)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float d = xv[c].get(k) - mu;
          const float u = dv[c].get(k) * g[c].get(k);
          t[0] += u;
          t[1] = fmaf(u, d, t[1]);
          t[2] += d;
        }
      }
    }
    block_sum_all<3>(t, slots, parity, wave, lane);
    if (threadIdx.x == 0) {
      float* dst = sums + (row * nseg + ix.s) * 3;
      dst[0] = t[0];
      dst[1] = t[1];
      dst[2] = t[2];
    }
  }
}

__global__ __launch_bounds__(256) void ln_split_bwd_finish_kernel(
    const float* __restrict__ sums, const float* __restrict__ rstd, float* __restrict__ coef,
    int64_t M, int N, int nseg) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= M) return;
  double su = 0.0, sud = 0.0, sd = 0.0;
  const float* src = sums + row * nseg * 3;
  for (int s = 0; s < nseg; ++s) {
    su += static_cast<double>(src[3 * s]);
    sud += static_cast<double>(src[3 * s + 1]);
    sd += static_cast<double>(src[3 * s + 2]);
  }
  const double inv_n = 1.0 / static_cast<double>(N);
  const double r = static_cast<double>(rstd[row]);
  const double c = sd * inv_n;
  float* dst = coef + row * 3;
  dst[0] = static_cast<float>(c);
  dst[1] = static_cast<float>(su * inv_n);
  dst[2] = static_cast<float>(r * (sud - c * su) * inv_n);
}

template <int DT, int VEC>
__global__ __launch_bounds__(kSplitBlock) void ln_split_bwd_apply_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ mean, const float* __restrict__ rstd,
    const float* __restrict__ coef, void* __restrict__ dx, float* __restrict__ part, int64_t M,
    int N, int nseg, int64_t P, int64_t lddy, int64_t ldx, int64_t lddx) {
#pragma clang fp contract(off)
  using PK = Pack<DT, VEC>;
  constexpr int CH = SplitGeom<DT, VEC>::kCh;
  const SegIndex ix = seg_index<DT, VEC>(M, nseg, P);
  PK g[CH];
  load_weight<DT, VEC, CH>(g, gamma, ix.e0, N);
  float ag[CH][VEC], ab[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) ag[c][k] = ab[c][k] = 0.f;
  // One row per step, rows in order: each column sum adds its rows in row
  // order.
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
    const float mu = mean[row], r = rstd[row];
    const float* k3 = coef + row * 3;
    const float rc = r * k3[0], c1 = k3[1], c2 = k3[2];
    const char* dxr = row_ptr<DT>(dx, row, lddx);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g[c].opaque();
      const int e = chunk_elem<VEC>(ix.e0, c);
      if (e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float dyf = dv[c].get(k);
          const float u = dyf * g[c].get(k);
          const float xh = fmaf(xv[c].get(k) - mu, r, -rc);
          o[k] = r * fmaf(-xh, c2, u - c1);
          ag[c][k] = fmaf(dyf, xh, ag[c][k]);
          ab[c][k] += dyf;
        }
        PK out;
        out.set(o);
        store_at<DT, VEC>(out, dxr, e);
      }
    }
  }
  const int64_t p = blockIdx.x / nseg;
  float* dg = part + p * N;
  float* db = part + (P + p) * N;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = chunk_elem<VEC>(ix.e0, c);
    if (e < N) {
      store_f32<VEC>(dg + e, ag[c]);
      store_f32<VEC>(db + e, ab[c]);
    }
  }
}

// ---- host side ---------------------------------------------------------------

template <int DT, int VEC>
hipError_t ln_split_fwd_vec(const SplitPlan& sp, const LnFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  const int64_t ldx = a.x_pitch / es, ldy = a.y_pitch / es;
  const int64_t grid = sp.P * sp.nseg;
  const int64_t rows_grid = (a.M + 255) / 256;
  hipError_t e = launch(ln_split_fwd_stats_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.x, a.y,
                        a.M, a.N, sp.nseg, sp.P, ldx, ldy);
  if (e != hipSuccess) return e;
  e = launch(ln_split_fwd_finish_kernel<DT>, rows_grid, 256, 0, s, a.y, a.mean, a.rstd, a.M, a.N,
             sp.nseg, SplitGeom<DT, VEC>::kSeg, ldy, a.eps);
  if (e != hipSuccess) return e;
  e = launch(ln_split_fwd_apply_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.x, a.gamma, a.beta,
             a.mean, a.rstd, a.y, a.M, a.N, sp.nseg, sp.P, ldx, ldy);
  if (e != hipSuccess) return e;
  return launch(ln_split_fwd_head_kernel<DT, head_elems<DT, VEC>()>, rows_grid, 256, 0, s, a.x,
                a.gamma, a.beta, a.mean, a.rstd, a.y, a.M, ldx, ldy);
}

template <int DT, int VEC>
hipError_t ln_split_bwd_vec(const SplitPlan& sp, const LnBwdArgs& a, float* sums, float* coef,
                            hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  const int64_t lddy = a.dy_pitch / es, ldx = a.x_pitch / es, lddx = a.dx_pitch / es;
  const int64_t grid = sp.P * sp.nseg;
  // The stats pass keeps no column sums, so it may cut the rows finer than
  // the apply pass (more workgroups in flight; its sums do not depend on it).
  const int64_t Ps = sp.P_free > 0 ? sp.P_free : sp.P;
  hipError_t e = launch(ln_split_bwd_stats_kernel<DT, VEC>, Ps * sp.nseg, kSplitBlock, 0, s, a.dy,
                        a.x, a.gamma, a.mean, sums, a.M, a.N, sp.nseg, Ps, lddy, ldx);
  if (e != hipSuccess) return e;
  e = launch(ln_split_bwd_finish_kernel, (a.M + 255) / 256, 256, 0, s, sums, a.rstd, coef, a.M,
             a.N, sp.nseg);
  if (e != hipSuccess) return e;
  return launch(ln_split_bwd_apply_kernel<DT, VEC>, grid, kSplitBlock, 0, s, a.dy, a.x, a.gamma,
                a.mean, a.rstd, coef, a.dx, a.part, a.M, a.N, sp.nseg, sp.P, lddy, ldx, lddx);
}

template <int DT>
hipError_t ln_split_fwd_dt(const SplitPlan& sp, const LnFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (sp.vec * es) {
    case 16: return ln_split_fwd_vec<DT, 16 / es>(sp, a, s);
    case 8: return ln_split_fwd_vec<DT, 8 / es>(sp, a, s);
    case 4: return ln_split_fwd_vec<DT, 4 / es>(sp, a, s);
    case 2:
      if constexpr (es == 2) return ln_split_fwd_vec<DT, 1>(sp, a, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t ln_split_bwd_dt(const SplitPlan& sp, const LnBwdArgs& a, float* sums, float* coef,
                           hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (sp.vec * es) {
    case 16: return ln_split_bwd_vec<DT, 16 / es>(sp, a, sums, coef, s);
    case 8: return ln_split_bwd_vec<DT, 8 / es>(sp, a, sums, coef, s);
    case 4: return ln_split_bwd_vec<DT, 4 / es>(sp, a, sums, coef, s);
    case 2:
      if constexpr (es == 2) return ln_split_bwd_vec<DT, 1>(sp, a, sums, coef, s);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t ln_split_fwd_launch(int dtype, const SplitPlan& sp, const LnFwdArgs& a,
                               hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_split_fwd_dt<kF32>(sp, a, s);
    case kF16: return ln_split_fwd_dt<kF16>(sp, a, s);
    case kBF16: return ln_split_fwd_dt<kBF16>(sp, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t ln_split_bwd_launch(int dtype, const SplitPlan& sp, const LnBwdArgs& a, float* sums,
                               float* coef, hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_split_bwd_dt<kF32>(sp, a, sums, coef, s);
    case kF16: return ln_split_bwd_dt<kF16>(sp, a, sums, coef, s);
    case kBF16: return ln_split_bwd_dt<kBF16>(sp, a, sums, coef, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
