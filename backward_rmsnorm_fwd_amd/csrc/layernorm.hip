// LayerNorm forward and backward for gfx950 (the sibling of RMSNorm on the
// page "PyTorch torch.compile ... LayerNorm and RMSNorm", section 1.1: each
// row normalised by its mean and variance, then scaled by gamma and shifted
// by beta; section 2: the backward yields dx, dgamma and dbeta; section 1.4:
// the forward keeps the row statistics for the backward).
//
// Per row of N elements (float32 after widening the inputs):
//   forward   mu = sum(x)/N;  var = sum((x - mu)^2)/N;  r = 1/sqrt(var + eps)
//             y = ((x - mu)*r)*gamma + beta;  mean[i] = mu, rstd[i] = r
// The row sum is accumulated in float64 (every widened element is exact
// there) and rounded once to the float32 mean mu; the variance is taken from
// the float32 deviations d = x - mu held in registers, less the square of the
// exactly known offset c = (sum/N) - mu between the exact and the rounded
// mean (sum(d^2)/N - c^2 is the variance about the exact mean), and c is
// also taken out of d before scaling.  The statistics thus stay within about
// one float32 rounding of their exact values even when a row's mean is large
// against its spread.
//   backward  xhat = (x - mu)*r;  u = dy*gamma
//             dx = r*((u - sum(u)/N) - xhat*(sum(u*xhat)/N))
//             dgamma += dy*xhat;  dbeta += dy   (column sums over rows)
// The backward takes the offset c = sum(x)/N - mean of the stored float32
// mean out of x - mean, as the forward does, with c = sum(x - mean)/N from
// the float32 deviations d = x - mean: where the mean is large against the
// spread d is exact (x and mean within a factor of two), and elsewhere c is
// below the rounding of xhat anyway.  With xhat = (d - c)*r,
// sum(u*xhat) = r*(sum(u*d) - c*sum(u)).  sum(u), sum(u*d) and sum(d) share
// one exchange.
//
// Geometry: a row is spread over `wpr` wavefronts (64*wpr lanes: a power of
// two up to 16, or for backward rows over four wavefronts the exact divisor
// of the row the plan picks); lane t of a row owns vectors c*64*wpr + t for
// c < chunks, so each chunk is one coalesced sweep.  A workgroup of B
// threads (256, or 64*wpr for longer rows; at most 1024) holds
// G = B/(64*wpr) rows at a time.  Lanes past N take no part in the row
// sums or the stores.
//
// Backward stage 1: the rows are cut into steps of G*R consecutive rows (R
// rows per row group) and workgroup w takes steps w, w+P, w+2P, ..., so the
// P workgroups stream one contiguous window of the matrices at a time.  It
// accumulates the column sums of dy*xhat and dy in float32 registers (each
// row group adds its rows in row order), adds its G groups in group order
// through LDS and writes part[w, :] (dgamma) and part[P + w, :] (dbeta).
// Stage 2 adds each [P, N] block by column in float64 (the RMSNorm reduce
// kernels).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"

namespace rmsnorm_hip {
namespace {

using namespace rowres;
constexpr int kLnWaves = kRowWaves;

// BLK: 256 for 256-thread workgroups (at least 3 wavefronts per SIMD, up to
// 168 VGPRs), else 1024 (512- and 1024-thread workgroups, 128 VGPRs).
// WREG keeps gamma and beta in registers across rows; without it (rows of
// more than four 16-byte chunks per lane, up to 64 KiB of bf16 or 128 KiB
// of float32) they are read from cache at each use.
template <int DT, int VEC, int MAXC, int BLK, bool WREG = true>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void ln_fwd_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta,
    void* __restrict__ y, float* __restrict__ mean, float* __restrict__ rstd, int64_t M, int N,
    int chunks, int wpr, float eps, int64_t ldx, int64_t ldy) {
  using PK = Pack<DT, VEC>;
  constexpr int R = rows_per_step<DT, VEC, MAXC, 1, BLK>();
  __shared__ float slots[2 * kLnWaves * R];
  __shared__ double slots64[2 * kLnWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  PK g[WREG ? MAXC : 1], b[WREG ? MAXC : 1];
  if constexpr (WREG) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * rg.tpr + rg.t) * VEC;
      g[c].zero();
      b[c].zero();
      if (c < chunks && e < N) {
        ld<DT, VEC, false>(g[c], static_cast<const char*>(gamma), e);
        if (beta) ld<DT, VEC, false>(b[c], static_cast<const char*>(beta), e);
      }
    }
  }
  // ok[c]: this lane's vector of chunk c lies inside the row.
  bool ok[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) ok[c] = c < chunks && (c * rg.tpr + rg.t) * VEC < N;
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * step; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * step) {
    if constexpr (WREG) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        g[c].opaque();
        b[c].opaque();
      }
    }
    // The loads carry no lane condition (a row past the matrix reads its
    // last row, a lane past the row reads the row's first vector); the
    // values are masked where they are used.  x is loaded with the default
    // cache policy (y is stored streaming): the backward reads x again, and
    // the rows this sweep touched last stay in the Infinity Cache for a
    // backward that starts there (bf16 32768 x 4096: stage 1 122 against
    // 137 us right after a forward that streamed x).
    int64_t row[R];
    PK xv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = row0 + j * rg.G + rg.group;
      const char* xr = row_base<DT>(x, row[j] < M ? row[j] : M - 1, ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks) ld<DT, VEC, false>(xv[j][c], xr, e < N ? e : 0);  // c is uniform
        else xv[j][c].zero();
      }
    }
    // Float64 row sums, pairwise within each vector and across chunks (a
    // short dependency chain; the order does not matter to the exact sum
    // of widened 16-bit elements, and float32 elements round at 2^-53).
    double s[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      double cs[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        double v[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[k] = static_cast<double>(xv[j][c].get(k));
#pragma unroll
        for (int h = VEC / 2; h > 0; h /= 2)
#pragma unroll
          for (int k = 0; k < h; ++k) v[k] += v[k + h];
        cs[c] = ok[c] ? v[0] : 0.0;
        // Without the weights in registers the rows are long: widen one
        // chunk at a time (no instruction crosses the fence) and from the
        // packed registers again in each pass.
        if constexpr (!WREG) {
          xv[j][c].opaque();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int h = MAXC / 2; h > 0; h /= 2)
#pragma unroll
        for (int c = 0; c < h; ++c) cs[c] += cs[c + h];
      s[j] = cs[0];
    }
    row_sums<R, 0, R, R>(s, nullptr, slots64, slots, parity, wpr, rg);
    float mu[R], cm[R], q[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const double mu64 = s[j] / static_cast<double>(N);
      mu[j] = static_cast<float>(mu64);
      cm[j] = static_cast<float>(mu64 - static_cast<double>(mu[j]));
      q[j] = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        float qc = 0.f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float d = xv[j][c].get(k) - mu[j];
          qc = fmaf(d, d, qc);
        }
        q[j] += ok[c] ? qc : 0.f;
        if constexpr (!WREG) {
          xv[j][c].opaque();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    row_sums<0, R, R, R>(nullptr, q, slots64, slots, parity, wpr, rg);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float r = 1.0f / sqrtf((q[j] / n_f - cm[j] * cm[j]) + eps);
      if (row[j] >= M) continue;
      if (rg.t == 0) {
        mean[row[j]] = mu[j];
        rstd[row[j]] = r;
      }
      // xhat = (x - mu - c)*r as one fma from the deviation.
      const float ncr = -(cm[j] * r);
      const char* yr = row_base<DT>(y, row[j], ldy);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        if (!ok[c]) continue;
        const int e = (c * rg.tpr + rg.t) * VEC;
        float o[VEC];
        if constexpr (WREG) {
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = fmaf(fmaf(xv[j][c].get(k) - mu[j], r, ncr), g[c].get(k), b[c].get(k));
        } else {
          PK gv, bv;
          ld<DT, VEC, false>(gv, static_cast<const char*>(gamma), e);
          bv.zero();
          if (beta) ld<DT, VEC, false>(bv, static_cast<const char*>(beta), e);
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = fmaf(fmaf(xv[j][c].get(k) - mu[j], r, ncr), gv.get(k), bv.get(k));
        }
        PK out;
        out.set(o);
        st<DT, VEC>(out, yr, e);
        if constexpr (!WREG) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int DT, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 2 : 1) void ln_bwd_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ mean, const float* __restrict__ rstd, void* __restrict__ dx,
    float* __restrict__ part, int64_t M, int N, int chunks, int wpr, int64_t P, int64_t lddy,
    int64_t ldx, int64_t lddx) {
  // No implicit contraction: u = dy*gamma must round the same way in the row
  // sum and in u - sum(u)/N, so that term is exactly 0 where the row is (an
  // FMA would leave the product's rounding error, scaled by r).  The fmaf
  // calls below are deliberate.
#pragma clang fp contract(off)
  using PK = Pack<DT, VEC>;
  constexpr int R = rows_per_step<DT, VEC, MAXC, 2, BLK>();
  constexpr bool kTwoSets = BLK == 256;  // larger workgroups have 128 VGPRs: one set
  extern __shared__ __align__(16) float comb[];  // [blockDim.x * VEC] when G > 1
  __shared__ float slots[2 * kLnWaves * 3 * R];
  const RowGeom rg = row_geom(wpr);
  const float inv_n = 1.0f / static_cast<float>(N);
  int parity = 0;
  const int64_t w = blockIdx.x;
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  const int64_t nsteps = (M + step - 1) / step;
  const int64_t iters = w < nsteps ? (nsteps - w + P - 1) / P : 0;
  PK g[MAXC];
  float ag[MAXC][VEC], ab[MAXC][VEC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * rg.tpr + rg.t) * VEC;
    g[c].zero();
    if (c < chunks && e < N) ld<DT, VEC, false>(g[c], static_cast<const char*>(gamma), e);
#pragma unroll
    for (int k = 0; k < VEC; ++k) ag[c][k] = ab[c][k] = 0.f;
  }

  // The rows of one step, held in registers.  In 256-thread workgroups two
  // sets alternate: the next step's loads are issued into one while the
  // other is reduced and written, so every row group keeps a step of loads
  // in flight across its barriers.  Those loads carry no condition (a row
  // past the matrix reads its last row, a lane past the row reads
  // the row's first vector, and both are masked where the values are used),
  // so the compiler can count them and wait for the older set alone.  With
  // one set, out-of-row lanes skip their loads and hold zeros.
  struct Rows {
    PK dv[R][MAXC], xv[R][MAXC];
    float mu[R], r[R];
  };
  auto row_of = [&](int64_t it, int j) __attribute__((always_inline)) {
    return (it * P + w) * step + j * rg.G + rg.group;
  };
  auto load_rows = [&](int64_t it, Rows& s) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int64_t row = row_of(it, j);
      const int64_t rr = row < M ? row : M - 1;
      s.mu[j] = mean[rr];
      s.r[j] = rstd[rr];
      const char* dyr = row_base<DT>(dy, rr, lddy);
      const char* xr = row_base<DT>(x, rr, ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if constexpr (kTwoSets) {
          const int el = c < chunks && e < N ? e : 0;
          ld<DT, VEC, true>(s.dv[j][c], dyr, el);
          ld<DT, VEC, true>(s.xv[j][c], xr, el);
        } else if (c < chunks && e < N) {
          ld<DT, VEC, true>(s.dv[j][c], dyr, e);
          ld<DT, VEC, true>(s.xv[j][c], xr, e);
        } else {
          s.dv[j][c].zero();
          s.xv[j][c].zero();
        }
      }
    }
  };
  auto process = [&](int64_t it, Rows& s) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      g[c].opaque();
      const int e = (c * rg.tpr + rg.t) * VEC;
      if (kTwoSets && !(c < chunks && e < N)) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          s.dv[j][c].zero();
          s.xv[j][c].zero();
        }
      }
    }
    // Lanes past N hold x = dy = 0 and add 0 to sum(u) and sum(u*d); their
    // d = -mean is left out of sum(d).
    float sums[3 * R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float d = s.xv[j][c].get(k) - s.mu[j];
          const float u = s.dv[j][c].get(k) * g[c].get(k);
          s1 += u;
          s2 = fmaf(u, d, s2);
          t += d;
        }
        if (c < chunks && e < N) s3 += t;
      }
      sums[3 * j] = s1;
      sums[3 * j + 1] = s2;
      sums[3 * j + 2] = s3;
    }
    row_sums<0, 3 * R, 1, 3 * R>(nullptr, sums, nullptr, slots, parity, wpr, rg);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        s.dv[j][c].opaque();
        s.xv[j][c].opaque();
      }
    }
    // Rows in order (j = 0, 1, ...), so each column sum adds its rows in
    // row order.
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int64_t row = row_of(it, j);
      if (row >= M) continue;
      const float mu = s.mu[j], r = s.r[j];
      const float s1 = sums[3 * j], s2 = sums[3 * j + 1];
      const float cm = sums[3 * j + 2] * inv_n;
      const float c1 = s1 * inv_n;
      const float c2 = (r * (s2 - cm * s1)) * inv_n;
      const float rcm = r * cm;
      const char* dxr = row_base<DT>(dx, row, lddx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float dyf = s.dv[j][c].get(k);
            const float xh = fmaf(s.xv[j][c].get(k) - mu, r, -rcm);
            const float u = dyf * g[c].get(k);
            o[k] = r * fmaf(-xh, c2, u - c1);
            ag[c][k] = fmaf(dyf, xh, ag[c][k]);
            ab[c][k] += dyf;
          }
          PK out;
          out.set(o);
          st<DT, VEC>(out, dxr, e);
        }
      }
    }
  };

  Rows a;
  if constexpr (kTwoSets) {
    Rows b;
    int64_t it = 0;
    if (iters > 0) load_rows(0, a);
    for (; it + 2 < iters; it += 2) {
      load_rows(it + 1, b);
      process(it, a);
      load_rows(it + 2, a);
      process(it + 1, b);
    }
    if (it + 1 < iters) {
      load_rows(it + 1, b);
      process(it, a);
      process(it + 1, b);
    } else if (it < iters) {
      process(it, a);
    }
  } else {
    for (int64_t it = 0; it < iters; ++it) {
      load_rows(it, a);
      process(it, a);
    }
  }

  // Column sums of the G row groups, added in group order: dgamma partials
  // to part[w, :], dbeta partials to part[P + w, :].
  for (int which = 0; which < 2; ++which) {
    float* dst = part + (which * P + w) * static_cast<int64_t>(N);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c >= chunks) continue;  // uniform: chunks is a kernel argument
      const int e = (c * rg.tpr + rg.t) * VEC;
      float v[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) v[k] = which ? ab[c][k] : ag[c][k];
      if (rg.G == 1) {
        if (e < N) store_f32<VEC>(dst + e, v);
        continue;
      }
      float* mine = comb + (rg.group * rg.tpr + rg.t) * VEC;
#pragma unroll
      for (int k = 0; k < VEC; ++k) mine[k] = v[k];
      __syncthreads();
      if (rg.group == 0 && e < N) {
        float tot[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) tot[k] = comb[rg.t * VEC + k];
        for (int h = 1; h < rg.G; ++h) {
#pragma unroll
          for (int k = 0; k < VEC; ++k) tot[k] += comb[(h * rg.tpr + rg.t) * VEC + k];
        }
        store_f32<VEC>(dst + e, tot);
      }
      __syncthreads();
    }
  }
}

template <int DT, int VEC, int MAXC>
hipError_t ln_fwd_maxc(const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  auto* k = p.block == 256 ? ln_fwd_kernel<DT, VEC, MAXC, 256> : ln_fwd_kernel<DT, VEC, MAXC, 1024>;
  return launch(k, p.grid, p.block, 0, s, a.x, a.gamma, a.beta, a.y,
                a.mean, a.rstd, a.M, a.N, p.chunks, p.wpr, a.eps, a.x_pitch / es,
                a.y_pitch / es);
}

template <int DT, int VEC, int MAXC>
hipError_t ln_bwd_maxc(const LnPlan& p, const LnBwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  auto* k = p.block == 256 ? ln_bwd_kernel<DT, VEC, MAXC, 256> : ln_bwd_kernel<DT, VEC, MAXC, 1024>;
  return launch(k, p.grid, p.block, static_cast<size_t>(p.lds), s,
                a.dy, a.x, a.gamma, a.mean, a.rstd, a.dx, a.part, a.M, a.N, p.chunks, p.wpr,
                p.grid, a.dy_pitch / es, a.x_pitch / es, a.dx_pitch / es);
}

template <int DT>
hipError_t ln_fwd_dt(const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(ln_fwd_maxc, DT, false, p, a, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t ln_bwd_dt(const LnPlan& p, const LnBwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(ln_bwd_maxc, DT, true, p, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Full-width rows of five to eight 16-byte chunks per lane over 16
// wavefronts (bf16/fp16 N <= 65536, float32 N <= 32768): the weights are not
// held in registers.
template <int DT>
hipError_t ln_fwd_long_dt(const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  constexpr int VEC = 16 / es;
  if (p.vec != VEC || p.block != 1024 || p.wpr != 16 || p.chunks > 8) return hipErrorInvalidValue;
  return launch(ln_fwd_kernel<DT, VEC, 8, 1024, false>, p.grid, p.block, 0, s, a.x, a.gamma,
                a.beta, a.y, a.mean, a.rstd, a.M, a.N, p.chunks, p.wpr, a.eps, a.x_pitch / es,
                a.y_pitch / es);
}

hipError_t ln_fwd_long_launch(int dtype, const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_fwd_long_dt<kF32>(p, a, s);
    case kF16: return ln_fwd_long_dt<kF16>(p, a, s);
    case kBF16: return ln_fwd_long_dt<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t ln_fwd_launch(int dtype, const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_fwd_dt<kF32>(p, a, s);
    case kF16: return ln_fwd_dt<kF16>(p, a, s);
    case kBF16: return ln_fwd_dt<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t ln_bwd_launch(int dtype, const LnPlan& p, const LnBwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_bwd_dt<kF32>(p, a, s);
    case kF16: return ln_bwd_dt<kF16>(p, a, s);
    case kBF16: return ln_bwd_dt<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
