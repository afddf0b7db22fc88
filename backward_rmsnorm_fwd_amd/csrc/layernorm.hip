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
// The backward recomputes the row sum of x in float64 alongside sum(u) and
// sum(u*(x - mean)) (one exchange) and takes the offset c = sum/N - mean of
// the stored float32 mean out of x - mean, as the forward does: with
// xhat = ((x - mean) - c)*r, sum(u*xhat) = r*(sum(u*(x - mean)) - c*sum(u)).
//
// Geometry: a row is spread over `wpr` wavefronts (64*wpr lanes, a power of
// two up to 16); lane t of a row owns vectors c*64*wpr + t for c < chunks,
// so each chunk is one coalesced sweep.  A workgroup of B threads (256, or
// 64*wpr for longer rows; at most 1024) holds G = B/(64*wpr) rows at a time.  Elements past N are loaded as 0 and left out of
// the variance and of every store.
//
// Backward stage 1: workgroup w owns rows [w*M/P, (w+1)*M/P) (its G row
// groups take them in turn), accumulates the column sums of dy*xhat and dy in
// float32 registers, adds its G groups in group order through LDS and writes
// part[w, :] (dgamma) and part[P + w, :] (dbeta).  Stage 2 adds each [P, N]
// block by column in float64 (the RMSNorm reduce kernels).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"

namespace rmsnorm_hip {
namespace {

using namespace rowres;
constexpr int kLnMaxBlock = kRowMaxBlock;
constexpr int kLnWaves = kRowWaves;

// BLK: 256 for 256-thread workgroups (at least 3 wavefronts per SIMD, up to
// 168 VGPRs), else 1024 (512- and 1024-thread workgroups, 128 VGPRs).
template <int DT, int VEC, int MAXC, int BLK>
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
  PK g[MAXC], b[MAXC];
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
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * step; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * step) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      g[c].opaque();
      b[c].opaque();
    }
    int64_t row[R];
    bool active[R];
    PK xv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = row0 + j * rg.G + rg.group;
      active[j] = row[j] < M;
      const char* xr = row_base<DT>(x, row[j], ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        xv[j][c].zero();
        if (active[j] && c < chunks && e < N) ld<DT, VEC, true>(xv[j][c], xr, e);
      }
    }
    double s[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      s[j] = 0.0;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) s[j] += static_cast<double>(xv[j][c].get(k));
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
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float d = xv[j][c].get(k) - mu[j];
            q[j] = fmaf(d, d, q[j]);
          }
        }
      }
    }
    row_sums<0, R, R, R>(nullptr, q, slots64, slots, parity, wpr, rg);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float r = 1.0f / sqrtf((q[j] / n_f - cm[j] * cm[j]) + eps);
      if (!active[j]) continue;
      if (rg.t == 0) {
        mean[row[j]] = mu[j];
        rstd[row[j]] = r;
      }
      const char* yr = row_base<DT>(y, row[j], ldy);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = fmaf(((xv[j][c].get(k) - mu[j]) - cm[j]) * r, g[c].get(k), b[c].get(k));
          PK out;
          out.set(o);
          st<DT, VEC>(out, yr, e);
        }
      }
    }
  }
}

template <int DT, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void ln_bwd_kernel(
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
  extern __shared__ __align__(16) float comb[];  // [blockDim.x * VEC] when G > 1
  __shared__ float slots[2 * kLnWaves * 2 * R];
  __shared__ double slots64[2 * kLnWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  const int64_t w = blockIdx.x;
  const int64_t r0 = block_row_begin(w, M, P);
  const int64_t r1 = block_row_begin(w + 1, M, P);
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  const int64_t iters = (r1 - r0 + step - 1) / step;
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
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    int64_t row[R];
    bool active[R];
    float mu[R], r[R];
    PK dv[R][MAXC], xv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = r0 + it * step + j * rg.G + rg.group;
      active[j] = row[j] < r1;
      mu[j] = active[j] ? mean[row[j]] : 0.f;
      r[j] = active[j] ? rstd[row[j]] : 0.f;
      const char* dyr = row_base<DT>(dy, row[j], lddy);
      const char* xr = row_base<DT>(x, row[j], ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        dv[j][c].zero();
        xv[j][c].zero();
        if (active[j] && c < chunks && e < N) {
          ld<DT, VEC, true>(dv[j][c], dyr, e);
          ld<DT, VEC, true>(xv[j][c], xr, e);
        }
      }
    }
    // Lanes past N hold x = dy = 0, so they add 0 to every sum.
    double sx[R];
    float s12[2 * R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      sx[j] = 0.0;
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float xf = xv[j][c].get(k);
          const float u = dv[j][c].get(k) * g[c].get(k);
          sx[j] += static_cast<double>(xf);
          s1 += u;
          s2 = fmaf(u, xf - mu[j], s2);
        }
      s12[2 * j] = s1;
      s12[2 * j + 1] = s2;
    }
    row_sums<R, 2 * R, R, 2 * R>(sx, s12, slots64, slots, parity, wpr, rg);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        dv[j][c].opaque();
        xv[j][c].opaque();
      }
    }
    // Rows in order (j = 0, 1, ...), so each column sum adds its rows in
    // row order.
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (!active[j]) continue;
      const float cm = static_cast<float>(sx[j] / static_cast<double>(N) -
                                          static_cast<double>(mu[j]));
      const float s1 = s12[2 * j], s2 = s12[2 * j + 1];
      const float c1 = s1 / n_f;
      const float c2 = (r[j] * (s2 - cm * s1)) / n_f;
      const char* dxr = row_base<DT>(dx, row[j], lddx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float dyf = dv[j][c].get(k);
            const float xh = ((xv[j][c].get(k) - mu[j]) - cm) * r[j];
            const float u = dyf * g[c].get(k);
            o[k] = r[j] * ((u - c1) - xh * c2);
            ag[c][k] = fmaf(dyf, xh, ag[c][k]);
            ab[c][k] += dyf;
          }
          PK out;
          out.set(o);
          st<DT, VEC>(out, dxr, e);
        }
      }
    }
  }

  // Column sums of the G row groups, added in group order: dgamma partials
  // to part[w, :], dbeta partials to part[P + w, :].
  for (int which = 0; which < 2; ++which) {
    float* dst = part + (which * P + w) * static_cast<int64_t>(N);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c >= chunks) break;  // uniform: chunks is a kernel argument
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
