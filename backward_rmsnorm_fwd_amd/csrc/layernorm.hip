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
// so each chunk is one coalesced sweep.  A 1024-thread workgroup holds
// G = 16/wpr rows at a time.  Elements past N are loaded as 0 and left out of
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

namespace rmsnorm_hip {
namespace {

constexpr int kLnBlock = 1024;
constexpr int kLnWaves = kLnBlock / kWave;

// Sum of v over the wpr wavefronts of this thread's row (wpr uniform across
// the workgroup, so every thread takes the same path and the barrier is
// reached by all).  slots: [2][kLnWaves] floats; parity alternates.
__device__ __forceinline__ float row_sum(float v, float* slots, int& parity, int wpr,
                                         int first_wave, int wave, int lane) {
  v = wave_sum(v);
  if (wpr == 1) return v;
  float* s = slots + parity * kLnWaves;
  if (lane == 0) s[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < wpr; ++i) t += s[first_wave + i];
  parity ^= 1;
  return t;
}

// float64 sum over the 64 lanes: xor butterfly, every lane ends with the
// same bits (each pairwise add sees the same two operands).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ double row_sum_f64(double v, double* slots, int& parity, int wpr,
                                              int first_wave, int wave, int lane) {
  v = wave_sum_f64(v);
  if (wpr == 1) return v;
  double* s = slots + parity * kLnWaves;
  if (lane == 0) s[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < wpr; ++i) t += s[first_wave + i];
  parity ^= 1;
  return t;
}

// One float64 and two float32 sums in one exchange (one barrier).
// slots64: [2][kLnWaves]; slots: [2][kLnWaves][2].
__device__ __forceinline__ void row_sum3(double& a, float& b, float& c, double* slots64,
                                         float* slots, int& parity, int wpr, int first_wave,
                                         int wave, int lane) {
  a = wave_sum_f64(a);
  b = wave_sum(b);
  c = wave_sum(c);
  if (wpr == 1) return;
  double* s64 = slots64 + parity * kLnWaves;
  float* s = slots + parity * kLnWaves * 2;
  if (lane == 0) {
    s64[wave] = a;
    s[2 * wave] = b;
    s[2 * wave + 1] = c;
  }
  __syncthreads();
  double ta = 0.0;
  float tb = 0.f, tc = 0.f;
  for (int i = 0; i < wpr; ++i) {
    ta += s64[first_wave + i];
    tb += s[2 * (first_wave + i)];
    tc += s[2 * (first_wave + i) + 1];
  }
  a = ta;
  b = tb;
  c = tc;
  parity ^= 1;
}

template <int DT>
__device__ __forceinline__ const char* row_base(const void* base, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + row * ld * ElemBytes<DT>::value;
}

// Lane access at element e of a row: uniform row base plus an opaque 32-bit
// byte offset (no 64-bit address per chunk; loads stay inside the row loop).
template <int DT, int VEC, bool NT>
__device__ __forceinline__ void ld(Pack<DT, VEC>& v, const char* row, int e) {
  uint32_t off = static_cast<uint32_t>(e) * ElemBytes<DT>::value;
  asm volatile("" : "+v"(off));
  using R = typename Pack<DT, VEC>::raw_t;
  const R* a = reinterpret_cast<const R*>(row + off);
  if constexpr (NT) v.raw = __builtin_nontemporal_load(a);
  else v.raw = *a;
}

template <int DT, int VEC>
__device__ __forceinline__ void st(const Pack<DT, VEC>& v, const char* row, int e) {
  uint32_t off = static_cast<uint32_t>(e) * ElemBytes<DT>::value;
  asm volatile("" : "+v"(off));
  using R = typename Pack<DT, VEC>::raw_t;
  __builtin_nontemporal_store(v.raw, reinterpret_cast<R*>(const_cast<char*>(row) + off));
}

struct RowGeom {
  int tpr, G, t, group, first_wave, wave, lane;
};

__device__ __forceinline__ RowGeom row_geom(int wpr) {
  RowGeom g;
  g.tpr = kWave * wpr;
  g.G = kLnBlock / g.tpr;
  g.t = threadIdx.x % g.tpr;
  g.group = threadIdx.x / g.tpr;
  g.first_wave = g.group * wpr;
  g.wave = threadIdx.x / kWave;
  g.lane = threadIdx.x % kWave;
  return g;
}

template <int DT, int VEC, int MAXC>
__global__ __launch_bounds__(kLnBlock) void ln_fwd_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, const void* __restrict__ beta,
    void* __restrict__ y, float* __restrict__ mean, float* __restrict__ rstd, int64_t M, int N,
    int chunks, int wpr, float eps, int64_t ldx, int64_t ldy) {
  using PK = Pack<DT, VEC>;
  __shared__ float slots[2 * kLnWaves];
  __shared__ double slots64[2 * kLnWaves];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0, parity64 = 0;
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
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * rg.G; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * rg.G) {
    const int64_t row = row0 + rg.group;
    const bool active = row < M;
    const char* xr = row_base<DT>(x, row, ldx);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      g[c].opaque();
      b[c].opaque();
    }
    PK xv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * rg.tpr + rg.t) * VEC;
      xv[c].zero();
      if (active && c < chunks && e < N) ld<DT, VEC, true>(xv[c], xr, e);
    }
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
      for (int k = 0; k < VEC; ++k) s += static_cast<double>(xv[c].get(k));
    s = row_sum_f64(s, slots64, parity64, wpr, rg.first_wave, rg.wave, rg.lane);
    const double mu64 = s / static_cast<double>(N);
    const float mu = static_cast<float>(mu64);
    const float cm = static_cast<float>(mu64 - static_cast<double>(mu));
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * rg.tpr + rg.t) * VEC;
      if (c < chunks && e < N) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float d = xv[c].get(k) - mu;
          q = fmaf(d, d, q);
        }
      }
    }
    q = row_sum(q, slots, parity, wpr, rg.first_wave, rg.wave, rg.lane);
    const float r = 1.0f / sqrtf((q / n_f - cm * cm) + eps);
    if (active) {
      if (rg.t == 0) {
        mean[row] = mu;
        rstd[row] = r;
      }
      const char* yr = row_base<DT>(y, row, ldy);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = fmaf(((xv[c].get(k) - mu) - cm) * r, g[c].get(k), b[c].get(k));
          PK out;
          out.set(o);
          st<DT, VEC>(out, yr, e);
        }
      }
    }
  }
}

template <int DT, int VEC, int MAXC>
__global__ __launch_bounds__(kLnBlock) void ln_bwd_kernel(
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
  extern __shared__ __align__(16) float comb[];  // [kLnBlock * VEC] when G > 1
  __shared__ float slots[2 * kLnWaves * 2];
  __shared__ double slots64[2 * kLnWaves];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  const int64_t w = blockIdx.x;
  const int64_t r0 = block_row_begin(w, M, P);
  const int64_t r1 = block_row_begin(w + 1, M, P);
  const int64_t iters = (r1 - r0 + rg.G - 1) / rg.G;
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
    const int64_t row = r0 + it * rg.G + rg.group;
    const bool active = row < r1;
    const char* dyr = row_base<DT>(dy, row, lddy);
    const char* xr = row_base<DT>(x, row, ldx);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    PK dv[MAXC], xv[MAXC];
    float mu = 0.f, r = 0.f;
    if (active) {
      mu = mean[row];
      r = rstd[row];
    }
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * rg.tpr + rg.t) * VEC;
      dv[c].zero();
      xv[c].zero();
      if (active && c < chunks && e < N) {
        ld<DT, VEC, true>(dv[c], dyr, e);
        ld<DT, VEC, true>(xv[c], xr, e);
      }
    }
    // Lanes past N hold x = dy = 0, so they add 0 to every sum.
    double sx = 0.0;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float xf = xv[c].get(k);
        const float u = dv[c].get(k) * g[c].get(k);
        sx += static_cast<double>(xf);
        s1 += u;
        s2 = fmaf(u, xf - mu, s2);
      }
    row_sum3(sx, s1, s2, slots64, slots, parity, wpr, rg.first_wave, rg.wave, rg.lane);
    const float cm =
        active ? static_cast<float>(sx / static_cast<double>(N) - static_cast<double>(mu)) : 0.f;
    const float c1 = s1 / n_f;
    const float c2 = (r * (s2 - cm * s1)) / n_f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      dv[c].opaque();
      xv[c].opaque();
    }
    if (active) {
      const char* dxr = row_base<DT>(dx, row, lddx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float dyf = dv[c].get(k);
            const float xh = ((xv[c].get(k) - mu) - cm) * r;
            const float u = dyf * g[c].get(k);
            o[k] = r * ((u - c1) - xh * c2);
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
  return launch(ln_fwd_kernel<DT, VEC, MAXC>, p.grid, kLnBlock, 0, s, a.x, a.gamma, a.beta, a.y,
                a.mean, a.rstd, a.M, a.N, p.chunks, p.wpr, a.eps, a.x_pitch / es,
                a.y_pitch / es);
}

template <int DT, int VEC, int MAXC>
hipError_t ln_bwd_maxc(const LnPlan& p, const LnBwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  return launch(ln_bwd_kernel<DT, VEC, MAXC>, p.grid, kLnBlock, static_cast<size_t>(p.lds), s,
                a.dy, a.x, a.gamma, a.mean, a.rstd, a.dx, a.part, a.M, a.N, p.chunks, p.wpr,
                p.grid, a.dy_pitch / es, a.x_pitch / es, a.dx_pitch / es);
}

int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Largest chunk count the plan gives a vector width (N <= 16384): the
// forward aims at min(4, 32/VEC) chunks, the backward at min(8, 16/VEC), and
// a row of 16384 elements over 16 wavefronts needs 16/VEC.  Only these
// register-slot counts are instantiated.
constexpr int ln_cap(int vec, bool backward) {
  const int target = backward ? (16 / vec < 8 ? 16 / vec : 8) : (32 / vec < 4 ? 32 / vec : 4);
  const int need = 16 / vec;
  const int m = target > need ? target : need;
  int p = 1;
  while (p < m) p <<= 1;
  return p;
}

#define LN_MAXC_CASE(FN, DT, VEC, BWD, C, ...) \
  case C:                                      \
    if constexpr (C <= ln_cap(VEC, BWD)) return FN<DT, VEC, C>(__VA_ARGS__); \
    return hipErrorInvalidValue;

#define LN_MAXC_SWITCH(FN, DT, VEC, BWD, ...)         \
  switch (pow2_ceil(p.chunks)) {                      \
    LN_MAXC_CASE(FN, DT, VEC, BWD, 1, __VA_ARGS__)    \
    LN_MAXC_CASE(FN, DT, VEC, BWD, 2, __VA_ARGS__)    \
    LN_MAXC_CASE(FN, DT, VEC, BWD, 4, __VA_ARGS__)    \
    LN_MAXC_CASE(FN, DT, VEC, BWD, 8, __VA_ARGS__)    \
    LN_MAXC_CASE(FN, DT, VEC, BWD, 16, __VA_ARGS__)   \
    default: return hipErrorInvalidValue;             \
  }

template <int DT>
hipError_t ln_fwd_dt(const LnPlan& p, const LnFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (p.vec * es) {
    case 16: LN_MAXC_SWITCH(ln_fwd_maxc, DT, 16 / es, false, p, a, s)
    case 8: LN_MAXC_SWITCH(ln_fwd_maxc, DT, 8 / es, false, p, a, s)
    case 4: LN_MAXC_SWITCH(ln_fwd_maxc, DT, 4 / es, false, p, a, s)
    case 2:
      if constexpr (es == 2) {
        LN_MAXC_SWITCH(ln_fwd_maxc, DT, 1, false, p, a, s)
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t ln_bwd_dt(const LnPlan& p, const LnBwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  switch (p.vec * es) {
    case 16: LN_MAXC_SWITCH(ln_bwd_maxc, DT, 16 / es, true, p, a, s)
    case 8: LN_MAXC_SWITCH(ln_bwd_maxc, DT, 8 / es, true, p, a, s)
    case 4: LN_MAXC_SWITCH(ln_bwd_maxc, DT, 4 / es, true, p, a, s)
    case 2:
      if constexpr (es == 2) {
        LN_MAXC_SWITCH(ln_bwd_maxc, DT, 1, true, p, a, s)
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

#undef LN_MAXC_SWITCH
#undef LN_MAXC_CASE

}  // namespace

int ln_block_threads() { return kLnBlock; }

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
