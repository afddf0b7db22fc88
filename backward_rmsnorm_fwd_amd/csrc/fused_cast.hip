// RMSNorm with the cast of its output to a narrower dtype fused after it (the
// page "PyTorch torch.compile ... LayerNorm and RMSNorm", introduction: a
// normalisation kernel gains from fusing the operations around it; a float32
// residual stream is normalised and handed to a bfloat16 or float16
// consumer).
//
//   forward   r = 1/sqrt(sum(x^2)/N + eps),  y = TO((x*r)*g),  g = gamma or 1 + w
//             (the arithmetic of the RMSNorm kernels, then one
//             round-to-nearest-even cast to TO)
//   backward  dy arrives in TO and is widened exactly (a dtype conversion
//             passes its gradient through); then RMSNorm's backward:
//             u = dy*g,  c = sum(u*x)/N,  dx = r*u - x*(r^3*c)   (float32)
//             dgamma += dy*x*r                                  (column sums)
//
// Against the unfused pair (rmsnorm_fwd in float32, then a cast kernel) the
// forward writes 2 bytes per element once instead of 4, then reads 4 and
// writes 2 again; the backward reads the narrow dy directly instead of a
// widened copy.  Rows use the row-resident layout of rowres.hpp.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"

namespace rmsnorm_hip {
namespace {

using namespace rowres;

// x, gamma and dx are float32 (Pack<kF32, VEC>); y and dy have type DTO
// (Pack<DTO, VEC>: half the bytes per lane).  BLK: 256 for 256-thread
// workgroups (at least 3 wavefronts per SIMD), else 1024 (512- and
// 1024-thread workgroups, 128 VGPRs).
template <int DTO, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void cast_rms_fwd_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, void* __restrict__ y,
    float* __restrict__ rstd, int64_t M, int N, int chunks, int wpr, float eps, int offset,
    int64_t ldx, int64_t ldy) {
  using PI = Pack<kF32, VEC>;
  using PO = Pack<DTO, VEC>;
  constexpr int R = rows_per_step<kF32, VEC, MAXC, 1, BLK>();
  __shared__ float slots[2 * kRowWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  PI g[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * rg.tpr + rg.t) * VEC;
    g[c].zero();
    if (c < chunks && e < N) ld<kF32, VEC, false>(g[c], static_cast<const char*>(gamma), e);
  }
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * step; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * step) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    int64_t row[R];
    bool active[R];
    PI xv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = row0 + j * rg.G + rg.group;
      active[j] = row[j] < M;
      const char* xr = row_base<kF32>(x, row[j], ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        xv[j][c].zero();
        if (active[j] && c < chunks && e < N) ld<kF32, VEC, true>(xv[j][c], xr, e);
      }
    }
    float ss[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      ss[j] = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float f = xv[j][c].get(k);
          ss[j] = fmaf(f, f, ss[j]);
        }
    }
    row_sums<0, R, 1, R>(nullptr, ss, nullptr, slots, parity, wpr, rg);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float r = 1.0f / sqrtf(ss[j] / n_f + eps);
      if (!active[j]) continue;
      if (rg.t == 0) rstd[row[j]] = r;
      const char* yr = row_base<DTO>(y, row[j], ldy);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = (xv[j][c].get(k) * r) * weight_of(g[c].get(k), offset);
          PO out;
          out.set(o);
          st<DTO, VEC>(out, yr, e);
        }
      }
    }
  }
}

template <int DTO, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void cast_rms_bwd_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ rstd, void* __restrict__ dx, float* __restrict__ part,
    int64_t M, int N, int chunks, int wpr, int64_t P, int offset, int64_t lddy, int64_t ldx,
    int64_t lddx) {
  using PI = Pack<kF32, VEC>;
  using PO = Pack<DTO, VEC>;
  constexpr int R = rows_per_step<kF32, VEC, MAXC, 2, BLK>();
  extern __shared__ __align__(16) float comb[];  // [blockDim.x * VEC] when G > 1
  __shared__ float slots[2 * kRowWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  // Steps of G*R consecutive rows; workgroup w takes steps w, w+P, w+2P, ...
  // (one contiguous window of the matrices at a time across the grid), and
  // each row group adds its rows to the column sums in row order.
  const int64_t w = blockIdx.x;
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  const int64_t nsteps = (M + step - 1) / step;
  const int64_t iters = w < nsteps ? (nsteps - w + P - 1) / P : 0;
  PI g[MAXC];
  float acc[MAXC][VEC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * rg.tpr + rg.t) * VEC;
    g[c].zero();
    if (c < chunks && e < N) ld<kF32, VEC, false>(g[c], static_cast<const char*>(gamma), e);
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    int64_t row[R];
    bool active[R];
    float r[R];
    PO dv[R][MAXC];
    PI xv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = (it * P + w) * step + j * rg.G + rg.group;
      active[j] = row[j] < M;
      r[j] = active[j] ? rstd[row[j]] : 0.f;
      const char* dyr = row_base<DTO>(dy, row[j], lddy);
      const char* xr = row_base<kF32>(x, row[j], ldx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        dv[j][c].zero();
        xv[j][c].zero();
        if (active[j] && c < chunks && e < N) {
          ld<DTO, VEC, true>(dv[j][c], dyr, e);
          ld<kF32, VEC, true>(xv[j][c], xr, e);
        }
      }
    }
    float dot[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      dot[j] = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c)
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          dot[j] = fmaf(dv[j][c].get(k) * weight_of(g[c].get(k), offset), xv[j][c].get(k),
                        dot[j]);
    }
    row_sums<0, R, 1, R>(nullptr, dot, nullptr, slots, parity, wpr, rg);
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
      for (int j = 0; j < R; ++j) {
        dv[j][c].opaque();
        xv[j][c].opaque();
      }
    // Rows in order (j = 0, 1, ...), so each column sum adds its rows in
    // row order.
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (!active[j]) continue;
      const float r3c = ((r[j] * r[j]) * r[j]) * (dot[j] / n_f);
      const char* dxr = row_base<kF32>(dx, row[j], lddx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float xf = xv[j][c].get(k);
            const float dyf = dv[j][c].get(k);
            const float u = dyf * weight_of(g[c].get(k), offset);
            o[k] = fmaf(-xf, r3c, r[j] * u);
            acc[c][k] = fmaf(dyf * xf, r[j], acc[c][k]);
          }
          PI out;
          out.set(o);
          st<kF32, VEC>(out, dxr, e);
        }
      }
    }
  }

  // Column sums of the G row groups, added in group order, to part[w, :].
  float* dst = part + w * static_cast<int64_t>(N);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    if (c >= chunks) continue;  // uniform: chunks is a kernel argument
    const int e = (c * rg.tpr + rg.t) * VEC;
    if (rg.G == 1) {
      if (e < N) store_f32<VEC>(dst + e, acc[c]);
      continue;
    }
    float* mine = comb + (rg.group * rg.tpr + rg.t) * VEC;
#pragma unroll
    for (int k = 0; k < VEC; ++k) mine[k] = acc[c][k];
    __syncthreads();
    if (rg.group == 0 && e < N) {
      float tot[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) tot[k] = comb[rg.t * VEC + k];
      for (int gi = 1; gi < rg.G; ++gi) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) tot[k] += comb[(gi * rg.tpr + rg.t) * VEC + k];
      }
      store_f32<VEC>(dst + e, tot);
    }
    __syncthreads();
  }
}

// Launchers for output type DTO, in the form the row-resident dispatch
// macros call (FN<DT, VEC, MAXC>, DT the float32 input type).
template <int DTO>
struct CastTo {
  template <int DT, int VEC, int MAXC>
  static hipError_t fwd(const LnPlan& p, const CastFwdArgs& a, hipStream_t s) {
    constexpr int eo = ElemBytes<DTO>::value;
    auto* k = p.block == 256 ? cast_rms_fwd_kernel<DTO, VEC, MAXC, 256>
                             : cast_rms_fwd_kernel<DTO, VEC, MAXC, 1024>;
    return launch(k, p.grid, p.block, 0, s, a.x, a.gamma, a.y, a.rstd, a.M, a.N, p.chunks,
                  p.wpr, a.eps, a.offset, a.x_pitch / 4, a.y_pitch / eo);
  }
  template <int DT, int VEC, int MAXC>
  static hipError_t bwd(const LnPlan& p, const CastBwdArgs& a, hipStream_t s) {
    constexpr int eo = ElemBytes<DTO>::value;
    auto* k = p.block == 256 ? cast_rms_bwd_kernel<DTO, VEC, MAXC, 256>
                             : cast_rms_bwd_kernel<DTO, VEC, MAXC, 1024>;
    return launch(k, p.grid, p.block, static_cast<size_t>(p.lds), s, a.dy, a.x, a.gamma,
                  a.rstd, a.dx, a.part, a.M, a.N, p.chunks, p.wpr, p.grid, a.offset,
                  a.dy_pitch / eo, a.x_pitch / 4, a.dx_pitch / 4);
  }
};

template <int DTO>
hipError_t cast_fwd_dto(const LnPlan& p, const CastFwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(CastTo<DTO>::template fwd, kF32, false, p, a, s);
  return hipErrorInvalidValue;
}

template <int DTO>
hipError_t cast_bwd_dto(const LnPlan& p, const CastBwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(CastTo<DTO>::template bwd, kF32, true, p, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t cast_fwd_launch(int out_dtype, const LnPlan& p, const CastFwdArgs& a,
                           hipStream_t s) {
  switch (out_dtype) {
    case kF16: return cast_fwd_dto<kF16>(p, a, s);
    case kBF16: return cast_fwd_dto<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t cast_bwd_launch(int out_dtype, const LnPlan& p, const CastBwdArgs& a,
                           hipStream_t s) {
  switch (out_dtype) {
    case kF16: return cast_bwd_dto<kF16>(p, a, s);
    case kBF16: return cast_bwd_dto<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
