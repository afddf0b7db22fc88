// RMSNorm with the residual add fused before it (the page "PyTorch
// torch.compile ... LayerNorm and RMSNorm", introduction: a normalisation
// kernel gains from fusing the operations around it; in a transformer block
// the sublayer output is added to the residual stream right before the norm).
//
//   forward   h = T(x + res)   (float32 sum of the widened operands, rounded
//                               to nearest even once: the dtype's own add)
//             y = (h*r)*g,  r = 1/sqrt(sum(h^2)/N + eps),  g = gamma or 1 + w
//   backward  u = dy*g,  c = sum(u*h)/N
//             dx = (r*u - h*(r^3*c)) + dh    (the gradient of x and of res;
//                                             dh, the gradient arriving on h
//                                             from the residual stream, may
//                                             be absent)
//             dgamma += dy*h*r               (column sums over rows)
//
// One pass over each operand: the unfused pair (an add kernel, then the
// norm) reads x and res, writes h, then reads h again; the backward's
// separate add would read dx back.  The norm arithmetic is that of the
// RMSNorm kernels; the row handling is the row-resident layout of rowres.hpp.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"
#include "rmsnorm_launch.hpp"
#include "rowres.hpp"

namespace rmsnorm_hip {
namespace {

using namespace rowres;

// BLK: 256 for 256-thread workgroups (at least 3 wavefronts per SIMD, up to
// 168 VGPRs), else 1024 (512- and 1024-thread workgroups, 128 VGPRs).
template <int DT, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void add_rms_fwd_kernel(
    const void* __restrict__ x, const void* __restrict__ res, const void* __restrict__ gamma,
    void* __restrict__ y, void* __restrict__ h, float* __restrict__ rstd, int64_t M, int N,
    int chunks, int wpr, float eps, int offset, int64_t ldx, int64_t ldr, int64_t ldy,
    int64_t ldh) {
  using PK = Pack<DT, VEC>;
  constexpr int R = rows_per_step<DT, VEC, MAXC, 2, BLK>();
  __shared__ float slots[2 * kRowWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  PK g[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * rg.tpr + rg.t) * VEC;
    g[c].zero();
    if (c < chunks && e < N) ld<DT, VEC, false>(g[c], static_cast<const char*>(gamma), e);
  }
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * step; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * step) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    int64_t row[R];
    bool active[R];
    PK xv[R][MAXC], rv[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = row0 + j * rg.G + rg.group;
      active[j] = row[j] < M;
      const char* xr = row_base<DT>(x, row[j], ldx);
      const char* rr = row_base<DT>(res, row[j], ldr);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        xv[j][c].zero();
        rv[j][c].zero();
        if (active[j] && c < chunks && e < N) {
          ld<DT, VEC, true>(xv[j][c], xr, e);
          ld<DT, VEC, true>(rv[j][c], rr, e);
        }
      }
    }
    // h in the dtype; the norm works on the rounded h, as the unfused model
    // normalises the tensor its add produced.
    PK hv[R][MAXC];
    float ss[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const char* hr = row_base<DT>(h, row[j], ldh);
      ss[j] = 0.f;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        float sum[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) sum[k] = xv[j][c].get(k) + rv[j][c].get(k);
        hv[j][c].set(sum);
        const int e = (c * rg.tpr + rg.t) * VEC;
        // h is stored cacheably: the backward reads it again
        if (active[j] && c < chunks && e < N) st<DT, VEC, false>(hv[j][c], hr, e);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float f = hv[j][c].get(k);
          ss[j] = fmaf(f, f, ss[j]);
        }
      }
    }
    row_sums<0, R, 1, R>(nullptr, ss, nullptr, slots, parity, wpr, rg);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float r = 1.0f / sqrtf(ss[j] / n_f + eps);
      if (!active[j]) continue;
      if (rg.t == 0) rstd[row[j]] = r;
      const char* yr = row_base<DT>(y, row[j], ldy);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = (hv[j][c].get(k) * r) * weight_of(g[c].get(k), offset);
          PK out;
          out.set(o);
          st<DT, VEC>(out, yr, e);
        }
      }
    }
  }
}

template <int DT, int VEC, int MAXC, int BLK>
__global__ __launch_bounds__(BLK, BLK == 256 ? 3 : 1) void add_rms_bwd_kernel(
    const void* __restrict__ dy, const void* __restrict__ dh, const void* __restrict__ h,
    const void* __restrict__ gamma, const float* __restrict__ rstd, void* __restrict__ dx,
    float* __restrict__ part, int64_t M, int N, int chunks, int wpr, int64_t P, int offset,
    int64_t lddy, int64_t lddh, int64_t ldh, int64_t lddx) {
  using PK = Pack<DT, VEC>;
  constexpr int R = rows_per_step<DT, VEC, MAXC, 3, BLK>();
  extern __shared__ __align__(16) float comb[];  // [blockDim.x * VEC] when G > 1
  __shared__ float slots[2 * kRowWaves * R];
  const RowGeom rg = row_geom(wpr);
  const float n_f = static_cast<float>(N);
  int parity = 0;
  // Steps of G*R consecutive rows; workgroup w takes steps w, w+P, w+2P, ...
  // counted from the last step (one contiguous window of the matrices at a
  // time across the grid, from the rows whose h the forward wrote last and
  // left in cache back to the first), and each row group adds its rows to
  // the column sums in step order, row order within a step.
  const int64_t w = blockIdx.x;
  const int64_t step = static_cast<int64_t>(rg.G) * R;
  const int64_t nsteps = (M + step - 1) / step;
  const int64_t iters = w < nsteps ? (nsteps - w + P - 1) / P : 0;
  const bool has_dh = dh != nullptr;
  PK g[MAXC];
  float acc[MAXC][VEC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * rg.tpr + rg.t) * VEC;
    g[c].zero();
    if (c < chunks && e < N) ld<DT, VEC, false>(g[c], static_cast<const char*>(gamma), e);
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    int64_t row[R];
    bool active[R];
    float r[R];
    PK dv[R][MAXC], hv[R][MAXC], ev[R][MAXC];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      row[j] = (nsteps - 1 - (it * P + w)) * step + j * rg.G + rg.group;
      active[j] = row[j] < M;
      r[j] = active[j] ? rstd[row[j]] : 0.f;
      const char* dyr = row_base<DT>(dy, row[j], lddy);
      const char* hr = row_base<DT>(h, row[j], ldh);
      const char* dhr = has_dh ? row_base<DT>(dh, row[j], lddh) : nullptr;
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        dv[j][c].zero();
        hv[j][c].zero();
        ev[j][c].zero();
        if (active[j] && c < chunks && e < N) {
          ld<DT, VEC, true>(dv[j][c], dyr, e);
          ld<DT, VEC, true>(hv[j][c], hr, e);
          if (has_dh) ld<DT, VEC, true>(ev[j][c], dhr, e);
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
          dot[j] = fmaf(dv[j][c].get(k) * weight_of(g[c].get(k), offset), hv[j][c].get(k), dot[j]);
    }
    row_sums<0, R, 1, R>(nullptr, dot, nullptr, slots, parity, wpr, rg);
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
      for (int j = 0; j < R; ++j) {
        dv[j][c].opaque();
        hv[j][c].opaque();
        ev[j][c].opaque();
      }
    // Rows in order (j = 0, 1, ...), so each column sum adds its rows in
    // row order.
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (!active[j]) continue;
      const float r3c = ((r[j] * r[j]) * r[j]) * (dot[j] / n_f);
      const char* dxr = row_base<DT>(dx, row[j], lddx);
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * rg.tpr + rg.t) * VEC;
        if (c < chunks && e < N) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float hf = hv[j][c].get(k);
            const float dyf = dv[j][c].get(k);
            const float u = dyf * weight_of(g[c].get(k), offset);
            o[k] = fmaf(-hf, r3c, r[j] * u) + ev[j][c].get(k);
            acc[c][k] = fmaf(dyf * hf, r[j], acc[c][k]);
          }
          PK out;
          out.set(o);
          st<DT, VEC>(out, dxr, e);
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

template <int DT, int VEC, int MAXC>
hipError_t add_fwd_maxc(const LnPlan& p, const AddFwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  auto* k = p.block == 256 ? add_rms_fwd_kernel<DT, VEC, MAXC, 256>
                           : add_rms_fwd_kernel<DT, VEC, MAXC, 1024>;
  return launch(k, p.grid, p.block, 0, s, a.x, a.res, a.gamma, a.y, a.h, a.rstd, a.M, a.N,
                p.chunks, p.wpr, a.eps, a.offset, a.x_pitch / es, a.res_pitch / es,
                a.y_pitch / es, a.h_pitch / es);
}

template <int DT, int VEC, int MAXC>
hipError_t add_bwd_maxc(const LnPlan& p, const AddBwdArgs& a, hipStream_t s) {
  constexpr int es = ElemBytes<DT>::value;
  auto* k = p.block == 256 ? add_rms_bwd_kernel<DT, VEC, MAXC, 256>
                           : add_rms_bwd_kernel<DT, VEC, MAXC, 1024>;
  return launch(k, p.grid, p.block, static_cast<size_t>(p.lds), s, a.dy, a.dh, a.h, a.gamma,
                a.rstd, a.dx, a.part, a.M, a.N, p.chunks, p.wpr, p.grid, a.offset,
                a.dy_pitch / es, a.dh_pitch / es, a.h_pitch / es, a.dx_pitch / es);
}

template <int DT>
hipError_t add_fwd_dt(const LnPlan& p, const AddFwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(add_fwd_maxc, DT, false, p, a, s);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t add_bwd_dt(const LnPlan& p, const AddBwdArgs& a, hipStream_t s) {
  ROWRES_VEC_SWITCH(add_bwd_maxc, DT, true, p, a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t add_fwd_launch(int dtype, const LnPlan& p, const AddFwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return add_fwd_dt<kF32>(p, a, s);
    case kF16: return add_fwd_dt<kF16>(p, a, s);
    case kBF16: return add_fwd_dt<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t add_bwd_launch(int dtype, const LnPlan& p, const AddBwdArgs& a, hipStream_t s) {
  switch (dtype) {
    case kF32: return add_bwd_dt<kF32>(p, a, s);
    case kF16: return add_bwd_dt<kF16>(p, a, s);
    case kBF16: return add_bwd_dt<kBF16>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
