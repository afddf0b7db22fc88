// LayerNorm backward stage 1 for full-width rows of 4-8 KiB (bf16/fp16
// 2048 < N <= 4096, float32 1024 < N <= 2048 with 16-byte rows and
// pointers), on the row geometry of RMSNorm's bwd_fast_kernel: four
// wavefronts per row, two 16-byte chunks per lane, two rows side by side in
// a 512-thread workgroup, x staged in LDS by DMA and dy in registers.
//
// Same arithmetic as the row-resident ln_bwd_kernel (page "PyTorch
// torch.compile ... LayerNorm and RMSNorm", section 2: dx, dgamma and dbeta
// from xhat and u = dy*gamma):
//   d = x - mean;  sums of u, u*d and d over the row (one exchange)
//   cm = sum(d)/N  (the offset between the exact and the float32 mean)
//   c1 = sum(u)/N;  c2 = r*(sum(u*d) - cm*sum(u))/N;  xhat = (d - cm)*r
//   dx = r*((u - c1) - xhat*c2);  dgamma += dy*xhat;  dbeta += dy
// Workgroup w takes the row groups of its RowSched order (the whole grid
// sweeps one window of the matrices from the last row to the first, the
// reverse of the forward's sweep) and accumulates dgamma and dbeta columns
// in float32 registers, each row group adding its rows in row order; the
// two groups are combined in group order through LDS into part[w, :]
// (dgamma) and part[P + w, :] (dbeta).  Stage 2 is unchanged.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_fast.hpp"
#include "rmsnorm_launch.hpp"

namespace rmsnorm_hip {
namespace {

// K row sums across the WPR wavefronts of a row group with one workgroup
// barrier.  slots: [2][G][WPR][K] floats; parity alternates between calls.
template <int WPR, int G, int K>
__device__ __forceinline__ void group_sums(float (&v)[K], float* slots, int& parity, int group,
                                           int wave_in_row, int lane) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum(v[k]);
  if constexpr (WPR > 1) {
    float* s = slots + (parity * G + group) * WPR * K;
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) s[wave_in_row * K + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float t = s[k];
#pragma unroll
      for (int i = 1; i < WPR; ++i) t += s[i * K + k];
      v[k] = t;
    }
    parity ^= 1;
  }
}

template <int DT, int CH, int WPR, int BLOCK, int ORD>
__global__ __launch_bounds__(BLOCK) void ln_bwd_rows_kernel(
    const void* __restrict__ dy, const void* __restrict__ x, const void* __restrict__ gamma,
    const float* __restrict__ mean, const float* __restrict__ rstd, void* __restrict__ dx,
    float* __restrict__ part, int64_t M, int N, int64_t P, int64_t dy_pitch, int64_t x_pitch,
    int64_t dx_pitch) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, G = Geo::G, SWEEP = Geo::SWEEP;
  constexpr uint32_t kChunk = TPR * 16;
  using PK = Pack<DT, VEC>;
  // [G][N] elements of x while the rows run; afterwards [G][SWEEP] float32
  // for the combine.
  extern __shared__ __align__(16) char dyn[];
  __shared__ float slots[WPR > 1 ? 2 * G * WPR * 3 : 1];
  const int t = threadIdx.x % TPR;
  const int group = uniform(static_cast<int>(threadIdx.x / TPR));
  const int wave_in_row = uniform(t / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  int parity = 0;
  const int64_t w = blockIdx.x;
  const RowSched<ORD> rs(w, M, P, G);
  const float inv_n = 1.0f / static_cast<float>(N);
  char* xrow = dyn + static_cast<int64_t>(group) * row_bytes;
  // only the last chunk can reach past the row
  auto in_row = [&](int c) __attribute__((always_inline)) {
    return c < CH - 1 || voff + c * kChunk < row_bytes;
  };

  // gamma widened once; the row's deviations d = x - mean, u = dy*gamma and
  // dy stay in float32 registers between the two sweeps (x is read from
  // LDS once), so the second sweep converts nothing.
  const GRow gbuf(gamma);
  float gf[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    PK gv;
    if (in_row(c)) gv.raw = gbuf.template load<false>(voff, c * kChunk);
    else gv.zero();
#pragma unroll
    for (int k = 0; k < VEC; ++k) gf[c][k] = gv.get(k);
  }
  float ag[CH][VEC], ab[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) ag[c][k] = ab[c][k] = 0.f;

  for (int64_t it = 0; it < rs.iters; ++it) {
    const int64_t row = rs.base + it * rs.stride + group;
    const bool active = row < rs.limit;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int k = 0; k < VEC; ++k) asm volatile("" : "+v"(gf[c][k]));
    PK dv[CH];
    float mu = 0.f, r = 0.f;
    if (active) {
      mu = mean[row];
      r = rstd[row];
      const GRow xb(static_cast<const char*>(x) + row * x_pitch);
      const GRow db(static_cast<const char*>(dy) + row * dy_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (in_row(c)) {
          dv[c].raw = db.template load<true>(voff, c * kChunk);
          xb.to_lds(xrow + c * kChunk + wave_in_row * kWave * 16, voff, c * kChunk);
        } else {
          dv[c].zero();
        }
      }
      // The DMA is not tracked by the compiler: wait for it (and the rest)
      // before the LDS reads.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) dv[c].zero();
    }
    float sums[3] = {0.f, 0.f, 0.f};
    float d[CH][VEC], u[CH][VEC], dyf[CH][VEC];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      PK xc;
      if (active && in_row(c)) xc.raw = *reinterpret_cast<const u32x4*>(xrow + c * kChunk + voff);
      else xc.zero();
      float td = 0.f;
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        dyf[c][k] = dv[c].get(k);
        d[c][k] = xc.get(k) - mu;
        u[c][k] = dyf[c][k] * gf[c][k];
        sums[0] += u[c][k];
        sums[1] = fmaf(u[c][k], d[c][k], sums[1]);
        td += d[c][k];
      }
      // lanes past the row hold d = -mean: left out of sum(d)
      if (in_row(c)) sums[2] += td;
      chunk_fence();
    }
    group_sums<WPR, G, 3>(sums, slots, parity, group, wave_in_row, lane);
    if (active) {
      const float cm = sums[2] * inv_n;
      const float c1 = sums[0] * inv_n;
      const float c2 = (r * (sums[1] - cm * sums[0])) * inv_n;
      const float rcm = r * cm;
      const GRow ob(static_cast<char*>(dx) + row * dx_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (in_row(c)) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float xh = fmaf(d[c][k], r, -rcm);
            o[k] = r * fmaf(-xh, c2, u[c][k] - c1);
            ag[c][k] = fmaf(dyf[c][k], xh, ag[c][k]);
            ab[c][k] += dyf[c][k];
          }
          PK out;
          out.set(o);
          ob.template store<true>(out.raw, voff, c * kChunk);
        }
        chunk_fence();
      }
    }
  }

  // Fixed-order combine of the G groups, one chunk sweep (SWEEP columns) at
  // a time: part[which*P + w, col] = ((acc_0 + acc_1) + acc_2) + ...
  float* comb = reinterpret_cast<float*>(dyn);
  __syncthreads();  // the LDS area still holds staged rows
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float* dst = part + (which * P + w) * static_cast<int64_t>(N);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if constexpr (G == 1) {
        const int e = (c * TPR + t) * VEC;
        if (c < CH - 1 || e < N) store_f32<VEC>(dst + e, which ? ab[c] : ag[c]);
      } else {
        store_f32<VEC>(comb + group * SWEEP + t * VEC, which ? ab[c] : ag[c]);
        __syncthreads();
        for (int j = threadIdx.x; j < SWEEP; j += BLOCK) {
          const int col = c * SWEEP + j;
          if (col < N) {
            float s = comb[j];
#pragma unroll
            for (int gi = 1; gi < G; ++gi) s += comb[gi * SWEEP + j];
            dst[col] = s;
          }
        }
        __syncthreads();
      }
    }
  }
}

template <int DT>
hipError_t ln_bwd_rows_dt(int64_t P, int64_t lds, const LnBwdArgs& a, hipStream_t s) {
  // 16-byte rows that fill more than the first of the two chunk sweeps (only
  // the last may be partial), and LDS for both rows of x.
  constexpr int64_t kSweepBytes = 4 * kWave * 16;
  const int64_t row_bytes = int64_t(a.N) * ElemBytes<DT>::value;
  if (row_bytes % 16 != 0 || row_bytes <= kSweepBytes || row_bytes > 2 * kSweepBytes ||
      lds < 2 * row_bytes || P < 1)
    return hipErrorInvalidValue;
  return launch(ln_bwd_rows_kernel<DT, 2, 4, 512, kRowsReverse>, P, 512,
                static_cast<size_t>(lds), s, a.dy, a.x, a.gamma, a.mean, a.rstd, a.dx, a.part,
                a.M, a.N, P, a.dy_pitch, a.x_pitch, a.dx_pitch);
}

}  // namespace

hipError_t ln_bwd_rows_launch(int dtype, int64_t P, int64_t lds, const LnBwdArgs& a,
                              hipStream_t s) {
  switch (dtype) {
    case kF32: return ln_bwd_rows_dt<kF32>(P, lds, a, s);
    case kF16: return ln_bwd_rows_dt<kF16>(P, lds, a, s);
    case kBF16: return ln_bwd_rows_dt<kBF16>(P, lds, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rmsnorm_hip
