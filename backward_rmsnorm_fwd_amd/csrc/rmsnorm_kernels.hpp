// RMSNorm forward / backward kernels for gfx950 (CDNA4, wave64).
//
// Math (page "Check an AI model calculation before accelerating it",
// sections "Problem and reference formula" and "Input backward pass: keep the
// right N"): r = 1/sqrt(mean(x^2) + eps), y = x*r*g; u = dy*g,
// dx = r*u - x*r^3*mean(u*x), dgamma = sum over rows of dy*x*r.
//
// Layout of work:
//  * A row is split into `chunks` vector accesses per thread.  Thread t of the
//    row's threads covers elements (c*tpr + t)*VEC .. +VEC-1 for chunk c, so
//    each chunk is one fully coalesced sweep of tpr*VEC*sizeof(T) bytes.
//  * Elements past N are loaded as 0 (they add nothing to the sums) and never
//    stored; the mean divides by the logical N.
//  * Values are widened to float32 as they leave the load, before squaring.
//  * Row sums: per-lane float32 FMA chain -> wave64 butterfly with DPP adds
//    (quad_perm, half-row mirror, row mirror) -> 4 readlanes summed in a fixed
//    order -> (workgroup-per-row only) an LDS exchange between wavefronts,
//    summed in wavefront order.  Every lane gets the same bits.
//  * Backward: each workgroup owns a fixed, contiguous block of rows (a pure
//    function of M and the number of workgroups P), accumulates dy*x*r per
//    column in float32 registers, combines its row groups in a fixed order
//    and stores one [N] partial row.  A second kernel adds the P partials per
//    column in float64, in order.  No atomics: results are reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsnorm_hip {

typedef uint32_t u32;
typedef uint16_t u16;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxWavesPerBlock = 16;

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2 };

template <int DT>
struct ElemBytes { static constexpr int value = (DT == kF32) ? 4 : 2; };

template <int BYTES> struct RawOf;
template <> struct RawOf<16> { using type = u32x4; };
template <> struct RawOf<8> { using type = u32x2; };
template <> struct RawOf<4> { using type = u32; };
template <> struct RawOf<2> { using type = u16; };

// VEC elements of dtype DT, kept in storage format (packed) in registers.
template <int DT, int VEC>
struct Pack {
  static constexpr int kBytes = VEC * ElemBytes<DT>::value;
  using raw_t = typename RawOf<kBytes>::type;
  raw_t raw;

  __device__ __forceinline__ void zero() { raw = raw_t(0); }

  // Optimization barrier: the compiler must assume `raw` changed here, so it
  // re-widens elements from the packed registers after this point instead of
  // hoisting or keeping all the widened float32 copies alive (which doubles
  // the register footprint and spills).
  __device__ __forceinline__ void opaque() {
    if constexpr (kBytes == 2) {
      u32 v = raw;
      asm volatile("" : "+v"(v));
      raw = static_cast<raw_t>(v);
    } else {
      asm volatile("" : "+v"(raw));
    }
  }

  __device__ __forceinline__ void load(const void* base, int64_t elem) {
    raw = *reinterpret_cast<const raw_t*>(
        static_cast<const char*>(base) + elem * ElemBytes<DT>::value);
  }
  __device__ __forceinline__ void store(void* base, int64_t elem) const {
    *reinterpret_cast<raw_t*>(static_cast<char*>(base) +
                              elem * ElemBytes<DT>::value) = raw;
  }
  // Streaming variants: the data is touched once, so hint the caches not to
  // keep it (nontemporal loads/stores).
  template <bool NT>
  __device__ __forceinline__ void load_s(const void* base, int64_t elem) {
    const raw_t* p = reinterpret_cast<const raw_t*>(
        static_cast<const char*>(base) + elem * ElemBytes<DT>::value);
    if constexpr (NT) raw = __builtin_nontemporal_load(p);
    else raw = *p;
  }
  template <bool NT>
  __device__ __forceinline__ void store_s(void* base, int64_t elem) const {
    raw_t* p = reinterpret_cast<raw_t*>(static_cast<char*>(base) +
                                        elem * ElemBytes<DT>::value);
    if constexpr (NT) __builtin_nontemporal_store(raw, p);
    else *p = raw;
  }

  __device__ __forceinline__ u32 word(int w) const {
    if constexpr (kBytes >= 8) return raw[w];
    else return static_cast<u32>(raw);
  }
  __device__ __forceinline__ void set_word(int w, u32 v) {
    if constexpr (kBytes >= 8) raw[w] = v;
    else raw = static_cast<raw_t>(v);
  }

  // Element k widened to float32 (exact for every dtype).
  __device__ __forceinline__ float get(int k) const {
    if constexpr (DT == kF32) {
      return __builtin_bit_cast(float, word(k));
    } else if constexpr (DT == kBF16) {
      const u32 w = word(k >> 1);
      return __builtin_bit_cast(float, (k & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      if constexpr (kBytes == 2) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<u16>(raw)));
      } else {
        const f16x2 h = __builtin_bit_cast(f16x2, word(k >> 1));
        return static_cast<float>(h[k & 1]);
      }
    }
  }

  // Round VEC float32 values to dtype DT (nearest even) and pack them.
  __device__ __forceinline__ void set(const float (&f)[VEC]) {
    if constexpr (DT == kF32) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) set_word(k, __builtin_bit_cast(u32, f[k]));
    } else if constexpr (VEC == 1) {
      if constexpr (DT == kBF16)
        raw = __builtin_bit_cast(u16, static_cast<__bf16>(f[0]));
      else
        raw = __builtin_bit_cast(u16, static_cast<_Float16>(f[0]));
    } else {
#pragma unroll
      for (int k = 0; k < VEC; k += 2) {
        const f32x2 v = {f[k], f[k + 1]};
        if constexpr (DT == kBF16)
          set_word(k >> 1, __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2)));
        else
          set_word(k >> 1, __builtin_bit_cast(u32, __builtin_convertvector(v, f16x2)));
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, true));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes of a wavefront; every lane receives the same bits.
// Must be called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror: 8-lane sums
  v += dpp_move<0x140>(v);  // row_mirror: 16-lane sums
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Sum over the `nwaves` wavefronts of a workgroup (all threads must call it,
// the same number of times).  `slots` is a [2][kMaxWavesPerBlock] LDS array;
// `parity` alternates between calls so one barrier per call suffices.
__device__ __forceinline__ float block_sum(float v, float* slots, int& parity,
                                           int wave, int nwaves, int lane) {
  v = wave_sum(v);
  if (nwaves == 1) return v;
  float* s = slots + parity * kMaxWavesPerBlock;
  if (lane == 0) s[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nwaves; ++w) t += s[w];
  parity ^= 1;
  return t;
}

__device__ __forceinline__ float weight_of(float w, int offset) {
  // One add per use: the uniform bias (1 or 0) is selected once per kernel.
  // w + 0 equals w except that a weight of -0 is read as +0, so the zero
  // products it scales may come out with the other sign (equal in value).
  return w + (offset ? 1.0f : 0.0f);
}

// ---------------------------------------------------------------------------
// Forward, one wavefront per row.  Each workgroup of G wavefronts walks rows
// blockIdx.x*G + g, then strides by gridDim.x*G; the weight stays in
// registers for all of them.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int MAXC>
__global__ __launch_bounds__(256) void fwd_wave_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma,
    void* __restrict__ y, float* __restrict__ rstd, int64_t M, int N,
    int chunks, float eps, int offset, int64_t ldx, int64_t ldy) {
  using P = Pack<DT, VEC>;
  const int lane = threadIdx.x & (kWave - 1);
  const int group = threadIdx.x / kWave;
  const int groups = blockDim.x / kWave;

  P g[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * kWave + lane) * VEC;
    if (c < chunks && e < N) g[c].load(gamma, e);
    else g[c].zero();
  }
  const float n_f = static_cast<float>(N);

  for (int64_t row = static_cast<int64_t>(blockIdx.x) * groups + group; row < M;
       row += static_cast<int64_t>(gridDim.x) * groups) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    P xv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * kWave + lane) * VEC;
      if (c < chunks && e < N) xv[c].load(x, row * ldx + e);
      else xv[c].zero();
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c < chunks) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float f = xv[c].get(k);
          ss = fmaf(f, f, ss);
        }
      }
    }
    ss = wave_sum(ss);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) xv[c].opaque();
    const float r = 1.0f / sqrtf(ss / n_f + eps);
    if (lane == 0) rstd[row] = r;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * kWave + lane) * VEC;
      if (c < chunks && e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          o[k] = (xv[c].get(k) * r) * weight_of(g[c].get(k), offset);
        P out;
        out.set(o);
        out.store(y, row * ldy + e);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Forward, one workgroup per row (long rows).  x stays in registers between
// the reduction and the scale pass; the weight is re-read (cache resident).
// ---------------------------------------------------------------------------
template <int DT, int VEC, int MAXC>
__global__ __launch_bounds__(1024) void fwd_block_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma,
    void* __restrict__ y, float* __restrict__ rstd, int64_t M, int N,
    int chunks, float eps, int offset, int64_t ldx, int64_t ldy) {
  using P = Pack<DT, VEC>;
  __shared__ float slots[2 * kMaxWavesPerBlock];
  const int tpr = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int nwaves = tpr / kWave;
  int parity = 0;
  const float n_f = static_cast<float>(N);

  for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
    P xv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * tpr + t) * VEC;
      if (c < chunks && e < N) xv[c].load(x, row * ldx + e);
      else xv[c].zero();
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c < chunks) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float f = xv[c].get(k);
          ss = fmaf(f, f, ss);
        }
      }
    }
    ss = block_sum(ss, slots, parity, wave, nwaves, lane);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) xv[c].opaque();
    const float r = 1.0f / sqrtf(ss / n_f + eps);
    if (t == 0) rstd[row] = r;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * tpr + t) * VEC;
      if (c < chunks && e < N) {
        P gv;
        gv.load(gamma, e);
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          o[k] = (xv[c].get(k) * r) * weight_of(gv.get(k), offset);
        P out;
        out.set(o);
        out.store(y, row * ldy + e);
      }
    }
  }
}

// Store VEC float32 values (columns e..e+VEC-1) with the widest aligned stores.
template <int VEC>
__device__ __forceinline__ void store_f32(float* p, const float (&v)[VEC]) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      const f32x4 q = {v[k], v[k + 1], v[k + 2], v[k + 3]};
      *reinterpret_cast<f32x4*>(p + k) = q;
    }
  } else if constexpr (VEC == 2) {
    const f32x2 q = {v[0], v[1]};
    *reinterpret_cast<f32x2*>(p) = q;
  } else {
    p[0] = v[0];
  }
}

template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float (&v)[VEC]) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int k = 0; k < VEC; k += 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(p + k);
      v[k] = q[0]; v[k + 1] = q[1]; v[k + 2] = q[2]; v[k + 3] = q[3];
    }
  } else if constexpr (VEC == 2) {
    const f32x2 q = *reinterpret_cast<const f32x2*>(p);
    v[0] = q[0]; v[1] = q[1];
  } else {
    v[0] = p[0];
  }
}

// First row of workgroup w's block when M rows are split over P workgroups.
__device__ __forceinline__ int64_t block_row_begin(int64_t w, int64_t M, int64_t P) {
  return (w * M) / P;
}

// ---------------------------------------------------------------------------
// Backward stage 1, one wavefront per row.  Workgroup w owns rows
// [w*M/P, (w+1)*M/P); its G wavefronts take them round-robin.  Per row:
// dot = sum(dy*g*x) (wave reduction), dx = r*u - x*(r^3*dot/N), and
// acc_j += (dy_j*x_j)*r.  At the end the G accumulators are added in
// wavefront order through LDS and the last wavefront stores the partial row.
// ---------------------------------------------------------------------------
template <int DT, int VEC, int MAXC>
__global__ __launch_bounds__(512) void bwd_wave_kernel(
    const void* __restrict__ dy, const void* __restrict__ x,
    const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ dx, float* __restrict__ part, int64_t M, int N,
    int chunks, int offset, int64_t P, int64_t lddy, int64_t ldx, int64_t lddx) {
  using PK = Pack<DT, VEC>;
  extern __shared__ float comb[];  // [N] running sum of the groups' partials
  const int lane = threadIdx.x & (kWave - 1);
  const int group = threadIdx.x / kWave;
  const int groups = blockDim.x / kWave;
  const int64_t w = blockIdx.x;
  const int64_t r0 = block_row_begin(w, M, P);
  const int64_t r1 = block_row_begin(w + 1, M, P);
  const float n_f = static_cast<float>(N);

  PK g[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * kWave + lane) * VEC;
    if (c < chunks && e < N) g[c].load(gamma, e);
    else g[c].zero();
  }
  float acc[MAXC][VEC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;

  for (int64_t row = r0 + group; row < r1; row += groups) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) g[c].opaque();
    PK xv[MAXC], dv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * kWave + lane) * VEC;
      if (c < chunks && e < N) {
        xv[c].load(x, row * ldx + e);
        dv[c].load(dy, row * lddy + e);
      } else {
        xv[c].zero();
        dv[c].zero();
      }
    }
    const float r = rstd[row];
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      if (c < chunks) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float u = dv[c].get(k) * weight_of(g[c].get(k), offset);
          dot = fmaf(u, xv[c].get(k), dot);
        }
      }
    }
    dot = wave_sum(dot);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      xv[c].opaque();
      dv[c].opaque();
      g[c].opaque();
    }
    const float r3c = ((r * r) * r) * (dot / n_f);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * kWave + lane) * VEC;
      if (c < chunks && e < N) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float xf = xv[c].get(k);
          const float dyf = dv[c].get(k);
          const float u = dyf * weight_of(g[c].get(k), offset);
          o[k] = fmaf(-xf, r3c, r * u);
          acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
        }
        PK out;
        out.set(o);
        out.store(dx, row * lddx + e);
      }
    }
  }

  // Fixed-order combine of the G row groups: ((acc_0 + acc_1) + acc_2) + ...
  float* dst = part + w * static_cast<int64_t>(N);
  for (int gi = 0; gi < groups; ++gi) {
    if (group == gi) {
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = (c * kWave + lane) * VEC;
        if (c < chunks && e < N) {
          float v[VEC];
          if (gi > 0) {
            float prev[VEC];
            load_f32<VEC>(comb + e, prev);
#pragma unroll
            for (int k = 0; k < VEC; ++k) v[k] = prev[k] + acc[c][k];
          } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) v[k] = acc[c][k];
          }
          if (gi == groups - 1) store_f32<VEC>(dst + e, v);
          else store_f32<VEC>(comb + e, v);
        }
      }
    }
    if (gi + 1 < groups) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Backward stage 1, one workgroup per row (long rows).  The row of x is
// staged in LDS (XLDS) or kept in registers, dy stays in registers, the
// weight is re-read from cache, and the dgamma contribution is accumulated
// while the row streams in (r is known before the row reduction).
// ---------------------------------------------------------------------------
template <int DT, int VEC, int MAXC, bool XLDS>
__global__ __launch_bounds__(1024) void bwd_block_kernel(
    const void* __restrict__ dy, const void* __restrict__ x,
    const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ dx, float* __restrict__ part, int64_t M, int N,
    int chunks, int offset, int64_t P, int64_t lddy, int64_t ldx, int64_t lddx) {
  using PK = Pack<DT, VEC>;
  extern __shared__ __align__(16) char xrow[];  // [N] elements of x when XLDS
  __shared__ float slots[2 * kMaxWavesPerBlock];
  const int tpr = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const int nwaves = tpr / kWave;
  int parity = 0;
  const int64_t w = blockIdx.x;
  const int64_t r0 = block_row_begin(w, M, P);
  const int64_t r1 = block_row_begin(w + 1, M, P);
  const float n_f = static_cast<float>(N);

  float acc[MAXC][VEC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;

  for (int64_t row = r0; row < r1; ++row) {
    PK dv[MAXC];
    PK xv[XLDS ? 1 : MAXC];
    const float r = rstd[row];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * tpr + t) * VEC;
      PK& xc = xv[XLDS ? 0 : c];
      if (c < chunks && e < N) {
        xc.load(x, row * ldx + e);
        dv[c].load(dy, row * lddy + e);
        if constexpr (XLDS) xc.store(xrow, e);
      } else {
        xc.zero();
        dv[c].zero();
      }
    }
    // Second sweep over registers so the loads above are all in flight
    // before the first use.
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * tpr + t) * VEC;
      if (c < chunks && e < N) {
        PK xc;
        if constexpr (XLDS) xc.load(xrow, e);
        else xc = xv[c];
        PK gv;
        gv.load(gamma, e);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float xf = xc.get(k);
          const float dyf = dv[c].get(k);
          dot = fmaf(dyf * weight_of(gv.get(k), offset), xf, dot);
          acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
        }
      }
    }
    dot = block_sum(dot, slots, parity, wave, nwaves, lane);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      dv[c].opaque();
      if constexpr (!XLDS) xv[c].opaque();
    }
    const float r3c = ((r * r) * r) * (dot / n_f);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = (c * tpr + t) * VEC;
      if (c < chunks && e < N) {
        PK xc;
        if constexpr (XLDS) xc.load(xrow, e);
        else xc = xv[c];
        PK gv;
        gv.load(gamma, e);
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float u = dv[c].get(k) * weight_of(gv.get(k), offset);
          o[k] = fmaf(-xc.get(k), r3c, r * u);
        }
        PK out;
        out.set(o);
        out.store(dx, row * lddx + e);
      }
    }
  }

  float* dst = part + w * static_cast<int64_t>(N);
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = (c * tpr + t) * VEC;
    if (c < chunks && e < N) store_f32<VEC>(dst + e, acc[c]);
  }
}

// ---------------------------------------------------------------------------
// Backward stage 2: dgamma[j] = sum_{p<P} part[p][j] in float64, fixed order.
// A workgroup covers 64 columns; its S = blockDim.x/64 slices take partial
// rows p = s, s+S, ...; the slices are then added in slice order.
// ---------------------------------------------------------------------------
// dgamma output type of stage 2: float32, or the input dtype (kF16/kBF16/kF32)
// rounded to nearest even from the float32 value.
constexpr int kOutF32 = -1;

template <int OUT>
__device__ __forceinline__ void store_dgamma(void* dgamma, int64_t j, double tot) {
  // The float32 value is materialised first: the compiler may not fold the
  // two conversions into one rounding from float64 (which differs when the
  // float32 value falls exactly halfway between two values of T).
  float f32 = static_cast<float>(tot);
  asm volatile("" : "+v"(f32));
  const float f[1] = {f32};
  if constexpr (OUT == kOutF32) {
    static_cast<float*>(dgamma)[j] = f[0];
  } else {
    Pack<OUT, 1> v;
    v.set(f);
    v.store(dgamma, j);
  }
}

template <int OUT>
static __global__ __launch_bounds__(1024) __attribute__((unused)) void bwd_reduce_kernel(
    const float* __restrict__ part, void* __restrict__ dgamma, int64_t P, int N,
    const float* __restrict__ part_b, void* __restrict__ dgamma_b) {
  __shared__ double sums[kMaxWavesPerBlock][kWave];
  // A second [P, N] block (part_b, for LayerNorm's dbeta): the grid's
  // second half reduces it into dgamma_b, the same way.
  int bx = static_cast<int>(blockIdx.x);
  if (part_b != nullptr && bx >= static_cast<int>(gridDim.x / 2)) {
    bx -= static_cast<int>(gridDim.x / 2);
    part = part_b;
    dgamma = dgamma_b;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int s = threadIdx.x / kWave;
  const int S = blockDim.x / kWave;
  const int col = bx * kWave + lane;
  double acc = 0.0;
  if (col < N) {
    for (int64_t p = s; p < P; p += S)
      acc += static_cast<double>(part[p * N + col]);
  }
  sums[s][lane] = acc;
  __syncthreads();
  if (s == 0 && col < N) {
    double tot = 0.0;
    for (int i = 0; i < S; ++i) tot += sums[i][lane];
    store_dgamma<OUT>(dgamma, col, tot);
  }
}

}  // namespace rmsnorm_hip
