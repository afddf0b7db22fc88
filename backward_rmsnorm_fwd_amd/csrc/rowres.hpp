// Shared pieces of the row-resident kernels (LayerNorm and the fused
// residual-add RMSNorm): a row spread over `wpr` wavefronts of a workgroup,
// lane t owning vectors c*64*wpr + t, row sums exchanged through LDS, and
// row access through a uniform row base plus an opaque 32-bit lane offset.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"

namespace rmsnorm_hip {
namespace rowres {

constexpr int kRowMaxBlock = 1024;
constexpr int kRowWaves = kRowMaxBlock / kWave;

// ---- row reductions ---------------------------------------------------------
//
// Every sum below is over the wpr wavefronts of one row: each wavefront sums
// its 64 lanes (every lane ends with the same bits), then, when wpr > 1, the
// wavefronts' sums are added in wavefront order through LDS.  `slots` hold
// [2][kRowWaves][K] values; parity alternates so one barrier per exchange
// suffices.  wpr is uniform across the workgroup, so every thread takes the
// same path and reaches the same barriers.

// float64 move between lanes with a DPP control (two 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(b)),
                                             CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(b >> 32)),
                                             CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}

__device__ __forceinline__ double lane_value_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), lane));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// float64 sum over the 64 lanes, in the same pattern as wave_sum.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_move_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move_f64<0x141>(v);  // row_half_mirror: 8-lane sums
  v += dpp_move_f64<0x140>(v);  // row_mirror: 16-lane sums
  return (lane_value_f64(v, 0) + lane_value_f64(v, 16)) +
         (lane_value_f64(v, 32) + lane_value_f64(v, 48));
}

struct RowGeom {
  int tpr, G, t, group, first_wave, wave, lane;
};

__device__ __forceinline__ RowGeom row_geom(int wpr) {
  RowGeom g;
  g.tpr = kWave * wpr;
  g.G = blockDim.x / g.tpr;
  g.t = threadIdx.x % g.tpr;
  g.group = threadIdx.x / g.tpr;
  g.first_wave = g.group * wpr;
  g.wave = threadIdx.x / kWave;
  g.lane = threadIdx.x % kWave;
  return g;
}

// Adds slot[first], ..., slot[first + W - 1] in that order.  With a
// compile-time W every LDS read is issued before the first is needed; W = 0
// takes the count `w` at run time (one read at a time, few registers: the
// wide rows of 512- and 1024-thread workgroups, whose register budget is
// already spent on the row).
template <int W, typename T>
__device__ __forceinline__ T sum_slots(const T* slot, int first, int w) {
  if constexpr (W == 0) {
    T t = slot[first];
    for (int i = 1; i < w; ++i) t += slot[first + i];
    return t;
  } else {
    T v[W];
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = slot[first + i];
    T t = v[0];
#pragma unroll
    for (int i = 1; i < W; ++i) t += v[i];
    return t;
  }
}

template <int W, int KD, int KF>
__device__ __forceinline__ void gather_sums(double* a, float* b, const double* d,
                                            const float* f, int first, int w) {
#pragma unroll
  for (int i = 0; i < KD; ++i) a[i] = sum_slots<W>(d + i * kRowWaves, first, w);
#pragma unroll
  for (int i = 0; i < KF; ++i) b[i] = sum_slots<W>(f + i * kRowWaves, first, w);
}

// KD float64 and KF float32 row sums in one exchange.  The slot arrays are
// [2][SD][kRowWaves] doubles and [2][SF][kRowWaves] floats with the same
// SD >= KD, SF >= KF in every call of a kernel, so the two parity halves are
// disjoint whatever KD and KF are: an exchange writes only the half the
// previous one did not read, and the half it reads is rewritten two
// exchanges later, after a barrier every reader has passed.  Sum i of wave
// w sits at [i][w], so a row's wpr partial sums are adjacent.
template <int KD, int KF, int SD, int SF>
__device__ __forceinline__ void row_sums(double* a, float* b, double* s64, float* s32,
                                         int& parity, int wpr, const RowGeom& rg) {
  static_assert(KD <= SD && KF <= SF, "slot layout");
#pragma unroll
  for (int i = 0; i < KD; ++i) a[i] = wave_sum_f64(a[i]);
#pragma unroll
  for (int i = 0; i < KF; ++i) b[i] = wave_sum(b[i]);
  if (wpr == 1) return;
  double* d = KD > 0 ? s64 + parity * kRowWaves * SD : nullptr;
  float* f = KF > 0 ? s32 + parity * kRowWaves * SF : nullptr;
  if (rg.lane == 0) {
    if constexpr (KD > 0) {
#pragma unroll
      for (int i = 0; i < KD; ++i) d[i * kRowWaves + rg.wave] = a[i];
    }
    if constexpr (KF > 0) {
#pragma unroll
      for (int i = 0; i < KF; ++i) f[i * kRowWaves + rg.wave] = b[i];
    }
  }
  __syncthreads();
  switch (wpr) {  // uniform across the workgroup
    case 2: gather_sums<2, KD, KF>(a, b, d, f, rg.first_wave, 2); break;
    case 4: gather_sums<4, KD, KF>(a, b, d, f, rg.first_wave, 4); break;
    default: gather_sums<0, KD, KF>(a, b, d, f, rg.first_wave, wpr); break;
  }
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

// NT: streaming store (the default); without it the line is cached as
// usual, for data a later kernel reads back.
template <int DT, int VEC, bool NT = true>
__device__ __forceinline__ void st(const Pack<DT, VEC>& v, const char* row, int e) {
  uint32_t off = static_cast<uint32_t>(e) * ElemBytes<DT>::value;
  asm volatile("" : "+v"(off));
  using R = typename Pack<DT, VEC>::raw_t;
  R* a = reinterpret_cast<R*>(const_cast<char*>(row) + off);
  if constexpr (NT) __builtin_nontemporal_store(v.raw, a);
  else *a = v.raw;
}

// Rows each row group takes per step: two when the rows' data fits in 16
// VGPRs per row in 256-thread workgroups (8 in larger ones, whose register
// budget is 128): both rows' loads are then in flight at once and their
// reductions share one exchange.  Else one.
__host__ __device__ constexpr int row_step_rows(int vec_bytes, int maxc, int matrices,
                                                 bool blk256) {
  return maxc * ((vec_bytes + 3) / 4) * matrices <= (blk256 ? 16 : 8) ? 2 : 1;
}

template <int DT, int VEC, int MAXC, int MATRICES, int BLK>
constexpr int rows_per_step() {
  return row_step_rows(VEC * ElemBytes<DT>::value, MAXC, MATRICES, BLK == 256);
}

__host__ __device__ constexpr int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Largest chunk count a row-resident plan gives a vector width (N <= 16384):
// the forward aims at min(4, 32/VEC) chunks, the backward at min(8, 16/VEC),
// and a row of 16384 elements over 16 wavefronts needs 16/VEC.  Only these
// register-slot counts are instantiated.
constexpr int row_cap(int vec, bool backward) {
  const int target = backward ? (16 / vec < 8 ? 16 / vec : 8) : (32 / vec < 4 ? 32 / vec : 4);
  const int need = 16 / vec;
  const int m = target > need ? target : need;
  int p = 1;
  while (p < m) p <<= 1;
  return p;
}

}  // namespace rowres

// Dispatch over the register-slot count (a power of two >= p.chunks) for a
// plan `p`, calling FN<DT, VEC, MAXC>(args...).
#define ROWRES_MAXC_CASE(FN, DT, VEC, BWD, C, ...)                                \
  case C:                                                                       \
    if constexpr (C <= rowres::row_cap(VEC, BWD)) return FN<DT, VEC, C>(__VA_ARGS__); \
    return hipErrorInvalidValue;

#define ROWRES_MAXC_SWITCH(FN, DT, VEC, BWD, ...)         \
  switch (rowres::pow2_ceil(p.chunks)) {                  \
    ROWRES_MAXC_CASE(FN, DT, VEC, BWD, 1, __VA_ARGS__)    \
    ROWRES_MAXC_CASE(FN, DT, VEC, BWD, 2, __VA_ARGS__)    \
    ROWRES_MAXC_CASE(FN, DT, VEC, BWD, 4, __VA_ARGS__)    \
    ROWRES_MAXC_CASE(FN, DT, VEC, BWD, 8, __VA_ARGS__)    \
    ROWRES_MAXC_CASE(FN, DT, VEC, BWD, 16, __VA_ARGS__)   \
    default: return hipErrorInvalidValue;                 \
  }

// The same over the vector width p.vec for dtype DT.
#define ROWRES_VEC_SWITCH(FN, DT, BWD, ...)                                       \
  do {                                                                          \
    constexpr int es_ = ElemBytes<DT>::value;                                   \
    switch (p.vec * es_) {                                                      \
      case 16: ROWRES_MAXC_SWITCH(FN, DT, 16 / es_, BWD, __VA_ARGS__)           \
      case 8: ROWRES_MAXC_SWITCH(FN, DT, 8 / es_, BWD, __VA_ARGS__)             \
      case 4: ROWRES_MAXC_SWITCH(FN, DT, 4 / es_, BWD, __VA_ARGS__)             \
      case 2:                                                                   \
        if constexpr (es_ == 2) {                                               \
          ROWRES_MAXC_SWITCH(FN, DT, 1, BWD, __VA_ARGS__)                       \
        }                                                                       \
        break;                                                                  \
      default: break;                                                           \
    }                                                                           \
  } while (0)
}  // namespace rmsnorm_hip
