// Helpers shared by the split-row plans (rmsnorm_split.hip, layernorm_split.hip):
// rows too long for one workgroup are cut into segments of 16 KiB per
// matrix (256 threads x 64 bytes; the last segment may be shorter), and
// workgroup p*nseg + s owns segment s of the rows of block p.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rmsnorm_kernels.hpp"

namespace rmsnorm_hip {
namespace split {

constexpr int kSplitBlock = 256;
constexpr int kSplitWaves = kSplitBlock / kWave;
constexpr int kBytesPerThread = 64;  // per matrix and row segment

template <int DT, int VEC>
struct SplitGeom {
  static constexpr int kCh = kBytesPerThread / (VEC * ElemBytes<DT>::value);
  static constexpr int kSeg = kSplitBlock * kCh * VEC;  // elements per segment
};

// Sums of two values over the workgroup's wavefronts, for thread 0 only,
// added in wavefront order.  One barrier per call; `parity` alternates the
// slot set so the next call cannot overwrite values still being read.
__device__ __forceinline__ void block_sum2(float& a, float& b, float (*slots)[kSplitWaves][2],
                                           int& parity, int wave, int lane) {
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane == 0) {
    slots[parity][wave][0] = a;
    slots[parity][wave][1] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float ta = 0.f, tb = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      ta += slots[parity][w][0];
      tb += slots[parity][w][1];
    }
    a = ta;
    b = tb;
  }
  parity ^= 1;
}

struct SegIndex {
  int64_t r0, r1;  // rows of this workgroup
  int s;           // segment
  int e0;          // first element of this thread's chunk 0
};

template <int DT, int VEC>
__device__ __forceinline__ SegIndex seg_index(int64_t M, int nseg, int64_t P) {
  const int64_t p = blockIdx.x / nseg;
  SegIndex ix;
  ix.s = static_cast<int>(blockIdx.x - p * nseg);
  ix.r0 = block_row_begin(p, M, P);
  ix.r1 = block_row_begin(p + 1, M, P);
  ix.e0 = ix.s * SplitGeom<DT, VEC>::kSeg + threadIdx.x * VEC;
  return ix;
}

// Element of chunk c for this thread (chunk c is one coalesced sweep).
template <int VEC>
__device__ __forceinline__ int chunk_elem(int e0, int c) {
  return e0 + c * kSplitBlock * VEC;
}

// Row access: the row's base address is workgroup-uniform (scalar
// registers) and each lane adds a 32-bit byte offset, made opaque so the
// compiler neither keeps 64-bit addresses per chunk nor hoists loads out of
// the row loop.  Offsets stay below 2^26 (N <= 2^24 elements of <= 4 bytes).
template <int DT>
__device__ __forceinline__ const char* row_ptr(const void* base, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + row * ld * ElemBytes<DT>::value;
}

template <int DT, int VEC, bool NT>
__device__ __forceinline__ void load_at(Pack<DT, VEC>& v, const char* row, int e) {
  uint32_t off = static_cast<uint32_t>(e) * ElemBytes<DT>::value;
  asm volatile("" : "+v"(off));
  using R = typename Pack<DT, VEC>::raw_t;
  const R* a = reinterpret_cast<const R*>(row + off);
  if constexpr (NT) v.raw = __builtin_nontemporal_load(a);
  else v.raw = *a;
}

template <int DT, int VEC>
__device__ __forceinline__ void store_at(const Pack<DT, VEC>& v, const char* row, int e) {
  uint32_t off = static_cast<uint32_t>(e) * ElemBytes<DT>::value;
  asm volatile("" : "+v"(off));
  using R = typename Pack<DT, VEC>::raw_t;
  __builtin_nontemporal_store(v.raw, reinterpret_cast<R*>(const_cast<char*>(row) + off));
}

template <int DT, int VEC, int CH>
__device__ __forceinline__ void load_weight(Pack<DT, VEC> (&g)[CH], const void* gamma, int e0,
                                            int N) {
  const char* base = static_cast<const char*>(gamma);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = chunk_elem<VEC>(e0, c);
    g[c].zero();
    if (e < N) load_at<DT, VEC, false>(g[c], base, e);
  }
}

}  // namespace split
}  // namespace rmsnorm_hip
