// Full-width (16-byte vector) RMSNorm kernels for gfx950.
//
// Same arithmetic as rmsnorm_kernels.hpp (page "Check an AI model
// calculation before accelerating it": r = 1/sqrt(mean(x^2) + eps),
// y = x*r*g; dx = r*u - x*r^3*mean(u*x) with u = dy*g; dgamma = sum over rows
// of dy*x*r), with the row geometry fixed at compile time:
//
//   VEC  = 16 / sizeof(T)   elements per 16-byte access
//   WPR  wavefronts per row (1 = wavefront per row; up to 16 = a 1024-thread
//        workgroup per row), TPR = 64*WPR threads per row
//   CH   accesses per thread per row: thread t of a row owns elements
//        (c*TPR + t)*VEC .. +VEC-1 for c < CH; only the last chunk can be
//        partial, so only it carries a bounds test
//   G    = BLOCK/TPR rows processed side by side by one workgroup
//
// Row i of a matrix starts at byte i*pitch (pitch = the row stride times the
// element size; pitch = N*sizeof(T) for dense matrices).  Each lane adds its
// own byte offset t*16 and the chunk offset c*TPR*16.  Streaming accesses
// carry the cache-policy bit "nt" (no temporal reuse expected).
//
// The kernels are picked by the host plan when N*sizeof(T), every pitch and
// every pointer are 16-byte aligned; rmsnorm_kernels.hpp covers the others.
#pragma once

#include "rmsnorm_kernels.hpp"

namespace rmsnorm_hip {

typedef __attribute__((address_space(3))) void lds_void_t;

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Access to one row (or one vector) of 16-byte elements at byte offsets
// voff (per thread) + soff (uniform), with plain global addresses.
struct GRow {
  char* p;
  __device__ __forceinline__ explicit GRow(const void* base)
      : p(static_cast<char*>(const_cast<void*>(base))) {}
  template <bool NT>
  __device__ __forceinline__ u32x4 load(uint32_t voff, uint32_t soff) const {
    const u32x4* a = reinterpret_cast<const u32x4*>(p + soff + voff);
    if constexpr (NT) return __builtin_nontemporal_load(a);
    else return *a;
  }
  template <bool NT>
  __device__ __forceinline__ void store(u32x4 v, uint32_t voff, uint32_t soff) const {
    u32x4* a = reinterpret_cast<u32x4*>(p + soff + voff);
    if constexpr (NT) __builtin_nontemporal_store(v, a);
    else *a = v;
  }
  // The same load issued by an asm statement, so the compiler does not
  // track it: the caller waits for it with an explicit count and then ties
  // the register (an asm with it as operand) before any use.  A tracked
  // load read after stores were issued makes the compiler wait for every
  // access in flight (it cannot count loads past pending stores).
  template <bool NT>
  __device__ __forceinline__ u32x4 load_untracked(uint32_t voff, uint32_t soff) const {
    const char* a = p + soff + voff;
    u32x4 v;
    if constexpr (NT) asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(v) : "v"(a) : "memory");
    else asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(a) : "memory");
    return v;
  }
  __device__ __forceinline__ void to_lds(void* lds_wave_base, uint32_t voff, uint32_t soff) const {
    __builtin_amdgcn_global_load_lds(p + soff + voff, (lds_void_t*)lds_wave_base, 16, 0, 0);
  }
};

// Row access in the scalar-base form: the row base is wave-uniform (kernel
// argument plus a uniform row offset, held in SGPRs) and each lane adds one
// 32-bit byte offset, so no chunk costs a 64-bit address in VGPRs.  The lane
// offset is made opaque per use: the compiler can then neither hoist a load
// out of the row loop nor merge two loads of one address (either would keep
// values live across a whole row and exhaust the register file).
struct URow {
  const char* p;
  __device__ __forceinline__ explicit URow(const void* base) : p(static_cast<const char*>(base)) {}
  __device__ __forceinline__ const char* at(uint32_t voff, uint32_t soff) const {
    uint32_t o = voff + soff;
    asm volatile("" : "+v"(o));
    return p + o;
  }
  template <bool NT>
  __device__ __forceinline__ u32x4 load(uint32_t voff, uint32_t soff) const {
    const u32x4* a = reinterpret_cast<const u32x4*>(at(voff, soff));
    if constexpr (NT) return __builtin_nontemporal_load(a);
    else return *a;
  }
  template <bool NT>
  __device__ __forceinline__ void store(u32x4 v, uint32_t voff, uint32_t soff) const {
    u32x4* a = reinterpret_cast<u32x4*>(const_cast<char*>(at(voff, soff)));
    if constexpr (NT) __builtin_nontemporal_store(v, a);
    else *a = v;
  }
  __device__ __forceinline__ void to_lds(void* lds_wave_base, uint32_t voff, uint32_t soff) const {
    __builtin_amdgcn_global_load_lds(const_cast<char*>(at(voff, soff)),
                                     (lds_void_t*)lds_wave_base, 16, 0, 0);
  }
};

// Scheduling fence: no instruction moves across it.  Placed between the
// chunks of a sweep so the scheduler does not widen every chunk at once
// (which multiplies the live float32 temporaries and spills).
__device__ __forceinline__ void chunk_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int DT, int CH, int WPR, int BLOCK>
struct Geometry {
  static constexpr int VEC = 16 / ElemBytes<DT>::value;
  static constexpr int TPR = kWave * WPR;
  static constexpr int G = BLOCK / TPR;
  static constexpr int SWEEP = TPR * VEC;  // elements covered by one chunk
  static_assert(BLOCK % TPR == 0 && G >= 1, "block must hold whole rows");
  static_assert(CH >= 1 && CH <= 16, "chunks per thread");
};

// Row sum across the WPR wavefronts of a row group.  All threads of the
// workgroup call it the same number of times (the row loops below have a
// workgroup-uniform trip count), since WPR > 1 needs a workgroup barrier.
// slots: [2][G][WPR] floats in LDS; parity alternates between calls.
template <int WPR, int G>
__device__ __forceinline__ float group_sum(float v, float* slots, int& parity, int group,
                                           int wave_in_row, int lane) {
  v = wave_sum(v);
  if constexpr (WPR == 1) {
    return v;
  } else {
    float* s = slots + (parity * G + group) * WPR;
    if (lane == 0) s[wave_in_row] = v;
    __syncthreads();
    float t = s[0];
#pragma unroll
    for (int i = 1; i < WPR; ++i) t += s[i];
    parity ^= 1;
    return t;
  }
}

// Order in which a workgroup takes its rows.  Either way the rows of
// workgroup w (of P) are a fixed function of (M, P, G), so every reduction
// order is reproducible; row group `group` of the G in a workgroup takes row
// base + it*stride + group.
//   kRowsBlocked: the contiguous rows [w*M/P, (w+1)*M/P)
//   kRowsCyclic:  row groups w, w+P, w+2P, ... counted from the first (all
//                 workgroups sweep the tensor together, front to back)
//   kRowsReverse: the same row groups counted from the last (the sweep runs
//                 back to front)
// A grid that sweeps the tensor together keeps the rows in flight within one
// window of the matrix, which the HBM serves far better than P streams at
// once when the data is not in cache.  Running the backward's sweep in the
// direction opposite to the forward's starts it on the rows the forward
// touched last.
constexpr int kRowsBlocked = 0;
constexpr int kRowsCyclic = 1;
constexpr int kRowsReverse = 2;

template <int ORD>
struct RowSched {
  int64_t base, stride, limit, iters;
  __device__ __forceinline__ RowSched(int64_t w, int64_t M, int64_t P, int G) {
    if constexpr (ORD == kRowsBlocked) {
      const int64_t r0 = block_row_begin(w, M, P), r1 = block_row_begin(w + 1, M, P);
      base = r0;
      stride = G;
      limit = r1;
      iters = (r1 - r0 + G - 1) / G;
    } else {
      const int64_t groups = (M + G - 1) / G;
      iters = w < groups ? (groups - w + P - 1) / P : 0;
      limit = M;
      if constexpr (ORD == kRowsCyclic) {
        base = w * G;
        stride = P * G;
      } else {
        // Row group groups-1-w first; the partial group (if any) is the
        // last one, so only workgroup 0's first step can reach past M.
        base = (groups - 1 - w) * G;
        stride = -P * G;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Forward.  Workgroup b handles rows b*G + g, then strides by gridDim.x*G.
// GREG keeps the weight in registers across rows (else it is re-read from
// cache each row); NT marks x loads and y stores as streaming.
// ADD (the residual add fused before the norm): the row is h = T(x + res),
// formed from the two loaded rows, written to h and then normalised; res, h
// and their pitches are unused otherwise.
// ---------------------------------------------------------------------------
template <int DT, int CH, int WPR, int BLOCK, bool GREG, bool NT, int MINW = 1, bool ADD = false>
__global__ __launch_bounds__(BLOCK, MINW) void fwd_fast_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, void* __restrict__ y,
    float* __restrict__ rstd, int64_t M, int N, float eps, int offset, int64_t x_pitch,
    int64_t y_pitch, const void* __restrict__ res, void* __restrict__ h, int64_t res_pitch,
    int64_t h_pitch) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, G = Geo::G;
  constexpr uint32_t kChunk = TPR * 16;  // bytes per chunk sweep
  using PK = Pack<DT, VEC>;
  __shared__ float slots[WPR > 1 ? 2 * G * WPR : 1];
  const int t = threadIdx.x % TPR;
  const int group = uniform(static_cast<int>(threadIdx.x / TPR));
  const int wave_in_row = uniform(t / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  int parity = 0;
  const float n_f = static_cast<float>(N);
  const GRow gbuf(gamma);

  PK g[GREG ? CH : 1];
  if constexpr (GREG) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < CH - 1 || voff + c * kChunk < row_bytes) g[c].raw = gbuf.template load<false>(voff, c * kChunk);
      else g[c].zero();
    }
  }

  for (int64_t row0 = static_cast<int64_t>(blockIdx.x) * G; row0 < M;
       row0 += static_cast<int64_t>(gridDim.x) * G) {
    const int64_t row = row0 + group;
    const bool active = row < M;
    if constexpr (GREG) {
#pragma unroll
      for (int c = 0; c < CH; ++c) g[c].opaque();
    }
    PK xv[CH];
    if (active) {
      const GRow xb(static_cast<const char*>(x) + row * x_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) xv[c].raw = xb.template load<NT>(voff, c * kChunk);
        else xv[c].zero();
      }
      if constexpr (ADD) {
        // h = T(x + res): the float32 sum rounded once on packing; the
        // norm below reads the rounded h.  Every chunk of res is in flight
        // before the first sum.
        const GRow rb(static_cast<const char*>(res) + row * res_pitch);
        const GRow hb(static_cast<char*>(h) + row * h_pitch);
        PK rv[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          if (c < CH - 1 || voff + c * kChunk < row_bytes) rv[c].raw = rb.template load<NT>(voff, c * kChunk);
          else rv[c].zero();
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          float sum[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) sum[k] = xv[c].get(k) + rv[c].get(k);
          xv[c].set(sum);
          if (c < CH - 1 || voff + c * kChunk < row_bytes) hb.template store<NT>(xv[c].raw, voff, c * kChunk);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) xv[c].zero();
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float f = xv[c].get(k);
        ss = fmaf(f, f, ss);
      }
    ss = group_sum<WPR, G>(ss, slots, parity, group, wave_in_row, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) xv[c].opaque();
    const float r = 1.0f / sqrtf(ss / n_f + eps);
    if (active) {
      if (t == 0) rstd[row] = r;
      const GRow yb(static_cast<char*>(y) + row * y_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          PK gv;
          if constexpr (GREG) gv = g[c];
          else gv.raw = gbuf.template load<false>(voff, c * kChunk);
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            o[k] = (xv[c].get(k) * r) * weight_of(gv.get(k), offset);
          PK out;
          out.set(o);
          yb.template store<NT>(out.raw, voff, c * kChunk);
        }
        chunk_fence();
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Backward stage 1.  Workgroup w takes the rows RowSched<ORD> gives it; its G
// row groups take them in turn (row = base + it*stride + g), all groups
// running the same number of iterations.  Per row: dot = sum(dy*g*x) over the row, then one
// sweep computes dx = r*u - x*(r^3*dot/N) and acc_j += (dy_j*x_j)*r.  Then the
// G accumulators are added in group order, one chunk-wide slice at a time
// through LDS, and the workgroup writes its partial row part[w, :].
//
// XLDS: x arrives by DMA straight into LDS (one row per group, no VGPRs while
// in flight) and is read back for both sweeps.
// GREG: the weight lives in registers; otherwise it is re-read from cache.
// ---------------------------------------------------------------------------
template <int DT, int CH, int WPR, int BLOCK, bool GREG, bool XLDS, bool NT, int ORD,
          int MINW = 1>
__global__ __launch_bounds__(BLOCK, MINW) void bwd_fast_kernel(
    const void* __restrict__ dy, const void* __restrict__ x,
    const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ dx, float* __restrict__ part, int64_t M, int N, int offset,
    int64_t P, int64_t dy_pitch, int64_t x_pitch, int64_t dx_pitch) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, G = Geo::G, SWEEP = Geo::SWEEP;
  constexpr uint32_t kChunk = TPR * 16;
  using PK = Pack<DT, VEC>;
  // XLDS: [G][N] elements of x; after the row loop: [G][SWEEP] float32 for
  // the combine (G > 1).
  extern __shared__ __align__(16) char dyn[];
  __shared__ float slots[WPR > 1 ? 2 * G * WPR : 1];
  const int t = threadIdx.x % TPR;
  const int group = uniform(static_cast<int>(threadIdx.x / TPR));
  const int wave_in_row = uniform(t / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  int parity = 0;
  const int64_t w = blockIdx.x;
  const RowSched<ORD> rs(w, M, P, G);
  const int64_t iters = rs.iters;
  const float n_f = static_cast<float>(N);
  char* xrow = dyn + static_cast<int64_t>(group) * row_bytes;
  const GRow gbuf(gamma);

  PK g[GREG ? CH : 1];
  if constexpr (GREG) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < CH - 1 || voff + c * kChunk < row_bytes) g[c].raw = gbuf.template load<false>(voff, c * kChunk);
      else g[c].zero();
    }
  }
  float acc[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;

  for (int64_t it = 0; it < iters; ++it) {
    const int64_t row = rs.base + it * rs.stride + group;
    const bool active = row < rs.limit;
    if constexpr (GREG) {
#pragma unroll
      for (int c = 0; c < CH; ++c) g[c].opaque();
    }
    PK xv[XLDS ? 1 : CH], dv[CH];
    float r = 0.f;
    if (active) {
      r = rstd[row];
      const GRow xb(static_cast<const char*>(x) + row * x_pitch);
      const GRow db(static_cast<const char*>(dy) + row * dy_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          dv[c].raw = db.template load<NT>(voff, c * kChunk);
          if constexpr (XLDS) xb.to_lds(xrow + c * kChunk + wave_in_row * kWave * 16, voff, c * kChunk);
          else xv[c].raw = xb.template load<NT>(voff, c * kChunk);
        } else {
          dv[c].zero();
          if constexpr (!XLDS) xv[c].zero();
        }
      }
      if constexpr (XLDS) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        dv[c].zero();
        if constexpr (!XLDS) xv[c].zero();
      }
    }
    float dot = 0.f;
    if (active) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          PK xc, gv;
          if constexpr (XLDS) xc.raw = *reinterpret_cast<const u32x4*>(xrow + c * kChunk + voff);
          else xc = xv[c];
          if constexpr (GREG) gv = g[c];
          else gv.raw = gbuf.template load<false>(voff, c * kChunk);
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            dot = fmaf(dv[c].get(k) * weight_of(gv.get(k), offset), xc.get(k), dot);
        }
        chunk_fence();
      }
    }
    dot = group_sum<WPR, G>(dot, slots, parity, group, wave_in_row, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      dv[c].opaque();
      if constexpr (!XLDS) xv[c].opaque();
      if constexpr (GREG) g[c].opaque();
    }
    const float r3c = ((r * r) * r) * (dot / n_f);
    if (active) {
      const GRow ob(static_cast<char*>(dx) + row * dx_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          PK xc, gv;
          if constexpr (XLDS) xc.raw = *reinterpret_cast<const u32x4*>(xrow + c * kChunk + voff);
          else xc = xv[c];
          if constexpr (GREG) gv = g[c];
          else gv.raw = gbuf.template load<false>(voff, c * kChunk);
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float xf = xc.get(k);
            const float dyf = dv[c].get(k);
            const float u = dyf * weight_of(gv.get(k), offset);
            o[k] = fmaf(-xf, r3c, r * u);
            acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
          }
          PK out;
          out.set(o);
          ob.template store<NT>(out.raw, voff, c * kChunk);
        }
        chunk_fence();
      }
    }
  }

  float* dst = part + w * static_cast<int64_t>(N);
  if constexpr (G == 1) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = (c * TPR + t) * VEC;
      if (c < CH - 1 || e < N) store_f32<VEC>(dst + e, acc[c]);
    }
  } else {
    // Fixed-order combine of the G groups, one chunk sweep (SWEEP columns) at
    // a time: part[w, col] = ((acc_0 + acc_1) + acc_2) + ...
    float* comb = reinterpret_cast<float*>(dyn);
    __syncthreads();  // the LDS area may still hold staged rows
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      store_f32<VEC>(comb + group * SWEEP + t * VEC, acc[c]);
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

// ---------------------------------------------------------------------------
// Software-pipelined row kernels.
//
// On gfx9 one counter tracks every outstanding vector memory operation, loads
// and stores alike, and they retire in issue order.  A row loop that loads
// row i, reduces, then stores row i makes each wavefront wait for its own
// stores of row i-1 before the loads of row i can be consumed; a workgroup
// barrier that also orders global memory (__syncthreads) waits for them too.
// The pipelined kernels below instead
//   * issue the loads of row i+1 right after the row-i reduction, before
//     the row-i stores, so those stores stay in flight while row i+1 arrives,
//   * exchange the partial row sums with a barrier that orders LDS only.
// The two register sets (rows i and i+1) alternate by unrolling the row loop
// twice, so no register copy ever waits on a load in flight.
// ---------------------------------------------------------------------------

// Wait until at most N vector memory operations of this wavefront are
// outstanding.  The "memory" clobber keeps the compiler from moving memory
// accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Compiler-only fence: no memory access and no instruction is moved across
// it (so the number of operations issued after a group of loads is exactly
// what the source says).
__device__ __forceinline__ void order_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier for the row-sum exchange: this wavefront's LDS
// instructions complete (lgkmcnt), then every wavefront meets.  Unlike
// __syncthreads (or an LDS-scoped fence, which also covers DMA writes into
// LDS) it does not wait for vector memory operations in flight: global
// stores and prefetches keep streaming across it.  The memory clobber keeps
// the compiler from moving any access across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// group_sum with the LDS-only barrier (same slots, parity and result).
template <int WPR, int G>
__device__ __forceinline__ float group_sum_lds(float v, float* slots, int& parity, int group,
                                               int wave_in_row, int lane) {
  v = wave_sum(v);
  if constexpr (WPR == 1) {
    return v;
  } else {
    float* s = slots + (parity * G + group) * WPR;
    if (lane == 0) s[wave_in_row] = v;
    lds_barrier();
    float t = s[0];
#pragma unroll
    for (int i = 1; i < WPR; ++i) t += s[i];
    parity ^= 1;
    return t;
  }
}

// 16 bytes from LDS, complete on return.  Written as one asm statement (read
// and wait together) so the compiler neither sees an LDS read it would guard
// with a wait for every DMA in flight, nor can touch the destination
// registers before the data has arrived.
__device__ __forceinline__ u32x4 lds_read16(const void* p) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}

// Forward, pipelined.  Workgroup w of P = gridDim.x takes the rows
// RowSched<ORD> gives it; its G row groups take rows base + it*stride + group.
// The weight stays in registers for the whole launch.  x is prefetched one
// row ahead either into LDS by DMA (XL, two stage buffers of [G][N] elements,
// read back with lds_read16 after an explicit wait) or into the second of two
// register sets.
template <int DT, int CH, int WPR, int BLOCK, bool NT, bool XL, int ORD, int MINW = 1>
__global__ __launch_bounds__(BLOCK, MINW) void fwd_pipe_kernel(
    const void* __restrict__ x, const void* __restrict__ gamma, void* __restrict__ y,
    float* __restrict__ rstd, int64_t M, int N, float eps, int offset, int64_t x_pitch,
    int64_t y_pitch) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, G = Geo::G;
  constexpr uint32_t kChunk = TPR * 16;
  using PK = Pack<DT, VEC>;
  extern __shared__ __align__(16) char dyn[];
  __shared__ float slots[WPR > 1 ? 2 * G * WPR : 1];
  const int t = threadIdx.x % TPR;
  const int group = uniform(static_cast<int>(threadIdx.x / TPR));
  const int wave_in_row = uniform(t / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  int parity = 0;
  const float n_f = static_cast<float>(N);
  const RowSched<ORD> rs(blockIdx.x, M, gridDim.x, G);
  const int64_t iters = rs.iters;
  char* const xstage = dyn + static_cast<int64_t>(group) * row_bytes;
  const int64_t stage_stride = static_cast<int64_t>(G) * row_bytes;
  const uint32_t dma_off = wave_in_row * kWave * 16;
  const GRow gbuf(gamma);

  PK g[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < CH - 1 || voff + c * kChunk < row_bytes) g[c].raw = gbuf.template load<false>(voff, c * kChunk);
    else g[c].zero();
  }

  auto issue = [&](int64_t row, int64_t it, PK(&xv)[CH]) __attribute__((always_inline)) {
    const GRow xb(static_cast<const char*>(x) + row * x_pitch);
    char* xs = xstage + (it & 1) * stage_stride;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < CH - 1 || voff + c * kChunk < row_bytes) {
        if constexpr (XL) xb.to_lds(xs + c * kChunk + dma_off, voff, c * kChunk);
        else xv[c].raw = xb.template load<NT>(voff, c * kChunk);
      } else if constexpr (!XL) {
        xv[c].zero();
      }
    }
  };

  // Lower bound on the vector memory operations issued after a row's loads:
  // the previous row's y stores (the rstd store is not counted).
  const bool has_last = uniform(static_cast<uint32_t>(wave_in_row * kWave * 16) +
                                (CH - 1) * kChunk) < row_bytes;

  auto step = [&](int64_t it, PK(&xc)[CH], PK(&xn)[CH]) __attribute__((always_inline)) {
    const int64_t row = rs.base + it * rs.stride + group;
    const bool active = row < rs.limit;
    if constexpr (XL) {
      if (active) {
        if (has_last) wait_vmem<CH>();
        else wait_vmem<CH - 1>();
      }
    }
    // Prefetch row it+1; it has the whole of this step to arrive.
    order_fence();
    if (it + 1 < iters && row + rs.stride < rs.limit) issue(row + rs.stride, it + 1, xn);
    order_fence();
    PK xv[CH];
    float ss = 0.f;
    if (active) {
      const char* xs = xstage + (it & 1) * stage_stride;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if constexpr (XL) {
          if (c < CH - 1 || voff + c * kChunk < row_bytes) xv[c].raw = lds_read16(xs + c * kChunk + voff);
          else xv[c].zero();
        } else {
          xv[c] = xc[c];
        }
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float f = xv[c].get(k);
          ss = fmaf(f, f, ss);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) xv[c].zero();
    }
    ss = group_sum_lds<WPR, G>(ss, slots, parity, group, wave_in_row, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      xv[c].opaque();
      g[c].opaque();
    }
    const float r = 1.0f / sqrtf(ss / n_f + eps);
    if (active) {
      if (t == 0) rstd[row] = r;
      const GRow yb(static_cast<char*>(y) + row * y_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) o[k] = (xv[c].get(k) * r) * weight_of(g[c].get(k), offset);
          PK out;
          out.set(o);
          yb.template store<NT>(out.raw, voff, c * kChunk);
        }
        chunk_fence();
      }
    }
  };

  PK xa[CH], xb2[CH];  // register sets (unused with XL)
  if (iters > 0 && rs.base + group < rs.limit) issue(rs.base + group, 0, xa);
  else if constexpr (!XL) {
#pragma unroll
    for (int c = 0; c < CH; ++c) xa[c].zero();
  }
  // Settle the first row's loads (and the weight) before the loop, so the
  // loop body's waits count only its own operations.
  wait_vmem<0>();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if constexpr (!XL) xa[c].opaque();
    g[c].opaque();
  }
  int64_t it = 0;
  for (; it + 1 < iters; it += 2) {
    step(it, xa, xb2);
    step(it + 1, xb2, xa);
  }
  if (it < iters) step(it, xa, xb2);
}

template <int DT, int CH, int WPR, int BLOCK, bool XL>
inline int64_t fwd_pipe_lds_bytes(int N) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  return XL ? 2 * static_cast<int64_t>(Geo::G) * N * ElemBytes<DT>::value : 0;
}

// Backward stage 1, pipelined.  Rows taken as in bwd_fast_kernel (P = gridDim.x
// workgroups, RowSched<ORD>, one fp32 dgamma partial row each).  x (and,
// with DLDS, dy) reaches LDS by DMA into one of two stage buffers
// ([2][DLDS ? 2 : 1][G][N] elements); without DLDS dy is loaded into one of
// two register sets.  Each wavefront reads back exactly the bytes its own DMA
// wrote, so the staging needs no barrier; the wait for row it's data is an
// explicit count (see `step`).
template <int DT, int CH, int WPR, int BLOCK, bool NT, bool DLDS, int ORD, int MINW = 1>
__global__ __launch_bounds__(BLOCK, MINW) void bwd_pipe_kernel(
    const void* __restrict__ dy, const void* __restrict__ x,
    const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ dx, float* __restrict__ part, int64_t M, int N, int offset,
    int64_t P, int64_t dy_pitch, int64_t x_pitch, int64_t dx_pitch) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, G = Geo::G, SWEEP = Geo::SWEEP;
  constexpr uint32_t kChunk = TPR * 16;
  constexpr int kSets = DLDS ? 2 : 1;  // staged tensors per buffer
  using PK = Pack<DT, VEC>;
  extern __shared__ __align__(16) char dyn[];
  __shared__ float slots[WPR > 1 ? 2 * G * WPR : 1];
  const int t = threadIdx.x % TPR;
  const int group = uniform(static_cast<int>(threadIdx.x / TPR));
  const int wave_in_row = uniform(t / kWave);
  const int lane = threadIdx.x % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  int parity = 0;
  const int64_t w = blockIdx.x;
  const RowSched<ORD> rs(w, M, P, G);
  const int64_t iters = rs.iters;
  const float n_f = static_cast<float>(N);
  // Stage buffer b: x row of this group at xstage + b*stage_stride, dy row
  // (DLDS) G rows further.
  char* const xstage = dyn + static_cast<int64_t>(group) * row_bytes;
  const int64_t stage_stride = static_cast<int64_t>(kSets) * G * row_bytes;
  const int64_t dy_off = static_cast<int64_t>(G) * row_bytes;
  const uint32_t dma_off = wave_in_row * kWave * 16;
  const GRow gbuf(gamma);

  // With dy in registers the weight (gamma, or 1 + w in offset mode) is
  // widened once and held in float32 registers for the whole kernel, instead
  // of a conversion and an add per element and row (fp16 262144 x 1024: 271.5
  // -> 268.8 us).  With dy staged in LDS that measured slower (bf16
  // 65536 x 5120: 333 -> 352 us), so there the packed weight is re-widened
  // per row as before.
  constexpr bool kHoldW = !DLDS;
  PK g[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < CH - 1 || voff + c * kChunk < row_bytes) g[c].raw = gbuf.template load<false>(voff, c * kChunk);
    else g[c].zero();
  }
  float gw[CH][VEC];
  auto weight = [&](int c, int k) __attribute__((always_inline)) {
    if constexpr (kHoldW) return gw[c][k];
    else return weight_of(g[c].get(k), offset);
  };
  float acc[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;

  auto issue = [&](int64_t row, int64_t it, PK(&dv)[CH]) __attribute__((always_inline)) {
    char* xs = xstage + (it & 1) * stage_stride;
    const GRow xb(static_cast<const char*>(x) + row * x_pitch);
    const GRow db(static_cast<const char*>(dy) + row * dy_pitch);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c < CH - 1 || voff + c * kChunk < row_bytes) {
        xb.to_lds(xs + c * kChunk + dma_off, voff, c * kChunk);
        if constexpr (DLDS) db.to_lds(xs + dy_off + c * kChunk + dma_off, voff, c * kChunk);
        else dv[c].raw = db.template load_untracked<NT>(voff, c * kChunk);
      } else if constexpr (!DLDS) {
        dv[c].zero();
      }
    }
  };

  // Vector memory operations this wavefront issues after the loads of a row:
  // the stores of the previous row, CH of them, or CH-1 when no lane of the
  // wavefront reaches the last chunk (that store is branched around).
  const bool has_last = uniform(static_cast<uint32_t>(wave_in_row * kWave * 16) +
                                (CH - 1) * kChunk) < row_bytes;

  // `last`: the final step, which has no next row to prefetch (stated so
  // that no load is emitted there at all).
  auto step = [&](int64_t it, PK(&dc)[CH], PK(&dn)[CH], bool last) __attribute__((always_inline)) {
    const int64_t row = rs.base + it * rs.stride + group;
    const bool active = row < rs.limit;
    const char* xs = xstage + (it & 1) * stage_stride;
    if (active) {
      // Row it's DMA (and dy loads) were issued before the previous row's
      // stores: wait for them only, the stores may stay in flight.  The
      // count is a lower bound on the operations issued since, so the wait
      // is never too short.  (Row it active implies row it-1 was.)
      if (has_last) wait_vmem<CH>();
      else wait_vmem<CH - 1>();
    }
    // The dy registers were loaded untracked: their uses follow the wait.
    if constexpr (!DLDS) {
#pragma unroll
      for (int c = 0; c < CH; ++c) dc[c].opaque();
    }
    // Prefetch row it+1 into the other stage buffer (and register set); it
    // has the whole of this step to arrive.
    order_fence();
    if (!last && it + 1 < iters && row + rs.stride < rs.limit) issue(row + rs.stride, it + 1, dn);
    order_fence();
    float r = 0.f;
    PK xv[CH], dv[CH];
    float dot = 0.f;
    if (active) {
      r = rstd[row];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          xv[c].raw = lds_read16(xs + c * kChunk + voff);
          if constexpr (DLDS) dv[c].raw = lds_read16(xs + dy_off + c * kChunk + voff);
          else dv[c] = dc[c];
#pragma unroll
          for (int k = 0; k < VEC; ++k)
            dot = fmaf(dv[c].get(k) * weight(c, k), xv[c].get(k), dot);
        } else {
          xv[c].zero();
          dv[c].zero();
        }
        chunk_fence();
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        xv[c].zero();
        dv[c].zero();
      }
    }
    dot = group_sum_lds<WPR, G>(dot, slots, parity, group, wave_in_row, lane);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      xv[c].opaque();
      dv[c].opaque();
      if constexpr (!kHoldW) g[c].opaque();
    }
    const float r3c = ((r * r) * r) * (dot / n_f);
    if (active) {
      const GRow ob(static_cast<char*>(dx) + row * dx_pitch);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (c < CH - 1 || voff + c * kChunk < row_bytes) {
          float o[VEC];
#pragma unroll
          for (int k = 0; k < VEC; ++k) {
            const float xf = xv[c].get(k);
            const float dyf = dv[c].get(k);
            const float u = dyf * weight(c, k);
            o[k] = fmaf(-xf, r3c, r * u);
            acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
          }
          PK out;
          out.set(o);
          ob.template store<NT>(out.raw, voff, c * kChunk);
        }
        chunk_fence();
      }
    }
  };

  PK da[CH], db2[CH];  // dy register sets (unused with DLDS)
  if (iters > 0 && rs.base + group < rs.limit) issue(rs.base + group, 0, da);
  else if constexpr (!DLDS) {
#pragma unroll
    for (int c = 0; c < CH; ++c) da[c].zero();
  }
  // Settle the first row's loads (and the weight) before the loop.
  wait_vmem<0>();
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if constexpr (!DLDS) da[c].opaque();
    if constexpr (kHoldW) {
#pragma unroll
      for (int k = 0; k < VEC; ++k) gw[c][k] = weight_of(g[c].get(k), offset);
    } else {
      g[c].opaque();
    }
  }
  int64_t it = 0;
  for (; it + 1 < iters; it += 2) {
    step(it, da, db2, false);
    step(it + 1, db2, da, false);
  }
  if (it < iters) step(it, da, db2, true);

  float* dst = part + w * static_cast<int64_t>(N);
  if constexpr (G == 1) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int e = (c * TPR + t) * VEC;
      if (c < CH - 1 || e < N) store_f32<VEC>(dst + e, acc[c]);
    }
  } else {
    float* comb = reinterpret_cast<float*>(dyn);
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      store_f32<VEC>(comb + group * SWEEP + t * VEC, acc[c]);
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

template <int DT, int CH, int WPR, int BLOCK, bool DLDS>
inline int64_t bwd_pipe_lds_bytes(int N) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  const int64_t stage = 2 * (DLDS ? 2 : 1) * static_cast<int64_t>(Geo::G) * N * ElemBytes<DT>::value;
  const int64_t comb = Geo::G > 1 ? static_cast<int64_t>(Geo::G) * Geo::SWEEP * 4 : 0;
  return stage > comb ? stage : comb;
}

// ---------------------------------------------------------------------------
// Backward stage 1 for long rows (16 KiB < row <= 128 KiB): one 512-thread
// workgroup streams whole rows, CH = ceil(row / 8 KiB) chunks per lane.
//
// Per row, x sits in LDS (DMA) and dy in registers, so x, dy and the dgamma
// accumulators of a 128 KiB row stay on chip: 8 wavefronts of 512 threads
// may hold 256 VGPRs each (dy: 4*CH, accumulators: VEC*CH).
//   pass A  dot = sum(dy*g*x)               (x read back from LDS)
//   reduce  across the 8 wavefronts (LDS-only barrier)
//   pass B  dx = r*u - x*(r^3*dot/N), acc += (dy*x)*r; after chunk c is done
//           its LDS slot and dy registers take the next row's chunk c, so the
//           next row streams in behind the current row's dx stores.
// The weight is read from cache one chunk ahead of its use, so its wait
// never covers a store issued after it (one in-order counter for all vector
// memory operations).  An LDS read of x waits, through an operand
// dependency, for the dy load of the same chunk; that load was issued right
// after the chunk's DMA, so its completion implies the DMA's.
// ---------------------------------------------------------------------------

// Pins a value at this point of the program: its computation cannot be
// sunk below (or hoisted above) the statement, so a chunk's arithmetic stays
// with its chunk and dead inputs free their registers.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

// 16 bytes from LDS once `dep` (a register loaded after the DMA that filled
// this LDS address) has arrived; complete on return.
__device__ __forceinline__ u32x4 lds_read16_after(const void* p, const u32x4& dep) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a), "v"(dep) : "memory");
  return v;
}

// DH (the residual add fused before the norm, x being h): dx also adds the
// gradient dh arriving on h, read like the weight one chunk ahead of its use.
template <int DT, int CH, bool NT, bool DH = false>
__global__ __launch_bounds__(512) void bwd_longrow_kernel(
    const void* __restrict__ dy, const void* __restrict__ x,
    const void* __restrict__ gamma, const float* __restrict__ rstd,
    void* __restrict__ dx, float* __restrict__ part, int64_t M, int N, int offset,
    int64_t P, int64_t dy_pitch, int64_t x_pitch, int64_t dx_pitch,
    const void* __restrict__ dh, int64_t dh_pitch) {
  constexpr int WPR = 8, BLOCK = 512;
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR;
  constexpr uint32_t kChunk = TPR * 16;
  using PK = Pack<DT, VEC>;
  extern __shared__ __align__(16) char dyn[];  // [N] elements of x
  __shared__ float slots[2 * WPR];
  const int t = threadIdx.x;
  const int wave = uniform(t / kWave);
  const int lane = t % kWave;
  const uint32_t voff = t * 16;
  const uint32_t row_bytes = static_cast<uint32_t>(N) * ElemBytes<DT>::value;
  const uint32_t dma_off = wave * kWave * 16;
  int parity = 0;
  const int64_t w = blockIdx.x;
  const RowSched<kRowsCyclic> rs(w, M, P, 1);
  const float n_f = static_cast<float>(N);
  const URow gbuf(gamma);

  PK dv[CH];
  float acc[CH][VEC];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[c][k] = 0.f;

  auto in_row = [&](int c) __attribute__((always_inline)) {
    return c < CH - 1 || voff + c * kChunk < row_bytes;
  };
  auto issue_chunk = [&](int64_t row, int c) __attribute__((always_inline)) {
    if (in_row(c)) {
      const URow xb(static_cast<const char*>(x) + row * x_pitch);
      const URow db(static_cast<const char*>(dy) + row * dy_pitch);
      xb.to_lds(dyn + c * kChunk + dma_off, voff, c * kChunk);  // DMA first,
      dv[c].raw = db.template load<NT>(voff, c * kChunk);        // then dy
    } else {
      dv[c].zero();
    }
  };
  auto load_g = [&](int c) __attribute__((always_inline)) {
    PK g;
    if (in_row(c)) g.raw = gbuf.template load<false>(voff, c * kChunk);
    else g.zero();
    return g;
  };

  if (rs.iters > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) issue_chunk(rs.base, c);
  }
  for (int64_t it = 0; it < rs.iters; ++it) {
    const int64_t row = rs.base + it * rs.stride;  // always < M here
    const bool has_next = it + 1 < rs.iters;
    const float r = rstd[row];

    // pass A
    float dot = 0.f;
    PK gc = load_g(0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      PK gn;
      if (c + 1 < CH) gn = load_g(c + 1);
      dv[c].opaque();  // widen this chunk here, not where it was loaded
      if (in_row(c)) {
        PK xv;
        xv.raw = lds_read16_after(dyn + c * kChunk + voff, dv[c].raw);
#pragma unroll
        for (int k = 0; k < VEC; ++k)
          dot = fmaf(dv[c].get(k) * weight_of(gc.get(k), offset), xv.get(k), dot);
      }
      pin(dot);
      if (c + 1 < CH) gc = gn;
      chunk_fence();
    }
    dot = group_sum_lds<WPR, 1>(dot, slots, parity, 0, wave, lane);
    const float r3c = ((r * r) * r) * (dot / n_f);

    // pass B
    const URow ob(static_cast<char*>(dx) + row * dx_pitch);
    const URow hb(static_cast<const char*>(dh) + (DH ? row * dh_pitch : 0));
    auto load_dh = [&](int c) __attribute__((always_inline)) {
      PK e;
      if (DH && in_row(c)) e.raw = hb.template load<NT>(voff, c * kChunk);
      else e.zero();
      return e;
    };
    gc = load_g(0);
    PK ec = load_dh(0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      PK gn, en;
      if (c + 1 < CH) gn = load_g(c + 1);
      dv[c].opaque();  // re-widen here rather than keep pass A's floats
      if (in_row(c)) {
        PK xv;
        xv.raw = lds_read16_after(dyn + c * kChunk + voff, dv[c].raw);
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float xf = xv.get(k);
          const float dyf = dv[c].get(k);
          const float u = dyf * weight_of(gc.get(k), offset);
          o[k] = fmaf(-xf, r3c, r * u);
          if constexpr (DH) o[k] = o[k] + ec.get(k);
          acc[c][k] = fmaf(dyf * xf, r, acc[c][k]);
        }
        PK out;
        out.set(o);
        // dh of the next chunk: issued once this chunk's dh is consumed
        // (one set live) and before this chunk's store, so its wait does
        // not cover the store.  (Only the last chunk can lie outside the
        // row, and it has no next chunk.)
        if constexpr (DH) {
          order_fence();
          if (c + 1 < CH) en = load_dh(c + 1);
        }
        ob.template store<NT>(out.raw, voff, c * kChunk);
      }
#pragma unroll
      for (int k = 0; k < VEC; ++k) pin(acc[c][k]);
      order_fence();
      if (has_next) issue_chunk(row + rs.stride, c);
      order_fence();
      if (c + 1 < CH) {
        gc = gn;
        ec = en;
      }
    }
  }

  float* dst = part + w * static_cast<int64_t>(N);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = (c * TPR + t) * VEC;
    if (c < CH - 1 || e < N) store_f32<VEC>(dst + e, acc[c]);
  }
}

// LDS bytes the backward kernel needs for a given N.
template <int DT, int CH, int WPR, int BLOCK, bool XLDS>
constexpr int64_t bwd_fast_lds_bytes(int N) {
  using Geo = Geometry<DT, CH, WPR, BLOCK>;
  const int64_t stage = static_cast<int64_t>(XLDS ? 1 : 0) * Geo::G * N * ElemBytes<DT>::value;
  const int64_t comb = Geo::G > 1 ? static_cast<int64_t>(Geo::G) * Geo::SWEEP * 4 : 0;
  return stage > comb ? stage : comb;
}

// ---------------------------------------------------------------------------
// Backward stage 2 over a 16-column tile per workgroup: 4 float4 column
// quads x 64 slices of partial rows; slice s adds rows s, s+64, ... in
// float64, then 16 threads add the 64 slice sums in slice order.  Needs
// N % 4 == 0 (16-byte partial rows).
// ---------------------------------------------------------------------------
template <int OUT>
static __global__ __launch_bounds__(256) __attribute__((unused)) void bwd_reduce16_kernel(
    const float* __restrict__ part, void* __restrict__ dgamma, int64_t P, int N,
    const float* __restrict__ part_b, void* __restrict__ dgamma_b) {
  // A second [P, N] block (part_b, for LayerNorm's dbeta): the grid's
  // second half reduces it into dgamma_b, the same way.
  int bx = static_cast<int>(blockIdx.x);
  if (part_b != nullptr && bx >= static_cast<int>(gridDim.x / 2)) {
    bx -= static_cast<int>(gridDim.x / 2);
    part = part_b;
    dgamma = dgamma_b;
  }
  constexpr int kQuads = 4, kSlices = 64;
  __shared__ double sums[kSlices][kQuads * 4 + 1];
  const int q = threadIdx.x % kQuads;
  const int s = threadIdx.x / kQuads;
  const int col = bx * (kQuads * 4) + q * 4;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (col < N) {
    // Unrolled so that a thread's loads are in flight together; the adds
    // keep partial-row order.
#pragma unroll 8
    for (int64_t p = s; p < P; p += kSlices) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + p * N + col);
      a0 += v[0];
      a1 += v[1];
      a2 += v[2];
      a3 += v[3];
    }
  }
  sums[s][q * 4 + 0] = a0;
  sums[s][q * 4 + 1] = a1;
  sums[s][q * 4 + 2] = a2;
  sums[s][q * 4 + 3] = a3;
  __syncthreads();
  if (threadIdx.x < kQuads * 4) {
    const int c = bx * (kQuads * 4) + threadIdx.x;
    if (c < N) {
      double tot = 0.0;
      for (int i = 0; i < kSlices; ++i) tot += sums[i][threadIdx.x];
      store_dgamma<OUT>(dgamma, c, tot);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward stage 2 for long rows: each lane adds 4 adjacent columns with
// 16-byte loads, so one wavefront reads 1 KiB of a partial row; the S
// wavefronts of a workgroup (S = blockDim.x / 64, a power of two <= 16) take
// the partial rows s, s+S, ... of the same 256 columns in float64, and the
// S slice sums are then added in slice order.  Needs N % 4 == 0.
// ---------------------------------------------------------------------------
template <int OUT>
static __global__ __launch_bounds__(1024) __attribute__((unused)) void bwd_reduce_wide_kernel(
    const float* __restrict__ part, void* __restrict__ dgamma, int64_t P, int N,
    const float* __restrict__ part_b, void* __restrict__ dgamma_b) {
  // A second [P, N] block (part_b, for LayerNorm's dbeta): the grid's
  // second half reduces it into dgamma_b, the same way.
  int bx = static_cast<int>(blockIdx.x);
  if (part_b != nullptr && bx >= static_cast<int>(gridDim.x / 2)) {
    bx -= static_cast<int>(gridDim.x / 2);
    part = part_b;
    dgamma = dgamma_b;
  }
  constexpr int kCols = 256;
  __shared__ double sums[kMaxWavesPerBlock][kCols];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = threadIdx.x / kWave;
  const int S = blockDim.x / kWave;
  const int64_t col = static_cast<int64_t>(bx) * kCols + lane * 4;
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  if (col < N) {
#pragma unroll 8
    for (int64_t p = s; p < P; p += S) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + p * N + col);
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] += static_cast<double>(v[k]);
    }
  }
  if (S == 1) {
    if (col < N) {
#pragma unroll
      for (int k = 0; k < 4; ++k) store_dgamma<OUT>(dgamma, col + k, a[k]);
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) sums[s][lane * 4 + k] = a[k];
  __syncthreads();
  // blockDim.x is 128 .. 1024: each thread finishes every blockDim.x-th column.
  for (int j = threadIdx.x; j < kCols; j += blockDim.x) {
    const int64_t c = static_cast<int64_t>(bx) * kCols + j;
    if (c < N) {
      double tot = 0.0;
      for (int i = 0; i < S; ++i) tot += sums[i][j];
      store_dgamma<OUT>(dgamma, c, tot);
    }
  }
}

}  // namespace rmsnorm_hip
