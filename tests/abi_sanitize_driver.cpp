// Host-side driver for the argument validation and plan arithmetic of the
// C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code only (tests/test_abi_sanitize_cpu.py builds and runs it).
//
// Every call below is one the library must reject before it enqueues
// anything (the page "Check an AI model calculation before accelerating it",
// section "The memory contract is part of the computation": a contract
// violation is refused before any output is written), or a pure query
// (workspace sizes, plans).  Pointers are fake addresses that are never
// dereferenced.  The driver refuses to run when a GPU is visible, so that no
// call can ever reach a device.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include <hip/hip_runtime_api.h>

#include "layernorm.h"
#include "rmsnorm.h"
#include "rmsnorm_add.h"
#include "rmsnorm_cast.h"

namespace {

int failures = 0;
int checks = 0;

void expect(const char* what, int got, int want) {
  ++checks;
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

void* at(uint64_t a) { return reinterpret_cast<void*>(a); }
float* fat(uint64_t a) { return reinterpret_cast<float*>(a); }

constexpr uint64_t A = 0x10000000ull;  // 16-byte aligned fake base
constexpr int64_t T40 = int64_t(1) << 40;
constexpr int64_t T22 = int64_t(1) << 22;

const rmsnorm_dtype_t kDtypes[] = {RMSNORM_F32, RMSNORM_F16, RMSNORM_BF16};

// Row pitches that make (M - 1) * pitch pass 2^63 (or 2^57) with y == x: the
// layouts must be refused as strides that do not fit, never launched.
void address_limits() {
  for (rmsnorm_dtype_t dt : kDtypes) {
    for (int64_t ld : {T40, T22, int64_t(1) << 30}) {
      expect("rmsnorm_fwd_strided y==x huge pitch",
             rmsnorm_fwd_strided(at(A), ld, at(A), 1e-6f, T40, 1, dt, 0, at(A), ld, fat(A),
                                 nullptr),
             RMSNORM_ERR_STRIDE);
      expect("rmsnorm_fwd_strided disjoint huge pitch",
             rmsnorm_fwd_strided(at(A), ld, at(A + (1ull << 20)), 1e-6f, T40, 1, dt, 0,
                                 at(A + (2ull << 20)), ld, fat(A + (3ull << 20)), nullptr),
             RMSNORM_ERR_STRIDE);
      expect("rmsnorm_bwd_strided huge pitch",
             rmsnorm_bwd_strided(at(A), ld, at(A), ld, at(A + 64), fat(A + 128), T40, 1, dt, 0,
                                 at(A), ld, at(A + 256), at(A + 512), size_t(1) << 40, nullptr),
             RMSNORM_ERR_STRIDE);
      expect("layernorm_fwd huge pitch",
             layernorm_fwd(at(A), ld, at(A + 64), at(A + 128), 1e-5f, T40, 1, dt, 0, at(A), ld,
                           fat(A + 256), fat(A + 512), nullptr),
             RMSNORM_ERR_STRIDE);
      expect("rmsnorm_add_fwd huge pitch",
             rmsnorm_add_fwd(at(A), ld, at(A), ld, at(A + 64), 1e-6f, T40, 1, dt, 0, at(A), ld,
                             at(A), ld, fat(A + 128), nullptr),
             RMSNORM_ERR_STRIDE);
      expect("rmsnorm_cast_fwd huge pitch",
             rmsnorm_cast_fwd(at(A), ld, at(A + 64), 1e-6f, T40, 1, RMSNORM_F32, RMSNORM_BF16, 0,
                              at(A), ld, fat(A + 128), nullptr),
             RMSNORM_ERR_STRIDE);
    }
  }
  // Dense rows ending past 2^57 (a base near the top of the address space).
  const uint64_t top = (uint64_t(1) << 57) - 1024;
  expect("rmsnorm_fwd past the address limit",
         rmsnorm_fwd(at(top), at(A), 1e-6f, 4, 256, RMSNORM_BF16, 0, at(A + 4096),
                     fat(A + 8192), nullptr),
         RMSNORM_ERR_SHAPE);
  // Overlap found through the row-against-row test at pitches near 2^41 bytes:
  // y's row 0 is x's row 1.
  expect("rmsnorm_fwd_strided y = next row of x",
         rmsnorm_fwd_strided(at(A), T40, at(A + 64), 1e-6f, int64_t(1) << 14, 8, RMSNORM_BF16, 0,
                             at(A + (uint64_t(T40) << 1)), T40, fat(A + 128), nullptr),
         RMSNORM_ERR_OVERLAP);
}

void plain_rejections() {
  for (rmsnorm_dtype_t dt : kDtypes) {
    expect("fwd null x", rmsnorm_fwd(nullptr, at(A), 1e-6f, 4, 256, dt, 0, at(A + 4096),
                                     fat(A + 8192), nullptr),
           RMSNORM_ERR_NULL_POINTER);
    expect("fwd bad eps", rmsnorm_fwd(at(A), at(A + 1024), 0.0f, 4, 256, dt, 0, at(A + 4096),
                                      fat(A + 8192), nullptr),
           RMSNORM_ERR_EPS);
    expect("fwd N too large", rmsnorm_fwd(at(A), at(A), 1e-6f, 4, RMSNORM_MAX_N + 1, dt, 0,
                                          at(A), fat(A), nullptr),
           RMSNORM_ERR_SHAPE);
    expect("fwd M*N too large", rmsnorm_fwd(at(A), at(A), 1e-6f, RMSNORM_MAX_M, 65537, dt, 0,
                                            at(A), fat(A), nullptr),
           RMSNORM_ERR_SHAPE);
    expect("fwd y overlaps x", rmsnorm_fwd(at(A), at(A + (1u << 24)), 1e-6f, 4, 256, dt, 0,
                                           at(A + 8), fat(A + (3u << 24)), nullptr),
           RMSNORM_ERR_OVERLAP);
    expect("bwd short workspace",
           rmsnorm_bwd(at(A), at(A + (1u << 24)), at(A + (2u << 24)), fat(A + (3u << 24)), 64,
                       4096, dt, 0, at(A + (4u << 24)), at(A + (5u << 24)), at(A + (6u << 24)),
                       16, nullptr),
           RMSNORM_ERR_WORKSPACE);
    expect("bwd bad flags",
           rmsnorm_bwd(at(A), at(A), at(A), fat(A), 64, 4096, dt, 8, at(A), at(A), at(A), 0,
                       nullptr),
           RMSNORM_ERR_FLAGS);
    expect("bwd_reduce short workspace",
           rmsnorm_bwd_reduce(at(A), 4, 1 << 20, 4096, dt, 0, at(A + (1u << 26)), nullptr),
           RMSNORM_ERR_WORKSPACE);
    expect("layernorm N too large",
           layernorm_fwd(at(A), LAYERNORM_MAX_N + 1, at(A), at(A), 1e-5f, 4, LAYERNORM_MAX_N + 1,
                         dt, 0, at(A), LAYERNORM_MAX_N + 1, fat(A), fat(A), nullptr),
           RMSNORM_ERR_SHAPE);
    expect("layernorm M*N too large",
           layernorm_fwd(at(A), 65537, at(A), at(A), 1e-5f, RMSNORM_MAX_M, 65537, dt, 0, at(A),
                         65537, fat(A), fat(A), nullptr),
           RMSNORM_ERR_SHAPE);
    expect("add stride below N",
           rmsnorm_add_fwd(at(A), 100, at(A), 256, at(A), 1e-6f, 4, 256, dt, 0, at(A), 256,
                           at(A), 256, fat(A), nullptr),
           RMSNORM_ERR_STRIDE);
  }
  {
    // The allocation-free backward: the need above its fixed buffer, and
    // caller arguments, are refused before the buffer is looked up.
    const uint64_t big = uint64_t(32) << 26;
    expect("bwd_noalloc beyond its buffer",
           rmsnorm_bwd_noalloc(at(A), at(A + big), at(A + 2 * big), fat(A + 3 * big), 32,
                               RMSNORM_MAX_N, RMSNORM_F32, 0, at(A + 4 * big), at(A + 5 * big),
                               nullptr),
           RMSNORM_ERR_WORKSPACE);
    expect("bwd_noalloc null dy",
           rmsnorm_bwd_noalloc(nullptr, at(A), at(A), fat(A), 4, 256, RMSNORM_BF16, 0, at(A),
                               at(A), nullptr),
           RMSNORM_ERR_NULL_POINTER);
    expect("bwd_noalloc dx overlaps x",
           rmsnorm_bwd_noalloc(at(A), at(A + (1u << 24)), at(A + (2u << 24)),
                               fat(A + (3u << 24)), 4, 256, RMSNORM_BF16, 0,
                               at(A + (1u << 24) + 64), at(A + (5u << 24)), nullptr),
           RMSNORM_ERR_OVERLAP);
    expect("bwd_noalloc huge M*N",
           rmsnorm_bwd_noalloc(at(A), at(A), at(A), fat(A), RMSNORM_MAX_M, 4096, RMSNORM_BF16, 0,
                               at(A), at(A), nullptr),
           RMSNORM_ERR_SHAPE);
  }
  expect("cast same dtype",
         rmsnorm_cast_fwd(at(A), 256, at(A + 4096), 1e-6f, 4, 256, RMSNORM_F32, RMSNORM_F32, 0,
                          at(A + 8192), 256, fat(A + 16384), nullptr),
         RMSNORM_ERR_DTYPE);
  expect("bad dtype", rmsnorm_fwd(at(A), at(A), 1e-6f, 4, 256, static_cast<rmsnorm_dtype_t>(7),
                                  0, at(A), fat(A), nullptr),
         RMSNORM_ERR_DTYPE);
}

// Workspace sizes and plans over the whole accepted domain, so that the plan
// arithmetic runs under the sanitizers at its extremes.
void queries() {
  const int64_t Ms[] = {0, 1, 2, 63, 65, 4096, 32768, 262144, int64_t(1) << 30,
                        RMSNORM_MAX_M};
  const int64_t Ns[] = {1, 2, 3, 127, 128, 1024, 4096, 5120, 16384, 65535, 65536, 65537,
                        131072, 1000003, RMSNORM_MAX_N};
  rmsnorm_plan_t plan;
  for (rmsnorm_dtype_t dt : kDtypes) {
    for (int64_t M : Ms) {
      for (int64_t N : Ns) {
        if (M > 0 && M > RMSNORM_MAX_ELEMENTS / N) continue;
        for (uint32_t flags : {0u, 1u, 2u, 3u}) {
          ++checks;
          (void)rmsnorm_bwd_workspace_bytes(M, N, dt, flags);
          for (int pass = 0; pass < 3; ++pass)
            for (int align : {2, 4, 8, 16}) (void)rmsnorm_query_plan(M, N, dt, flags, pass, align, &plan);
        }
        (void)layernorm_bwd_workspace_bytes(M, N, dt, 0);
        for (int pass = 0; pass < 3; ++pass)
          for (int align : {2, 4, 8, 16}) (void)layernorm_query_plan(M, N, dt, 0, pass, align, &plan);
        if (N <= RMSNORM_ADD_MAX_N) {
          (void)rmsnorm_add_bwd_workspace_bytes(M, N, dt, 0);
          for (int pass = 0; pass < 3; ++pass)
            for (int align : {2, 4, 8, 16}) (void)rmsnorm_add_query_plan(M, N, dt, 0, pass, align, &plan);
        }
      }
    }
  }
  for (int64_t M : Ms)
    for (int64_t N : Ns)
      if (N <= RMSNORM_CAST_MAX_N)
        (void)rmsnorm_cast_bwd_workspace_bytes(M, N, RMSNORM_F32, RMSNORM_BF16, 0);
  for (int code = -12; code <= 1; ++code) (void)rmsnorm_status_string(code);
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("SKIP: a GPU is visible; this driver runs on hosts without one\n");
    return 77;
  }
  address_limits();
  plain_rejections();
  queries();
  std::printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
