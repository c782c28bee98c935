// frt_host.h -- host-side helpers shared by the C ABI's translation units:
// the per-thread last-error text, status-returning checks of HIP calls, the
// device guard, workspace alignment and the prefill GEMM's configuration
// choice.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/frt_ffn.h"

namespace frt {

// one text per thread for every entry point of the library (inline: a single
// instance across translation units)
inline std::string& last_error_text() {
  static thread_local std::string s;
  return s;
}

inline frt_status fail(frt_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  last_error_text() = buf;
  return st;
}

// Keep the plan's device current for the duration of a call, then restore.
struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

int env_int(const char* name, int dflt);
// LDS-DMA GEMM (k_mm) tile configuration (and K split when allowed) for an
// [M] x [N] output over K; cfg < 0 when no configuration fits.
// Configurations [0, ncfg) are considered: the FFN GEMMs use the first six,
// the attention input all eight (6 and 7 are small tiles for short outputs).
constexpr int kMMConfigCount = 6;     // FFN candidates 0..5 of the cost model
constexpr int kMMConfigCountAll = 8;  // 6, 7: the attention input's small tiles
constexpr int kMMConfigTwoPerCU = 8;  // 128 x 256, two workgroups per CU (FFN)
constexpr int kMMConfigEightWaves = 9;  // 256 x 192, eight waves: configuration 2 on the f16 cores (FFN)
inline bool mm_config_ffn(int c) {
  return (c >= 0 && c < kMMConfigCount) || c == kMMConfigTwoPerCU || c == kMMConfigEightWaves;
}
void choose_mm(int M, int N, int K, bool allow_split, int& cfg, int& split, int ncfg = kMMConfigCount);
int mm_config_bm(int);
int mm_config_bn(int);
int mm_config_ks(int);

}  // namespace frt

#define HIP_CHECK(call)                                                                    \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return frt::fail(FRT_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

#define KERNEL_CHECK(call, name)                                                           \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) return frt::fail(FRT_ERR_HIP, "launch of %s failed: %s", name, hipGetErrorString(e_)); \
  } while (0)
