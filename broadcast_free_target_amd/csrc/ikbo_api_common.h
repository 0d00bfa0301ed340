// Host-side helpers shared by the exported C functions of libikbo.so: the
// per-thread last error, status returns, grow-only device and pinned host
// buffers, range checks.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <string>

#include "ikbo.h"

namespace ikbo_host {

// Message of the last failing call on this thread (ikbo_last_error).
extern thread_local std::string g_last_error;

inline int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

inline int fail_hip(hipError_t e, const char* what) {
  return fail(IKBO_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define IKBO_HIP(call)                          \
  do {                                          \
    hipError_t e_ = (call);                     \
    if (e_ != hipSuccess) return fail_hip(e_, #call); \
  } while (0)

inline int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (!s || !*s) return dflt;
  return std::atoi(s);
}

inline size_t elem_size(int32_t dtype) { return dtype == IKBO_DTYPE_F32 ? 4 : 2; }

constexpr int kMaxTimed = 4096;  // launches a plan can time between resets

// Grow-only device buffer.
struct DevBuf {
  void* ptr = nullptr;
  size_t cap = 0;
  int ensure(size_t bytes, bool zero) {
    if (bytes <= cap) return IKBO_OK;
    if (ptr) {
      hipError_t e = hipFree(ptr);  // hipFree waits for work that may still use the buffer
      ptr = nullptr;
      cap = 0;
      if (e != hipSuccess) return fail_hip(e, "hipFree");
    }
    size_t want = std::max<size_t>(bytes, 256);
    hipError_t e = hipMalloc(&ptr, want);
    if (e != hipSuccess) {
      ptr = nullptr;
      return fail(IKBO_ERR_NOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
    }
    if (zero) {
      e = hipMemset(ptr, 0, want);
      if (e != hipSuccess) return fail_hip(e, "hipMemset");
    }
    cap = want;
    return IKBO_OK;
  }
  void release() {
    if (ptr) (void)hipFree(ptr);
    ptr = nullptr;
    cap = 0;
  }
};

// Grow-only pinned host buffer (host-cached).  Work lists read in place by a
// kernel are written before the launch that reads them and never rewritten
// until that launch has completed (stage events), so the kernel boundary
// orders every host write before the device reads it.
struct PinnedBuf {
  void* ptr = nullptr;
  size_t cap = 0;
  int ensure(size_t bytes, bool coherent = false) {
    if (bytes <= cap) return IKBO_OK;
    if (ptr) (void)hipHostFree(ptr);
    ptr = nullptr;
    cap = 0;
    size_t want = std::max<size_t>(bytes, 4096);
    hipError_t e = hipHostMalloc(&ptr, want, coherent ? hipHostMallocCoherent : hipHostMallocDefault);
    if (e != hipSuccess) {
      ptr = nullptr;
      return fail(IKBO_ERR_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    }
    cap = want;
    return IKBO_OK;
  }
  void release() {
    if (ptr) (void)hipHostFree(ptr);
    ptr = nullptr;
    cap = 0;
  }
};

inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

inline int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

}  // namespace ikbo_host
