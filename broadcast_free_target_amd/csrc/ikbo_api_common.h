// Host-side helpers shared by the exported C functions of libikbo.so: the
// per-thread last error, status returns, grow-only device and pinned host
// buffers, range checks.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <string>
#include <vector>

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
  void* dev = nullptr;  // the device's address of the same memory, taken once per allocation
  size_t cap = 0;
  int ensure(size_t bytes, bool coherent = false) {
    if (bytes <= cap) return IKBO_OK;
    if (ptr) (void)hipHostFree(ptr);
    ptr = dev = nullptr;
    cap = 0;
    size_t want = std::max<size_t>(bytes, 4096);
    hipError_t e = hipHostMalloc(&ptr, want, coherent ? hipHostMallocCoherent : hipHostMallocDefault);
    if (e != hipSuccess) {
      ptr = nullptr;
      return fail(IKBO_ERR_NOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    }
    e = hipHostGetDevicePointer(&dev, ptr, 0);
    if (e != hipSuccess) {
      (void)hipHostFree(ptr);
      ptr = dev = nullptr;
      return fail_hip(e, "hipHostGetDevicePointer");
    }
    cap = want;
    return IKBO_OK;
  }
  void release() {
    if (ptr) (void)hipHostFree(ptr);
    ptr = dev = nullptr;
    cap = 0;
  }
};

// Pinned host buffers handed out in turn to successive calls whose kernels
// read them in place (work lists).  A buffer is reused only after the last
// launch that read it has finished.  Completion is tracked by an event
// recorded every kEventEvery launches, not after each one: an event after
// every launch puts a barrier packet between consecutive calls on the stream
// (measured at about 4.5 us per call).  Reusing a buffer means waiting for the
// first periodic event at or after its last reader, which has normally long
// fired: with kStages > kEventEvery buffers a call waits only when the host
// is more than kStages - kEventEvery launches ahead of the device.  If that
// event has not been recorded yet, one is recorded on the last launch's
// stream and waited for.  The events only order launches on their own stream,
// so before anything is enqueued on a different stream than the previous
// launch's, on_stream waits for the previous stream to drain (every buffer,
// and whatever else the owner's launches share, is then free).  One host
// thread per ring.
struct PinnedRing {
  static constexpr int kStages = 16;
  static constexpr int kEventEvery = 8;
  static constexpr int kEvents = 4;
  PinnedBuf buf[kStages];
  int64_t last[kStages];        // last launch that read the buffer, -1 if none
  hipEvent_t ev[kEvents] = {};
  int64_t ev_seq[kEvents];      // launch each event was recorded after, -1 if none
  hipEvent_t flush = nullptr;
  int64_t n_launch = 0;
  hipStream_t last_stream = nullptr;
  bool launched_any = false;
  int next = 0;

  int init() {
    for (int i = 0; i < kStages; ++i) last[i] = -1;
    for (int i = 0; i < kEvents; ++i) {
      ev_seq[i] = -1;
      IKBO_HIP(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming));
    }
    IKBO_HIP(hipEventCreateWithFlags(&flush, hipEventDisableTiming));
    return IKBO_OK;
  }
  void release() {
    for (int i = 0; i < kEvents; ++i)
      if (ev[i]) (void)hipEventDestroy(ev[i]);
    if (flush) (void)hipEventDestroy(flush);
    for (int i = 0; i < kStages; ++i) buf[i].release();
  }
  // Waits until launch L and every earlier one have finished.
  int wait(int64_t L) {
    if (L < 0) return IKBO_OK;
    const int64_t n_e = (L / kEventEvery) * kEventEvery + kEventEvery - 1;  // first event covering L
    const int slot = static_cast<int>((n_e / kEventEvery) % kEvents);
    if (ev_seq[slot] >= n_e) {  // that event, or a later one recorded in its slot
      IKBO_HIP(hipEventSynchronize(ev[slot]));
      return IKBO_OK;
    }
    IKBO_HIP(hipEventRecord(flush, last_stream));
    IKBO_HIP(hipEventSynchronize(flush));
    return IKBO_OK;
  }
  // The next buffer, at least `bytes` long, once its last reader is done.
  // When a request outgrows the buffers, all of them are reallocated at once
  // (with half again as much room), after every launch that may still read
  // one has finished: buffers are never allocated one call at a time, so a
  // steady stream of requests of similar size allocates nothing after its
  // first call.
  int acquire(size_t bytes, int* idx) {
    const int s = next;
    next = (s + 1) % kStages;
    int rc = IKBO_OK;
    if (bytes > buf[s].cap) {
      if ((rc = wait(n_launch - 1)) != IKBO_OK) return rc;
      const size_t want = bytes + bytes / 2;
      for (int i = 0; i < kStages; ++i) {
        if ((rc = buf[i].ensure(want)) != IKBO_OK) return rc;
        last[i] = -1;
      }
    } else if ((rc = wait(last[s])) != IKBO_OK) {
      return rc;
    }
    *idx = s;
    return IKBO_OK;
  }
  // To be called before enqueuing work on `stream`: if the previous launch
  // went to another stream, waits for that stream to drain.
  int on_stream(hipStream_t stream) {
    if (launched_any && stream != last_stream) {
      IKBO_HIP(hipStreamSynchronize(last_stream));
      for (int i = 0; i < kStages; ++i) last[i] = -1;
      for (int i = 0; i < kEvents; ++i) ev_seq[i] = -1;
      last_stream = stream;
    }
    return IKBO_OK;
  }
  // Notes that the launch just enqueued on `stream` reads buffer idx.
  int launched(int idx, hipStream_t stream) {
    launched_any = true;
    const int64_t seq = n_launch++;
    last[idx] = seq;
    last_stream = stream;
    if (seq % kEventEvery == kEventEvery - 1) {
      const int slot = static_cast<int>((seq / kEventEvery) % kEvents);
      IKBO_HIP(hipEventRecord(ev[slot], stream));
      ev_seq[slot] = seq;
    }
    return IKBO_OK;
  }
};

// Timing events of the measurement entry points: four per timed call (two
// kernels' start and end, stamped by their dispatches), created in batches
// when timing is switched on and when a batch runs out, so that a timed call
// normally creates none.  `flag` records per timed call whether its optional
// second kernel ran.
struct TimedEvents {
  static constexpr int kBatch = 256;  // calls per batch of events
  std::vector<hipEvent_t> ev;
  std::vector<char> flag;
  int n = 0;
  bool on = false;

  int reserve(int calls) {
    calls = std::min(calls, kMaxTimed);
    while (ev.size() < static_cast<size_t>(4 * calls)) {
      hipEvent_t e;
      IKBO_HIP(hipEventCreate(&e));
      ev.push_back(e);
    }
    if (flag.size() < static_cast<size_t>(calls)) flag.resize(calls);
    return IKBO_OK;
  }
  // Switches timing on or off; both reset the record.
  int enable(bool e) {
    on = e;
    n = 0;
    return e ? reserve(kBatch) : IKBO_OK;
  }
  // The four events of the next timed call (null when timing is off or the
  // record is full) and notes its flag.
  int next(hipEvent_t** te, bool flag_value) {
    *te = nullptr;
    if (!on || n >= kMaxTimed) return IKBO_OK;
    if (static_cast<size_t>(4 * (n + 1)) > ev.size()) {
      int rc = reserve(n + kBatch);
      if (rc != IKBO_OK) return rc;
    }
    *te = &ev[4 * n];
    flag[n] = flag_value ? 1 : 0;
    ++n;
    return IKBO_OK;
  }
  void release() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    ev.clear();
    flag.clear();
    n = 0;
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
