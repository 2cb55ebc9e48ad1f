// Host-side helpers of the libmoefp8 C ABI: status/detail reporting,
// argument checks that never touch the device, and the post-launch check.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/moefp8.h"

namespace moefp8 {

// Sets the calling thread's detail message and returns `s`.
moe_status fail(moe_status s, const char* fmt, ...);
// Clears the detail message (called on entry by every ABI function).
void clear_detail();
// After enqueueing: hipGetLastError -> MOE_ERR_HIP; with MOEFP8_SYNC_CHECK=1
// also synchronises `stream` and reports asynchronous errors.
moe_status after_launch(const char* what, hipStream_t stream);
// Compute units of the current device (256 if the runtime cannot say).
int device_cu_count();

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline unsigned ceil_div_u(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Element counts above 2^40 exceed any device memory; entry points refuse
// them (MOE_ERR_UNSUPPORTED) before any size arithmetic that could overflow.
constexpr int64_t kMaxElems = int64_t(1) << 40;
// a * b <= kMaxElems for non-negative a, b (no overflow in the test itself).
inline bool elems_ok(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (b == 0 || a <= kMaxElems / b); }

}  // namespace moefp8

#define MOE_REQUIRE(cond, status, ...)                  \
  do {                                                  \
    if (!(cond)) return ::moefp8::fail(status, __VA_ARGS__); \
  } while (0)
