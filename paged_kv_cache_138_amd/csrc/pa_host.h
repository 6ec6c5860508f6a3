// Host-side helpers of libpa: error reporting and argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "pa.h"

namespace pa {

// Records a failure for pa_last_error() and returns the status.
pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Checks a kernel launch that just happened.
pa_status check_launch(const char* what);

}  // namespace pa

#define PA_REQUIRE(cond, status, ...)                 \
    do {                                              \
        if (!(cond)) return ::pa::fail(status, __VA_ARGS__); \
    } while (0)
