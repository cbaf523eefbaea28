// Host-side helpers shared by the entry points of libqmv.so: the thread-local
// error message, argument checks and per-device launch facts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "qmv.h"

namespace qmv {

// Records the message for qmv_last_error() and returns code.
int32_t fail(int32_t code, const char* fmt, ...);
// Clears the message (called on every successful return).
int32_t ok();

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Workgroups of `kernel` (block threads, dynamic LDS bytes) that fit on one
// compute unit at once (cached per kernel and LDS size; at least 1).
int resident_wgs(const void* kernel, int threads, size_t lds);

// Maps the status of the launch just issued to a return code.
int32_t check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace qmv
