// qg_internal.h -- host helpers shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemv.h"

namespace qg {

// Records `status` and a printf-style detail for qg_last_error_detail (per
// thread) and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();

// QG_OK when the current device is a gfx950 GPU (cached per device).
int check_device();

// Maps a failed HIP call to QG_ELAUNCH with the call's name.
int hip_status(hipError_t e, const char* what);

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace qg
