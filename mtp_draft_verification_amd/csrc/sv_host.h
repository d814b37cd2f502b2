// sv_host.h -- host-side helpers of libspecverify (argument checks, launch status).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/specverify.h"

namespace sv {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// SV_OK if the current device is a gfx950 (cached per device after the first query).
int check_device();

// number of compute units of the current device (cached)
int device_cus();

// SV_OK, or SV_ERR_LAUNCH if the runtime recorded a failed launch
inline int launch_status() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH; }

}  // namespace sv
