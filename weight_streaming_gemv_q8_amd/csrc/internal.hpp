// Host-side helpers shared by the wsgemv translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wsgemv.h"

namespace wsg {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

// Status of the most recent launch on this thread (clears the sticky error).
inline int launch_status() { return hipGetLastError() == hipSuccess ? WSG_OK : WSG_ERR_HIP; }

// Per-device facts used to size grids (looked up once per device).
struct DeviceInfo {
    int cus = 0;
    int max_lds = 0;
};
const DeviceInfo& device_info();

// Waves per row the Q8_0 GEMV uses for this shape (the persistent kernel
// uses the same, so its rows are reduced in the same order).
int gemv_split(bool f32_act, int64_t n, int64_t k);

// Writes y[0..n) = 0 (the empty sum for k == 0).
int fill_zero_f32(float* y, int64_t n, hipStream_t stream);

}  // namespace wsg
