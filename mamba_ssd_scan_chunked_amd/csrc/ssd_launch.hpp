// Internal interface between the host library (ssd_api.cpp) and the kernel
// instantiations (ssd_bf16.hip, ssd_f32.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {
struct ScanParams;

// Return hipSuccess, hipErrorInvalidValue for a shape with no instantiation,
// or the launch error.
// seq: sequence ids present (segment handling compiled in); euler: dt scales x
hipError_t launch_scan_bf16(int P, int N, int QB, bool seq, bool euler, const ScanParams& prm, int64_t grid,
                            hipStream_t s);
hipError_t launch_scan_f32(int P, int N, int QB, bool seq, bool euler, const ScanParams& prm, int64_t grid,
                           hipStream_t s);
#define SSD_DECLARE_SCAN(tag, sq, eu) \
    hipError_t launch_scan_##tag##_s##sq##_e##eu(int P, int N, int QB, const ScanParams& prm, int64_t grid, hipStream_t s);
SSD_DECLARE_SCAN(bf16, 0, 0)
SSD_DECLARE_SCAN(bf16, 0, 1)
SSD_DECLARE_SCAN(bf16, 1, 0)
SSD_DECLARE_SCAN(bf16, 1, 1)
SSD_DECLARE_SCAN(f32, 0, 0)
SSD_DECLARE_SCAN(f32, 0, 1)
SSD_DECLARE_SCAN(f32, 1, 0)
SSD_DECLARE_SCAN(f32, 1, 1)
#undef SSD_DECLARE_SCAN

bool supported_bf16(int P, int N, int QB);
bool supported_f32(int P, int N, int QB);
}  // namespace ssd
