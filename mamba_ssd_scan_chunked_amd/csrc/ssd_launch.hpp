// Internal interface between the host library (ssd_api.cpp) and the kernel
// instantiations (ssd_bf16.hip, ssd_f32.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {
struct PrepParams;
struct ScanParams;

// Return hipSuccess, hipErrorInvalidValue for a shape with no instantiation,
// or the launch error.
hipError_t launch_prep_bf16(int N, int QB, const PrepParams& prm, int64_t grid, hipStream_t s);
hipError_t launch_scan_bf16(int P, int N, int QB, const ScanParams& prm, int64_t grid, hipStream_t s);
hipError_t launch_prep_f32(int N, int QB, const PrepParams& prm, int64_t grid, hipStream_t s);
hipError_t launch_scan_f32(int P, int N, int QB, const ScanParams& prm, int64_t grid, hipStream_t s);

bool supported_bf16(int P, int N, int QB);
bool supported_f32(int P, int N, int QB);
}  // namespace ssd
