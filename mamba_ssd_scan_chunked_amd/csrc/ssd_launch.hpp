// Internal interface between the host library (ssd_api.cpp) and the kernel
// instantiations (ssd_bf16.hip, ssd_f32.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {
struct ScanParams;
struct CombineParams;
struct StepParams;
struct BwdParams;

// Return hipSuccess, hipErrorInvalidValue for a shape with no instantiation,
// or the launch error.
// seq: sequence ids present (segment handling compiled in); xscale: x scaled per token (Euler or zero-order hold);
// local: the local pass of a row split into segments (else the scan proper);
// spw: 16-channel slices per workgroup (P / 16: one head per workgroup)
hipError_t launch_scan_bf16(int P, int N, int QB, bool seq, bool xscale, bool local, int spw, const ScanParams& prm,
                            int64_t grid, hipStream_t s);
hipError_t launch_scan_f32(int P, int N, int QB, bool seq, bool xscale, bool local, int spw, const ScanParams& prm,
                           int64_t grid, hipStream_t s);
hipError_t launch_combine(const CombineParams& prm, hipStream_t s);
hipError_t launch_step_bf16(int P, int N, const StepParams& prm, int64_t grid, hipStream_t s);
hipError_t launch_step_f32(int P, int N, const StepParams& prm, int64_t grid, hipStream_t s);
#define SSD_DECLARE_SCAN(tag, sq, eu, lo) \
    hipError_t launch_scan_##tag##_s##sq##_e##eu##_l##lo(int P, int N, int QB, int spw, const ScanParams& prm, int64_t grid, hipStream_t s);
#define SSD_DECLARE_SCAN2(tag, sq, eu) SSD_DECLARE_SCAN(tag, sq, eu, 0) SSD_DECLARE_SCAN(tag, sq, eu, 1)
SSD_DECLARE_SCAN2(bf16, 0, 0)
SSD_DECLARE_SCAN2(bf16, 0, 1)
SSD_DECLARE_SCAN2(bf16, 1, 0)
SSD_DECLARE_SCAN2(bf16, 1, 1)
SSD_DECLARE_SCAN2(f32, 0, 0)
SSD_DECLARE_SCAN2(f32, 0, 1)
SSD_DECLARE_SCAN2(f32, 1, 0)
SSD_DECLARE_SCAN2(f32, 1, 1)
#undef SSD_DECLARE_SCAN2
#undef SSD_DECLARE_SCAN

bool supported_bf16(int P, int N, int QB);
bool supported_f32(int P, int N, int QB);

// Backward: the forward pass then the reverse pass, one workgroup per (row, head).
hipError_t launch_bwd_bf16(int P, int N, const BwdParams& prm, int64_t grid, hipStream_t s);
hipError_t launch_bwd_f32(int P, int N, const BwdParams& prm, int64_t grid, hipStream_t s);
bool supported_bwd_bf16(int P, int N);
bool supported_bwd_f32(int P, int N);
int bwd_block_bf16();   // tokens per block of the backward kernels
int bwd_block_f32();
// Reverse local pass of rows split into segments (one workgroup per (row, head, segment > 0)).
hipError_t launch_bwd_klocal_bf16(int P, int N, const BwdParams& prm, float* kloc, float* kcarry, int64_t grid,
                                  hipStream_t s);
hipError_t launch_bwd_klocal_f32(int P, int N, const BwdParams& prm, float* kloc, float* kcarry, int64_t grid,
                                 hipStream_t s);
}  // namespace ssd
