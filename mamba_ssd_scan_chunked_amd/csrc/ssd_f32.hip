// Kernel instantiations for f32 inputs.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
bool supported_f32(int P, int N, int QB) {
    const bool p = P == 16 || P == 32 || P == 64;
    const bool n = N == 16 || N == 32 || N == 64 || N == 128;
    const bool q = QB == 32 || QB == 64;
    return p && n && q;
}

hipError_t launch_prep_f32(int N, int QB, const PrepParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_prep_kernel<float, 16, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_prep_kernel<float, 16, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_prep_kernel<float, 32, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_prep_kernel<float, 32, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_prep_kernel<float, 64, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_prep_kernel<float, 64, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_prep_kernel<float, 128, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_prep_kernel<float, 128, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}

hipError_t launch_scan_f32(int P, int N, int QB, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 16 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 32>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 64>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 32>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 64>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 32>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 64>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 32>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 64>), dim3((unsigned)grid), dim3(64), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 32>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 64>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 32>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 64>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 32>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 64>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 32>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 64>), dim3((unsigned)grid), dim3(128), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
