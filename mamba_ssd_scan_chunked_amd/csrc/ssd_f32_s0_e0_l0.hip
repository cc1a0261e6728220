// Kernel instantiations: f32 inputs, without sequence ids, without Euler input scaling, scan.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
hipError_t launch_scan_f32_s0_e0_l0(int P, int N, int QB, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (P == 16 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 16, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 16, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 32, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 32, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 64, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 64, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 128, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 128, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 16, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 16, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 32, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 32, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 64, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 64, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 128, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 128, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 16, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 16, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 32, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 32, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 64, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 64, 64>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 32) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 32, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 128, 32>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 64) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 64, false, false, false>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 128, 64>::NT), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
