// Kernel instantiations: f32 inputs, with sequence ids, without input scaling, scan.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
hipError_t launch_scan_f32_s1_e0_l0(int P, int N, int QB, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (P == 16 && N == 16 && QB == 32 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 32, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 16, 32, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 16 && QB == 64 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 16, 64, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 16, 64, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 32 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 32, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 32, 32, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32 && QB == 64 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 32, 64, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 32, 64, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 32 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 32, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 64, 32, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64 && QB == 64 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 64, 64, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 64, 64, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 32 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 32, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 128, 32, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128 && QB == 64 && spw == 1) { hipLaunchKernelGGL((ssd_scan_kernel<float, 16, 128, 64, true, false, false, 1>), dim3((unsigned)grid), dim3(ScanCfg<float, 16, 128, 64, 1>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 32, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 16, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 16, 64, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 16, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 32, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 32, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 32, 64, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 32, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 32, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 64, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 64, 64, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 64, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 32, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 128, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<float, 32, 128, 64, true, false, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<float, 32, 128, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 32, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 16, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 16, 64, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 16, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 32, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 32, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 32, 64, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 32, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 32, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 64, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 64, 64, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 64, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 32, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 128, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<float, 64, 128, 64, true, false, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<float, 64, 128, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
