// Kernel instantiations: bf16 inputs, with sequence ids, with input scaling, scan.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
hipError_t launch_scan_bf16_s1_e1_l0(int P, int N, int QB, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (P == 32 && N == 64 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 64, 32, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 64, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 64, 64, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 64, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 128, 32, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 128, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 128, 64, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 128, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 256 && QB == 32 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 256, 32, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 256, 32, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 256 && QB == 64 && spw == 2) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 32, 256, 64, true, true, false, 2>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 32, 256, 64, 2>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 64, 32, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 64, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 64, 64, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 64, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 128, 32, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 128, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 128, 64, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 128, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 256 && QB == 32 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 256, 32, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 256, 32, 4>::NT), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 256 && QB == 64 && spw == 4) { hipLaunchKernelGGL((ssd_scan_kernel<__bf16, 64, 256, 64, true, true, false, 4>), dim3((unsigned)grid), dim3(ScanCfg<__bf16, 64, 256, 64, 4>::NT), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
