// Shape table and variant dispatch for f32 inputs.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
bool supported_f32(int P, int N, int QB) {
    const bool p = P == 16 || P == 32 || P == 64;
    const bool n = N == 16 || N == 32 || N == 64 || N == 128;
    const bool q = QB == 32 || QB == 64;
    return p && n && q;
}

hipError_t launch_scan_f32(int P, int N, int QB, bool seq, bool xscale, bool local, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (seq == false && xscale == false && local == false) return launch_scan_f32_s0_e0_l0(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == false && local == true) return launch_scan_f32_s0_e0_l1(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == true && local == false) return launch_scan_f32_s0_e1_l0(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == true && local == true) return launch_scan_f32_s0_e1_l1(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == false && local == false) return launch_scan_f32_s1_e0_l0(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == false && local == true) return launch_scan_f32_s1_e0_l1(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == true && local == false) return launch_scan_f32_s1_e1_l0(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == true && local == true) return launch_scan_f32_s1_e1_l1(P, N, QB, spw, prm, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_step_f32(int P, int N, const StepParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 16 && N == 16) { hipLaunchKernelGGL((ssd_step_kernel<float, 16, 16>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 32) { hipLaunchKernelGGL((ssd_step_kernel<float, 16, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 64) { hipLaunchKernelGGL((ssd_step_kernel<float, 16, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 16 && N == 128) { hipLaunchKernelGGL((ssd_step_kernel<float, 16, 128>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 16) { hipLaunchKernelGGL((ssd_step_kernel<float, 32, 16>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 32) { hipLaunchKernelGGL((ssd_step_kernel<float, 32, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 64) { hipLaunchKernelGGL((ssd_step_kernel<float, 32, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128) { hipLaunchKernelGGL((ssd_step_kernel<float, 32, 128>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 16) { hipLaunchKernelGGL((ssd_step_kernel<float, 64, 16>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 32) { hipLaunchKernelGGL((ssd_step_kernel<float, 64, 32>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64) { hipLaunchKernelGGL((ssd_step_kernel<float, 64, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128) { hipLaunchKernelGGL((ssd_step_kernel<float, 64, 128>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
