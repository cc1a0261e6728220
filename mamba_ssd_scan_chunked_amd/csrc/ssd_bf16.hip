// Shape table and variant dispatch for bf16 inputs.
#include "ssd_kernels.hpp"
#include "ssd_launch.hpp"

namespace ssd {
bool supported_bf16(int P, int N, int QB) {
    const bool p = P == 32 || P == 64;
    const bool n = N == 64 || N == 128 || N == 256;
    const bool q = QB == 32 || QB == 64;
    return p && n && q;
}

hipError_t launch_scan_bf16(int P, int N, int QB, bool seq, bool xscale, bool local, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (seq == false && xscale == false && local == false) return launch_scan_bf16_s0_e0_l0(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == false && local == true) return launch_scan_bf16_s0_e0_l1(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == true && local == false) return launch_scan_bf16_s0_e1_l0(P, N, QB, spw, prm, grid, s);
    if (seq == false && xscale == true && local == true) return launch_scan_bf16_s0_e1_l1(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == false && local == false) return launch_scan_bf16_s1_e0_l0(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == false && local == true) return launch_scan_bf16_s1_e0_l1(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == true && local == false) return launch_scan_bf16_s1_e1_l0(P, N, QB, spw, prm, grid, s);
    if (seq == true && xscale == true && local == true) return launch_scan_bf16_s1_e1_l1(P, N, QB, spw, prm, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_step_bf16(int P, int N, const StepParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 32 && N == 64) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 32, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 128) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 32, 128>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 32 && N == 256) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 32, 256>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 64) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 64, 64>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 128) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 64, 128>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    if (P == 64 && N == 256) { hipLaunchKernelGGL((ssd_step_kernel<__bf16, 64, 256>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
