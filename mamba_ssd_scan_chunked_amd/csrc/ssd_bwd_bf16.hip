// Backward kernels (forward and reverse pass) for bf16 inputs.
#include "ssd_bwd.hpp"
#include "ssd_launch.hpp"

namespace ssd {
bool supported_bwd_bf16(int P, int N) {
    return (P == 32 || P == 64) && (N == 64 || N == 128 || N == 256);
}

int bwd_block_bf16() { return 64; }

hipError_t launch_bwd_bf16(int P, int N, const BwdParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 32 && N == 64) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 32, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 64, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 32, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 64, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 128) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 32, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 128, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 32, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 128, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 256) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 32, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 256, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 32, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 256, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 64) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 64, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 64, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 64, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 64, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 128) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 64, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 128, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 64, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 128, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 256) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<__bf16, 64, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 256, 64>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<__bf16, 64, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 256, 64>::REV), 0, s, prm);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_klocal_bf16(int P, int N, const BwdParams& prm, float* kloc, float* kcarry, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 32 && N == 64) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 32, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 64, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 128) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 32, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 128, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 256) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 32, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 32, 256, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 64) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 64, 64, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 64, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 128) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 64, 128, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 128, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 256) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<__bf16, 64, 256, 64>), dim3((unsigned)grid), dim3(64 * BwdWaves<__bf16, 64, 256, 64>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
