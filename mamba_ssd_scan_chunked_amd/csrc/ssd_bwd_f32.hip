// Backward kernels (forward and reverse pass) for f32 inputs.
#include "ssd_bwd.hpp"
#include "ssd_launch.hpp"

namespace ssd {
bool supported_bwd_f32(int P, int N) {
    return (P == 16 || P == 32 || P == 64) && (N == 16 || N == 32 || N == 64 || N == 128);
}

int bwd_block_f32() { return 32; }

hipError_t launch_bwd_f32(int P, int N, const BwdParams& prm, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 16 && N == 16) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 16, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 16, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 16, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 16, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 16 && N == 32) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 16, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 32, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 16, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 32, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 16 && N == 64) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 16, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 64, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 16, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 64, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 16 && N == 128) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 16, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 128, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 16, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 128, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 16) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 32, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 16, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 32, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 16, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 32) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 32, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 32, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 32, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 32, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 64) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 32, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 64, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 32, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 64, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 32 && N == 128) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 32, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 128, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 32, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 128, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 16) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 64, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 16, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 64, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 16, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 32) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 64, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 32, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 64, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 32, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 64) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 64, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 64, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 64, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 64, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    if (P == 64 && N == 128) {
        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<float, 64, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 128, 32>::FWD), 0, s, prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((ssd_bwd_rev_kernel<float, 64, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 128, 32>::REV), 0, s, prm);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_klocal_f32(int P, int N, const BwdParams& prm, float* kloc, float* kcarry, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (P == 16 && N == 16) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 16, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 16, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 16 && N == 32) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 16, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 32, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 16 && N == 64) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 16, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 64, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 16 && N == 128) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 16, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 16, 128, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 16) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 32, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 16, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 32) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 32, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 32, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 64) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 32, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 64, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 32 && N == 128) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 32, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 32, 128, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 16) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 64, 16, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 16, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 32) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 64, 32, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 32, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 64) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 64, 64, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 64, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    if (P == 64 && N == 128) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<float, 64, 128, 32>), dim3((unsigned)grid), dim3(64 * BwdWaves<float, 64, 128, 32>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }
    return hipErrorInvalidValue;
}
}  // namespace ssd
