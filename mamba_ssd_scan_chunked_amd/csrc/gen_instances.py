"""Write the kernel-instantiation sources (ssd_<dtype>.hip, ssd_<dtype>_s<seq>_e<xscale>_l<local>.hip).

Each file instantiates the scan kernel for one (dtype, sequence ids, input scaling (Euler or zero-order hold),
local pass or scan) combination over the supported (headdim, dstate, block) shapes, so the build compiles
them in parallel.  Run it after changing the shape lists below; the outputs are
committed sources.
"""
import itertools
def gen(tag, TI, Ps, Ns, QBs, seq, eul, loc):
    out = ['// Kernel instantiations: %s inputs, %s sequence ids, %s input scaling, %s.\n#include "ssd_kernels.hpp"\n#include "ssd_launch.hpp"\n\nnamespace ssd {\n' % (tag, "with" if seq else "without", "with" if eul else "without", "local pass" if loc else "scan")]
    fn = "launch_scan_%s_s%d_e%d_l%d" % (tag, seq, eul, loc)
    out.append("hipError_t %s(int P, int N, int QB, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {\n" % fn)
    b = lambda v: "true" if v else "false"
    for P in Ps:
        for N in Ns:
            for Q in QBs:
                # one head per workgroup, and for bf16 64-channel heads without sequence
                # ids, in the scan proper, also five slices per workgroup
                spws = [P // 16] + ([5] if (tag, P, seq, loc) == ("bf16", 64, 0, 0) else [])
                for spw in spws:
                    out.append("    if (P == %d && N == %d && QB == %d && spw == %d) { hipLaunchKernelGGL((ssd_scan_kernel<%s, %d, %d, %d, %s, %s, %s, %d>), dim3((unsigned)grid), dim3(ScanCfg<%s, %d, %d, %d, %d>::NT), 0, s, prm); return hipGetLastError(); }\n"
                               % (P, N, Q, spw, TI, P, N, Q, b(seq), b(eul), b(loc), spw, TI, P, N, Q, spw))
    out.append("    return hipErrorInvalidValue;\n}\n}  // namespace ssd\n")
    return "".join(out)

def gen_common(tag, TI, Ps, Ns, QBs):
    out = ['// Shape table and variant dispatch for %s inputs.\n#include "ssd_kernels.hpp"\n#include "ssd_launch.hpp"\n\nnamespace ssd {\n' % tag]
    out.append("bool supported_%s(int P, int N, int QB) {\n" % tag)
    out.append("    const bool p = %s;\n" % " || ".join("P == %d" % v for v in Ps))
    out.append("    const bool n = %s;\n" % " || ".join("N == %d" % v for v in Ns))
    out.append("    const bool q = %s;\n" % " || ".join("QB == %d" % v for v in QBs))
    out.append("    return p && n && q;\n}\n\n")
    out.append("hipError_t launch_scan_%s(int P, int N, int QB, bool seq, bool xscale, bool local, int spw, const ScanParams& prm, int64_t grid, hipStream_t s) {\n" % tag)
    out.append("    if (grid <= 0) return hipSuccess;\n")
    for sq, eu, lo in itertools.product((0, 1), (0, 1), (0, 1)):
        out.append("    if (seq == %s && xscale == %s && local == %s) return launch_scan_%s_s%d_e%d_l%d(P, N, QB, spw, prm, grid, s);\n" % ("true" if sq else "false", "true" if eu else "false", "true" if lo else "false", tag, sq, eu, lo))
    out.append("    return hipErrorInvalidValue;\n}\n\n")
    out.append("hipError_t launch_step_%s(int P, int N, const StepParams& prm, int64_t grid, hipStream_t s) {\n" % tag)
    out.append("    if (grid <= 0) return hipSuccess;\n")
    for P in Ps:
        for N in Ns:
            out.append("    if (P == %d && N == %d) { hipLaunchKernelGGL((ssd_step_kernel<%s, %d, %d>), dim3((unsigned)grid), dim3(256), 0, s, prm); return hipGetLastError(); }\n" % (P, N, TI, P, N))
    out.append("    return hipErrorInvalidValue;\n}\n}  // namespace ssd\n")
    return "".join(out)

def gen_bwd(tag, TI, Ps, Ns, QB):
    out = ['// Backward kernels (forward and reverse pass) for %s inputs.\n#include "ssd_bwd.hpp"\n#include "ssd_launch.hpp"\n\nnamespace ssd {\n' % tag]
    out.append("bool supported_bwd_%s(int P, int N) {\n" % tag)
    out.append("    return (%s) && (%s);\n}\n\n" % (" || ".join("P == %d" % v for v in Ps), " || ".join("N == %d" % v for v in Ns)))
    out.append("int bwd_block_%s() { return %d; }\n\n" % (tag, QB))
    out.append("hipError_t launch_bwd_%s(int P, int N, const BwdParams& prm, int64_t grid, hipStream_t s) {\n" % tag)
    out.append("    if (grid <= 0) return hipSuccess;\n")
    for P in Ps:
        for N in Ns:
            out.append("    if (P == %d && N == %d) {\n" % (P, N))
            out.append("        hipLaunchKernelGGL((ssd_bwd_fwd_kernel<%s, %d, %d, %d>), dim3((unsigned)grid), dim3(64 * BwdWaves<%s, %d, %d, %d>::FWD), 0, s, prm);\n" % (TI, P, N, QB, TI, P, N, QB))
            out.append("        hipError_t e = hipGetLastError();\n        if (e != hipSuccess) return e;\n")
            out.append("        hipLaunchKernelGGL((ssd_bwd_rev_kernel<%s, %d, %d, %d>), dim3((unsigned)grid), dim3(64 * BwdWaves<%s, %d, %d, %d>::REV), 0, s, prm);\n" % (TI, P, N, QB, TI, P, N, QB))
            out.append("        return hipGetLastError();\n    }\n")
    out.append("    return hipErrorInvalidValue;\n}\n\n")
    out.append("hipError_t launch_bwd_klocal_%s(int P, int N, const BwdParams& prm, float* kloc, float* kcarry, int64_t grid, hipStream_t s) {\n" % tag)
    out.append("    if (grid <= 0) return hipSuccess;\n")
    for P in Ps:
        for N in Ns:
            out.append("    if (P == %d && N == %d) { hipLaunchKernelGGL((ssd_bwd_klocal_kernel<%s, %d, %d, %d>), dim3((unsigned)grid), dim3(64 * BwdWaves<%s, %d, %d, %d>::KLOC), 0, s, prm, kloc, kcarry); return hipGetLastError(); }\n" % (P, N, TI, P, N, QB, TI, P, N, QB))
    out.append("    return hipErrorInvalidValue;\n}\n}  // namespace ssd\n")
    return "".join(out)

import os
d = os.path.dirname(os.path.abspath(__file__)) + "/"
cfg = {"bf16": ("__bf16", [32, 64], [64, 128, 256], [32, 64]), "f32": ("float", [16, 32, 64], [16, 32, 64, 128], [32, 64])}
files = []
for tag, (TI, Ps, Ns, QBs) in cfg.items():
    open(d + "ssd_%s.hip" % tag, "w").write(gen_common(tag, TI, Ps, Ns, QBs))
    files.append("ssd_%s.hip" % tag)
    for sq, eu, lo in itertools.product((0, 1), (0, 1), (0, 1)):
        fn = "ssd_%s_s%d_e%d_l%d.hip" % (tag, sq, eu, lo)
        open(d + fn, "w").write(gen(tag, TI, Ps, Ns, QBs, sq, eu, lo))
        files.append(fn)
bwd = {"bf16": ("__bf16", [32, 64], [64, 128, 256], 64), "f32": ("float", [16, 32, 64], [16, 32, 64, 128], 32)}
for tag, (TI, Ps, Ns, QB) in bwd.items():
    fn = "ssd_bwd_%s.hip" % tag
    open(d + fn, "w").write(gen_bwd(tag, TI, Ps, Ns, QB))
    files.append(fn)
print(files)
