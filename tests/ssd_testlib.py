"""Shared helpers of the test suite: moving seeded problems to the GPU, running
the HIP path through the C ABI, and comparing with the CPU oracle (whole
problems, or sampled (row, head) pairs of large ones)."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle

# Tolerances: max |y - y_ref| <= TOL * max |y_ref|, the same rule for final states.
TOL = {"bf16": 2e-2, "f32": 1e-5}


def dtype_name(prob) -> str:
    return "bf16" if prob["x"].dtype == torch.bfloat16 else "f32"


def to_device(prob, device="cuda"):
    out = {}
    for k, v in prob.items():
        out[k] = v.to(device) if isinstance(v, torch.Tensor) else v
    return out


def run_gpu(prob, chunk_len=256, dt_scales_x=False, **kw):
    import mamba_ssd_scan_chunked_amd as ssd
    d = to_device(prob)
    y, f = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=chunk_len,
                       init_state=d["init"], seq_idx=d["seq_idx"],
                       nseqs=prob["nseqs"] if prob["seq_idx"] is not None else None,
                       dt_scales_x=dt_scales_x, **kw)
    torch.cuda.synchronize()
    return y.cpu().double().numpy(), (f.cpu().double().numpy() if f is not None else None)


def run_oracle(prob, dt_scales_x=False, nthreads=0, **kw):
    return oracle.recurrence(prob["x"], prob["dt"], prob["A_log"], prob["B"], prob["C"], prob["D"],
                             prob["init"], prob["seq_idx"], prob["nseqs"] if prob["seq_idx"] is not None else None,
                             dt_scales_x=dt_scales_x, nthreads=nthreads, **kw)


def sub_problem(prob, b, h):
    """The (row b, head h) slice as a one-row, one-head, one-group problem."""
    H = prob["x"].shape[2]
    G = prob["B"].shape[2]
    g = h // (H // G)
    sub = {
        "x": prob["x"][b:b + 1, :, h:h + 1],
        "dt": prob["dt"][b:b + 1, :, h:h + 1],
        "A_log": prob["A_log"][h:h + 1],
        "B": prob["B"][b:b + 1, :, g:g + 1],
        "C": prob["C"][b:b + 1, :, g:g + 1],
        "D": prob["D"][h:h + 1] if prob["D"] is not None else None,
    }
    if prob["seq_idx"] is None:
        sub["seq_idx"] = None
        sub["nseqs"] = 1
        sub["init"] = prob["init"][b:b + 1, h:h + 1] if prob["init"] is not None else None
        sub["seqs"] = [b]
    else:
        row = prob["seq_idx"][b]
        seqs = sorted(set(row.tolist()))
        lo = seqs[0]
        sub["seq_idx"] = (row - lo).to(torch.int32).unsqueeze(0).contiguous()
        sub["nseqs"] = seqs[-1] - lo + 1
        sub["init"] = prob["init"][lo:lo + sub["nseqs"], h:h + 1] if prob["init"] is not None else None
        sub["seqs"] = list(range(lo, lo + sub["nseqs"]))
    return sub


def oracle_pairs(prob, pairs, dt_scales_x=False, workers=None):
    """Oracle y[b, :, h] and final[seqs, h] for each sampled (b, h), run concurrently."""
    workers = workers or max(1, min(len(pairs), os.cpu_count() or 1, 16))

    def one(bh):
        b, h = bh
        sub = sub_problem(prob, b, h)
        y, f = oracle.recurrence(sub["x"], sub["dt"], sub["A_log"], sub["B"], sub["C"], sub["D"], sub["init"],
                                 sub["seq_idx"], sub["nseqs"], dt_scales_x=dt_scales_x, nthreads=1)
        return y[0, :, 0], f[:, 0], sub["seqs"]

    with cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, pairs))


def rel_err(got, ref) -> float:
    scale = float(np.abs(ref).max())
    if scale == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max()) / scale


def assert_parity(got, ref, tol, what="y"):
    assert np.isfinite(got).all(), "%s has non-finite values" % what
    e = rel_err(got, ref)
    assert e <= tol, "%s: max|err| / max|ref| = %.3e > %.1e" % (what, e, tol)
    return e


# Per-head sums over every token (dA_log, ddt_bias, dD of the backward): their
# rounding error grows with the sum of the absolute per-token terms, not with the
# sum itself, which cancellation can make small.  Each term carries a relative
# error of a few units of the operand precision, so the error of the sum is
# bounded by about that times the absolute sum; the test allows tol * max(max|ref|,
# SUM_FRACTION * max_h sum_t |term|), i.e. 2e-3 (bf16) or 1e-6 (fp32) of the
# absolute sum.
SUM_FRACTION = 0.1


def assert_parity_sum(got, ref, abs_terms, tol, what):
    assert np.isfinite(got).all(), "%s has non-finite values" % what
    scale = max(float(np.abs(ref).max()), SUM_FRACTION * float(np.abs(abs_terms).max()))
    e = float(np.abs(got - ref).max()) / scale if scale > 0 else float(np.abs(got).max())
    assert e <= tol, "%s: max|err| / scale = %.3e > %.1e (scale %.3e)" % (what, e, tol, scale)
    return e


def sample_pairs(b, H, k, seed=0):
    rng = np.random.default_rng(seed)
    allp = [(i, j) for i in range(b) for j in range(H)]
    if len(allp) <= k:
        return allp
    pick = rng.choice(len(allp), size=k, replace=False)
    # always include the first and last unit (first/last row, first/last head)
    out = {allp[0], allp[-1]} | {allp[i] for i in pick}
    return sorted(out)[: max(k, 2)]
