"""Parity of the backward pass (ssd_backward, through the C ABI) with the CPU
oracle's adjoint recurrence (oracle.gradients, fp64, pinned by finite
differences in test_oracle_grad_pins.py).

Every output is compared element by element: max |got - ref| <= tol * max |ref|
per tensor, with tol = 2e-2 for bf16 inputs (bf16 MFMA operands, fp32
accumulation) and 1e-5 for fp32 inputs.  The per-head sums over all tokens
(dA_log, ddt_bias, dD) are judged against max(max|ref|, 0.1 * the sum of their
absolute per-token terms) instead: cancellation can make a sum far smaller than
the rounding its terms carry.  The loss is L = <dy, y> + <dfinal, final> with
seeded random dy and dfinal.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
from ssd_testlib import TOL, assert_parity, assert_parity_sum, dtype_name, to_device

pytestmark = pytest.mark.gpu

OUTS = ("dx", "ddt", "dA_log", "dB", "dC", "dD", "dinit", "ddt_bias")


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def cotangents(prob, seed):
    b, T, H, P = prob["x"].shape
    N = prob["B"].shape[3]
    ns = prob["nseqs"]
    rng = np.random.default_rng(seed)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return f32(rng.standard_normal((b, T, H, P))), f32(rng.standard_normal((ns, H, P, N)))


def run_both(prob, dy, dfinal, *, dt_bias=None, dt_softplus=False, zoh=False, dt_scales_x=False, workers=0,
             segments=0):
    import mamba_ssd_scan_chunked_amd as ssd
    d = to_device(prob)
    packed = prob["seq_idx"] is not None
    g = ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], dy.cuda(), D=d["D"], init_state=d["init"],
                     dfinal=dfinal.cuda() if dfinal is not None else None, dt_scales_x=dt_scales_x,
                     dt_bias=dt_bias.cuda() if dt_bias is not None else None, dt_softplus=dt_softplus, zoh=zoh,
                     seq_idx=d["seq_idx"], nseqs=prob["nseqs"] if packed else None, segments=segments)
    torch.cuda.synchronize()
    got = {k: v.cpu().double().numpy() for k, v in g.items()}
    ref = oracle.gradients(prob["x"], prob["dt"], prob["A_log"], prob["B"], prob["C"], dy, prob["D"], prob["init"],
                           dfinal, prob["seq_idx"], prob["nseqs"] if packed else None, dt_scales_x=dt_scales_x,
                           dt_bias=dt_bias, dt_softplus=dt_softplus, zoh=zoh, nthreads=workers)
    return got, ref


SUMS = ("dA_log", "ddt_bias", "dD")


def check(got, ref, tol, outs=OUTS):
    errs = {}
    for k in outs:
        if k in SUMS:
            errs[k] = assert_parity_sum(got[k], ref[k], ref["abs_terms"][k], tol, k)
        else:
            errs[k] = assert_parity(got[k], ref[k], tol, k)
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)


SHAPES = [
    # dtype, b, T, H, P, N, G   (ragged last blocks; G < H exercises the sum over a group's heads)
    ("bf16", 2, 200, 4, 64, 128, 2),
    ("bf16", 1, 130, 2, 32, 64, 2),
    ("bf16", 1, 100, 2, 64, 256, 1),
    ("bf16", 2, 64, 3, 32, 128, 1),
    ("f32", 2, 150, 2, 64, 128, 1),
    ("f32", 1, 77, 4, 16, 16, 2),
    ("f32", 1, 65, 2, 32, 64, 2),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-b%d-T%d-H%d-P%d-N%d-G%d" % s)
def test_backward_matches_oracle(shape):
    dt, b, T, H, P, N, G = shape
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + N + 5, d_skip=True, init_std=0.5)
    dy, dfinal = cotangents(prob, T + 1)
    announce("backward %s" % (shape,))
    got, ref = run_both(prob, dy, dfinal)
    check(got, ref, TOL[dt])


MODES = {
    "euler": dict(dt_scales_x=True),
    "zoh": dict(zoh=True),
    "softplus_bias": dict(dt_softplus=True, bias=True),
    "softplus_zoh": dict(dt_softplus=True, zoh=True, bias=True),
}


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_step_size_map_and_scaling(dt, mode):
    kw = dict(MODES[mode])
    bias = kw.pop("bias", False)
    b, T, H, P, N, G = 2, 140, 4, 64, 128 if dt == "bf16" else 64, 2
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=11, d_skip=True, init_std=0.5)
    if kw.get("dt_softplus"):
        raw = si.raw_step_sizes(b, T, H, seed=12)
        prob = dict(prob, dt=raw["dt"])
        dtb = raw["dt_bias"]
    else:
        dtb = si.raw_step_sizes(b, T, H, seed=12, bias_range=(0.0, 0.2))["dt_bias"] if bias else None
    dy, dfinal = cotangents(prob, 13)
    announce("backward mode=%s dtype=%s" % (mode, dt))
    got, ref = run_both(prob, dy, dfinal, dt_bias=dtb, **kw)
    check(got, ref, TOL[dt])


def test_backward_without_init_dfinal_and_skip():
    prob = si.make_problem(1, 96, 2, 64, 128, 1, dtype="bf16", seed=17)
    dy, _ = cotangents(prob, 18)
    announce("backward without init/dfinal/D")
    got, ref = run_both(prob, dy, None)
    check(got, ref, TOL["bf16"], outs=("dx", "ddt", "dA_log", "dB", "dC", "dinit", "dD"))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_sums_without_cancellation(dt):
    """With x, B, C, dy, dfinal and the initial states nonnegative, every state H_t
    and every gradient G_t = dL/dH_t is nonnegative elementwise, so each per-token
    term of dA_log, ddt_bias (dl_t = <G_t, a_t H_{t-1}>) and dD (x_t . dy_t) has one
    sign: the sums have no cancellation, and all eight outputs are held to the plain
    max|ref| rule."""
    b, T, H, P, N, G = 2, 200, 4, 64, 128 if dt == "bf16" else 64, 2
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=41, d_skip=True, init_std=0.5)
    prob = dict(prob, x=prob["x"].abs(), B=prob["B"].abs(), C=prob["C"].abs(), init=prob["init"].abs())
    dy, dfinal = cotangents(prob, 42)
    dtb = si.raw_step_sizes(b, T, H, seed=43, bias_range=(0.0, 0.2))["dt_bias"]
    announce("backward, sums without cancellation, dtype=%s" % dt)
    got, ref = run_both(prob, dy.abs(), dfinal.abs(), dt_bias=dtb)
    for k in SUMS:      # the construction: |sum| equals the sum of the absolute terms
        assert np.all(np.abs(ref[k]) >= 0.999999 * ref["abs_terms"][k]), k
    errs = {k: assert_parity(got[k], ref[k], TOL[dt], k) for k in OUTS}
    print("[errors] " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)


def test_backward_no_tokens():
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(2, 0, 2, 64, 128, 1, dtype="bf16", seed=19, d_skip=True, init_std=0.5)
    _, dfinal = cotangents(prob, 20)
    d = to_device(prob)
    announce("backward T=0")
    g = ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], torch.zeros(2, 0, 2, 64, device="cuda"), D=d["D"],
                     init_state=d["init"], dfinal=dfinal.cuda())
    torch.cuda.synchronize()
    assert torch.equal(g["dinit"].cpu(), dfinal)
    assert not g["dA_log"].any() and not g["dD"].any() and not g["ddt_bias"].any()


def test_backward_is_deterministic():
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(2, 300, 4, 64, 128, 2, dtype="bf16", seed=23, d_skip=True, init_std=0.5)
    dy, dfinal = cotangents(prob, 24)
    d = to_device(prob)
    announce("backward determinism")
    runs = [ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], dy.cuda(), D=d["D"], init_state=d["init"],
                         dfinal=dfinal.cuda()) for _ in range(2)]
    torch.cuda.synchronize()
    for k in OUTS:
        assert torch.equal(runs[0][k], runs[1][k]), k


PACKED = [
    # dtype, b, T, H, P, N, G, sequence lengths per row (starts at, inside and across block edges; length 1)
    ("bf16", 2, 300, 4, 64, 128, 2, [[100, 1, 199], [64, 236]]),
    ("bf16", 1, 257, 2, 32, 64, 1, [[1, 63, 64, 128, 1]]),
    ("f32", 1, 200, 2, 64, 64, 1, [[37, 64, 99]]),
    ("f32", 2, 96, 3, 16, 32, 3, [[32, 32, 32], [95, 1]]),
]


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "%s-b%d-T%d-H%d-P%d-N%d-G%d" % c[:7])
def test_backward_packed_sequences(case):
    dt, b, T, H, P, N, G, lens = case
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + 3, d_skip=True, init_std=0.5, seqlens=lens)
    dy, dfinal = cotangents(prob, T + 4)
    announce("backward packed %s" % (case[:7],))
    got, ref = run_both(prob, dy, dfinal)
    check(got, ref, TOL[dt])


def test_backward_packed_with_absent_sequence_ids():
    """Ids 1, 2 and 3 of 0..4 never occur: their dinit is 0; the others as the oracle."""
    prob = si.make_problem(1, 200, 2, 64, 128, 1, dtype="bf16", seed=33, d_skip=True, init_std=0.5,
                           seqlens=[[80, 120]])
    seq = prob["seq_idx"].clone()
    seq[seq == 1] = 4                          # sequences 0 and 4; 1, 2, 3 absent
    prob = dict(prob, seq_idx=seq, nseqs=5,
                init=torch.from_numpy(np.random.default_rng(34).normal(0, 0.5, (5, 2, 64, 128)).astype(np.float32)))
    dy, dfinal = cotangents(prob, 35)
    announce("backward packed, absent ids")
    got, ref = run_both(prob, dy, dfinal)
    check(got, ref, TOL["bf16"])
    assert not got["dinit"][1:4].any()


def test_backward_packed_workload():
    """The packed workload at full size: 16 sequences (minimum length 64) in one row of
    8192 tokens, 48 heads in 8 groups, init states, every output against the oracle."""
    w = si.WORKLOADS["packed_bf16"]
    prob = si.make_workload(w)
    dy, dfinal = cotangents(prob, 37)
    announce("backward packed workload")
    got, ref = run_both(prob, dy, dfinal)
    check(got, ref, TOL["bf16"])


def test_backward_headline_shape():
    """The 2.7B-layer shape (b=4, T=4096, H=80, P=64, N=128, bf16), every output
    against the oracle over the whole problem."""
    w = si.WORKLOADS["m2p7_bf16"]
    prob = si.make_workload(w)
    dy, dfinal = cotangents(prob, 29)
    announce("backward 2.7B-layer shape")
    got, ref = run_both(prob, dy, dfinal)
    check(got, ref, TOL["bf16"])


SPLIT = [
    # dtype, b, T, H, P, N, G, forced segments (0: the automatic choice)
    ("bf16", 1, 1000, 2, 64, 128, 1, 0),       # 2 items: split automatically
    ("bf16", 2, 700, 2, 64, 128, 2, 3),        # ragged last segment
    ("bf16", 1, 640, 3, 32, 64, 3, 5),
    ("f32", 1, 500, 2, 64, 64, 1, 2),
    ("f32", 2, 300, 2, 16, 32, 2, 0),
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: "%s-b%d-T%d-H%d-P%d-N%d-G%d-S%d" % c)
def test_backward_split_rows(case):
    """Rows cut into segments (the state entering each segment from the forward's local
    pass and combine step, the gradient leaving each from the reverse local pass and
    combine step): every output against the oracle."""
    dt, b, T, H, P, N, G, S = case
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + 7, d_skip=True, init_std=0.5)
    dy, dfinal = cotangents(prob, T + 8)
    announce("backward split rows %s" % (case,))
    got, ref = run_both(prob, dy, dfinal, segments=S)
    check(got, ref, TOL[dt])


@pytest.mark.parametrize("mode", ["softplus_zoh", "euler"])
def test_backward_split_rows_step_size_modes(mode):
    kw = dict(MODES[mode])
    kw.pop("bias", None)
    b, T, H = 1, 600, 2
    prob = si.make_problem(b, T, H, 64, 128, 1, dtype="bf16", seed=41, d_skip=True, init_std=0.5)
    dtb = None
    if kw.get("dt_softplus"):
        raw = si.raw_step_sizes(b, T, H, seed=42)
        prob = dict(prob, dt=raw["dt"])
        dtb = raw["dt_bias"]
    dy, dfinal = cotangents(prob, 43)
    announce("backward split rows mode=%s" % mode)
    got, ref = run_both(prob, dy, dfinal, dt_bias=dtb, segments=4, **kw)
    check(got, ref, TOL["bf16"])


def test_backward_split_equals_unsplit():
    """The same problem with 1 and 4 segments: equal within the tolerance."""
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(1, 512, 2, 64, 128, 1, dtype="bf16", seed=47, d_skip=True, init_std=0.5)
    dy, dfinal = cotangents(prob, 48)
    d = to_device(prob)
    outs = []
    for S in (1, 4):
        g = ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], dy.cuda(), D=d["D"], init_state=d["init"],
                         dfinal=dfinal.cuda(), segments=S)
        torch.cuda.synchronize()
        outs.append({k: v.cpu().double().numpy() for k, v in g.items()})
    for k in OUTS:
        assert_parity(outs[1][k], outs[0][k], TOL["bf16"], k)
