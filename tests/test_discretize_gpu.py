"""Parity of the fused step-size map and input discretisations with the CPU oracle.

The GPU path maps the dt input to the step size itself (dt + dt_bias, through
softplus when asked) and scales x in the state write by nothing, by the step
size (Euler) or by the exact zero-order hold (exp(step A) - 1) / A.  The oracle
does the same in fp64 from the same raw inputs.  Covered: the one-pass scan,
rows split into segments (local pass, combine, scan), packed sequences and the
single-token step, for bf16 and fp32 inputs.  Tolerance as everywhere:
max |got - ref| <= tol * max |ref| (2e-2 bf16, 1e-5 fp32), y and final states.
"""
import sys

import pytest
import torch

import ssd_inputs as si
from ssd_testlib import TOL, assert_parity, dtype_name, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu

MODES = {
    # name: (softplus, with bias, Euler, zero-order hold)
    "softplus": (True, True, False, False),
    "softplus_euler": (True, True, True, False),
    "softplus_zoh": (True, True, False, True),
    "zoh": (False, False, False, True),
    "bias_zoh": (False, True, False, True),
}


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def with_raw_dt(prob, seed, softplus):
    """Pre-activation dt and a bias for the softplus map; without it, the problem's
    positive step sizes and a small positive bias (a negative step size would make
    the decay exceed 1 and the state grow without bound)."""
    b, T, H = prob["dt"].shape
    q = dict(prob)
    if softplus:
        raw = si.raw_step_sizes(b, T, H, seed=seed)
        q["dt"] = raw["dt"]
    else:
        raw = si.raw_step_sizes(b, T, H, seed=seed, bias_range=(0.0, 0.2))
    q["dt_bias"] = raw["dt_bias"]
    return q


def check(prob, chunk_len, mode, label):
    softplus, bias, euler, zoh = MODES[mode]
    announce("%s mode=%s dtype=%s x=%s chunk=%d" % (label, mode, dtype_name(prob), tuple(prob["x"].shape), chunk_len))
    kw = dict(dt_softplus=softplus, zoh=zoh, dt_scales_x=euler)
    dtb = prob["dt_bias"] if bias else None
    y, f = run_gpu(prob, chunk_len=chunk_len, dt_bias=dtb.cuda() if dtb is not None else None, **kw)
    yr, fr = run_oracle(prob, dt_bias=dtb, **kw)
    tol = TOL[dtype_name(prob)]
    assert_parity(y, yr, tol, "y")
    assert_parity(f, fr, tol, "final")


SHAPES = [
    # dtype, b, T, H, P, N, G, chunk  (2-8 (row, head) items: rows are split into segments)
    ("bf16", 2, 700, 4, 64, 128, 1, 256),
    ("bf16", 1, 333, 2, 32, 64, 1, 64),
    ("f32", 2, 300, 2, 64, 128, 1, 64),
    ("f32", 1, 150, 3, 16, 32, 3, 32),
]


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-b%d-T%d-H%d-P%d-N%d-G%d-Q%d" % s)
def test_step_size_map_and_scaling(shape, mode):
    dt, b, T, H, P, N, G, Q = shape
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + H, d_skip=True, init_std=0.5)
    check(with_raw_dt(prob, 100 + T, MODES[mode][0]), Q, mode, "scan")


@pytest.mark.parametrize("mode", ["softplus_zoh", "softplus_euler"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_packed_sequences(dt, mode):
    prob = si.make_problem(2, 640, 4, 64, 64 if dt == "f32" else 128, 2, dtype=dt, seed=31, init_std=0.5,
                           packed_nseqs=4, min_len=64)
    check(with_raw_dt(prob, 131, MODES[mode][0]), 64, mode, "packed")


@pytest.mark.parametrize("mode", ["softplus_zoh", "zoh"])
def test_many_items_one_pass(mode):
    """Enough (row, head) items that each row runs in one workgroup pass (no segments),
    including five-slice workgroups (bf16, P = 64, between 256 and 320 items)."""
    prob = si.make_problem(4, 256, 80, 64, 128, 1, dtype="bf16", seed=41)
    check(with_raw_dt(prob, 141, MODES[mode][0]), 256, mode, "one pass")


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_single_token_step(dt, mode):
    import mamba_ssd_scan_chunked_amd as ssd
    softplus, bias, euler, zoh = MODES[mode]
    b, H, P, N, G = 3, 6, 64, 128 if dt == "bf16" else 64, 2
    prob = with_raw_dt(si.make_problem(b, 1, H, P, N, G, dtype=dt, seed=51, d_skip=True, init_std=0.5), 151,
                       softplus)
    announce("step mode=%s dtype=%s" % (mode, dt))
    d = to_device(prob)
    state = d["init"].clone()
    y = ssd.step(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], state, dt_scales_x=euler,
                 dt_bias=d["dt_bias"] if bias else None, dt_softplus=softplus, zoh=zoh)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_scales_x=euler, dt_bias=prob["dt_bias"] if bias else None, dt_softplus=softplus,
                        zoh=zoh)
    assert_parity(y.cpu().double().numpy(), yr, TOL[dt], "y")
    assert_parity(state.cpu().double().numpy(), fr, TOL[dt], "state")
