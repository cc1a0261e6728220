"""The recurrent single-token step (ssd_step) against the CPU oracle.

One step is the oracle's recurrence over one token from the given state; a
chunked prefill of T tokens followed by K steps must equal the chunked forward
over all T + K tokens.  Tolerance as for the forward: max |got - ref| <=
tol * max |ref|, 2e-2 for bf16 inputs, 1e-5 for fp32.
"""
import sys

import numpy as np
import pytest
import torch

import ssd_inputs as si
from ssd_testlib import TOL, assert_parity, run_oracle, to_device

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


SHAPES = [
    # dtype, b, H, P, N, G
    ("bf16", 3, 8, 64, 128, 1),
    ("bf16", 2, 6, 32, 256, 3),
    ("bf16", 1, 4, 64, 64, 2),
    ("bf16", 2, 4, 64, 256, 1),     # a state row spans the whole wave (64 float4 per row)
    ("f32", 2, 4, 16, 16, 1),
    ("f32", 1, 6, 32, 64, 2),
    ("f32", 2, 2, 64, 128, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-b%d-H%d-P%d-N%d-G%d" % s)
@pytest.mark.parametrize("euler", [False, True])
def test_step_matches_one_oracle_step(shape, euler):
    import mamba_ssd_scan_chunked_amd as ssd
    dt_, b, H, P, N, G = shape
    prob = si.make_problem(b, 1, H, P, N, G, dtype=dt_, seed=H * N + P, d_skip=True, init_std=0.5)
    announce("step %s euler=%s" % (shape, euler))
    d = to_device(prob)
    state = d["init"].clone()
    y = ssd.step(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], state, dt_scales_x=euler)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_scales_x=euler)
    assert_parity(y.cpu().double().numpy(), yr, TOL[dt_], "y")
    assert_parity(state.cpu().double().numpy(), fr, TOL[dt_], "state")


@pytest.mark.parametrize("dt_", ["bf16", "f32"])
def test_prefill_then_steps_equals_the_whole_sequence(dt_):
    import mamba_ssd_scan_chunked_amd as ssd
    b, T, K, H, P, N, G = 2, 200, 16, 4, 64, 128 if dt_ == "bf16" else 64, 1
    prob = si.make_problem(b, T + K, H, P, N, G, dtype=dt_, seed=7, d_skip=True, init_std=0.5)
    announce("prefill %d + %d steps %s" % (T, K, dt_))
    d = to_device(prob)
    head = {k: (v[:, :T].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    _, state = ssd.forward(head["x"], head["dt"], head["A_log"], head["B"], head["C"], head["D"], chunk_len=64,
                           init_state=d["init"])
    ys = []
    for t in range(T, T + K):
        ys.append(ssd.step(d["x"][:, t], d["dt"][:, t], d["A_log"], d["B"][:, t], d["C"][:, t], d["D"], state))
    torch.cuda.synchronize()
    y_steps = torch.cat(ys, dim=1).cpu().double().numpy()
    yr, fr = run_oracle(prob)
    assert_parity(y_steps, yr[:, T:], TOL[dt_], "y (steps)")
    assert_parity(state.cpu().double().numpy(), fr, TOL[dt_], "state after the steps")


def test_step_updates_the_state_in_place_and_is_deterministic():
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(2, 1, 4, 64, 128, 1, dtype="bf16", seed=3, d_skip=True, init_std=0.5)
    d = to_device(prob)
    announce("step in place")
    outs = []
    for _ in range(2):
        state = d["init"].clone()
        y = ssd.step(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], state)
        torch.cuda.synchronize()
        assert not torch.equal(state, d["init"])
        outs.append((y.cpu(), state.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
