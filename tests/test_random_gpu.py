"""Seeded random problems through the forward and the backward, against the oracle.

Each case draws its shape and options from a fixed seed: dtype, batch rows,
length (ragged against the 32- and 64-token blocks), heads and groups, head and
state sizes from the supported sets, chunk length, a skip term, an initial
state, packed sequences, and the step-size map with the input scaling.  The
forward is compared on y and the final states, the backward on every gradient,
with the parity rules of the other tests (per-head sums over tokens judged
against the sum of their absolute terms).  The draws are listed by seed, so a
failing case can be rerun alone.
"""
import random
import sys

import pytest
import torch

import oracle
import ssd_inputs as si
from ssd_testlib import TOL, assert_parity, assert_parity_sum, run_oracle, to_device

pytestmark = pytest.mark.gpu

MODES = [
    # softplus, bias, Euler, zero-order hold
    (False, False, False, False),
    (False, False, True, False),
    (True, True, False, False),
    (True, True, True, False),
    (True, True, False, True),
    (False, True, False, True),
]


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def draw(seed, backward=False):
    r = random.Random(seed)
    dt = r.choice(["bf16", "f32"])
    P = r.choice([32, 64] if dt == "bf16" else [16, 32, 64])
    N = r.choice([64, 128, 256] if dt == "bf16" else [16, 32, 64, 128])
    G = r.choice([1, 2, 4])
    H = G * r.randint(1, 6 if not backward else 3)
    packed = r.random() < 0.3
    b = r.randint(1, 3)
    tmax = 400 if not backward else 220
    T = r.randint(40, tmax) if packed else (r.choice([1, 2]) if r.random() < 0.15 else r.randint(3, tmax))
    chunk = r.choice([32, 64, 128, 256])
    return dict(dtype=dt, b=b, T=T, H=H, G=G, P=P, N=N, chunk=chunk, d_skip=r.random() < 0.5,
                init_std=0.5 if r.random() < 0.5 else 0.0, packed=(r.randint(2, 3) if packed else 0),
                mode=r.randrange(len(MODES)), seed=seed)


def problem(c):
    prob = si.make_problem(c["b"], c["T"], c["H"], c["P"], c["N"], c["G"], dtype=c["dtype"], seed=c["seed"],
                           d_skip=c["d_skip"], init_std=c["init_std"], packed_nseqs=c["packed"], min_len=8)
    softplus, bias, euler, zoh = MODES[c["mode"]]
    dt_bias = None
    if softplus or bias:
        raw = si.raw_step_sizes(c["b"], c["T"], c["H"], seed=c["seed"] + 7,
                                bias_range=(-0.5, 0.5) if softplus else (0.0, 0.2))
        if softplus:
            prob["dt"] = raw["dt"]
        dt_bias = raw["dt_bias"] if bias else None
    return prob, dt_bias, dict(dt_softplus=softplus, dt_scales_x=euler, zoh=zoh)


def describe(c):
    return "seed=%(seed)d %(dtype)s b=%(b)d T=%(T)d H=%(H)d G=%(G)d P=%(P)d N=%(N)d chunk=%(chunk)d D=%(d_skip)s " \
           "init=%(init_std)s packed=%(packed)d mode=%(mode)d" % c


@pytest.mark.parametrize("seed", range(100, 148))
def test_random_forward(seed):
    import mamba_ssd_scan_chunked_amd as ssd
    c = draw(seed)
    announce("forward " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    packed = prob["seq_idx"] is not None
    y, f = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=c["chunk"],
                       init_state=d["init"], seq_idx=d["seq_idx"], nseqs=prob["nseqs"] if packed else None,
                       dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_bias=dt_bias, **kw)
    tol = TOL[c["dtype"]]
    assert_parity(y.cpu().double().numpy(), yr, tol, "y")
    assert_parity(f.cpu().double().numpy(), fr, tol, "final")


@pytest.mark.parametrize("seed", range(200, 224))
def test_random_backward(seed):
    import numpy as np

    import mamba_ssd_scan_chunked_amd as ssd
    c = draw(seed, backward=True)
    announce("backward " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    packed = prob["seq_idx"] is not None
    rng = np.random.default_rng(seed)
    b, T, H, P = prob["x"].shape
    N = prob["B"].shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32))
    dfinal = torch.from_numpy(rng.standard_normal((prob["nseqs"], H, P, N)).astype(np.float32))
    g = ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], dy.cuda(), D=d["D"], init_state=d["init"],
                     dfinal=dfinal.cuda(), chunk_len=c["chunk"], seq_idx=d["seq_idx"],
                     nseqs=prob["nseqs"] if packed else None,
                     dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    ref = oracle.gradients(prob["x"], prob["dt"], prob["A_log"], prob["B"], prob["C"], dy, prob["D"], prob["init"],
                           dfinal, prob["seq_idx"], prob["nseqs"] if packed else None, dt_bias=dt_bias, **kw)
    tol = TOL[c["dtype"]]
    for k in ("dx", "ddt", "dB", "dC", "dinit"):
        assert_parity(g[k].cpu().double().numpy(), ref[k], tol, k)
    for k in ("dA_log", "ddt_bias", "dD"):
        assert_parity_sum(g[k].cpu().double().numpy(), ref[k], ref["abs_terms"][k], tol, k)


def draw_five_slice(seed):
    """Shapes with 256 < b*H <= 320 heads of 64 channels (bf16, no sequence ids), which the
    library packs five 16-channel slices per workgroup: the headline layout."""
    r = random.Random(seed)
    H = r.choice([65, 70, 75, 80])
    G = r.choice([g for g in (1, 5, 13, 2, 4) if H % g == 0 and (H // g) % 5 == 0] or [1])
    T = r.choice([1, 2]) if r.random() < 0.15 else r.randint(3, 300)
    return dict(dtype="bf16", b=4, T=T, H=H, G=G, P=64, N=r.choice([64, 128, 256]), chunk=r.choice([32, 64, 256]),
                d_skip=r.random() < 0.5, init_std=0.5 if r.random() < 0.5 else 0.0, packed=0,
                mode=r.randrange(len(MODES)), seed=seed)


@pytest.mark.parametrize("seed", range(300, 312))
def test_random_five_slice_forward(seed):
    import mamba_ssd_scan_chunked_amd as ssd
    c = draw_five_slice(seed)
    announce("five-slice forward " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    y, f = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=c["chunk"],
                       init_state=d["init"], dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_bias=dt_bias, **kw)
    assert_parity(y.cpu().double().numpy(), yr, TOL["bf16"], "y")
    assert_parity(f.cpu().double().numpy(), fr, TOL["bf16"], "final")


def draw_split(seed):
    """Few (row, head) items on long rows, which the library cuts into segments (a local
    pass, the combine step, then every segment's scan)."""
    r = random.Random(seed)
    c = draw(seed)
    G = r.choice([1, 2])
    blk = 64 if c["chunk"] >= 64 else 32           # rows under 16 blocks are not split
    c.update(b=r.randint(1, 2), G=G, H=G * r.randint(1, 2), T=r.randint(16 * blk + 8, 2000),
             packed=(r.randint(2, 5) if r.random() < 0.3 else 0))
    return c


@pytest.mark.parametrize("seed", range(400, 410))
def test_random_split_rows_forward(seed):
    import mamba_ssd_scan_chunked_amd as ssd
    c = draw_split(seed)
    announce("split-row forward " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    packed = prob["seq_idx"] is not None
    p = ssd.problem(c["b"], c["T"], c["H"], c["P"], c["N"], c["G"], c["chunk"], prob["nseqs"],
                    ssd.DTYPE_BF16 if c["dtype"] == "bf16" else ssd.DTYPE_F32, 0)
    assert ssd.workspace_size(p) > 0, "rows are split"
    y, f = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=c["chunk"],
                       init_state=d["init"], seq_idx=d["seq_idx"], nseqs=prob["nseqs"] if packed else None,
                       dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_bias=dt_bias, **kw)
    tol = TOL[c["dtype"]]
    assert_parity(y.cpu().double().numpy(), yr, tol, "y")
    assert_parity(f.cpu().double().numpy(), fr, tol, "final")


@pytest.mark.parametrize("seed", range(500, 506))
def test_random_split_rows_backward(seed):
    import numpy as np

    import mamba_ssd_scan_chunked_amd as ssd
    c = draw_split(seed)
    c["T"] = min(c["T"], 1200)
    announce("split-row backward " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    packed = prob["seq_idx"] is not None
    rng = np.random.default_rng(seed)
    b, T, H, P = prob["x"].shape
    N = prob["B"].shape[3]
    dy = torch.from_numpy(rng.standard_normal((b, T, H, P)).astype(np.float32))
    dfinal = torch.from_numpy(rng.standard_normal((prob["nseqs"], H, P, N)).astype(np.float32))
    g = ssd.backward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], dy.cuda(), D=d["D"], init_state=d["init"],
                     dfinal=dfinal.cuda(), chunk_len=c["chunk"], seq_idx=d["seq_idx"],
                     nseqs=prob["nseqs"] if packed else None,
                     dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    ref = oracle.gradients(prob["x"], prob["dt"], prob["A_log"], prob["B"], prob["C"], dy, prob["D"], prob["init"],
                           dfinal, prob["seq_idx"], prob["nseqs"] if packed else None, dt_bias=dt_bias, **kw)
    tol = TOL[c["dtype"]]
    for k in ("dx", "ddt", "dB", "dC", "dinit"):
        assert_parity(g[k].cpu().double().numpy(), ref[k], tol, k)
    for k in ("dA_log", "ddt_bias", "dD"):
        assert_parity_sum(g[k].cpu().double().numpy(), ref[k], ref["abs_terms"][k], tol, k)


@pytest.mark.parametrize("seed", range(600, 616))
def test_random_step(seed):
    """One decoding step from a random state: shape, skip term and step-size mode drawn per seed."""
    import mamba_ssd_scan_chunked_amd as ssd
    c = draw(seed)
    c.update(T=1, packed=0, init_std=0.5)
    announce("step " + describe(c))
    prob, dt_bias, kw = problem(c)
    d = to_device(prob)
    state = d["init"].clone()
    y = ssd.step(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], state,
                 dt_bias=dt_bias.cuda() if dt_bias is not None else None, **kw)
    torch.cuda.synchronize()
    yr, fr = run_oracle(prob, dt_bias=dt_bias, **kw)
    tol = TOL[c["dtype"]]
    assert_parity(y.cpu().double().numpy(), yr, tol, "y")
    assert_parity(state.cpu().double().numpy(), fr, tol, "state")
