"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerance (both y and final states): max |got - ref| <= tol * max |ref| with
tol = 2e-2 for bf16 inputs (fp32 accumulation) and 1e-5 for fp32 inputs.
Small problems are compared element by element on every output; the measured
workloads are compared on sampled (row, head) pairs that the oracle computes
one by one over the full sequence length.
"""
import sys

import numpy as np
import pytest
import torch

import ssd_inputs as si
from ssd_testlib import (TOL, assert_parity, dtype_name, oracle_pairs, run_gpu, run_oracle, sample_pairs,
                         to_device)

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def check_full(prob, chunk_len, dt_scales_x=False, label=""):
    announce("%s dtype=%s x=%s chunk=%d euler=%s" % (label, dtype_name(prob), tuple(prob["x"].shape), chunk_len,
                                                   dt_scales_x))
    y, f = run_gpu(prob, chunk_len=chunk_len, dt_scales_x=dt_scales_x)
    yr, fr = run_oracle(prob, dt_scales_x=dt_scales_x)
    tol = TOL[dtype_name(prob)]
    ey = assert_parity(y, yr, tol, "y")
    ef = assert_parity(f, fr, tol, "final")
    return ey, ef


# ------------------------------------------------------------------ small shapes, every output

def test_tiny_f32_workload():
    w = si.WORKLOADS["tiny_f32"]
    check_full(si.make_workload(w), w.chunk_len, label="tiny_f32")


SHAPES = [
    # dtype, b, T, H, P, N, G, chunk
    ("bf16", 2, 200, 4, 64, 128, 2, 64),
    ("bf16", 1, 333, 2, 64, 64, 1, 256),
    ("bf16", 2, 97, 2, 32, 256, 1, 32),
    ("bf16", 1, 130, 3, 32, 128, 3, 128),
    ("f32", 2, 150, 2, 64, 128, 1, 64),
    ("f32", 1, 77, 4, 16, 16, 2, 32),
    ("f32", 1, 129, 2, 32, 64, 1, 256),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%s-b%d-T%d-H%d-P%d-N%d-G%d-Q%d" % s)
def test_parity_shapes(shape):
    dt, b, T, H, P, N, G, Q = shape
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + N, d_skip=True, init_std=0.5)
    check_full(prob, Q, label="shape")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_euler_input_scaling(dt):
    prob = si.make_problem(1, 150, 2, 32, 64, 1, dtype=dt, seed=21, d_skip=True, init_std=0.3)
    check_full(prob, 64, dt_scales_x=True, label="euler")


SEQ_CASES = [
    # lengths per row; boundaries at a block edge, inside a block, several in one block, length 1
    [[64, 64, 72]],
    [[10, 1, 1, 50, 20, 118]],
    [[1, 63, 1, 135]],
    [[100, 100], [37, 163]],
    [[200]],
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("idx", range(len(SEQ_CASES)))
@pytest.mark.parametrize("with_init", [True, False])
def test_packed_sequences(dt, idx, with_init):
    lens = SEQ_CASES[idx]
    T = sum(lens[0])
    prob = si.make_problem(len(lens), T, 2, 32, 64, 1, dtype=dt, seed=31 + idx, d_skip=True,
                           seqlens=lens, init_std=0.5 if with_init else 0.0)
    check_full(prob, 64, label="packed%s" % lens)


def test_worked_example_split_at_a_block_boundary():
    """The three-step a = 1/2 example embedded at positions Q-2, Q-1, Q: y_Q must be 8.5, not 6."""
    for dt in ("bf16", "f32"):
        Q = 64
        T = 2 * Q
        prob = si.make_problem(1, T, 1, 32, 64, 1, dtype=dt, seed=1)
        tdt = prob["x"].dtype
        x = torch.zeros(1, T, 1, 32, dtype=tdt)
        x[0, Q - 2, 0, 0], x[0, Q - 1, 0, 0], x[0, Q, 0, 0] = 2.0, 4.0, 6.0
        Bm = torch.zeros(1, T, 1, 64, dtype=tdt)
        Bm[..., 0] = 1.0
        prob.update(x=x, B=Bm, C=Bm.clone(), dt=torch.ones(1, T, 1), D=None, init=None,
                    A_log=torch.tensor([float(np.log(np.log(2.0)))], dtype=torch.float32))
        announce("worked example dtype=%s" % dt)
        y, _ = run_gpu(prob, chunk_len=Q)
        np.testing.assert_allclose(y[0, Q - 2:Q + 1, 0, 0], [2.0, 5.0, 8.5], rtol=0, atol=1e-5)
        assert abs(y[0, Q, 0, 0] - 6.0) > 1.0


def test_chunk_length_invariance():
    prob = si.make_problem(1, 300, 2, 64, 128, 1, dtype="bf16", seed=41, d_skip=True, init_std=0.5)
    yr, fr = run_oracle(prob)
    outs = {}
    for Q in (16, 32, 64, 128, 256):
        announce("chunk invariance Q=%d" % Q)
        y, f = run_gpu(prob, chunk_len=Q)
        assert_parity(y, yr, TOL["bf16"], "y Q=%d" % Q)
        assert_parity(f, fr, TOL["bf16"], "final Q=%d" % Q)
        outs[Q] = (y, f)
    # chunk lengths that are multiples of 64 run the same kernel
    np.testing.assert_array_equal(outs[64][0], outs[256][0])


def test_empty_and_single_token():
    import mamba_ssd_scan_chunked_amd as ssd
    for T in (0, 1):
        prob = si.make_problem(2, T, 2, 32, 64, 1, dtype="bf16", seed=5, init_std=0.5)
        announce("T=%d" % T)
        y, f = run_gpu(prob, chunk_len=64)
        yr, fr = run_oracle(prob)
        if T == 0:
            assert y.size == 0
            np.testing.assert_array_equal(f, prob["init"].double().numpy())   # state after no token
        else:
            assert_parity(y, yr, TOL["bf16"], "y")
            assert_parity(f, fr, TOL["bf16"], "final")
    announce("batch=0")
    prob = si.make_problem(0, 64, 2, 32, 64, 1, dtype="bf16", seed=5)
    y, f = run_gpu(prob, chunk_len=64)
    assert y.size == 0 and f.size == 0


def test_outputs_fully_written_and_deterministic():
    prob = si.make_problem(2, 190, 2, 64, 128, 1, dtype="bf16", seed=51, d_skip=True, init_std=0.5,
                           seqlens=[[60, 70, 60], [190]])
    d = to_device(prob)
    import mamba_ssd_scan_chunked_amd as ssd
    announce("nan-poisoned outputs")
    res = []
    for _ in range(2):
        y = torch.full((2, 190, 2, 64), float("nan"), device="cuda")
        f = torch.full((prob["nseqs"], 2, 64, 128), float("nan"), device="cuda")
        ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=64, init_state=d["init"],
                    seq_idx=d["seq_idx"], nseqs=prob["nseqs"], y=y, final_state=f)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all() and torch.isfinite(f).all()
        res.append((y.cpu(), f.cpu()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_sequences_do_not_leak():
    lens = [[50, 80, 70]]
    prob = si.make_problem(1, 200, 2, 32, 64, 1, dtype="bf16", seed=61, init_std=0.5, seqlens=lens)
    announce("no leak")
    y, f = run_gpu(prob, chunk_len=64)
    p2 = dict(prob)
    x = prob["x"].clone()
    x[:, 50:130] *= 1e4
    p2["x"] = x
    y2, f2 = run_gpu(p2, chunk_len=64)
    np.testing.assert_array_equal(y[:, :50], y2[:, :50])
    np.testing.assert_array_equal(y[:, 130:], y2[:, 130:])
    np.testing.assert_array_equal(f[0], f2[0])
    np.testing.assert_array_equal(f[2], f2[2])


def test_forward_into_preallocated_outputs():
    """The raw entry point on caller-owned outputs, with no workspace, equals forward()."""
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(2, 160, 4, 64, 128, 2, dtype="bf16", seed=71, d_skip=True, init_std=0.5)
    d = to_device(prob)
    announce("forward_into")
    y1, f1 = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], chunk_len=64, init_state=d["init"])
    p = ssd.problem(2, 160, 4, 64, 128, 2, 64, 2, ssd.DTYPE_BF16, 0)
    assert ssd.workspace_size(p) == 0
    y2 = torch.empty_like(y1)
    f2 = torch.empty_like(f1)
    ssd.forward_into(p, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], None, y2, f2, None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_in_place_state_carry():
    """final_state may alias init_state: a split run chained in place equals the unsplit run."""
    import mamba_ssd_scan_chunked_amd as ssd
    prob = si.make_problem(2, 256, 2, 64, 128, 1, dtype="bf16", seed=81, init_std=0.5)
    d = to_device(prob)
    announce("in-place carry")
    yfull, ffull = ssd.forward(d["x"], d["dt"], d["A_log"], d["B"], d["C"], chunk_len=64, init_state=d["init"])
    st = d["init"].clone()
    ys = []
    for lo, hi in ((0, 100), (100, 256)):
        sl = slice(lo, hi)
        y, _ = ssd.forward(d["x"][:, sl].contiguous(), d["dt"][:, sl].contiguous(), d["A_log"],
                           d["B"][:, sl].contiguous(), d["C"][:, sl].contiguous(), chunk_len=64,
                           init_state=st, final_state=st)
        ys.append(y)
    torch.cuda.synchronize()
    y2 = torch.cat(ys, dim=1)
    assert_parity(y2.cpu().double().numpy(), yfull.cpu().double().numpy(), 2e-2, "y")
    assert_parity(st.cpu().double().numpy(), ffull.cpu().double().numpy(), 2e-2, "final")


# ------------------------------------------------------------------ measured workloads, sampled heads

@pytest.mark.parametrize("name,k", [("m130_bf16", 6), ("m2p7_bf16", 8), ("long_n64", 3), ("long_n128", 3),
                                    ("long_n256", 3), ("packed_bf16", 6)])
def test_workload_sampled(name, k):
    w = si.WORKLOADS[name]
    prob = si.make_workload(w)
    announce("workload %s (sampled %d pairs)" % (name, k))
    y, f = run_gpu(prob, chunk_len=w.chunk_len)
    pairs = sample_pairs(w.batch, w.nheads, k, seed=w.seed)
    tol = TOL[w.dtype]
    for (b, h), (yr, fr, seqs) in zip(pairs, oracle_pairs(prob, pairs)):
        assert_parity(y[b, :, h], yr, tol, "y[%d,:,%d]" % (b, h))
        assert_parity(f[seqs, h], fr, tol, "final[%s,%d]" % (seqs[:3], h))


# ------------------------------------------------------------------ five slices per workgroup
# Between 256 and 320 (row, head) items of 64 channels: the library packs five
# 16-channel slices into a workgroup, so a workgroup may hold parts of two heads.

@pytest.mark.parametrize("case", [
    # b, T, H, N, G, chunk, euler
    (1, 130, 260, 64, 1, 64, False),
    (2, 70, 150, 128, 1, 64, True),
    (1, 100, 300, 64, 5, 32, False),      # (H/G)*4 = 240 slices per group: still five per workgroup
    (1, 90, 265, 64, 5, 64, False),       # (H/G)*4 = 212: not a multiple of five, one head per workgroup
    # N = 128 with 64-token blocks: the swizzled B and X tiles
    (1, 65, 260, 128, 1, 64, False),      # one token past a block
    (2, 129, 140, 128, 4, 64, False),     # four groups of 35 heads
    (3, 1, 100, 128, 1, 64, True),        # a single token
])
def test_five_slice_workgroups(case):
    b, T, H, N, G, Q, euler = case
    prob = si.make_problem(b, T, H, 64, N, G, dtype="bf16", seed=H + T, d_skip=True, init_std=0.5)
    check_full(prob, Q, dt_scales_x=euler, label="five slices b=%d H=%d G=%d" % (b, H, G))


# ------------------------------------------------------------------ no leak of Inf or NaN
# "088 Mamba-2", section 5: independent documents packed into one row must not
# leak into each other.  An Inf or NaN planted in one sequence's inputs may ruin
# that sequence's outputs, but every other sequence's y and final state must stay
# finite and bit-identical to the clean run (the kernels select rather than
# multiply by zero wherever sequences meet inside a block).

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("field,value", [("x", float("inf")), ("x", float("-inf")), ("x", float("nan")),
                                         ("B", float("inf")), ("C", float("-inf")), ("dt", float("inf")),
                                         ("dt", float("nan"))])
@pytest.mark.parametrize("shape", ["blocks", "segments"])
def test_inf_in_one_sequence_does_not_leak(dtype, field, value, shape):
    if shape == "blocks":
        b, T, H, P, N, lens, bad = 2, 200, 2, 32, 64, [[50, 80, 70], [200]], 1     # boundaries inside blocks
    else:
        b, T, H, P, N, lens, bad = 1, 1600, 2, 32, 64, [[500, 600, 500]], 1        # rows split into segments
    if dtype == "f32":
        P, N = 16, 32
    prob = si.make_problem(b, T, H, P, N, 1, dtype=dtype, seed=97, d_skip=True, init_std=0.5, seqlens=lens)
    seq = prob["seq_idx"]
    announce("inf no-leak %s %s=%s %s" % (dtype, field, value, shape))
    y0, f0 = run_gpu(prob, chunk_len=64)
    p2 = dict(prob)
    t = prob[field].clone()
    rows, toks = torch.nonzero(seq == bad, as_tuple=True)
    pick = torch.tensor([0, len(toks) // 2, len(toks) - 1])       # first, a middle and the last token of it
    r, tk = rows[pick], toks[pick]
    if field == "dt":
        t[r, tk, 0] = value
    else:
        t[r, tk] = value
    p2[field] = t
    y1, f1 = run_gpu(p2, chunk_len=64)
    others = (seq != bad).numpy()
    assert np.isfinite(y1[others]).all()
    np.testing.assert_array_equal(y1[others], y0[others])
    keep = [k for k in range(prob["nseqs"]) if k != bad]
    assert np.isfinite(f1[keep]).all()
    np.testing.assert_array_equal(f1[keep], f0[keep])
    yr, fr = run_oracle(prob)
    assert_parity(y0, yr, TOL[dtype], "y (clean)")
    assert_parity(f0, fr, TOL[dtype], "final (clean)")


def test_headline_row_every_head():
    """At the full 2.7B-layer shape, every head of one row (all 80 heads, so every
    five-slice workgroup of the row, including those that straddle two heads)
    against the oracle over the whole 4096-token length."""
    w = si.WORKLOADS["m2p7_bf16"]
    prob = si.make_workload(w)
    announce("m2p7 row 2, all %d heads" % w.nheads)
    y, f = run_gpu(prob, chunk_len=w.chunk_len)
    pairs = [(2, h) for h in range(w.nheads)]
    for (b, h), (yr, fr, seqs) in zip(pairs, oracle_pairs(prob, pairs)):
        assert_parity(y[b, :, h], yr, TOL["bf16"], "y[%d,:,%d]" % (b, h))
        assert_parity(f[seqs, h], fr, TOL["bf16"], "final[%d,%d]" % (b, h))
