"""The library's calls recorded into a HIP graph (through torch.cuda.graph) and replayed.

Every entry point only launches kernels on the caller's stream: no allocation,
memset, copy or synchronisation.  A whole forward, a decoding loop of
single-token steps or a whole backward can therefore be captured once and
replayed.  Each replay, with eager work and synchronisations between the
replays, must reproduce the eager result bit for bit (every kernel is
deterministic); output buffers are poisoned with NaN before each replay so that
an element the graph did not write shows.
"""
import sys

import pytest
import torch

import ssd_inputs as si
from ssd_testlib import to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3
F32 = dict(dtype=torch.float32, device="cuda")


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def _dtype_code(ssd, dt_):
    return ssd.DTYPE_BF16 if dt_ == "bf16" else ssd.DTYPE_F32


def _poison(*ts):
    for t in ts:
        t.fill_(float("nan"))


FWD = [
    # dtype, b, T, H, P, N, G
    ("bf16", 4, 200, 80, 64, 128, 1),    # 320 (row, head) items: five-slice workgroups, one launch
    ("bf16", 1, 1000, 4, 64, 128, 2),    # 4 items: rows split (local pass, combine, scan), workspace
    ("f32", 2, 130, 2, 16, 16, 1),
]


@pytest.mark.parametrize("shape", FWD, ids=lambda s: "%s-b%d-T%d-H%d-P%d-N%d-G%d" % s)
def test_forward_graph_replays_equal_eager(shape):
    import mamba_ssd_scan_chunked_amd as ssd
    dt_, b, T, H, P, N, G = shape
    announce("graph forward %s" % (shape,))
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt_, seed=11, d_skip=True, init_std=0.5)
    d = to_device(prob)
    p = ssd.problem(b, T, H, P, N, G, 256, b, _dtype_code(ssd, dt_), 0)
    wsb = ssd.workspace_size(p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb > 0 else None

    def run(y, f):
        ssd.forward_into(p, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], None, y, f, ws)

    y0, f0 = torch.empty((b, T, H, P), **F32), torch.empty((b, H, P, N), **F32)
    run(y0, f0)
    torch.cuda.synchronize()
    yg, fg = torch.empty_like(y0), torch.empty_like(f0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(yg, fg)
    ye, fe = torch.empty_like(y0), torch.empty_like(f0)
    for rep in range(REPLAYS):
        _poison(yg, fg, ye, fe)
        torch.cuda.synchronize()
        g.replay()
        run(ye, fe)                      # eager work on the same stream between replays
        torch.cuda.synchronize()
        assert torch.equal(yg, y0) and torch.equal(fg, f0), "replay %d differs from the eager forward" % rep
        assert torch.equal(ye, y0) and torch.equal(fe, f0), "eager forward after replay %d differs" % rep


@pytest.mark.parametrize("dt_", ["bf16", "f32"])
def test_decode_loop_graph_replays_equal_eager(dt_):
    """Eight single-token steps on one state, captured as one graph."""
    import mamba_ssd_scan_chunked_amd as ssd
    b, K, H, P, N, G = 4, 8, 80 if dt_ == "bf16" else 4, 64, 128, 1
    announce("graph decode loop %s b=%d H=%d" % (dt_, b, H))
    prob = si.make_problem(b, K, H, P, N, G, dtype=dt_, seed=5, d_skip=True, init_std=0.5)
    d = to_device(prob)
    xs = [d["x"][:, k:k + 1].contiguous() for k in range(K)]
    dts = [d["dt"][:, k:k + 1].contiguous() for k in range(K)]
    Bs = [d["B"][:, k:k + 1].contiguous() for k in range(K)]
    Cs = [d["C"][:, k:k + 1].contiguous() for k in range(K)]
    state0 = d["init"].clone()

    def loop(state, ys):
        for k in range(K):
            ssd.step(xs[k], dts[k], d["A_log"], Bs[k], Cs[k], d["D"], state, y=ys[k])

    st_ref = state0.clone()
    y_ref = [torch.empty((b, 1, H, P), **F32) for _ in range(K)]
    loop(st_ref, y_ref)
    torch.cuda.synchronize()
    st_g = state0.clone()
    y_g = [torch.empty((b, 1, H, P), **F32) for _ in range(K)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop(st_g, y_g)
    st_e = state0.clone()
    y_e = [torch.empty((b, 1, H, P), **F32) for _ in range(K)]
    for rep in range(REPLAYS):
        _poison(*y_g, *y_e)
        st_g.copy_(state0)
        st_e.copy_(state0)
        torch.cuda.synchronize()
        g.replay()
        loop(st_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(st_g, st_ref), "replay %d: state differs" % rep
        assert all(torch.equal(a, r) for a, r in zip(y_g, y_ref)), "replay %d: y differs" % rep
        assert torch.equal(st_e, st_ref) and all(torch.equal(a, r) for a, r in zip(y_e, y_ref))


BWD = [
    # dtype, b, T, H, P, N, G
    ("bf16", 1, 1000, 4, 64, 128, 2),    # rows split in segments; per-head sums over the group
    ("bf16", 3, 200, 4, 64, 128, 4),     # one head per group: passes write dB, dC directly
    ("f32", 2, 130, 2, 16, 16, 1),
]


@pytest.mark.parametrize("shape", BWD, ids=lambda s: "%s-b%d-T%d-H%d-P%d-N%d-G%d" % s)
def test_backward_graph_replays_equal_eager(shape):
    import mamba_ssd_scan_chunked_amd as ssd
    dt_, b, T, H, P, N, G = shape
    announce("graph backward %s" % (shape,))
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt_, seed=13, d_skip=True, init_std=0.5)
    d = to_device(prob)
    gen = torch.Generator(device="cpu").manual_seed(17)
    dy = torch.randn((b, T, H, P), generator=gen, dtype=torch.float32).cuda()
    dfinal = torch.randn((b, H, P, N), generator=gen, dtype=torch.float32).cuda()
    p = ssd.problem(b, T, H, P, N, G, 256, b, _dtype_code(ssd, dt_), 0)
    ws = torch.empty(ssd.backward_workspace_size(p), dtype=torch.uint8, device="cuda")
    shapes = {"dx": (b, T, H, P), "ddt": (b, T, H), "dA_log": (H,), "dB": (b, T, G, N), "dC": (b, T, G, N),
              "dD": (H,), "dinit": (b, H, P, N), "ddt_bias": (H,)}

    def outs():
        return {k: torch.empty(s, **F32) for k, s in shapes.items()}

    def run(out):
        ssd.backward_into(p, d["x"], d["dt"], None, d["A_log"], d["B"], d["C"], d["D"], d["init"], dy, dfinal,
                          out, ws)

    ref = outs()
    run(ref)
    torch.cuda.synchronize()
    og = outs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(og)
    oe = outs()
    for rep in range(REPLAYS):
        _poison(*og.values(), *oe.values())
        torch.cuda.synchronize()
        g.replay()
        run(oe)
        torch.cuda.synchronize()
        for k in shapes:
            assert torch.equal(og[k], ref[k]), "replay %d: %s differs from the eager backward" % (rep, k)
            assert torch.equal(oe[k], ref[k]), "eager backward after replay %d: %s differs" % (rep, k)
