"""ssd_forward_noalloc (the entry point that allocates nothing; its scratch is a
static device array) against ssd_forward with a caller workspace, through the C
ABI, on problems whose rows are split into segments (so the scratch is used):
two calls in a row, the second with a smaller input, each bit-equal to
ssd_forward on the same inputs and within the bf16 tolerance of the oracle."""
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


def both(prob, chunk_len=64):
    import mamba_ssd_scan_chunked_amd as ssd
    d = to_device(prob)
    b, T, H, P = prob["x"].shape
    G, N = prob["B"].shape[2], prob["B"].shape[3]
    packed = prob["seq_idx"] is not None
    ns = prob["nseqs"] if packed else b
    p = ssd.problem(b, T, H, P, N, G, chunk_len, ns, ssd.DTYPE_BF16, 0)
    need = ssd.workspace_size(p)
    assert 0 < need <= ssd.noalloc_scratch_bytes()        # rows split: the scratch is in use
    f32 = dict(dtype=torch.float32, device="cuda")
    y1, f1 = torch.full((b, T, H, P), float("nan"), **f32), torch.full((ns, H, P, N), float("nan"), **f32)
    y2, f2 = torch.full_like(y1, float("nan")), torch.full_like(f1, float("nan"))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ssd.forward_into(p, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], d["seq_idx"], y1, f1, ws)
    ssd.forward_into_noalloc(p, d["x"], d["dt"], d["A_log"], d["B"], d["C"], d["D"], d["init"], d["seq_idx"], y2, f2)
    torch.cuda.synchronize()
    return (y1.cpu(), f1.cpu()), (y2.cpu(), f2.cpu())


def test_noalloc_equals_forward_on_two_calls_in_a_row():
    cases = [
        # b, T, H, P, N, G, seqlens: the first call larger than the second
        (2, 2000, 4, 64, 128, 2, None),                 # 8 items: 8 segments of 4 blocks per row
        (1, 1100, 2, 32, 64, 1, [[450, 1, 649]]),       # packed sequences, 2 items: 4 segments
    ]
    sizes = []
    for i, (b, T, H, P, N, G, lens) in enumerate(cases):
        prob = si.make_problem(b, T, H, P, N, G, dtype="bf16", seed=300 + i, d_skip=True, init_std=0.5,
                               seqlens=lens)
        announce("noalloc call %d: b=%d T=%d H=%d P=%d N=%d G=%d packed=%s" % (i + 1, b, T, H, P, N, G, lens is not None))
        (y1, f1), (y2, f2) = both(prob)
        assert torch.isfinite(y2).all() and torch.isfinite(f2).all()
        assert torch.equal(y1, y2) and torch.equal(f1, f2)
        yr, fr = run_oracle(prob)
        assert_parity(y2.double().numpy(), yr, TOL["bf16"], "y")
        assert_parity(f2.double().numpy(), fr, TOL["bf16"], "final")
        sizes.append(b * T * H * P)
    assert sizes[1] < sizes[0]
