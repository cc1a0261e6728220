"""Rows split into segments that run in parallel (local pass, combine, scan from
each segment's incoming state), against the CPU oracle.

The library picks the number of segments from the problem; the problem's
`segments` field forces it, so each case runs unsplit and split into several
segments (including a ragged last one).  Same tolerance as the other parity tests: max |got - ref| <=
tol * max |ref|, tol = 2e-2 for bf16 inputs and 1e-5 for fp32.
"""
import sys

import numpy as np
import pytest
import torch

import ssd_inputs as si
from ssd_testlib import TOL, assert_parity, dtype_name, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def run_split(prob, chunk_len, nseg, dt_scales_x=False):
    return run_gpu(prob, chunk_len=chunk_len, dt_scales_x=dt_scales_x, segments=nseg)


CASES = [
    # dtype, b, T, H, P, N, G, chunk, seqlens (None = one sequence per row)
    ("bf16", 2, 640, 3, 64, 128, 1, 64, None),
    ("bf16", 1, 700, 2, 32, 256, 1, 256, None),
    ("bf16", 1, 1000, 2, 64, 64, 2, 32, None),
    ("f32", 1, 330, 2, 32, 64, 1, 32, None),
    ("f32", 2, 260, 2, 16, 16, 1, 64, None),
    # sequence boundaries exactly at segment edges (4 blocks of 64), inside segments, spanning several
    ("bf16", 1, 640, 2, 64, 128, 1, 64, [[256, 256, 128]]),
    ("bf16", 2, 640, 2, 64, 128, 1, 64, [[1, 255, 1, 300, 83], [640]]),
    ("f32", 1, 640, 2, 32, 64, 1, 64, [[100, 156, 256, 128]]),
]


@pytest.mark.parametrize("nseg", [1, 2, 3, 5])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-b%d-T%d-H%d-P%d-N%d-G%d-Q%d-%s" % (c[:8] + ("seq" if c[8] else "rows",)))
@pytest.mark.parametrize("with_init", [True, False])
def test_split_rows_match_the_oracle(case, nseg, with_init):
    dt, b, T, H, P, N, G, Q, lens = case
    prob = si.make_problem(b, T, H, P, N, G, dtype=dt, seed=T + N + nseg, d_skip=True, seqlens=lens,
                           init_std=0.5 if with_init else 0.0)
    announce("split nseg=%d %s init=%s" % (nseg, case, with_init))
    y, f = run_split(prob, Q, nseg)
    yr, fr = run_oracle(prob)
    tol = TOL[dt]
    assert_parity(y, yr, tol, "y")
    assert_parity(f, fr, tol, "final")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_split_rows_euler(dt):
    prob = si.make_problem(1, 512, 2, 32, 64, 1, dtype=dt, seed=91, d_skip=True, init_std=0.3,
                           seqlens=[[200, 312]])
    announce("split euler %s" % dt)
    y, f = run_split(prob, 64, 4, dt_scales_x=True)
    yr, fr = run_oracle(prob, dt_scales_x=True)
    assert_parity(y, yr, TOL[dt], "y")
    assert_parity(f, fr, TOL[dt], "final")


def test_split_and_unsplit_agree_closely():
    """Splitting only regroups the same sums: results differ by rounding only."""
    prob = si.make_problem(2, 1024, 4, 64, 128, 1, dtype="bf16", seed=93, d_skip=True, init_std=0.5)
    announce("split vs unsplit")
    y1, f1 = run_split(prob, 256, 1)
    y8, f8 = run_split(prob, 256, 8)
    scale_y, scale_f = np.abs(y1).max(), np.abs(f1).max()
    assert np.abs(y8 - y1).max() <= 1e-2 * scale_y
    assert np.abs(f8 - f1).max() <= 1e-2 * scale_f


def test_default_split_on_a_long_row():
    """Few (row, head) items and a long row: the library splits it by itself."""
    import mamba_ssd_scan_chunked_amd as ssd
    p = ssd.problem(1, 4096, 4, 64, 128, 1, 256, 1, ssd.DTYPE_BF16, 0)
    assert ssd.workspace_size(p) > 0
    prob = si.make_problem(1, 4096, 4, 64, 128, 1, dtype="bf16", seed=95, d_skip=True, init_std=0.5)
    announce("default split T=4096 H=4")
    y, f = run_gpu(prob, chunk_len=256)
    yr, fr = run_oracle(prob)
    assert_parity(y, yr, TOL["bf16"], "y")
    assert_parity(f, fr, TOL["bf16"], "final")
