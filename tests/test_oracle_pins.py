"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test compares the oracle (fp64 recurrence in C) with something other than
itself: values printed on the pages (tests/golden/*.json, each with its
source), closed forms, the independently written dense dual form, invariants
(rank of past-to-future blocks, continuation, packing, linearity) and special
cases that reduce to textbook results.  ``test_planted_mistakes_are_caught``
compiles mutated copies of the oracle source and checks that this suite's
checks reject each of them.
"""
import json
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import brute
import ssd_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def scalar_problem(a, x, B=1.0, C=1.0, init=None):
    """N = P = 1, one head, dt = 1 and A_log chosen so that exp(dt * A) == a."""
    T = len(x)
    A_log = np.array([math.log(-math.log(a))])
    xs = np.asarray(x, dtype=np.float64).reshape(1, T, 1, 1)
    dt = np.ones((1, T, 1))
    Bm = np.full((1, T, 1, 1), B)
    Cm = np.full((1, T, 1, 1), C)
    ini = None if init is None else np.full((1, 1, 1, 1), float(init))
    return dict(x=xs, dt=dt, A_log=A_log, B=Bm, C=Cm, init=ini)


def run(p, fn=None, **kw):
    fn = fn or oracle.recurrence
    return fn(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p.get("D"), p.get("init"),
              p.get("seq_idx"), p.get("nseqs"), **kw)


# ---------------------------------------------------------------- worked examples

def test_w1_three_steps():
    g = golden("w1_three_steps.json")
    y, fin = run(scalar_problem(g["a"], g["x"], g["B"], g["C"]))
    np.testing.assert_allclose(y.ravel(), g["h"], rtol=0, atol=1e-12)
    assert abs(fin.item() - g["h"][-1]) < 1e-12


def test_w1_matrix_form():
    g = golden("w1_three_steps.json")
    T = len(g["x"])
    M = brute.semiseparable_matrix(np.full(T, g["a"]), np.ones((T, 1)), np.ones((T, 1)))
    np.testing.assert_allclose(M, g["M"], atol=1e-15)
    np.testing.assert_allclose(M @ np.array(g["x"]), g["h"], atol=1e-12)


def test_w1_split_state_handoff():
    g = golden("w1_three_steps.json")["split"]
    a = golden("w1_three_steps.json")["a"]
    y1, s1 = run(scalar_problem(a, g["first_block"]))
    assert abs(s1.item() - g["first_block_end_state"]) < 1e-12
    y2, _ = run(scalar_problem(a, g["second_block"], init=s1.item()))
    assert abs(y2.item() - g["y3"]) < 1e-12
    # the local part alone (zero initial state) is the wrong answer the page warns about
    y_local, _ = run(scalar_problem(a, g["second_block"]))
    assert abs(y_local.item() - g["second_block_local"]) < 1e-12
    assert abs(y_local.item() - g["y3_if_zero_initial_state"]) < 1e-12
    assert abs((y2.item() - y_local.item()) - g["incoming"]) < 1e-12


def test_w2_past_to_future_block_is_rank_one():
    g = golden("w2_rank_cut.json")
    T, m = g["T"], g["cut_after"]
    M = brute.semiseparable_matrix(np.full(T, g["a"]), np.ones((T, 1)), np.ones((T, 1)))
    blk = M[m:, :m]
    np.testing.assert_allclose(blk, g["past_to_future_block"], atol=1e-15)
    np.testing.assert_allclose(np.outer(g["left_factor"], g["right_factor"]), blk, atol=1e-15)
    assert abs(np.linalg.det(blk) - g["block_det"]) < 1e-15
    assert np.linalg.matrix_rank(blk) == g["block_rank"]
    assert abs(np.linalg.det(M) - g["full_matrix_det"]) < 1e-12
    assert np.linalg.matrix_rank(M) == g["full_matrix_rank"]
    # the carried state after the cut is x1/2 + x2 (the oracle's final state after 2 steps)
    rng = np.random.default_rng(0)
    for _ in range(3):
        x12 = rng.standard_normal(2)
        _, s = run(scalar_problem(g["a"], x12))
        assert abs(s.item() - float(np.dot(g["carried_state_coeffs"], x12))) < 1e-12


def test_w3_one_dimensional_example():
    g = golden("w3_one_dim.json")
    y, _ = run(scalar_problem(g["Abar"], g["x"], B=g["Bbar"], C=g["C"]))
    np.testing.assert_allclose(y.ravel(), g["h"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.round(y.ravel(), g["printed_decimals"]), g["printed_h"], atol=1e-12)


# ---------------------------------------------------------------- dual form / closed form

CASES = [
    dict(b=1, T=17, H=2, P=3, N=4, G=1),
    dict(b=2, T=33, H=4, P=5, N=3, G=2, d_skip=True),
    dict(b=2, T=40, H=6, P=4, N=6, G=3, init_std=0.7, seqlens=[[7, 1, 32], [40]]),
    dict(b=1, T=64, H=2, P=8, N=8, G=1, d_skip=True, init_std=0.5, seqlens=[[1, 63]]),
    dict(b=3, T=29, H=2, P=2, N=5, G=1, init_std=1.0),
]


def _case_problem(c, seed):
    c = dict(c)
    return si.make_problem(c.pop("b"), c.pop("T"), c.pop("H"), c.pop("P"), c.pop("N"), c.pop("G"),
                           dtype="f32", seed=seed, **c)


@pytest.mark.parametrize("idx", range(len(CASES)))
@pytest.mark.parametrize("euler", [False, True])
def test_recurrence_matches_dual_form(idx, euler):
    p = _case_problem(CASES[idx], seed=100 + idx)
    y, f = run(p, dt_scales_x=euler)
    y2, f2 = run(p, fn=brute.dual_form, dt_scales_x=euler)
    scale = max(np.abs(y2).max(), 1.0)
    assert np.abs(y - y2).max() <= 1e-12 * scale
    assert np.abs(f - f2).max() <= 1e-12 * max(np.abs(f2).max(), 1.0)


def test_past_to_future_rank_at_most_N():
    rng = np.random.default_rng(7)
    T, N = 24, 3
    for _ in range(5):
        a = rng.uniform(0.3, 1.0, T)
        B = rng.standard_normal((T, N))
        C = rng.standard_normal((T, N))
        M = brute.semiseparable_matrix(a, B, C)
        for m in range(N, T - N):
            blk = M[m:, :m]
            sv = np.linalg.svd(blk, compute_uv=False)
            rank = int((sv > 1e-10 * sv[0]).sum())
            assert rank <= N
            assert rank == N            # generic inputs reach the bound
        assert np.linalg.matrix_rank(M) == T    # the whole matrix is not low rank


def test_state_is_the_only_path_across_a_cut():
    """y after a cut depends on the past only through the P x N state at the cut."""
    p = _case_problem(dict(b=1, T=50, H=3, P=4, N=5, G=1, d_skip=True), seed=11)
    y, _ = run(p)
    for m in (1, 13, 31, 49):
        first = {k: (v[:, :m] if k in ("x", "dt", "B", "C") and v is not None else v) for k, v in p.items()}
        rest = {k: (v[:, m:] if k in ("x", "dt", "B", "C") and v is not None else v) for k, v in p.items()}
        y1, s1 = run(first)
        rest["init"] = s1
        y2, _ = run(rest)
        np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- special cases

def test_no_decay_is_a_prefix_sum_of_outer_products():
    p = _case_problem(dict(b=1, T=30, H=2, P=3, N=4, G=1), seed=5)
    p["dt"] = np.zeros_like(p["dt"].numpy())            # a_t = exp(0) = 1
    y, f = run(p)
    x = p["x"].double().numpy()[0]
    B = p["B"].double().numpy()[0, :, 0]
    C = p["C"].double().numpy()[0, :, 0]
    for h in range(2):
        S = np.cumsum(np.einsum("tp,tn->tpn", x[:, h], B), axis=0)   # S_t = sum_{s<=t} x_s B_s^T
        np.testing.assert_allclose(y[0, :, h], np.einsum("tpn,tn->tp", S, C), atol=1e-12)
        np.testing.assert_allclose(f[0, h], S[-1], atol=1e-12)


def test_constant_decay_is_a_geometric_series():
    a, xv, T = 0.8, 1.5, 20
    y, _ = run(scalar_problem(a, [xv] * T))
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(y.ravel(), xv * (1 - a ** t) / (1 - a), rtol=1e-13)


def test_full_decay_keeps_only_the_diagonal():
    p = _case_problem(dict(b=1, T=12, H=2, P=3, N=4, G=1, d_skip=True), seed=6)
    p["dt"] = np.full(p["dt"].shape, 1e6)                 # a_t = exp(-1e6 * |A|) = 0
    y, _ = run(p)
    x = p["x"].double().numpy()[0]
    B = p["B"].double().numpy()[0, :, 0]
    C = p["C"].double().numpy()[0, :, 0]
    D = p["D"].double().numpy()
    expect = np.einsum("tn,tn->t", C, B)[:, None, None] * x + D[None, :, None] * x
    np.testing.assert_allclose(y[0], expect, atol=1e-12)


# ---------------------------------------------------------------- identities

def test_packed_rows_equal_separate_runs():
    lens = [9, 1, 23, 31]
    p = _case_problem(dict(b=1, T=64, H=2, P=3, N=4, G=1, init_std=0.6, seqlens=[lens], d_skip=True), seed=9)
    y, f = run(p)
    start = 0
    for k, L in enumerate(lens):
        sl = slice(start, start + L)
        q = {kk: (v[:, sl] if kk in ("x", "dt", "B", "C") else v) for kk, v in p.items()}
        q["seq_idx"] = None
        q["init"] = p["init"][k:k + 1]
        q["nseqs"] = None
        yk, fk = run(q)
        np.testing.assert_allclose(y[:, sl], yk, atol=1e-12)
        np.testing.assert_allclose(f[k], fk[0], atol=1e-12)
        start += L


def test_packed_sequences_do_not_leak():
    lens = [20, 20, 24]
    p = _case_problem(dict(b=1, T=64, H=2, P=3, N=4, G=1, seqlens=[lens]), seed=10)
    y, _ = run(p)
    q = dict(p)
    x = p["x"].clone()
    x[:, 20:40] *= 1e4
    q["x"] = x
    y2, _ = run(q)
    np.testing.assert_array_equal(y[:, :20], y2[:, :20])
    np.testing.assert_array_equal(y[:, 40:], y2[:, 40:])


def test_linear_in_skip_and_initial_state():
    p = _case_problem(dict(b=2, T=25, H=2, P=3, N=4, G=1, d_skip=True, init_std=1.0), seed=12)
    y, f = run(p)
    q = dict(p, D=None, init=None)
    y0, f0 = run(q)
    x = p["x"].double().numpy()
    yd, _ = run(dict(p, init=None))
    np.testing.assert_allclose(yd - y0, p["D"].double().numpy()[None, None, :, None] * x, atol=1e-12)
    init = p["init"].double().numpy()
    yi1, fi1 = run(dict(q, init=init))
    yi2, fi2 = run(dict(q, init=2.5 * init))
    np.testing.assert_allclose(yi2 - y0, 2.5 * (yi1 - y0), atol=1e-11)
    np.testing.assert_allclose(fi2 - f0, 2.5 * (fi1 - f0), atol=1e-11)


def test_euler_flag_equals_prescaled_input():
    p = _case_problem(dict(b=1, T=30, H=3, P=4, N=2, G=1, d_skip=True), seed=13)
    y, f = run(p, dt_scales_x=True)
    x = p["x"].double().numpy()
    xs = x * p["dt"].double().numpy()[..., None]
    y2, f2 = run(dict(p, x=xs, D=None))
    np.testing.assert_allclose(y, y2 + p["D"].double().numpy()[None, None, :, None] * x, atol=1e-12)
    np.testing.assert_allclose(f, f2, atol=1e-12)


def test_group_mapping_contiguous_heads():
    """Head h reads group h // (H/G); replicated groups equal a single group."""
    p = _case_problem(dict(b=1, T=20, H=4, P=3, N=4, G=2), seed=14)
    y, _ = run(p)
    for h in range(4):
        g = h // 2
        q = dict(p, x=p["x"][:, :, h:h + 1], dt=p["dt"][:, :, h:h + 1], A_log=p["A_log"][h:h + 1],
                 B=p["B"][:, :, g:g + 1], C=p["C"][:, :, g:g + 1])
        yh, _ = run(q)
        np.testing.assert_allclose(y[:, :, h:h + 1], yh, atol=1e-12)
    rep = dict(p, B=p["B"][:, :, :1].repeat(1, 1, 2, 1), C=p["C"][:, :, :1].repeat(1, 1, 2, 1))
    one = dict(p, B=p["B"][:, :, :1], C=p["C"][:, :, :1])
    np.testing.assert_allclose(run(rep)[0], run(one)[0], atol=1e-12)


# ------------------------------------------- step-size map and input discretisation

def _w1_with_step_map(dt_raw, dt_bias, A_log, **kw):
    g = golden("w1_three_steps.json")
    p = scalar_problem(g["a"], g["x"], g["B"], g["C"])
    T = len(g["x"])
    p = dict(p, dt=np.full((1, T, 1), float(dt_raw)), A_log=np.array([float(A_log)]))
    y, fin = run(p, dt_bias=np.array([float(dt_bias)]), **kw)
    return g, y, fin


def test_softplus_step_size_reproduces_w1():
    """softplus(v) == 1 exactly at v = ln(e - 1): with the bias carrying part of v and
    A = -ln 2 the decay is 1/2 again and the printed three-step example comes back."""
    v = math.log(math.e - 1.0)
    g, y, fin = _w1_with_step_map(v - 0.25, 0.25, math.log(math.log(2.0)), dt_softplus=True)
    np.testing.assert_allclose(y.ravel(), g["h"], rtol=0, atol=1e-12)
    assert abs(fin.item() - g["h"][-1]) < 1e-12


def test_softplus_at_zero_is_ln2():
    """softplus(0) = ln 2, so with A = -1 the decay is exp(-ln 2) = 1/2: the printed example."""
    g, y, _ = _w1_with_step_map(-0.5, 0.5, 0.0, dt_softplus=True)
    np.testing.assert_allclose(y.ravel(), g["h"], rtol=0, atol=1e-12)


def test_softplus_tails():
    """softplus(v) - v -> 0 for large v (about e^-v), and softplus(v) -> 0 for very
    negative v: then a = 1 and the map is a prefix sum."""
    p = _case_problem(dict(b=1, T=12, H=2, P=3, N=2, G=1), seed=21)
    big = dict(p, dt=np.full((1, 12, 2), 36.0))
    y_sp, f_sp = run(big, dt_softplus=True)
    y_id, f_id = run(big)
    np.testing.assert_allclose(y_sp, y_id, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(f_sp, f_id, rtol=1e-12, atol=1e-14)
    neg = dict(p, dt=np.full((1, 12, 2), -800.0))
    y0, _ = run(neg, dt_softplus=True)
    x = p["x"].double().numpy()
    B = p["B"].double().numpy()
    C = p["C"].double().numpy()
    cb = np.einsum("btgn,bsgn->bts", C, B)[0]           # (t, s), one group
    expect = np.einsum("ts,shp->thp", np.tril(cb), x[0])
    np.testing.assert_allclose(y0[0], expect, atol=1e-12)


def test_zoh_scales_w1_by_the_hold_factor():
    """Exact zero-order hold with a = 1/2, dt = 1, A = -ln 2: every write is scaled by
    (1/2 - 1) / (-ln 2) = 1 / (2 ln 2), and the map is linear in the writes."""
    g = golden("w1_three_steps.json")
    y, fin = run(scalar_problem(g["a"], g["x"], g["B"], g["C"]), zoh=True)
    k = 1.0 / (2.0 * math.log(2.0))
    np.testing.assert_allclose(y.ravel(), np.array(g["h"]) * k, rtol=1e-14, atol=0)
    assert abs(fin.item() - g["h"][-1] * k) < 1e-12


def test_zoh_steps_compose():
    """With x and B held for two steps, the exact hold over dt1 then dt2 equals one
    step over dt1 + dt2 (the solution operator of h' = A h + B x is a semigroup);
    Euler scaling does not have this property, which shows the check can fail."""
    rng = np.random.default_rng(22)
    H, P, N = 3, 4, 5
    x1 = rng.standard_normal((1, 1, H, P))
    B1 = rng.standard_normal((1, 1, 1, N))
    C1 = rng.standard_normal((1, 1, 1, N))
    init = rng.standard_normal((1, H, P, N))
    A_log = rng.uniform(-1.0, 1.0, H)
    dt1, dt2 = rng.uniform(0.1, 1.5, (1, 1, H)), rng.uniform(0.1, 1.5, (1, 1, H))
    two = dict(x=np.concatenate([x1, x1], 1), dt=np.concatenate([dt1, dt2], 1), A_log=A_log,
               B=np.concatenate([B1, B1], 1), C=np.concatenate([C1, C1], 1), init=init)
    one = dict(x=x1, dt=dt1 + dt2, A_log=A_log, B=B1, C=C1, init=init)
    _, f2 = run(two, zoh=True)
    _, f1 = run(one, zoh=True)
    np.testing.assert_allclose(f2, f1, rtol=1e-12, atol=1e-12)
    _, e2 = run(two, dt_scales_x=True)
    _, e1 = run(one, dt_scales_x=True)
    assert not np.allclose(e2, e1, rtol=1e-6, atol=1e-6)


def test_zoh_tends_to_euler_as_A_vanishes():
    """(e^{dt A} - 1) / A = dt (1 + dt A / 2 + ...): as A -> 0 the hold becomes Euler."""
    p = _case_problem(dict(b=1, T=16, H=2, P=3, N=4, G=1, init_std=1.0), seed=23)
    p = dict(p, A_log=np.full(2, -25.0))
    yz, fz = run(p, zoh=True)
    ye, fe = run(p, dt_scales_x=True)
    np.testing.assert_allclose(yz, ye, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(fz, fe, rtol=1e-9, atol=1e-12)
    yn, _ = run(p)
    assert not np.allclose(yz, yn, rtol=1e-3)


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "no_decay": ("S[p * N + n] = a * S[p * N + n] + xs[p] * Bt[n];", "S[p * N + n] = S[p * N + n] + xs[p] * Bt[n];"),
    "read_before_write": ("/* decay, then write: H_t = a_t H_{t-1} + x_t B_t^T */",
                          "for (int64_t p = 0; p < P; ++p) { double acc = 0.0; for (int64_t n = 0; n < N; ++n) acc += S[p*N+n]*Ct[n]; yt[p] = acc + Dh*xt[p]; } if (0)"),
    "decay_sign": ("const double A = -exp(A_log[h]);", "const double A = exp(A_log[h]);"),
    "b_c_swapped": ("acc += S[p * N + n] * Ct[n];", "acc += S[p * N + n] * Bt[n];"),
    "init_ignored": ("memcpy(S, init + (k * H + h) * P * N, (size_t)(P * N) * sizeof(double));",
                     "memset(S, 0, (size_t)(P * N) * sizeof(double));"),
    "group_interleaved": ("g = h / heads_per_group;", "g = h % G;"),
    "skip_on_scaled_x": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc + Dh * xs[p];"),
    "no_reset_at_boundary": ("if (t == 0 || k != cur) {", "if (t == 0) {"),
    "bias_ignored": ("+ (dt_bias ? dt_bias[h] : 0.0);", "+ 0.0;"),
    "softplus_wrong_branch": ("dtv + log1p(exp(-dtv))", "dtv + log1p(exp(dtv))"),
    "softplus_without_log": ("log1p(exp(dtv));", "exp(dtv);"),
    "zoh_as_euler": ("expm1(dtv * A) / A", "dtv"),
    "zoh_sign": ("expm1(dtv * A) / A", "expm1(-dtv * A) / -A"),
}


def _build_mutant(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    old, new = MUTANTS[name]
    assert old in src, name
    d = tempfile.mkdtemp()
    cpath = os.path.join(d, "m.c")
    lib = os.path.join(d, "m.so")
    open(cpath, "w").write(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", cpath, "-o", lib, "-lm"], check=True)
    return lib


def _pin_suite_passes(lib_path) -> bool:
    import ctypes
    lib = ctypes.CDLL(lib_path)
    f = lib.ssd_oracle_f64
    f.argtypes = oracle._load().ssd_oracle_f64.argtypes
    f.restype = ctypes.c_int
    saved = oracle._lib
    oracle._lib = type("L", (), {"ssd_oracle_f64": f, "ssd_oracle_max_threads": saved.ssd_oracle_max_threads})()
    try:
        checks = [test_w1_three_steps, test_w1_split_state_handoff, test_w3_one_dimensional_example,
                  test_packed_rows_equal_separate_runs, test_group_mapping_contiguous_heads,
                  test_linear_in_skip_and_initial_state, test_euler_flag_equals_prescaled_input,
                  test_softplus_step_size_reproduces_w1, test_softplus_at_zero_is_ln2, test_softplus_tails,
                  test_zoh_scales_w1_by_the_hold_factor, test_zoh_steps_compose,
                  test_zoh_tends_to_euler_as_A_vanishes]
        for c in checks:
            c()
        for idx in range(len(CASES)):
            test_recurrence_matches_dual_form(idx, False)
            test_recurrence_matches_dual_form(idx, True)
        return True
    except AssertionError:
        return False
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    assert not _pin_suite_passes(_build_mutant(name)), "mutant %s survived the pins" % name


def test_zero_tokens_leave_the_initial_state():
    """No token means no step of the recurrence: the final state is the initial one."""
    p = _case_problem(dict(b=2, T=0, H=2, P=3, N=4, G=1, init_std=1.0), seed=15)
    y, f = run(p)
    assert y.size == 0
    np.testing.assert_array_equal(f, p["init"].double().numpy())
    _, f0 = run(dict(p, init=None))
    assert not f0.any()
