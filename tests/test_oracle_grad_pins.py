"""Pins of the oracle's gradients (the adjoint recurrence) against what does
not depend on them: central finite differences of the forward oracle (itself
pinned in test_oracle_pins.py), gradients of the three-step worked example
derived by hand from its closed form, and special cases.  Planted mistakes in
copies of the oracle source are each rejected by these checks.
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

INPUTS = ("x", "dt", "A_log", "B", "C", "D", "init", "dt_bias")


def problem(b, T, H, P, N, G, seed, packed=False, softplus=False):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((b, T, H, P)),
        "dt": rng.uniform(-1.0, 0.5, (b, T, H)) if softplus else rng.uniform(0.05, 0.6, (b, T, H)),
        "A_log": rng.uniform(-0.5, 1.0, H),
        "B": rng.standard_normal((b, T, G, N)) / math.sqrt(N),
        "C": rng.standard_normal((b, T, G, N)) / math.sqrt(N),
        "D": rng.normal(1.0, 0.2, H),
        "dt_bias": rng.uniform(-0.3, 0.3, H) if softplus else rng.uniform(0.0, 0.1, H),
        "seq_idx": None, "nseqs": b,
    }
    if packed:
        # row 0: sequences of lengths 2, 1, T-3; row 1: one sequence
        ids = [[0, 0, 1] + [2] * (T - 3), [3] * T] if b == 2 else None
        p["seq_idx"] = np.array(ids, dtype=np.int32)
        p["nseqs"] = 4
    p["init"] = rng.standard_normal((p["nseqs"], H, P, N)) * 0.5
    p["dy"] = rng.standard_normal((b, T, H, P))
    p["dfinal"] = rng.standard_normal((p["nseqs"], H, P, N))
    return p


def loss(p, **flags):
    y, f = oracle.recurrence(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["D"], p["init"], p["seq_idx"],
                             p["nseqs"] if p["seq_idx"] is not None else None, dt_bias=p["dt_bias"], **flags)
    seen = np.zeros(f.shape[0], dtype=bool)      # final rows of sequences that occur
    if p["seq_idx"] is not None:
        seen[np.unique(p["seq_idx"])] = True
    else:
        seen[:] = True
    return float((p["dy"] * y).sum() + (p["dfinal"][seen] * f[seen]).sum())


def grads(p, **flags):
    return oracle.gradients(p["x"], p["dt"], p["A_log"], p["B"], p["C"], p["dy"], p["D"], p["init"], p["dfinal"],
                            p["seq_idx"], p["nseqs"] if p["seq_idx"] is not None else None, dt_bias=p["dt_bias"],
                            **flags)


def finite_difference(p, name, eps=1e-6, **flags):
    base = p[name]
    out = np.empty_like(base)
    for i in np.ndindex(base.shape):
        old = base[i]
        base[i] = old + eps
        lp = loss(p, **flags)
        base[i] = old - eps
        lm = loss(p, **flags)
        base[i] = old
        out[i] = (lp - lm) / (2 * eps)
    return out


FLAGS = {
    "plain": {},
    "euler": {"dt_scales_x": True},
    "zoh": {"zoh": True},
    "softplus": {"dt_softplus": True},
    "softplus_zoh": {"dt_softplus": True, "zoh": True},
}


@pytest.mark.parametrize("mode", sorted(FLAGS))
@pytest.mark.parametrize("G", [1, 2])
def test_gradients_match_finite_differences(mode, G):
    flags = FLAGS[mode]
    p = problem(2, 6, 2, 3, 2, G, seed=7 + G, softplus=flags.get("dt_softplus", False))
    g = grads(p, **flags)
    for name in INPUTS:
        fd = finite_difference(p, name, **flags)
        key = "d" + name
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(g[key], fd, rtol=0, atol=2e-7 * scale, err_msg="%s (%s)" % (key, mode))


@pytest.mark.parametrize("mode", ["plain", "softplus_zoh"])
def test_gradients_with_packed_sequences(mode):
    flags = FLAGS[mode]
    p = problem(2, 7, 2, 3, 2, 1, seed=19, packed=True, softplus=flags.get("dt_softplus", False))
    g = grads(p, **flags)
    for name in INPUTS:
        fd = finite_difference(p, name, **flags)
        scale = max(1.0, float(np.abs(fd).max()))
        np.testing.assert_allclose(g["d" + name], fd, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_w1_gradients_by_hand():
    """The three-step example (a = 1/2, x = 2, 4, 6, B = C = 1) with L = y1 + y2 + y3.
    From y = M x with M = [[1,0,0],[a,1,0],[a^2,a,1]]: dL/dx = (1 + a + a^2, 1 + a, 1)
    = (1.75, 1.5, 1); dL/dC_t = h_t = (2, 5, 8.5); dL/dB_t = x_t dL/dx_t = (3.5, 6, 6);
    dL/dD = sum x = 12.  With one decay a shared by the steps, sum y = 2(1 + a + a^2)
    + 4(1 + a) + 6, so dL/da = 2(1 + 2a) + 4 = 8, split over the steps as
    G_t h_{t-1} = (0, 3, 5); a = exp(dt A) with dt = 1, A = -ln 2 gives
    da/ddt = a A and da/dA_log = a A, so ddt = (0, -1.5 ln 2, -2.5 ln 2) and
    dA_log = -4 ln 2; and dL/dinit = a + a^2 + a^3 = 0.875."""
    x = np.array([2.0, 4.0, 6.0]).reshape(1, 3, 1, 1)
    ones = np.ones((1, 3, 1, 1))
    g = oracle.gradients(x, np.ones((1, 3, 1)), np.array([math.log(math.log(2.0))]), ones, ones, ones,
                         D=np.zeros(1), init=np.zeros((1, 1, 1, 1)))
    ln2 = math.log(2.0)
    np.testing.assert_allclose(g["dx"].ravel(), [1.75, 1.5, 1.0], atol=1e-14)
    np.testing.assert_allclose(g["dC"].ravel(), [2.0, 5.0, 8.5], atol=1e-14)
    np.testing.assert_allclose(g["dB"].ravel(), [3.5, 6.0, 6.0], atol=1e-14)
    np.testing.assert_allclose(g["dD"], [12.0], atol=1e-14)
    np.testing.assert_allclose(g["ddt"].ravel(), [0.0, -1.5 * ln2, -2.5 * ln2], atol=1e-14)
    np.testing.assert_allclose(g["dA_log"], [-4.0 * ln2], atol=1e-14)
    np.testing.assert_allclose(g["dinit"].ravel(), [0.875], atol=1e-14)


def test_zero_tokens_pass_dfinal_to_dinit():
    p = problem(2, 0, 2, 3, 2, 1, seed=3)
    g = grads(p)
    np.testing.assert_array_equal(g["dinit"], p["dfinal"])
    assert g["dx"].size == 0 and not g["dA_log"].any()


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "adjoint_decay_of_own_step": ("Gs[i] *= av[t + 1];", "Gs[i] *= av[t];"),
    "dB_without_input_factor": ("dBt[n] = fv[t] * sb;", "dBt[n] = sb;"),
    "dinit_without_decay": ("di[i] = a * Gs[i];", "di[i] = Gs[i];"),
    "softplus_derivative": ("g_dt *= 1.0 / (1.0 + exp(-pre[t]));", "g_dt *= 1.0 / (1.0 + exp(pre[t]));"),
    "zoh_dA_term": ("dfdA = (Dv * A * a - a + 1.0) / (A * A);", "dfdA = 0.0;"),
    "dfinal_decayed": ("dfinal[(k * H + h) * (int64_t)PN + (int64_t)i] : 0.0;",
                       "av[t] * dfinal[(k * H + h) * (int64_t)PN + (int64_t)i] : 0.0;"),
}


def _mutant_gradients(name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    old, new = MUTANTS[name]
    assert old in src, name
    d = tempfile.mkdtemp()
    cpath, lib = os.path.join(d, "m.c"), os.path.join(d, "m.so")
    open(cpath, "w").write(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-std=c11", cpath, "-o", lib, "-lm"], check=True)
    import ctypes
    m = ctypes.CDLL(lib)
    f = m.ssd_oracle_bwd_f64
    f.argtypes = oracle._load().ssd_oracle_bwd_f64.argtypes
    f.restype = ctypes.c_int
    return f


def _pins_pass_with(fn) -> bool:
    saved = oracle._lib
    oracle._lib = type("L", (), {"ssd_oracle_bwd_f64": fn, "ssd_oracle_f64": saved.ssd_oracle_f64,
                                 "ssd_oracle_max_threads": saved.ssd_oracle_max_threads})()
    try:
        test_w1_gradients_by_hand()
        for mode in ("plain", "zoh", "softplus_zoh"):
            test_gradients_match_finite_differences(mode, 2)
        test_gradients_with_packed_sequences("plain")
        return True
    except AssertionError:
        return False
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_gradient_mistakes_are_caught(name):
    assert not _pins_pass_with(_mutant_gradients(name)), "mutant %s survived" % name
