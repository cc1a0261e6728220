"""CPU oracle for the Mamba-2 SSD forward (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it and shares no code with it.

* :func:`recurrence` — the plain fp64 step-by-step recurrence (C, OpenMP over
  (row, head) units).  This is the definition the GPU path must match.
* :func:`gradients` — reverse-mode differentiation of that recurrence, step by
  step (C): the gradients of <dy, y> + <dfinal, final> with respect to every input.
* :mod:`oracle.brute` — the dual (masked-attention) matrix form and the
  unrolled closed form in numpy, written independently, for tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_ssd.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    f = lib.ssd_oracle_f64
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    ci = ctypes.c_int
    f.argtypes = [i64, i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci,
                  vp, vp, ci]
    f.restype = ctypes.c_int
    b = lib.ssd_oracle_bwd_f64
    b.argtypes = [i64, i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, vp, vp,
                  vp, vp, vp, vp, vp, vp, vp, vp, vp, ci]
    b.restype = ctypes.c_int
    lib.ssd_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):          # torch tensor: exact upcast (bf16/f32 -> f64)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def recurrence(x, dt, A_log, B, C, D=None, init=None, seq_idx=None, nseqs: Optional[int] = None,
               dt_scales_x: bool = False, nthreads: int = 0, dt_bias=None, dt_softplus: bool = False,
               zoh: bool = False):
    """Run the fp64 recurrence.  Arrays may be numpy or torch (any float dtype).

    Shapes: x (b,T,H,P), dt (b,T,H), A_log (H), B/C (b,T,G,N), D (H), init (nseqs,H,P,N),
    seq_idx (b,T) int32, dt_bias (H).  The step size is dt + dt_bias, passed through
    softplus when ``dt_softplus``; x is written to the state unscaled, times the step
    size (``dt_scales_x``, Euler) or times (exp(step A) - 1) / A (``zoh``, exact
    zero-order hold).  Returns (y (b,T,H,P), final (nseqs,H,P,N)) as float64.
    """
    if dt_scales_x and zoh:
        raise ValueError("Euler and zero-order-hold input scaling are exclusive")
    lib = _load()
    x, dt, A_log, B, C = (_f64(v) for v in (x, dt, A_log, B, C))
    D = _f64(D)
    init = _f64(init)
    dt_bias = _f64(dt_bias)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        seq_idx = np.ascontiguousarray(seq_idx, dtype=np.int32)
        if nseqs is None:
            nseqs = int(seq_idx.max()) + 1 if seq_idx.size else 0
    else:
        nseqs = b
    assert dt.shape == (b, T, H) and A_log.shape == (H,)
    assert dt_bias is None or dt_bias.shape == (H,)
    assert B.shape == (b, T, G, N) and C.shape == (b, T, G, N)
    y = np.empty((b, T, H, P), dtype=np.float64)
    final = np.zeros((nseqs, H, P, N), dtype=np.float64)

    def p(a):
        return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None

    rc = lib.ssd_oracle_f64(b, T, H, P, N, G, nseqs, p(x), p(dt), p(A_log), p(B), p(C), p(D), p(init),
                            p(seq_idx), p(dt_bias), int(bool(dt_softplus)), 2 if zoh else int(bool(dt_scales_x)),
                            p(y), p(final), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    return y, final


def gradients(x, dt, A_log, B, C, dy, D=None, init=None, dfinal=None, seq_idx=None, nseqs: Optional[int] = None,
              dt_scales_x: bool = False, dt_bias=None, dt_softplus: bool = False, zoh: bool = False,
              nthreads: int = 0):
    """Gradients of L = <dy, y> + <dfinal, final_state> for the forward map of
    :func:`recurrence` (same arguments), by the adjoint recurrence in fp64.

    Returns a dict of float64 arrays: dx (b,T,H,P), ddt (b,T,H) (with respect to
    the dt input), dA_log (H), dB and dC (b,T,G,N), dD (H), dinit (nseqs,H,P,N),
    ddt_bias (H), and under "abs_terms" the per-head sums of the absolute
    per-token terms of dA_log, ddt_bias and dD.  dD, dinit and ddt_bias are returned whether or not D, init and
    dt_bias were given (the gradient at zero / no bias).
    """
    if dt_scales_x and zoh:
        raise ValueError("Euler and zero-order-hold input scaling are exclusive")
    lib = _load()
    x, dt, A_log, B, C, dy = (_f64(v) for v in (x, dt, A_log, B, C, dy))
    D, init, dfinal, dt_bias = (_f64(v) for v in (D, init, dfinal, dt_bias))
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if seq_idx is not None:
        if hasattr(seq_idx, "detach"):
            seq_idx = seq_idx.detach().cpu().numpy()
        seq_idx = np.ascontiguousarray(seq_idx, dtype=np.int32)
        if nseqs is None:
            nseqs = int(seq_idx.max()) + 1 if seq_idx.size else 0
    else:
        nseqs = b
    assert dy.shape == (b, T, H, P)
    assert dfinal is None or dfinal.shape == (nseqs, H, P, N)
    out = {"dx": np.empty((b, T, H, P)), "ddt": np.empty((b, T, H)), "dA_log": np.empty(H),
           "dB": np.empty((b, T, G, N)), "dC": np.empty((b, T, G, N)), "dD": np.empty(H),
           "dinit": np.empty((nseqs, H, P, N)), "ddt_bias": np.empty(H)}
    abs_sums = np.empty((H, 3))

    def p(a):
        return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None

    rc = lib.ssd_oracle_bwd_f64(b, T, H, P, N, G, nseqs, p(x), p(dt), p(A_log), p(B), p(C), p(D), p(init),
                                p(seq_idx), p(dt_bias), int(bool(dt_softplus)), 2 if zoh else int(bool(dt_scales_x)),
                                p(dy), p(dfinal), p(out["dx"]), p(out["ddt"]), p(out["dA_log"]), p(out["dB"]),
                                p(out["dC"]), p(out["dD"]), p(out["dinit"]), p(out["ddt_bias"]), p(abs_sums),
                                int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)
    # per head: sums over rows and tokens of the absolute per-token terms of each reduced gradient
    out["abs_terms"] = {"dA_log": abs_sums[:, 0].copy(), "ddt_bias": abs_sums[:, 1].copy(), "dD": abs_sums[:, 2].copy()}
    return out
