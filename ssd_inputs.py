"""Seeded synthetic inputs for the SSD chunked-scan forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the HIP path (through the Python binding) and the
CPU oracle consume what it returns, so the two sides always see bit-identical
inputs.

Distributions follow the workload descriptions this project is measured on
(one Mamba-2 layer at several model sizes):

* ``A_log ~ U(0, ln 16)`` so that ``A_h = -exp(A_log_h)`` lies in [-16, -1];
* ``dt = softplus(u)`` with ``u ~ U(lo, hi)`` per (row, token, head);
* ``x ~ N(0, 1)``; ``B, C ~ N(0, 1) / sqrt(N)``;
* ``D_h ~ N(1, 0.1)`` where the workload has a skip term, else zero;
* packed batches: sequence lengths ``64 + Multinomial(T - 64*nseq, p)`` with
  ``p ~ Dirichlet(1)``, initial states ``~ N(0, 0.5)``.

Draw order per problem is fixed: A_log, u, x, B, C, D, then (packed only) the
length split and the initial states.  Values are drawn in float64, softplus is
taken in float64, every array is then stored as float32, and x, B, C are cast
to bfloat16 with round-to-nearest-even where the workload is bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    dtype: str                      # "bf16" or "f32": dtype of x, B, C
    dt_range: tuple                 # (lo, hi) of u, dt = softplus(u)
    d_skip: bool                    # D_h ~ N(1, 0.1) if True, else D = 0
    nseqs_packed: int = 0           # > 0: one row packed with this many sequences
    init_std: float = 0.0           # > 0: per-sequence initial states ~ N(0, init_std)
    min_len: int = 64               # minimum packed-sequence length
    seed: int = 0


# The five measured workloads.  Index 0 is the small fp32 case the oracle
# finishes in well under a second; index 2 is the headline layer shape.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 256, 2, 16, 16, 1, 32, "f32", (-4.0, -1.0), False, seed=1),
    "m130_bf16": Workload("m130_bf16", 8, 2048, 24, 64, 128, 1, 256, "bf16", (-5.0, -2.0), True, seed=2),
    "m2p7_bf16": Workload("m2p7_bf16", 4, 4096, 80, 64, 128, 1, 256, "bf16", (-4.0, -1.0), False, seed=3),
    "long_n64": Workload("long_n64", 1, 16384, 32, 64, 64, 1, 256, "bf16", (-6.0, -3.0), False, seed=4),
    "long_n128": Workload("long_n128", 1, 16384, 32, 64, 128, 1, 256, "bf16", (-6.0, -3.0), False, seed=4),
    "long_n256": Workload("long_n256", 1, 16384, 32, 64, 256, 1, 256, "bf16", (-6.0, -3.0), False, seed=4),
    "packed_bf16": Workload("packed_bf16", 1, 8192, 48, 64, 128, 8, 256, "bf16", (-4.0, -1.0), False,
                            nseqs_packed=16, init_std=0.5, seed=5),
}


def _softplus64(u: np.ndarray) -> np.ndarray:
    # log(1 + e^u) evaluated stably in float64 (input transform of the workload)
    return np.logaddexp(0.0, u)


def packed_lengths(rng: np.random.Generator, total: int, nseq: int, min_len: int) -> np.ndarray:
    """Dirichlet-multinomial split of ``total`` tokens into ``nseq`` lengths >= min_len."""
    spare = total - nseq * min_len
    if spare < 0:
        raise ValueError("total too small for nseq * min_len")
    p = rng.dirichlet(np.ones(nseq))
    extra = rng.multinomial(spare, p)
    return (min_len + extra).astype(np.int64)


def seq_idx_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Per-token sequence id (int32) for one packed row."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths, dtype=np.int64))


def make_problem(batch: int, seqlen: int, nheads: int, headdim: int, dstate: int, ngroups: int = 1,
                 *, dtype: str = "bf16", seed: int = 0, dt_range=(-4.0, -1.0), d_skip: bool = False,
                 seqlens: Optional[Sequence[Sequence[int]]] = None, init_std: float = 0.0,
                 packed_nseqs: int = 0, min_len: int = 64) -> dict:
    """Draw one seeded problem.

    Returns a dict of CPU torch tensors: x (b,T,H,P), dt (b,T,H) f32, A_log (H) f32,
    B, C (b,T,G,N), D (H) f32 or None, init (nseqs,H,P,N) f32 or None,
    seq_idx (b,T) int32 or None, nseqs (int).

    ``seqlens``: explicit per-row lists of sequence lengths (each row must sum
    to seqlen); ids are numbered consecutively across rows.
    ``packed_nseqs``: draw a Dirichlet-multinomial split of each row instead.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    b, T, H, P, N, G = batch, seqlen, nheads, headdim, dstate, ngroups
    A_log = rng.uniform(0.0, math.log(16.0), size=(H,))
    u = rng.uniform(dt_range[0], dt_range[1], size=(b, T, H))
    dt = _softplus64(u)
    x = rng.standard_normal(size=(b, T, H, P))
    Bm = rng.standard_normal(size=(b, T, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal(size=(b, T, G, N)) / math.sqrt(N)
    D = rng.normal(1.0, 0.1, size=(H,)) if d_skip else None

    seq_idx = None
    nseqs = b
    if packed_nseqs and seqlens is None:
        seqlens = [packed_lengths(rng, T, packed_nseqs, min_len) for _ in range(b)]
    if seqlens is not None:
        rows = []
        base = 0
        for r in range(b):
            lens = np.asarray(seqlens[r], dtype=np.int64)
            if lens.sum() != T or (lens <= 0).any():
                raise ValueError("row %d: lengths must be positive and sum to seqlen" % r)
            rows.append(seq_idx_from_lengths(lens) + base)
            base += len(lens)
        seq_idx = np.stack(rows).astype(np.int32)
        nseqs = base
    init = rng.normal(0.0, init_std, size=(nseqs, H, P, N)) if init_std > 0 else None

    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))

    return {
        "x": f32(x).to(tdt),
        "dt": f32(dt),
        "A_log": f32(A_log),
        "B": f32(Bm).to(tdt),
        "C": f32(Cm).to(tdt),
        "D": f32(D) if D is not None else None,
        "init": f32(init) if init is not None else None,
        "seq_idx": torch.from_numpy(seq_idx) if seq_idx is not None else None,
        "nseqs": nseqs,
    }


def raw_step_sizes(batch: int, seqlen: int, nheads: int, *, seed: int = 0, lo: float = -4.0,
                   hi: float = 1.0, bias_range=(-0.5, 0.5)) -> dict:
    """Pre-activation step sizes for the fused step-size map: dt_raw (b,T,H) f32 and a
    per-head bias (H) f32, with dt_raw + bias ~ U(lo, hi) and bias ~ U(bias_range).
    Both sides take these values as given."""
    rng = np.random.default_rng(seed)
    bias = rng.uniform(bias_range[0], bias_range[1], size=(nheads,))
    u = rng.uniform(lo, hi, size=(batch, seqlen, nheads))
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return {"dt": f32(u - bias[None, None, :]), "dt_bias": f32(bias)}


def make_workload(w: Workload) -> dict:
    """Inputs of one named workload (seeded by the workload's own seed)."""
    return make_problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
                        dtype=w.dtype, seed=w.seed, dt_range=w.dt_range, d_skip=w.d_skip,
                        init_std=w.init_std, packed_nseqs=w.nseqs_packed, min_len=w.min_len)
