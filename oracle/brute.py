"""Dense dual form of the SSD map, in numpy float64 (test infrastructure only).

This is a second, independent formulation used to pin the recurrence oracle:
instead of stepping a state it builds, per (row, head), the full T x T matrix

    M[t, s] = L[t, s] * (C_t . B_s),   L[t, s] = prod_{j=s+1..t} a_j  (s <= t), else 0

and returns Y = M X (+ the initial-state and skip terms).  Sources:

* the unrolled closed form y_t = sum_{s<=t} (prod_{j=s+1..t} a_j)(C_t^T B_s) x_s
  with the empty product equal to 1: "088 Mamba-2" (wq-win.github.io), section
  2.1 "unrolling the history contribution";
* the dual masked-attention form Y = [L o (C B^T)] X with L lower triangular:
  same page, section 2.2;
* the cut factorisation M[t,s] = (prod_{m+1..t} a) C_t^T (prod_{s+1..m} a) B_s
  for s <= m < t, so every past-to-future block has rank <= N: same page, the
  boxed derivation in section 2.2.

For packed rows, L[t, s] is zero whenever t and s belong to different
sequences; a sequence that starts at st with initial state S0 adds
(prod_{j=st..t} a_j) S0 C_t to y_t (the state replaced at the boundary, then
decayed by each of the sequence's own steps).  Intended for T up to a few
hundred: it is O(T^2) per head.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _np64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def decay_products(a: np.ndarray) -> np.ndarray:
    """L[t, s] = prod_{j=s+1..t} a_j for s <= t, 0 above the diagonal (empty product = 1)."""
    T = a.shape[0]
    L = np.zeros((T, T), dtype=np.float64)
    for s in range(T):
        L[s, s] = 1.0
        if s + 1 < T:
            L[s + 1:, s] = np.cumprod(a[s + 1:])
    return L


def semiseparable_matrix(a: np.ndarray, B: np.ndarray, C: np.ndarray) -> np.ndarray:
    """M = L o (C B^T) for one head: a (T,), B and C (T, N)."""
    return decay_products(np.asarray(a, np.float64)) * (np.asarray(C, np.float64) @ np.asarray(B, np.float64).T)


def dual_form(x, dt, A_log, B, C, D=None, init=None, seq_idx=None, nseqs: Optional[int] = None,
              dt_scales_x: bool = False):
    """Same contract as ``oracle.recurrence`` but evaluated as dense matrices."""
    x, dt, A_log, B, C = (_np64(v) for v in (x, dt, A_log, B, C))
    D = _np64(D)
    init = _np64(init)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    if seq_idx is not None:
        seq = np.asarray(seq_idx.cpu().numpy() if hasattr(seq_idx, "cpu") else seq_idx, dtype=np.int64)
        if nseqs is None:
            nseqs = int(seq.max()) + 1
    else:
        seq = np.repeat(np.arange(b, dtype=np.int64)[:, None], T, axis=1)
        nseqs = b
    y = np.zeros((b, T, H, P))
    final = np.zeros((nseqs, H, P, N))
    for r in range(b):
        sr = seq[r]
        same = sr[:, None] == sr[None, :]
        starts = {}
        ends = {}
        for t in range(T):
            starts.setdefault(int(sr[t]), t)
            ends[int(sr[t])] = t
        for h in range(H):
            g = h // hpg
            A = -np.exp(A_log[h])
            a = np.exp(dt[r, :, h] * A)
            Bg, Cg = B[r, :, g, :], C[r, :, g, :]
            xs = x[r, :, h, :] * (dt[r, :, h][:, None] if dt_scales_x else 1.0)
            M = semiseparable_matrix(a, Bg, Cg) * same
            Y = M @ xs
            if init is not None:
                for k, st in starts.items():
                    rows = np.nonzero(sr == k)[0]
                    dec = np.cumprod(a[st:ends[k] + 1])        # prod_{j=st..t} a_j
                    Y[rows] += dec[:, None] * (Cg[rows] @ init[k, h].T)
            if D is not None:
                Y = Y + D[h] * x[r, :, h, :]
            y[r, :, h, :] = Y
            for k, e in ends.items():
                st = starts[k]
                F = np.zeros((P, N))
                if init is not None:
                    F += np.prod(a[st:e + 1]) * init[k, h]
                for s in range(st, e + 1):
                    F += np.prod(a[s + 1:e + 1]) * np.outer(xs[s], Bg[s])
                final[k, h] = F
    return y, final
