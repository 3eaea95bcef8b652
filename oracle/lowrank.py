"""Oracle: the decomposed linear layer (test infrastructure only).

A dense weight W[d_in, d_out] is replaced by two smaller matrices whose
product approximates it (W ~ A B; DeInfer/en §1 "Problem Statement", and
DeInfer/es "Resumen Técnico" §1).  Inference applies the downward projection
first, into the rank-r latent space, then the upward projection back to
d_out (DeInfer/en §2.A; DeInfer/es §2, "proyecciones hacia abajo / arriba").

Notation of this repository: U_r[d_in, r] is the downward factor, V_r[r, d_out]
the upward factor, t = x U_r the rank-r intermediate, y = t V_r the output.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def rank_for_ratio(rho, d_in: int, d_out: int) -> int:
    """Largest r whose two factors hold at most the fraction rho of the dense
    parameters: r (d_in + d_out) <= rho d_in d_out, i.e.
    r = floor(rho d_in d_out / (d_in + d_out)).  rho is taken as the decimal
    it is written as (exact rational arithmetic)."""
    f = Fraction(str(rho)) if not isinstance(rho, Fraction) else rho
    return int((f * d_in * d_out) // (d_in + d_out))


def truncated_factors(W: np.ndarray, r: int):
    """Rank-r factors of W from its singular value decomposition
    W = P diag(s) Q^T (s descending): U_r = P[:, :r] diag(sqrt s_r),
    V_r = diag(sqrt s_r) Q^T[:r, :].  Their product is the best rank-r
    approximation of W (Eckart-Young); splitting sqrt(s) evenly keeps both
    factors on the same scale.  Returns fp64 (U_r, V_r, s)."""
    W = np.asarray(W, dtype=np.float64)
    P, s, Qt = np.linalg.svd(W, full_matrices=False)
    root = np.sqrt(s[:r])
    U_r = P[:, :r] * root[None, :]
    V_r = root[:, None] * Qt[:r, :]
    return U_r, V_r, s


def linear(x: np.ndarray, U_r: np.ndarray, V_r: np.ndarray):
    """Decomposed linear: down projection t = x U_r, then up projection
    y = t V_r, both in fp64 (DeInfer/en §2.A).  Returns (t, y)."""
    x = np.asarray(x, dtype=np.float64)
    t = x @ np.asarray(U_r, dtype=np.float64)
    y = t @ np.asarray(V_r, dtype=np.float64)
    return t, y


def linear_loops(x, U_r, V_r):
    """The same two contractions as explicit Python loops, for tiny shapes."""
    T, d_in = len(x), len(x[0])
    r, d_out = len(U_r[0]), len(V_r[0])
    t = [[0.0] * r for _ in range(T)]
    for i in range(T):
        for j in range(r):
            acc = 0.0
            for k in range(d_in):
                acc += float(x[i][k]) * float(U_r[k][j])
            t[i][j] = acc
    y = [[0.0] * d_out for _ in range(T)]
    for i in range(T):
        for n in range(d_out):
            acc = 0.0
            for j in range(r):
                acc += t[i][j] * float(V_r[j][n])
            y[i][n] = acc
    return np.array(t), np.array(y)


def _shard(n: int, s: int, P: int):
    if n % P:
        raise ValueError("dimension %d not divisible by %d shares" % (n, P))
    w = n // P
    return slice(s * w, (s + 1) * w)


def tp_share_stage1(x, U_r, s: int, P: int):
    """One tensor-parallel share's downward projection with U_r split by input
    rows: t_s = x[:, R_s] U_r[R_s, :], the partial rank-r intermediate that
    the shares would exchange in rank space (DeInfer/en §2.A: communication
    moved into the low-rank latent space).  Sum over s of t_s equals x U_r."""
    R = _shard(np.shape(U_r)[0], s, P)
    return np.asarray(x, np.float64)[:, R] @ np.asarray(U_r, np.float64)[R, :]


def tp_share_stage2(t, V_r, s: int, P: int):
    """One share's upward projection on its output-column shard, 'shard mode'
    (DeInfer/en §2.A): y_s = t V_r[:, C_s]."""
    C = _shard(np.shape(V_r)[1], s, P)
    return np.asarray(t, np.float64) @ np.asarray(V_r, np.float64)[:, C]
