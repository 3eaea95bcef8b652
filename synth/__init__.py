"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and lays them out; it computes none of the
low-rank method's arithmetic (no projection, gather, remap, norm, rotary or
attention).  Both the fp64 oracle and the HIP path receive exactly the arrays
produced here, so quantisation of inputs is never counted as error.

Citation key used across this repository: "DeInfer/en" is the English
technical summary page of *DeInfer: Efficient Parallel Inferencing for
Decomposed Large Language Models* (gist.science); "DeInfer/es" the Spanish
page ("Resumen Técnico"); "DeInfer/zh" the Chinese page.

Seed convention: ``seed = 1_000_000*cfg + 1_000*layer + 10*role + kind`` with
roles q,k,v,o,gate,up,down = 0..6 and kinds W=0, x/h=1, norm=2, lengths=3,
placement=4, latents=5.
"""
from __future__ import annotations

import numpy as np

ROLES = ("q", "k", "v", "o", "gate", "up", "down")
KIND_W, KIND_X, KIND_NORM, KIND_LEN, KIND_PLACE, KIND_LAT = 0, 1, 2, 3, 4, 5


def seed_of(cfg: int, layer: int = 0, role: int = 0, kind: int = 0) -> int:
    return 1_000_000 * cfg + 1_000 * layer + 10 * role + kind


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- bf16 bits
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (fp64 -> fp32 by numpy's RNE cast, then fp32 -> bf16
    round-to-nearest-even on the bit pattern).  Returns uint16 bit patterns."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    out = u.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def quantize(a: np.ndarray, dtype: str):
    """Return (storage array, exact fp64 values).  dtype 'bf16' -> uint16 bits,
    'f32' -> float32."""
    if dtype == "bf16":
        b = bf16_bits(a)
        return b, bf16_value(b)
    if dtype == "f32":
        f = np.ascontiguousarray(a, dtype=np.float32)
        return f, f.astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- tensors
def gaussian(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    return rng(seed).standard_normal(shape) * scale


def dense_weight(seed: int, d_in: int, d_out: int) -> np.ndarray:
    """W[d_in, d_out] with iid N(0, 1/d_in) entries (fp64)."""
    return gaussian(seed, (d_in, d_out), 1.0 / np.sqrt(d_in))


def tokens(seed: int, T: int, d: int) -> np.ndarray:
    """Activations x[T, d] ~ N(0, 1) (fp64)."""
    return gaussian(seed, (T, d))


def ternary(seed: int, shape) -> np.ndarray:
    """Entries uniform in {-1, 0, 1} (fp64): integer cases whose products and
    short sums are exact in bf16 and fp32."""
    return rng(seed).integers(-1, 2, size=shape).astype(np.float64)


# ------------------------------------------------------- factor synthesis
def svd_factors(W: np.ndarray, r: int):
    """Factors of a seeded dense weight by LAPACK SVD, truncated to rank r,
    with sqrt(sigma) folded into both sides: returns (U_r[d_in,r], V_r[r,d_out]).
    This is the decomposition that precedes inference (W ~ A B,
    DeInfer/en §1); the oracle owns an independent statement of it."""
    U, s, Vt = np.linalg.svd(W, full_matrices=False)
    rs = np.sqrt(s[:r])
    return U[:, :r] * rs[None, :], rs[:, None] * Vt[:r, :]


def _haar_columns(g: np.random.Generator, d: int, r: int) -> np.ndarray:
    """First r columns of a Haar-distributed orthogonal d x d matrix: QR of a
    Gaussian d x r matrix with the signs of R's diagonal made positive
    (Mezzadri, 'How to generate random matrices from the classical compact
    groups', 2007)."""
    Q, R = np.linalg.qr(g.standard_normal((d, r)))
    return Q * np.sign(np.diag(R))[None, :]


def _gaussian_singular_values(g: np.random.Generator, m: int, n: int) -> np.ndarray:
    """Singular values, descending, distributed as those of an m x n matrix of
    iid N(0,1) entries, drawn from the bidiagonal model of Dumitriu and
    Edelman ('Matrix models for beta ensembles', 2002; beta = 1): with
    p = min(m, n), q = max(m, n), B is p x p upper bidiagonal with diagonal
    chi_{q}, chi_{q-1}, ..., chi_{q-p+1} and super-diagonal chi_{p-1}, ..., chi_1.
    The squared singular values of B are the eigenvalues of the symmetric
    tridiagonal B^T B."""
    from scipy.linalg import eigvalsh_tridiagonal

    p, q = min(m, n), max(m, n)
    a = np.sqrt(g.chisquare(np.arange(q, q - p, -1)))
    b = np.sqrt(g.chisquare(np.arange(p - 1, 0, -1)))
    diag = a * a
    diag[1:] += b * b
    off = a[:-1] * b
    ev = eigvalsh_tridiagonal(diag, off)
    return np.sqrt(np.clip(ev, 0.0, None))[::-1]


def fast_factors(seed: int, d_in: int, d_out: int, r: int):
    """Rank-r factors with the same joint law as ``svd_factors`` applied to
    ``dense_weight(seed', d_in, d_out)``: for a Gaussian matrix the left and
    right singular vectors are Haar-distributed and independent of the
    singular values, so U_r = H1 diag(sqrt s), V_r = diag(sqrt s) H2^T with
    H1, H2 Haar column sets and s the r largest singular values of an
    N(0, 1/d_in) matrix.  O(d r^2) instead of the O(d^3) SVD; used for the
    7B/13B-shaped workloads."""
    if not 0 < r <= min(d_in, d_out):
        raise ValueError("rank %d outside 1..min(d_in, d_out)" % r)
    g = rng(seed)
    s = _gaussian_singular_values(g, d_in, d_out)[:r] / np.sqrt(d_in)
    rs = np.sqrt(s)
    H1 = _haar_columns(g, d_in, r)
    H2 = _haar_columns(g, d_out, r)
    return H1 * rs[None, :], rs[:, None] * H2.T


# --------------------------------------------- paged latent cache inputs
def decode_lengths(seed: int, B: int, lo: int = 128, hi: int = 4096) -> np.ndarray:
    """Cached length L_i ~ U{lo..hi} for each of B sequences (int64)."""
    return rng(seed).integers(lo, hi + 1, size=B)


def block_tables(seed: int, lengths: np.ndarray, block: int = 16,
                 max_extent: int = 8, slack_blocks: int = 0):
    """Seeded physical placement of a paged cache.

    Each sequence i needs ceil((L_i + 1) / block) blocks (its cached rows and
    the slot of the token being decoded).  The pool's block range is cut into
    extents of 1..max_extent consecutive blocks, the extents are shuffled, and
    the sequences take blocks in order from the concatenated shuffled extents.
    Returns (tables: list of int32 arrays, n_pool_blocks)."""
    g = rng(seed)
    need = [(int(L) + 1 + block - 1) // block for L in lengths]
    total = sum(need) + slack_blocks
    extents = []
    start = 0
    while start < total:
        n = int(g.integers(1, max_extent + 1))
        n = min(n, total - start)
        extents.append(np.arange(start, start + n, dtype=np.int32))
        start += n
    order = g.permutation(len(extents))
    flat = np.concatenate([extents[i] for i in order])
    tables, pos = [], 0
    for n in need:
        tables.append(flat[pos:pos + n].copy())
        pos += n
    return tables, total


# ------------------------------------- counter-based generator (numpy/torch)
# value(seed, i) for a flat element index i: two rounds of the MurmurHash3
# 32-bit finaliser give four 16-bit uniforms u_k; their centred, scaled sum
# (Irwin-Hall with n = 4) approximates N(0, 1).  Integer steps are identical
# in numpy (uint64) and torch (int64, low 32 bits kept after each product),
# the final scaling is one IEEE double division, so both twins agree bit for
# bit and a GPU can materialise gigabytes of inputs whose rows the CPU side
# regenerates one by one.
_M32 = 0xFFFFFFFF
_IH_MEAN = 4 * 65535 / 2.0
_IH_SD = float(np.sqrt(4 * (65536.0 ** 2 - 1) / 12.0))


def _fmix32_np(h):
    h = h & _M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def hash_normal(seed: int, index) -> np.ndarray:
    """Approximately N(0,1) values at flat indices (numpy, fp64)."""
    i = np.asarray(index, dtype=np.uint64)
    s = np.uint64(seed & _M32)
    a = _fmix32_np((i * np.uint64(2) * np.uint64(0x9E3779B1) + s) & np.uint64(_M32))
    b = _fmix32_np(((i * np.uint64(2) + np.uint64(1)) * np.uint64(0x9E3779B1) + s)
                   & np.uint64(_M32))
    tot = (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)
    return (tot.astype(np.float64) - _IH_MEAN) / _IH_SD


def hash_normal_torch(seed: int, index):
    """The same values as hash_normal for an int64 torch tensor of indices
    (any device); returns float64."""
    import torch

    m = 0xFFFFFFFF

    def fmix(h):
        h = h & m
        h = h ^ (h >> 16)
        h = (h * 0x85EBCA6B) & m
        h = h ^ (h >> 13)
        h = (h * 0xC2B2AE35) & m
        return h ^ (h >> 16)

    i = index.to(torch.int64)
    s = seed & m
    a = fmix((i * 2 * 0x9E3779B1 + s) & m)
    b = fmix(((i * 2 + 1) * 0x9E3779B1 + s) & m)
    tot = (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)
    return (tot.to(torch.float64) - _IH_MEAN) / _IH_SD


def hash_bf16_rows_torch(seed: int, rows: int, ld: int, device):
    """Device [rows, ld] bf16 tensor of hash_normal(seed, row * ld + col),
    rounded fp64 -> fp32 -> bf16 as bf16_bits does; built in row chunks."""
    import torch

    out = torch.empty((rows, ld), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 24) // ld)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        idx = torch.arange(r0 * ld, r1 * ld, dtype=torch.int64, device=device)
        out[r0:r1] = hash_normal_torch(seed, idx).to(torch.float32).to(torch.bfloat16).view(
            r1 - r0, ld)
    return out


def hash_rows(seed: int, rows, ld: int) -> np.ndarray:
    """fp64 values of the bf16-rounded hash_normal rows (numpy twin of
    hash_bf16_rows_torch) for the given physical row indices."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = rows[:, None] * ld + np.arange(ld)[None, :]
    return bf16_value(bf16_bits(hash_normal(seed, idx)))


def rank_permutation(seed: int, r: int):
    """Seeded permutation and signs of the rank components: (U_r P D, D P^T V_r)
    has the same product and the same law as (U_r, V_r)."""
    g = rng(seed)
    return g.permutation(r), g.choice(np.array([-1.0, 1.0]), r)


# -------------------------------------------- 32-layer decode-step workload
DECODE_STEP_7B = {"d_model": 4096, "n_heads": 32, "n_kv_heads": 32, "head_dim": 128,
                  "d_ffn": 11008, "eps": 1e-5, "rho": 0.2, "B": 64, "n_layers": 32,
                  "block": 16, "len_lo": 128, "len_hi": 4096}
