"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-8, 8, 20000),
                        [0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, 1e-40, np.inf, -np.inf]])
    a32 = a.astype(np.float32)
    ref = torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(a), ref)
    # exact round trip of representable values
    b = synth.bf16_bits(a)
    assert np.array_equal(synth.bf16_bits(synth.bf16_value(b)), b)


def test_svd_factors_match_oracle_truncation():
    W = synth.dense_weight(3, 48, 80)
    U1, V1 = synth.svd_factors(W, 17)
    U2, V2, _ = oracle.truncated_factors(W, 17)
    assert np.max(np.abs(U1 @ V1 - U2 @ V2)) <= 1e-12


@pytest.mark.parametrize("shape", [(64, 160), (160, 64), (96, 96)])
def test_fast_factors_structure(shape):
    d_in, d_out = shape
    r = 20
    U, V = synth.fast_factors(5, d_in, d_out, r)
    sig = np.diag(U.T @ U)
    assert np.allclose(U.T @ U, np.diag(sig), atol=1e-12)
    assert np.allclose(V @ V.T, np.diag(sig), atol=1e-12)
    assert np.all(np.diff(sig) <= 0)
    # the product has exactly these singular values
    s = np.linalg.svd(U @ V, compute_uv=False)[:r]
    assert np.allclose(s, sig, rtol=1e-10)


def test_fast_factor_spectrum_law():
    # bidiagonal model vs singular values of actual Gaussian matrices
    m, n, reps = 24, 40, 400
    g = np.random.default_rng(0)
    emp = np.mean([np.linalg.svd(g.standard_normal((m, n)), compute_uv=False)
                   for _ in range(reps)], axis=0)
    mod = np.mean([synth._gaussian_singular_values(np.random.default_rng(1000 + k), m, n)
                   for k in range(reps)], axis=0)
    assert np.max(np.abs(emp - mod) / emp) < 0.03
    # E sum sigma^2 = m n exactly; check the model's mean within sampling error
    tot = np.mean([np.sum(synth._gaussian_singular_values(np.random.default_rng(k), m, n) ** 2)
                   for k in range(reps)])
    assert abs(tot - m * n) < 4 * np.sqrt(2 * m * n / reps)


def test_block_tables_partition_pool():
    lengths = synth.decode_lengths(1, 20, 1, 200)
    tables, nb = synth.block_tables(2, lengths, block=16, slack_blocks=5)
    used = np.concatenate(tables)
    assert len(np.unique(used)) == len(used)
    assert used.min() >= 0 and used.max() < nb
    for L, t in zip(lengths, tables):
        assert len(t) == (L + 1 + 15) // 16


def test_hash_generator_numpy_torch_twins_agree_bitwise():
    idx = np.concatenate([np.arange(5000), np.array([2**31 - 1, 2**32 + 7, 10**12])])
    a = synth.hash_normal(12345, idx)
    b = synth.hash_normal_torch(12345, torch.from_numpy(idx)).numpy()
    assert np.array_equal(a, b)
    rows = synth.hash_rows(77, [0, 3, 9], 24)
    full = synth.hash_bf16_rows_torch(77, 10, 24, "cpu")
    got = full.float().double().numpy()[[0, 3, 9]]
    assert np.array_equal(rows, got)
    # roughly standard normal
    v = synth.hash_normal(1, np.arange(200000))
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.01
    assert abs(np.mean(v ** 4) - 3.0) < 0.5   # Irwin-Hall(4) kurtosis 2.7


def test_rank_permutation_keeps_the_product():
    U, V = synth.fast_factors(3, 40, 50, 12)
    perm, sign = synth.rank_permutation(9, 12)
    U2, V2 = U[:, perm] * sign[None, :], V[perm, :] * sign[:, None]
    assert np.allclose(U2 @ V2, U @ V, atol=1e-13)
