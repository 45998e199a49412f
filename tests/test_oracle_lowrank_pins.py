"""Pins of the oracle's quantization residual and truncated SVD (CPU only).

The plain SVD compensation on the EoRA page (section 1) factors the quantization
error Delta W = W - W_hat as U Sigma V^T and keeps B = U Sigma, A = V^T (LoRA factors)
at rank r.  ``oracle.hqq_residual`` is Delta W with W_hat = s (W_q - z) from the stored
codes and binary16 s, z (section 2 of the HQQ page); ``oracle.lowrank_svd`` is the
truncation.  Pins (facts that do not come from these functions themselves):
  * the residual is zero on weights the quantizer reproduces exactly, equals
    W - (the separately written dequantizer's binary16 output) within that output's
    half-ulp, and stays within s/2 where the code is not clamped;
  * on matrices with a planted spectrum the truncation returns the planted singular
    values and the planted rank-r part, its error is the Eckart-Young value
    sum_{i>r} sigma_i^2, the rows of A are orthonormal and the columns of B orthogonal
    with norms sigma_i, and r >= rank reconstructs exactly.
"""
import numpy as np
import pytest

import oracle


def _planted(m, n, sig, seed):
    rng = np.random.default_rng(seed)
    k = len(sig)
    U, _ = np.linalg.qr(rng.standard_normal((m, k)))
    V, _ = np.linalg.qr(rng.standard_normal((n, k)))
    return U, np.asarray(sig, np.float64), V


def test_residual_is_zero_on_grid_and_matches_the_dequantizer():
    rng = np.random.default_rng(5)
    nbits, g, N, K = 4, 64, 12, 256
    W = np.empty((N, K), np.float16)
    for n in range(N):
        for j in range(K // g):
            c = rng.integers(0, 16, g)
            c[0], c[1] = 0, 15
            a = 2.0 ** -int(rng.integers(5, 9))
            W[n, j * g:(j + 1) * g] = (a * (c - int(rng.integers(0, 16)))).astype(np.float16)
    r = oracle.hqq_quantize(W, nbits, g)
    assert np.array_equal(oracle.hqq_residual(W, r.packed, r.scale_f16, r.zero_f16, nbits, g),
                          np.zeros((N, K)))
    # general weights: Delta W = W - (exact dequantization), the binary16 dequantizer is its
    # single rounding
    for nbits, g in ((4, 64), (2, 16), (3, 32), (8, 128)):
        W = np.asarray(rng.standard_t(4, (16, 256)) * 0.02, np.float16)
        r = oracle.hqq_quantize(W, nbits, g)
        dW = oracle.hqq_residual(W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
        deq = oracle.f16_to_f64(oracle.hqq_dequantize(r.packed, r.scale_f16, r.zero_f16, 16, 256,
                                                      nbits, g))
        half_ulp = np.spacing(np.abs(deq).astype(np.float16)).astype(np.float64) / 2
        assert np.all(np.abs(dW - (W.astype(np.float64) - deq)) <= half_ulp + 1e-300)
        # |Delta W| <= s/2 on the solver's fp64 grid (plus fp64 rounding) where the code is
        # not clamped, plus what the binary16 storage of s and z moves
        q = r.codes.astype(np.float64)
        s64 = np.repeat(r.scale, g, axis=1)
        z64 = np.repeat(r.zero, g, axis=1)
        s16 = np.repeat(oracle.f16_to_f64(r.scale_f16), g, axis=1)
        z16 = np.repeat(oracle.f16_to_f64(r.zero_f16), g, axis=1)
        storage = np.abs(s16 * (q - z16) - s64 * (q - z64))
        inner = (r.codes > 0) & (r.codes < (1 << nbits) - 1)
        assert np.all(np.abs(dW[inner]) <= (s64 * (0.5 + 1e-6) + storage * (1 + 1e-9))[inner])


def test_singular_values_are_the_planted_ones():
    sig = [7.0, 3.0, 2.0, 0.5]
    U, S, V = _planted(50, 30, sig, seed=3)
    s = oracle.singular_values((U * S) @ V.T)
    assert s.shape == (30,)
    assert np.allclose(s[:4], sig, rtol=1e-12) and np.all(np.abs(s[4:]) <= 1e-12)


@pytest.mark.parametrize("m,n", [(60, 40), (40, 70)])
def test_planted_spectrum(m, n):
    sig = [9.0, 5.0, 4.0, 2.5, 1.0, 0.5, 0.25]
    U, S, V = _planted(m, n, sig, seed=m + n)
    M = (U * S) @ V.T
    for r in (1, 3, 5):
        B, A, s_all = oracle.lowrank_svd(M, r)
        assert B.shape == (m, r) and A.shape == (r, n)
        assert np.allclose(s_all[:len(sig)], S, rtol=1e-12, atol=1e-12)
        assert np.allclose(s_all[len(sig):], 0.0, atol=1e-12)
        Mr = (U[:, :r] * S[:r]) @ V[:, :r].T  # the planted rank-r part (distinct sigmas)
        assert np.allclose(B @ A, Mr, atol=1e-12)
        err = np.sum((M - B @ A) ** 2)
        assert abs(err - np.sum(S[r:] ** 2)) <= 1e-10  # Eckart-Young
        assert np.allclose(A @ A.T, np.eye(r), atol=1e-12)
        G = B.T @ B
        assert np.allclose(G, np.diag(S[:r] ** 2), atol=1e-10)
        # sign convention: the largest-magnitude entry of each row of A is positive
        assert np.all(A[np.arange(r), np.argmax(np.abs(A), axis=1)] > 0)
    B, A, _ = oracle.lowrank_svd(M, len(sig) + 3)  # r >= rank: exact
    assert np.allclose(B @ A, M, atol=1e-12)


def test_truncation_beats_random_rank_r_approximations():
    rng = np.random.default_rng(3)
    M = rng.standard_normal((50, 30))
    B, A, s = oracle.lowrank_svd(M, 4)
    best = np.sum((M - B @ A) ** 2)
    for _ in range(20):
        Q, _ = np.linalg.qr(rng.standard_normal((30, 4)))
        assert np.sum((M - (M @ Q) @ Q.T) ** 2) >= best - 1e-9
