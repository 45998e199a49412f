"""Pins of the oracle's product with the quantized weight (CPU only).

The operation is y = x Q^-1(W_q)^T with the inverse quantizer Q^-1(W_q) = s (W_q - z)
of section 2 of "Half-Quadratic Quantization of Large Machine Learning Models", applied
to the codes and binary16 s and z that the quantizer stores (row n of the weight holds
output n, grouped along the input dimension K).  These tests tie
``oracle.hqq_matmul`` to facts that do not come from its own formula:
  * a unit activation x = 2^j e_k picks column k of the dequantized weight, which the
    separately written dequantizer rounds once to binary16 (scaled exactly by 2^j);
  * on weights the quantizer reproduces exactly (every group on its code grid), the
    product equals numpy's fp64 matmul of the original binary16 weights;
  * brute force in exact rational arithmetic on small random operands;
  * linearity in x on exactly representable activations, and empty shapes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _quantized(rows, cols, nbits, g, seed):
    rng = np.random.default_rng(seed)
    W = np.asarray(rng.standard_t(4, (rows, cols)) * 0.02, np.float16)
    return W, oracle.hqq_quantize(W, nbits, g)


@pytest.mark.parametrize("nbits,g", [(4, 64), (3, 32), (2, 16), (8, 128)])
def test_unit_activations_pick_dequantized_columns(nbits, g):
    N, K = 24, 256
    _, r = _quantized(N, K, nbits, g, seed=nbits * 10 + g)
    deq = oracle.hqq_dequantize(r.packed, r.scale_f16, r.zero_f16, N, K, nbits, g)
    ks = [0, 1, g - 1, g, K // 2 + 3, K - 1]
    for j in (0, -3, 2):
        X = np.zeros((len(ks), K), np.float16)
        for m, k in enumerate(ks):
            X[m, k] = np.float16(2.0 ** j)
        Y = oracle.hqq_matmul(X, r.packed, r.scale_f16, r.zero_f16, N, nbits, g)
        for m, k in enumerate(ks):
            got = oracle.f64_to_f16(Y[m] * 2.0 ** -j)
            assert np.array_equal(got, deq[:, k]), (j, k)


def test_on_grid_weights_give_the_plain_product():
    # every group is a*(c - c0) for integer codes c spanning 0..qmax, a a power of two:
    # min-max init gives s = a and z = c0 exactly, so W is reproduced bit for bit
    rng = np.random.default_rng(3)
    nbits, g, N, K = 4, 64, 16, 192
    W = np.empty((N, K), np.float16)
    for n in range(N):
        for j in range(K // g):
            c = rng.integers(0, 16, g)
            c[rng.integers(0, g)] = 0
            c[(rng.integers(1, g) + 7) % g] = 15
            c[0], c[1] = 0, 15
            a = 2.0 ** -int(rng.integers(5, 9))
            c0 = int(rng.integers(0, 16))
            W[n, j * g:(j + 1) * g] = (a * (c - c0)).astype(np.float16)
    r = oracle.hqq_quantize(W, nbits, g)
    deq = oracle.hqq_dequantize(r.packed, r.scale_f16, r.zero_f16, N, K, nbits, g)
    assert np.array_equal(deq, W.view(np.uint16))  # the quantizer is exact here
    X = np.asarray(rng.standard_normal((5, K)), np.float16)
    Y = oracle.hqq_matmul(X, r.packed, r.scale_f16, r.zero_f16, N, nbits, g)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    scale = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    assert np.all(np.abs(Y - ref) <= 4 * K * 2.0 ** -53 * scale)


def _exact(X, codes, s16, z16, g):
    M, K = X.shape
    N = codes.shape[0]
    fx = [[Fraction(float(v)) for v in row] for row in X.astype(np.float64)]
    out = np.empty((M, N), object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                s = Fraction(float(s16[n, k // g]))
                z = Fraction(float(z16[n, k // g]))
                acc += fx[m][k] * s * (int(codes[n, k]) - z)
            out[m, n] = acc
    return out


@pytest.mark.parametrize("nbits,g", [(4, 16), (2, 32), (3, 16), (8, 32)])
def test_exact_rational_brute_force(nbits, g):
    rng = np.random.default_rng(nbits + g)
    M, N, K = 3, 4, 64
    qmax = (1 << nbits) - 1
    codes = rng.integers(0, qmax + 1, (N, K)).astype(np.uint8)
    packed = np.zeros((N * K * nbits + 7) // 8, np.uint8)
    oracle._load().oracle_pack_codes(oracle._ptr(codes.ravel().copy()), N * K, nbits,
                                     oracle._ptr(packed))
    s16 = np.asarray(rng.uniform(1e-3, 0.05, (N, K // g)), np.float16)
    z16 = np.asarray(rng.uniform(-2, qmax + 2, (N, K // g)), np.float16)
    X = np.asarray(rng.standard_normal((M, K)) * 3, np.float16)
    Y = oracle.hqq_matmul(X, packed, s16, z16, N, nbits, g)
    ex = _exact(X, codes, s16, z16, g)
    for m in range(M):
        for n in range(N):
            e = ex[m, n]
            bound = Fraction(K + 2, 2 ** 52) * sum(
                abs(Fraction(float(X[m, k])) * Fraction(float(s16[n, k // g])) *
                    (int(codes[n, k]) - Fraction(float(z16[n, k // g])))) for k in range(K))
            assert abs(Fraction(Y[m, n]) - e) <= bound


def test_linearity_and_empty_shapes():
    nbits, g, N, K = 4, 64, 8, 128
    _, r = _quantized(N, K, nbits, g, seed=9)
    rng = np.random.default_rng(9)
    X1 = rng.integers(-8, 9, (4, K)).astype(np.float16)  # small integers: sums stay exact
    X2 = rng.integers(-8, 9, (4, K)).astype(np.float16)
    args = (r.packed, r.scale_f16, r.zero_f16, N, nbits, g)
    Y1, Y2 = oracle.hqq_matmul(X1, *args), oracle.hqq_matmul(X2, *args)
    Y12 = oracle.hqq_matmul((X1.astype(np.float64) + X2).astype(np.float16), *args)
    tol = 4 * K * 2.0 ** -53 * (np.abs(Y1) + np.abs(Y2) + 1e-3)
    assert np.all(np.abs(Y12 - (Y1 + Y2)) <= tol)
    assert np.array_equal(oracle.hqq_matmul(np.zeros((2, K), np.float16), *args), np.zeros((2, N)))
    assert oracle.hqq_matmul(np.zeros((0, K), np.float16), *args).shape == (0, N)
    # K not a multiple of the group size is rejected before any pointer is read
    assert oracle._load().oracle_hqq_matmul(None, 1, K + 8, None, None, None, N, nbits, g,
                                            None) == -1
