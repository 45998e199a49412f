"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what it pins.  Sources: the page "Half-Quadratic Quantization
of Large Machine Learning Models" (section 2: quantizer and its inverse;
section 2.1: lp shrink and its l1 special case, soft-thresholding; section 2.2:
the z update as the minimizer of a quadratic, i.e. a mean; section 4.1: default
parameters), IEEE 754 binary16 as implemented by numpy, numpy's bit packing,
brute force on tiny inputs, and hand-derived worked examples (derivations
written next to each example).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ binary16 --

def test_f16_decode_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy_and_ties_go_to_even():
    rng = np.random.default_rng(7)
    # random magnitudes over the whole binary16 range, both signs
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),
        rng.uniform(-70000, 70000, 2000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1e-30]),
    ])
    ours = oracle.f64_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    # exact midpoints between consecutive finite binary16 values: RNE picks the even code
    h = np.arange(0, 0x7bff, 37, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0  # exact in fp64
    got = oracle.f64_to_f16(mid)
    want = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.f64_to_f16(-mid), want | 0x8000)


# ------------------------------------------------------------ section 2.1 --

def _soft_threshold(x, t):
    return np.sign(x) * np.maximum(np.abs(x) - t, 0.0)


def test_shrink_at_p1_is_soft_threshold():
    """Section 2.1: for the l1 norm the shrink is the soft-thresholding operator."""
    for beta in (0.5, 1.0, 3.0, 1e4):
        for x in np.linspace(-5, 5, 401):
            assert oracle.shrink_lp(x, beta, 1.0) == pytest.approx(_soft_threshold(x, 1.0 / beta),
                                                                   abs=1e-15)
    # spot values at beta = 1, derived by hand
    assert oracle.shrink_lp(3.0, 1.0, 1.0) == 2.0
    assert oracle.shrink_lp(-2.5, 1.0, 1.0) == -1.5
    assert oracle.shrink_lp(-0.5, 1.0, 1.0) == 0.0


def test_shrink_at_p1_is_the_l1_proximal_operator_by_brute_force():
    """argmin_y |y| + beta/2 (y - x)^2, found on a fine grid, equals shrink(x, beta) at p = 1."""
    ys = np.linspace(-6, 6, 1_200_001)  # spacing 1e-5
    for beta in (0.7, 1.0, 2.5):
        for x in (-4.2, -1.3, -0.2, 0.0, 0.9, 1.01, 3.7):
            y = ys[np.argmin(np.abs(ys) + 0.5 * beta * (ys - x) ** 2)]
            assert abs(y - oracle.shrink_lp(x, beta, 1.0)) <= 1e-5


def test_shrink_threshold_sign_and_zero():
    """shrink(x) != 0 exactly when |x| - |x|^(p-1)/beta > 0, i.e. |x|^(2-p) > 1/beta."""
    for p in (0.0, 0.3, 0.7, 1.0):
        for beta in (0.5, 1.0, 1e4):
            tau = beta ** (-1.0 / (2.0 - p))
            assert oracle.shrink_lp(tau * (1 - 1e-9), beta, p) == 0.0
            assert oracle.shrink_lp(tau * (1 + 1e-6), beta, p) > 0.0
            assert oracle.shrink_lp(-tau * (1 + 1e-6), beta, p) < 0.0
            assert oracle.shrink_lp(0.0, beta, p) == 0.0
            for x in (0.1, 1.7, 42.0):
                assert oracle.shrink_lp(-x, beta, p) == -oracle.shrink_lp(x, beta, p)
                assert abs(oracle.shrink_lp(x, beta, p)) <= x


def test_shrink_scaling_identity_pins_the_exponent():
    """shrink(a x, beta a^(p-2)) = a shrink(x, beta): |a x|^(p-1) / (beta a^(p-2)) = a |x|^(p-1)/beta.
    A wrong exponent (p instead of p-1, or a missing 1/beta) breaks it."""
    rng = np.random.default_rng(3)
    for p in (0.0, 0.5, 0.7, 1.0):
        for a in (0.25, 2.0, 8.0):
            for x in rng.uniform(-3, 3, 50):
                for beta in (0.3, 1.0, 5.0):
                    lhs = oracle.shrink_lp(a * x, beta * a ** (p - 2.0), p)
                    rhs = a * oracle.shrink_lp(x, beta, p)
                    assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-15)


# -------------------------------------------------------------- section 2 --

def test_quantize_rounds_half_to_even_and_clamps():
    q = lambda v, qmax=3: oracle.quantize_value(v, 1.0, 0.0, qmax)  # noqa: E731
    assert [q(0.5), q(1.5), q(2.5), q(0.49), q(0.51)] == [0.0, 2.0, 2.0, 0.0, 1.0]
    assert [q(-0.5), q(-3.0), q(3.4), q(3.5), q(99.0)] == [0.0, 0.0, 3.0, 3.0, 3.0]
    assert q(254.5, 255) == 254.0 and q(253.5, 255) == 254.0
    # the decision is taken on the fp64 value itself: values off a half-integer by far less
    # than a binary32 half-ulp still go to the nearer integer
    assert [q(0.5 + 2**-40), q(2.5 - 2**-40), q(1.5 + 2**-35), q(2.5 + 2**-45)] == [1.0, 2.0, 2.0, 3.0]
    assert q(128.5 - 2**-30, 255) == 128.0 and q(127.5 + 2**-30, 255) == 128.0


def _exact_half_even(num: Fraction) -> int:
    """Round half to even of an exact rational (Python integers only)."""
    k = num.numerator // num.denominator
    rem = num - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k


def test_round_ratio_is_exact_rational_rounding():
    """The exact ratio rounding of the initial quantizer against Python's rationals, on
    differences of random binary16 values (every magnitude, subnormals included) and on exact
    midpoints."""
    rng = np.random.default_rng(31)
    bits = rng.integers(0, 0x7BFF, (20000, 3)).astype(np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    for qmax in (3, 7, 15, 255):
        for a, b, c in v[:5000]:
            lo, hi = min(a, b), max(a, b)
            if not hi > lo:
                continue
            w = lo + (hi - lo) * (c / 65504.0)
            w = float(np.float16(w))
            if not lo <= w <= hi:
                continue
            num = (w - lo) * qmax  # exact in fp64
            assert Fraction(num) == (Fraction(w) - Fraction(lo)) * qmax
            exact = _exact_half_even((Fraction(w) - Fraction(lo)) * qmax / (Fraction(hi) - Fraction(lo)))
            assert oracle.round_ratio(num, hi - lo) == exact
    # exact midpoints: (2k+1)/2 of any binary16 difference goes to the even neighbour
    for k in range(0, 255):
        d = float(np.float16(rng.uniform(1e-3, 10)))
        assert oracle.round_ratio((2 * k + 1) * d / 2, d) == (k if k % 2 == 0 else k + 1)


# binary16 groups (min, max, w) whose exact ratio (w - min) qmax / (max - min) lies off a
# half-integer by less than a binary32 half-ulp: the exact code is the nearer integer,
# while rounding the ratio to binary32 first would make it a tie and pick the even one.
# Found by a search over exact rationals (Python fractions); the expected code is computed
# below from the rationals, not stored.
NEAR_TIE_TRIPLES = {
    15: [(-0.375, 0.286865234375, 5.698204040527344e-05),
         (-0.375, 0.11407470703125, -4.273653030395508e-05),
         (-0.375, 0.01293182373046875, 7.748603820800781e-07),
         (-0.63232421875, 18.34375, 0.00021159648895263672),
         (-0.63232421875, 5.69140625, 4.881620407104492e-05),
         (-0.63232421875, 0.365966796875, -7.325410842895508e-05)],
    7: [(-1.0859375, 14.1171875, 5.960464477539063e-08),
        (-1.0859375, 3.982421875, 0.00013947486877441406),
        (-1.0859375, 0.08355712890625, 2.181529998779297e-05),
        (-0.49609375, 0.275634765625, 1.7464160919189453e-05)],
    3: [(-0.36279296875, 1.8134765625, -8.13603401184082e-05),
        (-1.6845703125, 1.6845703125, -5.960464477539063e-08),
        (-1.6845703125, 0.3369140625, 5.960464477539063e-08),
        (-0.75146484375, 0.1502685546875, -2.0325183868408203e-05)],
    255: [(-0.04083251953125, 0.0210418701171875, 5.310773849487305e-05),
          (-0.0085906982421875, 0.0135040283203125, 3.057718276977539e-05),
          (-1.435546875, -0.0307769775390625, -0.64501953125),
          (0.0102386474609375, 1.3017578125, 0.89404296875)],
}


def test_init_codes_are_exact_next_to_half_integers():
    """Section 2's round(W/s + z) at the min-max initialisation, decided on the exact value:
    for every triple the ratio is within a binary32 half-ulp of a half-integer, so the exact
    code and the code of the binary32-rounded ratio differ; the oracle must give the exact
    one, in the whole solver at T = 0 too."""
    bits = {3: 2, 7: 3, 15: 4, 255: 8}
    for qmax, triples in NEAR_TIE_TRIPLES.items():
        for mn, mx, w in triples:
            assert all(float(np.float16(x)) == x for x in (mn, mx, w))
            ratio = (Fraction(w) - Fraction(mn)) * qmax / (Fraction(mx) - Fraction(mn))
            exact = _exact_half_even(ratio)
            half = Fraction(2 * (exact if ratio > exact else exact - 1) + 1, 2)
            assert 0 < abs(ratio - half) <= Fraction(1, 2 ** 24) * half  # off the tie, below 2^-24
            b32 = int(np.rint(np.float64(np.float32(float(ratio)))))
            assert b32 != exact  # the case exists only below binary32 resolution
            assert oracle.quantize_init_value(w, mn, mx, qmax) == exact
            r = oracle.hqq_group(np.array([mn, mx, w]), bits[qmax], iters=0)
            assert r.codes.tolist() == [0, qmax, exact]


def test_exact_midpoint_tie_at_init_is_half_even():
    """An element at the exact midpoint of min and max has w/s + z = qmax/2 exactly (a tie for
    odd qmax).  Exact arithmetic rounds 7.5 to 8 (half-even); evaluating w * (1/s) + z0 in
    fp64 would leave it on either side of 7.5 by rounding noise."""
    rng = np.random.default_rng(17)
    hits = 0
    for _ in range(2000):
        w = (rng.standard_normal(16) * 0.02).astype(np.float16).astype(np.float64)
        mid = (w.min() + w.max()) / 2
        if np.float16(mid).astype(np.float64) != mid:
            continue
        k = [i for i in range(16) if i not in (int(w.argmin()), int(w.argmax()))][0]
        w[k] = mid
        assert oracle.quantize_init_value(mid, w.min(), w.max(), 15) == 8.0
        assert oracle.hqq_group(w, 4, iters=0).codes[k] == 8
        hits += 1
    assert hits > 100


def test_minmax_init_maps_min_and_max_to_the_ends_of_the_code_range():
    rng = np.random.default_rng(11)
    for nbits in (2, 3, 4, 8):
        qmax = (1 << nbits) - 1
        for _ in range(50):
            w = rng.standard_normal(64) * 0.02
            s, inv_s, z = oracle.minmax_init(w, nbits)
            assert s == pytest.approx((w.max() - w.min()) / qmax, rel=1e-15)
            assert s * inv_s == pytest.approx(1.0, rel=1e-15)
            assert oracle.quantize_value(w.min(), inv_s, z, qmax) == 0.0
            assert oracle.quantize_value(w.max(), inv_s, z, qmax) == qmax
            assert w.min() * inv_s + z == pytest.approx(0.0, abs=1e-12)
    # constant group: s = 1, z = -min
    assert oracle.minmax_init(np.full(16, 0.375), 4) == (1.0, 1.0, -0.375)


def test_group_error_closed_values():
    r = np.array([3.0, -4.0, 0.0, 0.0])
    assert oracle.group_error(r, 2.0) == 25.0
    assert oracle.group_error(r, 1.0) == 7.0
    assert oracle.group_error(r, 0.0) == 2.0  # |0|^0 := 0, counts the non-zero residuals
    assert oracle.group_error(np.array([0.25]), 0.5) == 0.5


# ------------------------------------------------------------ section 2.2 --

def test_z_update_minimizes_its_quadratic_by_brute_force():
    """Section 2.2: z^(t+1) = argmin_z 1/2 || Q^-1_z(W_q) - (W - W_e) ||^2 with W_q frozen.
    The oracle's z must sit at the grid minimum of f(z) = sum (s(q - z) - (w - W_e))^2
    and satisfy the optimality condition f'(z) = 0."""
    rng = np.random.default_rng(5)
    for g in (4, 8):
        for _ in range(40):
            s = float(rng.uniform(0.005, 0.5))
            q = rng.integers(0, 16, g).astype(np.float64)
            w = rng.standard_normal(g) * 8 * s
            we = np.where(rng.random(g) < 0.5, rng.standard_normal(g) * s, 0.0)
            z = oracle.z_update(q, w, we, 1.0 / s)
            grid = z + np.arange(-2000, 2001) * 1e-6
            f = ((s * (q[None, :] - grid[:, None]) - (w - we)[None, :]) ** 2).sum(1)
            assert abs(grid[np.argmin(f)] - z) <= 1e-6
            fprime = -2.0 * s * np.sum(s * (q - z) - (w - we))
            assert abs(fprime) <= 1e-12 * max(1.0, np.sum(np.abs(w)) / s)


# ---------------------------------------------------------- whole solver --

def test_hand_example_stops_at_the_first_evaluation():
    """Worked by hand (g=4, b=2, p=0.7, beta=1, kappa=1.01, T=20), w = [-1, 0, 0.5, 2]:
    min-max init gives s = 1, z0 = 1; codes round(w + 1) = [0, 1, 2, 3] (1.5 -> 2, half-even);
    residuals [0, 0, -0.5, 0], e0 = 0.5^0.7.  The shrink is zero (0.5 - 0.5^-0.3 < 0), so
    z1 = mean(q - w) = 1.125; codes stay [0,1,2,3], residuals [0.125, 0.125, -0.375, 0.125],
    e1 = 3 * 0.125^0.7 + 0.375^0.7 > e0, so the solver stops and keeps z0."""
    w = np.array([-1.0, 0.0, 0.5, 2.0])
    r = oracle.hqq_group(w, 2, p=0.7, beta=1.0, kappa=1.01, iters=20)
    assert r.stop_step == 0 and r.n_eval == 2
    assert r.scale == 1.0 and r.zero == 1.0
    assert r.codes.tolist() == [0, 1, 2, 3]
    assert r.err_init == pytest.approx(0.5 ** 0.7, rel=1e-15)
    assert r.trace[1] == pytest.approx(3 * 0.125 ** 0.7 + 0.375 ** 0.7, rel=1e-15)
    assert r.err_best == r.err_init
    # same under the l1 reading of "the error" (0.75 >= 0.5) ...
    assert oracle.hqq_group(w, 2, iters=20, err_pow=1.0).stop_step == 0
    # ... but under l2 the first update is accepted (0.1875 < 0.25)
    assert oracle.hqq_group(w, 2, iters=20, err_pow=2.0).stop_step >= 1
    # with the early stop disabled and T = 1 the solver returns z1 = 1.125, same codes
    r1 = oracle.hqq_group(w, 2, iters=1, early_stop=False)
    assert r1.zero == 1.125 and r1.stop_step == 1 and r1.codes.tolist() == [0, 1, 2, 3]
    # packed 2-bit byte of codes [0,1,2,3] is 0b11100100
    assert oracle.pack_codes(r.codes, 2).tolist() == [0xE4]


def test_hand_example_accepts_one_update():
    """Worked by hand (g=8, b=2, p=0.7, beta=1): w = [0, .25 x6, 3] -> s = 1, z0 = 0,
    codes [0 x7, 3], residuals [0, .25 x6, 0], e0 = 6 * .25^.7.  No shrink (|r| < 1), so
    z1 = mean(q - w) = (3 - 4.5)/8 = -0.1875; codes unchanged; residuals w - q + z1 =
    [-.1875, .0625 x6, -.1875]; e1 = 6 * .0625^.7 + 2 * .1875^.7 < e0 -> accepted.
    z2 = mean(q - w) = z1 again, so e2 = e1 and the solver stops with t* = 1."""
    w = np.array([0.0] + [0.25] * 6 + [3.0])
    r = oracle.hqq_group(w, 2, p=0.7, beta=1.0, kappa=1.01, iters=20)
    assert r.stop_step == 1 and r.n_eval == 3
    assert r.zero == -0.1875 and r.scale == 1.0
    assert r.codes.tolist() == [0] * 7 + [3]
    assert r.err_init == pytest.approx(6 * 0.25 ** 0.7, rel=1e-15)
    assert r.err_best == pytest.approx(6 * 0.0625 ** 0.7 + 2 * 0.1875 ** 0.7, rel=1e-15)
    assert r.trace[2] == r.trace[1]


def test_hand_example_with_active_shrink_and_beta_schedule():
    """Worked by hand in exact dyadic arithmetic (g=8, b=2, p=1, beta0=8, kappa=2, T=3),
    w = [0, .25 x6, 3], s = 1, codes stay [0 x7, 3] throughout:
      t=0: z=0,        r=[0, .25 x6, 0],            e=1.5;   W_e=[0, .125 x6, 0] (thr 1/8)
           z1 = (-1.5 + .75)/8 = -0.09375
      t=1: r=[-.09375, .15625 x6, -.09375],         e=1.125; thr 1/16 -> sum W_e = .5625 - .0625
           z2 = (-1.5 + .5)/8 = -0.125
      t=2: r=[-.125, .125 x6, -.125],               e=1.0;   thr 1/32 -> sum W_e = .375
           z3 = (-1.5 + .375)/8 = -0.140625
      t=3: r=[-.140625, .109375 x6, -.140625],      e=0.9375 accepted, t = T -> stop."""
    w = np.array([0.0] + [0.25] * 6 + [3.0])
    r = oracle.hqq_group(w, 2, p=1.0, beta=8.0, kappa=2.0, iters=3)
    assert r.trace.tolist() == [1.5, 1.125, 1.0, 0.9375]
    assert r.stop_step == 3 and r.zero == -0.140625
    assert r.codes.tolist() == [0] * 7 + [3]
    # one more iteration continues the same exact sequence: thr 1/64, sum W_e = .3125
    r4 = oracle.hqq_group(w, 2, p=1.0, beta=8.0, kappa=2.0, iters=4)
    assert r4.zero == (-1.5 + 0.3125) / 8 and r4.trace[4] == 0.90625


def test_zero_iterations_is_round_to_nearest():
    """T = 0: the solver reduces to asymmetric min-max round-to-nearest (numpy fp64, half-even)."""
    rng = np.random.default_rng(21)
    n_near = 0
    for nbits in (2, 3, 4, 8):
        qmax = (1 << nbits) - 1
        W = (rng.standard_normal((16, 128)) * 0.02).astype(np.float16)
        # plant exact ties: the midpoint of a group's min and max, where it is a binary16
        Wv = W.reshape(-1, 32)
        for grp in Wv[::3]:
            mid = (float(grp.min()) + float(grp.max())) / 2
            j = [i for i in range(32) if i not in (int(grp.argmin()), int(grp.argmax()))][0]
            if float(np.float16(mid)) == mid:
                grp[j] = mid
        res = oracle.hqq_quantize(W, nbits, 32, iters=0)
        Wg = W.astype(np.float64).reshape(-1, 32)
        mn, mx = Wg.min(1, keepdims=True), Wg.max(1, keepdims=True)
        s = (mx - mn) / qmax
        pre = (Wg - mn) / s
        ref = np.clip(np.round(pre), 0, qmax)
        # within fp64 noise of a half-integer numpy's two roundings cannot decide: those
        # elements take the exact rational answer instead, so every code is compared
        near = np.abs(np.abs(pre - np.floor(pre)) - 0.5) < 1e-9
        for i, j in zip(*np.nonzero(near)):
            ratio = (Fraction(Wg[i, j]) - Fraction(mn[i, 0])) * qmax / (Fraction(mx[i, 0]) - Fraction(mn[i, 0]))
            ref[i, j] = _exact_half_even(ratio)
        n_near += int(near.sum())
        assert np.array_equal(res.codes.reshape(-1, 32), ref)
        assert (res.stop_step == 0).all()
        assert np.allclose(res.zero.reshape(-1, 1), -mn / s, rtol=1e-14, atol=1e-12)
    assert n_near > 0  # the exact ties of binary16 data are part of the comparison


def test_early_stop_invariants_on_layer_like_groups():
    """Per group: e_0 >= e_best; the accepted errors strictly decrease; the evaluation after
    the last accepted one did not improve; t* in [0, T]."""
    for wl_name in ("single_256x512", "mlp_11008x4096"):
        wl = workloads.WORKLOADS[wl_name]
        W = workloads.generate(64, 512, wl.dist, 123, "cpu").numpy().astype(np.float64)
        for nbits, g in ((4, 64), (2, 16), (2, 32), (3, 64)):
            for row in W[:16]:
                for grp in row.reshape(-1, g)[:8]:
                    r = oracle.hqq_group(grp, nbits, iters=20)
                    t = r.stop_step
                    assert 0 <= t <= 20 and r.err_best <= r.err_init
                    assert np.all(np.diff(r.trace[: t + 1]) < 0)
                    assert r.err_best == r.trace[t]
                    if t < 20:
                        assert r.n_eval == t + 2 and r.trace[t + 1] >= r.trace[t]
                    else:
                        assert r.n_eval == 21


def test_unchanged_zero_point_repeats_the_error():
    """The error of an evaluation depends on z alone, so a z update that leaves z unchanged
    repeats the last error: under the strict-improvement stop that step is rejected and
    the group ends with the last accepted z (which the device uses to stop such a group
    without evaluating the repeat).  Checked on the no-stop trajectory: wherever z after
    t + 1 updates equals z after t updates, error t + 1 equals error t exactly; and the
    early-stop run then stops at the first such repeat (if not earlier)."""
    wl = workloads.WORKLOADS["llama70b_stack"]
    W = workloads.generate(16, 512, wl.dist, 321, "cpu").numpy().astype(np.float64)
    repeats = groups = 0
    for nbits, g in ((2, 32), (4, 64)):
        for grp in W.reshape(-1, g)[:48]:
            full = oracle.hqq_group(grp, nbits, iters=20, early_stop=False)
            z = [oracle.hqq_group(grp, nbits, iters=t, early_stop=False).zero for t in range(21)]
            first = None
            for t in range(20):
                if z[t + 1] == z[t]:
                    assert full.trace[t + 1] == full.trace[t]
                    first = t if first is None else first
            r = oracle.hqq_group(grp, nbits, iters=20)
            if first is not None:
                assert r.stop_step <= first
                repeats += r.stop_step == first
            groups += 1
    # the early stop ends at such a repeat for about a third of these groups
    assert repeats >= groups // 5


def test_constant_and_on_grid_groups_are_exact():
    # constant group: s = 1, z = -w, all codes 0, e0 = 0, t* = 0
    r = oracle.hqq_group(np.full(32, -0.0625), 4)
    assert (r.scale, r.zero, r.stop_step, r.err_init) == (1.0, 0.0625, 0, 0.0)
    assert (r.codes == 0).all()
    # values on the grid s (k - z): s = 0.5, z = 3 (min -1.5 -> code 0, max 6 -> code 15)
    rng = np.random.default_rng(2)
    k = np.concatenate([[0, 15], rng.integers(0, 16, 62)]).astype(np.float64)
    w = 0.5 * (k - 3.0)
    r = oracle.hqq_group(w, 4)
    assert r.scale == 0.5 and r.zero == 3.0 and r.err_init == 0.0 and r.stop_step == 0
    assert np.array_equal(r.codes, k.astype(np.uint8))


def test_exact_ties_follow_half_even():
    # s = 1 and integer z make w + z an exact half-integer in fp64 (and fp32)
    w = np.array([0.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.5, 3.0])
    r = oracle.hqq_group(w, 2, iters=0)
    assert r.codes.tolist() == [0, 0, 2, 2, 1, 2, 0, 3]


def test_power_of_two_scaling_invariance():
    """Scaling W by a = 2^k with beta' = beta a^(p-2) scales s by a and leaves codes, z and t*
    unchanged: shrink(a x, beta') = a shrink(x, beta) and every error scales by a^p.
    Bit-exact for p = 1 and p = 0, where no pow() rounding enters."""
    wl = workloads.WORKLOADS["mlp_11008x4096"]
    W = workloads.generate(32, 256, wl.dist, 77, "cpu").numpy()
    for p in (1.0, 0.0, 0.7):
        for k in (1, 4):  # upward only: fp16 subnormals would lose bits going down
            a = 2.0 ** k
            Wa = (W.astype(np.float64) * a).astype(np.float16)  # exact: no overflow/underflow
            assert np.array_equal(Wa.astype(np.float64), W.astype(np.float64) * a)
            for nbits, g, beta in ((2, 32, 1.0), (4, 64, 1e4)):
                r0 = oracle.hqq_quantize(W, nbits, g, p=p, beta=beta)
                r1 = oracle.hqq_quantize(Wa, nbits, g, p=p, beta=beta * a ** (p - 2.0))
                assert np.array_equal(r1.scale, r0.scale * a)
                if p in (0.0, 1.0):
                    assert np.array_equal(r1.codes, r0.codes)
                    assert np.array_equal(r1.zero, r0.zero)
                    assert np.array_equal(r1.stop_step, r0.stop_step)
                else:
                    same = r1.stop_step == r0.stop_step
                    assert same.mean() >= 0.999
                    assert np.allclose(r1.zero[same], r0.zero[same], rtol=0, atol=1e-9)


def test_reflection_invariance():
    """W -> -W maps codes q -> qmax - q, z -> qmax - z, keeps s and t*.  Half-even rounding
    is not symmetric about an odd qmax, so groups holding an exact tie at init (an element
    at an exact half-code, e.g. the midpoint of min and max) are left out."""
    wl = workloads.WORKLOADS["attn_4096x4096"]
    W = workloads.generate(32, 256, wl.dist, 5, "cpu").numpy()
    for nbits, g, beta in ((4, 64, 1.0), (3, 64, 1.0), (2, 16, 1e4)):
        qmax = (1 << nbits) - 1
        r0 = oracle.hqq_quantize(W, nbits, g, beta=beta)
        r1 = oracle.hqq_quantize(-W, nbits, g, beta=beta)
        assert np.array_equal(r1.scale, r0.scale)
        Wg = W.astype(np.float64).reshape(32, -1, g)
        mn, mx = Wg.min(2, keepdims=True), Wg.max(2, keepdims=True)
        pre = (Wg - mn) * qmax / (mx - mn)
        tie = (np.abs(pre - np.floor(pre) - 0.5) < 1e-9).any(2)
        same = r1.stop_step == r0.stop_step
        assert same[~tie].all() and (~tie).mean() > 0.9
        same &= ~tie
        assert np.allclose(r1.zero[same], qmax - r0.zero[same], atol=1e-9)
        rows_same = np.repeat(same, g, axis=1)
        assert np.array_equal(r1.codes[rows_same], qmax - r0.codes[rows_same])


def test_permutation_within_a_group_and_row_independence():
    rng = np.random.default_rng(9)
    W = (rng.standard_t(4, size=(8, 256)) * 0.014).astype(np.float16)
    base = oracle.hqq_quantize(W, 4, 64)
    perm = rng.permutation(64)
    Wp = W.reshape(8, 4, 64)[:, :, perm].reshape(8, 256)
    rp = oracle.hqq_quantize(Wp, 4, 64)
    assert np.array_equal(rp.scale, base.scale)
    assert np.array_equal(rp.stop_step, base.stop_step)
    assert np.allclose(rp.zero, base.zero, rtol=0, atol=1e-12)
    assert np.array_equal(rp.codes.reshape(8, 4, 64), base.codes.reshape(8, 4, 64)[:, :, perm])
    # each row alone gives the same result as inside the matrix; meta is row-major
    for i in range(8):
        ri = oracle.hqq_quantize(W[i: i + 1], 4, 64)
        assert np.array_equal(ri.codes[0], base.codes[i])
        assert np.array_equal(ri.zero_f16[0], base.zero_f16[i])
        assert np.array_equal(ri.packed, base.packed[i * 128:(i + 1) * 128])


def test_whole_matrix_equals_per_group_solver():
    W = workloads.generate(4, 128, workloads.WORKLOADS["single_256x512"].dist, 3, "cpu").numpy()
    res = oracle.hqq_quantize(W, 3, 32)
    Wd = W.astype(np.float64)
    for i in range(4):
        for j in range(4):
            r = oracle.hqq_group(Wd[i, j * 32:(j + 1) * 32], 3)
            assert res.zero[i, j] == r.zero and res.stop_step[i, j] == r.stop_step
            assert np.array_equal(res.codes[i, j * 32:(j + 1) * 32], r.codes)
    assert np.array_equal(res.scale_f16, oracle.f64_to_f16(res.scale))
    assert np.array_equal(res.zero_f16, oracle.f64_to_f16(res.zero))


# ---------------------------------------------------------------- storage --

def test_pack_hand_examples():
    assert oracle.pack_codes(np.array([1, 2, 3, 0]), 2).tolist() == [0x39]
    assert oracle.pack_codes(np.array([1, 2]), 4).tolist() == [0x21]
    # 3-bit: sum c_k << 3k for c = 1..7,0 is 0x1F58D1, stored little-endian
    assert oracle.pack_codes(np.array([1, 2, 3, 4, 5, 6, 7, 0]), 3).tolist() == [0xD1, 0x58, 0x1F]
    assert oracle.pack_codes(np.array([7, 200, 255]), 8).tolist() == [7, 200, 255]


def test_pack_matches_numpy_little_endian_bitstream():
    rng = np.random.default_rng(4)
    for nbits in (2, 3, 4, 8):
        codes = rng.integers(0, 1 << nbits, 8 * 37).astype(np.uint8)
        bits = ((codes[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.uint8).ravel()
        ref = np.packbits(bits, bitorder="little")
        got = oracle.pack_codes(codes, nbits)
        assert np.array_equal(got, ref)
        assert np.array_equal(oracle.unpack_codes(got, codes.size, nbits), codes)


def test_dequantize_matches_numpy_single_rounding():
    """Q^-1(W_q) = s (W_q - z) from the stored binary16 s, z; numpy evaluates it in fp64 (exact)
    and rounds once to binary16."""
    W = workloads.generate(16, 256, workloads.WORKLOADS["attn_4096x4096"].dist, 8, "cpu").numpy()
    for nbits, g in ((4, 64), (3, 64), (2, 16), (8, 128)):
        res = oracle.hqq_quantize(W, nbits, g)
        deq = oracle.hqq_dequantize(res.packed, res.scale_f16, res.zero_f16, 16, 256, nbits, g)
        s = np.repeat(res.scale_f16.view(np.float16).astype(np.float64), g, axis=1)
        z = np.repeat(res.zero_f16.view(np.float16).astype(np.float64), g, axis=1)
        ref = (s * (res.codes.astype(np.float64) - z)).astype(np.float16).view(np.uint16)
        assert np.array_equal(deq, ref)


# ------------------------------------------------------------- page values --

def test_default_solver_settings_are_the_pages():
    with open(os.path.join(HERE, "golden", "hqq_page_settings.json")) as f:
        page = json.load(f)["solver"]
    s = workloads.Solver()
    assert (s.p, s.beta, s.kappa, s.iters, s.early_stop) == (
        page["p"], page["beta"], page["kappa"], page["iters"], page["early_stop"])


def test_replay_hook_without_events_is_the_solver_and_flips_move_one_code():
    """The tie-replay entry (test infrastructure) with no events equals the solver; a flip at
    evaluation 0 moves exactly that element's code to the other neighbour of its pre-round value."""
    w = np.array([-1.0, 0.0, 0.5, 2.0])  # w + 1 = [0, 1, 1.5, 3]: element 2 is an exact tie
    base = oracle.hqq_group(w, 2)
    rep, ztr = oracle.hqq_group_replay(w, 2)
    assert rep.codes.tolist() == base.codes.tolist() and rep.zero == base.zero
    assert ztr[0] == 1.0 and len(ztr) == base.n_eval
    r1, _ = oracle.hqq_group_replay(w, 2, flips=((0, 2),), iters=0)
    assert r1.codes.tolist() == [0, 1, 1, 3]  # 1.5 -> 1 instead of 2
    # inverting the first stop decision (e1 >= e0) accepts z1 = 1.125
    r2, _ = oracle.hqq_group_replay(w, 2, inverts=(1,), iters=1)
    assert r2.stop_step == 1 and r2.zero == 1.125


# ---------------------------------------------------------------- whole-tensor stop --

def test_tensor_stop_of_one_group_is_the_group_stop():
    # a single group: the total error is the group's error, so the tensor stop is the
    # per-group early stop (pinned above by the hand examples)
    rng = np.random.default_rng(11)
    cases = [np.asarray([-1, 0, 0.5, 2], np.float16)]
    cases += [np.asarray(rng.standard_t(4, 64) * 0.02, np.float16) for _ in range(20)]
    for w in cases:
        g = w.size
        W = w.reshape(1, g).view(np.uint16)
        r_t, t_star, E = oracle.hqq_quantize_tensor_stop(W, 4 if g > 4 else 2, g)
        r_g = oracle.hqq_quantize(W, 4 if g > 4 else 2, g)
        assert t_star == int(r_g.stop_step[0, 0])
        assert r_t.zero[0, 0] == r_g.zero[0, 0]
        assert np.array_equal(r_t.codes, r_g.codes)


def test_tensor_stop_of_replicated_groups():
    # k copies of one group: E_t = k e_t, so t* is the single group's stop step
    rng = np.random.default_rng(12)
    for _ in range(5):
        w = np.asarray(rng.standard_t(3, 32) * 0.02, np.float16)
        W = np.tile(w, (7, 1)).view(np.uint16)
        _, t_star, E = oracle.hqq_quantize_tensor_stop(W, 2, 32)
        r_g = oracle.hqq_quantize(w.reshape(1, 32).view(np.uint16), 2, 32)
        assert t_star == int(r_g.stop_step[0, 0])


def test_tensor_stop_invariants_and_totals():
    W = workloads.generate_matrix(workloads.WORKLOADS["single_256x512"], 0).numpy().view(np.uint16)
    iters = 20
    r, t_star, E = oracle.hqq_quantize_tensor_stop(W, 4, 64, iters=iters)
    assert np.all(np.diff(E[: t_star + 1]) < 0)                  # strictly improving to t*
    assert t_star == iters or E[t_star + 1] >= E[t_star]          # stops at the first non-improvement
    assert np.all(r.stop_step == t_star)
    # E_0 is the sum of the min-max init errors, computed here from the quantizer alone
    Wd = oracle.f16_to_f64(W).reshape(-1, 64)
    e0 = 0.0
    for w in Wd:
        s, inv_s, z = oracle.minmax_init(w, 4)
        q = np.array([oracle.quantize_value(x, inv_s, z, 15) for x in w])
        e0 += oracle.group_error(w - s * (q - z), 0.7)
    assert abs(E[0] - e0) <= 1e-9 * e0
    # E_{t*} is the sum of the returned groups' errors
    assert abs(E[t_star] - r.err_best.sum()) <= 1e-9 * E[t_star]
    # the whole-tensor reading iterates longer than most groups would alone
    assert t_star > np.median(oracle.hqq_quantize(W, 4, 64).stop_step)
