"""Pins of the oracle's meta quantization (CPU only).

Section 4.1 of "Half-Quadratic Quantization of Large Machine Learning Models"
stores the zero-points in 8 bits without grouping or optimization, and the note
under its Llama-2 table quantizes the scales to 8 bits in groups of 128.  The
oracle reads this as affine min-max round-to-nearest over the stored binary16
values (one group per array for the zero-points, runs of 128 for the scales).
These tests pin that function to facts that do not come from the oracle itself:
a hand-worked example, the min/max mapping, the half-even tie rule, constant
groups, the group structure, monotonicity, the reconstruction bound, exact
power-of-two scaling and reflection, and the single rounding of the
dequantization (checked against numpy's own binary16 conversion).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f16(x):
    return np.asarray(x, dtype=np.float16)


def test_hand_example_whole_array():
    # w = [-1, 0, 0.5, 2]: min -1, max 2, d = 3; codes (v + 1) * 255 / 3 = 0, 85, 127.5, 255;
    # 127.5 is an exact tie and rounds half to even, to 128.
    v = f16([-1, 0, 0.5, 2])
    codes, sc, off = oracle.meta_quantize(v.view(np.uint16), 0)
    assert codes.tolist() == [0, 85, 128, 255]
    assert sc.view(np.float16)[0] == np.float16(3.0 / 255.0)
    assert off.view(np.float16)[0] == np.float16(-1.0)
    back = oracle.meta_dequantize(codes, sc, off, 0).view(np.float16)
    s = float(np.float16(3.0 / 255.0))
    expect = [np.float16(-1.0 + s * c) for c in (0, 85, 128, 255)]
    assert back.tolist() == expect


def test_half_even_ties():
    # min 0, max 255: the quotient is v itself, so v = k + 1/2 is an exact tie
    v = f16([0, 255, 2.5, 3.5, 4.5, 0.5, 1.5, 254.5])
    codes, sc, off = oracle.meta_quantize(v.view(np.uint16), 0)
    assert codes.tolist() == [0, 255, 2, 4, 4, 0, 2, 254]
    assert sc.view(np.float16)[0] == np.float16(1.0)
    assert off.view(np.float16)[0] == np.float16(0.0)


def test_min_and_max_map_to_0_and_255():
    rng = np.random.default_rng(0)
    for group in (0, 16, 128):
        v = f16(rng.standard_normal(1000) * 3 + 5)
        codes, sc, off = oracle.meta_quantize(v.view(np.uint16), group)
        gs = v.size if group == 0 else group
        for g0 in range(0, v.size, gs):
            blk = v[g0:g0 + gs].astype(np.float64)
            c = codes[g0:g0 + gs]
            assert c[np.argmin(blk)] == 0 and c[np.argmax(blk)] == 255
            assert off.view(np.float16)[g0 // gs] == np.float16(blk.min())


def test_constant_group():
    v = f16([0.75] * 5 + [1, 2, 3])
    codes, sc, off = oracle.meta_quantize(v.view(np.uint16), 5)
    assert codes[:5].tolist() == [0] * 5
    assert sc.view(np.float16)[0] == np.float16(1.0)
    assert off.view(np.float16)[0] == np.float16(0.75)
    back = oracle.meta_dequantize(codes, sc, off, 5).view(np.float16)
    assert back[:5].tolist() == [np.float16(0.75)] * 5


def test_groups_are_independent_and_ragged_last_group():
    rng = np.random.default_rng(1)
    v = f16(rng.standard_normal(300) * 0.01 + 0.02)
    codes, sc, off = oracle.meta_quantize(v.view(np.uint16), 128)
    assert sc.size == 3 and off.size == 3
    for k, (a, b) in enumerate(((0, 128), (128, 256), (256, 300))):
        c1, s1, o1 = oracle.meta_quantize(v[a:b].view(np.uint16), 0)
        assert np.array_equal(codes[a:b], c1)
        assert sc[k] == s1[0] and off[k] == o1[0]
    # a group at least as long as the array is one group
    c_all, s_all, o_all = oracle.meta_quantize(v.view(np.uint16), 0)
    c_big, s_big, o_big = oracle.meta_quantize(v.view(np.uint16), 512)
    assert np.array_equal(c_all, c_big) and s_all[0] == s_big[0] and o_all[0] == o_big[0]


def test_codes_are_monotone_in_the_value():
    rng = np.random.default_rng(2)
    v = f16(np.sort(rng.standard_normal(4000)))
    codes, _, _ = oracle.meta_quantize(v.view(np.uint16), 0)
    assert np.all(np.diff(codes.astype(int)) >= 0)


def test_reconstruction_bound():
    # |v' - v| <= d/510 (rounding of the code) + 255 |s16 - d/255| (stored meta scale)
    #            + one binary16 half-ulp of v' (final rounding)
    rng = np.random.default_rng(3)
    for group in (0, 128):
        v = f16(rng.standard_t(4, 2000) * 2 + 7)
        codes, sc, off = oracle.meta_quantize(v.view(np.uint16), group)
        back = oracle.meta_dequantize(codes, sc, off, group).view(np.float16).astype(np.float64)
        gs = v.size if group == 0 else group
        for k, g0 in enumerate(range(0, v.size, gs)):
            blk = v[g0:g0 + gs].astype(np.float64)
            d = blk.max() - blk.min()
            s16 = float(sc.view(np.float16)[k])
            b = back[g0:g0 + gs]
            half_ulp = np.spacing(np.abs(b).astype(np.float16)).astype(np.float64) / 2
            bound = d / 510 + 255 * abs(s16 - d / 255) + half_ulp + 1e-12
            assert np.all(np.abs(b - blk) <= bound)


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(4)
    v = f16(rng.standard_normal(500) + 3)
    codes, sc, off = oracle.meta_quantize(v.view(np.uint16), 128)
    for k in (-3, 2):
        w = f16(v.astype(np.float64) * 2.0 ** k)
        c2, s2, o2 = oracle.meta_quantize(w.view(np.uint16), 128)
        assert np.array_equal(codes, c2)
        assert np.array_equal(s2.view(np.float16), f16(sc.view(np.float16).astype(np.float64) * 2.0 ** k))
        assert np.array_equal(o2.view(np.float16), f16(off.view(np.float16).astype(np.float64) * 2.0 ** k))


def test_reflection():
    # v -> -v maps codes to 255 - code, except at exact ties (half-even is not symmetric)
    rng = np.random.default_rng(5)
    v = f16(rng.standard_normal(3000))
    codes, _, _ = oracle.meta_quantize(v.view(np.uint16), 0)
    c2, _, _ = oracle.meta_quantize((-v).view(np.uint16), 0)
    x = v.astype(np.float64)
    u = (x - x.min()) * 255 / (x.max() - x.min())
    tie = np.abs(u - np.floor(u) - 0.5) < 1e-6
    assert np.array_equal(c2[~tie], 255 - codes[~tie])


def test_dequantize_single_rounding():
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 256, 1000).astype(np.uint8)
    sc = f16(rng.uniform(1e-3, 0.1, 8)).view(np.uint16)
    off = f16(rng.standard_normal(8)).view(np.uint16)
    out = oracle.meta_dequantize(codes, sc, off, 128).view(np.float16)
    g = np.arange(1000) // 128
    exact = off.view(np.float16)[g].astype(np.float64) + \
        sc.view(np.float16)[g].astype(np.float64) * codes.astype(np.float64)
    assert np.array_equal(out, exact.astype(np.float16))


def test_empty_and_invalid():
    codes, sc, off = oracle.meta_quantize(np.zeros(0, np.uint16), 128)
    assert codes.size == 0 and sc.size == 0
    with pytest.raises(ValueError):
        oracle.meta_quantize(np.zeros(4, np.uint16), -1)


def _exact_half_even(x: Fraction) -> int:
    k = x.numerator // x.denominator
    rem = x - k
    return k + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1) else k


# Groups (min, max, v) whose exact quotient (v - min) * 255 / (max - min) lies off a
# half-integer by less than a binary32 half-ulp, so that rounding the quotient to binary32
# first would turn it into a tie (191.4999949... -> 191.5 -> 192, 248.5000057... -> 248.5
# -> 248).  Found by a search over exact rationals; the expected codes are computed from the
# rationals in the test.
NEAR_TIES = [(-1.3779296875, 286.25, 214.625), (-1.009765625, 170.625, 166.25),
             (-0.04083251953125, 0.0210418701171875, 5.310773849487305e-05),
             (-3.36766242980957e-05, 0.04107666015625, 0.029388427734375),
             (-0.0085906982421875, 0.0135040283203125, 3.057718276977539e-05),
             (-0.025665283203125, 0.018890380859375, 0.00010710954666137695),
             (0.00022685527801513672, 0.0225677490234375, 0.0106964111328125),
             (-0.016876220703125, 0.01096343994140625, 0.00020968914031982422),
             (-1.435546875, -0.0307769775390625, -0.64501953125),
             (-1.287109375, 1.068359375, 0.0014705657958984375),
             (-0.1456298828125, 0.7490234375, -2.944469451904297e-05),
             (0.0102386474609375, 1.3017578125, 0.89404296875),
             (-0.00853729248046875, 1.9033203125, 1.5546875),
             (-0.8896484375, 0.047882080078125, -0.0017518997192382812)]


def test_code_is_the_exact_rounding_next_to_half_integers():
    """The code is round(v/s' + z') of the affine 8-bit quantizer taken on the exact quotient:
    for each triple the exact code differs from the code of the binary32-rounded quotient."""
    v = f16(np.array(NEAR_TIES).reshape(-1))
    assert np.array_equal(v.astype(np.float64), np.array(NEAR_TIES).reshape(-1))
    codes, _, _ = oracle.meta_quantize(v.view(np.uint16), 3)
    for i, (mn, mx, x) in enumerate(NEAR_TIES):
        q = (Fraction(x) - Fraction(mn)) * 255 / (Fraction(mx) - Fraction(mn))
        exact = _exact_half_even(q)
        assert int(np.rint(np.float64(np.float32(float(q))))) != exact
        assert codes[3 * i:3 * i + 3].tolist() == [0, 255, exact]
    assert codes[:6].tolist() == [0, 255, 191, 0, 255, 249]


def test_zero_minimum_is_stored_as_plus_zero():
    # zero-point arrays hold both -0 (z = -(0 * 1/s)) and +0; min(+0, -0) has no order, so
    # the offset of a group whose minimum is zero is +0 whichever comes first
    for vals in ([-0.0, 0.0, 1.0], [0.0, -0.0, 1.0], [-0.0, 2.0, -0.0]):
        _, _, off = oracle.meta_quantize(f16(vals).view(np.uint16), 0)
        assert off[0] == 0
