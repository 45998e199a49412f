"""The GPU-vs-oracle comparison procedure (``tests/parity.py``) checked on the CPU.

The procedure must accept what a correct fp32 solver can produce -- the oracle's own
result carried in binary32, and a group that left the oracle's trajectory at a rounding
tie (made here by the oracle's tie replay, the way the device's binary32 decision
leaves it) -- and must reject results that are wrong: a divergent group whose codes or
e_best do not follow the replayed trajectory, a z off by more than the tolerance, a code
off away from a tie, and reported errors off by 1%.
"""
import numpy as np
import pytest

import oracle
from tests import parity
from tests.test_oracle_pins import NEAR_TIE_TRIPLES


def _as_device(ref, nbits):
    """The oracle's result as an fp32 solver would report it."""
    s32 = ref.scale.astype(np.float32)
    z32 = ref.zero.astype(np.float32)
    return parity.DeviceResult(
        packed=ref.packed.copy(), scale16=oracle.f64_to_f16(s32.astype(np.float64)),
        zero16=oracle.f64_to_f16(z32.astype(np.float64)), scale32=s32, zero32=z32,
        stop=ref.stop_step.copy(), err_init=ref.err_init.astype(np.float32),
        err_best=ref.err_best.astype(np.float32))


def _tie_group(seed):
    """A 16-element 4-bit group holding a near-tie triple (the exact init code and the
    binary32 one differ at element 2), whose trajectory changes when that code flips."""
    rng = np.random.default_rng(seed)
    for mn, mx, v in NEAR_TIE_TRIPLES[15] * 50:
        w = np.concatenate([[mn, mx, v], rng.uniform(mn, mx, 13)]).astype(np.float16)
        if w.min() != np.float16(mn) or w.max() != np.float16(mx):
            continue
        w = w.astype(np.float64)
        base = oracle.hqq_group(w, 4)
        flip, ztr = oracle.hqq_group_replay(w, 4, flips=((0, 2),))
        if flip.stop_step != base.stop_step or abs(flip.zero - base.zero) > 2e-3:
            return w, base, flip
    raise AssertionError("no tie group found")


def _matrix_with_tie_group():
    rng = np.random.default_rng(3)
    W = (rng.standard_t(4, (4, 64)) * 0.02).astype(np.float16)
    w, base, flip = _tie_group(5)
    W[1, 16:32] = w.astype(np.float16)
    return W, flip


def test_accepts_the_oracle_in_binary32():
    rng = np.random.default_rng(0)
    W = (rng.standard_t(4, (32, 256)) * 0.02).astype(np.float16)
    ref = oracle.hqq_quantize(W, 4, 64)
    rep = parity.compare(W, _as_device(ref, 4), 4, 64, ref=ref)
    assert rep["group_agree"] == 1.0 and rep["code_mismatch_total"] == 0


def test_divergence_at_a_rounding_tie_is_explained():
    W, flip = _matrix_with_tie_group()
    ref = oracle.hqq_quantize(W, 4, 16)
    dev = _as_device(ref, 4)
    codes = ref.codes.copy()
    codes[1, 16:32] = flip.codes
    dev.packed = oracle.pack_codes(codes, 4)
    dev.stop[1, 1] = flip.stop_step
    dev.zero32[1, 1] = np.float32(flip.zero)
    dev.zero16 = oracle.f64_to_f16(dev.zero32.astype(np.float64))
    dev.err_best[1, 1] = np.float32(flip.err_best)
    rep = parity.compare(W, dev, 4, 16, ref=ref, min_agree=0.9, min_code_agree=0.9)
    assert rep["divergent"]["rounding_tie"] == 1
    return W, ref, dev, codes


def test_divergent_group_with_wrong_codes_is_rejected():
    W, ref, dev, codes = test_divergence_at_a_rounding_tie_is_explained()
    # one code of the divergent group moved by one away from any rounding tie
    w = W[1, 16:32].astype(np.float64)
    _, inv_s, _ = oracle.minmax_init(w, 4)
    _, flip_z = dev.stop[1, 1], float(dev.zero32[1, 1])
    pre = w * inv_s + flip_z
    far = int(np.argmax(np.abs(np.abs(pre - np.floor(pre)) - 0.5)))
    bad = codes.copy()
    bad[1, 16 + far] = bad[1, 16 + far] + 1 if bad[1, 16 + far] < 15 else bad[1, 16 + far] - 1
    dev.packed = oracle.pack_codes(bad, 4)
    with pytest.raises(AssertionError):
        parity.compare(W, dev, 4, 16, ref=ref, min_agree=0.9, min_code_agree=0.9)


def test_divergent_group_with_wrong_error_is_rejected():
    W, ref, dev, codes = test_divergence_at_a_rounding_tie_is_explained()
    dev.err_best[1, 1] *= np.float32(1.01)
    with pytest.raises(AssertionError):
        parity.compare(W, dev, 4, 16, ref=ref, min_agree=0.9, min_code_agree=0.9)


def test_wrong_z_code_and_errors_are_rejected():
    rng = np.random.default_rng(1)
    W = (rng.standard_t(4, (16, 256)) * 0.02).astype(np.float16)
    ref = oracle.hqq_quantize(W, 4, 64)
    # z off by 2e-3 in one group (same stop step): neither agreeing nor explainable
    dev = _as_device(ref, 4)
    dev.zero32[3, 2] += np.float32(2e-3)
    dev.zero16 = oracle.f64_to_f16(dev.zero32.astype(np.float64))
    with pytest.raises(AssertionError):
        parity.compare(W, dev, 4, 64, ref=ref, min_agree=0.9)
    # a code off by one away from a tie in an agreeing group
    dev = _as_device(ref, 4)
    codes = ref.codes.copy()
    w = W[0, :64].astype(np.float64)
    _, inv_s, _ = oracle.minmax_init(w, 4)
    pre = w * inv_s + ref.zero[0, 0]
    far = int(np.argmax(np.abs(np.abs(pre - np.floor(pre)) - 0.5) * (ref.codes[0, :64] < 15)))
    codes[0, far] += 1
    dev.packed = oracle.pack_codes(codes, 4)
    with pytest.raises(AssertionError):
        parity.compare(W, dev, 4, 64, ref=ref, min_code_agree=0.99)
    # reported e_best off by 1% in 1% of the groups
    dev = _as_device(ref, 4)
    dev.err_best.reshape(-1)[::50] *= np.float32(1.01)
    with pytest.raises(AssertionError):
        parity.compare(W, dev, 4, 64, ref=ref)
