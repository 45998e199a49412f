"""GPU-vs-oracle comparison procedure (test infrastructure).

Tolerances (fp32 device solver against the fp64 oracle on the same fp16 bits):
  * s: |s32 - s64| / s64 <= 1e-6; binary16 s bit-equal, or 1 ulp apart where
    s64 lies within 1e-6 (relative) of a binary16 rounding midpoint;
  * a group agrees when its stop step t* is identical and |z32 - z64| <= 1e-3
    code units; >= 99.9% of the groups must agree; binary16 z of an agreeing
    group is within 1 ulp of the binary16 cast of z64;
  * codes: >= 99.99% equal overall; in agreeing groups every mismatch is
    |delta| = 1 at a rounding tie (the oracle's w/s + z within 2e-3 code units of
    a half-integer);
  * every group that does not agree must be explained (``explain_divergence``):
    replaying the oracle with at most four tie events reproduces the device's t*,
    z (within 1e-3), codes (equal, or |delta| = 1 at a rounding tie of the
    replay's z) and e_best (within 1e-4).  A tie event is either a rounding tie
    (an element whose pre-round value lies within 8 binary32 ulps of a rounding
    boundary -- within the device's working precision -- takes the other
    neighbour) or an error tie (the stop test of an evaluation whose error equals
    the best so far to within 1e-5 is inverted).  A single code flip moves the
    next z by 1/G, so fp32 and fp64 trajectories part at such ties; the replay
    shows that this, and nothing else, happened.  With p = 1 the error is
    piecewise linear in z and runs of exactly equal errors are common, so the
    p = 1 cases use a lower agreement floor; their divergent groups must still
    all be explained;
  * the reported errors e_0 and e_best (debug outputs, weight units) agree with the
    oracle's to 1e-4 relative in >= 99.9% of the agreeing groups.

The oracle decides the codes of the first evaluation exactly and later ones on fp64
values; the device decides all of them on binary32 values.  Codes whose exact value
lies within a binary32 rounding of a half-integer can therefore differ by one; the
tie band above covers them, and ``compare`` reports how many there were.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import oracle

S_REL = 1e-6
Z_ABS = 1e-3
TIE_BAND = 2e-3
STOP_AGREE = 0.999
CODE_AGREE = 0.9999
FLIP_REL = 1e-5
ERR_REL = 1e-4


@dataclass
class DeviceResult:
    packed: np.ndarray      # uint8
    scale16: np.ndarray     # uint16 bits, rows x ng
    zero16: np.ndarray      # uint16 bits
    scale32: np.ndarray | None = None
    zero32: np.ndarray | None = None
    stop: np.ndarray | None = None
    err_init: np.ndarray | None = None
    err_best: np.ndarray | None = None


def from_quantized(q) -> DeviceResult:
    """Copy a QuantizedWeight (torch, device) to host numpy arrays."""
    def h(t):
        return None if t is None else t.cpu().numpy()
    return DeviceResult(packed=h(q.packed), scale16=h(q.scale).view(np.uint16),
                        zero16=h(q.zero).view(np.uint16), scale32=h(q.scale_f32),
                        zero32=h(q.zero_f32), stop=h(q.stop_step), err_init=h(q.err_init),
                        err_best=h(q.err_best))


def _ulp_distance16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in binary16 ulps between bit patterns (sign-magnitude ordered)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(key(a) - key(b))


def _near_f16_midpoint(v: np.ndarray, rel: float) -> np.ndarray:
    lo = oracle.f64_to_f16(v * (1 - rel))
    hi = oracle.f64_to_f16(v * (1 + rel))
    return lo != hi


def compare(W16: np.ndarray, dev: DeviceResult, nbits: int, group_size: int, p=0.7, beta=1.0,
            kappa=1.01, iters=20, early_stop=True, ref=None, strict_ties_only=True,
            min_agree=STOP_AGREE, min_code_agree=CODE_AGREE, err_pow=None) -> dict:
    """Assert the tolerances above for rows x cols binary16 input bits W16."""
    W16 = np.ascontiguousarray(W16).view(np.uint16)
    rows, cols = W16.shape
    qmax = (1 << nbits) - 1
    if ref is None:
        ref = oracle.hqq_quantize(W16, nbits, group_size, p=p, beta=beta, kappa=kappa, iters=iters,
                                  early_stop=early_stop, err_pow=err_pow)
    rep = {"groups": ref.scale.size, "weights": W16.size}

    # ---- s
    if dev.scale32 is not None:
        rel = np.abs(dev.scale32.astype(np.float64) - ref.scale) / ref.scale
        assert rel.max() <= S_REL, f"s rel err {rel.max():.3g}"
    if dev.scale32 is not None:
        assert np.array_equal(dev.scale16, oracle.f64_to_f16(dev.scale32.astype(np.float64))), \
            "binary16 s is not the round-to-nearest-even cast of s32"
    d = _ulp_distance16(dev.scale16, ref.scale_f16)
    assert d.max() <= 1, "binary16 s off by more than 1 ulp"
    bad = (d == 1) & ~_near_f16_midpoint(ref.scale, S_REL)
    assert not bad.any(), f"binary16 s differs away from a rounding midpoint in {bad.sum()} groups"
    rep["s16_ulp1"] = int((d == 1).sum())

    # ---- per-group agreement: same stop step and |z32 - z64| <= Z_ABS
    same_t = np.ones(ref.stop_step.shape, bool) if dev.stop is None else dev.stop == ref.stop_step
    agree = same_t.copy()
    if dev.zero32 is not None:
        dz = np.abs(dev.zero32.astype(np.float64) - ref.zero)
        agree &= dz <= Z_ABS
        rep["z_maxdiff"] = float(dz[agree].max(initial=0.0))
    rep["stop_agree"] = float(same_t.mean())
    rep["group_agree"] = float(agree.mean())
    assert agree.mean() >= min_agree, f"group agreement {agree.mean():.5f}"
    # binary16 z is the RNE cast of the device's z32 (and z32 is within Z_ABS of z64)
    if dev.zero32 is not None:
        assert np.array_equal(dev.zero16, oracle.f64_to_f16(dev.zero32.astype(np.float64))), \
            "binary16 z is not the round-to-nearest-even cast of z32"
    dz16 = _ulp_distance16(dev.zero16, ref.zero_f16)
    big = np.abs(ref.zero) >= 1.0  # where one binary16 ulp is at least 2^-10
    assert dz16[agree & big].max(initial=0) <= 1, "binary16 z off by more than 1 ulp"

    # ---- codes
    codes = oracle.unpack_codes(dev.packed, rows * cols, nbits).reshape(rows, cols)
    eq = codes == ref.codes
    rep["code_agree"] = float(eq.mean())
    assert eq.mean() >= min_code_agree, f"code agreement {eq.mean():.6f}"
    agree_el = np.repeat(agree, group_size, axis=1)
    mism = ~eq & agree_el
    Wd = oracle.f16_to_f64(W16).reshape(rows, -1, group_size)
    if mism.any():
        r_i, c_i = np.nonzero(mism)
        g_i = c_i // group_size
        w = oracle.f16_to_f64(W16[r_i, c_i])
        inv_s = np.array([oracle.minmax_init(Wd[a, b], nbits)[1] for a, b in zip(r_i, g_i)])
        pre = w * inv_s + ref.zero[r_i, g_i]
        tie = np.abs(pre - np.floor(pre) - 0.5) <= TIE_BAND
        delta = np.abs(codes[mism].astype(int) - ref.codes[mism].astype(int))
        assert (delta == 1).all(), "code mismatch larger than 1"
        if strict_ties_only:
            assert tie.all(), f"{(~tie).sum()} code mismatches away from a rounding tie"
    rep["code_mismatch_agreeing"] = int(mism.sum())
    rep["code_mismatch_total"] = int((~eq).sum())

    # ---- groups that left the oracle's trajectory: each must be explained
    kinds = {"error_tie": 0, "rounding_tie": 0}
    params = dict(p=p, beta=beta, kappa=kappa, iters=iters, early_stop=early_stop, err_pow=err_pow)
    for (i, j) in np.argwhere(~agree):
        assert dev.zero32 is not None and dev.stop is not None, "divergent group without debug outputs"
        kind = explain_divergence(Wd[i, j], nbits, int(dev.stop[i, j]), float(dev.zero32[i, j]),
                                  codes[i, j * group_size:(j + 1) * group_size], params,
                                  None if dev.err_best is None else float(dev.err_best[i, j]))
        assert kind is not None, (f"group {(i, j)}: device t*={dev.stop[i, j]} z={dev.zero32[i, j]} "
                                  f"vs oracle t*={ref.stop_step[i, j]} z={ref.zero[i, j]} unexplained")
        kinds[kind] += 1
    rep["divergent"] = kinds

    # ---- reported errors (debug outputs): fp32 sums of hardware log2/exp2 terms
    for name, dv, rv in (("err_init", dev.err_init, ref.err_init),
                         ("err_best", dev.err_best, ref.err_best)):
        if dv is None:
            continue
        ok = np.abs(dv.astype(np.float64) - rv) <= ERR_REL * np.maximum(rv, 1e-6)
        rep[f"{name}_off"] = int((~ok & agree).sum())
        assert ok[agree].mean() >= STOP_AGREE, f"{name} agreement {ok[agree].mean():.5f}"
    return rep


def _near_ties(w, inv_s, z, qmax, window_ulps=8.0):
    """Elements whose pre-round value lies within a few binary32 ulps (the device's working
    precision) of a rounding boundary."""
    x = w * inv_s + z
    dist = np.abs(np.abs(x - np.floor(x)) - 0.5)
    win = window_ulps * 2.0 ** -23 * np.maximum(np.abs(x), 1.0)
    inside = (x > -0.5 - win) & (x < qmax + 0.5 + win)
    idx = np.nonzero((dist <= win) & inside)[0]
    return idx[np.argsort(dist[idx])]


def _error_at(w, nbits, z, p):
    s64, inv_s64, _ = oracle.minmax_init(w, nbits)
    qmax = (1 << nbits) - 1
    q = np.array([oracle.quantize_value(x, inv_s64, z, qmax) for x in w])
    return oracle.group_error(w - s64 * (q - z), p)


def _codes_match(w, inv_s, z, qmax, dev_codes, ref_codes):
    """Device codes equal the reference codes at z, except |delta| = 1 where the pre-round
    value w/s + z lies within TIE_BAND of a half-integer."""
    dc, rc = np.asarray(dev_codes, np.int64), np.asarray(ref_codes, np.int64)
    diff = dc != rc
    if not diff.any():
        return True
    pre = w[diff] * inv_s + z
    tie = np.abs(pre - np.floor(pre) - 0.5) <= TIE_BAND
    return bool((np.abs(dc[diff] - rc[diff]) == 1).all() and tie.all())


def explain_divergence(w, nbits, dev_t, dev_z, dev_codes, params, dev_err_best=None,
                       max_events=4):
    """Why a device group left the oracle's trajectory, or None if unexplained.

    Replays the oracle with at most `max_events` tie events and looks for the device's
    stop step, z (within Z_ABS), codes (equal, or one apart at a rounding tie of the
    replay's z) and e_best (within ERR_REL, when the device reported it).  Events are
    (a) a rounding tie: an element whose pre-round value lies within 8 binary32 ulps of
    a rounding boundary gets the other neighbour; (b) an error tie: an evaluation whose
    error equals the best error so far to within FLIP_REL has its stop decision
    inverted.  Returns "error_tie" if only events of kind (b) were needed, else
    "rounding_tie"."""
    qmax = (1 << nbits) - 1
    _, inv_s, _ = oracle.minmax_init(w, nbits)

    def run(flips, inverts):
        return oracle.hqq_group_replay(w, nbits, flips, inverts, **params)

    def matches(res):
        if res.stop_step != dev_t or abs(res.zero - dev_z) > Z_ABS:
            return False
        if not _codes_match(w, inv_s, res.zero, qmax, dev_codes, res.codes):
            return False
        if dev_err_best is not None and \
                abs(dev_err_best - res.err_best) > ERR_REL * max(res.err_best, 1e-6):
            return False
        return True

    def events(res, ztr, after):
        ev = []
        for t in range(max(after, 1), len(res.trace)):
            prev = np.min(res.trace[:t])
            if abs(res.trace[t] - prev) <= FLIP_REL * max(prev, 1e-30):
                ev.append(("inv", t, -1))
        for t in range(after, len(ztr)):
            for k in _near_ties(w, inv_s, ztr[t], qmax)[:4]:
                ev.append(("flip", t, int(k)))
        return ev

    frontier = [((), ())]
    for _depth in range(max_events):
        nxt = []
        for flips, inverts in frontier:
            res, ztr = run(flips, inverts)
            after = max([f[0] for f in flips] + [v for v in inverts] + [0])
            for kind, t, k in events(res, ztr, after):
                f2 = flips + ((t, k),) if kind == "flip" else flips
                i2 = inverts + (t,) if kind == "inv" else inverts
                r2, _ = run(f2, i2)
                if matches(r2):
                    return "error_tie" if not f2 else "rounding_tie"
                nxt.append((f2, i2))
        frontier = nxt[:24]
    return None
