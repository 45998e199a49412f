"""GPU parity of the 8-bit meta quantization (through the C ABI) against the oracle.

The meta codes are the exact half-even rounding of (v - min) 255 / (max - min) on
both sides, and the meta scale, offset and dequantized values are single roundings
of exact values, so every output is compared bit for bit: on the s and z arrays the
solver produces for workload matrices (z as one group per array, s in groups of
128), on ragged group counts, and on edge cases (constant arrays, +0/-0 minima, one
value, groups of 1, 3, 5 and 1000 values, binary16 triples whose ratio lies off a
half-integer by less than a binary32 rounding, and triples whose ratio is on a
half-integer or within 2^-11 of one -- on both sides of the margin at which the
kernels leave the group's reciprocal for the exact comparison -- including groups
whose minimum is near -6e4 next to values near 2^-14, and groups a few binary16
ulps wide).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.test_oracle_meta_pins import NEAR_TIES

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    import bit_weight_quantization_amd as m
    m.load_library()
    return m


def _say(msg):
    print(f"[gpu-meta] {msg}", flush=True)


def _check(hq, values16: np.ndarray, group: int):
    """Meta-quantize binary16 bit patterns on the GPU and compare with the oracle."""
    v = torch.from_numpy(values16.view(np.int16).copy()).view(torch.float16).cuda()
    m = hq.meta_quantize(v, group)
    back = hq.meta_dequantize(m)
    torch.cuda.synchronize()
    codes, sc, off = oracle.meta_quantize(values16, group)
    assert np.array_equal(m.codes.cpu().numpy(), codes)
    assert np.array_equal(m.scale.cpu().numpy().view(np.uint16), sc)
    assert np.array_equal(m.offset.cpu().numpy().view(np.uint16), off)
    ref = oracle.meta_dequantize(codes, sc, off, group)
    assert np.array_equal(back.cpu().numpy().view(np.uint16), ref)
    return m


@pytest.mark.parametrize("name,nbits,g", [("attn_4096x4096", 4, 64), ("single_256x512", 4, 64),
                                         ("mlp_11008x4096", 2, 16)])
def test_meta_of_solver_outputs(hq, name, nbits, g):
    wl = workloads.WORKLOADS[name]
    _say(f"{name} b{nbits} g{g}: z whole-array, s groups of 128")
    W = workloads.generate_matrix(wl, 0, "cuda")
    q = hq.quantize(W, nbits, g)
    torch.cuda.synchronize()
    z16 = q.zero.cpu().numpy().view(np.uint16).ravel()
    s16 = q.scale.cpu().numpy().view(np.uint16).ravel()
    mz = _check(hq, z16, 0)
    ms = _check(hq, s16, 128)
    # the full dequantization from the meta-dequantized s and z, against the oracle's
    zb = hq.meta_dequantize(mz).view(q.zero.shape)
    sb = hq.meta_dequantize(ms).view(q.scale.shape)
    qm = hq.QuantizedWeight(packed=q.packed, scale=sb, zero=zb, rows=q.rows, cols=q.cols,
                            nbits=nbits, group_size=g)
    Wd = hq.dequantize(qm)
    torch.cuda.synchronize()
    rows = min(q.rows, 256)
    ref = oracle.hqq_dequantize(q.packed.cpu().numpy()[: rows * q.cols * nbits // 8],
                                sb.cpu().numpy()[:rows], zb.cpu().numpy()[:rows], rows, q.cols,
                                nbits, g)
    assert np.array_equal(Wd[:rows].cpu().numpy().view(np.uint16), ref)


def test_meta_of_largest_70b_matrix(hq):
    wl = workloads.WORKLOADS["llama70b_stack"]
    m = wl.matrices[6]  # 8192 x 28672
    _say(f"70B {m.rows}x{m.cols} b2 g32: z whole-array ({m.rows * m.cols // 32} values), s g128")
    W = workloads.generate(m.rows, m.cols, wl.dist, m.seed, "cuda")
    q = hq.quantize(W, 2, 32)
    torch.cuda.synchronize()
    _check(hq, q.zero.cpu().numpy().view(np.uint16).ravel(), 0)
    _check(hq, q.scale.cpu().numpy().view(np.uint16).ravel(), 128)


def test_meta_ragged_and_small_groups(hq):
    rng = np.random.default_rng(7)
    _say("ragged group counts, groups of 1, 3, 5, 1000")
    W = workloads.generate(1001, 80, workloads.WORKLOADS["mlp_11008x4096"].dist, 77, "cuda")
    q = hq.quantize(W, 2, 16)  # 5005 groups: 39 full meta groups of 128 and one of 13
    torch.cuda.synchronize()
    _check(hq, q.scale.cpu().numpy().view(np.uint16).ravel(), 128)
    _check(hq, q.zero.cpu().numpy().view(np.uint16).ravel(), 0)
    v = np.asarray(rng.standard_normal(5003) * 4, np.float16).view(np.uint16)
    for group in (1, 3, 5, 64, 65, 1000, 4096):  # n % 8 != 0: the per-value kernels
        _check(hq, v, group)
    v8 = np.asarray(rng.standard_normal(5008) * 4, np.float16).view(np.uint16)
    for group in (0, 16, 32, 64, 128):  # the 8-values-per-lane kernels, ragged last group
        _check(hq, v8, group)


def test_meta_edge_cases(hq):
    f16 = lambda x: np.asarray(x, np.float16).view(np.uint16)
    _say("constant, +0/-0, single value, ties off by less than a binary32 rounding")
    _check(hq, f16([0.75] * 300), 0)
    _check(hq, f16([0.75] * 300), 128)
    _check(hq, f16([-0.0, 0.0, 1.0, -0.0]), 0)
    _check(hq, f16([0.0, -0.0, 2.0, 3.0, -0.0, 0.0]), 3)
    _check(hq, f16([3.5]), 0)
    _check(hq, f16(np.array(NEAR_TIES).reshape(-1)), 3)
    _check(hq, f16([0, 255, 2.5, 3.5, 4.5, 0.5, 1.5, 254.5]), 0)
    _check(hq, f16([-1, 0, 0.5, 2]), 0)


def test_meta_empty(hq):
    v = torch.empty(0, dtype=torch.float16, device="cuda")
    m = hq.meta_quantize(v, 0)
    assert m.codes.numel() == 0 and m.scale.numel() == 0


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 32)])
def test_meta_batch_equals_per_matrix(hq, nbits, g):
    """hqq_meta_quantize_batch over a quantize_batch arena equals hqq_meta_quantize on each
    matrix's slice (z: one group per matrix, with empty and tiny entries and blocks that
    span several entries; s: groups of 128 where every group count is a multiple of 128)."""
    _say(f"hqq_meta_quantize_batch vs per-matrix hqq_meta_quantize, b{nbits} g{g}")
    dist = workloads.WORKLOADS["attn_4096x4096"].dist
    shapes = [(37, 5 * g), (0, g), (1, g), (1024, 64 * g), (3, g), (2049, g), (4096, 4096)]
    Ws = [workloads.generate(r, c, dist, 500 + i, "cuda") if r * c else
          torch.empty((r, c), dtype=torch.float16, device="cuda") for i, (r, c) in enumerate(shapes)]
    b = hq.quantize_batch(Ws, nbits, g)
    mz = hq.meta_quantize_batch(b, "zero", 0)
    torch.cuda.synchronize()
    for i, (r, c) in enumerate(shapes):
        g0, ng = b.first_group[i], r * c // g
        if ng == 0:
            continue
        one = hq.meta_quantize(b.zero[g0:g0 + ng].contiguous(), 0)
        torch.cuda.synchronize()
        assert torch.equal(mz.codes[g0:g0 + ng], one.codes)
        assert torch.equal(mz.scale[i:i + 1].view(torch.int16), one.scale.view(torch.int16))
        assert torch.equal(mz.offset[i:i + 1].view(torch.int16), one.offset.view(torch.int16))
    # scales: a 70B layer, every matrix's group count a multiple of 128
    wl = workloads.WORKLOADS["llama70b_stack"]
    Ws = [workloads.generate(m.rows, m.cols, wl.dist, m.seed, "cuda") for m in wl.matrices[:7]]
    b = hq.quantize_batch(Ws, nbits, g)
    ms = hq.meta_quantize_batch(b, "scale", 128)
    mz = hq.meta_quantize_batch(b, "zero", 0)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        g0, ng = b.first_group[i], W.numel() // g
        one_s = hq.meta_quantize(b.scale[g0:g0 + ng].contiguous(), 128)
        one_z = hq.meta_quantize(b.zero[g0:g0 + ng].contiguous(), 0)
        torch.cuda.synchronize()
        assert torch.equal(ms.codes[g0:g0 + ng], one_s.codes)
        assert torch.equal(ms.scale[g0 // 128:(g0 + ng) // 128].view(torch.int16),
                           one_s.scale.view(torch.int16))
        assert torch.equal(mz.codes[g0:g0 + ng], one_z.codes)
        assert torch.equal(mz.offset[i:i + 1].view(torch.int16), one_z.offset.view(torch.int16))


BANDS = ((0.0, 0.0), (0.0, 2.0 ** -15), (2.0 ** -15, 2.0 ** -12), (2.0 ** -12, 2.0 ** -11))


def _near_half_triples(seed, want, draw, bands=BANDS):
    """binary16 triples (min, max, v) from ``draw(rng, n)`` whose ratio
    (v - min) 255 / (max - min) is on a half-integer or within 2^-11 of one, ``want`` of
    each distance band in ``bands``: exactly on it, within 2^-15, from 2^-15 to 2^-12
    (just inside the kernels' margin) and from 2^-12 to 2^-11 (just outside it)."""
    rng = np.random.default_rng(seed)
    found = [[] for _ in bands]
    for _ in range(200):
        if min(len(f) for f in found) >= want:
            break
        a = draw(rng, 1 << 20)
        a = a[np.isfinite(a).all(axis=1)]
        lo = np.minimum(a[:, 0], a[:, 1]).astype(np.float64)
        hi = np.maximum(a[:, 0], a[:, 1]).astype(np.float64)
        v = a[:, 2].astype(np.float64)
        ok = (hi > lo) & (v >= lo) & (v <= hi)
        u = (v - lo) * 255.0 / np.where(ok, hi - lo, 1.0)
        off = np.abs(u - np.floor(u) - 0.5)
        trip = np.stack([lo, hi, v], axis=1).astype(np.float16)
        for f, (b0, b1) in zip(found, bands):
            sel = ok & (off == 0.0) if b1 == 0.0 else ok & (off > b0) & (off < b1)
            f += list(trip[sel][:max(want - len(f), 0)])
    assert min(len(f) for f in found) >= want, [len(f) for f in found]
    return [np.array(f[:want]) for f in found]


def _draw_normal(rng, n):
    return rng.standard_normal((n, 3)).astype(np.float16)


def _draw_mixed_magnitudes(rng, n):
    """A minimum near -6e4 beside values near 2^-14: v - min rounds in fp32."""
    lo = -rng.uniform(2e4, 6.5e4, n)
    hi = rng.uniform(-1.0, 50.0, n)
    v = rng.standard_normal(n) * 2.0 ** -14
    return np.stack([lo, hi, v], axis=1).astype(np.float16)


@pytest.mark.parametrize("draw,bands", [(_draw_normal, BANDS),
                                        (_draw_mixed_magnitudes, BANDS[1:])])
def test_meta_codes_at_and_near_half_integers(hq, draw, bands):
    """Ratios on a half-integer or up to 2^-11 from one, in groups of three: the codes must
    match the exact definition bit for bit on both sides of the kernels' 2^-12 margin (the
    mixed-magnitude draw has no exact ties)."""
    found = _near_half_triples(7, 64, draw, bands)
    vals = np.concatenate(found).reshape(-1).view(np.uint16)
    _check(hq, vals, 3)
    _say(f"{draw.__name__}: {[len(b) for b in found]} triples per band {bands}: bit-exact")


def test_meta_codes_of_narrow_groups(hq):
    """Groups a few binary16 ulps wide (d tiny, so fl32(255/d) is large): ratios k 255 / m
    with small m, exact ties among them."""
    rng = np.random.default_rng(8)
    groups = []
    for _ in range(512):
        base = np.float16(rng.standard_normal() * 10.0 ** rng.uniform(-4, 4))
        if not np.isfinite(base):
            continue
        m = int(rng.integers(1, 12))
        steps = np.concatenate([[0, m], rng.integers(0, m + 1, 6)])
        vals = base.view(np.uint16).astype(np.int64) + np.where(base >= 0, steps, -steps)
        grp = vals.astype(np.uint16)
        if np.isfinite(grp.view(np.float16)).all():
            groups.append(grp)
    vals = np.concatenate(groups)
    _check(hq, vals, 8)
    _say(f"{len(groups)} groups of 8 values at most 11 ulps apart: bit-exact")
