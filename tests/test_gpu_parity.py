"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs are seeded synthetic matrices with the shapes and distributions of the
workload table in ``workloads``; both sides read the same fp16 bits.  Small
matrices are compared in full; full-size matrices of the 7B/70B stacks are
quantized whole (the call the benchmark times) and compared on sampled rows,
which the oracle computes on its own (rows are independent).  Tolerances are in
``tests/parity.py``.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import parity

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
    print(f"[gpu-parity] {msg}", flush=True)


def _run(hq, W, nbits, g, **kw):
    q = hq.quantize(W, nbits, g, debug=True, **kw)
    torch.cuda.synchronize()
    return q


def _check_full(hq, W, nbits, g, p=0.7, beta=1.0, kappa=1.01, iters=20, early_stop=True,
                **floors):
    q = _run(hq, W, nbits, g, p=p, beta=beta, kappa=kappa, iters=iters, early_stop=early_stop)
    dev = parity.from_quantized(q)
    W16 = W.cpu().numpy().view(np.uint16)
    rep = parity.compare(W16, dev, nbits, g, p=p, beta=beta, kappa=kappa, iters=iters,
                         early_stop=early_stop, **floors)
    _say(f"  {rep}")
    return q, rep


def _sample_rows(rows, seed, n=62):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, rows - 1), size=min(n, rows - 2), replace=False)
    return np.unique(np.concatenate([[0, rows - 1], mid]))


def _check_sampled(hq, W, nbits, g, seed, **kw):
    """Quantize the whole matrix on the GPU, compare sampled rows against the oracle."""
    q = _run(hq, W, nbits, g, **kw)
    rows, cols = W.shape
    idx = _sample_rows(rows, seed)
    it = torch.as_tensor(idx, device=W.device)
    ngr = cols // g
    bytes_per_row = cols * nbits // 8
    packed = q.packed.view(rows, bytes_per_row)[it].cpu().numpy().ravel()
    dev = parity.DeviceResult(
        packed=packed, scale16=q.scale[it].cpu().numpy().view(np.uint16),
        zero16=q.zero[it].cpu().numpy().view(np.uint16), scale32=q.scale_f32[it].cpu().numpy(),
        zero32=q.zero_f32[it].cpu().numpy(), stop=q.stop_step[it].cpu().numpy(),
        err_init=q.err_init[it].cpu().numpy(), err_best=q.err_best[it].cpu().numpy())
    assert dev.scale16.shape == (len(idx), ngr)
    W16 = W[it].cpu().numpy().view(np.uint16)
    rep = parity.compare(W16, dev, nbits, g, **kw)
    _say(f"  sampled {len(idx)} rows: {rep}")
    return rep


# ------------------------------------------------------------- workloads --

def test_single_256x512_full(hq):
    wl = workloads.WORKLOADS["single_256x512"]
    _say("single_256x512 b4 g64 seed 1")
    W = workloads.generate_matrix(wl, 0, "cuda")
    _check_full(hq, W, 4, 64)


def test_attn_4096x4096_full(hq):
    wl = workloads.WORKLOADS["attn_4096x4096"]
    _say("attn_4096x4096 b4 g64 seed 2")
    W = workloads.generate_matrix(wl, 0, "cuda")
    _check_full(hq, W, 4, 64)


@pytest.mark.parametrize("nbits,g", [(2, 16), (2, 32)])
def test_mlp_11008x4096(hq, nbits, g):
    wl = workloads.WORKLOADS["mlp_11008x4096"]
    _say(f"mlp 11008x4096 (full) and 4096x11008 (sampled) b{nbits} g{g} seeds 3, 4")
    W = workloads.generate_matrix(wl, 0, "cuda")
    _check_full(hq, W, nbits, g)
    W = workloads.generate_matrix(wl, 1, "cuda")
    _check_sampled(hq, W, nbits, g, seed=4)


@pytest.mark.parametrize("nbits,g", [(4, 64), (3, 64)])
def test_llama7b_stack_sampled(hq, nbits, g):
    wl = workloads.WORKLOADS["llama7b_stack"]
    for m in (0, 4, 6, 7 * 31 + 5):  # 4096x4096, 11008x4096, 4096x11008 (layer 0), 11008x4096 (layer 31)
        mat = wl.matrices[m]
        _say(f"llama7b matrix {m} {mat.rows}x{mat.cols} seed {mat.seed} b{nbits} g{g}")
        W = workloads.generate_matrix(wl, m, "cuda")
        _check_sampled(hq, W, nbits, g, seed=mat.seed)


@pytest.mark.parametrize("nbits,g", [(2, 32), (4, 64)])
def test_llama70b_stack_sampled(hq, nbits, g):
    wl = workloads.WORKLOADS["llama70b_stack"]
    for m in (0, 2, 4, 6, 7 * 79 + 4):  # 8192^2, 1024x8192, 28672x8192, 8192x28672, last layer
        mat = wl.matrices[m]
        _say(f"llama70b matrix {m} {mat.rows}x{mat.cols} seed {mat.seed} b{nbits} g{g}")
        W = workloads.generate_matrix(wl, m, "cuda")
        _check_sampled(hq, W, nbits, g, seed=mat.seed)
        del W
        torch.cuda.empty_cache()


# ---------------------------------------------------- branches and extremes --

def _c1(device="cuda"):
    return workloads.generate_matrix(workloads.WORKLOADS["single_256x512"], 0, device)


# With 8-bit codes the code grid is 16-64 times finer relative to a binary32 ulp than at
# 2-4 bits, so after the first update (where the device's binary32 iterate u + delta and
# the oracle's fp64 value are two approximations of the same step) pre-round values fall
# within that noise of a half-integer correspondingly more often, and a few groups in a
# thousand take another path.  The floor is 99.5% there; every such group must still be
# explained by the tie replay.
BITS8_FLOOR = dict(min_agree=0.995)


@pytest.mark.parametrize("nbits,g", [(8, 64), (3, 64), (4, 128), (4, 16), (8, 128), (3, 16)])
def test_bits_and_group_sizes(hq, nbits, g):
    _say(f"single_256x512 b{nbits} g{g}")
    _check_full(hq, _c1(), nbits, g, **(BITS8_FLOOR if nbits == 8 else {}))


def test_active_shrink_large_beta(hq):
    _say("single_256x512 beta=1e4 (shrink active)")
    _check_full(hq, _c1(), 4, 64, beta=1e4)
    _check_full(hq, _c1(), 2, 32, beta=3e3, kappa=1.1)


def test_scaled_weights(hq):
    _say("single_256x512 x50 (shrink active near outliers)")
    W = (_c1().float() * 50).half()
    _check_full(hq, W, 4, 64)
    _check_full(hq, W, 2, 16)


@pytest.mark.parametrize("p", [1.0, 0.0, 0.5])
def test_other_p(hq, p):
    """p = 1 (l1, soft-threshold shrink) and p = 0 (l0) are the ends of the range the page
    allows.  The l1 error is piecewise linear in z: runs of exactly equal errors make the
    stop test a coin toss between fp32 and fp64, so p = 1 only needs 75% of the groups on
    the oracle's exact trajectory, and every other group explained as a tie."""
    _say(f"single_256x512 p={p}")
    floors = dict(min_agree=0.75, min_code_agree=0.999) if p == 1.0 else {}
    _check_full(hq, _c1(), 4, 64, p=p, **floors)
    _check_full(hq, _c1(), 2, 32, p=p, beta=1e3, **floors)


@pytest.mark.parametrize("err_metric,err_pow,floors", [(1, 1.0, dict(min_agree=0.95)),
                                                      (2, 2.0, dict(min_agree=0.99))])
def test_error_metric_variants(hq, err_metric, err_pow, floors):
    """The l1 and l2 early-stop errors (hqq_options_t.err_metric) against the oracle's
    err_pow switch; the shrink keeps p = 0.7.  With codes fixed, the z update is the exact
    l2 minimizer, so consecutive l2 errors sit on a flat quadratic minimum and differ by
    amounts at fp32 noise level: the stop floor is lower (as for p = 1), and every
    divergent group must still be explained as an error or rounding tie."""
    for name in ("single_256x512", "attn_4096x4096"):
        _say(f"{name} b4 g64, early-stop error l{err_metric}")
        W = workloads.generate_matrix(workloads.WORKLOADS[name], 0, "cuda")
        q = _run(hq, W, 4, 64, err_metric=err_metric)
        rep = parity.compare(W.cpu().numpy().view(np.uint16), parity.from_quantized(q), 4, 64,
                             err_pow=err_pow, **floors)
        _say(f"  {rep}")


def test_no_early_stop_and_zero_iters(hq):
    _say("single_256x512 early_stop=0 T=20; T=0; T=255")
    _check_full(hq, _c1(), 4, 64, early_stop=False)
    _check_full(hq, _c1(), 4, 64, iters=0)
    _check_full(hq, _c1(), 3, 32, iters=255)


def test_ragged_shapes(hq):
    """Group counts that fill no whole wavefront or queue; one row; one group."""
    dist = workloads.WORKLOADS["attn_4096x4096"].dist
    for rows, cols, nbits, g, seed in [(37, 96, 4, 32, 11), (1, 16, 2, 16, 12), (3, 128, 3, 128, 13),
                                       (1001, 80, 4, 16, 14), (5, 4224, 8, 64, 15),
                                       (2049, 64, 2, 64, 16)]:
        _say(f"ragged {rows}x{cols} b{nbits} g{g} seed {seed}")
        W = workloads.generate(rows, cols, dist, seed, "cuda")
        _check_full(hq, W, nbits, g)


def test_constant_same_sign_and_grid_groups(hq):
    _say("constant / same-sign / on-grid groups")
    rng = np.random.default_rng(0)
    rows, cols = 64, 256
    W = np.empty((rows, cols), np.float16)
    W[:16] = np.repeat(rng.standard_normal((16, 4)) * 0.02, 64, axis=1)            # constant groups
    W[16:32] = np.abs(rng.standard_normal((16, cols)) * 0.02) + 0.01               # all positive
    W[32:48] = -np.abs(rng.standard_normal((16, cols)) * 0.02) - 0.01              # all negative
    k = rng.integers(0, 16, (16, cols)).astype(np.float64)
    k[:, ::64] = 0
    k[:, 1::64] = 15
    W[48:] = (0.5 * (k - 3.0)).astype(np.float16)                                 # on a code grid
    Wt = torch.from_numpy(W).cuda()
    q, _ = _check_full(hq, Wt, 4, 64)
    ref = oracle.hqq_quantize(W, 4, 64)
    codes = oracle.unpack_codes(q.packed.cpu().numpy(), rows * cols, 4).reshape(rows, cols)
    assert np.array_equal(codes[:16], ref.codes[:16]) and (codes[:16] == 0).all()
    assert np.array_equal(codes[48:], ref.codes[48:])
    assert (q.stop_step[48:].cpu().numpy() == 0).all()


def test_exact_ties_round_half_even(hq):
    """s = 1 and integer z: every w/s + z is exact in fp32 and fp64, ties are real ties."""
    _say("tie-engineered groups")
    rng = np.random.default_rng(1)
    rows, cols = 32, 64
    v = rng.integers(0, 7, (rows, cols)).astype(np.float64) / 2.0  # multiples of 1/2 in [0, 3]
    v[:, ::16] = 0.0
    v[:, 1::16] = 3.0  # min 0, max 3 -> s = 1, z = 0 for 2-bit groups of 16
    W = torch.from_numpy(v.astype(np.float16)).cuda()
    q = _run(hq, W, 2, 16, iters=0)
    ref = oracle.hqq_quantize(v.astype(np.float16), 2, 16, iters=0)
    codes = oracle.unpack_codes(q.packed.cpu().numpy(), rows * cols, 2).reshape(rows, cols)
    assert np.array_equal(codes, ref.codes)


def test_init_near_ties_below_binary32_resolution(hq):
    """Groups holding a binary16 triple (min, max, w) whose exact initial ratio
    (w - min) qmax / (max - min) lies off a half-integer by less than a binary32 rounding:
    its fp32 rounding lands on the half-integer, and the device must still take the exact
    code (the oracle's).  At T = 0 (the initial quantizer alone) every code must equal the
    oracle's bit for bit; with the full solver, the usual tolerances apply."""
    from tests.test_oracle_pins import NEAR_TIE_TRIPLES
    rng = np.random.default_rng(12)
    total = {}
    for qmax, nbits in ((15, 4), (7, 3), (3, 2), (255, 8)):
        rows = []
        for mn, mx, w in NEAR_TIE_TRIPLES[qmax]:
            for _ in range(64):
                grp = np.concatenate([[mn, mx, w], rng.uniform(mn, mx, 13)]).astype(np.float16)
                grp[3:] = np.clip(grp[3:], np.float16(mn), np.float16(mx))
                rows.append(grp)
        W = np.stack(rows).reshape(-1, 64)
        _say(f"init near ties b{nbits}: {W.shape[0] * 4} groups of 16")
        Wt = torch.from_numpy(W).cuda()
        q0 = _run(hq, Wt, nbits, 16, iters=0)
        ref0 = oracle.hqq_quantize(W, nbits, 16, iters=0)
        codes0 = oracle.unpack_codes(q0.packed.cpu().numpy(), W.size, nbits).reshape(W.shape)
        assert np.array_equal(codes0, ref0.codes), "initial codes differ from the exact ones"
        q = _run(hq, Wt, nbits, 16)
        rep = parity.compare(W.view(np.uint16), parity.from_quantized(q), nbits, 16, min_agree=0.99)
        total[nbits] = (rep["code_mismatch_total"], rep["divergent"])
        _say(f"  {rep}")
    _say(f"near-tie code mismatches and divergent groups per bit width: {total}")


def test_hand_examples_are_exact_on_gpu(hq):
    """The worked examples of the oracle pins, duplicated to a group of 16, in dyadic arithmetic."""
    _say("hand examples")
    w8 = np.array([0.0] + [0.25] * 6 + [3.0])
    W = torch.from_numpy(np.tile(w8, 2)[None, :].astype(np.float16)).cuda()
    q = _run(hq, W, 2, 16, p=0.7)
    assert q.stop_step.item() == 1 and q.zero_f32.item() == -0.1875
    q = _run(hq, W, 2, 16, p=1.0, beta=8.0, kappa=2.0, iters=3)
    assert q.stop_step.item() == 3 and q.zero_f32.item() == -0.140625
    assert abs(q.err_best.item() - 2 * 0.9375) <= 1e-6
    codes = oracle.unpack_codes(q.packed.cpu().numpy(), 16, 2)
    assert codes.tolist() == ([0] * 7 + [3]) * 2


# ------------------------------------------------------- dequant and API --

@pytest.mark.parametrize("nbits,g", [(4, 64), (3, 64), (2, 16), (2, 32), (8, 128)])
def test_dequantize_is_single_rounding(hq, nbits, g):
    _say(f"dequant b{nbits} g{g}")
    W = workloads.generate(512, 1024, workloads.WORKLOADS["mlp_11008x4096"].dist, 21, "cuda")
    q = hq.quantize(W, nbits, g)
    Wd = hq.dequantize(q)
    torch.cuda.synchronize()
    ref = oracle.hqq_dequantize(q.packed.cpu().numpy(), q.scale.cpu().numpy(),
                                q.zero.cpu().numpy(), 512, 1024, nbits, g)
    assert np.array_equal(Wd.cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("nbits,g", [(4, 64), (8, 128), (2, 32), (3, 16)])
def test_packed_stream_four_byte_aligned(hq, nbits, g):
    """The packed stream needs only 4-byte alignment: quantizing into a buffer 4 bytes past
    an aligned allocation gives the same bytes, and hqq_dequantize reads them back from
    there bit for bit."""
    _say(f"packed stream at a 4-byte offset, b{nbits} g{g}")
    W = workloads.generate(256, 512, workloads.WORKLOADS["mlp_11008x4096"].dist, 23, "cuda")
    ref = hq.quantize(W, nbits, g)
    nb = hq.hqq_packed_bytes(256, 512, nbits)
    buf = torch.full((nb + 16,), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.empty_like(ref.scale)
    z = torch.empty_like(ref.zero)
    st = hq.hqq_quantize(W.data_ptr(), 256, 512, nbits, g, 0.7, 1.0, 1.01, 20,
                         buf.data_ptr() + 4, s.data_ptr(), z.data_ptr())
    assert st == hq.HQQ_OK, hq.hqq_status_string(st)
    out = torch.empty_like(W)
    st = hq.hqq_dequantize(buf.data_ptr() + 4, s.data_ptr(), z.data_ptr(), 256, 512, nbits, g,
                           out.data_ptr())
    assert st == hq.HQQ_OK, hq.hqq_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(buf[4:4 + nb], ref.packed)
    assert int(buf[:4].ne(0xA5).sum()) == 0 and int(buf[4 + nb:].ne(0xA5).sum()) == 0
    assert torch.equal(out.view(torch.int16), hq.dequantize(ref).view(torch.int16))


def test_plain_entry_point_equals_debug_entry_point_and_is_deterministic(hq):
    _say("hqq_quantize vs hqq_quantize_ex, repeatability, side stream")
    W = workloads.generate_matrix(workloads.WORKLOADS["attn_4096x4096"], 0, "cuda")
    a = hq.quantize(W, 4, 64)
    b = hq.quantize(W, 4, 64, debug=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = hq.quantize(W, 4, 64, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    for x, y in ((a, b), (a, c)):
        assert torch.equal(x.packed, y.packed)
        assert torch.equal(x.scale.view(torch.int16), y.scale.view(torch.int16))
        assert torch.equal(x.zero.view(torch.int16), y.zero.view(torch.int16))
    # rows are independent: a block of rows gives the bit-identical result
    top = hq.quantize(W[:100].contiguous(), 4, 64)
    torch.cuda.synchronize()
    assert torch.equal(top.packed, a.packed[: 100 * 2048])
    assert torch.equal(top.zero.view(torch.int16), a.zero[:100].view(torch.int16))


@pytest.mark.parametrize("nbits,g", [(2, 16), (2, 32), (4, 64)])
def test_refill_threshold_changes_no_output(hq, nbits, g):
    """The hand-over threshold only changes the schedule.  A high threshold lets up to
    every segment of a wavefront stop before the hand-over, more than the done ring holds
    at g <= 32 (those groups are written straight from registers), and the result must be
    bit-identical to the default schedule."""
    _say(f"refill thresholds, b{nbits} g{g}")
    W = workloads.generate_matrix(workloads.WORKLOADS["attn_4096x4096"], 0, "cuda")
    ref = hq.quantize(W, nbits, g)
    slots = 64 * 16 // g
    for thr in (2, 5, slots // 2 + 1, slots):
        q = hq.quantize(W, nbits, g, refill_threshold=thr)
        torch.cuda.synchronize()
        assert torch.equal(q.packed, ref.packed), thr
        assert torch.equal(q.scale.view(torch.int16), ref.scale.view(torch.int16)), thr
        assert torch.equal(q.zero.view(torch.int16), ref.zero.view(torch.int16)), thr


def test_empty_input(hq):
    W = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    q = hq.quantize(W, 4, 64)
    assert q.packed.numel() == 0 and q.scale.numel() == 0


# ----------------------------------------------------------- batched launch --

def _assert_same_outputs(x, y):
    assert torch.equal(x.packed, y.packed)
    assert torch.equal(x.scale.reshape(-1).view(torch.int16), y.scale.reshape(-1).view(torch.int16))
    assert torch.equal(x.zero.reshape(-1).view(torch.int16), y.zero.reshape(-1).view(torch.int16))


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 32), (2, 16), (3, 128), (8, 64)])
def test_batch_equals_per_matrix_calls(hq, nbits, g):
    """One batched launch writes, bit for bit, what one hqq_quantize per matrix writes
    (the per-matrix path is the one compared with the oracle above): empty entries,
    entries with fewer groups than a wavefront holds, ragged group counts and entry
    boundaries inside a wavefront's queue."""
    shapes = [(37, 5 * g), (0, g), (1, g), (3, g), (1024, 64 * g), (5, 0), (129, 2 * g),
              (2049, g), (7, 3 * g), (1, g)]
    _say(f"hqq_quantize_batch vs per-matrix calls, b{nbits} g{g}, {len(shapes)} entries")
    dist = workloads.WORKLOADS["mlp_11008x4096"].dist
    Ws = [workloads.generate(r, c, dist, 900 + i, "cuda") if r * c else
          torch.empty((r, c), dtype=torch.float16, device="cuda") for i, (r, c) in enumerate(shapes)]
    b = hq.quantize_batch(Ws, nbits, g)
    torch.cuda.synchronize()
    assert b.packed.numel() == sum(r * c for r, c in shapes) * nbits // 8
    for i, W in enumerate(Ws):
        one = hq.quantize(W, nbits, g)
        torch.cuda.synchronize()
        _assert_same_outputs(b.matrix(i), one)
    # the arena can be reused for the same shapes (same stream)
    b2 = hq.quantize_batch(Ws, nbits, g, out=b)
    torch.cuda.synchronize()
    assert b2 is b
    _assert_same_outputs(b.matrix(4), hq.quantize(Ws[4], nbits, g))


def test_batch_rejects_a_device_table_that_differs(hq):
    """The kernel checks its device copy of the entry table against the validated host
    table before it reads any weight.  With two entries swapped in the copy (every pointer
    still a valid tensor of the same shape, so an undetected mismatch could not fault) or
    one pointer replaced by another tensor's, the launch writes nothing and reports
    HQQ_ERR_TABLE_MISMATCH in its status word; with the right copy it reports HQQ_OK."""
    import ctypes
    dist = workloads.WORKLOADS["attn_4096x4096"].dist
    Ws = [workloads.generate(64, 256, dist, 950 + i, "cuda") for i in range(4)]
    b = hq.quantize_batch(Ws[:3], 4, 64)
    b.check()
    _say("batched launch with a device table that differs from the host table")
    entries, _ = hq.batch_table(Ws[:3], 64)
    for wrong in ([Ws[1], Ws[0], Ws[2]], [Ws[0], Ws[1], Ws[3]]):
        dev_entries, _ = hq.batch_table(wrong, 64)
        b.table.copy_(torch.frombuffer(bytearray(bytes(dev_entries)), dtype=torch.uint8))
        b.packed.fill_(0xA5)
        b.scale.fill_(7.0)
        b.zero.fill_(-3.0)
        b.status.fill_(-1)
        st = hq.hqq_quantize_batch(entries, b.table.data_ptr(), 3, 4, 64, 0.7, 1.0, 1.01, 20,
                                   b.packed.data_ptr(), b.scale.data_ptr(), b.zero.data_ptr(),
                                   b.status.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == hq.HQQ_OK  # the host side validated its own table and launched
        torch.cuda.synchronize()
        assert int(b.status.item()) == hq.HQQ_ERR_TABLE_MISMATCH
        assert bool((b.packed == 0xA5).all()) and bool((b.scale == 7.0).all())
        assert bool((b.zero == -3.0).all())
        with pytest.raises(hq.HQQError):
            b.check()
    b2 = hq.quantize_batch(Ws[:3], 4, 64, out=b)
    b2.check()
    assert ctypes.sizeof(hq.hqq_batch_entry_t) == 32
    for i, W in enumerate(Ws[:3]):
        _assert_same_outputs(b2.matrix(i), hq.quantize(W, 4, 64))


def test_batch_out_must_match(hq):
    """An arena passed as out is reused only for the shapes and settings it was made for."""
    dist = workloads.WORKLOADS["attn_4096x4096"].dist
    Ws = [workloads.generate(64, 256, dist, 960 + i, "cuda") for i in range(3)]
    b = hq.quantize_batch(Ws[:2], 4, 64)
    other = [Ws[0], workloads.generate(64, 128, dist, 963, "cuda")]
    for args in ((Ws, 4, 64), (Ws[:2], 2, 64), (Ws[:2], 4, 32), (other, 4, 64)):
        with pytest.raises(ValueError):
            hq.quantize_batch(*args, out=b)
    q = hq.quantize(Ws[0], 4, 64)
    with pytest.raises(ValueError):
        hq.quantize(Ws[0][:32].contiguous(), 4, 64, out=q)
    with pytest.raises(ValueError):
        hq.dequantize(q, out=torch.empty((64, 128), dtype=torch.float16, device="cuda"))


@pytest.mark.parametrize("nbits,g", [(2, 32), (4, 64)])
def test_batch_llama70b_layer(hq, nbits, g):
    """The benchmark's call: a 70B-shaped layer (7 matrices) in one launch equals the
    per-matrix results."""
    wl = workloads.WORKLOADS["llama70b_stack"]
    mats = wl.matrices[:7]
    _say(f"hqq_quantize_batch on 70B layer 0 (7 matrices), b{nbits} g{g}")
    Ws = [workloads.generate(m.rows, m.cols, wl.dist, m.seed, "cuda") for m in mats]
    b = hq.quantize_batch(Ws, nbits, g)
    torch.cuda.synchronize()
    for i, W in enumerate(Ws):
        one = hq.quantize(W, nbits, g)
        torch.cuda.synchronize()
        _assert_same_outputs(b.matrix(i), one)
