"""GPU parity of hqq_matmul (Y = X Q^-1(W_q)^T, through the C ABI) against the oracle.

Weights are stored-format inputs built on the host (random codes packed by the
oracle's packer, binary16 s and z), so nothing on the oracle side comes from the
device.  Two kinds of checks:
  * exact cases: s a power of two, z an integer, X small integers: every product and
    partial sum is exact in fp32 whatever the order, so fp32 outputs equal the oracle
    bit for bit and binary16 outputs equal the oracle's value rounded once.  This pins
    the indexing of every kernel (few rows of X: the per-row kernel; up to 64: the
    skinny matrix-core kernels; above: the tiled one) over ragged tiles, all bit widths
    and group sizes;
  * general inputs: |y_dev - y_oracle| within a bound derived from the arithmetic of the
    path (``_bound``), on full small products and on sampled outputs of the Llama-2-70B
    layer shapes at full size.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
U16 = 2.0 ** -11


@pytest.fixture(scope="module")
def hq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    import bit_weight_quantization_amd as m
    m.load_library()
    return m


def _say(msg):
    print(f"[gpu-matmul] {msg}", flush=True)


def _weight(N, K, nbits, g, seed, exact=False):
    rng = np.random.default_rng(seed)
    qmax = (1 << nbits) - 1
    codes = rng.integers(0, qmax + 1, (N, K), dtype=np.uint8)
    G = K // g
    if exact:
        s = (2.0 ** -rng.integers(3, 7, (N, G))).astype(np.float16)
        z = rng.integers(0, qmax + 1, (N, G)).astype(np.float16)
    else:
        s = np.asarray(rng.uniform(2e-4, 4e-3, (N, G)), np.float16)
        z = np.asarray(rng.uniform(-0.5, qmax + 0.5, (N, G)), np.float16)
    packed = oracle.pack_codes(codes.ravel(), nbits)
    return codes, packed, s, z


def _run(hq, X, packed, s, z, N, nbits, g, out_f32, sz_offset=0):
    """sz_offset binary16 elements of padding in front of s and z (their device pointers
    then lose 16-byte alignment when it is odd)."""
    M, K = X.shape
    Xd = torch.from_numpy(X.view(np.int16).copy()).view(torch.float16).cuda()
    pd = torch.from_numpy(packed.copy()).cuda()
    pad = np.zeros(sz_offset, np.int16)
    sd = torch.from_numpy(np.concatenate([pad, s.view(np.int16).ravel()])).cuda()
    zd = torch.from_numpy(np.concatenate([pad, z.view(np.int16).ravel()])).cuda()
    Y = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.float16, device="cuda")
    wb = hq.hqq_matmul_workspace_bytes(M, N, K, nbits, g)
    assert wb >= 0
    ws = torch.empty(max(wb, 1), dtype=torch.uint8, device="cuda")
    st = hq.hqq_matmul(Xd.data_ptr(), M, K, pd.data_ptr(), sd.data_ptr() + 2 * sz_offset,
                       zd.data_ptr() + 2 * sz_offset, N, nbits, g, Y.data_ptr(), int(out_f32),
                       ws.data_ptr() if wb > 0 else 0)
    assert st == hq.HQQ_OK, hq.hqq_status_string(st)
    torch.cuda.synchronize()
    return Y.cpu().numpy().astype(np.float64)


def _per_row_path(M, K, nbits, g):
    """hqq_matmul's per-row path (exact codes): M <= 2 where the aligned small-batch
    kernel applies (2, 4, 8 bits, g >= 32, K % 256 == 0; these tests' s and z are
    16-byte aligned), else M <= 8."""
    aligned = nbits != 3 and g >= 32 and K % 256 == 0
    return M <= (2 if aligned else 8)


def _bound(X, codes, s, z, g, gemv, out_f32, y):
    """Worst-case |y_dev - y_exact| of the device path, elementwise (M x N).
    per-row path: per 16 codes fp32 sums of x q and x, then s (p - z sx) accumulated over
      K/16 blocks and a 64-lane tree: <= (K/16 + 30) u32 sum_k |x| |s| (|q| + |z|);
    matrix-core path: the weight rounded to fp32 then binary16 (<= (u16 + 2 u32) |w| +
      2^-25 absolute, binary16 subnormals), exact products, fp32 sums over K:
      <= sum_k |x| ((u16 + 2 u32) |w| + 2^-25) + (K + 8) u32 sum_k |x| |w| (1 + 2 u16);
    plus u16 |y| for a binary16 output."""
    K = X.shape[1]
    x = np.abs(X.astype(np.float64))
    sk = np.repeat(s.astype(np.float64), g, axis=1)
    zk = np.repeat(z.astype(np.float64), g, axis=1)
    w = sk * (codes.astype(np.float64) - zk)
    if gemv:
        b = (K / 16 + 30) * U32 * (x @ (np.abs(sk) * (codes + np.abs(zk))).T)
    else:
        aw = np.abs(w)
        b = x @ ((U16 + 2 * U32) * aw + 2.0 ** -25).T + (K + 8) * U32 * (1 + 2 * U16) * (x @ aw.T)
    if not out_f32:
        b = b + U16 * np.abs(y) + 2.0 ** -25
    return b


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 32), (2, 16), (3, 32), (8, 128), (4, 16)])
def test_exact_products_all_paths(hq, nbits, g):
    rng = np.random.default_rng(nbits * 100 + g)
    shapes = [(1, 7, 128), (2, 3, 256), (3, 128, 64 if g <= 64 else 128), (5, 300, 256),
              (8, 129, 384), (9, 128, 128), (16, 257, 256), (20, 33, 160 if g <= 32 else 256),
              (33, 70, 256), (64, 129, 384), (130, 300, 512), (257, 64, 1024)]
    for M, N, K in shapes:
        if K % g:
            continue
        codes, packed, s, z = _weight(N, K, nbits, g, seed=M * 7 + N, exact=True)
        X = rng.integers(-2, 3, (M, K)).astype(np.float16)
        ref = oracle.hqq_matmul(X, packed, s, z, N, nbits, g)
        for out_f32 in (1, 0):
            Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32)
            want = ref if out_f32 else oracle.f16_to_f64(oracle.f64_to_f16(ref))
            bad = np.argwhere(Y != want)
            assert bad.size == 0, (M, N, K, out_f32, bad[:5], Y[tuple(bad[0])], want[tuple(bad[0])])
    _say(f"b{nbits} g{g}: exact on {len(shapes)} shapes, fp32 and binary16 outputs")


@pytest.mark.parametrize("nbits", [2, 4, 8])
def test_exact_products_skinny_paths(hq, nbits):
    """Small batches (2 < M <= 64) on the matrix-core skinny kernels: K a multiple of 256
    with 1, 2, 9 and 16 blocks of 256 (split over 1, 2 and 16 partial sums; the general
    kernel splits 9 unevenly over the 8 wavefronts of a block), one and two 16-row weight
    groups per wavefront (N below and above 4096, ragged), every 16-row tile count of X
    (M = 3 .. 64), groups of 32, 64 and 128, and s, z off 16-byte alignment (the general
    kernel): bit-exact on exact inputs."""
    rng = np.random.default_rng(400 + nbits)
    cases = [(3, 100, 512, 32, 0), (4, 130, 2304, 128, 0), (8, 4100, 256, 64, 0),
             (9, 100, 256, 32, 0), (16, 300, 2304, 64, 0), (17, 129, 4096, 128, 0),
             (32, 4100, 2304, 32, 0), (33, 70, 2304, 64, 0), (64, 4097, 512, 128, 0),
             (40, 200, 4096, 32, 0), (24, 130, 2304, 64, 1), (48, 4100, 768, 32, 3)]
    for M, N, K, g, off in cases:
        codes, packed, s, z = _weight(N, K, nbits, g, seed=M + N + K, exact=True)
        X = rng.integers(-2, 3, (M, K)).astype(np.float16)
        ref = oracle.hqq_matmul(X, packed, s, z, N, nbits, g)
        for out_f32 in (1, 0):
            Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32, sz_offset=off)
            want = ref if out_f32 else oracle.f16_to_f64(oracle.f64_to_f16(ref))
            bad = np.argwhere(Y != want)
            assert bad.size == 0, (M, N, K, g, off, out_f32, bad[:5], Y[tuple(bad[0])], want[tuple(bad[0])])
        _say(f"b{nbits} M={M} N={N} K={K} g{g} s/z offset {off}: exact")


def test_split_k_is_deterministic_and_exact(hq):
    """The split-K path (17 to 64 rows of X): many partial slabs (N = 1024, K = 8192: 32
    splits; N = 8192, K = 4096: 4) are added in a fixed order, so repeated calls give
    identical bits on general inputs, and exact inputs give the exact product."""
    rng = np.random.default_rng(77)
    for M, N, K, nbits, g in [(64, 1024, 8192, 4, 64), (24, 8192, 4096, 2, 32),
                              (37, 1000, 8192, 8, 128)]:
        wb = hq.hqq_matmul_workspace_bytes(M, N, K, nbits, g)
        assert wb > 0
        codes, packed, s, z = _weight(N, K, nbits, g, seed=M + N)
        X = np.asarray(rng.standard_normal((M, K)), np.float16)
        Y1 = _run(hq, X, packed, s, z, N, nbits, g, out_f32=1)
        Y2 = _run(hq, X, packed, s, z, N, nbits, g, out_f32=1)
        assert np.array_equal(Y1, Y2)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)]))
        bpr = K * nbits // 8
        ref = oracle.hqq_matmul(X, packed.reshape(N, bpr)[rows].ravel(), s[rows], z[rows],
                                len(rows), nbits, g)
        b = _bound(X, codes[rows], s[rows], z[rows], g, False, 1, ref)
        assert np.all(np.abs(Y1[:, rows] - ref) <= b)
        codes, packed, s, z = _weight(N, K, nbits, g, seed=M + N + 1, exact=True)
        Xe = rng.integers(-2, 3, (M, K)).astype(np.float16)
        Ye = _run(hq, Xe, packed, s, z, N, nbits, g, out_f32=1)
        ref = oracle.hqq_matmul(Xe, packed.reshape(N, bpr)[rows].ravel(), s[rows], z[rows],
                                len(rows), nbits, g)
        assert np.array_equal(Ye[:, rows], ref)
        _say(f"split-K M={M} N={N} K={K} b{nbits} g{g}: {wb} workspace bytes, repeatable, exact")


@pytest.mark.parametrize("nbits,g", [(2, 32), (4, 64)])
def test_split_k_unsplit_odd_block_count(hq, nbits, g):
    """The split-K kernel with one split over many blocks of K: a ragged 28722-row weight
    (225 blocks of 128 rows, so K is not split) with an odd count of 7 blocks of 256.
    This runs full rounds of its loop, whose loads run a block ahead, and then a last
    block that loads nothing.  Exact inputs give the exact product on sampled rows
    (including the ragged last ones); repeated calls are bit-identical."""
    N, K = 28722, 7 * 256
    assert hq.hqq_matmul_workspace_bytes(64, N, K, nbits, g) == 0  # one split: no slabs
    codes, packed, s, z = _weight(N, K, nbits, g, seed=N + nbits, exact=True)
    rng = np.random.default_rng(5 + nbits)
    rows = np.unique(np.concatenate([[0, N - 2, N - 1], rng.choice(N, 40, replace=False)]))
    bpr = K * nbits // 8
    for M in (64, 20):
        X = rng.integers(-2, 3, (M, K)).astype(np.float16)
        Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32=1)
        assert np.array_equal(Y, _run(hq, X, packed, s, z, N, nbits, g, out_f32=1))
        ref = oracle.hqq_matmul(X, packed.reshape(N, bpr)[rows].ravel(), s[rows], z[rows],
                                len(rows), nbits, g)
        assert np.array_equal(Y[:, rows], ref)
        _say(f"split-K unsplit M={M} N={N} K={K} b{nbits} g{g}: exact, repeatable")


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 16), (3, 32), (8, 128)])
def test_exact_products_large_tiles(hq, nbits, g):
    """A large ragged product on the matrix-core kernel (M = 1040 and N = 16500, 645+
    tiles, ragged against 128 and 256): bit-exact on exact inputs, checked on sampled
    weight rows (every activation row)."""
    rng = np.random.default_rng(nbits * 7 + g)
    M, N, K = 1040, 16500, 256
    codes, packed, s, z = _weight(N, K, nbits, g, seed=N + nbits, exact=True)
    X = rng.integers(-2, 3, (M, K)).astype(np.float16)
    rows = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 36, replace=False)]))
    bpr = K * nbits // 8
    sub_packed = packed.reshape(N, bpr)[rows].ravel()
    ref = oracle.hqq_matmul(X, sub_packed, s[rows], z[rows], len(rows), nbits, g)
    Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32=1)
    bad = np.argwhere(Y[:, rows] != ref)
    assert bad.size == 0, (bad[:5],)
    _say(f"b{nbits} g{g}: {M}x{N}x{K} exact on {len(rows)} sampled weight rows")


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 32), (3, 64), (8, 32)])
def test_general_inputs_within_the_bound(hq, nbits, g):
    rng = np.random.default_rng(nbits + 7 * g)
    for M in (1, 4, 8, 24, 40, 64, 200):
        N, K = 160, 1024
        codes, packed, s, z = _weight(N, K, nbits, g, seed=M + 1000)
        X = np.asarray(rng.standard_normal((M, K)), np.float16)
        ref = oracle.hqq_matmul(X, packed, s, z, N, nbits, g)
        for out_f32 in (1, 0):
            Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32)
            b = _bound(X, codes, s, z, g, _per_row_path(M, K, nbits, g), out_f32, ref)
            err = np.abs(Y - ref)
            assert np.all(err <= b), (M, out_f32, float((err / b).max()))
            _say(f"b{nbits} g{g} M={M} out_f32={out_f32}: max err/bound {float((err / b).max()):.3g}, "
                 f"max rel err {float((err / np.maximum(np.abs(ref), 1e-6)).max()):.3g}")


@pytest.mark.parametrize("nbits,g", [(4, 64), (2, 32)])
def test_llama70b_layer_shapes_sampled(hq, nbits, g):
    """The 7 weight shapes of a Llama-2-70B layer at full size (N x K = 8192 x 8192,
    1024 x 8192, 28672 x 8192, 8192 x 28672), decode (M = 1), small-batch (M = 16, 64) and
    prefill (M = 512) activations; outputs checked on sampled weight rows and activation
    rows."""
    rng = np.random.default_rng(70 + nbits)
    for N, K in [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)]:
        codes, packed, s, z = _weight(N, K, nbits, g, seed=N + K + nbits)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 46, replace=False)]))
        bpr = K * nbits // 8
        sub_packed = packed.reshape(N, bpr)[rows].ravel()
        for M in (1, 16, 64, 512):
            X = np.asarray(rng.standard_normal((M, K)) * 0.5, np.float16)
            Y = _run(hq, X, packed, s, z, N, nbits, g, out_f32=1)
            ms = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 6), replace=False)]))
            ref = oracle.hqq_matmul(X[ms], sub_packed, s[rows], z[rows], len(rows), nbits, g)
            b = _bound(X[ms], codes[rows], s[rows], z[rows], g, _per_row_path(M, K, nbits, g), 1, ref)
            err = np.abs(Y[np.ix_(ms, rows)] - ref)
            assert np.all(err <= b)
            _say(f"{N}x{K} b{nbits} g{g} M={M}: max err/bound {float((err / b).max()):.3g}")


def test_quantize_then_matmul_matches_dequantize(hq):
    """The device quantizer's output fed to the product equals (within the bound of the
    matrix-core path) the product with the device's binary16 dequantization."""
    import workloads
    W = workloads.generate_matrix(workloads.WORKLOADS["attn_4096x4096"], 0, "cuda")
    q = hq.quantize(W, 4, 64)
    Wd = hq.dequantize(q).float()
    X = torch.randn((64, 4096), device="cuda").half()
    Y = hq.matmul(X, q, out_f32=True)
    ref = X.float() @ Wd.T
    torch.cuda.synchronize()
    err = (Y - ref).abs()
    scale = X.float().abs() @ Wd.abs().T
    assert float((err / (scale * 2.0 ** -9 + 1e-6)).max()) <= 1.0
    Y1 = hq.matmul(X[:1].contiguous(), q, out_f32=True)
    torch.cuda.synchronize()
    assert float(((Y1 - Y[:1]).abs() / (scale[:1] * 2.0 ** -9 + 1e-6)).max()) <= 1.0


def test_empty_and_zero_k(hq):
    X = torch.zeros((0, 64), dtype=torch.float16, device="cuda")
    assert hq.hqq_matmul(X.data_ptr(), 0, 64, 0, 0, 0, 5, 4, 64, 0, 0, 0) == hq.HQQ_OK
    Y = torch.full((3, 5), 7.0, dtype=torch.float32, device="cuda")
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    st = hq.hqq_matmul(dummy.data_ptr(), 3, 0, dummy.data_ptr(), dummy.data_ptr(),
                       dummy.data_ptr(), 5, 4, 64, Y.data_ptr(), 1, 0)
    torch.cuda.synchronize()
    assert st == hq.HQQ_OK and torch.equal(Y, torch.zeros_like(Y))
    Y2 = torch.full((12, 5), 7.0, dtype=torch.float32, device="cuda")  # matrix-core path
    st = hq.hqq_matmul(dummy.data_ptr(), 12, 0, dummy.data_ptr(), dummy.data_ptr(),
                       dummy.data_ptr(), 5, 4, 64, Y2.data_ptr(), 1, 0)
    torch.cuda.synchronize()
    assert st == hq.HQQ_OK and torch.equal(Y2, torch.zeros_like(Y2))
