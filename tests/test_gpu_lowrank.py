"""GPU parity of the low-rank compensation path (hqq_residual, hqq_lowrank) against the
oracle.

The weights' quantization (codes, binary16 s and z) comes from the oracle's quantizer or
is built on the host, so nothing on the oracle side comes from the device.
  * residual: every element within the rounding bound of the device arithmetic
    (s q - s z in fp32, the difference in fp32, then binary16) of the oracle's fp64
    residual; the transposed copy is the exact transpose;
  * planted spectrum (codes 0, z = 0, s = 1, so Delta W is W itself): singular values,
    the rank-r part B A, orthonormality, against the exact truncated SVD of the oracle;
  * a quantization residual (flat spectrum), against the oracle's exact truncation: the
    captured energy sum sigma_i^2 at least (1 - eps) of the exact rank-r part's, the top
    singular value and every singular value above a fixed fraction of the exact ones, and
    below them (Ritz values); eps and the fractions rest on what the same iteration
    achieves in fp64 on these inputs (see LOWRANK_FLOORS).  The same run is also compared
    with an fp64 run of the same iteration and test matrix (a check of the binary16 /
    fp32 products only);
  * a 70B layer matrix at full size: the same floors against the exact singular values of
    the oracle's residual, and the structure (orthonormal A, B A consistent with the
    singular values and with the residual's norm).
Tolerances: Delta W and the iterates Q enter the matrix-core products as binary16
(relative 2^-11 per entry), sums are fp32; the resulting singular values agree to a few
units of 2^-11 relative, which is what the bounds below allow.
"""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

U16 = 2.0 ** -11
U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def hq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    import bit_weight_quantization_amd as m
    m.load_library()
    return m


def _say(msg):
    print(f"[gpu-lowrank] {msg}", flush=True)


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).cuda()


def _quantized_weight(hq, W16, packed, s16, z16, nbits, g):
    rows, cols = W16.shape
    return hq.QuantizedWeight(packed=torch.from_numpy(packed.copy()).cuda(),
                              scale=_dev16(s16).view(torch.float16),
                              zero=_dev16(z16).view(torch.float16), rows=rows, cols=cols,
                              nbits=nbits, group_size=g)


def _randomized_svd64(dW, omega, rank, q):
    """The same subspace iteration in fp64 (numpy QR for the orthonormalizations: the
    spanned subspaces, hence the results, do not depend on the basis chosen)."""
    Om = omega.astype(np.float64).T
    Y = dW @ Om
    for _ in range(q):
        Q, _ = np.linalg.qr(Y)
        P, _ = np.linalg.qr(dW.T @ Q)
        Y = dW @ P
    Q, _ = np.linalg.qr(Y)
    Bm = Q.T @ dW
    Ub, S, Vt = np.linalg.svd(Bm, full_matrices=False)
    return (Q @ Ub[:, :rank]) * S[:rank], Vt[:rank], S[:rank]


@pytest.mark.parametrize("rows,cols,nbits,g", [(128, 256, 4, 64), (192, 512, 2, 16),
                                               (64, 128, 3, 32), (256, 256, 8, 128)])
def test_residual_within_rounding_of_the_oracle(hq, rows, cols, nbits, g):
    rng = np.random.default_rng(rows + cols + nbits)
    W = np.asarray(rng.standard_t(4, (rows, cols)) * 0.02, np.float16)
    r = oracle.hqq_quantize(W, nbits, g)
    ref = oracle.hqq_residual(W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    q = _quantized_weight(hq, W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    Wd = _dev16(W).view(torch.float16)
    dW, dWT = hq.residual(Wd, q, transposed=True)
    torch.cuda.synchronize()
    dev = dW.cpu().numpy().astype(np.float64)
    what = np.abs(W.astype(np.float64) - ref)  # |W_hat|
    bound = U32 * what + U32 * np.abs(ref) + U16 * np.abs(dev) + 2.0 ** -25
    assert np.all(np.abs(dev - ref) <= bound)
    assert torch.equal(dWT.view(torch.int16), dW.t().contiguous().view(torch.int16))
    _say(f"residual {rows}x{cols} b{nbits} g{g}: max err/bound {float((np.abs(dev - ref) / bound).max()):.3g}")


def _zero_quantization(rows, cols, nbits, g):
    packed = np.zeros((rows * cols * nbits + 7) // 8, np.uint8)
    s16 = np.full((rows, cols // g), np.float16(1.0))
    z16 = np.zeros((rows, cols // g), np.float16)
    return packed, s16, z16


# widths rank + over: 64, 96 (factorizations in LDS), 32, 128 and 512 (in global memory)
@pytest.mark.parametrize("rows,cols,rank,over,decay", [(256, 512, 32, 32, 0.9),
                                                       (512, 256, 64, 32, 0.9),
                                                       (128, 1024, 16, 16, 0.9),
                                                       (256, 512, 96, 32, 0.99),
                                                       (640, 768, 448, 64, 0.995)])
def test_planted_spectrum_matches_the_exact_truncation(hq, rows, cols, rank, over, decay):
    rng = np.random.default_rng(rows * 3 + rank)
    k = rank + 24
    U, _ = np.linalg.qr(rng.standard_normal((rows, k)))
    V, _ = np.linalg.qr(rng.standard_normal((cols, k)))
    sig = decay ** np.arange(k)
    sig[rank:] *= 0.2  # a clear gap after the rank-r part
    W = np.asarray((U * sig) @ V.T + rng.standard_normal((rows, cols)) * 1e-4, np.float16)
    packed, s16, z16 = _zero_quantization(rows, cols, 4, 64)
    dW = oracle.hqq_residual(W, packed, s16, z16, 4, 64)  # = W exactly
    B64, A64, s_all = oracle.lowrank_svd(dW, rank)
    q = _quantized_weight(hq, W, packed, s16, z16, 4, 64)
    Wd = _dev16(W).view(torch.float16)
    B, A, S = hq.lowrank(Wd, q, rank, oversample=over, power_iters=4, seed=rows)
    torch.cuda.synchronize()
    B, A, S = (t.cpu().numpy().astype(np.float64) for t in (B, A, S))
    rel = np.abs(S - s_all[:rank]) / s_all[:rank]
    assert rel.max() <= 8 * U16, rel.max()
    BA, ref = B @ A, B64 @ A64
    err = np.linalg.norm(BA - ref) / np.linalg.norm(ref)
    assert err <= 16 * U16, err
    assert np.abs(A @ A.T - np.eye(rank)).max() <= 8 * U16
    G = B.T @ B
    assert np.abs(G - np.diag(S ** 2)).max() <= 8 * U16 * S[0] ** 2
    _say(f"planted {rows}x{cols} r={rank}: max rel sigma err {rel.max():.3g}, rel |BA - B64 A64| {err:.3g}")


# Floors of the randomized truncation (width rank + 32, 4 power steps) against the exact
# one on quantization residuals, whose spectra are nearly flat: fraction of the exact
# rank-r energy captured, of the top singular value, and of every singular value.  The same
# iteration in fp64 (numpy QR, 20 test matrices) reaches at least 0.976 / 0.993 / 0.975 of
# them on the 512 x 1024 residuals and 0.909 / 0.960 / 0.942 on the 8192 x 8192 70B one
# (b4 g64, rank 64; 3 test matrices); the floors leave room for a further loss of a few
# percent, far more than the binary16 products cost (a few 2^-11 relative).
LOWRANK_FLOORS = {"512x1024": (0.95, 0.98, 0.95), "8192x8192": (0.88, 0.94, 0.92)}


def _check_against_exact(S, s_exact, rank, floors, where):
    energy, top, each = floors
    cap, opt = np.sum(S ** 2), np.sum(s_exact[:rank] ** 2)
    assert cap >= energy * opt, f"{where}: captured {cap / opt:.4f} of the exact rank-{rank} energy"
    assert S[0] >= top * s_exact[0], f"{where}: top sigma {S[0] / s_exact[0]:.4f} of the exact"
    ratio = S / s_exact[:rank]
    assert ratio.min() >= each, f"{where}: sigma ratio {ratio.min():.4f}"
    assert np.all(S <= s_exact[:rank] * (1 + 4 * U16))  # Ritz values stay below the exact ones
    return cap / opt, S[0] / s_exact[0], ratio.min()


@pytest.mark.parametrize("nbits,g,rank", [(4, 64, 64), (2, 32, 32)])
def test_quantization_residual_against_the_exact_truncation(hq, nbits, g, rank):
    """The device's rank-r compensation of a real quantization residual against the oracle's
    exact truncated SVD of the same residual (codes from the oracle's quantizer)."""
    wl = workloads.WORKLOADS["attn_4096x4096"]
    W = workloads.generate(512, 1024, wl.dist, 11, "cpu").numpy()
    r = oracle.hqq_quantize(W, nbits, g)
    dW = oracle.hqq_residual(W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    B64, A64, s_exact = oracle.lowrank_svd(dW, rank)
    q = _quantized_weight(hq, W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    Wd = _dev16(W).view(torch.float16)
    for seed in (1, 2, 3):
        B, A, S = hq.lowrank(Wd, q, rank, oversample=32, power_iters=4, seed=seed)
        torch.cuda.synchronize()
        B, A, S = (t.cpu().numpy().astype(np.float64) for t in (B, A, S))
        cap, top, each = _check_against_exact(S, s_exact, rank, LOWRANK_FLOORS["512x1024"],
                                              f"b{nbits} g{g} seed {seed}")
        # what B A leaves is the energy not captured, and never below the Eckart-Young value
        left, cap_dev = np.sum((dW - B @ A) ** 2), np.sum(S ** 2)
        assert abs(left - (np.sum(dW ** 2) - cap_dev)) <= 32 * U16 * cap_dev
        assert left >= np.sum(s_exact[rank:] ** 2) * (1 - 16 * U16)
        _say(f"b{nbits} g{g} r={rank} seed {seed}: {cap:.4f} of the exact rank-r energy, "
             f"top sigma {top:.4f}, smallest sigma ratio {each:.4f}")


@pytest.mark.parametrize("nbits,g,rank", [(4, 64, 64), (2, 32, 32)])
def test_quantization_residual_against_the_same_iteration(hq, nbits, g, rank):
    """A numerical check of the matrix-core products only: the device against the same
    iteration run in fp64 with the same test matrix."""
    wl = workloads.WORKLOADS["attn_4096x4096"]
    W = workloads.generate(512, 1024, wl.dist, 11, "cpu").numpy()
    r = oracle.hqq_quantize(W, nbits, g)
    dW = oracle.hqq_residual(W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    s_exact = np.linalg.svd(dW, compute_uv=False)
    over, q_it = 32, 4
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    omega = torch.randn((rank + over, 1024), generator=gen, device="cuda").half()
    q = _quantized_weight(hq, W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
    B, A, S = hq.lowrank(_dev16(W).view(torch.float16), q, rank, oversample=over,
                         power_iters=q_it, omega=omega)
    torch.cuda.synchronize()
    B, A, S = (t.cpu().numpy().astype(np.float64) for t in (B, A, S))
    Be, Ae, Se = _randomized_svd64(dW, omega.cpu().numpy(), rank, q_it)
    rel = np.abs(S - Se) / Se
    assert rel.max() <= 8 * U16, rel.max()
    assert np.all(S <= s_exact[:rank] * (1 + 4 * U16))  # Ritz values stay below the exact ones
    cap_dev, cap_emu, cap_opt = np.sum(S ** 2), np.sum(Se ** 2), np.sum(s_exact[:rank] ** 2)
    assert abs(cap_dev - cap_emu) <= 16 * U16 * cap_emu
    assert np.abs(A @ A.T - np.eye(rank)).max() <= 8 * U16
    res = np.sum((dW - B @ A) ** 2)
    assert abs(res - (np.sum(dW ** 2) - cap_dev)) <= 32 * U16 * cap_dev
    _say(f"b{nbits} g{g} r={rank}: captured {cap_dev / np.sum(dW ** 2):.4f} of |dW|^2 "
         f"({cap_dev / cap_opt:.4f} of the exact truncation's), sigma vs fp64 iteration "
         f"{rel.max():.3g}")


def test_llama70b_matrix_against_the_exact_truncation(hq):
    """A 70B-shaped 8192 x 8192 matrix at full size: the oracle's fp64 residual of the
    device's stored quantization, its exact singular values (LAPACK on the host), and the
    device's rank-64 compensation of the same matrix against them; then the structure of
    the factors."""
    wl = workloads.WORKLOADS["llama70b_stack"]
    m = wl.matrices[0]  # 8192 x 8192
    _say(f"70B {m.rows}x{m.cols} b4 g64, rank 64: against the exact singular values")
    W = workloads.generate(m.rows, m.cols, wl.dist, m.seed, "cuda")
    q = hq.quantize(W, 4, 64)
    B, A, S = hq.lowrank(W, q, 64, oversample=32, power_iters=4, seed=1)
    dW = hq.residual(W, q).float()
    torch.cuda.synchronize()
    dW64 = oracle.hqq_residual(W.cpu().numpy(), q.packed.cpu().numpy(), q.scale.cpu().numpy(),
                               q.zero.cpu().numpy(), 4, 64)
    s_exact = oracle.singular_values(dW64)
    del dW64
    cap, top, each = _check_against_exact(S.cpu().numpy().astype(np.float64), s_exact, 64,
                                          LOWRANK_FLOORS["8192x8192"], "70B 8192x8192")
    _say(f"  {cap:.4f} of the exact rank-64 energy, top sigma {top:.4f}, smallest ratio {each:.4f}")
    assert bool((S[1:] <= S[:-1]).all())
    eye = torch.eye(64, device="cuda")
    assert float((A @ A.T - eye).abs().max()) <= 8 * U16
    G = B.T @ B
    assert float((G - torch.diag(S ** 2)).abs().max()) <= 8 * U16 * float(S[0]) ** 2
    tot = float((dW.double() ** 2).sum())
    res = float(((dW - B @ A).double() ** 2).sum())
    cap = float((S.double() ** 2).sum())
    assert abs(res - (tot - cap)) <= 32 * U16 * cap + 1e-6 * tot
    _say(f"  captured {cap / tot:.4f} of |dW|^2 with rank 64")


def test_concurrent_calls_on_two_streams_match_sequential(hq):
    """Two matrices' calls on streams of their own, each with its own workspace, run at
    the same time and give bit for bit what the same calls give one after the other (the
    library keeps no state between calls, and every sum has a fixed order)."""
    wl = workloads.WORKLOADS["attn_4096x4096"]
    cases = [(512, 1024, 4, 64, 21), (384, 2048, 2, 32, 22)]
    inputs = []
    for rows, cols, nbits, g, seed in cases:
        W = workloads.generate(rows, cols, wl.dist, seed, "cpu").numpy()
        r = oracle.hqq_quantize(W, nbits, g)
        q = _quantized_weight(hq, W, r.packed, r.scale_f16, r.zero_f16, nbits, g)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        omega = torch.randn((64 + 32, cols), generator=gen, device="cuda").half()
        inputs.append((_dev16(W).view(torch.float16), q, omega))
    seq = [hq.lowrank(W, q, 64, oversample=32, power_iters=4, omega=om) for W, q, om in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in inputs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    conc = []
    for s, (W, q, om) in zip(streams, inputs):
        ws = torch.empty(hq.hqq_lowrank_workspace_bytes(W.shape[0], W.shape[1], 64, 32),
                         dtype=torch.uint8, device="cuda")
        conc.append((hq.lowrank(W, q, 64, oversample=32, power_iters=4, omega=om, workspace=ws,
                                stream=s), ws))
    torch.cuda.synchronize()
    for (rows, cols, nbits, g, _), a, (b, _) in zip(cases, seq, conc):
        for x, y in zip(a, b):
            assert torch.equal(x, y), (rows, cols, nbits, g)
        _say(f"{rows}x{cols} b{nbits} g{g}: concurrent call bit-identical to the sequential one")
