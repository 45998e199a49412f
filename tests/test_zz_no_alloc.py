"""The no-allocation whole-tensor stop (hqq_quantize_tensor_stop_noalloc, through the C ABI)
against the entry point with a caller workspace (hqq_quantize_tensor_stop).

The two share every kernel; only the scratch differs (a static device array inside the
library instead of the caller's workspace), so the outputs, the totals E_t and t* must be
bit-identical.  Two calls in a row, the second on a smaller input with fewer steps, show
that the array keeps no state a later call depends on; the outputs are first filled with
a pattern, so a call that wrote nothing would fail too.  The totals of the first call are
recomputed independently by the oracle-compared path (hqq_quantize_tensor_stop) only.
"""
import ctypes

import numpy as np
import pytest

import workloads

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
    print(f"[gpu-no-alloc] {msg}", flush=True)


def _buffers(rows, cols, nbits, g, iters):
    dev = "cuda"
    ng = rows * cols // g
    b = {"packed": torch.full((rows * cols * nbits // 8,), 0xA5, dtype=torch.uint8, device=dev),
         "scale": torch.full((ng,), 7.0, dtype=torch.float16, device=dev),
         "zero": torch.full((ng,), -3.0, dtype=torch.float16, device=dev),
         "zero32": torch.full((ng,), -1.0, dtype=torch.float32, device=dev),
         "stop": torch.full((ng,), 255, dtype=torch.uint8, device=dev),
         "totals": torch.full((iters + 1,), -1.0, dtype=torch.float64, device=dev),
         "t_star": torch.full((1,), -1, dtype=torch.int32, device=dev)}
    return b


def _call(hq, noalloc, W, nbits, g, iters, b, workspace=None):
    rows, cols = W.shape
    opts = hq.hqq_options_t(1, 0, b["zero32"].data_ptr(), b["stop"].data_ptr(), 0, 0, 0, 0)
    args = (W.data_ptr(), rows, cols, nbits, g, 0.7, 1.0, 1.01, iters, b["packed"].data_ptr(),
            b["scale"].data_ptr(), b["zero"].data_ptr(), opts, b["totals"].data_ptr(),
            b["t_star"].data_ptr())
    sh = torch.cuda.current_stream().cuda_stream
    if noalloc:
        st = hq.hqq_quantize_tensor_stop_noalloc(*args, sh)
    else:
        st = hq.hqq_quantize_tensor_stop(*args, workspace.data_ptr(), sh)
    assert st == hq.HQQ_OK, hq.hqq_status_string(st)


def _same(a, b):
    for k in a:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_noalloc_tensor_stop_equals_the_workspace_entry_point(hq):
    wl = workloads.WORKLOADS["attn_4096x4096"]
    cases = [(1024, 4096, 4, 64, 20, 31), (300, 512, 2, 32, 7, 32)]  # the second smaller
    for rows, cols, nbits, g, iters, seed in cases:
        _say(f"{rows}x{cols} b{nbits} g{g} iters {iters}: noalloc vs workspace entry point")
        W = workloads.generate(rows, cols, wl.dist, seed, "cuda")
        ws = torch.empty(hq.hqq_tensor_stop_workspace_bytes(iters), dtype=torch.uint8,
                         device="cuda")
        ref = _buffers(rows, cols, nbits, g, iters)
        out = _buffers(rows, cols, nbits, g, iters)
        _call(hq, False, W, nbits, g, iters, ref, ws)
        _call(hq, True, W, nbits, g, iters, out)
        torch.cuda.synchronize()
        _same(ref, out)
        t = int(out["t_star"].item())
        assert 0 <= t <= iters and bool((out["stop"] == t).all())
        E = out["totals"].cpu().numpy()
        assert np.all(np.diff(E[:t + 1]) < 0) and (t == iters or E[t + 1] >= E[t])
        _say(f"  bit-identical; t* = {t}, E_0 = {E[0]:.6g}, E_t* = {E[t]:.6g}")
    assert hq.hqq_tensor_stop_noalloc_max_bytes() >= hq.hqq_tensor_stop_workspace_bytes(255)
    assert ctypes.sizeof(hq.hqq_options_t) > 0
