"""MI355X (gfx950) group-wise HQQ weight quantizer: thin Python binding.

Every step of the quantization runs in the HIP kernels of ``libhqq_mi355x.so``
(built from ``csrc/`` by ``build.py``); this module only marshals arguments
through ctypes.  PyTorch provides device memory and the current stream.  There
is no fallback: if the library is missing or no device is usable, calls raise.

Low-level functions carry the names of the C ABI in ``include/hqq.h`` and take
raw device addresses; :func:`quantize` and :func:`dequantize` wrap them for
torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhqq_mi355x.so")

HQQ_OK = 0
HQQ_ERR_INVALID_ARG = 1
HQQ_ERR_UNSUPPORTED = 2
HQQ_ERR_ALIGNMENT = 3
HQQ_ERR_LAUNCH = 4
HQQ_ERR_TABLE_MISMATCH = 5

# Symbols declared in include/hqq.h.
EXPORTED_SYMBOLS = ("hqq_quantize", "hqq_quantize_ex", "hqq_quantize_batch", "hqq_dequantize",
                    "hqq_quantize_tensor_stop", "hqq_tensor_stop_workspace_bytes", "hqq_matmul",
                    "hqq_matmul_workspace_bytes",
                    "hqq_residual", "hqq_lowrank", "hqq_lowrank_workspace_bytes",
                    "hqq_meta_quantize", "hqq_meta_dequantize", "hqq_meta_groups",
                    "hqq_meta_workspace_bytes", "hqq_meta_quantize_batch",
                    "hqq_packed_bytes", "hqq_num_groups", "hqq_status_string",
                    "hqq_quantize_tensor_stop_noalloc", "hqq_tensor_stop_noalloc_max_bytes")


class HQQError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {hqq_status_string(status)} (status {status})")
        self.status = status


class hqq_options_t(ctypes.Structure):
    _fields_ = [("early_stop", ctypes.c_int),
                ("scale_f32", ctypes.c_void_p), ("zero_f32", ctypes.c_void_p),
                ("stop_step", ctypes.c_void_p), ("err_init", ctypes.c_void_p),
                ("err_best", ctypes.c_void_p), ("refill_threshold", ctypes.c_int),
                ("err_metric", ctypes.c_int)]


class hqq_batch_entry_t(ctypes.Structure):
    _fields_ = [("W_f16", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("first_group", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m bit_weight_quantization_amd.build`")
    lib = ctypes.CDLL(path)
    I, I64, F, P = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.hqq_quantize.restype = I
    lib.hqq_quantize.argtypes = [P, I64, I64, I, I, F, F, F, I, P, P, P, P]
    lib.hqq_quantize_ex.restype = I
    lib.hqq_quantize_ex.argtypes = [P, I64, I64, I, I, F, F, F, I, P, P, P,
                                    ctypes.POINTER(hqq_options_t), P]
    lib.hqq_quantize_tensor_stop.restype = I
    lib.hqq_quantize_tensor_stop.argtypes = [P, I64, I64, I, I, F, F, F, I, P, P, P,
                                             ctypes.POINTER(hqq_options_t), P, P, P, P]
    lib.hqq_quantize_tensor_stop_noalloc.restype = I
    lib.hqq_quantize_tensor_stop_noalloc.argtypes = [P, I64, I64, I, I, F, F, F, I, P, P, P,
                                                     ctypes.POINTER(hqq_options_t), P, P, P]
    lib.hqq_tensor_stop_noalloc_max_bytes.restype = I64
    lib.hqq_tensor_stop_noalloc_max_bytes.argtypes = []
    lib.hqq_residual.restype = I
    lib.hqq_residual.argtypes = [P, P, P, P, I64, I64, I, I, P, P, P]
    lib.hqq_lowrank.restype = I
    lib.hqq_lowrank.argtypes = [P, P, P, P, I64, I64, I, I, I, I, I, P, P, P, P, P, P]
    lib.hqq_lowrank_workspace_bytes.restype = I64
    lib.hqq_lowrank_workspace_bytes.argtypes = [I64, I64, I, I]
    lib.hqq_matmul.restype = I
    lib.hqq_matmul.argtypes = [P, I64, I64, P, P, P, I64, I, I, P, I, P, P]
    lib.hqq_matmul_workspace_bytes.restype = I64
    lib.hqq_matmul_workspace_bytes.argtypes = [I64, I64, I64, I, I]
    lib.hqq_tensor_stop_workspace_bytes.restype = I64
    lib.hqq_tensor_stop_workspace_bytes.argtypes = [I]
    lib.hqq_quantize_batch.restype = I
    lib.hqq_quantize_batch.argtypes = [ctypes.POINTER(hqq_batch_entry_t), P, I, I, I, F, F, F, I,
                                       P, P, P, P, P]
    lib.hqq_meta_quantize.restype = I
    lib.hqq_meta_quantize.argtypes = [P, I64, I64, P, P, P, P, P]
    lib.hqq_meta_dequantize.restype = I
    lib.hqq_meta_dequantize.argtypes = [P, P, P, I64, I64, P, P]
    lib.hqq_meta_groups.restype = I64
    lib.hqq_meta_groups.argtypes = [I64, I64]
    lib.hqq_meta_quantize_batch.restype = I
    lib.hqq_meta_quantize_batch.argtypes = [ctypes.POINTER(hqq_batch_entry_t), P, I, I, P, I64, P,
                                            P, P, P, P]
    lib.hqq_meta_workspace_bytes.restype = I64
    lib.hqq_meta_workspace_bytes.argtypes = []
    lib.hqq_dequantize.restype = I
    lib.hqq_dequantize.argtypes = [P, P, P, I64, I64, I, I, P, P]
    lib.hqq_packed_bytes.restype = I64
    lib.hqq_packed_bytes.argtypes = [I64, I64, I]
    lib.hqq_num_groups.restype = I64
    lib.hqq_num_groups.argtypes = [I64, I64, I]
    lib.hqq_status_string.restype = ctypes.c_char_p
    lib.hqq_status_string.argtypes = [I]
    _lib = lib
    return lib


# ------------------------------------------------------------- C ABI names --

def hqq_status_string(status: int) -> str:
    return load_library().hqq_status_string(int(status)).decode()


def hqq_packed_bytes(rows: int, cols: int, nbits: int) -> int:
    return load_library().hqq_packed_bytes(rows, cols, nbits)


def hqq_num_groups(rows: int, cols: int, group_size: int) -> int:
    return load_library().hqq_num_groups(rows, cols, group_size)


def hqq_quantize(W_f16: int, rows: int, cols: int, nbits: int, group_size: int, p: float,
                 beta: float, kappa: float, iters: int, packed_codes: int, scale_f16: int,
                 zero_f16: int, stream: int = 0) -> int:
    return load_library().hqq_quantize(W_f16, rows, cols, nbits, group_size, p, beta, kappa,
                                       iters, packed_codes, scale_f16, zero_f16, stream)


def hqq_quantize_ex(W_f16: int, rows: int, cols: int, nbits: int, group_size: int, p: float,
                    beta: float, kappa: float, iters: int, packed_codes: int, scale_f16: int,
                    zero_f16: int, options: Optional[hqq_options_t], stream: int = 0) -> int:
    opt = ctypes.byref(options) if options is not None else None
    return load_library().hqq_quantize_ex(W_f16, rows, cols, nbits, group_size, p, beta, kappa,
                                          iters, packed_codes, scale_f16, zero_f16, opt, stream)


def hqq_quantize_tensor_stop(W_f16: int, rows: int, cols: int, nbits: int, group_size: int,
                             p: float, beta: float, kappa: float, iters: int, packed_codes: int,
                             scale_f16: int, zero_f16: int, options: Optional[hqq_options_t],
                             totals_f64: int, t_star_i32: int, workspace: int,
                             stream: int = 0) -> int:
    opt = ctypes.byref(options) if options is not None else None
    return load_library().hqq_quantize_tensor_stop(W_f16, rows, cols, nbits, group_size, p, beta,
                                                   kappa, iters, packed_codes, scale_f16, zero_f16,
                                                   opt, totals_f64, t_star_i32, workspace, stream)


def hqq_quantize_tensor_stop_noalloc(W_f16: int, rows: int, cols: int, nbits: int,
                                     group_size: int, p: float, beta: float, kappa: float,
                                     iters: int, packed_codes: int, scale_f16: int,
                                     zero_f16: int, options: Optional[hqq_options_t],
                                     totals_f64: int, t_star_i32: int, stream: int = 0) -> int:
    opt = ctypes.byref(options) if options is not None else None
    return load_library().hqq_quantize_tensor_stop_noalloc(
        W_f16, rows, cols, nbits, group_size, p, beta, kappa, iters, packed_codes, scale_f16,
        zero_f16, opt, totals_f64, t_star_i32, stream)


def hqq_tensor_stop_noalloc_max_bytes() -> int:
    return load_library().hqq_tensor_stop_noalloc_max_bytes()


def hqq_matmul(X_f16: int, M: int, K: int, packed_codes: int, scale_f16: int, zero_f16: int,
               N: int, nbits: int, group_size: int, Y: int, out_f32: int, workspace: int = 0,
               stream: int = 0) -> int:
    return load_library().hqq_matmul(X_f16, M, K, packed_codes, scale_f16, zero_f16, N, nbits,
                                     group_size, Y, out_f32, workspace, stream)


def hqq_matmul_workspace_bytes(M: int, N: int, K: int, nbits: int, group_size: int) -> int:
    return load_library().hqq_matmul_workspace_bytes(M, N, K, nbits, group_size)


def hqq_residual(W_f16: int, packed_codes: int, scale_f16: int, zero_f16: int, rows: int,
                 cols: int, nbits: int, group_size: int, dW_f16: int, dWT_f16: int,
                 stream: int = 0) -> int:
    return load_library().hqq_residual(W_f16, packed_codes, scale_f16, zero_f16, rows, cols, nbits,
                                       group_size, dW_f16, dWT_f16, stream)


def hqq_lowrank(W_f16: int, packed_codes: int, scale_f16: int, zero_f16: int, rows: int,
                cols: int, nbits: int, group_size: int, rank: int, oversample: int,
                power_iters: int, omega_f16: int, B_f32: int, A_f32: int, sigma_f32: int,
                workspace: int, stream: int = 0) -> int:
    return load_library().hqq_lowrank(W_f16, packed_codes, scale_f16, zero_f16, rows, cols, nbits,
                                      group_size, rank, oversample, power_iters, omega_f16, B_f32,
                                      A_f32, sigma_f32, workspace, stream)


def hqq_lowrank_workspace_bytes(rows: int, cols: int, rank: int, oversample: int) -> int:
    return load_library().hqq_lowrank_workspace_bytes(rows, cols, rank, oversample)


def hqq_tensor_stop_workspace_bytes(iters: int) -> int:
    return load_library().hqq_tensor_stop_workspace_bytes(iters)


def hqq_quantize_batch(entries, entries_device: int, count: int, nbits: int, group_size: int,
                       p: float, beta: float, kappa: float, iters: int, packed_codes: int,
                       scale_f16: int, zero_f16: int, status_device: int, stream: int = 0) -> int:
    """``entries``: a ctypes array of ``hqq_batch_entry_t`` (host copy)."""
    return load_library().hqq_quantize_batch(entries, entries_device, count, nbits, group_size, p,
                                             beta, kappa, iters, packed_codes, scale_f16, zero_f16,
                                             status_device, stream)


def hqq_meta_groups(n: int, meta_group: int) -> int:
    return load_library().hqq_meta_groups(n, meta_group)


def hqq_meta_workspace_bytes() -> int:
    return load_library().hqq_meta_workspace_bytes()


def hqq_meta_quantize(values_f16: int, n: int, meta_group: int, codes_u8: int, mscale_f16: int,
                      moffset_f16: int, workspace: int = 0, stream: int = 0) -> int:
    return load_library().hqq_meta_quantize(values_f16, n, meta_group, codes_u8, mscale_f16,
                                            moffset_f16, workspace, stream)


def hqq_meta_quantize_batch(entries, entries_device: int, count: int, group_size: int,
                            values_f16: int, meta_group: int, codes_u8: int, mscale_f16: int,
                            moffset_f16: int, workspace: int = 0, stream: int = 0) -> int:
    return load_library().hqq_meta_quantize_batch(entries, entries_device, count, group_size,
                                                  values_f16, meta_group, codes_u8, mscale_f16,
                                                  moffset_f16, workspace, stream)


def hqq_meta_dequantize(codes_u8: int, mscale_f16: int, moffset_f16: int, n: int,
                        meta_group: int, values_f16: int, stream: int = 0) -> int:
    return load_library().hqq_meta_dequantize(codes_u8, mscale_f16, moffset_f16, n, meta_group,
                                              values_f16, stream)


def hqq_dequantize(packed_codes: int, scale_f16: int, zero_f16: int, rows: int, cols: int,
                   nbits: int, group_size: int, W_out_f16: int, stream: int = 0) -> int:
    return load_library().hqq_dequantize(packed_codes, scale_f16, zero_f16, rows, cols, nbits,
                                         group_size, W_out_f16, stream)


# ----------------------------------------------------------- torch helpers --

@dataclass
class QuantizedWeight:
    packed: "torch.Tensor"            # uint8, hqq_packed_bytes(rows, cols, nbits)
    scale: "torch.Tensor"             # fp16, rows x cols/group_size
    zero: "torch.Tensor"              # fp16, rows x cols/group_size (code units)
    rows: int
    cols: int
    nbits: int
    group_size: int
    scale_f32: Optional["torch.Tensor"] = None
    zero_f32: Optional["torch.Tensor"] = None
    stop_step: Optional["torch.Tensor"] = None
    err_init: Optional["torch.Tensor"] = None
    err_best: Optional["torch.Tensor"] = None


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _addr(t) -> int:
    return int(t.data_ptr()) if t is not None else 0


def _alloc_on(stream):
    """Context for allocating the outputs of a launch on ``stream``: the caching allocator
    then ties them to that stream, so memory the caller drops early is not handed to
    other streams while the launch may still write it."""
    import contextlib

    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _check_tensor(t, name: str, dtype, numel: int, shape=None):
    import torch
    if t is None or not isinstance(t, torch.Tensor):
        raise ValueError(f"out.{name} is missing")
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"out.{name} must be a contiguous {dtype} CUDA tensor")
    if t.numel() != numel or (shape is not None and tuple(t.shape) != tuple(shape)):
        raise ValueError(f"out.{name} has {tuple(t.shape)}, expected {shape or (numel,)}")


def quantize(W, nbits: int, group_size: int, p: float = 0.7, beta: float = 1.0,
             kappa: float = 1.01, iters: int = 20, early_stop: bool = True, debug: bool = False,
             out: Optional[QuantizedWeight] = None, stream=None,
             refill_threshold: int = 0, err_metric: int = 0) -> QuantizedWeight:
    """Quantize a contiguous rows x cols fp16 CUDA tensor on the given (or current) stream.

    ``out`` may supply preallocated output tensors (reused as-is).  With ``debug`` the
    fp32 s and z, the stop step and the initial/best errors per group are returned too.
    """
    out = _outputs(W, nbits, group_size, debug, out, "quantize", stream)
    rows, cols = W.shape
    opts = None
    if debug or not early_stop or refill_threshold or err_metric:
        opts = _options(out, debug, early_stop, refill_threshold, err_metric)
    st = hqq_quantize_ex(_addr(W), rows, cols, nbits, group_size, float(p), float(beta),
                         float(kappa), int(iters), _addr(out.packed), _addr(out.scale),
                         _addr(out.zero), opts, _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_quantize_ex")
    return out


def quantize_tensor_stop(W, nbits: int, group_size: int, p: float = 0.7, beta: float = 1.0,
                         kappa: float = 1.01, iters: int = 20, debug: bool = False,
                         err_metric: int = 0, out: Optional[QuantizedWeight] = None,
                         workspace=None, stream=None):
    """Quantize with the early stop taken over the whole matrix (hqq_quantize_tensor_stop).

    Returns ``(QuantizedWeight, totals, t_star)`` where ``totals`` is a float64 CUDA tensor
    of the iters + 1 total errors E_t and ``t_star`` a one-element int32 CUDA tensor (both
    filled on the stream; read them after synchronizing).  ``workspace`` may supply a uint8
    CUDA tensor of at least hqq_tensor_stop_workspace_bytes(iters) bytes.
    """
    import torch
    out = _outputs(W, nbits, group_size, debug, out, "quantize_tensor_stop", stream)
    rows, cols = W.shape
    wb = hqq_tensor_stop_workspace_bytes(int(iters))
    if wb < 0:
        raise HQQError(HQQ_ERR_INVALID_ARG, "quantize_tensor_stop")
    with _alloc_on(stream):
        if workspace is None:
            workspace = torch.empty(wb, dtype=torch.uint8, device=W.device)
        elif workspace.numel() < wb or not workspace.is_cuda:
            raise ValueError(f"workspace needs {wb} bytes of device memory")
        totals = torch.empty(int(iters) + 1, dtype=torch.float64, device=W.device)
        t_star = torch.empty(1, dtype=torch.int32, device=W.device)
    opts = _options(out, debug, True, 0, err_metric)
    st = hqq_quantize_tensor_stop(_addr(W), rows, cols, nbits, group_size, float(p), float(beta),
                                  float(kappa), int(iters), _addr(out.packed), _addr(out.scale),
                                  _addr(out.zero), opts, _addr(totals), _addr(t_star),
                                  _addr(workspace), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_quantize_tensor_stop")
    return out, totals, t_star


def _outputs(W, nbits: int, group_size: int, debug: bool, out: Optional[QuantizedWeight],
             where: str, stream=None) -> QuantizedWeight:
    """Checks W, checks a supplied ``out`` against W's shape and the settings, and
    allocates the output tensors that ``out`` does not supply."""
    import torch
    if W.dtype != torch.float16 or W.dim() != 2 or not W.is_cuda or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D float16 CUDA tensor")
    rows, cols = W.shape
    ng = hqq_num_groups(rows, cols, group_size)
    nb = hqq_packed_bytes(rows, cols, nbits)
    if ng < 0 or nb < 0:
        raise HQQError(HQQ_ERR_INVALID_ARG if nb >= 0 else HQQ_ERR_UNSUPPORTED, where)
    dev = W.device
    shp = (rows, cols // group_size)
    if out is not None:
        if (out.rows, out.cols, out.nbits, out.group_size) != (rows, cols, nbits, group_size):
            raise ValueError(f"{where}: out was made for {out.rows}x{out.cols} b{out.nbits} "
                             f"g{out.group_size}, not {rows}x{cols} b{nbits} g{group_size}")
        _check_tensor(out.packed, "packed", torch.uint8, nb)
        _check_tensor(out.scale, "scale", torch.float16, ng, shp)
        _check_tensor(out.zero, "zero", torch.float16, ng, shp)
        if debug and out.stop_step is not None:
            for name, dt in (("scale_f32", torch.float32), ("zero_f32", torch.float32),
                             ("stop_step", torch.uint8), ("err_init", torch.float32),
                             ("err_best", torch.float32)):
                _check_tensor(getattr(out, name), name, dt, ng, shp)
    with _alloc_on(stream):
        if out is None:
            out = QuantizedWeight(
                packed=torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)[:nb],
                scale=torch.empty(shp, dtype=torch.float16, device=dev),
                zero=torch.empty(shp, dtype=torch.float16, device=dev),
                rows=rows, cols=cols, nbits=nbits, group_size=group_size)
        if debug and out.stop_step is None:
            out.scale_f32 = torch.empty(shp, dtype=torch.float32, device=dev)
            out.zero_f32 = torch.empty(shp, dtype=torch.float32, device=dev)
            out.stop_step = torch.empty(shp, dtype=torch.uint8, device=dev)
            out.err_init = torch.empty(shp, dtype=torch.float32, device=dev)
            out.err_best = torch.empty(shp, dtype=torch.float32, device=dev)
    return out


def _options(out: QuantizedWeight, debug: bool, early_stop: bool, refill_threshold: int,
             err_metric: int) -> hqq_options_t:
    return hqq_options_t(int(bool(early_stop)), _addr(out.scale_f32 if debug else None),
                         _addr(out.zero_f32 if debug else None),
                         _addr(out.stop_step if debug else None),
                         _addr(out.err_init if debug else None),
                         _addr(out.err_best if debug else None), int(refill_threshold),
                         int(err_metric))


def matmul(X, q: "QuantizedWeight", out_f32: bool = False, out=None, workspace=None,
           stream=None):
    """Y = X Q^-1(W_q)^T (hqq_matmul) for a contiguous M x K float16 CUDA tensor X and a
    weight quantized as q (rows = N outputs, cols = K inputs).  Returns an M x N float16
    (or float32) tensor, or fills ``out``.  ``workspace`` may supply a uint8 CUDA tensor of
    at least hqq_matmul_workspace_bytes(M, N, K, nbits, group_size) bytes."""
    import torch
    if X.dtype != torch.float16 or X.dim() != 2 or not X.is_cuda or not X.is_contiguous():
        raise ValueError("X must be a contiguous 2-D float16 CUDA tensor")
    M, K = X.shape
    if K != q.cols:
        raise ValueError(f"X has {K} columns, the weight {q.cols}")
    dt = torch.float32 if out_f32 else torch.float16
    wb = hqq_matmul_workspace_bytes(M, q.rows, K, q.nbits, q.group_size)
    if wb < 0:
        raise HQQError(HQQ_ERR_INVALID_ARG, "hqq_matmul")
    with _alloc_on(stream):
        if out is None:
            out = torch.empty((M, q.rows), dtype=dt, device=X.device)
        if wb > 0 and workspace is None:
            workspace = torch.empty(wb, dtype=torch.uint8, device=X.device)
    if out.dtype != dt or tuple(out.shape) != (M, q.rows) or not out.is_contiguous():
        raise ValueError("out has the wrong dtype or shape")
    if wb > 0 and (workspace.numel() < wb or not workspace.is_cuda):
        raise ValueError(f"workspace needs {wb} bytes of device memory")
    st = hqq_matmul(_addr(X), M, K, _addr(q.packed), _addr(q.scale), _addr(q.zero), q.rows,
                    q.nbits, q.group_size, _addr(out), int(bool(out_f32)),
                    _addr(workspace) if wb > 0 else 0, _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_matmul")
    return out


def residual(W, q: "QuantizedWeight", transposed: bool = False, stream=None):
    """Delta W = W - Q^-1(W_q) as float16 (hqq_residual); with ``transposed`` also its
    transpose.  Returns dW or (dW, dWT)."""
    import torch
    with _alloc_on(stream):
        dW = torch.empty_like(W)
        dWT = torch.empty((W.shape[1], W.shape[0]), dtype=W.dtype, device=W.device) if transposed else None
    st = hqq_residual(_addr(W), _addr(q.packed), _addr(q.scale), _addr(q.zero), q.rows, q.cols,
                      q.nbits, q.group_size, _addr(dW), _addr(dWT), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_residual")
    return (dW, dWT) if transposed else dW


def lowrank(W, q: "QuantizedWeight", rank: int, oversample: int = 32, power_iters: int = 4,
            omega=None, seed: int = 0, workspace=None, stream=None):
    """LoRA factors (B: rows x rank, A: rank x cols, sigma) of the quantization error of W
    under q (hqq_lowrank).  ``omega`` may supply the (rank + oversample) x cols float16 test
    matrix; otherwise it is drawn from a standard normal with ``seed`` on W's device."""
    import torch
    rows, cols = W.shape
    width = rank + oversample
    if omega is None:
        gen = torch.Generator(device=W.device)
        gen.manual_seed(int(seed))
        omega = torch.randn((width, cols), generator=gen, device=W.device).half()
    wb = hqq_lowrank_workspace_bytes(rows, cols, rank, oversample)
    if wb < 0:
        raise HQQError(HQQ_ERR_INVALID_ARG, "lowrank")
    with _alloc_on(stream):
        if workspace is None:
            workspace = torch.empty(wb, dtype=torch.uint8, device=W.device)
        B = torch.empty((rows, rank), dtype=torch.float32, device=W.device)
        A = torch.empty((rank, cols), dtype=torch.float32, device=W.device)
        sigma = torch.empty(rank, dtype=torch.float32, device=W.device)
    st = hqq_lowrank(_addr(W), _addr(q.packed), _addr(q.scale), _addr(q.zero), rows, cols, q.nbits,
                     q.group_size, rank, oversample, power_iters, _addr(omega), _addr(B), _addr(A),
                     _addr(sigma), _addr(workspace), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_lowrank")
    return B, A, sigma


@dataclass
class QuantizedBatch:
    """Outputs of :func:`quantize_batch`: one arena for all matrices, in list order."""
    packed: "torch.Tensor"            # uint8, total_groups * group_size * nbits / 8
    scale: "torch.Tensor"             # fp16, total_groups
    zero: "torch.Tensor"              # fp16, total_groups (code units)
    shapes: list                      # (rows, cols) per matrix
    first_group: list                 # first group index per matrix
    nbits: int
    group_size: int
    table: "torch.Tensor"             # device copy of the entry table (kept for the launch)
    status: "torch.Tensor"            # int32 status word the launch writes (table check)

    def check(self) -> None:
        """Synchronizes on the status word and raises if the launch found its device
        entry table different from the validated host table (then it wrote nothing)."""
        st = int(self.status.item())
        if st != HQQ_OK:
            raise HQQError(st, "hqq_quantize_batch")

    def matrix(self, i: int) -> QuantizedWeight:
        """Views of matrix i's outputs (no copy)."""
        rows, cols = self.shapes[i]
        g0, ng = self.first_group[i], rows * cols // self.group_size
        b0 = g0 * self.group_size * self.nbits // 8
        nb = ng * self.group_size * self.nbits // 8
        return QuantizedWeight(packed=self.packed[b0:b0 + nb],
                               scale=self.scale[g0:g0 + ng].view(rows, cols // self.group_size),
                               zero=self.zero[g0:g0 + ng].view(rows, cols // self.group_size),
                               rows=rows, cols=cols, nbits=self.nbits, group_size=self.group_size)


def batch_table(Ws, group_size: int):
    """Host entry table (ctypes array) for a list of contiguous 2-D fp16 CUDA tensors."""
    entries = (hqq_batch_entry_t * max(len(Ws), 1))()
    total = 0
    for i, W in enumerate(Ws):
        rows, cols = W.shape
        entries[i].W_f16 = _addr(W)
        entries[i].rows, entries[i].cols, entries[i].first_group = rows, cols, total
        total += rows * cols // group_size
    return entries, total


def quantize_batch(Ws, nbits: int, group_size: int, p: float = 0.7, beta: float = 1.0,
                   kappa: float = 1.01, iters: int = 20, out: Optional[QuantizedBatch] = None,
                   stream=None) -> QuantizedBatch:
    """Quantize a list of contiguous rows x cols fp16 CUDA tensors in one launch.

    Results equal those of :func:`quantize` on each tensor; the outputs go to one arena
    (``QuantizedBatch.matrix(i)`` gives the views of tensor i).  ``out`` may supply a
    previous result for the same shapes, whose buffers and entry table are reused.
    """
    import torch
    for W in Ws:
        if W.dtype != torch.float16 or W.dim() != 2 or not W.is_cuda or not W.is_contiguous():
            raise ValueError("every W must be a contiguous 2-D float16 CUDA tensor")
    entries, total = batch_table(Ws, group_size)
    nb = total * group_size * nbits // 8
    table_bytes = max(len(Ws), 1) * ctypes.sizeof(hqq_batch_entry_t)
    shapes = [tuple(W.shape) for W in Ws]
    if out is None:
        dev = Ws[0].device if Ws else torch.device("cuda")
        starts, g = [], 0
        for W in Ws:
            starts.append(g)
            g += W.numel() // group_size
        with _alloc_on(stream):
            out = QuantizedBatch(
                packed=torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)[:nb],
                scale=torch.empty(total, dtype=torch.float16, device=dev),
                zero=torch.empty(total, dtype=torch.float16, device=dev),
                shapes=shapes, first_group=starts, nbits=nbits, group_size=group_size,
                table=torch.empty(table_bytes, dtype=torch.uint8, device=dev),
                status=torch.empty(1, dtype=torch.int32, device=dev))
    else:  # reuse only an arena made for exactly these shapes and settings
        if (list(out.shapes) != shapes or out.nbits != nbits or out.group_size != group_size):
            raise ValueError("quantize_batch: out was made for other shapes, nbits or group_size")
        _check_tensor(out.packed, "packed", torch.uint8, nb)
        _check_tensor(out.scale, "scale", torch.float16, total)
        _check_tensor(out.zero, "zero", torch.float16, total)
        _check_tensor(out.table, "table", torch.uint8, table_bytes)
        _check_tensor(out.status, "status", torch.int32, 1)
    host = torch.frombuffer(bytearray(bytes(entries)), dtype=torch.uint8)
    out.table.copy_(host, non_blocking=False)
    st = hqq_quantize_batch(entries, _addr(out.table), len(Ws), nbits, group_size, float(p),
                            float(beta), float(kappa), int(iters), _addr(out.packed),
                            _addr(out.scale), _addr(out.zero), _addr(out.status),
                            _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_quantize_batch")
    return out


@dataclass
class MetaQuantized:
    """8-bit meta quantization of a per-group array (codes, binary16 meta scale and offset)."""
    codes: "torch.Tensor"             # uint8, n
    scale: "torch.Tensor"             # fp16, hqq_meta_groups(n, meta_group)
    offset: "torch.Tensor"            # fp16, hqq_meta_groups(n, meta_group)
    n: int
    meta_group: int
    workspace: Optional["torch.Tensor"] = None  # kept alive until the launch has completed


def meta_quantize(values, meta_group: int, workspace=None, stream=None) -> MetaQuantized:
    """8-bit meta quantization of a contiguous fp16 CUDA tensor (e.g. ``QuantizedWeight.zero``
    with meta_group 0, ``QuantizedWeight.scale`` with meta_group 128)."""
    import torch
    if values.dtype != torch.float16 or not values.is_cuda or not values.is_contiguous():
        raise ValueError("values must be a contiguous float16 CUDA tensor")
    n = values.numel()
    ng = hqq_meta_groups(n, meta_group)
    if ng < 0:
        raise HQQError(HQQ_ERR_INVALID_ARG, "meta_quantize")
    dev = values.device
    with _alloc_on(stream):
        out = MetaQuantized(codes=torch.empty(n, dtype=torch.uint8, device=dev),
                            scale=torch.empty(ng, dtype=torch.float16, device=dev),
                            offset=torch.empty(ng, dtype=torch.float16, device=dev),
                            n=n, meta_group=meta_group)
        if meta_group == 0 and workspace is None:
            workspace = torch.empty(hqq_meta_workspace_bytes(), dtype=torch.uint8, device=dev)
    out.workspace = workspace
    st = hqq_meta_quantize(_addr(values), n, meta_group, _addr(out.codes), _addr(out.scale),
                           _addr(out.offset), _addr(workspace), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_meta_quantize")
    return out


def meta_quantize_batch(b: "QuantizedBatch", which: str, meta_group: int, stream=None,
                        entries=None) -> MetaQuantized:
    """Meta-quantize the zero (``which="zero"``, meta_group 0: one group per matrix) or scale
    (meta_group dividing every matrix's group count) arena of a :func:`quantize_batch` result
    in one launch sequence."""
    import torch
    values = b.zero if which == "zero" else b.scale
    n = values.numel()
    count = len(b.shapes)
    if entries is None:
        entries = (hqq_batch_entry_t * max(count, 1))()
        for i, ((rows, cols), g0) in enumerate(zip(b.shapes, b.first_group)):
            entries[i].W_f16, entries[i].rows, entries[i].cols, entries[i].first_group = \
                0, rows, cols, g0
    ng = count if meta_group == 0 else (n // meta_group if meta_group else 0)
    dev = values.device
    with _alloc_on(stream):
        out = MetaQuantized(codes=torch.empty(n, dtype=torch.uint8, device=dev),
                            scale=torch.empty(ng, dtype=torch.float16, device=dev),
                            offset=torch.empty(ng, dtype=torch.float16, device=dev),
                            n=n, meta_group=meta_group)
        if meta_group == 0:
            out.workspace = torch.empty(max(8 * count, 4), dtype=torch.uint8, device=dev)
    st = hqq_meta_quantize_batch(entries, _addr(b.table), count, b.group_size, _addr(values),
                                 meta_group, _addr(out.codes), _addr(out.scale), _addr(out.offset),
                                 _addr(out.workspace), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_meta_quantize_batch")
    return out


def meta_dequantize(m: MetaQuantized, out=None, stream=None):
    """offset + scale * code as a flat fp16 tensor of n values (single rounding)."""
    import torch
    if out is None:
        with _alloc_on(stream):
            out = torch.empty(m.n, dtype=torch.float16, device=m.codes.device)
    else:
        _check_tensor(out, "values", torch.float16, m.n)
    st = hqq_meta_dequantize(_addr(m.codes), _addr(m.scale), _addr(m.offset), m.n, m.meta_group,
                             _addr(out), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_meta_dequantize")
    return out


def dequantize(q: QuantizedWeight, out=None, stream=None):
    """Return s*(W_q - z) as a rows x cols fp16 tensor (single rounding from the exact value)."""
    import torch
    if out is None:
        with _alloc_on(stream):
            out = torch.empty((q.rows, q.cols), dtype=torch.float16, device=q.scale.device)
    else:
        _check_tensor(out, "W", torch.float16, q.rows * q.cols, (q.rows, q.cols))
    st = hqq_dequantize(_addr(q.packed), _addr(q.scale), _addr(q.zero), q.rows, q.cols, q.nbits,
                        q.group_size, _addr(out), _stream_handle(stream))
    if st != HQQ_OK:
        raise HQQError(st, "hqq_dequantize")
    return out
