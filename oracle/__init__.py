"""fp64 CPU oracle for group-wise HQQ quantization -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``bit_weight_quantization_amd``) never imports it, and this package imports
nothing from the product path.

The arithmetic lives in ``hqq_oracle.c`` (plain C, fp64, one thread), which
follows the page "Half-Quadratic Quantization of Large Machine Learning
Models": section 2 (objective, quantizer Q and Q^-1, half-quadratic split with
s fixed, alternating updates), section 2.1 (lp shrink), section 2.2 (closed
form z mean with the inverse scale), section 4.1 (default parameters, early
exit).  This module only marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hqq_oracle.c")
_LIB = os.path.join(_HERE, "libhqq_oracle.so")

# Plain IEEE fp64: no contraction into FMA, no fast-math.
GCC_CMD = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-o", _LIB, _SRC, "-lm"]


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    subprocess.run(GCC_CMD, check=True, cwd=_HERE)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    D, I, I64 = ctypes.c_double, ctypes.c_int, ctypes.c_int64
    P = ctypes.c_void_p
    lib.oracle_f16_to_f64.restype = D
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_f64_to_f16.argtypes = [D]
    lib.oracle_f16_to_f64_array.argtypes = [P, I64, P]
    lib.oracle_f64_to_f16_array.argtypes = [P, I64, P]
    lib.oracle_shrink_lp.restype = D
    lib.oracle_shrink_lp.argtypes = [D, D, D]
    lib.oracle_quantize_value.restype = D
    lib.oracle_quantize_value.argtypes = [D, D, D, I]
    lib.oracle_round_ratio.restype = D
    lib.oracle_round_ratio.argtypes = [D, D]
    lib.oracle_quantize_init_value.restype = D
    lib.oracle_quantize_init_value.argtypes = [D, D, D, I]
    lib.oracle_minmax_init.argtypes = [P, I, I, P, P, P]
    lib.oracle_group_error.restype = D
    lib.oracle_group_error.argtypes = [P, I, D]
    lib.oracle_z_update.restype = D
    lib.oracle_z_update.argtypes = [P, P, P, D, I]
    lib.oracle_hqq_group.restype = I
    lib.oracle_hqq_group.argtypes = [P, I, I, D, D, D, I, I, D, P, P, P, P]
    lib.oracle_hqq_group_replay.restype = I
    lib.oracle_hqq_group_replay.argtypes = [P, I, I, D, D, D, I, I, D, P, P, P, P, P, I, P, P, I, P]
    lib.oracle_packed_bytes.restype = I64
    lib.oracle_packed_bytes.argtypes = [I64, I]
    lib.oracle_pack_codes.argtypes = [P, I64, I, P]
    lib.oracle_unpack_codes.argtypes = [P, I64, I, P]
    lib.oracle_hqq_quantize.restype = I
    lib.oracle_hqq_quantize.argtypes = [P, I64, I64, I, I, D, D, D, I, I, D] + [P] * 9
    lib.oracle_hqq_dequantize.restype = I
    lib.oracle_hqq_dequantize.argtypes = [P, P, P, I64, I64, I, I, P]
    lib.oracle_hqq_quantize_tensor_stop.restype = I
    lib.oracle_hqq_quantize_tensor_stop.argtypes = [P, I64, I64, I, I, D, D, D, I, D] + [P] * 10
    lib.oracle_meta_quantize.restype = I64
    lib.oracle_meta_quantize.argtypes = [P, I64, I64, P, P, P]
    lib.oracle_meta_dequantize.restype = I
    lib.oracle_meta_dequantize.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_hqq_residual.restype = I
    lib.oracle_hqq_residual.argtypes = [P, P, P, P, I64, I64, I, I, P]
    lib.oracle_hqq_matmul.restype = I
    lib.oracle_hqq_matmul.argtypes = [P, I64, I64, P, P, P, I64, I, I, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class _GroupResult(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("inv_scale", ctypes.c_double),
                ("zero", ctypes.c_double), ("stop_step", ctypes.c_int),
                ("err_init", ctypes.c_double), ("err_best", ctypes.c_double),
                ("n_eval", ctypes.c_int)]


# ---------------------------------------------------------------- binary16 ---

def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_f16_to_f64_array(_ptr(bits), bits.size, _ptr(out))
    return out


def f64_to_f16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_f64_to_f16_array(_ptr(v), v.size, _ptr(out))
    return out


# ------------------------------------------------------------------ steps ---

def shrink_lp(x: float, beta: float, p: float) -> float:
    return _load().oracle_shrink_lp(float(x), float(beta), float(p))


def quantize_value(w: float, inv_s: float, z: float, qmax: int) -> float:
    return _load().oracle_quantize_value(float(w), float(inv_s), float(z), int(qmax))


def round_ratio(num: float, den: float) -> float:
    return _load().oracle_round_ratio(float(num), float(den))


def quantize_init_value(w: float, mn: float, mx: float, qmax: int) -> float:
    return _load().oracle_quantize_init_value(float(w), float(mn), float(mx), int(qmax))


def minmax_init(w: np.ndarray, nbits: int):
    w = np.ascontiguousarray(w, dtype=np.float64)
    s, inv_s, z = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _load().oracle_minmax_init(_ptr(w), w.size, (1 << nbits) - 1, ctypes.byref(s),
                               ctypes.byref(inv_s), ctypes.byref(z))
    return s.value, inv_s.value, z.value


def group_error(r: np.ndarray, err_pow: float) -> float:
    r = np.ascontiguousarray(r, dtype=np.float64)
    return _load().oracle_group_error(_ptr(r), r.size, float(err_pow))


def z_update(q, w, we, inv_s: float) -> float:
    q = np.ascontiguousarray(q, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    we = np.ascontiguousarray(we, dtype=np.float64)
    return _load().oracle_z_update(_ptr(q), _ptr(w), _ptr(we), float(inv_s), q.size)


@dataclass
class GroupResult:
    codes: np.ndarray
    scale: float
    inv_scale: float
    zero: float
    stop_step: int
    err_init: float
    err_best: float
    n_eval: int
    trace: np.ndarray


def hqq_group(w, nbits: int, p: float = 0.7, beta: float = 1.0, kappa: float = 1.01,
              iters: int = 20, early_stop: bool = True, err_pow: float | None = None) -> GroupResult:
    """One group through the solver (fp64).  ``err_pow`` defaults to ``p``."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    g = w.size
    codes = np.empty(g, np.uint8)
    trace = np.empty(iters + 1, np.float64)
    n_trace = ctypes.c_int()
    res = _GroupResult()
    rc = _load().oracle_hqq_group(_ptr(w), g, nbits, float(p), float(beta), float(kappa), int(iters),
                                  int(bool(early_stop)), float(p if err_pow is None else err_pow),
                                  _ptr(codes), ctypes.byref(res), _ptr(trace), ctypes.byref(n_trace))
    if rc != 0:
        raise ValueError("oracle_hqq_group rejected its arguments")
    return GroupResult(codes, res.scale, res.inv_scale, res.zero, res.stop_step, res.err_init,
                       res.err_best, res.n_eval, trace[: n_trace.value].copy())


def hqq_group_replay(w, nbits: int, flips=(), inverts=(), p: float = 0.7, beta: float = 1.0,
                     kappa: float = 1.01, iters: int = 20, early_stop: bool = True,
                     err_pow: float | None = None):
    """hqq_group with the codes of (evaluation, element) pairs in ``flips`` moved to the
    other rounding neighbour and the stop decision of the evaluations in ``inverts``
    inverted; also returns the z of every evaluation.  Test infrastructure for showing
    that a divergent device trajectory left the oracle's at a rounding or error tie."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    g = w.size
    codes = np.empty(g, np.uint8)
    trace = np.empty(iters + 1, np.float64)
    ztr = np.empty(iters + 1, np.float64)
    n_trace = ctypes.c_int()
    res = _GroupResult()
    fe = np.ascontiguousarray([f[0] for f in flips] or [0], dtype=np.int32)
    fk = np.ascontiguousarray([f[1] for f in flips] or [0], dtype=np.int32)
    rc = _load().oracle_hqq_group_replay(
        _ptr(w), g, nbits, float(p), float(beta), float(kappa), int(iters), int(bool(early_stop)),
        float(p if err_pow is None else err_pow), _ptr(codes), ctypes.byref(res), _ptr(trace),
        _ptr(ztr), ctypes.byref(n_trace), len(flips), _ptr(fe), _ptr(fk), len(inverts),
        _ptr(np.ascontiguousarray(list(inverts) or [0], dtype=np.int32)))
    if rc != 0:
        raise ValueError("oracle_hqq_group_replay rejected its arguments")
    n = n_trace.value
    return GroupResult(codes, res.scale, res.inv_scale, res.zero, res.stop_step, res.err_init,
                       res.err_best, res.n_eval, trace[:n].copy()), ztr[:n].copy()


# ---------------------------------------------------------------- packing ---

def packed_bytes(n: int, nbits: int) -> int:
    return _load().oracle_packed_bytes(int(n), int(nbits))


def pack_codes(codes: np.ndarray, nbits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.empty(packed_bytes(codes.size, nbits), np.uint8)
    _load().oracle_pack_codes(_ptr(codes), codes.size, nbits, _ptr(out))
    return out


def unpack_codes(packed: np.ndarray, n: int, nbits: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(n, np.uint8)
    _load().oracle_unpack_codes(_ptr(packed), n, nbits, _ptr(out))
    return out


# ----------------------------------------------------------- whole matrix ---

@dataclass
class QuantResult:
    packed: np.ndarray      # uint8, rows*cols*nbits/8
    scale_f16: np.ndarray   # uint16 bits, rows x cols/g
    zero_f16: np.ndarray    # uint16 bits, rows x cols/g
    scale: np.ndarray       # float64
    zero: np.ndarray        # float64
    stop_step: np.ndarray   # uint8
    err_init: np.ndarray    # float64
    err_best: np.ndarray    # float64
    codes: np.ndarray       # uint8, rows x cols


def hqq_quantize(W_f16_bits: np.ndarray, nbits: int, group_size: int, p: float = 0.7,
                 beta: float = 1.0, kappa: float = 1.01, iters: int = 20,
                 early_stop: bool = True, err_pow: float | None = None) -> QuantResult:
    """Quantize a rows x cols matrix given as binary16 bit patterns (uint16)."""
    W = np.ascontiguousarray(W_f16_bits)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    assert W.dtype == np.uint16 and W.ndim == 2
    rows, cols = W.shape
    if cols % group_size:
        raise ValueError("cols must be a multiple of group_size")
    ng = rows * cols // group_size
    mshape = (rows, cols // group_size)
    out = QuantResult(
        packed=np.empty(packed_bytes(rows * cols, nbits), np.uint8),
        scale_f16=np.empty(mshape, np.uint16), zero_f16=np.empty(mshape, np.uint16),
        scale=np.empty(mshape, np.float64), zero=np.empty(mshape, np.float64),
        stop_step=np.empty(mshape, np.uint8), err_init=np.empty(mshape, np.float64),
        err_best=np.empty(mshape, np.float64), codes=np.empty((rows, cols), np.uint8))
    assert ng == out.scale.size
    rc = _load().oracle_hqq_quantize(
        _ptr(W), rows, cols, nbits, group_size, float(p), float(beta), float(kappa), int(iters),
        int(bool(early_stop)), float(p if err_pow is None else err_pow), _ptr(out.packed),
        _ptr(out.scale_f16), _ptr(out.zero_f16), _ptr(out.scale), _ptr(out.zero),
        _ptr(out.stop_step), _ptr(out.err_init), _ptr(out.err_best), _ptr(out.codes))
    if rc != 0:
        raise ValueError("oracle_hqq_quantize rejected its arguments")
    return out


def hqq_quantize_tensor_stop(W_f16_bits: np.ndarray, nbits: int, group_size: int,
                             p: float = 0.7, beta: float = 1.0, kappa: float = 1.01,
                             iters: int = 20, err_pow: float | None = None):
    """Whole-tensor early stop (hqq_oracle.c, oracle_hqq_quantize_tensor_stop).
    Returns (QuantResult, t_star, E) with E the total error of every step 0..iters."""
    W = np.ascontiguousarray(W_f16_bits)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    assert W.dtype == np.uint16 and W.ndim == 2
    rows, cols = W.shape
    mshape = (rows, cols // group_size)
    out = QuantResult(
        packed=np.empty(packed_bytes(rows * cols, nbits), np.uint8),
        scale_f16=np.empty(mshape, np.uint16), zero_f16=np.empty(mshape, np.uint16),
        scale=np.empty(mshape, np.float64), zero=np.empty(mshape, np.float64),
        stop_step=np.empty(mshape, np.uint8), err_init=np.empty(mshape, np.float64),
        err_best=np.empty(mshape, np.float64), codes=np.empty((rows, cols), np.uint8))
    E = np.empty(iters + 1, np.float64)
    t_star = _load().oracle_hqq_quantize_tensor_stop(
        _ptr(W), rows, cols, nbits, group_size, float(p), float(beta), float(kappa), int(iters),
        float(p if err_pow is None else err_pow), _ptr(E), _ptr(out.packed), _ptr(out.scale_f16),
        _ptr(out.zero_f16), _ptr(out.scale), _ptr(out.zero), _ptr(out.stop_step),
        _ptr(out.err_init), _ptr(out.err_best), _ptr(out.codes))
    if t_star < 0:
        raise ValueError("oracle_hqq_quantize_tensor_stop rejected its arguments")
    return out, t_star, E


def hqq_dequantize(packed: np.ndarray, scale_f16: np.ndarray, zero_f16: np.ndarray, rows: int,
                   cols: int, nbits: int, group_size: int) -> np.ndarray:
    """Return the binary16 bit patterns of s*(W_q - z), rounded once from fp64."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scale_f16 = np.ascontiguousarray(scale_f16).view(np.uint16)
    zero_f16 = np.ascontiguousarray(zero_f16).view(np.uint16)
    out = np.empty((rows, cols), np.uint16)
    rc = _load().oracle_hqq_dequantize(_ptr(packed), _ptr(scale_f16), _ptr(zero_f16), rows, cols,
                                       nbits, group_size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_hqq_dequantize rejected its arguments")
    return out


def meta_groups(n: int, group: int) -> int:
    """Number of meta groups: 1 for group = 0 (one group of all n values), else ceil(n/group)."""
    if n == 0:
        return 0
    return 1 if group == 0 else -(-n // group)


def meta_quantize(values_f16: np.ndarray, group: int):
    """8-bit min-max meta quantization (hqq_oracle.c, oracle_meta_quantize) of binary16 bit
    patterns in groups of `group` (0 = one group).  Returns (codes u8, scale16, offset16)."""
    v = np.ascontiguousarray(values_f16).view(np.uint16).ravel()
    n = v.size
    ng = meta_groups(n, group)
    codes = np.empty(n, np.uint8)
    sc = np.empty(max(ng, 1), np.uint16)
    off = np.empty(max(ng, 1), np.uint16)
    rc = _load().oracle_meta_quantize(_ptr(v), n, group, _ptr(codes), _ptr(sc), _ptr(off))
    if rc != ng:
        raise ValueError("oracle_meta_quantize rejected its arguments")
    return codes, sc[:ng], off[:ng]


def meta_dequantize(codes: np.ndarray, scale16: np.ndarray, offset16: np.ndarray,
                    group: int) -> np.ndarray:
    """binary16 bit patterns of offset + scale * code, rounded once from fp64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    sc = np.ascontiguousarray(scale16).view(np.uint16).ravel()
    off = np.ascontiguousarray(offset16).view(np.uint16).ravel()
    out = np.empty(codes.size, np.uint16)
    rc = _load().oracle_meta_dequantize(_ptr(codes), _ptr(sc), _ptr(off), codes.size, group,
                                        _ptr(out))
    if rc != 0:
        raise ValueError("oracle_meta_dequantize rejected its arguments")
    return out


def hqq_matmul(X_f16: np.ndarray, packed: np.ndarray, scale_f16: np.ndarray,
               zero_f16: np.ndarray, N: int, nbits: int, group_size: int) -> np.ndarray:
    """Y = X Q^-1(W_q)^T in fp64 (hqq_oracle.c, oracle_hqq_matmul): X is M x K binary16
    (bit patterns or float16), the weight N x K as hqq_quantize stores it."""
    X = np.ascontiguousarray(X_f16)
    if X.dtype == np.float16:
        X = X.view(np.uint16)
    assert X.dtype == np.uint16 and X.ndim == 2
    M, K = X.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    sc = np.ascontiguousarray(scale_f16).view(np.uint16).ravel()
    zr = np.ascontiguousarray(zero_f16).view(np.uint16).ravel()
    assert sc.size == N * (K // group_size) and zr.size == sc.size
    assert packed.size >= (N * K * nbits + 7) // 8
    Y = np.empty((M, N), np.float64)
    rc = _load().oracle_hqq_matmul(_ptr(X), M, K, _ptr(packed), _ptr(sc), _ptr(zr), N, nbits,
                                   group_size, _ptr(Y))
    if rc != 0:
        raise ValueError("oracle_hqq_matmul rejected its arguments")
    return Y


def hqq_residual(W_f16: np.ndarray, packed: np.ndarray, scale_f16: np.ndarray,
                 zero_f16: np.ndarray, nbits: int, group_size: int) -> np.ndarray:
    """Delta W = W - s (W_q - z) in fp64 (hqq_oracle.c, oracle_hqq_residual)."""
    W = np.ascontiguousarray(W_f16)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    assert W.dtype == np.uint16 and W.ndim == 2
    rows, cols = W.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8).ravel()
    sc = np.ascontiguousarray(scale_f16).view(np.uint16).ravel()
    zr = np.ascontiguousarray(zero_f16).view(np.uint16).ravel()
    assert sc.size == rows * (cols // group_size) and zr.size == sc.size
    out = np.empty((rows, cols), np.float64)
    rc = _load().oracle_hqq_residual(_ptr(W), _ptr(packed), _ptr(sc), _ptr(zr), rows, cols, nbits,
                                     group_size, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_hqq_residual rejected its arguments")
    return out


def singular_values(dW: np.ndarray) -> np.ndarray:
    """All singular values of Delta W in decreasing order (fp64, LAPACK as the library
    step): the exact rank-r truncation of the EoRA page's plain SVD compensation captures
    the sum of the r largest squares of them."""
    return np.linalg.svd(np.asarray(dW, np.float64), compute_uv=False)


def lowrank_svd(dW: np.ndarray, rank: int):
    """The LoRA factors of the plain SVD compensation (EoRA page, section 1): with
    Delta W = U Sigma V^T (singular values in decreasing order), B = U_r Sigma_r (rows x r)
    and A = V_r^T (r x cols), so that B A is the best rank-r approximation of Delta W in
    the Frobenius norm.  fp64, LAPACK's SVD as the library step.  Returns (B, A, sigma)
    with sigma all min(rows, cols) singular values.  Each pair of singular vectors is
    signed so that the largest-magnitude entry of the column of A^T is positive (the
    SVD fixes the pair only up to a common sign)."""
    dW = np.asarray(dW, np.float64)
    U, sig, Vt = np.linalg.svd(dW, full_matrices=False)
    r = min(rank, sig.size)
    U, S, Vt = U[:, :r], sig[:r], Vt[:r]
    flip = np.sign(Vt[np.arange(r), np.argmax(np.abs(Vt), axis=1)])
    flip[flip == 0] = 1.0
    B = U * (S * flip)
    A = Vt * flip[:, None]
    return B, A, sig
