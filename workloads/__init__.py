"""Seeded synthetic weight matrices and the workload table.

This module holds no arithmetic of the quantization method: it only draws
random fp16 matrices with the layer shapes and heavy-tailed value distributions
of the Llama-2 linear layers that the HQQ page quantizes ("Half-Quadratic
Quantization of Large Machine Learning Models", sections 3 and 4.1), which are
not available here.  Both the HIP path and the oracle read the same fp16 bits
produced here, which is the only thing the two sides share.

Recipe (per matrix):
  * a ``torch.Generator`` on the target device, seeded with the matrix seed;
  * N(0, sigma): sigma * Z;
  * Student-t with integer nu: Z0 / sqrt((Z1^2 + ... + Znu^2) / nu), drawn in
    that order, rescaled to standard deviation sigma by sqrt((nu - 2) / nu);
  * outliers: k = round(frac * N) distinct flat indices, the first k of
    ``randperm(N)`` from the same generator, multiplied by ``factor``;
  * everything in fp32, then one cast to fp16 (round to nearest even).
Streams differ between CPU and GPU generators; a parity test always feeds the
very same fp16 bits to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Dist:
    kind: str            # "normal" or "student_t"
    std: float
    nu: int = 0
    outlier_frac: float = 0.0
    outlier_factor: float = 1.0


@dataclass(frozen=True)
class Matrix:
    rows: int
    cols: int
    seed: int


@dataclass(frozen=True)
class Solver:
    """Solver settings of section 4.1 of the HQQ page."""
    p: float = 0.7
    beta: float = 1.0
    kappa: float = 1.01
    iters: int = 20
    early_stop: bool = True


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    dist: Dist
    matrices: tuple
    settings: tuple      # ((nbits, group_size), ...)
    solver: Solver = field(default_factory=Solver)

    @property
    def weights(self) -> int:
        return sum(m.rows * m.cols for m in self.matrices)


def _stack(layers: int, shapes, seed_base: int):
    mats = []
    for layer in range(layers):
        for m, (r, c) in enumerate(shapes):
            mats.append(Matrix(r, c, seed_base + 16 * layer + m))
    return tuple(mats)


_S7B = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
_S70B = [(8192, 8192)] * 2 + [(1024, 8192)] * 2 + [(28672, 8192)] * 2 + [(8192, 28672)]

WORKLOADS = {
    "single_256x512": Workload(
        "single_256x512", "one 256x512 matrix, N(0,0.02) with 0.1% x20 outliers",
        Dist("normal", 0.02, outlier_frac=0.001, outlier_factor=20.0),
        (Matrix(256, 512, 1),), ((4, 64),)),
    "attn_4096x4096": Workload(
        "attn_4096x4096", "one 4096x4096 attention-projection matrix, Student-t nu=4, std 0.02",
        Dist("student_t", 0.02, nu=4), (Matrix(4096, 4096, 2),), ((4, 64),)),
    "mlp_11008x4096": Workload(
        "mlp_11008x4096", "11008x4096 and 4096x11008 MLP matrices, Student-t nu=3, std 0.02, "
        "0.05% x50 outliers",
        Dist("student_t", 0.02, nu=3, outlier_frac=0.0005, outlier_factor=50.0),
        (Matrix(11008, 4096, 3), Matrix(4096, 11008, 4)), ((2, 16), (2, 32))),
    "llama7b_stack": Workload(
        "llama7b_stack", "7B-shaped stack: 32 layers x {4x 4096x4096, 2x 11008x4096, "
        "1x 4096x11008}, Student-t nu=4, std 0.02",
        Dist("student_t", 0.02, nu=4), _stack(32, _S7B, 100000), ((4, 64), (3, 64))),
    "llama70b_stack": Workload(
        "llama70b_stack", "70B-shaped stack: 80 layers x {2x 8192x8192, 2x 1024x8192, "
        "2x 28672x8192, 1x 8192x28672}, Student-t nu=4, std 0.015",
        Dist("student_t", 0.015, nu=4), _stack(80, _S70B, 200000), ((2, 32), (4, 64))),
}


def generate(rows: int, cols: int, dist: Dist, seed: int, device="cpu") -> torch.Tensor:
    """Draw one rows x cols fp16 matrix with the recipe in the module docstring."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    shape = (rows, cols)
    if dist.kind == "normal":
        w = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).mul_(dist.std)
    elif dist.kind == "student_t":
        nu = int(dist.nu)
        if nu <= 2:
            raise ValueError("Student-t needs nu > 2 for a finite standard deviation")
        w = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        chi = torch.zeros(shape, device=dev, dtype=torch.float32)
        for _ in range(nu):
            z = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
            chi.addcmul_(z, z)
            del z
        chi.div_(nu).sqrt_()
        w.div_(chi)
        del chi
        w.mul_(dist.std * ((nu - 2) / nu) ** 0.5)
    else:
        raise ValueError(f"unknown distribution {dist.kind!r}")
    n = rows * cols
    k = int(round(dist.outlier_frac * n))
    if k > 0:
        idx = torch.randperm(n, generator=gen, device=dev)[:k]
        flat = w.view(-1)
        flat[idx] = flat[idx] * dist.outlier_factor
        del idx
    return w.to(torch.float16)


def generate_matrix(workload: Workload, index: int, device="cpu") -> torch.Tensor:
    m = workload.matrices[index]
    return generate(m.rows, m.cols, workload.dist, m.seed, device)
