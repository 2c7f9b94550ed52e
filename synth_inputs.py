"""Seeded synthetic inputs for the dense-layer training path.

This module only draws random numbers and lays them out; it holds none of the
arithmetic of the method.  Both the HIP path (through tests and bench.py) and
the float64 oracle consume what it returns, so the two sides always see the
same bits.

Draw order is fixed so that a workload is reproducible from its seed alone:
X, labels, then (W_l, b_l) for l = 1..L, then the upstream gradient dY.
All floating-point draws are made in float32 (``standard_normal(dtype=float32)``
then scaled in float32); labels are int32 drawn uniformly from [0, C).

Workloads (shapes from the noeira.nn docs, "A complete example" -- the
784-256-128-10 MLP -- and from the wide-MLP, transformer-MLP and
classifier-head stress shapes this library is measured on):

* ``mlp_small``   784->256->128->10 ReLU MLP, batch 64, SGD(lr=1e-3)
* ``mlp_adamw``   same MLP, batch 8192, 100 AdamW steps on one fixed batch
* ``mlp_wide``    1024->4096->4096->4096->1000 ReLU MLP, batch 16384, SGD
* ``tmlp_bf16``   1024->4096(GELU tanh)->1024, 32768 tokens, bf16 operands
* ``head_xent``   768->32000 linear head + softmax-xent, 65536 rows, AdamW
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

ACT_IDENTITY = 0
ACT_RELU = 1
ACT_GELU_TANH = 2


@dataclasses.dataclass
class Optim:
    kind: str  # "sgd" or "adamw"
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    batch: int
    dims: List[int]             # [in_0, out_0 = in_1, ..., out_{L-1}]
    acts: List[int]             # one per layer
    init: str                   # "kaiming" or "normal002"
    bias: str                   # "zero" or "uniform001"
    dtype: str                  # "f32", "bf16" or "f16"
    optim: Optional[Optim]      # None for fwd+vjp-only workloads
    steps: int = 1
    has_loss: bool = True       # softmax-xent closes the step
    has_dy: bool = False        # an upstream gradient dY is drawn instead

    @property
    def n_layers(self) -> int:
        return len(self.dims) - 1

    @property
    def n_classes(self) -> int:
        return self.dims[-1]

    def gemm_flops_per_step(self) -> int:
        """2*M*N*K summed over fwd, dW and dX (dX skipped for layer 1)."""
        total = 0
        for l in range(self.n_layers):
            mnk = self.batch * self.dims[l] * self.dims[l + 1]
            total += 2 * mnk * (2 if l == 0 else 3)
        return total

    def n_params(self) -> int:
        return sum(self.dims[l] * self.dims[l + 1] + self.dims[l + 1]
                   for l in range(self.n_layers))

    def scaled(self, batch: int) -> "Workload":
        return dataclasses.replace(self, batch=batch)


ADAMW = Optim("adamw", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.01)
SGD = Optim("sgd", lr=1e-3)

WORKLOADS = {
    "mlp_small": Workload("mlp_small", 1, 64, [784, 256, 128, 10],
                          [ACT_RELU, ACT_RELU, ACT_IDENTITY], "kaiming",
                          "zero", "f32", SGD),
    "mlp_adamw": Workload("mlp_adamw", 2, 8192, [784, 256, 128, 10],
                          [ACT_RELU, ACT_RELU, ACT_IDENTITY], "kaiming",
                          "zero", "f32", ADAMW, steps=100),
    "mlp_wide": Workload("mlp_wide", 3, 16384, [1024, 4096, 4096, 4096, 1000],
                         [ACT_RELU, ACT_RELU, ACT_RELU, ACT_IDENTITY],
                         "kaiming", "uniform001", "f32", SGD),
    "tmlp_bf16": Workload("tmlp_bf16", 4, 32768, [1024, 4096, 1024],
                          [ACT_GELU_TANH, ACT_IDENTITY], "normal002", "zero",
                          "bf16", None, has_loss=False, has_dy=True),
    "head_xent": Workload("head_xent", 5, 65536, [768, 32000],
                          [ACT_IDENTITY], "normal002", "zero", "f32", ADAMW),
}


@dataclasses.dataclass
class Inputs:
    X: np.ndarray                 # [B, in_0] float32
    labels: Optional[np.ndarray]  # [B] int32
    W: List[np.ndarray]           # [out_l, in_l] float32 (fp32 master)
    b: List[np.ndarray]           # [out_l] float32
    dY: Optional[np.ndarray]      # [B, out_L] float32 (values bf16-exact when bf16)


def _to_bf16_exact(a: np.ndarray) -> np.ndarray:
    """Make a draw bf16-representable by clearing the low 16 bits of each
    float32 (a property of the draw, not the method's round-to-nearest-even):
    inputs that the workload declares bf16 then reach both sides exactly."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def generate(w: Workload, batch: Optional[int] = None) -> Inputs:
    B = w.batch if batch is None else batch
    rng = np.random.default_rng(w.seed)
    X = rng.standard_normal((B, w.dims[0]), dtype=np.float32)
    labels = None
    if w.has_loss:
        labels = rng.integers(0, w.n_classes, size=B, dtype=np.int32)
    Ws, bs = [], []
    for l in range(w.n_layers):
        fan_in, fan_out = w.dims[l], w.dims[l + 1]
        Wl = rng.standard_normal((fan_out, fan_in), dtype=np.float32)
        if w.init == "kaiming":
            Wl *= np.float32(np.sqrt(2.0 / fan_in))
        else:
            Wl *= np.float32(0.02)
        if w.bias == "zero":
            bl = np.zeros(fan_out, dtype=np.float32)
        else:
            bl = rng.uniform(-0.01, 0.01, size=fan_out).astype(np.float32)
        Ws.append(Wl)
        bs.append(bl)
    dY = None
    if w.has_dy:
        dY = rng.standard_normal((B, w.dims[-1]), dtype=np.float32)
    if w.dtype == "bf16":
        X = _to_bf16_exact(X)
        if dY is not None:
            dY = _to_bf16_exact(dY)
    elif w.dtype == "f16":
        X = X.astype(np.float16).astype(np.float32)
        if dY is not None:
            dY = dY.astype(np.float16).astype(np.float32)
    return Inputs(X, labels, Ws, bs, dY)


def random_matrix(seed: int, shape, scale: float = 1.0,
                  bf16_exact: bool = False, f16_exact: bool = False) -> np.ndarray:
    """Standalone float32 N(0, scale^2) matrix for kernel-level cases.
    bf16_exact / f16_exact make every value representable in that 16-bit
    format (bits cleared, or NumPy's half cast), so such inputs reach both
    sides exactly."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if f16_exact:
        return a.astype(np.float16).astype(np.float32)
    return _to_bf16_exact(a) if bf16_exact else a


def random_labels(seed: int, n: int, n_classes: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, n_classes, size=n, dtype=np.int32)
