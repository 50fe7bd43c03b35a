"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the quantization method: it only draws
weights and activations with the shapes, scales and tails of the workloads
(Llama-3-8B, a 27B model with hidden 5120 / intermediate 17408, Llama-3-70B)
and hands the same tensors to the HIP library and to the CPU oracle.

Every draw goes through a ``torch.Generator`` seeded from
(config, layer, tensor) so that a run is reproducible on a given device.
The CPU and GPU generators produce different streams for the same seed; a
parity check always copies the exact device tensor to the host.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------

LLAMA8B = {            # name -> (N rows, K cols); y = W x with W [N, K]
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}
LLAMA8B_LAYERS = 32

QWEN27B = {            # hidden 5120, intermediate 17408, 8 KV heads x 128
    "q": (5120, 5120), "k": (1024, 5120), "v": (1024, 5120), "o": (5120, 5120),
    "gate": (17408, 5120), "up": (17408, 5120), "down": (5120, 17408),
}
QWEN27B_LAYERS = 64

LLAMA70B = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
LLAMA70B_LAYERS = 80

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}

# The decode step feeds one activation to q|k|v and one to gate|up, so the
# row-concatenated groups are what a GEMV launch sees.
LLAMA8B_GROUPS = {
    "qkv": (4096 + 1024 + 1024, 4096), "o": (4096, 4096),
    "gate_up": (2 * 14336, 4096), "down": (4096, 14336),
}


def seed_of(config: int, layer: int = 0, tensor: int = 0, salt: int = 0) -> int:
    return (config * 1_000_003 + layer * 10_007 + tensor * 101 + salt) & 0x7FFF_FFFF_FFFF


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def add_outliers(w: torch.Tensor, frac: float, factor: float, g: torch.Generator) -> torch.Tensor:
    """Multiply exactly round(frac * numel) distinct, uniformly drawn entries by ``factor``."""
    n = w.numel()
    count = int(round(frac * n))
    if count == 0:
        return w
    pos = torch.randperm(n, generator=g, device=w.device)[:count]
    flat = w.reshape(-1)
    flat[pos] = flat[pos] * factor
    return w


def normal_weight(n: int, k: int, std: float, g: torch.Generator, device, dtype) -> torch.Tensor:
    w = torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std
    return w.to(dtype)


def student_t4_weight(n: int, k: int, g: torch.Generator, device, dtype) -> torch.Tensor:
    """Student-t with 4 degrees of freedom, scaled to variance 1/K.

    t = z / sqrt(chi2_4 / 4) with chi2_4 the sum of four squared normals;
    Var(t_4) = 2, so the scale is sqrt(1 / (2K)).
    """
    z = torch.randn(n, k, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros_like(z)
    for _ in range(4):
        e = torch.randn(n, k, generator=g, device=device, dtype=torch.float32)
        chi += e * e
    t = z / torch.sqrt(chi / 4.0)
    return (t * math.sqrt(1.0 / (2.0 * k))).to(dtype)


def activation(m: int, k: int, g: torch.Generator, device, dtype) -> torch.Tensor:
    return torch.randn(m, k, generator=g, device=device, dtype=torch.float32).to(dtype)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def tiny_tq(device="cpu", seed: int = 1):
    """W fp32 [256, 512] ~ N(0, 0.02^2) with 0.1% of entries x10; x fp32 [512] ~ N(0, 1)."""
    g = generator(seed, device)
    w = normal_weight(256, 512, 0.02, g, device, torch.float32)
    w = add_outliers(w, 0.001, 10.0, g)
    x = activation(1, 512, g, device, torch.float32)[0]
    return w, x


def llama8b_weight(name: str, layer: int, device, variant: str = "gauss", dtype=torch.bfloat16,
                   rows: int | None = None):
    """One Llama-3-8B-shaped tensor: bf16 N(0, 1/K) or the Student-t(4) variant."""
    n, k = LLAMA8B[name]
    if rows is not None:
        n = rows
    g = generator(seed_of(2, layer, TENSOR_IDS[name], salt=0 if variant == "gauss" else 7), device)
    if variant == "t4":
        return student_t4_weight(n, k, g, device, dtype)
    return normal_weight(n, k, 1.0 / math.sqrt(k), g, device, dtype)


def layer_variant(layer: int) -> str:
    """Even layers Gaussian, odd layers Student-t(4): both tails in every stream."""
    return "gauss" if layer % 2 == 0 else "t4"


def qwen27b_weight(name: str, layer: int, device, dtype=torch.bfloat16, rows: int | None = None):
    """27B-shaped tensor: bf16 N(0, 1/K) with 0.1% of entries x20."""
    n, k = QWEN27B[name]
    if rows is not None:
        n = rows
    g = generator(seed_of(4, layer, TENSOR_IDS[name]), device)
    w = normal_weight(n, k, 1.0 / math.sqrt(k), g, device, torch.float32)
    w = add_outliers(w, 0.001, 20.0, g)
    return w.to(dtype)


def qwen27b_format(layer: int, name: str) -> str:
    """Seeded per-tensor format choice: MXFP6 with probability 0.1, else NVFP4."""
    g = generator(seed_of(4, layer, TENSOR_IDS[name], salt=99), "cpu")
    return "mxfp6" if torch.rand(1, generator=g).item() < 0.1 else "nvfp4"


def llama70b_layer_drift(layer: int) -> float:
    """Per-layer std multiplier ~ U(0.5, 2), one draw per layer."""
    g = generator(seed_of(5, layer, 0, salt=1), "cpu")
    return 0.5 + 1.5 * torch.rand(1, generator=g).item()


def llama70b_weight(name: str, layer: int, device, dtype=torch.bfloat16, rows: int | None = None):
    n, k = LLAMA70B[name]
    if rows is not None:
        n = rows
    g = generator(seed_of(5, layer, TENSOR_IDS[name]), device)
    std = llama70b_layer_drift(layer) / math.sqrt(k)
    return normal_weight(n, k, std, g, device, dtype)


@dataclass(frozen=True)
class Shape:
    name: str
    n: int
    k: int

    @property
    def weights(self) -> int:
        return self.n * self.k
