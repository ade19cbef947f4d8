"""Seeded synthetic inputs for the NF4+DQ LoRA linear.

This module holds no arithmetic of the method: it only draws Gaussian tensors with
fixed seeds, so the HIP path and the CPU oracle can be fed identical data.  The
distributions follow the pages' model of weights (zero-mean normal, "QLoRA -- Fine-Tuning
a 65B Model on One GPU", section "NF4") at the sizes of the workloads below.

Seed rule: 1000*cfg + 10*linear_idx + t (+ 100000*layer), t in {W:0, X:1, A:2, B:3, dY:4}.
BF16 tensors are drawn in FP32 and cast with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses

import torch

T_W, T_X, T_A, T_B, T_DY = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class LinearShape:
    name: str
    d_out: int
    d_in: int


# Workload shapes (d_out x d_in)
LLAMA7B_QPROJ = [LinearShape("q_proj", 4096, 4096)]
LLAMA3_8B_LAYER = [
    LinearShape("q_proj", 4096, 4096),
    LinearShape("k_proj", 1024, 4096),
    LinearShape("v_proj", 1024, 4096),
    LinearShape("o_proj", 4096, 4096),
    LinearShape("gate_proj", 14336, 4096),
    LinearShape("up_proj", 14336, 4096),
    LinearShape("down_proj", 4096, 14336),
]
SEVENTY_B_LAYER = [
    LinearShape("q_proj", 8192, 8192),
    LinearShape("k_proj", 1024, 8192),
    LinearShape("v_proj", 1024, 8192),
    LinearShape("o_proj", 8192, 8192),
    LinearShape("gate_proj", 28672, 8192),
    LinearShape("up_proj", 28672, 8192),
    LinearShape("down_proj", 8192, 28672),
]

WORKLOADS = {
    1: dict(name="single-linear-256x256", shapes=[LinearShape("linear", 256, 256)], w_std=0.02, r=8, alpha=16.0, Ms=[4]),
    2: dict(name="llama7b-qproj-4096x4096-stream", shapes=LLAMA7B_QPROJ, w_std=0.02, r=16, alpha=32.0, Ms=[1, 16]),
    3: dict(name="llama7b-qproj-4096x4096-M4096-train", shapes=LLAMA7B_QPROJ, w_std=0.02, r=16, alpha=32.0, Ms=[4096]),
    4: dict(name="llama3-8b-layer-M8192-train", shapes=LLAMA3_8B_LAYER, w_std=0.02, r=16, alpha=32.0, Ms=[8192]),
    5: dict(name="70b-class-80-layer-stream", shapes=SEVENTY_B_LAYER, w_std=0.015, r=16, alpha=32.0, Ms=[1, 2048], layers=80),
}


def seed_for(cfg: int, linear_idx: int, t: int, layer: int = 0) -> int:
    return 1000 * cfg + 10 * linear_idx + t + 100000 * layer


def _randn(shape, seed: int, std: float, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device) * std


def weight(cfg: int, linear_idx: int, d_out: int, d_in: int, std: float, layer: int = 0, device="cpu") -> torch.Tensor:
    """FP32 W[d_out, d_in] ~ N(0, std^2)."""
    return _randn((d_out, d_in), seed_for(cfg, linear_idx, T_W, layer), std, device)


def activations(cfg: int, linear_idx: int, M: int, d_in: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """BF16 X[M, d_in] ~ N(0, 1)."""
    return _randn((M, d_in), seed_for(cfg, linear_idx, T_X, layer), 1.0, device).to(torch.bfloat16)


def lora_A(cfg: int, linear_idx: int, r: int, d_in: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """BF16 A[r, d_in] ~ N(0, 1/d_in)."""
    return _randn((r, d_in), seed_for(cfg, linear_idx, T_A, layer), d_in**-0.5, device).to(torch.bfloat16)


def lora_B(cfg: int, linear_idx: int, d_out: int, r: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """BF16 B[d_out, r] ~ N(0, 0.01^2)."""
    return _randn((d_out, r), seed_for(cfg, linear_idx, T_B, layer), 0.01, device).to(torch.bfloat16)


def grad_out(cfg: int, linear_idx: int, M: int, d_out: int, layer: int = 0, device="cpu") -> torch.Tensor:
    """BF16 dY[M, d_out] ~ N(0, 1e-2) (variance 1e-2, std 0.1)."""
    return _randn((M, d_out), seed_for(cfg, linear_idx, T_DY, layer), 0.1, device).to(torch.bfloat16)


def linear_case(cfg: int, linear_idx: int, d_out: int, d_in: int, M: int, r: int, w_std: float, layer: int = 0, device="cpu"):
    """All inputs of one linear: W (FP32), X, A, B, dY (BF16)."""
    return dict(
        W=weight(cfg, linear_idx, d_out, d_in, w_std, layer, device),
        X=activations(cfg, linear_idx, M, d_in, layer, device),
        A=lora_A(cfg, linear_idx, r, d_in, layer, device),
        B=lora_B(cfg, linear_idx, d_out, r, layer, device),
        dY=grad_out(cfg, linear_idx, M, d_out, layer, device),
    )


# Trainable adapter parameters of the Llama-3-8B layer shapes above with r = 16 on all seven
# linears, over 32 layers: 32 * 16 * sum(d_out + d_in) = 41,943,040 (the pages' 41.9M).
LLAMA3_8B_ADAPTER_PARAMS = 32 * 16 * sum(s.d_out + s.d_in for s in LLAMA3_8B_LAYER)


def optimizer_state(seed: int, n: int, device="cpu"):
    """Flat AdamW inputs for n adapter parameters: FP32 master ~ N(0, 0.02^2), FP32 first
    moment ~ N(0, (1e-3)^2), FP32 second moment ~ U(0, 1e-6), BF16 gradient ~ N(0, (1e-3)^2)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    master = torch.randn(n, generator=g, device=device) * 0.02
    m = torch.randn(n, generator=g, device=device) * 1e-3
    v = torch.rand(n, generator=g, device=device) * 1e-6
    grad = (torch.randn(n, generator=g, device=device) * 1e-3).to(torch.bfloat16)
    return master, m, v, grad
