"""Seeded synthetic inputs for the W4 + dynamic LoRA linear.

Shared by the tests, the smoke check and the benchmark; it holds none of the method's arithmetic
(no quantization, no decoding, no contraction) -- only seeded draws of the value distributions the
workloads name:
    x   ~ N(0, 1)      as bf16   (activation)
    pqs ~ U[0.5, 2]    as fp32   (per-input-channel pre_quant_scale)
    W   ~ N(0, 0.02)   as fp32   (weight before NVFP4 quantization)
    A,B ~ N(0, 0.01)   as bf16   (LoRA factors)
where N(0, s) names the standard deviation s. Draws use torch's seeded generators on the device
the tensor is made on; the same tensor is then handed to both sides of a comparison, so no two
implementations of a generator ever need to agree.
"""
from __future__ import annotations

import numpy as np
import torch

# tensor slots of a seed: seed = 1e6 * config + 1e3 * projection + slot
X, PQS, W, A1, B1, A2, B2 = range(7)

# projections of one DiT block (MiniMax-H3 Ultra Fast, "Why the pruned transformer matters":
# fused QKV, attention output, MLP up/gate and MLP down are the four NVFP4 matrices of a block)
QKV, ATTN_OUT, GATE_UP, DOWN = range(4)


def seed_of(config: int, proj: int, slot: int) -> int:
    return 1_000_000 * config + 1_000 * proj + slot


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    t = torch.randn(shape, generator=_generator(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    t = torch.rand(shape, generator=_generator(seed, device), device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def activation(S: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    return normal((S, K), 1.0, seed, device, torch.bfloat16)


def pre_quant_scale(K: int, seed: int, device="cpu") -> torch.Tensor:
    return uniform((K,), 0.5, 2.0, seed, device)


def weight_fp32(N: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    return normal((N, K), 0.02, seed, device, torch.float32)


def lora_factors(N: int, K: int, rank: int, seed_a: int, seed_b: int, device="cpu"):
    A = normal((rank, K), 0.01, seed_a, device, torch.bfloat16)
    B = normal((N, rank), 0.01, seed_b, device, torch.bfloat16)
    return A, B


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its uint16 bit patterns as a host numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16)


def rope_table(S: int, rot_dim: int, frame_hw=(48, 84), base: float = 10000.0, device="cpu"):
    """Per-token rotary angle table for a packed video sequence (the caller-side input of the Q/K
    RMSNorm + rotary epilogue): token s sits at (t, h, w) of a grid of frames of frame_hw latent
    cells (48 x 84: a 768 x 1344 canvas at 16 pixels per cell), and the rot_dim/2 rotated pairs are
    split evenly over the three axes, pair j of an axis turning at base^(-j/n) per position step
    (n pairs per axis). Returns (cos, sin) fp32 [S][rot_dim/2]."""
    half = rot_dim // 2
    s = torch.arange(S, dtype=torch.float64)
    H, W = frame_hw
    pos = torch.stack([torch.div(s, H * W, rounding_mode="floor"),
                       torch.remainder(torch.div(s, W, rounding_mode="floor"), H),
                       torch.remainder(s, W)], dim=1)                          # [S][3]
    per_axis = [half // 3 + (1 if a < half % 3 else 0) for a in range(3)]
    cols = []
    for a, n in enumerate(per_axis):
        if n == 0:
            continue
        freq = base ** (-torch.arange(n, dtype=torch.float64) / n)
        cols.append(pos[:, a:a + 1] * freq[None, :])
    theta = torch.cat(cols, dim=1) if cols else torch.zeros((S, 0), dtype=torch.float64)
    return theta.cos().float().to(device), theta.sin().float().to(device)
