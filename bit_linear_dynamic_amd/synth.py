"""Seeded synthetic inputs for the W4 + dynamic LoRA linear.

Shared by the tests, the smoke check and the benchmark; it holds none of the method's arithmetic
(no quantization, no decoding, no contraction) -- only seeded draws of the value distributions the
workloads name:
    x   ~ N(0, 1)      as bf16   (activation)
    pqs ~ U[0.5, 2]    as fp32   (per-input-channel pre_quant_scale)
    W   ~ N(0, 0.02)   as fp32   (weight before NVFP4 quantization)
    A,B ~ N(0, 0.01)   as bf16   (LoRA factors)
and, for the AdaLN modulation curve, smooth time coordinates and sinusoidal timestep features
(adaln_curve_inputs), where N(0, s) names the standard deviation s. Draws use torch's seeded generators on the device
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


def adaln_curve_inputs(blocks: int, samples: int, emb_dim: int, base_rank: int, lora_rank: int, rows: int,
                       seed: int, device="cpu"):
    """Synthetic inputs of the AdaLN modulation curve, at the sample points t_i = i / (samples - 1):
      u    fp32 [samples][base_rank]: the time coordinate, u_q(t) = a_q cos((q + 1) pi t + phi_q) with
           amplitudes a_q = 0.3^q * N(1, 0.1) (a smooth curve whose components decay like the
           singular values the pages list);
      emb  fp32 [samples][emb_dim]: sinusoidal features of 1000 t (half cosines, half sines, periods
           spread geometrically up to 10000), a stand-in for the model's timestep embedding;
      A    bf16 [blocks][lora_rank][emb_dim] ~ N(0, 0.01);
      M    bf16 [blocks][rows][base_rank + lora_rank] = [W_p ~ N(0, 0.1) | B ~ N(0, 0.01)];
      bias fp32 [blocks][rows] ~ N(0, 0.1)."""
    t = torch.linspace(0.0, 1.0, samples, dtype=torch.float64)
    amp = (0.3 ** torch.arange(base_rank, dtype=torch.float64)) * (1.0 + 0.1 * normal((base_rank,), 1.0, seed).double())
    phase = uniform((base_rank,), 0.0, 6.283185307179586, seed + 1).double()
    q = torch.arange(base_rank, dtype=torch.float64)
    u = amp[None, :] * torch.cos((q[None, :] + 1.0) * torch.pi * t[:, None] + phase[None, :])
    half = emb_dim // 2
    freq = 10000.0 ** (-torch.arange(half, dtype=torch.float64) / max(half, 1))
    arg = 1000.0 * t[:, None] * freq[None, :]
    emb = torch.cat([torch.cos(arg), torch.sin(arg)], dim=1)
    if emb.shape[1] < emb_dim:
        emb = torch.cat([emb, torch.zeros((samples, emb_dim - emb.shape[1]), dtype=torch.float64)], dim=1)
    A = normal((blocks, lora_rank, emb_dim), 0.01, seed + 2, device, torch.bfloat16)
    Wp = normal((blocks, rows, base_rank), 0.1, seed + 3, device, torch.bfloat16)
    B = normal((blocks, rows, lora_rank), 0.01, seed + 4, device, torch.bfloat16)
    bias = normal((blocks, rows), 0.1, seed + 5, device)
    return (u.float().to(device), emb.float().to(device), A, torch.cat([Wp, B], dim=2).contiguous(), bias)
