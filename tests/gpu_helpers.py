"""Shared fixtures for the GPU tests: packed projections whose inputs come from the seeded generators
and the oracle's NVFP4 weight quantizer, and comparisons of the HIP path with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bit_linear_dynamic_amd as h3q
import oracle
from bit_linear_dynamic_amd import synth

# Normwise relative error bar for floating-point outputs (||y - y_ref||_F / ||y_ref||_F).
TOL = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits(t)


def normwise(y_gpu: torch.Tensor, y_ref: np.ndarray) -> float:
    g = y_gpu.detach().float().cpu().double().numpy()
    den = np.linalg.norm(y_ref)
    return float(np.linalg.norm(g - y_ref) / (den if den > 0 else 1.0))


class Proj:
    """A packed NVFP4 projection with host copies of everything the oracle needs."""

    def __init__(self, N, K, seed, gate_up=False, codes=None, scales=None, ts=None):
        self.N, self.K, self.gate_up = N, K, gate_up
        if codes is None:
            w = synth.weight_fp32(N, K, seed)
            codes, scales, ts = oracle.nvfp4_weight_fixture(w.numpy())
        self.codes, self.scales, self.ts = codes, scales, ts
        self.handle = h3q.h3q_pack_weight(codes, scales, ts, N, K, h3q.H3Q_PACK_GATE_UP if gate_up else 0)
        self.adapters = {}

    def add_adapter(self, adapter_id, rank, alpha, seed_a, seed_b, A=None, B=None):
        if A is None:
            A, B = synth.lora_factors(self.N, self.K, rank, seed_a, seed_b)
        h3q.h3q_register_adapter(self.handle, adapter_id, A, B, rank, alpha)
        self.adapters[adapter_id] = (bits(A) if isinstance(A, torch.Tensor) else A,
                                     bits(B) if isinstance(B, torch.Tensor) else B, rank, alpha)

    def reference(self, x_bits, pqs, adapter_id=h3q.H3Q_ADAPTER_NONE, strength=0.0, w4a4=False):
        """fp64 oracle output for the given rows of x (bf16 bits)."""
        kw = {}
        if adapter_id != h3q.H3Q_ADAPTER_NONE and strength != 0.0:
            A, B, r, alpha = self.adapters[adapter_id]
            kw = dict(A_bits=A, B_bits=B, rank=r, alpha=alpha, strength=strength)
        if w4a4:
            ac, asc, ts_a = oracle.w4a4_activation(x_bits, pqs)
            kw.update(act_codes=ac, act_scales=asc, ts_a=ts_a)
        return oracle.linear(x_bits, pqs, self.codes, self.scales, self.ts, **kw)

    def run(self, x, pqs, adapter_id=h3q.H3Q_ADAPTER_NONE, strength=0.0, flags=0):
        y = h3q.h3q_linear_ex(x, pqs, self.handle, adapter_id, strength, flags)
        torch.cuda.synchronize()
        return y

    def free(self):
        if self.handle:
            h3q.h3q_free_weight(self.handle)
            self.handle = None
