"""Shapes of the projections and of the synthetic workloads the library is measured and checked on.

One DiT block of MiniMax-H3 has four NVFP4 matrices (MiniMax-H3 Ultra Fast, "Why the pruned
transformer matters"): fused QKV, attention output, fused MLP gate/up and MLP down. The adapters use
rank = alpha = 384 on fused QKV and 128 on the others (FL2VA Turbo, "Implementation"). The model
width d = 6144 and MLP width 16384 are not printed on the pages; they are the reading under which
one block at S = 37726 costs the ~70 TFLOP of GEMM plus attention that the MiniMax-H3 AoTI packages
card states (paragraph after its timing table) -- tests/test_pages_facts.py checks that arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

D_MODEL = 6144
D_FF = 16384


@dataclass(frozen=True)
class Projection:
    name: str
    N: int          # output features (rows of W)
    K: int          # input features
    rank: int
    alpha: float
    gate_up: bool = False   # rows [0, N/2) gate, [N/2, N) up


QKV = Projection("qkv", 3 * D_MODEL, D_MODEL, 384, 384.0)
ATTN_OUT = Projection("attn_out", D_MODEL, D_MODEL, 128, 128.0)
GATE_UP = Projection("gate_up", 2 * D_FF, D_MODEL, 128, 128.0, gate_up=True)
DOWN = Projection("down", D_MODEL, D_FF, 128, 128.0)
BLOCK = (QKV, ATTN_OUT, GATE_UP, DOWN)

# the small single fused-QKV-like projection used for exhaustive checks
SMALL_QKV = Projection("qkv_small", 3072, 1024, 384, 384.0)

# packed sequence lengths of the released 768x1344x124-frame canvas for a 16- and an 18-token
# prompt (MiniMax-H3 AoTI packages, "What is here")
S_CANVAS = 37726
S_CANVAS_ALT = 37728
S_MID = 8192
S_SWITCH = 16384
S_SMALL = 256


def effective_flops(S: int, p: Projection, with_adapter: bool = True) -> int:
    """Algorithmic FLOPs of one call: the dense base contraction plus, with an adapter, A x and B t.
    Decoding, quantization and padding are not counted."""
    f = 2 * S * p.N * p.K
    if with_adapter:
        f += 2 * S * p.rank * (p.K + p.N)
    return f


@dataclass(frozen=True)
class AdalnCurve:
    """The AdaLN modulation curve of the pruned model with the adapter folded in (MiniMax-H3 Turbo CMF
    card, "What the conversion did": [1025, 8] time table shared by the blocks, [96768, 8] per-block
    weights, lora_A [16, 2688], a [1025, 24] table per block; 50 denoiser blocks: FL2VA Turbo,
    "Implementation")."""
    blocks: int = 50
    samples: int = 1025
    emb_dim: int = 2688
    base_rank: int = 8
    lora_rank: int = 16
    rows: int = 96768


ADALN = AdalnCurve()
ADALN_SMALL = AdalnCurve(blocks=3, samples=33, emb_dim=200, base_rank=8, lora_rank=16, rows=1000)
