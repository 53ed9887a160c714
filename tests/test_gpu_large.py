"""Buffers larger than 4 GiB in one call: the activation operand (S x K_pad bf16) and the adapter's
t' (S x r_pad bf16). A 32-bit byte offset cannot reach past 4 GiB, so the kernels address these
buffers from each tile's first row; rows beyond the 4 GiB mark must come out like every other row.
The oracle checks the first rows, the rows on both sides of the mark and the last rows (the ragged
last tile), the rows past the mark on their own as well.
(FL2VA Turbo, "Implementation": the LoRA branch on the original x, folded into the base product.)"""
import numpy as np
import pytest
import torch

import bit_linear_dynamic_amd as h3q
from bit_linear_dynamic_amd import synth
from gpu_helpers import TOL, Proj, bits, normwise, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample(S: int, mark: int) -> np.ndarray:
    return np.unique(np.concatenate([np.arange(64), np.arange(mark - 96, mark + 96), np.arange(S - 300, S)]))


def check(pr: Proj, y, x, pqs, rows: np.ndarray, mark: int, what: str):
    idx = torch.from_numpy(rows).to(x.device)
    ref = pr.reference(bits(x.index_select(0, idx)), None if pqs is None else pqs.cpu().numpy(), 1, 1.0)
    got = y.index_select(0, idx)
    err = normwise(got, ref)
    past = rows >= mark
    err_past = normwise(got[torch.from_numpy(past).to(got.device)], ref[past])
    say(f"  {what}: {len(rows)} rows, normwise {err:.3e}; {int(past.sum())} rows past 4 GiB {err_past:.3e}")
    assert err <= TOL and err_past <= TOL, (what, err, err_past)


@pytest.fixture
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("use_pqs", [True, False])
def test_activation_operand_past_4gib(gpu, use_pqs):
    """S = 140000, K = 16384: the operand is 4.59 GB (x * pqs in the workspace, or x itself)."""
    N, K, r, S = 256, 16384, 128, 140000
    mark = (1 << 32) // (K * 2)  # first row whose operand bytes start at or past 2^32
    say(f"large activation S={S} K={K} N={N} r={r} pqs={use_pqs}")
    pr = Proj(N, K, synth.seed_of(21, 0, synth.W))
    try:
        pr.add_adapter(1, r, float(r), synth.seed_of(21, 0, synth.A1), synth.seed_of(21, 0, synth.B1))
        x = synth.activation(S, K, synth.seed_of(21, 0, synth.X), "cuda")
        pqs = synth.pre_quant_scale(K, synth.seed_of(21, 0, synth.PQS), "cuda") if use_pqs else None
        y = pr.run(x, pqs, 1, 1.0)
        check(pr, y, x, pqs, sample(S, mark), mark, "adapter 1, strength 1")
        del x, y
    finally:
        pr.free()


def test_lora_t_past_4gib(gpu):
    """S = 4.2 M, r = 512: t' is 4.3 GB (K = 64 keeps x and the GEMM small)."""
    N, K, r, S = 256, 64, 512, 4_200_000
    mark = (1 << 32) // (r * 2)
    say(f"large t' S={S} K={K} N={N} r={r}")
    pr = Proj(N, K, synth.seed_of(21, 1, synth.W))
    try:
        pr.add_adapter(1, r, float(r), synth.seed_of(21, 1, synth.A1), synth.seed_of(21, 1, synth.B1))
        x = synth.activation(S, K, synth.seed_of(21, 1, synth.X), "cuda")
        pqs = synth.pre_quant_scale(K, synth.seed_of(21, 1, synth.PQS), "cuda")
        y = pr.run(x, pqs, 1, 1.0)
        check(pr, y, x, pqs, sample(S, mark), mark, "adapter 1, strength 1")
        del x, y
    finally:
        pr.free()
