"""h3q_linear_ex_noalloc: the entry point for callers that cannot allocate (graph capture, tight
serving loops). It runs the kernels of h3q_linear_ex with the workspace in the library's fixed device
scratch, so its outputs must equal h3q_linear_ex's bit for bit; the library's own allocator is made
to fail while it runs, to show that it allocates nothing; two calls in a row (the second smaller)
show that the reused scratch carries nothing over; a call that needs more scratch than there is fails
with H3Q_E_SHAPE and writes nothing."""
import pytest
import torch

import bit_linear_dynamic_amd as h3q
from bit_linear_dynamic_amd import synth
from gpu_helpers import Proj, say

pytestmark = pytest.mark.gpu

NONE = h3q.H3Q_ADAPTER_NONE
SCRATCH = 64 << 20   # H3Q_NOALLOC_SCRATCH_BYTES


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _compare(p, x, pqs, aid, st, flags):
    ref = h3q.h3q_linear_ex(x, pqs, p.handle, aid, st, flags)
    torch.cuda.synchronize()
    return ref


@pytest.mark.parametrize("K,N,rank,gate_up", [(1040, 520, 384, False), (320, 2 * 200, 64, True)])
def test_noalloc_matches_linear_ex(monkeypatch, K, N, rank, gate_up):
    p = Proj(N, K, 2500 + K + N, gate_up=gate_up)
    try:
        p.add_adapter(1, rank, float(rank) / 2, 2501, 2502)
        pqs = synth.pre_quant_scale(K, 2503, "cuda")
        cases = [(1, 1.0, 0), (NONE, 0.0, 0), (1, 0.5, h3q.H3Q_ACT_NVFP4)]
        if gate_up:
            cases += [(1, 1.0, h3q.H3Q_EPI_SWIGLU), (1, 1.0, h3q.H3Q_EPI_SWIGLU | h3q.H3Q_ACT_NVFP4)]
        for S in (3000, 700):  # the second call is the smaller one
            x = synth.activation(S, K, 2504 + S, "cuda")
            for aid, st, flags in cases:
                for use_pqs in (True, False):
                    pq = pqs if use_pqs else None
                    say(f"noalloc K={K} N={N} r={rank} S={S} adapter={aid} flags={flags} pqs={use_pqs}")
                    ref = _compare(p, x, pq, aid, st, flags)
                    n_out = ref.shape[1]
                    out = torch.full((S, n_out), -7.0, dtype=torch.bfloat16, device="cuda")
                    # the library's allocator fails from here on: the call must not need it
                    monkeypatch.setenv("H3Q_TEST_FAIL_ALLOC_AFTER", "0")
                    try:
                        h3q.h3q_linear_ex_noalloc(x, pq, p.handle, aid, st, flags, out=out)
                    finally:
                        monkeypatch.delenv("H3Q_TEST_FAIL_ALLOC_AFTER")
                    torch.cuda.synchronize()
                    assert torch.equal(out, ref)
    finally:
        p.free()


def test_noalloc_rejects_calls_beyond_the_scratch():
    K, N, rank = 6144, 256, 384
    p = Proj(N, K, 2600)
    try:
        p.add_adapter(1, rank, float(rank), 2601, 2602)
        pqs = synth.pre_quant_scale(K, 2603, "cuda")
        per_row = K * 2 + rank * 2
        S_fit = (SCRATCH - 256) // per_row // 8 * 8
        S_big = S_fit + 600
        x = synth.activation(S_big, K, 2604, "cuda")
        out = torch.full((S_big, N), -7.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(h3q.H3QError) as e:
            h3q.h3q_linear_ex_noalloc(x, pqs, p.handle, 1, 1.0, 0, out=out)
        assert e.value.code == h3q.H3Q_E_SHAPE and "scratch" in str(e.value)
        torch.cuda.synchronize()
        assert (out == -7.0).all(), "a refused call wrote its output"
        # at the limit it runs, and without pqs and adapter (x feeds the GEMM directly) any S fits
        xs = x[:S_fit].contiguous()
        y = h3q.h3q_linear_ex_noalloc(xs, pqs, p.handle, 1, 1.0, 0)
        assert torch.equal(y, h3q.h3q_linear_ex(xs, pqs, p.handle, 1, 1.0, 0))
        y0 = h3q.h3q_linear_ex_noalloc(x, None, p.handle, NONE, 0.0, 0)
        assert torch.equal(y0, h3q.h3q_linear_ex(x, None, p.handle, NONE, 0.0, 0))
        torch.cuda.synchronize()
    finally:
        p.free()
