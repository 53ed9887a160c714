"""Producer fusion across the MLP (FL2VA Turbo, "Implementation": a producer that emits the next
projection's base input beside the exact bf16 LoRA input was bit-exact on the pages' hardware): the
gate/up SwiGLU epilogue also writes the down projection's base operand xs = bf16(h * pqs_down), and
the down projection takes (h, xs) instead of (h, pqs).

Checked: the emitted h is bit-identical to the plain SwiGLU call's; the chain gate/up -> down gives
bit-identical outputs fused and unfused, with and without adapters and with W4A4 on gate/up; the
emitted xs and the prescaled call each match the fp64 oracle; argument errors."""
import numpy as np
import pytest
import torch

import bit_linear_dynamic_amd as h3q
import oracle
from bit_linear_dynamic_amd import synth
from bit_linear_dynamic_amd import workloads as wl
from gpu_helpers import TOL, Proj, bits, normwise, say

pytestmark = pytest.mark.gpu

NONE = h3q.H3Q_ADAPTER_NONE


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def mlp(F, D, seed, rank_gu=16, rank_dn=16):
    gu = Proj(2 * F, D, seed, gate_up=True)
    dn = Proj(D, F, seed + 1)
    gu.add_adapter(1, rank_gu, float(rank_gu), seed + 2, seed + 3)
    dn.add_adapter(1, rank_dn, float(rank_dn), seed + 4, seed + 5)
    return gu, dn


def chain(gu, dn, x, pqs_gu, pqs_dn, aid, st, flags=0):
    h = h3q.h3q_linear_ex(x, pqs_gu, gu.handle, aid, st, flags | h3q.H3Q_EPI_SWIGLU)
    y = h3q.h3q_linear(h, pqs_dn, dn.handle, aid, st)
    h2, xs = h3q.h3q_linear_swiglu_emit(x, pqs_gu, gu.handle, aid, st, pqs_dn, flags=flags)
    y2 = h3q.h3q_linear_prescaled(h2, xs, dn.handle, aid, st)
    torch.cuda.synchronize()
    return h, y, h2, xs, y2


@pytest.mark.parametrize("S,F,D", [(300, 320, 192), (37, 64, 128), (513, 1024, 256)])
def test_mlp_chain_fused_is_bit_identical(S, F, D):
    say(f"fusion chain S={S} F={F} D={D}")
    gu, dn = mlp(F, D, 1600 + S)
    try:
        x = synth.activation(S, D, 1610 + S).cuda()
        pqs_gu = synth.pre_quant_scale(D, 1611).cuda()
        pqs_dn = synth.pre_quant_scale(F, 1612).cuda()
        for aid, st, flags in ((1, 1.0, 0), (NONE, 0.0, 0), (1, 0.5, h3q.H3Q_ACT_NVFP4)):
            h, y, h2, xs, y2 = chain(gu, dn, x, pqs_gu, pqs_dn, aid, st, flags)
            assert torch.equal(h, h2), ("emitted h differs", aid, st, flags)
            assert torch.equal(y, y2), ("fused chain differs", aid, st, flags)
            if flags == 0 and aid == 1:
                # the emitted operand against the oracle: SiLU(gate) * up of the fp64 projection, times pqs_down
                ref_h = oracle.swiglu(gu.reference(bits(x), pqs_gu.cpu().numpy(), 1, st))
                err = normwise(xs, ref_h * pqs_dn.cpu().numpy().astype(np.float64)[None, :])
                say(f"  xs vs oracle: normwise {err:.3e}")
                assert err <= TOL
            say(f"  adapter={aid} strength={st} flags={flags}: h, y bit-identical")
    finally:
        gu.free()
        dn.free()


@pytest.mark.parametrize("S,K,N", [(300, 512, 320), (129, 1024, 200)])
def test_prescaled_parity(S, K, N):
    """The prescaled call fed with the oracle's prescale of x (rounded to bf16) matches the oracle's
    linear, and equals h3q_linear(x, pqs) bit for bit."""
    say(f"prescaled S={S} K={K} N={N}")
    p = Proj(N, K, 1700 + S)
    try:
        p.add_adapter(1, 64, 32.0, 1701, 1702)
        x = synth.activation(S, K, 1703)
        pqs = synth.pre_quant_scale(K, 1704)
        xs = torch.from_numpy(oracle.prescale_f32(bits(x), pqs.numpy())).to(torch.bfloat16)
        for aid, st in ((1, 1.0), (NONE, 0.0)):
            y = h3q.h3q_linear_prescaled(x.cuda(), xs.cuda(), p.handle, aid, st)
            y_ref_path = h3q.h3q_linear(x.cuda(), pqs.cuda(), p.handle, aid, st)
            torch.cuda.synchronize()
            assert torch.equal(y, y_ref_path), (aid, st)
            err = normwise(y, p.reference(bits(x), pqs.numpy(), aid, st))
            say(f"  adapter={aid}: normwise {err:.3e}, bit-identical to h3q_linear")
            assert err <= TOL
    finally:
        p.free()


@pytest.mark.slow
def test_mlp_chain_full_s8192():
    """The block's gate/up (32768 x 6144) -> down (6144 x 16384) at S = 8192, adapters of rank 128."""
    S = wl.S_MID
    say(f"fusion chain full S={S}")
    gu = Proj(wl.GATE_UP.N, wl.GATE_UP.K, synth.seed_of(10, 2, synth.W), gate_up=True)
    dn = Proj(wl.DOWN.N, wl.DOWN.K, synth.seed_of(10, 3, synth.W))
    try:
        gu.add_adapter(1, 128, 128.0, synth.seed_of(10, 2, synth.A1), synth.seed_of(10, 2, synth.B1))
        dn.add_adapter(1, 128, 128.0, synth.seed_of(10, 3, synth.A1), synth.seed_of(10, 3, synth.B1))
        x = synth.activation(S, wl.D_MODEL, synth.seed_of(10, 2, synth.X), "cuda")
        pqs_gu = synth.pre_quant_scale(wl.D_MODEL, synth.seed_of(10, 2, synth.PQS), "cuda")
        pqs_dn = synth.pre_quant_scale(wl.D_FF, synth.seed_of(10, 3, synth.PQS), "cuda")
        h, y, h2, xs, y2 = chain(gu, dn, x, pqs_gu, pqs_dn, 1, 1.0)
        assert torch.equal(h, h2) and torch.equal(y, y2)
        say("  h and y bit-identical fused and unfused")
    finally:
        gu.free()
        dn.free()


def test_emit_past_2gib_of_activation():
    """K = 16384 puts more than 2 GiB of activation in S = 65836 rows (one launch; the GEMM addresses
    each tile from its own first row, so its 32-bit buffer offsets stay small). The emitted operand of
    the rows past the 2 GiB point must land in their own rows: the fused chain stays bit-identical to
    the unfused one on every row."""
    S, K, F, D = 65836, 16384, 256, 128
    say(f"fusion chain past 2 GiB of activation S={S} K={K}")
    gu = Proj(2 * F, K, 1900, gate_up=True)
    dn = Proj(D, F, 1901)
    try:
        gu.add_adapter(1, 16, 16.0, 1902, 1903)
        dn.add_adapter(1, 16, 16.0, 1904, 1905)
        x = synth.activation(S, K, 1906, "cuda")
        pqs_gu = synth.pre_quant_scale(K, 1907, "cuda")
        pqs_dn = synth.pre_quant_scale(F, 1908, "cuda")
        h, y, h2, xs, y2 = chain(gu, dn, x, pqs_gu, pqs_dn, 1, 1.0)
        assert torch.equal(h, h2)
        assert torch.equal(y, y2), "fused chain differs past 2 GiB of activation"
        say("  h and y bit-identical on all rows")
    finally:
        gu.free()
        dn.free()


def test_fusion_argument_errors():
    gu = Proj(2 * 36, 64, 1800, gate_up=True)     # F = 36: not a multiple of 8
    plain = Proj(64, 64, 1801)
    odd_k = Proj(64, 80, 1802)                    # K = 80: not a multiple of 64
    try:
        x = synth.activation(8, 64, 1803).cuda()
        pq = torch.ones(36, device="cuda")

        def expect(code, fn):
            with pytest.raises(h3q.H3QError) as e:
                fn()
            assert e.value.code == code, e.value

        expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_linear_swiglu_emit(x, None, gu.handle, NONE, 0.0, pq))
        expect(h3q.H3Q_E_ARG, lambda: h3q.h3q_linear_swiglu_emit(x, None, plain.handle, NONE, 0.0,
                                                                  torch.ones(32, device="cuda")))
        gu16 = Proj(2 * 32, 64, 1805, gate_up=True)
        try:
            big = torch.zeros(8 * 64 + 64, dtype=torch.bfloat16, device="cuda")
            xo = big[:8 * 64].view(8, 64)
            expect(h3q.H3Q_E_ARG, lambda: h3q.h3q_linear_swiglu_emit(xo, None, gu16.handle, NONE, 0.0,
                                                                      torch.ones(32, device="cuda"),
                                                                      xs_next=big[64:64 + 8 * 32].view(8, 32)))
        finally:
            gu16.free()
        x80 = synth.activation(8, 80, 1804).cuda()
        expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_linear_prescaled(x80, x80.clone(), odd_k.handle, NONE, 0.0))
        buf = torch.zeros(8 * 64 + 8, dtype=torch.bfloat16, device="cuda")
        expect(h3q.H3Q_E_ARG, lambda: h3q.h3q_linear_prescaled(x, buf[1:8 * 64 + 1].view(8, 64), plain.handle, NONE,
                                                                0.0))
    finally:
        gu.free()
        plain.free()
        odd_k.free()
