"""The fused QKV projection with per-head Q/K RMSNorm and partial split-half rotary embedding
(MiniMax-H3 Ultra Fast, "Active optimization stack" and "Kernel path"; 96 of 128 head dimensions
rotate: MiniMax-H3 Turbo CMF card, "On parity") against the fp64 oracle: small and ragged shapes,
the W4A4 activation path, the full QKV shape, and argument errors. The v columns must equal the plain
projection's output bit for bit (same GEMM, plain store)."""
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
EPS = 1e-6


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def gammas(q_width, seed):
    g = synth.uniform((2, q_width), 0.5, 1.5, seed)
    return g[0].contiguous(), g[1].contiguous()


def off_by_one_float(t):
    """A device copy of t whose data starts 4 bytes past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    v = buf[1:].view(t.shape)
    v.copy_(t.to("cuda"))
    assert v.data_ptr() % 16 == 4
    return v


def run_case(p: Proj, x, pqs, q_width, rot, adapter_id, strength, flags=0, rows=None, misaligned_tables=False,
             sections=None):
    S = x.shape[0]
    gq, gk = gammas(q_width, 900 + q_width + rot)
    cos, sin = synth.rope_table(S, rot)
    dev = "cuda"
    cos_d, sin_d = (cos.to(dev), sin.to(dev)) if rot else (None, None)
    if rot and misaligned_tables:
        cos_d, sin_d = off_by_one_float(cos), off_by_one_float(sin)
    y = h3q.h3q_linear_qk_norm_rope(x.to(dev), pqs.to(dev) if pqs is not None else None, p.handle, adapter_id,
                                    strength, q_width, rot, EPS, gq.to(dev), gk.to(dev), cos_d, sin_d, flags=flags,
                                    sections=sections)
    plain = h3q.h3q_linear_ex(x.to(dev), pqs.to(dev) if pqs is not None else None, p.handle, adapter_id, strength,
                              flags)
    torch.cuda.synchronize()
    assert torch.equal(y[:, 2 * q_width:], plain[:, 2 * q_width:]), "v columns differ from the plain projection"
    sel = np.arange(S) if rows is None else rows
    xb = bits(x[torch.from_numpy(sel)])
    pq = pqs.numpy() if pqs is not None else None
    lin = p.reference(xb, pq, adapter_id, strength, w4a4=bool(flags & h3q.H3Q_ACT_NVFP4)) if rows is None else None
    if rows is not None:  # W4A4 is not run on row samples (its activation scale spans all rows)
        lin = p.reference(xb, pq, adapter_id, strength)
    ref = oracle.qk_norm_rope(lin, q_width, rot, EPS, gq.numpy(), gk.numpy(), cos.numpy()[sel], sin.numpy()[sel],
                              sections=sections)
    ys = y.index_select(0, torch.from_numpy(sel).cuda())
    eq = normwise(ys[:, :q_width], ref[:, :q_width])
    ek = normwise(ys[:, q_width:2 * q_width], ref[:, q_width:2 * q_width])
    ev = normwise(ys[:, 2 * q_width:], ref[:, 2 * q_width:])
    say(f"  q {eq:.3e}  k {ek:.3e}  v {ev:.3e}")
    assert max(eq, ek, ev) <= TOL
    return y


CASES = [
    # S, K, q_width, v width (0: q_width), rot_dim, rank
    (300, 512, 256, 0, 96, 64),
    (37, 208, 256, 104, 96, 16),
    (129, 256, 512, 0, 128, 64),
    (64, 320, 256, 0, 0, 64),
    (513, 1024, 768, 0, 96, 384),
    (200, 256, 256, 0, 100, 64),   # rot/2 = 50, not a multiple of 8: the one-pair-at-a-time path
    (90, 256, 256, 0, 16, 64),     # rot/2 = 8: one group of 8 pairs, 112 pass-through dims
]


@pytest.mark.parametrize("S,K,q_width,extra,rot,rank", CASES)
def test_qk_norm_rope_parity(S, K, q_width, extra, rot, rank):
    N = 2 * q_width + (extra or q_width)  # a narrower v ends in a ragged column tile
    say(f"qk S={S} K={K} q_width={q_width} N={N} rot={rot} r={rank}")
    p = Proj(N, K, 1100 + S + K)
    try:
        p.add_adapter(1, rank, float(rank) / 2, 1101, 1102)
        x = synth.activation(S, K, 1103)
        pqs = synth.pre_quant_scale(K, 1104)
        for aid, st in ((NONE, 0.0), (1, 1.0)):
            run_case(p, x, pqs, q_width, rot, aid, st)
    finally:
        p.free()


SECTION_CASES = [
    # S, K, q_width, rank, sections: three axes of 32 dims each (the per-axis reading of the
    # three-axis split-half rotary), unequal axes, halves that are not multiples of 8 (one pair at a
    # time), two sections over all 128 dims
    (300, 512, 256, 64, (32, 32, 32)),
    (77, 208, 512, 16, (16, 48, 32)),
    (129, 256, 256, 64, (24, 40, 32)),
    (64, 320, 256, 384, (64, 64)),
]


@pytest.mark.parametrize("S,K,q_width,rank,sections", SECTION_CASES)
def test_qk_norm_rope_sections_parity(S, K, q_width, rank, sections):
    """Rotation within axis sections (h3q_linear_qk_norm_rope_sections) against the oracle."""
    rot = sum(sections)
    say(f"qk sections {sections} S={S} K={K} q_width={q_width} r={rank}")
    p = Proj(3 * q_width, K, 1400 + S + K)
    try:
        p.add_adapter(1, rank, float(rank), 1401, 1402)
        x, pqs = synth.activation(S, K, 1403), synth.pre_quant_scale(K, 1404)
        for aid, st in ((NONE, 0.0), (1, 1.0)):
            run_case(p, x, pqs, q_width, rot, aid, st, sections=sections)
        run_case(p, x, pqs, q_width, rot, 1, 1.0, flags=h3q.H3Q_ACT_NVFP4, sections=sections)
        run_case(p, x, pqs, q_width, rot, 1, 1.0, misaligned_tables=True, sections=sections)
    finally:
        p.free()


def test_qk_norm_rope_one_section_is_the_plain_call():
    """One section of rot_dim is the reading of h3q_linear_qk_norm_rope, bit for bit; three sections
    of 32 give a different result (the two readings differ)."""
    S, K, q_width = 200, 256, 256
    p = Proj(3 * q_width, K, 1500)
    try:
        p.add_adapter(1, 64, 64.0, 1501, 1502)
        x, pqs = synth.activation(S, K, 1503).cuda(), synth.pre_quant_scale(K, 1504).cuda()
        gq, gk = (g.cuda() for g in gammas(q_width, 1505))
        cos, sin = (t.cuda() for t in synth.rope_table(S, 96))
        args = (x, pqs, p.handle, 1, 1.0, q_width, 96, EPS, gq, gk, cos, sin)
        plain = h3q.h3q_linear_qk_norm_rope(*args)
        one = h3q.h3q_linear_qk_norm_rope(*args, sections=(96,))
        three = h3q.h3q_linear_qk_norm_rope(*args, sections=(32, 32, 32))
        torch.cuda.synchronize()
        assert torch.equal(plain, one)
        assert not torch.equal(plain[:, :2 * q_width], three[:, :2 * q_width])
        assert torch.equal(plain[:, 2 * q_width:], three[:, 2 * q_width:])
    finally:
        p.free()


def test_qk_norm_rope_misaligned_tables():
    """Angle tables that start 4 bytes past a 16-byte boundary take scalar table loads."""
    S, K, q_width = 150, 256, 256
    say("qk misaligned angle tables")
    p = Proj(3 * q_width, K, 1300)
    try:
        p.add_adapter(1, 64, 64.0, 1301, 1302)
        run_case(p, synth.activation(S, K, 1303), synth.pre_quant_scale(K, 1304), q_width, 96, 1, 1.0,
                 misaligned_tables=True)
    finally:
        p.free()


def test_qk_norm_rope_w4a4():
    S, K, q_width = 200, 512, 256
    say("qk W4A4")
    p = Proj(3 * q_width, K, 1200)
    try:
        p.add_adapter(1, 64, 64.0, 1201, 1202)
        run_case(p, synth.activation(S, K, 1203), synth.pre_quant_scale(K, 1204), q_width, 96, 1, 1.0,
                 flags=h3q.H3Q_ACT_NVFP4)
    finally:
        p.free()


@pytest.mark.slow
def test_qk_norm_rope_full_qkv_s8192():
    """The block's fused QKV projection (18432 x 6144, 48 heads each of q, k, v, rank 384) at S = 8192
    on sampled rows (first 256, last 256, every 128th)."""
    S, P = wl.S_MID, wl.QKV
    say(f"qk full QKV S={S}")
    p = Proj(P.N, P.K, synth.seed_of(2, 0, synth.W))
    try:
        p.add_adapter(1, P.rank, P.alpha, synth.seed_of(2, 0, synth.A1), synth.seed_of(2, 0, synth.B1))
        x = synth.activation(S, P.K, synth.seed_of(7, 0, synth.X))
        pqs = synth.pre_quant_scale(P.K, synth.seed_of(7, 0, synth.PQS))
        rows = np.unique(np.concatenate([np.arange(256), np.arange(256, S - 256, 128), np.arange(S - 256, S)]))
        run_case(p, x, pqs, wl.D_MODEL, 96, 1, 1.0, rows=rows)
        say("  per-axis sections (32, 32, 32)")
        run_case(p, x, pqs, wl.D_MODEL, 96, 1, 1.0, rows=rows, sections=(32, 32, 32))
    finally:
        p.free()


def test_qk_norm_rope_argument_errors():
    K, q_width = 64, 256
    p = Proj(3 * q_width, K, 1300)
    gu = Proj(2 * 256, K, 1301, gate_up=True)
    try:
        x = synth.activation(4, K, 1302).cuda()
        g = torch.ones(q_width, device="cuda")
        cos, sin = (t.cuda() for t in synth.rope_table(4, 96))
        ok = dict(q_width=q_width, rot_dim=96, eps=EPS, gamma_q=g, gamma_k=g, rope_cos=cos, rope_sin=sin)

        def expect(code, handle=p.handle, **kw):
            args = dict(ok, **kw)
            flags = args.pop("flags", 0)
            with pytest.raises(h3q.H3QError) as e:
                h3q.h3q_linear_qk_norm_rope(x, None, handle, NONE, 0.0, flags=flags, **args)
            assert e.value.code == code, (kw, e.value)

        expect(h3q.H3Q_E_SHAPE, q_width=128, gamma_q=g[:128].contiguous(), gamma_k=g[:128].contiguous())
        expect(h3q.H3Q_E_SHAPE, q_width=512, gamma_q=torch.ones(512, device="cuda"),
               gamma_k=torch.ones(512, device="cuda"))
        expect(h3q.H3Q_E_SHAPE, rot_dim=97, rope_cos=cos[:, :48].contiguous(), rope_sin=sin[:, :48].contiguous())
        expect(h3q.H3Q_E_ARG, eps=0.0)
        expect(h3q.H3Q_E_ARG, eps=float("nan"))
        expect(h3q.H3Q_E_ARG, flags=h3q.H3Q_EPI_SWIGLU)
        expect(h3q.H3Q_E_ARG, handle=gu.handle, q_width=256)
        expect(h3q.H3Q_E_ARG, flags=1 << 7)
        for bad in ((32, 32), (32, 33, 31), (0, 64, 32), (16, 16, 16, 16, 32), (-32, 64, 64)):
            expect(h3q.H3Q_E_SHAPE, sections=bad)
    finally:
        p.free()
        gu.free()
