"""Edge cases of the HIP path that the N(0, 1) workloads never reach.

* The W4A4 activation quantizer (MiniMax-H3 Ultra Fast, "Kernel path", item 1: activations quantized
  to NVFP4 on every call) on inputs built to take its rarer branches: block scales that are E4M3
  subnormals (and block maxima exactly on the midpoints between them), block scales that round to
  zero, all-zero 16-blocks beside non-zero ones, and an all-zero tensor (tensor scale 1, every code
  and scale 0). Codes, scales and the tensor scale must equal the oracle's bit for bit, both from the
  debug entry point and inside the linear: with an identity weight each output is one decoded
  activation value times the two tensor scales, so the linear's result is known exactly.
* The LoRA-down's K padding: with the library workspace filled with NaN bytes before every call (a
  test hook), outputs must still match the oracle when K is not a multiple of 64 -- nothing may read
  workspace columns that the call did not write -- and a row must not read past its own end into the
  next row (a neighbour holding inf must not turn it into NaN).
* Output sentinels: nothing is written before the first element, after the last row, or past the
  last column of a ragged last column tile.
"""
import numpy as np
import pytest
import torch

import bit_linear_dynamic_amd as h3q
import oracle
import pins
from bit_linear_dynamic_amd import synth
from gpu_helpers import TOL, Proj, bits, normwise, say

pytestmark = pytest.mark.gpu

NONE = h3q.H3Q_ADAPTER_NONE


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def dev(t):
    return t.to("cuda")


# --------------------------------------------------------------------------------------------
# inputs that reach the quantizer's rarer branches
# --------------------------------------------------------------------------------------------

def _bf16(v: np.ndarray) -> np.ndarray:
    """fp64 values rounded to bf16 (RNE), as bf16 bit patterns."""
    return synth.bf16_bits(torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(torch.bfloat16))


def x_spread(S=48, K=512, seed=71):
    """Each 16-block scaled by 2^u, u uniform in [-24, 6]: block maxima from ~1e-7 to ~200, so that
    amax_b / (6 ts) falls below 2^-6 (subnormal E4M3 scale) and below 2^-10 (scale 0) in many blocks."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((S, K)) * np.repeat(2.0 ** rng.uniform(-24, 6, (S, K // 16)), 16, axis=1)
    return _bf16(v)


def x_subnormal_midpoints(S=36, K=256, seed=72):
    """The tensor scale is exactly 2^-4 (one element equals 2688 * 2^-4 = 168 and every other is
    smaller), and block b of row s has the maximum 6 * 2^-4 * j * 2^-10 with j = (s * 16 + b) % 20: the
    quotient amax_b / (6 ts) is then j * 2^-10, i.e. 0, every E4M3 subnormal (even j), every midpoint
    between two of them (odd j: ties to the even code) and the first normal values. The other 15
    values of a block are uniform in [-amax_b, amax_b], rounded to bf16 towards zero."""
    rng = np.random.default_rng(seed)
    v = np.zeros((S, K))
    for s in range(S):
        for b in range(K // 16):
            j = (s * (K // 16) + b) % 20
            amax_b = 6.0 * 2.0 ** -4 * j * 2.0 ** -10
            blk = rng.uniform(-1, 1, 16) * amax_b
            blk[rng.integers(16)] = amax_b * (1 if rng.integers(2) else -1)
            v[s, 16 * b:16 * b + 16] = blk
    v[0, 0] = 168.0
    t = torch.from_numpy(v).to(torch.float32)
    # round towards zero to bf16, so that no value rounds above its block maximum
    b = (t.view(torch.int32) & ~0xFFFF).view(torch.float32).to(torch.bfloat16)
    out = synth.bf16_bits(b)
    assert np.max(np.abs(pins.bf16_values(out))) == 168.0
    return out


def x_zero_blocks(S=70, K=320, seed=73):
    """N(0, 1) activations with about 40 % of the 16-blocks all zero (and a few -0.0 entries)."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((S, K))
    zero = rng.random((S, K // 16)) < 0.4
    v[np.repeat(zero, 16, axis=1)] = 0.0
    out = _bf16(v)
    neg0 = np.repeat(zero, 16, axis=1) & (rng.random((S, K)) < 0.1)
    out[neg0] = 0x8000
    return out


def x_all_zero(S=33, K=64):
    return np.zeros((S, K), np.uint16)


QUANT_CASES = {
    "spread": (x_spread, False),
    "spread_pqs": (x_spread, True),
    "subnormal_midpoints": (x_subnormal_midpoints, False),
    "zero_blocks_pqs": (x_zero_blocks, True),
    "all_zero": (x_all_zero, False),
    "all_zero_pqs": (x_all_zero, True),
}


def _case(name):
    make, use_pqs = QUANT_CASES[name]
    xb = make()
    K = xb.shape[1]
    pqs = synth.pre_quant_scale(K, 74 + K).numpy() if use_pqs else None
    return xb, pqs


def _branches(oc, osc, ots, xb, pqs):
    """Which of the quantizer's branches the oracle took on this input."""
    v = oracle.prescale_f32(xb, pqs)
    blk_zero = np.all(v.reshape(v.shape[0], -1, 16) == 0, axis=2)
    return {"subnormal_scale": int(np.sum((osc > 0) & (osc < 8))),
            "zero_scale_nonzero_block": int(np.sum((osc == 0) & ~blk_zero)),
            "zero_block": int(np.sum(blk_zero)),
            "ts_one": ots == 1.0 and not np.any(v)}


@pytest.mark.parametrize("name", list(QUANT_CASES))
def test_quantizer_edge_branches_bit_exact(name):
    xb, pqs = _case(name)
    S, K = xb.shape
    say(f"act-quant edges {name} S={S} K={K}")
    x = dev(synth.from_bf16_bits(xb))
    pq = dev(torch.from_numpy(pqs)) if pqs is not None else None
    codes, scales, ts = h3q.h3q_debug_quantize_act(x, pq)
    torch.cuda.synchronize()
    oc, osc, ots = oracle.w4a4_activation(xb, pqs)
    br = _branches(oc, osc, ots, xb, pqs)
    say(f"  oracle branches: {br}")
    if name.startswith("spread"):
        assert br["subnormal_scale"] > 0 and br["zero_scale_nonzero_block"] > 0
    if name == "subnormal_midpoints":
        assert ots == 2.0 ** -4 and br["subnormal_scale"] > 0 and br["zero_block"] > 0
    if name.startswith("zero_blocks"):
        assert br["zero_block"] > 0
    if name.startswith("all_zero"):
        assert br["ts_one"] and not np.any(oc) and not np.any(osc)
    assert ts.item() == ots
    assert np.array_equal(scales.cpu().numpy(), osc)
    assert np.array_equal(codes.cpu().numpy(), oc)
    # the earlier name of the same entry point gives the same bits
    c2, s2, t2 = h3q.h3q_quantize_nvfp4(x, pq)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scales) and torch.equal(t2, ts)


def _identity_weight(K):
    """NVFP4 identity [K][K]: E2M1 1.0 (code 2) on the diagonal, block scales 1.0 (0x38), ts = 1."""
    nib = np.zeros((K, K), np.uint8)
    nib[np.arange(K), np.arange(K)] = 2
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((K, K // 16), 0x38, np.uint8)
    return codes, scales


@pytest.mark.parametrize("name", list(QUANT_CASES))
def test_w4a4_linear_edge_branches_bit_exact(name):
    """Through h3q_linear_ex(H3Q_ACT_NVFP4) with an identity weight, y[s][n] is one product:
    bf16(f32(f32(ts_w * ts_a) * Xd[s][n])) with Xd = E2M1 * E4M3 of the quantized activation, so the
    quantizer inside the linear is checked bit for bit, subnormal and zero scales included. An adapter
    on the same handle gives the oracle's normwise parity (the LoRA branch sees the original x)."""
    xb, pqs = _case(name)
    S, K = xb.shape
    say(f"w4a4 linear edges {name} S={S} K={K}")
    codes, scales = _identity_weight(K)
    p = Proj(K, K, 0, codes=codes, scales=scales, ts=1.0)
    try:
        x = dev(synth.from_bf16_bits(xb))
        pq = dev(torch.from_numpy(pqs)) if pqs is not None else None
        y = p.run(x, pq, flags=h3q.H3Q_ACT_NVFP4)
        oc, osc, ots = oracle.w4a4_activation(xb, pqs)
        xd = oracle.dequant(oc, osc, 1.0)                       # exact, at most 6 significant bits
        scale = np.float32(np.float32(1.0) * np.float32(ots))
        want = _bf16((xd.astype(np.float32) * scale).astype(np.float64))
        assert np.array_equal(bits(y), want)
        p.add_adapter(1, 24, 12.0, 75, 76)
        y1 = p.run(x, pq, 1, 0.75, flags=h3q.H3Q_ACT_NVFP4)
        ref = p.reference(xb, pqs, 1, 0.75, w4a4=True)
        if not np.any(ref):
            assert not np.any(bits(y1) & 0x7FFF), "an all-zero input must give zeros"
        else:
            err = normwise(y1, ref)
            say(f"  with adapter: normwise={err:.3e}")
            assert err <= TOL
    finally:
        p.free()


# --------------------------------------------------------------------------------------------
# LoRA-down padding: a poisoned workspace and non-finite neighbours
# --------------------------------------------------------------------------------------------

POISON_CASES = [
    # S, K, N, rank: K % 64 = 16 or 32 with 32-deep LoRA-down tiles (rank > 256, or 129..256 at large S)
    (300, 1040, 256, 384),
    (40000, 1056, 256, 256),
    (100, 1104, 300, 300),
    (64, 80, 96, 16),      # 64-deep tiles with K % 64 = 16
]


@pytest.mark.parametrize("S,K,N,rank", POISON_CASES)
def test_poisoned_workspace_k_padding(monkeypatch, S, K, N, rank):
    """Every call first fills its workspace with 0xFF bytes (bf16 NaN). The GEMM reads xs out to K
    rounded up to 64 and t' out to the padded rank: the LoRA-down must have written all of it."""
    say(f"poisoned workspace S={S} K={K} N={N} r={rank}")
    monkeypatch.setenv("H3Q_TEST_POISON_WORKSPACE", "1")
    p = Proj(N, K, 1700 + K)
    try:
        p.add_adapter(1, rank, float(rank) / 2, 1701, 1702)
        x = synth.activation(S, K, 1703)
        pqs = synth.pre_quant_scale(K, 1704)
        rows = np.unique(np.concatenate([np.arange(min(S, 160)), np.arange(max(0, S - 160), S),
                                         np.arange(0, S, max(1, S // 300))]))
        idx = torch.from_numpy(rows)
        for aid, st, flags in ((1, 1.0, 0), (NONE, 0.0, 0), (1, 0.5, h3q.H3Q_ACT_NVFP4)):
            y = p.run(dev(x), dev(pqs), aid, st, flags=flags)
            assert torch.isfinite(y).all(), (aid, flags)
            xs_rows = x if len(rows) == S else x.index_select(0, idx)
            if flags:
                # the W4A4 tensor scale is global: quantize the whole activation, then sample rows
                oc, osc, ots = oracle.w4a4_activation(bits(x), pqs.numpy())
                A, B, r, al = p.adapters[1]
                ref = oracle.linear(bits(xs_rows), pqs.numpy(), p.codes, p.scales, p.ts, A, B, r, al, st,
                                    act_codes=oc[rows], act_scales=osc[rows], ts_a=ots)
            else:
                ref = p.reference(bits(xs_rows), pqs.numpy(), aid, st)
            err = normwise(y.index_select(0, idx.cuda()), ref)
            say(f"  adapter={aid} flags={flags}: normwise={err:.3e}")
            assert err <= TOL
    finally:
        p.free()


@pytest.mark.parametrize("K,rank", [(1040, 384), (1040, 64), (208, 32)])
def test_rows_do_not_read_past_their_end(K, rank):
    """Odd rows hold +inf in their first 48 columns; the even rows' outputs must stay finite and match
    the oracle (the last K-tile of a row covers columns past K, which in memory are the next row's)."""
    S, N = 130, 256
    say(f"row tails K={K} r={rank}")
    p = Proj(N, K, 1800 + K + rank)
    try:
        p.add_adapter(1, rank, float(rank), 1801, 1802)
        x = synth.activation(S, K, 1803)
        x[1::2, :48] = float("inf")
        pqs = synth.pre_quant_scale(K, 1804)
        even = np.arange(0, S, 2)
        for pq in (dev(pqs), None):
            y = p.run(dev(x), pq, 1, 1.0)
            ye = y[torch.from_numpy(even).cuda()]
            assert torch.isfinite(ye).all()
            ref = p.reference(bits(x[torch.from_numpy(even)]), pqs.numpy() if pq is not None else None, 1, 1.0)
            err = normwise(ye, ref)
            say(f"  pqs={pq is not None}: even rows normwise={err:.3e}")
            assert err <= TOL
    finally:
        p.free()


# --------------------------------------------------------------------------------------------
# sentinels around the outputs
# --------------------------------------------------------------------------------------------

SENTINEL = -12345.0  # exact in bf16


def guarded(rows, cols, pre=64, post_rows=3):
    """A [rows][cols] bf16 view into a buffer with `pre` sentinel elements before it and `post_rows`
    sentinel rows (of cols elements, plus 256 more) after it; pre keeps the view 16-byte aligned."""
    buf = torch.full((pre + (rows + post_rows) * cols + 256,), SENTINEL, dtype=torch.bfloat16, device="cuda")
    view = buf[pre:pre + rows * cols].view(rows, cols)
    assert view.data_ptr() % 16 == 0
    return buf, view, pre, rows * cols


def sentinels_intact(buf, pre, n) -> bool:
    return bool((buf[:pre] == SENTINEL).all() and (buf[pre + n:] == SENTINEL).all())


@pytest.mark.parametrize("S,K,N,gate_up", [(261, 320, 300, False), (37, 208, 520, False), (100, 256, 2 * 200, True),
                                           (77, 96, 2 * 116, True)])
def test_output_sentinels_small(S, K, N, gate_up):
    """Ragged rows and ragged last column tiles (N % 256 != 0): the plain, SwiGLU, emit and W4A4 calls
    write inside their outputs only, through both store paths."""
    say(f"sentinels S={S} K={K} N={N} gate_up={gate_up}")
    p = Proj(N, K, 1900 + N + K, gate_up=gate_up)
    try:
        p.add_adapter(1, 64, 32.0, 1901, 1902)
        x, pqs = dev(synth.activation(S, K, 1903)), dev(synth.pre_quant_scale(K, 1904))
        flag_sets = [0, h3q.H3Q_ACT_NVFP4] + ([h3q.H3Q_EPI_SWIGLU, h3q.H3Q_EPI_SWIGLU | h3q.H3Q_ACT_NVFP4] if gate_up else [])
        for fl in flag_sets:
            n_out = N // 2 if fl & h3q.H3Q_EPI_SWIGLU else N
            for aid in (1, NONE):
                buf, y, pre, n = guarded(S, n_out)
                h3q.h3q_linear_ex(x, pqs, p.handle, aid, 1.0, fl, out=y)
                torch.cuda.synchronize()
                assert sentinels_intact(buf, pre, n), (fl, aid)
                assert not (y == SENTINEL).any(), "an output element was not written"
        if gate_up and (N // 2) % 8 == 0:
            F = N // 2
            pqs_next = dev(synth.pre_quant_scale(F, 1905))
            hb, h, hpre, hn = guarded(S, F)
            xb, xs, xpre, xn = guarded(S, F)
            h3q.h3q_linear_swiglu_emit(x, pqs, p.handle, 1, 1.0, pqs_next, h=h, xs_next=xs)
            torch.cuda.synchronize()
            assert sentinels_intact(hb, hpre, hn) and sentinels_intact(xb, xpre, xn)
    finally:
        p.free()
