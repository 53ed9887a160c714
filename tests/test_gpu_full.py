"""HIP path at the full projection shapes of one MiniMax-H3 DiT block (d = 6144, d_ff = 16384), in
the launch configuration the benchmark times: S = 8192; the packed canvas length S = 37726 and its
neighbour S = 37728 through the same call; adapter switching at S = 16384; and the W4A4 + SwiGLU
gate/up projection at S = 37726.

The oracle checks a deterministic row sample (the first 256 rows, the last 256 rows -- which hold
the ragged last row tile -- and every 64th row between). The bit-level contracts are checked on
every row: row locality across S, adapter none and strength 0 against a handle that never had an
adapter, determinism, the packed weight's checksum, and the W4A4 activation quantizer.
(FL2VA Turbo, "Implementation" and "Validation"; MiniMax-H3 Ultra Fast, "Kernel path".)"""
import numpy as np
import pytest
import torch

import bit_linear_dynamic_amd as h3q
import oracle
import pins
from bit_linear_dynamic_amd import synth
from bit_linear_dynamic_amd import workloads as wl
from gpu_helpers import TOL, Proj, bits, normwise, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

NONE = h3q.H3Q_ADAPTER_NONE
NAMES = [p.name for p in wl.BLOCK]
WEIGHT_CONFIG = 2   # one set of block weights serves every full-size case ("the same four projections")


def rows_sample(S: int, edge: int = 256, stride: int = 64) -> np.ndarray:
    r = np.concatenate([np.arange(min(edge, S)), np.arange(edge, max(S - edge, edge), stride),
                        np.arange(max(S - edge, 0), S)])
    return np.unique(r)


@pytest.fixture(scope="module")
def block():
    """The four projections: NVFP4 weights from the oracle's quantizer, two adapters each
    (distinct seeds, the projection's rank with alpha = rank)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    projs = {}
    try:
        for i, p in enumerate(wl.BLOCK):
            say(f"packing {p.name} {p.N}x{p.K} r={p.rank}")
            pr = Proj(p.N, p.K, synth.seed_of(WEIGHT_CONFIG, i, synth.W), gate_up=p.gate_up)
            pr.add_adapter(1, p.rank, p.alpha, synth.seed_of(WEIGHT_CONFIG, i, synth.A1),
                           synth.seed_of(WEIGHT_CONFIG, i, synth.B1))
            pr.add_adapter(2, p.rank, p.alpha, synth.seed_of(WEIGHT_CONFIG, i, synth.A2),
                           synth.seed_of(WEIGHT_CONFIG, i, synth.B2))
            projs[p.name] = (i, p, pr)
        yield projs
    finally:
        for _, _, pr in projs.values():
            pr.free()
        torch.cuda.synchronize()


def inputs(config: int, i: int, S: int, K: int):
    x = synth.activation(S, K, synth.seed_of(config, i, synth.X), "cuda")
    pqs = synth.pre_quant_scale(K, synth.seed_of(config, i, synth.PQS), "cuda")
    return x, pqs


def check_rows(pr: Proj, y: torch.Tensor, x: torch.Tensor, pqs: torch.Tensor, rows: np.ndarray,
               adapter_id: int, strength: float, what: str) -> float:
    idx = torch.from_numpy(rows).to(x.device)
    ref = pr.reference(bits(x.index_select(0, idx)), pqs.cpu().numpy(), adapter_id, strength)
    err = normwise(y.index_select(0, idx), ref)
    say(f"  {what}: {len(rows)} sampled rows, normwise={err:.3e}")
    assert err <= TOL, (what, err)
    return err


@pytest.mark.parametrize("name", NAMES)
def test_block_s8192(block, name):
    i, p, pr = block[name]
    S = wl.S_MID
    say(f"S={S} {name}")
    x, pqs = inputs(2, i, S, p.K)
    y = h3q.h3q_linear(x, pqs, pr.handle, 1, 1.0)
    torch.cuda.synchronize()
    check_rows(pr, y, x, pqs, rows_sample(S, stride=128), 1, 1.0, "adapter 1, strength 1")
    # the mirror oracle (the GPU's declared rounding points) on the first and last 48 rows: only the
    # fp32 accumulation order differs, so nearly every output is bit-identical
    rows = np.concatenate([np.arange(48), np.arange(S - 48, S)])
    idx = torch.from_numpy(rows).to(x.device)
    A, B, r, alpha = pr.adapters[1]
    mirror = oracle.linear_mirror(bits(x.index_select(0, idx)), pqs.cpu().numpy(), pr.codes, pr.scales, pr.ts,
                                  A, B, r, alpha, 1.0)
    yb = bits(y.index_select(0, idx))
    same = float(np.mean(yb == mirror))
    err = normwise(y.index_select(0, idx), pins.bf16_values(mirror))
    say(f"  mirror: {100 * same:.2f} % bit-identical, normwise {err:.2e}")
    assert same >= 0.98 and err <= 1e-3


@pytest.mark.parametrize("name", NAMES)
def test_canvas_s37726_and_s37728(block, name):
    """S = 37726 (a ragged last tile of 94 rows) and S = 37728 through the same call; the first
    37726 rows of the longer input are the shorter input, so their outputs must be bit-identical."""
    i, p, pr = block[name]
    say(f"S={wl.S_CANVAS}/{wl.S_CANVAS_ALT} {name}")
    x_long, pqs = inputs(3, i, wl.S_CANVAS_ALT, p.K)
    x_short = x_long[:wl.S_CANVAS].contiguous()
    y_short = h3q.h3q_linear(x_short, pqs, pr.handle, 1, 1.0)
    y_long = h3q.h3q_linear(x_long, pqs, pr.handle, 1, 1.0)
    y_again = h3q.h3q_linear(x_long, pqs, pr.handle, 1, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(y_short, y_long[:wl.S_CANVAS]), "row locality across S"
    assert torch.equal(y_long, y_again), "run-to-run determinism"
    del y_again, x_short
    check_rows(pr, y_long, x_long, pqs, rows_sample(wl.S_CANVAS_ALT), 1, 1.0, "adapter 1, strength 1")


@pytest.mark.parametrize("name", NAMES)
def test_adapter_switching_s16384(block, name):
    """Two resident adapters selected per call with strength 0, 0.5 and 1, and adapter none:
    none and strength 0 are bit-identical to a handle that never had an adapter, repeated calls
    agree bit for bit, the packed weight is never written, and the adapted outputs match the oracle."""
    i, p, pr = block[name]
    S = wl.S_SWITCH
    say(f"S={S} switching {name}")
    x, pqs = inputs(4, i, S, p.K)
    ck0 = h3q.h3q_weight_checksum(pr.handle)
    bare = Proj(p.N, p.K, 0, gate_up=p.gate_up, codes=pr.codes, scales=pr.scales, ts=pr.ts)
    try:
        base = bare.run(x, pqs)
    finally:
        bare.free()
    order = [(1, 1.0), (NONE, 0.0), (2, 0.5), (1, 0.0), (2, 1.0), (NONE, 1.0), (1, 0.5), (2, 0.0), (1, 1.0),
             (2, 0.5)]
    outs = {}
    for aid, st in order:
        outs.setdefault((aid, st), []).append(pr.run(x, pqs, aid, st))
    for key in ((NONE, 0.0), (1, 0.0), (NONE, 1.0), (2, 0.0)):
        for y in outs[key]:
            assert torch.equal(y, base), ("disabled path differs from the base-only path", key)
    for key in ((1, 1.0), (2, 0.5)):
        a, b = outs[key]
        assert torch.equal(a, b), ("repeat differs", key)
    assert not torch.equal(outs[(1, 1.0)][0], outs[(2, 1.0)][0])
    assert h3q.h3q_weight_checksum(pr.handle) == ck0, "packed weight modified"
    rows = rows_sample(S, stride=256)
    check_rows(pr, base, x, pqs, rows, NONE, 0.0, "adapter none")
    check_rows(pr, outs[(2, 0.5)][0], x, pqs, rows, 2, 0.5, "adapter 2, strength 0.5")
    check_rows(pr, outs[(1, 1.0)][0], x, pqs, rows, 1, 1.0, "adapter 1, strength 1")


def test_w4a4_swiglu_gate_up_s37726(block):
    """Activations quantized to NVFP4 on every call for the base GEMM (bit-exact against the oracle's
    quantizer over the whole tensor), LoRA on the original bf16 x, SiLU(gate) * up in the epilogue."""
    i, p, pr = block["gate_up"]
    S = wl.S_CANVAS
    say(f"W4A4 + SwiGLU gate/up S={S}")
    x, pqs = inputs(5, i, S, p.K)
    codes, scales, ts_a = h3q.h3q_quantize_nvfp4(x, pqs)
    h = h3q.h3q_linear_ex(x, pqs, pr.handle, 1, 1.0, h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU)
    torch.cuda.synchronize()
    assert tuple(h.shape) == (S, p.N // 2)
    xb, pq = bits(x), pqs.cpu().numpy()
    say("  oracle quantizer over the whole activation")
    oc, osc, ots = oracle.w4a4_activation(xb, pq)
    assert ts_a.item() == ots
    assert np.array_equal(scales.cpu().numpy(), osc)
    assert np.array_equal(codes.cpu().numpy(), oc)
    del codes, scales
    rows = rows_sample(S)
    A, B, r, alpha = pr.adapters[1]
    y_ref = oracle.linear(xb[rows], pq, pr.codes, pr.scales, pr.ts, A, B, r, alpha, 1.0,
                          act_codes=oc[rows], act_scales=osc[rows], ts_a=ots)
    err = normwise(h.index_select(0, torch.from_numpy(rows).cuda()), oracle.swiglu(y_ref))
    say(f"  h: {len(rows)} sampled rows, normwise={err:.3e}")
    assert err <= TOL


def test_rows_beyond_32bit_offsets(block):
    """The down projection (K = 16384) at S = 65836: the activation spans 2.16 GB, past what a 32-bit
    offset from the buffer's start reaches at 2 GiB (the GEMM addresses each tile from its first
    row). Rows on both sides of each 2 GiB boundary and the ragged tail match the oracle, and the
    first rows are bit-identical to a short call's."""
    i, p, pr = block["down"]
    S = 65836
    say(f"S={S} down, past 2 GiB of operand")
    x, pqs = inputs(6, i, S, p.K)
    y = h3q.h3q_linear(x, pqs, pr.handle, 1, 1.0)
    y_short = h3q.h3q_linear(x[:300].contiguous(), pqs, pr.handle, 1, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(y[:300], y_short)
    # the rows around each 1 GiB point of the activation (row 32768: 1 GiB, 65536: 2 GiB, the reach of
    # a signed 32-bit offset from the buffer's start)
    per_gib = (1 << 30) // (p.K * 2)
    edges = [np.arange(max(0, b - 96), min(S, b + 96)) for b in range(per_gib, S, per_gib)]
    rows = np.unique(np.concatenate([np.arange(64), np.arange(0, S, 509), np.arange(S - 160, S)] + edges))
    check_rows(pr, y, x, pqs, rows, 1, 1.0, "adapter 1, strength 1, around the 1 and 2 GiB points")


SENTINEL = -12345.0  # exact in bf16


def _guarded(rows, cols, post_rows=2):
    """A [rows][cols] bf16 view with 64 sentinel elements before it and post_rows sentinel rows after it."""
    buf = torch.full((64 + (rows + post_rows) * cols,), SENTINEL, dtype=torch.bfloat16, device="cuda")
    return buf, buf[64:64 + rows * cols].view(rows, cols), 64, rows * cols


def _intact(buf, pre, n) -> bool:
    return bool((buf[:pre] == SENTINEL).all() and (buf[pre + n:] == SENTINEL).all())


@pytest.mark.parametrize("S", [wl.S_CANVAS, wl.S_CANVAS_ALT])
def test_output_sentinels_full(block, S):
    """Sentinel rows after the last row (the 94-row tail tile at S = 37726) and sentinels before the
    first element stay untouched for the QKV projection (plain and with the fused Q/K epilogue) and the
    gate/up SwiGLU projection with the emitted down operand; every output element is written."""
    say(f"output sentinels S={S}")
    i, p, pr = block["qkv"]
    x, pqs = inputs(7, i, S, p.K)
    buf, y, pre, n = _guarded(S, p.N)
    h3q.h3q_linear(x, pqs, pr.handle, 1, 1.0, y=y)
    torch.cuda.synchronize()
    assert _intact(buf, pre, n) and not (y == SENTINEL).any(), "qkv plain"
    q_width, rot = 6144, 96
    g = synth.uniform((2, q_width), 0.5, 1.5, 7001, "cuda")
    cos, sin = synth.rope_table(S, rot)
    h3q.h3q_linear_qk_norm_rope(x, pqs, pr.handle, 1, 1.0, q_width, rot, 1e-6, g[0].contiguous(), g[1].contiguous(),
                                cos.cuda(), sin.cuda(), y=y)
    torch.cuda.synchronize()
    assert _intact(buf, pre, n) and not (y == SENTINEL).any(), "qkv with the Q/K epilogue"
    del buf, y, x
    i, p, pr = block["gate_up"]
    x, pqs = inputs(7, i, S, p.K)
    F = p.N // 2
    pqs_next = synth.pre_quant_scale(F, 7002, "cuda")
    hb, h, hpre, hn = _guarded(S, F)
    xb, xs, xpre, xn = _guarded(S, F)
    h3q.h3q_linear_swiglu_emit(x, pqs, pr.handle, 1, 1.0, pqs_next, h=h, xs_next=xs)
    torch.cuda.synchronize()
    assert _intact(hb, hpre, hn) and _intact(xb, xpre, xn), "gate/up SwiGLU with emit"
    assert not (h == SENTINEL).any() and not (xs == SENTINEL).any()
