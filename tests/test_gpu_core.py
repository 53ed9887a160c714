"""HIP path against the fp64 oracle on small and ragged shapes (several tiles plus ragged tails):
bit-exact decode, closed-form bit-exact GEMM cases, normwise parity, adapter switching and the
invariants of the method (FL2VA Turbo, "Implementation" and "Validation")."""
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


def bf16_bits_of_exact(values: np.ndarray) -> np.ndarray:
    """Bit patterns of fp64 values that must be exact in bf16."""
    return pins.bits_of(values)


# --------------------------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------------------------

def _dequant_matches(p: Proj):
    got = bits(h3q.h3q_debug_dequant(p.handle))
    want = bf16_bits_of_exact(oracle.dequant(p.codes, p.scales, 1.0))
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_dequant_every_code_and_scale():
    """All 16 element codes against all 127 valid scale codes, bit for bit (incl. -0)."""
    N, K = 127, 64
    row = np.concatenate([np.arange(16), np.arange(16)[::-1], np.arange(16), np.arange(16)])
    nib = np.tile(row, (N, 1)).astype(np.uint8)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.tile(np.arange(127, dtype=np.uint8)[:, None], (1, K // 16))
    say("dequant table N=127 K=64")
    p = Proj(N, K, 0, codes=codes, scales=scales, ts=1.0)
    try:
        _dequant_matches(p)
    finally:
        p.free()


@pytest.mark.parametrize("N,K,gate_up", [(300, 208, False), (512, 1024, False), (2 * 200, 80, True), (2 * 128, 64, True)])
def test_dequant_random_layouts(N, K, gate_up):
    say(f"dequant random N={N} K={K} gate_up={gate_up}")
    p = Proj(N, K, 101 + N + K, gate_up=gate_up)
    try:
        _dequant_matches(p)
    finally:
        p.free()


# --------------------------------------------------------------------------------------------
# closed forms through the production GEMM (bit-exact)
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("K,N", [(128, 300), (96, 70), (320, 256)])
def test_identity_activation_bit_exact(K, N):
    """x = I, pqs = 1, ts = 2^-3: each output is one product, y = bf16(ts * Wq^T) exactly."""
    say(f"identity S=K={K} N={N}")
    rng = np.random.default_rng(K + N)
    codes, scales, _ = pins.random_nvfp4(N, K, rng)
    p = Proj(N, K, 0, codes=codes, scales=scales, ts=0.125)
    try:
        x = dev(torch.eye(K, dtype=torch.bfloat16))
        for pqs in (None, dev(torch.ones(K))):
            y = p.run(x, pqs)
            want = bf16_bits_of_exact(oracle.dequant(codes, scales, 0.125).T)
            assert np.array_equal(bits(y), want)
    finally:
        p.free()


def _exact_bf16_bits(values: np.ndarray) -> np.ndarray:
    return synth.bf16_bits(torch.from_numpy(values).to(torch.bfloat16))


@pytest.mark.parametrize("rank,alpha,strength", [(1, 2.0, 0.5), (4, 1.0, 1.0), (70, 35.0, -2.0)])
def test_onehot_rank_closed_form(rank, alpha, strength):
    """x rows one-hot, pqs powers of two, dyadic A/B: every intermediate is exact, so
    y[s, n] = bf16(ts Wq[n,k] pqs[k] + strength*alpha/rank * sum_j A[j,k] B[n,j]) bit for bit."""
    K, N, S = 192, 300, 40
    say(f"one-hot closed form rank={rank} alpha={alpha} strength={strength}")
    rng = np.random.default_rng(rank)
    codes, scales, _ = pins.random_nvfp4(N, K, rng)
    ts = 0.25
    p = Proj(N, K, 0, codes=codes, scales=scales, ts=ts)
    try:
        ks = rng.choice(K, S, replace=False)
        x = np.zeros((S, K))
        x[np.arange(S), ks] = 1.0
        pqs = (2.0 ** rng.integers(-1, 2, K)).astype(np.float32)
        A = rng.integers(-4, 5, (rank, K)) / 8.0
        B = rng.integers(-4, 5, (N, rank)) / 8.0
        p.add_adapter(5, rank, alpha, 0, 0, A=pins.bits_of(A), B=pins.bits_of(B))
        y = p.run(dev(synth.from_bf16_bits(pins.bits_of(x))), dev(torch.from_numpy(pqs)), 5, strength)
        Wd = oracle.dequant(codes, scales, ts)
        c = strength * alpha / rank
        want = Wd[:, ks].T * pqs[ks][:, None].astype(np.float64) + c * (A[:, ks].T @ B.T)
        assert np.array_equal(bits(y), _exact_bf16_bits(want))
    finally:
        p.free()


# --------------------------------------------------------------------------------------------
# normwise parity with the oracle
# --------------------------------------------------------------------------------------------

CASES = [
    # S, K, N, rank, alpha, strength, gate_up
    (256, 1024, 3072, 384, 384.0, 1.0, False),   # single fused-QKV-like projection
    (1, 48, 40, 4, 1.0, 0.7, False),
    (37, 208, 300, 65, 16.0, -1.5, False),
    (300, 1024, 520, 128, 128.0, 1.0, False),
    (513, 320, 256, 512, 64.0, 0.5, False),
    (100, 512, 2 * 200, 128, 128.0, 1.0, True),
    (70, 96, 2 * 116, 16, 8.0, 1.0, True),       # F not a multiple of 8: the 2-byte store path
    (9000, 320, 256, 128, 128.0, 1.0, False),    # LoRA-down: 36 rows per workgroup (2 row tiles, 28 rows masked)
    (9001, 256, 192, 384, 384.0, 1.0, False),    # the same with 3 column tiles per wave (r = 384)
]


@pytest.mark.parametrize("S,K,N,rank,alpha,strength,gate_up", CASES)
def test_parity_with_oracle(S, K, N, rank, alpha, strength, gate_up):
    seed = synth.seed_of(1, 0, 0) + S + K + N
    say(f"parity S={S} K={K} N={N} r={rank} alpha={alpha} strength={strength} gate_up={gate_up}")
    p = Proj(N, K, seed + synth.W, gate_up=gate_up)
    try:
        p.add_adapter(1, rank, alpha, seed + synth.A1, seed + synth.B1)
        x = synth.activation(S, K, seed + synth.X)
        pqs = synth.pre_quant_scale(K, seed + synth.PQS)
        xb, pq = bits(x), pqs.numpy()
        for aid, st in ((NONE, 0.0), (1, strength)):
            y = p.run(dev(x), dev(pqs), aid, st)
            ref = p.reference(xb, pq, aid, st)
            err = normwise(y, ref)
            say(f"  adapter={aid} normwise={err:.3e}")
            assert err <= TOL
            if gate_up:
                h = p.run(dev(x), dev(pqs), aid, st, flags=h3q.H3Q_EPI_SWIGLU)
                herr = normwise(h, oracle.swiglu(ref))
                say(f"  swiglu normwise={herr:.3e}")
                assert herr <= TOL
    finally:
        p.free()


@pytest.mark.parametrize("N,gate_up", [(520, False), (2 * 200, True)])
def test_store_paths_agree(N, gate_up):
    """Outputs whose rows are 16-byte aligned go through the LDS-staged 16-byte stores; the same call
    into a buffer offset by one element takes the 2-byte store path. Both must agree bit for bit."""
    S, K = 261, 320
    say(f"store paths N={N} gate_up={gate_up}")
    p = Proj(N, K, 950 + N, gate_up=gate_up)
    try:
        p.add_adapter(1, 32, 16.0, 951, 952)
        x, pqs = dev(synth.activation(S, K, 953)), dev(synth.pre_quant_scale(K, 954))
        flags = (0,) + ((h3q.H3Q_EPI_SWIGLU,) if gate_up else ())
        for fl in flags:
            n_out = N // 2 if fl else N
            aligned = h3q.h3q_linear_ex(x, pqs, p.handle, 1, 1.0, fl)
            buf = torch.full((S * n_out + 1,), -1.0, dtype=torch.bfloat16, device="cuda")
            shifted = h3q.h3q_linear_ex(x, pqs, p.handle, 1, 1.0, fl, out=buf[1:].view(S, n_out))
            torch.cuda.synchronize()
            assert buf[0].item() == -1.0, "store before the output"
            assert torch.equal(aligned, shifted), fl
    finally:
        p.free()


@pytest.mark.parametrize("S,K,N,rank,alpha,strength", [(256, 1024, 3072, 384, 384.0, 1.0),
                                                       (37, 208, 300, 65, 16.0, -1.5),
                                                       (300, 6144, 520, 128, 32.0, 0.5),
                                                       (70, 320, 400, 150, 75.0, 1.0),
                                                       (48, 256, 260, 300, 64.0, 0.75)])
def test_mirror_tight_parity(S, K, N, rank, alpha, strength):
    """Against the mirror oracle (exact arithmetic with the GPU's declared rounding points: xs and t' in
    bf16, one fp32 scale, bf16 store) the only difference left is the GPU's fp32 accumulation, which
    moves an output across a bf16 rounding boundary with probability about 2 sqrt(K) 2^-24 / 2^-8
    (~0.1 %), by one unit: at least 98 % of outputs must be bit-identical and the normwise distance
    at most 1e-3 -- tight enough to show a scale or fold error of a fraction of a percent."""
    say(f"mirror S={S} K={K} N={N} r={rank} alpha={alpha} strength={strength}")
    p = Proj(N, K, 2300 + S + K)
    try:
        p.add_adapter(1, rank, alpha, 2301, 2302)
        x = synth.activation(S, K, 2303)
        pqs = synth.pre_quant_scale(K, 2304)
        for aid, st in ((1, strength), (NONE, 0.0)):
            y = p.run(dev(x), dev(pqs), aid, st)
            kw = {}
            if aid != NONE:
                A, B, r, al = p.adapters[aid]
                kw = dict(A_bits=A, B_bits=B, rank=r, alpha=al, strength=st)
            mirror = oracle.linear_mirror(bits(x), pqs.numpy(), p.codes, p.scales, p.ts, **kw)
            same = float(np.mean(bits(y) == mirror))
            err = normwise(y, pins.bf16_values(mirror))
            say(f"  adapter={aid}: {100 * same:.2f} % bit-identical, normwise {err:.2e}")
            assert same >= 0.98 and err <= 1e-3, (same, err)
    finally:
        p.free()


def test_lora_only_parity():
    """All-zero weight codes: the output is the LoRA term alone, B(A x) on the original x."""
    S, K, N, r = 200, 320, 300, 96
    say("lora-only")
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    p = Proj(N, K, 0, codes=codes, scales=scales, ts=0.01)
    try:
        p.add_adapter(3, r, 24.0, 11, 12)
        x = synth.activation(S, K, 13)
        pqs = synth.pre_quant_scale(K, 14)
        y = p.run(dev(x), dev(pqs), 3, 0.8)
        ref = p.reference(bits(x), pqs.numpy(), 3, 0.8)
        err = normwise(y, ref)
        say(f"  normwise={err:.3e}")
        assert err <= TOL
        # the LoRA branch must not see pqs: same output with pqs = 2 * pqs
        y2 = p.run(dev(x), dev(pqs * 2), 3, 0.8)
        assert torch.equal(y, y2)
    finally:
        p.free()


def test_no_pqs_direct_path():
    """pqs = NULL with K a multiple of 64 feeds x straight to the GEMM; K = 80 goes through the
    padded operand; both match the oracle with pqs = 1."""
    for K in (256, 80):
        S, N = 130, 200
        say(f"no-pqs K={K}")
        p = Proj(N, K, 77 + K)
        try:
            p.add_adapter(2, 16, 8.0, 1, 2)
            x = synth.activation(S, K, 3)
            for aid, st in ((NONE, 0.0), (2, 1.0)):
                y = p.run(dev(x), None, aid, st)
                err = normwise(y, p.reference(bits(x), None, aid, st))
                assert err <= TOL, err
        finally:
            p.free()


# --------------------------------------------------------------------------------------------
# adapter selection, exactness when disabled, immutability (FL2VA Turbo, "Hot API", "Validation")
# --------------------------------------------------------------------------------------------

def test_adapter_none_is_bit_identical_and_weight_immutable():
    S, K, N = 300, 512, 640
    say("switching / disabled exactness")
    p = Proj(N, K, 501)
    try:
        x = dev(synth.activation(S, K, 502))
        pqs = dev(synth.pre_quant_scale(K, 503))
        base0 = p.run(x, pqs)
        ck0 = h3q.h3q_weight_checksum(p.handle)
        p.add_adapter(1, 128, 128.0, 504, 505)
        p.add_adapter(2, 128, 128.0, 506, 507)
        assert h3q.h3q_list_adapters(p.handle) == [1, 2]
        outs = {}
        for aid, st in ((1, 1.0), (NONE, 0.0), (2, 0.5), (1, 0.0), (2, 1.0), (NONE, 1.0), (1, 1.0)):
            outs.setdefault((aid, st), []).append(p.run(x, pqs, aid, st))
        for y in outs[(NONE, 0.0)] + outs[(1, 0.0)] + outs[(NONE, 1.0)]:
            assert torch.equal(y, base0)
        a, b = outs[(1, 1.0)]
        assert torch.equal(a, b)                      # deterministic, order-independent
        assert not torch.equal(outs[(1, 1.0)][0], outs[(2, 1.0)][0])
        assert h3q.h3q_weight_checksum(p.handle) == ck0   # packed base never written
        h3q.h3q_unregister_adapter(p.handle, 1)
        assert torch.equal(p.run(x, pqs), base0)
        with pytest.raises(h3q.H3QError) as e:
            p.run(x, pqs, 1, 1.0)
        assert e.value.code == h3q.H3Q_E_ADAPTER
        with pytest.raises(h3q.H3QError) as e:
            p.add_adapter(2, 128, 128.0, 1, 2)
        assert e.value.code == h3q.H3Q_E_ADAPTER
    finally:
        p.free()


def test_row_locality_and_determinism_small():
    """Rows are independent: the first S rows do not change when more rows are appended."""
    K, N = 256, 300
    say("row locality small")
    p = Proj(N, K, 601)
    try:
        p.add_adapter(1, 64, 64.0, 602, 603)
        x2 = synth.activation(302, K, 604)
        pqs = dev(synth.pre_quant_scale(K, 605))
        for aid in (NONE, 1):
            y_short = p.run(dev(x2[:300].contiguous()), pqs, aid, 1.0)
            y_long = p.run(dev(x2), pqs, aid, 1.0)
            assert torch.equal(y_short, y_long[:300])
            assert torch.equal(y_long, p.run(dev(x2), pqs, aid, 1.0))
    finally:
        p.free()


def test_empty_and_argument_errors():
    K, N = 64, 64
    p = Proj(N, K, 701)
    try:
        x = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
        y = p.run(x, None)
        assert y.shape == (0, N)
        xs = dev(synth.activation(8, K, 1))
        with pytest.raises(h3q.H3QError) as e:
            p.run(xs, None, 42, 1.0)
        assert e.value.code == h3q.H3Q_E_ADAPTER
        with pytest.raises(h3q.H3QError) as e:
            p.run(xs, None, flags=h3q.H3Q_EPI_SWIGLU)  # not packed as gate/up
        assert e.value.code == h3q.H3Q_E_ARG
        big = torch.zeros((9 * K + 8,), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(h3q.H3QError) as e:  # misaligned x (offset of one element)
            h3q.h3q_linear(big[1:1 + 8 * K].view(8, K), None, p.handle, NONE, 0.0)
        assert e.value.code == h3q.H3Q_E_ARG
        buf = torch.zeros((8 * max(K, N),), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(h3q.H3QError) as e:  # y overlaps x
            h3q.h3q_linear(buf[:8 * K].view(8, K), None, p.handle, NONE, 0.0, y=buf[:8 * N].view(8, N))
        assert e.value.code == h3q.H3Q_E_ARG
        with pytest.raises(h3q.H3QError) as e:
            h3q.h3q_linear(xs, None, p.handle, NONE, float("nan"))
        assert e.value.code == h3q.H3Q_E_ARG
    finally:
        p.free()


def test_allocation_failure_hook(monkeypatch):
    """With allocations failing, pack and adapter registration report E_NOMEM and leave nothing."""
    N, K = 64, 64
    rng = np.random.default_rng(5)
    codes, scales, ts = pins.random_nvfp4(N, K, rng)
    monkeypatch.setenv("H3Q_TEST_FAIL_ALLOC_AFTER", "1")  # the codes buffer succeeds, scales fail
    with pytest.raises(h3q.H3QError) as e:
        h3q.h3q_pack_weight(codes, scales, ts, N, K)
    assert e.value.code == h3q.H3Q_E_NOMEM
    monkeypatch.delenv("H3Q_TEST_FAIL_ALLOC_AFTER")
    p = Proj(N, K, 0, codes=codes, scales=scales, ts=ts)
    try:
        monkeypatch.setenv("H3Q_TEST_FAIL_ALLOC_AFTER", "0")
        with pytest.raises(h3q.H3QError) as e:
            p.add_adapter(1, 8, 8.0, 1, 2)
        assert e.value.code == h3q.H3Q_E_NOMEM
        monkeypatch.delenv("H3Q_TEST_FAIL_ALLOC_AFTER")
        assert h3q.h3q_list_adapters(p.handle) == []
    finally:
        p.free()


# --------------------------------------------------------------------------------------------
# W4A4: the activation quantizer (bit-exact) and the linear with quantized activations
# --------------------------------------------------------------------------------------------

def test_activation_quantizer_bit_exact():
    for (S, K, seed, use_pqs) in ((37, 208, 1, True), (256, 1024, 2, True), (5, 16, 3, False)):
        say(f"act-quant S={S} K={K}")
        x = synth.activation(S, K, seed)
        pqs = synth.pre_quant_scale(K, seed + 1) if use_pqs else None
        codes, scales, ts = h3q.h3q_quantize_nvfp4(dev(x), dev(pqs) if use_pqs else None)
        torch.cuda.synchronize()
        oc, osc, ots = oracle.w4a4_activation(bits(x), pqs.numpy() if use_pqs else None)
        assert np.array_equal(codes.cpu().numpy(), oc)
        assert np.array_equal(scales.cpu().numpy(), osc)
        assert ts.item() == ots


def test_activation_quantizer_midpoints():
    """The hand-built block of tests/pins.py (E2M1 and E4M3 ties) through the device quantizer."""
    q = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0]
    blk1 = [6.375, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.0, -0.0, 0.25, 5.5, 0.75, -0.25, 2.75, 6.25]
    v = np.array([[a * 448 for a in q] + blk1])
    x = synth.from_bf16_bits(pins.bits_of(v))
    codes, scales, ts = h3q.h3q_quantize_nvfp4(dev(x))
    torch.cuda.synchronize()
    oc, osc, ots = oracle.w4a4_activation(pins.bits_of(v), None)
    assert ts.item() == 1.0 == ots
    assert list(scales.cpu().numpy()[0]) == [0x7E, 0x38] == list(osc[0])
    assert np.array_equal(codes.cpu().numpy(), oc)


@pytest.mark.parametrize("S,K,N,gate_up", [(256, 1024, 512, False), (77, 208, 2 * 160, True)])
def test_w4a4_linear_parity(S, K, N, gate_up):
    say(f"w4a4 S={S} K={K} N={N}")
    p = Proj(N, K, 801 + K, gate_up=gate_up)
    try:
        p.add_adapter(1, 128, 128.0, 802, 803)
        x = synth.activation(S, K, 804)
        pqs = synth.pre_quant_scale(K, 805)
        for aid, st in ((NONE, 0.0), (1, 1.0)):
            y = p.run(dev(x), dev(pqs), aid, st, flags=h3q.H3Q_ACT_NVFP4)
            ref = p.reference(bits(x), pqs.numpy(), aid, st, w4a4=True)
            err = normwise(y, ref)
            say(f"  adapter={aid} normwise={err:.3e}")
            assert err <= TOL
            if gate_up:
                h = p.run(dev(x), dev(pqs), aid, st, flags=h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU)
                assert normwise(h, oracle.swiglu(ref)) <= TOL
    finally:
        p.free()


def test_timing_counts_launches_per_kernel():
    """The per-kernel timing behind the benchmark's breakdown: each call records one launch of each
    kernel it runs, a read returns and clears that kernel's totals, and nothing is recorded while
    timing is off."""
    S, K, N = 200, 512, 512
    say("timing counts")
    p = Proj(N, K, 1700)
    try:
        p.add_adapter(1, 32, 32.0, 1701, 1702)
        x = dev(synth.activation(S, K, 1703))
        pqs = dev(synth.pre_quant_scale(K, 1704))
        kinds = (h3q.H3Q_KERNEL_GEMM, h3q.H3Q_KERNEL_LORA_DOWN, h3q.H3Q_KERNEL_PRESCALE, h3q.H3Q_KERNEL_ACT_QUANT)
        h3q.h3q_timing_enable(False)
        h3q.h3q_linear_ex(x, pqs, p.handle, 1, 1.0, 0)
        h3q.h3q_timing_enable(True)
        for _ in range(3):
            h3q.h3q_linear_ex(x, pqs, p.handle, 1, 1.0, 0)                      # LoRA-down + GEMM
        for _ in range(2):
            h3q.h3q_linear_ex(x, pqs, p.handle, h3q.H3Q_ADAPTER_NONE, 0.0, 0)   # prescale + GEMM
        h3q.h3q_linear_ex(x, pqs, p.handle, h3q.H3Q_ADAPTER_NONE, 0.0, h3q.H3Q_ACT_NVFP4)  # act-quant + GEMM
        torch.cuda.synchronize()
        got = {k: h3q.h3q_timing_get(k) for k in kinds}
        assert [got[k][1] for k in kinds] == [6, 3, 2, 1], got
        assert all(got[k][0] > 0.0 for k in kinds), got
        assert h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM) == (0.0, 0)  # read clears
        h3q.h3q_timing_enable(False)
        h3q.h3q_linear_ex(x, pqs, p.handle, 1, 1.0, 0)
        torch.cuda.synchronize()
        assert h3q.h3q_timing_get(h3q.H3Q_KERNEL_GEMM) == (0.0, 0)
    finally:
        h3q.h3q_timing_enable(False)
        p.free()
