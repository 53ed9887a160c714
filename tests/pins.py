"""Pins of the fp64 oracle: each check sets the oracle against something that is not the oracle.

Independent sources used here:
  * the published code tables of the format (tests/golden/nvfp4_format.txt) and torch's own
    float8_e4m3fn conversion (a library routine) for decoding and for RNE encoding of E4M3;
  * exact rational arithmetic (fractions.Fraction) with brute-force nearest-value search over the
    whole code table, for the encoders and the quantizer (the oracle instead brackets the value
    and compares with the midpoint in fp64);
  * numpy's fp64 matmul on an independently decoded weight, for the contraction;
  * closed forms: identity activations, one-hot activations against rank-1 adapters, zero weights;
  * torch's SiLU in fp64 and the identity SiLU(z) - SiLU(-z) = z.

Every pin is a function of the loaded oracle library (``lib``) so that tests/test_oracle_mutants.py
can re-run all of them against deliberately broken builds of the oracle and show each break is
caught. A pin raises AssertionError when the oracle disagrees.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------------------------------------
# independent references
# ------------------------------------------------------------------------------------------------

def read_format_tables():
    tables, cur = {}, None
    with open(os.path.join(GOLDEN, "nvfp4_format.txt")) as f:
        for raw in f:
            line = raw.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                tables[cur] = {}
                continue
            code, val = line.split()
            tables[cur][int(code, 0)] = float(val)
    return tables["e2m1"], tables["e4m3"]


E2M1_GOLDEN, E4M3_LANDMARKS = read_format_tables()
E2M1_ARRAY = np.array([E2M1_GOLDEN[c] for c in range(16)], np.float64)


def e4m3_torch(codes) -> np.ndarray:
    """Decode E4M3FN codes with torch's float8_e4m3fn dtype."""
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def e4m3_encode_torch(values) -> np.ndarray:
    """RNE-encode non-negative values <= 464 with torch's float8_e4m3fn cast."""
    t = torch.tensor(np.asarray(values, np.float64), dtype=torch.float64).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def decode_independent(codes: np.ndarray, scales: np.ndarray, ts: float) -> np.ndarray:
    """NVFP4 -> fp64 with the golden E2M1 table and torch's E4M3 (low nibble = even k)."""
    rows = codes.shape[0]
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(rows, -1)
    sc = np.repeat(e4m3_torch(scales), 16, axis=1)
    return E2M1_ARRAY[nib] * sc * float(ts)


E2M1_FRAC = {c: Fraction(E2M1_GOLDEN[c]) for c in range(8)}
E4M3_FRAC = {c: Fraction(float(v)) for c, v in enumerate(e4m3_torch(np.arange(0x7F, dtype=np.uint8)))}


def nearest_code(value: Fraction, table: dict) -> int:
    """Brute force: the code whose value is nearest; on a tie the code with even LSB (mantissa)."""
    best = None
    for c, v in table.items():
        d = abs(value - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def round_to_f32(fr: Fraction) -> float:
    """Correctly rounded (ties to even) binary32 of a non-negative rational, normal or subnormal."""
    if fr == 0:
        return 0.0
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    while Fraction(2) ** e > fr:
        e -= 1
    while Fraction(2) ** (e + 1) <= fr:
        e += 1
    e = max(e, -126)
    q = fr / Fraction(2) ** (e - 23)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(Fraction(n) * Fraction(2) ** (e - 23))


def quantize_exact(v: np.ndarray):
    """NVFP4 quantization of an fp32 [rows][K] array in exact rationals (reading of the scale rules:
    tensor scale = amax/(6*448) rounded to fp32; block scale = E4M3 nearest to amax_b/(6*ts);
    element = E2M1 nearest to v/(scale*ts), saturating; zero block scale -> zero codes)."""
    rows, K = v.shape
    fr = [[Fraction(float(a)) for a in row] for row in v]
    amax = max((abs(a) for row in fr for a in row), default=Fraction(0))
    ts = Fraction(1) if amax == 0 else Fraction(round_to_f32(amax / 2688))
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    for r in range(rows):
        for b in range(K // 16):
            blk = fr[r][16 * b:16 * b + 16]
            s = nearest_code(max(abs(a) for a in blk) / (6 * ts), E4M3_FRAC)
            scales[r, b] = s
            d = E4M3_FRAC[s] * ts
            for i, a in enumerate(blk):
                if d == 0:
                    c = 0
                else:
                    mag = nearest_code(abs(a) / d, E2M1_FRAC)
                    c = 0 if mag == 0 else (mag | (8 if a < 0 else 0))
                codes[r, 8 * b + i // 2] |= c << (4 * (i % 2))
    return codes, scales, float(ts)


def bits_of(values) -> np.ndarray:
    """fp64 values exactly representable in bf16 -> bf16 bit patterns (asserts exactness)."""
    t = torch.tensor(np.asarray(values, np.float64))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float64), t), "value not exact in bf16"
    return b.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def random_bf16(shape, std, rng) -> np.ndarray:
    return bits_of(torch.tensor(rng.standard_normal(shape) * std).to(torch.bfloat16).to(torch.float64).numpy())


def random_nvfp4(N, K, rng, std=0.02, lib=None):
    w = (rng.standard_normal((N, K)) * std).astype(np.float32)
    return oracle.quantize_nvfp4(w, lib=lib)


# ------------------------------------------------------------------------------------------------
# pins: codec
# ------------------------------------------------------------------------------------------------

def pin_e2m1_table(lib):
    for c in range(16):
        got, want = oracle.e2m1_value(c, lib), E2M1_GOLDEN[c]
        assert got == want and np.signbit(got) == np.signbit(want), (c, got, want)


def pin_e4m3_vs_torch(lib):
    want = e4m3_torch(np.arange(256, dtype=np.uint8))
    got = np.array([oracle.e4m3_value(c, lib) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def pin_e4m3_landmarks(lib):
    for c, v in E4M3_LANDMARKS.items():
        got = oracle.e4m3_value(c, lib)
        if np.isnan(v):
            assert np.isnan(got), hex(c)
        else:
            assert got == v and np.signbit(got) == np.signbit(v), (hex(c), got, v)


def pin_e4m3_encode_vs_torch(lib):
    rng = np.random.default_rng(11)
    finite = e4m3_torch(np.arange(0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2
    vals = np.concatenate([finite, mids, rng.uniform(0, 464, 2000), np.exp(rng.uniform(-12, 6, 2000)),
                           [448.0, 455.0, 464.0]])
    want = e4m3_encode_torch(vals)
    got = np.array([oracle.e4m3_encode(v, lib) for v in vals], np.uint8)
    assert np.array_equal(got, want), vals[got != want][:8]
    for v in (465.0, 1e6, 1e30):  # saturating, where torch would give NaN
        assert oracle.e4m3_encode(v, lib) == 0x7E


def pin_e2m1_encode_hand_vectors(lib):
    # midpoints of the E2M1 grid round to the neighbour with mantissa bit 0
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.2499: 0, 0.2501: 1, 0.7499: 1, 0.7501: 2, 1.2501: 3, 1.7499: 3, 2.5001: 5, 3.4999: 5,
             4.9999: 6, 5.0001: 7, 6.0: 7, 7.0: 7, 1e9: 7, 0.0: 0, 0.1: 0}
    for q, c in cases.items():
        assert oracle.e2m1_encode(q, lib) == c, (q, c)
        want_neg = 0 if c == 0 else (c | 8)
        assert oracle.e2m1_encode(-q, lib) == want_neg, (-q, want_neg)


def pin_e2m1_encode_bruteforce(lib):
    rng = np.random.default_rng(12)
    vals = np.concatenate([rng.uniform(-7, 7, 3000), np.arange(-28, 29) / 4.0])
    for v in vals:
        mag = nearest_code(abs(Fraction(float(v))), E2M1_FRAC)
        want = 0 if mag == 0 else (mag | (8 if v < 0 else 0))
        assert oracle.e2m1_encode(v, lib) == want, v


# ------------------------------------------------------------------------------------------------
# pins: quantizer
# ------------------------------------------------------------------------------------------------

def pin_quantizer_exact_random(lib):
    rng = np.random.default_rng(13)
    arrays = [
        rng.standard_normal((3, 64)).astype(np.float32),
        (rng.standard_normal((2, 48)) * np.exp(rng.uniform(-20, 5, (2, 48)))).astype(np.float32),
        np.zeros((1, 32), np.float32),
        np.concatenate([np.zeros(16), rng.standard_normal(16) * 1e-8]).reshape(1, 32).astype(np.float32),
    ]
    for v in arrays:
        got = oracle.quantize_nvfp4(v, lib=lib)
        want = quantize_exact(v)
        assert np.array_equal(got[0], want[0]), "codes"
        assert np.array_equal(got[1], want[1]), "scales"
        assert got[2] == want[2], "tensor scale"


def pin_quantizer_hand_block(lib):
    # amax = 2688 = 6 * 448 makes the tensor scale exactly 1 and block 0's scale 448 (code 0x7E);
    # every other element then sits on a known point of the E2M1 grid times 448.
    q = [2688 / 448, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0]
    # block 1: amax 6.375 = 6 * 1.0625, an E4M3 midpoint (1.0 | 1.125) -> scale 1.0 (code 0x38)
    blk1 = [6.375, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, -6.0, 0.0, -0.0, 0.24, 5.5, 0.75, -0.25, 2.9, 6.2]
    v = np.array([[x * 448 for x in q] + blk1], np.float32)
    codes, scales, ts = oracle.quantize_nvfp4(v, lib=lib)
    assert ts == 1.0
    assert list(scales[0]) == [0x7E, 0x38]
    want0 = [7, 0, 2, 2, 4, 4, 6, 6, 0, 10, 10, 12, 12, 14, 14, 15]
    want1 = [7, 1, 2, 3, 4, 5, 6, 15, 0, 0, 0, 7, 2, 0, 5, 7]
    nib = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=-1).reshape(-1)
    assert list(nib[:16]) == want0, list(nib[:16])
    assert list(nib[16:]) == want1, list(nib[16:])


def pin_quantizer_bounds(lib):
    rng = np.random.default_rng(14)
    v = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    codes, scales, ts = oracle.quantize_nvfp4(v, lib=lib)
    assert ts == np.float32(np.float64(np.abs(v).max()) / 2688)
    deq = decode_independent(codes, scales, ts)
    d = np.repeat(e4m3_torch(scales), 16, axis=1) * ts
    # every element is within half a grid step (at most 1 * d, between 4 and 6) of its value
    assert np.all(np.abs(deq - v) <= 1.0 * d + 1e-30)
    # the block maximum does not saturate beyond the grid: |v| <= 6 d (1 + 2^-4) per element
    assert np.all(np.abs(v) <= 6 * d * (1 + 2 ** -4))


# ------------------------------------------------------------------------------------------------
# pins: dequantization layout and the linear
# ------------------------------------------------------------------------------------------------

def pin_dequant_vs_independent(lib):
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 256, (5, 24), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (5, 3), dtype=np.uint8)
    got = oracle.dequant(codes, scales, 0.375, lib=lib)
    want = decode_independent(codes, scales, 0.375)
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))


def _lora_case(rng, M, K, N, r, lib):
    x = random_bf16((M, K), 1.0, rng)
    pqs = rng.uniform(0.5, 2.0, K).astype(np.float32)
    codes, scales, ts = random_nvfp4(N, K, rng, lib=lib)
    A = random_bf16((r, K), 0.01 * 8, rng)
    B = random_bf16((N, r), 0.01 * 8, rng)
    return x, pqs, codes, scales, ts, A, B


def pin_linear_vs_numpy(lib):
    rng = np.random.default_rng(16)
    for (M, K, N, r, alpha, strength) in [(5, 48, 7, 3, 1.5, 0.7), (9, 64, 33, 16, 16.0, 1.0), (4, 32, 6, 2, 8.0, -0.5)]:
        x, pqs, codes, scales, ts, A, B = _lora_case(rng, M, K, N, r, lib)
        got = oracle.linear(x, pqs, codes, scales, ts, A, B, r, alpha, strength, lib=lib)
        xv, Av, Bv = bf16_values(x), bf16_values(A), bf16_values(B)
        Wd = decode_independent(codes, scales, ts)
        want = (xv * pqs.astype(np.float64)) @ Wd.T + strength * alpha / r * ((xv @ Av.T) @ Bv.T)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
        # adapter absent: base only
        got0 = oracle.linear(x, pqs, codes, scales, ts, lib=lib)
        np.testing.assert_allclose(got0, (xv * pqs.astype(np.float64)) @ Wd.T, rtol=1e-12, atol=1e-14)


def pin_linear_exact_fractions(lib):
    # tiny shapes with few-bit dyadic inputs: every fp64 operation is exact, so the oracle must
    # equal the rational result bit for bit
    rng = np.random.default_rng(17)
    M, K, N, r = 3, 32, 4, 2
    x = bits_of(rng.integers(-8, 9, (M, K)) / 4.0)
    pqs = (2.0 ** rng.integers(-1, 2, K)).astype(np.float32)
    codes = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x3C, 0x40, 0x44], np.uint8), (N, K // 16))
    ts = 0.25
    A = bits_of(rng.integers(-4, 5, (r, K)) / 8.0)
    B = bits_of(rng.integers(-4, 5, (N, r)) / 8.0)
    alpha, strength = 3.0, 0.5
    got = oracle.linear(x, pqs, codes, scales, ts, A, B, r, alpha, strength, lib=lib)
    xv, Av, Bv = bf16_values(x), bf16_values(A), bf16_values(B)
    Wd = decode_independent(codes, scales, ts)
    c = Fraction(strength) * Fraction(alpha) / r
    for m in range(M):
        t = [sum(Fraction(xv[m, k]) * Fraction(Av[j, k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            base = sum(Fraction(xv[m, k]) * Fraction(float(pqs[k])) * Fraction(Wd[n, k]) for k in range(K))
            delta = sum(t[j] * Fraction(Bv[n, j]) for j in range(r))
            assert Fraction(got[m, n]) == base + c * delta, (m, n)


def pin_identity_activation(lib):
    # x = I (S = K), pqs = 1, no adapter: y[m][n] = ts * Wq[n][m], one product per output
    rng = np.random.default_rng(18)
    K, N = 32, 5
    x = bits_of(np.eye(K))
    codes, scales, ts = random_nvfp4(N, K, rng, lib=lib)
    got = oracle.linear(x, None, codes, scales, ts, lib=lib)
    assert np.array_equal(got, decode_independent(codes, scales, ts).T)


def pin_rank1_closed_form(lib):
    rng = np.random.default_rng(19)
    K, N = 48, 6
    codes, scales, ts = random_nvfp4(N, K, rng, lib=lib)
    Wd = decode_independent(codes, scales, ts)
    pqs = (2.0 ** rng.integers(-1, 2, K)).astype(np.float32)
    k = 37
    x = bits_of(np.eye(K)[k:k + 1])
    a = rng.integers(-4, 5, K) / 8.0
    b = rng.integers(-4, 5, N) / 8.0
    # rank 1, alpha 2, strength 0.5: y[n] = Wd[n,k] pqs[k] + 0.5 * 2 * a_k b_n
    got = oracle.linear(x, pqs, codes, scales, ts, bits_of(a[None, :]), bits_of(b[:, None]), 1, 2.0, 0.5, lib=lib)
    assert np.array_equal(got[0], Wd[:, k] * float(pqs[k]) + 1.0 * a[k] * b)
    # rank 4, alpha 1: the factor alpha / rank = 1/4 must be applied
    A4 = rng.integers(-4, 5, (4, K)) / 8.0
    B4 = rng.integers(-4, 5, (N, 4)) / 8.0
    got4 = oracle.linear(x, pqs, codes, scales, ts, bits_of(A4), bits_of(B4), 4, 1.0, 1.0, lib=lib)
    assert np.array_equal(got4[0], Wd[:, k] * float(pqs[k]) + 0.25 * (B4 @ A4[:, k]))


def pin_prescale_base_only(lib):
    # zero weights: the output is the pure LoRA term and does not depend on pqs (original x);
    # no adapter: the output does not depend on A or B
    rng = np.random.default_rng(20)
    M, K, N, r = 4, 32, 5, 3
    x, pqs, codes, scales, ts, A, B = _lora_case(rng, M, K, N, r, lib)
    zc = np.zeros_like(codes)
    y1 = oracle.linear(x, pqs, zc, scales, ts, A, B, r, 2.0, 1.0, lib=lib)
    y2 = oracle.linear(x, pqs * 2, zc, scales, ts, A, B, r, 2.0, 1.0, lib=lib)
    assert np.array_equal(y1, y2)
    xv, Av, Bv = bf16_values(x), bf16_values(A), bf16_values(B)
    np.testing.assert_allclose(y1, 2.0 / r * (xv @ Av.T) @ Bv.T, rtol=1e-12, atol=1e-15)
    assert np.any(y1 != 0)


def pin_strength_linearity(lib):
    rng = np.random.default_rng(21)
    x, pqs, codes, scales, ts, A, B = _lora_case(rng, 6, 64, 9, 4, lib)
    y = {s: oracle.linear(x, pqs, codes, scales, ts, A, B, 4, 4.0, s, lib=lib) for s in (0.0, 0.5, 1.0)}
    np.testing.assert_allclose(y[1.0] - y[0.0], 2 * (y[0.5] - y[0.0]), rtol=1e-9, atol=1e-14)
    assert np.array_equal(y[0.0], oracle.linear(x, pqs, codes, scales, ts, lib=lib))


def pin_w4a4_base(lib):
    rng = np.random.default_rng(22)
    M, K, N, r = 5, 64, 7, 4
    x, pqs, codes, scales, ts, A, B = _lora_case(rng, M, K, N, r, lib)
    ac, asc, ts_a = oracle.w4a4_activation(x, pqs, lib=lib)
    # the activation the quantizer sees is f32_rne(x * pqs), compared with torch's fp32 product
    v = oracle.prescale_f32(x, pqs, lib=lib)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(v, (xt * torch.from_numpy(pqs)).numpy())
    want_c, want_s, want_ts = quantize_exact(v)
    assert np.array_equal(ac, want_c) and np.array_equal(asc, want_s) and ts_a == want_ts
    got = oracle.linear(x, pqs, codes, scales, ts, A, B, r, 4.0, 1.0, act_codes=ac, act_scales=asc, ts_a=ts_a, lib=lib)
    Xd = decode_independent(ac, asc, ts_a)
    Wd = decode_independent(codes, scales, ts)
    xv, Av, Bv = bf16_values(x), bf16_values(A), bf16_values(B)
    np.testing.assert_allclose(got, Xd @ Wd.T + (xv @ Av.T) @ Bv.T, rtol=1e-12, atol=1e-14)


def pin_swiglu(lib):
    rng = np.random.default_rng(23)
    y = rng.standard_normal((3, 10)) * 4
    got = oracle.swiglu(y, lib=lib)
    g, u = torch.from_numpy(y[:, :5]), torch.from_numpy(y[:, 5:])
    np.testing.assert_allclose(got, (torch.nn.functional.silu(g) * u).numpy(), rtol=1e-14, atol=1e-300)
    z = rng.standard_normal(8) * 5
    ones = np.ones(8)
    sp = oracle.swiglu(np.concatenate([z, ones])[None, :], lib=lib)[0]
    sn = oracle.swiglu(np.concatenate([-z, ones])[None, :], lib=lib)[0]
    np.testing.assert_allclose(sp - sn, z, rtol=1e-14, atol=1e-14)
    assert oracle.swiglu(np.array([[0.0, 3.0]]), lib=lib)[0, 0] == 0.0


def _qkv_case(rng, M, heads):
    """A fused-QKV-shaped output with `heads` heads of 128 in q and in k, and as many columns of v."""
    qw = 128 * heads
    y = rng.standard_normal((M, 3 * qw)) * rng.uniform(0.5, 3.0, size=(M, 1))
    gq, gk = rng.uniform(0.5, 1.5, qw), rng.uniform(0.5, 1.5, qw)
    return y, qw, gq.astype(np.float32), gk.astype(np.float32)


def pin_qk_rmsnorm_vs_linalg(lib):
    """RMSNorm scope and weights: with no rotation and eps = 0 every 128-column head of q and k is
    y * sqrt(128) / ||y||_2 * gamma (numpy's norm); v is returned bit for bit; with eps > 0 a
    constant head c gives c / sqrt(c^2 + eps) * gamma."""
    rng = np.random.default_rng(29)
    M = 5
    y, qw, gq, gk = _qkv_case(rng, M, 2)
    for rot in (0, 96):
        half = rot // 2
        cos, sin = np.ones((M, half), np.float32), np.zeros((M, half), np.float32)
        got = oracle.qk_norm_rope(y, qw, rot, 0.0, gq, gk, cos, sin, lib=lib)
        assert np.array_equal(got[:, 2 * qw:], y[:, 2 * qw:])
        for c0 in range(0, 2 * qw, 128):
            yh = y[:, c0:c0 + 128]
            g = (gq[c0:c0 + 128] if c0 < qw else gk[c0 - qw:c0 - qw + 128]).astype(np.float64)
            want = yh * np.sqrt(128.0) / np.linalg.norm(yh, axis=1, keepdims=True) * g
            np.testing.assert_allclose(got[:, c0:c0 + 128], want, rtol=1e-13, atol=0)
    c, eps = 0.75, 0.4375
    yc = np.full((1, 3 * 128), c)
    g1 = np.full(128, 2.0, np.float32)
    got = oracle.qk_norm_rope(yc, 128, 0, eps, g1, g1, np.ones((1, 0)), np.zeros((1, 0)), lib=lib)
    np.testing.assert_allclose(got[0, :256], c / np.sqrt(c * c + eps) * 2.0, rtol=1e-15)


def pin_rope_complex_rotation(lib):
    """Split-half rotation: dims (i, i + rot/2) of a normalized head form the complex number
    u_i + j u_{i+rot/2}, multiplied by exp(j theta_i) with theta_i the table's angle (numpy complex
    arithmetic); dims rot..127 pass through. Checked for rot = 96 (the pages' 96 of 128), 128, 32."""
    rng = np.random.default_rng(31)
    M = 4
    y, qw, gq, gk = _qkv_case(rng, M, 2)
    for rot in (96, 128, 32):
        half = rot // 2
        theta = rng.uniform(-np.pi, np.pi, (M, half))
        cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
        flat = oracle.qk_norm_rope(y, qw, rot, 1e-6, gq, gk, np.ones((M, half)), np.zeros((M, half)), lib=lib)
        got = oracle.qk_norm_rope(y, qw, rot, 1e-6, gq, gk, cos, sin, lib=lib)
        rot_c = cos.astype(np.float64) + 1j * sin.astype(np.float64)
        for c0 in range(0, 2 * qw, 128):
            u = flat[:, c0:c0 + 128]
            z = (u[:, :half] + 1j * u[:, half:rot]) * rot_c
            np.testing.assert_allclose(got[:, c0:c0 + half], z.real, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(got[:, c0 + half:c0 + rot], z.imag, rtol=1e-12, atol=1e-12)
            assert np.array_equal(got[:, c0 + rot:c0 + 128], u[:, rot:])
        assert np.array_equal(got[:, 2 * qw:], y[:, 2 * qw:])


def pin_rope_sections_complex_rotation(lib):
    """Rotation within axis sections: with sections of widths w_j at dims [o_j, o_j + w_j), dims
    (o_j + i, o_j + i + w_j/2) of a normalized head form u + j v, multiplied by exp(j theta) with
    theta from table column o_j/2 + i (numpy complex arithmetic); three sections of 32 is the per-axis
    reading of the three-axis rotary, one section of rot_dim must equal the call without sections bit
    for bit, and sections of unequal widths are checked too."""
    rng = np.random.default_rng(37)
    M = 4
    y, qw, gq, gk = _qkv_case(rng, M, 2)
    for sections in ((32, 32, 32), (16, 48, 32), (8, 4, 20), (96,), (128,)):
        rot = sum(sections)
        half = rot // 2
        theta = rng.uniform(-np.pi, np.pi, (M, half))
        cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
        flat = oracle.qk_norm_rope(y, qw, rot, 1e-6, gq, gk, np.ones((M, half)), np.zeros((M, half)), lib=lib)
        got = oracle.qk_norm_rope(y, qw, rot, 1e-6, gq, gk, cos, sin, sections=sections, lib=lib)
        rot_c = cos.astype(np.float64) + 1j * sin.astype(np.float64)
        for c0 in range(0, 2 * qw, 128):
            u = flat[:, c0:c0 + 128]
            o = 0
            for w in sections:
                h = w // 2
                z = (u[:, o:o + h] + 1j * u[:, o + h:o + w]) * rot_c[:, o // 2:o // 2 + h]
                np.testing.assert_allclose(got[:, c0 + o:c0 + o + h], z.real, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(got[:, c0 + o + h:c0 + o + w], z.imag, rtol=1e-12, atol=1e-12)
                o += w
            assert np.array_equal(got[:, c0 + rot:c0 + 128], u[:, rot:])
        assert np.array_equal(got[:, 2 * qw:], y[:, 2 * qw:])
        if len(sections) == 1:
            plain = oracle.qk_norm_rope(y, qw, rot, 1e-6, gq, gk, cos, sin, lib=lib)
            assert np.array_equal(plain, got)


def pin_merge_reproduces_dynamic_linear(lib):
    """The merged fp32 weight applied to x (*) pqs reproduces the dynamic linear (itself pinned to
    numpy and exact fractions) up to m's one fp32 rounding, for pqs != 1, alpha != rank, negative
    strength and N != K; and with no adapter m is Wd rounded to fp32."""
    rng = np.random.default_rng(33)
    for (M, K, N, r, alpha, strength) in [(6, 48, 7, 3, 1.5, 0.7), (5, 64, 33, 16, 16.0, 1.0), (4, 32, 6, 2, 8.0, -1.5)]:
        x, pqs, codes, scales, ts, A, B = _lora_case(rng, M, K, N, r, lib)
        m = oracle.merge_lora(codes, scales, ts, A, B, r, alpha, strength, pqs, lib=lib)
        assert m.dtype == np.float32 and m.shape == (N, K)
        xs = bf16_values(x) * pqs.astype(np.float64)
        got = xs @ m.astype(np.float64).T
        want = oracle.linear(x, pqs, codes, scales, ts, A, B, r, alpha, strength, lib=lib)
        err = np.abs(got - want).max() / np.abs(want).max()
        assert err < 1e-6, err
        m0 = oracle.merge_lora(codes, scales, ts, pqs=pqs, lib=lib)
        assert np.array_equal(m0, decode_independent(codes, scales, ts).astype(np.float32))


def pin_merge_rank1_exact(lib):
    """Rank 1 with dyadic a, b and power-of-two pqs: every fp64 step is exact, so
    m[n][k] = f32(Wd[n][k] + c a_k b_n / pqs_k) with c = strength alpha / rank, element for element."""
    rng = np.random.default_rng(34)
    N, K = 5, 32
    codes, scales, ts = random_nvfp4(N, K, rng, lib=lib)
    a = rng.integers(-4, 5, K) / 8.0
    b = rng.integers(-4, 5, N) / 8.0
    pqs = (2.0 ** rng.integers(-2, 3, K)).astype(np.float32)
    m = oracle.merge_lora(codes, scales, ts, bits_of(a[None, :]), bits_of(b[:, None]), 1, 2.0, 0.75, pqs, lib=lib)
    want = decode_independent(codes, scales, ts) + 1.5 * np.outer(b, a) / pqs.astype(np.float64)
    assert np.array_equal(m, want.astype(np.float32))


def _adaln_case(rng, blocks=2, S=5, E=12, rb=3, rl=2, rows=7):
    u = rng.standard_normal((S, rb)).astype(np.float32)
    emb = rng.uniform(-4, 4, (S, E)).astype(np.float32)
    A = random_bf16((blocks, rl, E), 0.5, rng)
    Wp = random_bf16((blocks, rows, rb), 0.5, rng)
    B = random_bf16((blocks, rows, rl), 0.5, rng)
    bias = rng.standard_normal((blocks, rows)).astype(np.float32)
    return u, emb, A, Wp, B, bias


def pin_adaln_fold_identity(lib):
    """The folded form [W_p | B] [u ; c A silu(e)] + bias, evaluated through the table at the sample
    points, equals the unfolded W_p u + bias + c B (A silu(e)) computed with numpy, block by block."""
    rng = np.random.default_rng(35)
    u, emb, A, Wp, B, bias = _adaln_case(rng)
    blocks, rows, rb = Wp.shape
    S, c = u.shape[0], -0.75
    table = oracle.adaln_table(u, emb, A, c, lib=lib)
    M = np.concatenate([Wp, B], axis=2)
    ts = (np.arange(S) / (S - 1)).astype(np.float32)
    got = oracle.adaln_apply(M, bias, table, ts, lib=lib)
    e = emb.astype(np.float64)
    silu = e / (1.0 + np.exp(-e))
    for b in range(blocks):
        Av, Wv, Bv = bf16_values(A[b]), bf16_values(Wp[b]), bf16_values(B[b])
        want = (Wv @ u.astype(np.float64).T + bias[b].astype(np.float64)[:, None] + c * Bv @ (Av @ silu.T)).T
        np.testing.assert_allclose(got[:, b, :], want, rtol=1e-12, atol=1e-12)
    # no adapter term: the rank-8 base curve alone
    t0 = oracle.adaln_table(u, emb, A, 0.0, lib=lib)
    got0 = oracle.adaln_apply(M, None, t0, ts, lib=lib)
    np.testing.assert_allclose(got0[:, 0, :], (bf16_values(Wp[0]) @ u.astype(np.float64).T).T, rtol=1e-13, atol=1e-13)


def pin_adaln_silu_points(lib):
    """silu at points with closed forms: silu(0) = 0 and silu(ln 3) = 0.75 ln 3 (sigmoid(ln 3) = 3/4),
    through a one-hot A row."""
    E = 4
    emb = np.array([[0.0, 0.0, 0.0, 0.0], [np.log(3.0)] * 4], np.float32)
    u = np.zeros((2, 1), np.float32)
    A = bits_of(np.array([[[1.0, 0.0, 0.0, 0.0]]]))
    table = oracle.adaln_table(u, emb, A, 2.0, lib=lib)
    z = float(np.float32(np.log(3.0)))
    assert table[0, 0, 1] == 0.0
    np.testing.assert_allclose(table[0, 1, 1], 2.0 * z / (1.0 + np.exp(-z)), rtol=1e-15)
    np.testing.assert_allclose(table[0, 1, 1], 2.0 * 0.75 * np.log(3.0), rtol=1e-7)
    assert table.shape == (1, 2, 2) and E == 4


def pin_adaln_interpolation(lib):
    """Between samples the curve is the affine blend of its neighbours; t = 0 and t = 1 give the first
    and last samples exactly; t outside [0, 1] is clamped."""
    rng = np.random.default_rng(36)
    blocks, S, R, rows = 2, 9, 4, 5
    table = rng.standard_normal((blocks, S, R))
    M = random_bf16((blocks, rows, R), 1.0, rng)
    at = lambda t: oracle.adaln_apply(M, None, table, np.array([t], np.float32), lib=lib)[0]
    exact = lambda i: np.einsum("brq,bq->br", bf16_values(M), table[:, i, :])
    np.testing.assert_allclose(at(0.0), exact(0), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(at(1.0), exact(S - 1), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(at(-0.5), exact(0), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(at(2.0), exact(S - 1), rtol=1e-14, atol=1e-14)
    for i, th in ((2, 0.25), (5, 0.5), (7, 0.75)):
        t = (i + th) / (S - 1)   # exact in fp32 for S - 1 = 8
        np.testing.assert_allclose(at(t), (1 - th) * exact(i) + th * exact(i + 1), rtol=1e-12, atol=1e-12)


def pin_bf16_rne_vs_torch(lib):
    """The oracle's fp32 -> bf16 rounding against torch's conversion (round to nearest even) on random
    magnitudes and on constructed ties of both parities."""
    rng = np.random.default_rng(37)
    vals = (rng.standard_normal(4000) * 10.0 ** rng.integers(-20, 20, 4000)).astype(np.float32)
    hi = rng.integers(0, 0x7F7F, 400, dtype=np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)  # exactly halfway: the even neighbour must win
    near = (hi | 0x7FFF).view(np.float32)
    allv = np.concatenate([vals, ties, near, -ties, np.array([0.0, -0.0, 1.0, 3.0e38], np.float32)])
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v), lib=lib) for v in allv], np.uint16)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def pin_mirror_exact_cases(lib):
    """Mirror mode where every declared rounding is exact: identity activation with power-of-two pqs
    and ts gives bf16(ts Wq pqs) bit for bit; zero weight codes with a dyadic rank-1 adapter on a
    one-hot row give bf16(c a_k b_n) bit for bit."""
    rng = np.random.default_rng(38)
    K, N = 48, 6
    codes, scales, _ = random_nvfp4(N, K, rng, lib=lib)
    ts = 0.125
    pqs = (2.0 ** rng.integers(-1, 2, K)).astype(np.float32)
    x = bits_of(np.eye(K))
    got = oracle.linear_mirror(x, pqs, codes, scales, ts, lib=lib)
    want = bits_of(decode_independent(codes, scales, ts).T * pqs.astype(np.float64)[:, None])
    assert np.array_equal(got, want)
    k = 11
    pqs[k] = 2.0  # the adapter branch must see x itself, not x * pqs
    a = rng.integers(-4, 5, K) / 8.0
    b = rng.integers(-4, 5, N) / 8.0
    zc = np.zeros_like(codes)
    got = oracle.linear_mirror(bits_of(np.eye(K)[k:k + 1]), pqs, zc, scales, 0.25, bits_of(a[None, :]),
                               bits_of(b[:, None]), 1, 2.0, 0.25, lib=lib)
    assert np.array_equal(got[0], bits_of(0.5 * a[k] * b))


def pin_mirror_within_bar(lib):
    """On random inputs the mirror differs from the exact oracle only by its roundings: within the
    parity bar, and above zero (the roundings are really applied)."""
    rng = np.random.default_rng(39)
    x, pqs, codes, scales, ts, A, B = _lora_case(rng, 7, 96, 40, 8, lib)
    ref = oracle.linear(x, pqs, codes, scales, ts, A, B, 8, 4.0, 0.75, lib=lib)
    got = bf16_values(oracle.linear_mirror(x, pqs, codes, scales, ts, A, B, 8, 4.0, 0.75, lib=lib))
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-5 < err < 4e-3, err


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
