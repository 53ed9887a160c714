"""fp64 CPU oracle for the W4 (NVFP4) + dynamic LoRA linear -- TEST INFRASTRUCTURE ONLY.

The arithmetic lives in ``oracle.cpp`` (plain C++, fp64, scalar loops); this module compiles it with
g++ into ``liboracle.so`` and marshals numpy arrays through ctypes. It shares no code with the HIP
library in ``bit_linear_dynamic_amd`` and never imports it. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may use it.

Method (FL2VA Turbo page, section "Implementation"):
    y = NVFP4_base(x * pre_quant_scale) + strength * (alpha / rank) * B(A x)
with the LoRA branch on the original bf16 activation. W4A4 variant: the base path's activation is
itself quantized to NVFP4 per call (MiniMax-H3 Ultra Fast, "Kernel path"). Gate/up output feeds
SiLU(gate) * up (same page, "Active optimization stack", MLP row). For comparison only, the merged
route (the LoRA update merged into the weight before quantizing: MiniMax-H3 Turbo CMF card, "What the
conversion did") is ``merge_lora`` + ``quantize_nvfp4``. The AdaLN modulation curve of the same card
(the adapter folded into a rank-24 table by the same K-concatenation) is ``adaln_table`` +
``adaln_apply``.

Every function here is pinned by tests/test_oracle_*.py (pins in tests/pins.py) against things other
than itself: the format's published code tables and torch's float8 conversion, exact rational
arithmetic on small shapes, numpy's fp64 matmul, norms and complex arithmetic, rank-1 closed forms,
the unfolded form of every folded formula, and identities. Nothing in the oracle is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.cpp")
_LIB = os.path.join(_DIR, "liboracle.so")

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c++17",
           "-Wall", "-Wextra"]


def build(out: str = _LIB, src: str = _SRC) -> str:
    """Compile the oracle with g++ (never hipcc). ``src`` other than oracle.cpp is for the tests'
    deliberately broken copies only."""
    tmp = out + ".tmp"
    cmd = ["g++", *_CFLAGS, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def _declare(lib):
    i64, f64, f32, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_int
    vp = ctypes.c_void_p
    lib.orc_e2m1_value.argtypes, lib.orc_e2m1_value.restype = [i32], f64
    lib.orc_e4m3_value.argtypes, lib.orc_e4m3_value.restype = [i32], f64
    lib.orc_e2m1_encode.argtypes, lib.orc_e2m1_encode.restype = [f64], i32
    lib.orc_e4m3_encode_nonneg.argtypes, lib.orc_e4m3_encode_nonneg.restype = [f64], i32
    lib.orc_quantize_nvfp4.argtypes = [vp, i64, i64, vp, vp, ctypes.POINTER(f32)]
    lib.orc_quantize_nvfp4.restype = i32
    lib.orc_prescale_f32.argtypes, lib.orc_prescale_f32.restype = [vp, vp, i64, i64, vp], None
    lib.orc_dequant.argtypes, lib.orc_dequant.restype = [vp, vp, f64, i64, i64, vp], None
    lib.orc_linear.argtypes = [vp, i64, i64, vp, vp, vp, f32, i64, vp, vp, i64, f64, f64, vp, vp, f32, vp]
    lib.orc_linear.restype = i32
    lib.orc_swiglu.argtypes, lib.orc_swiglu.restype = [vp, i64, i64, vp], None
    lib.orc_qk_norm_rope.argtypes = [vp, i64, i64, i64, i32, f64, vp, vp, vp, vp, vp, i32, vp]
    lib.orc_qk_norm_rope.restype = None
    lib.orc_merge_lora.argtypes = [vp, vp, f32, i64, i64, vp, vp, i64, f64, f64, vp, vp]
    lib.orc_merge_lora.restype = i32
    lib.orc_adaln_table.argtypes = [vp, vp, vp, f64, i64, i64, i64, i64, i64, vp]
    lib.orc_adaln_table.restype = None
    lib.orc_adaln_apply.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.orc_adaln_apply.restype = None
    lib.orc_f32_to_bf16.argtypes, lib.orc_f32_to_bf16.restype = [f32], ctypes.c_uint16
    lib.orc_linear_mirror.argtypes = [vp, i64, i64, vp, vp, vp, f32, i64, vp, vp, i64, f64, f64, vp]
    lib.orc_linear_mirror.restype = i32
    lib.orc_num_threads.argtypes, lib.orc_num_threads.restype = [], i32
    return lib


def load(path: str | None = None):
    """Load liboracle.so, building it first if it is missing or older than its source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------------------------
# numpy-facing wrappers (bf16 arrays are passed as their uint16 bit patterns)
# --------------------------------------------------------------------------------------------

def e2m1_value(code: int, lib=None) -> float:
    return (lib or load()).orc_e2m1_value(int(code))


def e4m3_value(code: int, lib=None) -> float:
    return (lib or load()).orc_e4m3_value(int(code))


def e2m1_encode(q: float, lib=None) -> int:
    return (lib or load()).orc_e2m1_encode(float(q))


def e4m3_encode(v: float, lib=None) -> int:
    return (lib or load()).orc_e4m3_encode_nonneg(float(v))


def quantize_nvfp4(v: np.ndarray, lib=None):
    """fp32 [rows][K] -> (codes u8 [rows][K/2], scales u8 [rows][K/16], ts float)."""
    v = _c(v, np.float32)
    rows, K = v.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    ts = ctypes.c_float(0.0)
    rc = (lib or load()).orc_quantize_nvfp4(_ptr(v), rows, K, _ptr(codes), _ptr(scales), ctypes.byref(ts))
    if rc != 0:
        raise ValueError("orc_quantize_nvfp4: K must be a multiple of 16 and inputs finite")
    return codes, scales, float(ts.value)


def prescale_f32(x_bits: np.ndarray, pqs: np.ndarray | None, lib=None) -> np.ndarray:
    """bf16 bits [rows][K], fp32 [K] -> fp32 [rows][K] = f32_rne(x * pqs)."""
    x_bits = _c(x_bits, np.uint16)
    rows, K = x_bits.shape
    out = np.empty((rows, K), np.float32)
    pqs = _c(pqs, np.float32)  # kept alive by the local name across the call
    (lib or load()).orc_prescale_f32(_ptr(x_bits), _ptr(pqs), rows, K, _ptr(out))
    return out


def dequant(codes: np.ndarray, scales: np.ndarray, ts: float = 1.0, lib=None) -> np.ndarray:
    """(codes [rows][K/2], scales [rows][K/16]) -> fp64 [rows][K] = E2M1 * E4M3 * ts."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, K), np.float64)
    (lib or load()).orc_dequant(_ptr(codes), _ptr(scales), float(ts), rows, K, _ptr(out))
    return out


def linear(x_bits, pqs, codes, scales, ts, A_bits=None, B_bits=None, rank=0, alpha=0.0, strength=0.0,
           act_codes=None, act_scales=None, ts_a=1.0, lib=None) -> np.ndarray:
    """fp64 y [M][N] = base + strength*alpha/rank * B(A x)  (see oracle.cpp, orc_linear)."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    codes = _c(codes, np.uint8)
    N = codes.shape[0]
    y = np.empty((M, N), np.float64)
    # converted copies must stay referenced until the call returns (a raw pointer keeps nothing alive)
    pqs, scales = _c(pqs, np.float32), _c(scales, np.uint8)
    A_bits, B_bits = _c(A_bits, np.uint16), _c(B_bits, np.uint16)
    act_codes, act_scales = _c(act_codes, np.uint8), _c(act_scales, np.uint8)
    rc = (lib or load()).orc_linear(
        _ptr(x_bits), M, K, _ptr(pqs), _ptr(codes), _ptr(scales), float(ts), N,
        _ptr(A_bits), _ptr(B_bits), int(rank), float(alpha), float(strength),
        _ptr(act_codes), _ptr(act_scales), float(ts_a), _ptr(y))
    if rc != 0:
        raise ValueError("orc_linear: bad shape")
    return y


def swiglu(y: np.ndarray, lib=None) -> np.ndarray:
    """fp64 [M][2F] -> fp64 [M][F] = SiLU(gate) * up, gate = y[:, :F], up = y[:, F:]."""
    y = _c(y, np.float64)
    M, N2 = y.shape
    h = np.empty((M, N2 // 2), np.float64)
    (lib or load()).orc_swiglu(_ptr(y), M, N2 // 2, _ptr(h))
    return h


def qk_norm_rope(y: np.ndarray, q_width: int, rot_dim: int, eps: float, gamma_q, gamma_k, cos, sin,
                 sections=None, lib=None) -> np.ndarray:
    """fp64 [M][N] fused-QKV output -> per-head RMSNorm of q and k, then rotation of their first
    rot_dim dims with the [M][rot_dim/2] angle tables, in split halves within each section of
    `sections` (consecutive widths summing to rot_dim; None: one section of rot_dim); v unchanged
    (see oracle.cpp)."""
    y = _c(y, np.float64)
    M, N = y.shape
    if q_width % 128 or 2 * q_width > N or rot_dim % 2 or not 0 <= rot_dim <= 128:
        raise ValueError("qk_norm_rope: bad q_width or rot_dim")
    sec = None
    if sections is not None:
        sec = _c(np.asarray(sections, np.int32), np.int32)
        if sec.sum() != rot_dim or np.any(sec <= 0) or np.any(sec % 2):
            raise ValueError("qk_norm_rope: sections must be positive, even and sum to rot_dim")
    half = rot_dim // 2
    cos = _c(np.asarray(cos, np.float32).reshape(M, half), np.float32)
    sin = _c(np.asarray(sin, np.float32).reshape(M, half), np.float32)
    out = np.empty_like(y)
    gamma_q, gamma_k = _c(gamma_q, np.float32), _c(gamma_k, np.float32)
    (lib or load()).orc_qk_norm_rope(_ptr(y), M, N, int(q_width), int(rot_dim), float(eps),
                                     _ptr(gamma_q), _ptr(gamma_k), _ptr(cos), _ptr(sin),
                                     None if sec is None else _ptr(sec), 0 if sec is None else len(sec),
                                     _ptr(out))
    return out


def merge_lora(codes, scales, ts, A_bits=None, B_bits=None, rank=0, alpha=0.0, strength=0.0, pqs=None,
               lib=None) -> np.ndarray:
    """fp32 [N][K] merged weight m = f32(Wd + c * (B A) / pqs) (see oracle.cpp, orc_merge_lora); feed it
    to quantize_nvfp4 for the merged NVFP4 weight."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    m = np.empty((N, K), np.float32)
    A_bits, B_bits, pqs = _c(A_bits, np.uint16), _c(B_bits, np.uint16), _c(pqs, np.float32)
    rc = (lib or load()).orc_merge_lora(_ptr(codes), _ptr(scales), float(ts), N, K, _ptr(A_bits), _ptr(B_bits),
                                        int(rank), float(alpha), float(strength), _ptr(pqs), _ptr(m))
    if rc != 0:
        raise ValueError("orc_merge_lora: bad shape")
    return m


def merged_nvfp4(codes, scales, ts, A_bits=None, B_bits=None, rank=0, alpha=0.0, strength=0.0, pqs=None,
                 lib=None):
    """The merged route end to end: (codes, scales, ts) of NVFP4(merge_lora(...))."""
    return quantize_nvfp4(merge_lora(codes, scales, ts, A_bits, B_bits, rank, alpha, strength, pqs, lib=lib),
                          lib=lib)


def adaln_table(u, emb, A_bits, c, lib=None) -> np.ndarray:
    """fp64 [blocks][S][rb + rl] = [u ; c * A_b silu(e)] per sample (see oracle.cpp, orc_adaln_table).
    u: [S][rb]; emb: [S][E]; A_bits: bf16 bits [blocks][rl][E]."""
    u, emb, A_bits = _c(u, np.float32), _c(emb, np.float32), _c(A_bits, np.uint16)
    S, rb = u.shape
    blocks, rl, E = A_bits.shape
    if emb.shape != (S, E):
        raise ValueError("adaln_table: emb must be [S][E]")
    out = np.empty((blocks, S, rb + rl), np.float64)
    (lib or load()).orc_adaln_table(_ptr(u), _ptr(emb), _ptr(A_bits), float(c), blocks, S, E, rb, rl, _ptr(out))
    return out


def adaln_apply(M_bits, bias, table, t, lib=None) -> np.ndarray:
    """fp64 [T][blocks][rows] = bias + M v(t), v interpolated from the table (orc_adaln_apply).
    M_bits: bf16 bits [blocks][rows][R]; bias: [blocks][rows] or None; table: [blocks][S][R]; t: [T]."""
    M_bits, bias = _c(M_bits, np.uint16), _c(bias, np.float32)
    table, t = _c(table, np.float64), _c(np.atleast_1d(t), np.float32)
    blocks, rows, R = M_bits.shape
    S = table.shape[1]
    if table.shape != (blocks, S, R) or S < 2:
        raise ValueError("adaln_apply: table must be [blocks][S >= 2][R]")
    out = np.empty((t.shape[0], blocks, rows), np.float64)
    (lib or load()).orc_adaln_apply(_ptr(M_bits), _ptr(bias), _ptr(table), _ptr(t), t.shape[0], blocks, rows, S, R,
                                    _ptr(out))
    return out


def f32_to_bf16(v: float, lib=None) -> int:
    """bf16 bit pattern of an fp32 value, round to nearest even."""
    return int((lib or load()).orc_f32_to_bf16(float(v)))


def linear_mirror(x_bits, pqs, codes, scales, ts, A_bits=None, B_bits=None, rank=0, alpha=0.0, strength=0.0,
                  lib=None) -> np.ndarray:
    """Diagnostic: bf16 bits [M][N] of the linear with the GPU path's declared rounding points (see
    oracle.cpp, orc_linear_mirror)."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    codes = _c(codes, np.uint8)
    N = codes.shape[0]
    y = np.empty((M, N), np.uint16)
    pqs, scales = _c(pqs, np.float32), _c(scales, np.uint8)
    A_bits, B_bits = _c(A_bits, np.uint16), _c(B_bits, np.uint16)
    rc = (lib or load()).orc_linear_mirror(_ptr(x_bits), M, K, _ptr(pqs), _ptr(codes), _ptr(scales), float(ts), N,
                                           _ptr(A_bits), _ptr(B_bits), int(rank), float(alpha), float(strength),
                                           _ptr(y))
    if rc != 0:
        raise ValueError("orc_linear_mirror: bad shape")
    return y


def num_threads(lib=None) -> int:
    return (lib or load()).orc_num_threads()


def nvfp4_weight_fixture(w: np.ndarray, lib=None):
    """Synthetic NVFP4 weight from an fp32 [N][K] array: the same quantizer with pqs = 1."""
    return quantize_nvfp4(np.asarray(w, np.float32), lib=lib)


def w4a4_activation(x_bits, pqs, lib=None):
    """The W4A4 base path's activation: NVFP4 of f32_rne(x * pqs) with a per-call global scale."""
    return quantize_nvfp4(prescale_f32(x_bits, pqs, lib=lib), lib=lib)
