"""The C-ABI library on a machine without a GPU: it loads, exports every entry point that
include/h3q.h declares, and rejects bad arguments before touching the device."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import bit_linear_dynamic_amd as h3q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "h3q.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(h3q_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(h3q.LIB_PATH):
        pytest.fail("libh3q.so is not built (run __graft_entry__.build())")
    return h3q.lib()


# The boundary's entry points by the names the projection's C ABI gives them (the pack, register,
# linear and SwiGLU calls, the flags entry point, the error text, and the test/diagnostic exports).
SCOPE_NAMES = ("h3q_pack_weight", "h3q_free_weight", "h3q_register_adapter", "h3q_unregister_adapter",
               "h3q_linear", "h3q_linear_swiglu", "h3q_linear_ex", "h3q_last_error", "h3q_debug_dequant",
               "h3q_debug_quantize_act", "h3q_weight_checksum")
PAGES = ("FL2VA Turbo", "MiniMax-H3 Ultra Fast", "MiniMax-H3 Turbo CMF card")


def test_header_declares_the_entry_points():
    names = declared_functions()
    missing = [n for n in SCOPE_NAMES if n not in names]
    assert not missing, missing
    assert "h3q_quantize_nvfp4" in names  # the quantizer's earlier name stays as an alias


def test_every_entry_point_cites_a_page_or_says_it_is_a_convention():
    """The comment block in front of each declaration (or of the group it belongs to) names the page
    and section that defines the call, or says that the call is a library convention."""
    text = open(HEADER).read()
    for name in declared_functions():
        m = re.search(r"(h3q_status|const char\*)\s+" + name + r"\s*\(", text)
        before = text[:m.start()]
        comment = before[before.rfind("/*"):]
        assert "*/" in comment, name
        ok = any(pg in comment for pg in PAGES) or "convention" in comment.lower() or "earlier name" in comment
        # the no-allocation variant names the callers it is for instead
        ok = ok or (name.endswith("_noalloc") and "cannot allocate" in comment)
        assert ok, f"{name}: its comment cites no page and does not say it is a library convention"


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", h3q.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (h3q_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def test_binding_covers_the_header():
    for n in declared_functions():
        if n in ("h3q_last_error",):
            continue
        assert hasattr(h3q, n), f"binding lacks {n}"


def _pack(lib, codes, scales, ts, N, K, flags=0):
    out = ctypes.c_void_p()
    rc = lib.h3q_pack_weight(None, codes, scales, ts, N, K, flags, ctypes.byref(out))
    return rc, out


def test_pack_rejects_bad_arguments(lib):
    N, K = 4, 32
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    cp, sp = ctypes.c_void_p(codes.ctypes.data), ctypes.c_void_p(scales.ctypes.data)
    assert _pack(lib, None, sp, 1.0, N, K)[0] == h3q.H3Q_E_ARG
    assert _pack(lib, cp, None, 1.0, N, K)[0] == h3q.H3Q_E_ARG
    assert lib.h3q_pack_weight(None, cp, sp, 1.0, N, K, 0, None) == h3q.H3Q_E_ARG
    assert _pack(lib, cp, sp, 1.0, N, K, flags=0x80)[0] == h3q.H3Q_E_ARG
    assert _pack(lib, cp, sp, 1.0, N, 24)[0] == h3q.H3Q_E_SHAPE        # K % 16 != 0
    assert _pack(lib, cp, sp, 1.0, 0, K)[0] == h3q.H3Q_E_SHAPE
    assert _pack(lib, cp, sp, 1.0, N, 0)[0] == h3q.H3Q_E_SHAPE
    assert _pack(lib, cp, sp, 1.0, 3, K, flags=h3q.H3Q_PACK_GATE_UP)[0] == h3q.H3Q_E_SHAPE
    assert _pack(lib, cp, sp, 1.0, (1 << 20) + 1, K)[0] == h3q.H3Q_E_SHAPE
    for bad_ts in (0.0, -1.0, math.nan, math.inf):
        assert _pack(lib, cp, sp, bad_ts, N, K)[0] == h3q.H3Q_E_ARG
    assert "tensor_scale" in h3q.last_error()
    for bad in (0x7F, 0x80, 0xB8, 0xFF):
        s2 = scales.copy()
        s2[2, 1] = bad
        assert _pack(lib, cp, ctypes.c_void_p(s2.ctypes.data), 1.0, N, K)[0] == h3q.H3Q_E_FORMAT
        assert "row 2 block 1" in h3q.last_error()


def test_pack_without_gpu_fails_cleanly(lib):
    N, K = 4, 32
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.full((N, K // 16), 0x38, np.uint8)
    rc, out = _pack(lib, ctypes.c_void_p(codes.ctypes.data), ctypes.c_void_p(scales.ctypes.data), 1.0, N, K)
    if rc == h3q.H3Q_OK:  # a gfx950 is present after all
        assert lib.h3q_free_weight(out) == h3q.H3Q_OK
    else:
        assert rc in (h3q.H3Q_E_HIP, h3q.H3Q_E_UNSUPPORTED), rc
        assert h3q.last_error()


def test_dead_handles_are_rejected(lib):
    bogus = ctypes.c_void_p(0x1234)
    assert lib.h3q_free_weight(bogus) == h3q.H3Q_E_ARG
    assert lib.h3q_free_weight(None) == h3q.H3Q_E_ARG
    A = np.zeros(32, np.uint16)
    ap = ctypes.c_void_p(A.ctypes.data)
    assert lib.h3q_register_adapter(bogus, 1, ap, ap, 1, 1.0) == h3q.H3Q_E_ARG
    assert lib.h3q_unregister_adapter(bogus, 1) == h3q.H3Q_E_ARG
    cnt = ctypes.c_int32()
    assert lib.h3q_list_adapters(bogus, None, 0, ctypes.byref(cnt)) == h3q.H3Q_E_ARG
    assert lib.h3q_linear(None, ap, 1, None, bogus, -1, 1.0, ap) == h3q.H3Q_E_ARG
    assert lib.h3q_linear_ex(None, ap, 1, None, bogus, -1, 1.0, 0, ap) == h3q.H3Q_E_ARG
    assert lib.h3q_debug_dequant(None, bogus, ap) == h3q.H3Q_E_ARG
    h = ctypes.c_uint64()
    assert lib.h3q_weight_checksum(None, bogus, ctypes.byref(h)) == h3q.H3Q_E_ARG
    assert lib.h3q_weight_info(bogus, None, None, None) == h3q.H3Q_E_ARG
    assert "live weight handle" in h3q.last_error()


def test_quantize_and_timing_argument_checks(lib):
    buf = np.zeros(64, np.uint8)
    p = ctypes.c_void_p(buf.ctypes.data)
    for fn in (lib.h3q_debug_quantize_act, lib.h3q_quantize_nvfp4):
        assert fn(None, None, 1, 16, None, p, p, p) == h3q.H3Q_E_ARG
        assert fn(None, p, 1, 24, None, p, p, p) == h3q.H3Q_E_SHAPE
        assert fn(None, p, -1, 16, None, p, p, p) == h3q.H3Q_E_SHAPE
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.h3q_timing_get(7, ctypes.byref(ms), ctypes.byref(n)) == h3q.H3Q_E_ARG
    assert lib.h3q_timing_enable(0) == h3q.H3Q_OK
    assert lib.h3q_timing_get(h3q.H3Q_KERNEL_GEMM, ctypes.byref(ms), ctypes.byref(n)) == h3q.H3Q_OK
    assert (ms.value, n.value) == (0.0, 0)


def test_library_does_not_link_the_oracle():
    out = subprocess.run(["nm", "-D", h3q.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "orc_" not in out
    deps = subprocess.run(["ldd", h3q.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def test_gemm_steps_inc_is_current():
    """The inline-asm K-steps the GEMM includes are exactly what their generator writes today."""
    import importlib.util
    csrc = os.path.join(ROOT, "bit_linear_dynamic_amd", "csrc")
    spec = importlib.util.spec_from_file_location("gen_gemm_steps", os.path.join(csrc, "gen_gemm_steps.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(csrc, "gemm_w4_steps.inc")) as f:
        assert f.read() == gen.render(), "gemm_w4_steps.inc is stale: run csrc/gen_gemm_steps.py"


def test_side_entry_points_reject_bad_arguments(lib):
    """The Q/K epilogue, merged route, producer fusion and AdaLN entry points validate before any
    device work (dead handle, null or misshaped arguments)."""
    bogus = ctypes.c_void_p(0x1234)
    buf = np.zeros(4096, np.uint8)
    p = ctypes.c_void_p(buf.ctypes.data)
    f = ctypes.c_void_p(np.zeros(64, np.float32).ctypes.data)
    assert lib.h3q_linear_qk_norm_rope(None, p, 1, None, bogus, -1, 0.0, 0, 256, 96, 1e-6, f, f, f, f, p) == h3q.H3Q_E_ARG
    assert lib.h3q_merge_adapter(None, bogus, -1, 1.0, None, p, p, p, None) == h3q.H3Q_E_ARG
    assert lib.h3q_linear_swiglu_emit(None, p, 1, None, bogus, -1, 0.0, 0, p, f, p) == h3q.H3Q_E_ARG
    assert lib.h3q_linear_prescaled(None, p, p, 1, bogus, -1, 0.0, p) == h3q.H3Q_E_ARG
    assert "live weight handle" in h3q.last_error()
    # AdaLN table: null pointers, then shapes
    assert lib.h3q_adaln_table(None, None, f, p, 1.0, 1, 5, 8, 8, 16, f) == h3q.H3Q_E_ARG
    assert lib.h3q_adaln_table(None, f, f, None, 1.0, 1, 5, 8, 8, 16, f) == h3q.H3Q_E_ARG   # A needed for lora_rank > 0
    for blocks, samples, emb, rb, rl in ((0, 5, 8, 8, 16), (1, 1, 8, 8, 16), (1, 5, 0, 8, 16), (1, 5, 8, 0, 16),
                                         (1, 5, 8, 8, 33), (1, 5, 8, 40, 32), (70000, 5, 8, 8, 16),
                                         (1, 65535 * 16 + 1, 8, 8, 16)):
        assert lib.h3q_adaln_table(None, f, f, p, 1.0, blocks, samples, emb, rb, rl, f) == h3q.H3Q_E_SHAPE, \
            (blocks, samples, emb, rb, rl)
    assert lib.h3q_adaln_table(None, f, f, p, math.inf, 1, 5, 8, 8, 16, f) == h3q.H3Q_E_ARG
    # AdaLN apply: null pointers, then shapes, then alignment
    assert lib.h3q_adaln_apply(None, None, None, f, f, 1, 1, 16, 5, 24, f) == h3q.H3Q_E_ARG
    for T, blocks, rows, samples, R in ((0, 1, 16, 5, 24), (9, 1, 16, 5, 24), (1, 0, 16, 5, 24), (1, 1, -1, 5, 24),
                                        (1, 1, 16, 1, 24), (1, 1, 16, 5, 20), (1, 1, 16, 5, 72), (1, 1, 16, 5, 0)):
        assert lib.h3q_adaln_apply(None, p, None, f, f, T, blocks, rows, samples, R, f) == h3q.H3Q_E_SHAPE, \
            (T, blocks, rows, samples, R)
    odd = ctypes.c_void_p(buf.ctypes.data + 2)
    assert lib.h3q_adaln_apply(None, odd, None, f, f, 1, 1, 16, 5, 24, f) == h3q.H3Q_E_ARG
