"""bit_linear_dynamic_amd -- W4 (NVFP4) + dynamic LoRA linear for MI355X (gfx950).

    y = NVFP4_base(x * pre_quant_scale) + strength * (alpha / rank) * B(A x)

(FL2VA Turbo page, section "Implementation"). Every step runs in the hand-written HIP kernels of
``libh3q.so`` behind the C ABI of ``include/h3q.h``; this module only marshals arguments: numpy or
torch CPU arrays for packing and adapter registration, torch device tensors and the current torch
stream for the calls. The functions carry the C names. There is no fallback: if the library is not
built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libh3q.so")

H3Q_OK = 0
H3Q_E_ARG, H3Q_E_SHAPE, H3Q_E_FORMAT, H3Q_E_ADAPTER, H3Q_E_NOMEM, H3Q_E_HIP, H3Q_E_UNSUPPORTED = range(1, 8)
H3Q_ADAPTER_NONE = -1
H3Q_PACK_GATE_UP = 1
H3Q_ACT_NVFP4 = 1
H3Q_EPI_SWIGLU = 2
H3Q_KERNEL_GEMM, H3Q_KERNEL_LORA_DOWN, H3Q_KERNEL_PRESCALE, H3Q_KERNEL_ACT_QUANT = range(4)


class H3QError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"h3q error {code}: {message}")
        self.code = code


_lib = None


def _declare(lib):
    vp, i64, i32, u32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    sigs = {
        "h3q_pack_weight": [vp, vp, vp, f32, i64, i64, u32, ctypes.POINTER(vp)],
        "h3q_free_weight": [vp],
        "h3q_register_adapter": [vp, i32, vp, vp, i32, f32],
        "h3q_unregister_adapter": [vp, i32],
        "h3q_list_adapters": [vp, vp, i32, ctypes.POINTER(i32)],
        "h3q_weight_info": [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(u32)],
        "h3q_linear": [vp, vp, i64, vp, vp, i32, f32, vp],
        "h3q_linear_swiglu": [vp, vp, i64, vp, vp, i32, f32, vp],
        "h3q_linear_ex": [vp, vp, i64, vp, vp, i32, f32, u32, vp],
        "h3q_linear_ex_noalloc": [vp, vp, i64, vp, vp, i32, f32, u32, vp],
        "h3q_linear_qk_norm_rope": [vp, vp, i64, vp, vp, i32, f32, u32, i64, i32, f32, vp, vp, vp, vp, vp],
        "h3q_linear_qk_norm_rope_sections": [vp, vp, i64, vp, vp, i32, f32, u32, i64, i32, vp, i32, f32, vp, vp, vp,
                                             vp, vp],
        "h3q_quantize_nvfp4": [vp, vp, i64, i64, vp, vp, vp, vp],
        "h3q_debug_quantize_act": [vp, vp, i64, i64, vp, vp, vp, vp],
        "h3q_debug_dequant": [vp, vp, vp],
        "h3q_merge_adapter": [vp, vp, i32, f32, vp, vp, vp, vp, vp],
        "h3q_mfma_loop": [vp, vp, vp, i32, i32, vp],
        "h3q_linear_swiglu_emit": [vp, vp, i64, vp, vp, i32, f32, u32, vp, vp, vp],
        "h3q_linear_prescaled": [vp, vp, vp, i64, vp, i32, f32, vp],
        "h3q_adaln_table": [vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, vp],
        "h3q_adaln_apply": [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, vp],
        "h3q_weight_checksum": [vp, vp, ctypes.POINTER(ctypes.c_uint64)],
        "h3q_timing_enable": [i32],
        "h3q_timing_get": [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = i32
    lib.h3q_last_error.argtypes = []
    lib.h3q_last_error.restype = ctypes.c_char_p
    return lib


def lib():
    """The loaded libh3q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(rc: int):
    if rc != H3Q_OK:
        raise H3QError(rc, lib().h3q_last_error().decode())


def last_error() -> str:
    return lib().h3q_last_error().decode()


def _host_ptr(a, dtype):
    """Contiguous host array of `dtype` (bf16 travels as its uint16 bit patterns) + its pointer."""
    import torch
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError("expected a host (CPU) array")
        a = a.detach().contiguous()
        a = (a.view(torch.int16) if a.dtype == torch.bfloat16 else a).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        if a.dtype.kind in "iu" and a.dtype.itemsize == np.dtype(dtype).itemsize:
            a = a.view(dtype)
        else:
            raise TypeError(f"expected {np.dtype(dtype)} data, got {a.dtype}")
    return a, ctypes.c_void_p(a.ctypes.data)


def _dev_ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------------------------------------
# entry points (same names as include/h3q.h)
# ------------------------------------------------------------------------------------------------

def h3q_pack_weight(codes, scales, tensor_scale: float, N: int, K: int, flags: int = 0, stream=None) -> int:
    """Host uint8 codes [N][K/2] and scales [N][K/16] -> weight handle (int)."""
    c, cp = _host_ptr(codes, np.uint8)
    s, sp = _host_ptr(scales, np.uint8)
    if c.size != N * (K // 2) or s.size != N * (K // 16):
        raise ValueError("codes/scales do not match N, K")
    out = ctypes.c_void_p()
    st = None if stream is None else _stream(stream)  # packing copies synchronously
    _check(lib().h3q_pack_weight(st, cp, sp, float(tensor_scale), int(N), int(K), int(flags), ctypes.byref(out)))
    return out.value


def h3q_free_weight(w: int):
    _check(lib().h3q_free_weight(ctypes.c_void_p(w)))


def h3q_register_adapter(w: int, adapter_id: int, A, B, rank: int, alpha: float):
    """Host bf16 A [rank][K] and B [N][rank] (torch bf16 or uint16 bit patterns)."""
    a, ap = _host_ptr(A, np.uint16)
    b, bp = _host_ptr(B, np.uint16)
    N, K = h3q_weight_info(w)[:2]
    if a.size != rank * K or b.size != N * rank:
        raise ValueError("A/B do not match rank, N, K")
    _check(lib().h3q_register_adapter(ctypes.c_void_p(w), int(adapter_id), ap, bp, int(rank), float(alpha)))


def h3q_unregister_adapter(w: int, adapter_id: int):
    _check(lib().h3q_unregister_adapter(ctypes.c_void_p(w), int(adapter_id)))


def h3q_list_adapters(w: int) -> list[int]:
    cnt = ctypes.c_int32()
    _check(lib().h3q_list_adapters(ctypes.c_void_p(w), None, 0, ctypes.byref(cnt)))
    ids = (ctypes.c_int32 * max(cnt.value, 1))()
    _check(lib().h3q_list_adapters(ctypes.c_void_p(w), ids, cnt.value, ctypes.byref(cnt)))
    return list(ids[:cnt.value])


def h3q_weight_info(w: int):
    N, K, fl = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_uint32()
    _check(lib().h3q_weight_info(ctypes.c_void_p(w), ctypes.byref(N), ctypes.byref(K), ctypes.byref(fl)))
    return N.value, K.value, fl.value


def h3q_linear_ex(x, pqs, w: int, adapter_id: int, strength: float, flags: int = 0, out=None, stream=None):
    """x: device bf16 [S][K]; pqs: device fp32 [K] or None. Returns out (allocated if None)."""
    return _linear_ex(lib().h3q_linear_ex, x, pqs, w, adapter_id, strength, flags, out, stream)


def h3q_linear_ex_noalloc(x, pqs, w: int, adapter_id: int, strength: float, flags: int = 0, out=None, stream=None):
    """h3q_linear_ex with the workspace in the library's fixed device scratch (the library allocates
    nothing; `out` is allocated here by torch if None)."""
    return _linear_ex(lib().h3q_linear_ex_noalloc, x, pqs, w, adapter_id, strength, flags, out, stream)


def _linear_ex(fn, x, pqs, w, adapter_id, strength, flags, out, stream):
    import torch
    N, K, _ = h3q_weight_info(w)
    S = x.shape[0]
    n_out = N // 2 if flags & H3Q_EPI_SWIGLU else N
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [S][{K}]")
    if pqs is not None and tuple(pqs.shape) != (K,):
        raise ValueError(f"pqs must be [{K}]")
    if out is None:
        out = torch.empty((S, n_out), dtype=torch.bfloat16, device=x.device)
    elif tuple(out.shape) != (S, n_out):
        raise ValueError(f"out must be [{S}][{n_out}]")
    _check(fn(_stream(stream), _dev_ptr(x, torch.bfloat16, "x"), S, _dev_ptr(pqs, torch.float32, "pqs"),
              ctypes.c_void_p(w), int(adapter_id), float(strength), int(flags), _dev_ptr(out, torch.bfloat16, "out")))
    return out


def h3q_linear(x, pqs, w: int, adapter_id: int, strength: float, y=None, stream=None):
    return h3q_linear_ex(x, pqs, w, adapter_id, strength, 0, y, stream)


def h3q_linear_swiglu(x, pqs, w: int, adapter_id: int, strength: float, h=None, stream=None):
    return h3q_linear_ex(x, pqs, w, adapter_id, strength, H3Q_EPI_SWIGLU, h, stream)


def h3q_linear_swiglu_emit(x, pqs, w: int, adapter_id: int, strength: float, pqs_next, flags: int = 0, h=None,
                           xs_next=None, stream=None):
    """SwiGLU projection that also emits the next projection's base operand bf16(h * pqs_next).
    Returns (h, xs_next), both device bf16 [S][N/2]."""
    import torch
    N, K, _ = h3q_weight_info(w)
    S, F = x.shape[0], N // 2
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [S][{K}]")
    if tuple(pqs_next.shape) != (F,):
        raise ValueError(f"pqs_next must be [{F}]")
    h = torch.empty((S, F), dtype=torch.bfloat16, device=x.device) if h is None else h
    xs_next = torch.empty((S, F), dtype=torch.bfloat16, device=x.device) if xs_next is None else xs_next
    if tuple(h.shape) != (S, F) or tuple(xs_next.shape) != (S, F):
        raise ValueError(f"h and xs_next must be [{S}][{F}]")
    _check(lib().h3q_linear_swiglu_emit(_stream(stream), _dev_ptr(x, torch.bfloat16, "x"), S,
                                        _dev_ptr(pqs, torch.float32, "pqs"), ctypes.c_void_p(w), int(adapter_id),
                                        float(strength), int(flags), _dev_ptr(h, torch.bfloat16, "h"),
                                        _dev_ptr(pqs_next, torch.float32, "pqs_next"),
                                        _dev_ptr(xs_next, torch.bfloat16, "xs_next")))
    return h, xs_next


def h3q_linear_prescaled(x, xs, w: int, adapter_id: int, strength: float, y=None, stream=None):
    """h3q_linear with the base operand xs (= bf16(x * pqs)) given; x feeds the LoRA branch only."""
    import torch
    N, K, _ = h3q_weight_info(w)
    S = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K or tuple(xs.shape) != (S, K):
        raise ValueError(f"x and xs must be [S][{K}]")
    y = torch.empty((S, N), dtype=torch.bfloat16, device=x.device) if y is None else y
    if tuple(y.shape) != (S, N):
        raise ValueError(f"y must be [{S}][{N}]")
    _check(lib().h3q_linear_prescaled(_stream(stream), _dev_ptr(x, torch.bfloat16, "x"),
                                      _dev_ptr(xs, torch.bfloat16, "xs"), S, ctypes.c_void_p(w), int(adapter_id),
                                      float(strength), _dev_ptr(y, torch.bfloat16, "y")))
    return y


def h3q_linear_qk_norm_rope(x, pqs, w: int, adapter_id: int, strength: float, q_width: int, rot_dim: int,
                            eps: float, gamma_q, gamma_k, rope_cos=None, rope_sin=None, flags: int = 0, y=None,
                            stream=None, sections=None):
    """Fused QKV projection + per-head Q/K RMSNorm + split-half rotation of the first rot_dim dims
    (within each section of `sections`, consecutive widths summing to rot_dim, when given: the
    h3q_linear_qk_norm_rope_sections entry point). gamma_q, gamma_k: device fp32 [q_width];
    rope_cos, rope_sin: device fp32 [S][rot_dim/2]."""
    import torch
    N, K, _ = h3q_weight_info(w)
    S = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [S][{K}]")
    if pqs is not None and tuple(pqs.shape) != (K,):
        raise ValueError(f"pqs must be [{K}]")
    for name, g in (("gamma_q", gamma_q), ("gamma_k", gamma_k)):
        if tuple(g.shape) != (q_width,):
            raise ValueError(f"{name} must be [{q_width}]")
    if rot_dim > 0:
        for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            if t is None or tuple(t.shape) != (S, rot_dim // 2):
                raise ValueError(f"{name} must be [{S}][{rot_dim // 2}]")
    if y is None:
        y = torch.empty((S, N), dtype=torch.bfloat16, device=x.device)
    elif tuple(y.shape) != (S, N):
        raise ValueError(f"y must be [{S}][{N}]")
    common = (_dev_ptr(gamma_q, torch.float32, "gamma_q"), _dev_ptr(gamma_k, torch.float32, "gamma_k"),
              _dev_ptr(rope_cos, torch.float32, "rope_cos"), _dev_ptr(rope_sin, torch.float32, "rope_sin"),
              _dev_ptr(y, torch.bfloat16, "y"))
    head = (_stream(stream), _dev_ptr(x, torch.bfloat16, "x"), S, _dev_ptr(pqs, torch.float32, "pqs"),
            ctypes.c_void_p(w), int(adapter_id), float(strength), int(flags), int(q_width), int(rot_dim))
    if sections is None:
        _check(lib().h3q_linear_qk_norm_rope(*head, float(eps), *common))
    else:
        sec = (ctypes.c_int32 * max(len(sections), 1))(*[int(v) for v in sections])
        _check(lib().h3q_linear_qk_norm_rope_sections(*head, sec, len(sections), float(eps), *common))
    return y


def h3q_merge_adapter(w: int, adapter_id: int, strength: float, pqs=None, merged: bool = False, stream=None):
    """The merged route (for comparison): NVFP4 of Wq*ts + c*(B A)/pqs. Returns device tensors
    (codes u8 [N][K/2], scales u8 [N][K/16], ts fp32 [1]) and, if merged, the fp32 [N][K] m."""
    import torch
    N, K, _ = h3q_weight_info(w)
    dev = torch.device("cuda", torch.cuda.current_device())
    if pqs is not None and tuple(pqs.shape) != (K,):
        raise ValueError(f"pqs must be [{K}]")
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty((1,), dtype=torch.float32, device=dev)
    m = torch.empty((N, K), dtype=torch.float32, device=dev) if merged else None
    _check(lib().h3q_merge_adapter(_stream(stream), ctypes.c_void_p(w), int(adapter_id), float(strength),
                                   _dev_ptr(pqs, torch.float32, "pqs"), _dev_ptr(codes), _dev_ptr(scales),
                                   _dev_ptr(ts), _dev_ptr(m, torch.float32, "merged")))
    return (codes, scales, ts, m) if merged else (codes, scales, ts)


def h3q_adaln_table(u, emb, A, scale: float, stream=None):
    """Device u fp32 [S][rb], emb fp32 [S][E], A bf16 [blocks][rl][E] (or None) -> fp32 table
    [blocks][S][rb + rl] = [u ; scale * A_b silu(emb)]."""
    import torch
    S, rb = u.shape
    E = emb.shape[1]
    if tuple(emb.shape) != (S, E):
        raise ValueError("emb must be [S][E]")
    blocks, rl = (A.shape[0], A.shape[1]) if A is not None else (1, 0)
    if A is not None and A.shape[2] != E:
        raise ValueError("A must be [blocks][rl][E]")
    table = torch.empty((blocks, S, rb + rl), dtype=torch.float32, device=u.device)
    _check(lib().h3q_adaln_table(_stream(stream), _dev_ptr(u, torch.float32, "u"), _dev_ptr(emb, torch.float32, "emb"),
                                 _dev_ptr(A, torch.bfloat16, "A"), float(scale), blocks, S, E, rb, rl,
                                 _dev_ptr(table, torch.float32, "table")))
    return table


def h3q_adaln_apply(M, bias, table, t, out=None, stream=None):
    """Device M bf16 [blocks][rows][R], bias fp32 [blocks][rows] or None, table fp32 [blocks][S][R],
    t fp32 [T] -> out fp32 [T][blocks][rows] = bias + M v(t)."""
    import torch
    blocks, rows, R = M.shape
    S = table.shape[1]
    if tuple(table.shape) != (blocks, S, R):
        raise ValueError("table must be [blocks][S][R]")
    T = t.shape[0]
    if out is None:
        out = torch.empty((T, blocks, rows), dtype=torch.float32, device=M.device)
    elif tuple(out.shape) != (T, blocks, rows):
        raise ValueError(f"out must be [{T}][{blocks}][{rows}]")
    _check(lib().h3q_adaln_apply(_stream(stream), _dev_ptr(M, torch.bfloat16, "M"), _dev_ptr(bias, torch.float32, "bias"),
                                 _dev_ptr(table, torch.float32, "table"), _dev_ptr(t, torch.float32, "t"), T, blocks,
                                 rows, S, R, _dev_ptr(out, torch.float32, "out")))
    return out


def h3q_mfma_loop(ops_a, ops_b, iters: int, workgroups: int, sink=None, stream=None):
    """Pure matrix-core loop (measurement aid). ops_a, ops_b: device bf16 [8][256][8]. Returns the sink."""
    import torch
    if tuple(ops_a.shape) != (8, 256, 8) or tuple(ops_b.shape) != (8, 256, 8):
        raise ValueError("ops_a and ops_b must be [8][256][8]")
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device=ops_a.device) if sink is None else sink
    _check(lib().h3q_mfma_loop(_stream(stream), _dev_ptr(ops_a, torch.bfloat16, "ops_a"),
                               _dev_ptr(ops_b, torch.bfloat16, "ops_b"), int(iters), int(workgroups),
                               _dev_ptr(sink, torch.float32, "sink")))
    return sink


def _quantize_act(fn, x, pqs, stream):
    import torch
    S, K = x.shape
    codes = torch.empty((S, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((S, K // 16), dtype=torch.uint8, device=x.device)
    ts = torch.empty((1,), dtype=torch.float32, device=x.device)
    _check(fn(_stream(stream), _dev_ptr(x, torch.bfloat16, "x"), S, K, _dev_ptr(pqs, torch.float32, "pqs"),
              _dev_ptr(codes), _dev_ptr(scales), _dev_ptr(ts)))
    return codes, scales, ts


def h3q_debug_quantize_act(x, pqs=None, stream=None):
    """Device bf16 x [S][K] -> (codes u8 [S][K/2], scales u8 [S][K/16], ts fp32 [1]) on the device:
    the W4A4 activation quantizer exactly as the linear runs it."""
    return _quantize_act(lib().h3q_debug_quantize_act, x, pqs, stream)


def h3q_quantize_nvfp4(x, pqs=None, stream=None):
    """The same quantizer under its earlier name (kept as an alias)."""
    return _quantize_act(lib().h3q_quantize_nvfp4, x, pqs, stream)


def h3q_debug_dequant(w: int, out=None, stream=None):
    import torch
    N, K, _ = h3q_weight_info(w)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    _check(lib().h3q_debug_dequant(_stream(stream), ctypes.c_void_p(w), _dev_ptr(out, torch.bfloat16, "out")))
    return out


def h3q_weight_checksum(w: int, stream=None) -> int:
    h = ctypes.c_uint64()
    _check(lib().h3q_weight_checksum(_stream(stream), ctypes.c_void_p(w), ctypes.byref(h)))
    return h.value


def h3q_timing_enable(on: bool = True):
    _check(lib().h3q_timing_enable(1 if on else 0))


def h3q_timing_get(kind: int):
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().h3q_timing_get(int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def h3q_linear_qk_norm_rope_sections(x, pqs, w: int, adapter_id: int, strength: float, q_width: int, rot_dim: int,
                                     sections, eps: float, gamma_q, gamma_k, rope_cos=None, rope_sin=None,
                                     flags: int = 0, y=None, stream=None):
    """h3q_linear_qk_norm_rope with the rotated dims in axis sections, each rotated in split halves
    within itself (`sections`: consecutive even widths summing to rot_dim)."""
    return h3q_linear_qk_norm_rope(x, pqs, w, adapter_id, strength, q_width, rot_dim, eps, gamma_q, gamma_k,
                                   rope_cos, rope_sin, flags, y, stream, sections=list(sections))
