"""The library under HIP stream capture (how launch-bound small-S calls are driven): replays of a
captured sequence of calls equal the eager results bit for bit, over several replays with eager work
and synchronizations between them (the W4A4 call included: its activation scale word is zeroed by a
kernel, not a memset); a capture that would have to grow the stream's workspace is refused before
anything is enqueued; a workspace that a capture used survives a later growth on the same stream; and
calls on two streams run concurrently with their own workspaces."""
import pytest
import torch

import bit_linear_dynamic_amd as h3q
from bit_linear_dynamic_amd import synth
from gpu_helpers import Proj, say

pytestmark = pytest.mark.gpu

NONE = h3q.H3Q_ADAPTER_NONE


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def projs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qkv = Proj(3072, 1024, 2400)              # the single fused-QKV-like projection, rank = alpha = 384
    gu = Proj(2 * 512, 1024, 2401, gate_up=True)
    try:
        qkv.add_adapter(1, 384, 384.0, 2402, 2403)
        gu.add_adapter(1, 16, 16.0, 2404, 2405)
        yield qkv, gu
    finally:
        qkv.free()
        gu.free()
        torch.cuda.synchronize()


def _inputs(S, seed):
    return synth.activation(S, 1024, seed, "cuda"), synth.pre_quant_scale(1024, seed + 1, "cuda")


def test_graph_replays_match_eager(projs):
    qkv, gu = projs
    S = 256
    say(f"graph capture S={S}")
    s = torch.cuda.Stream()
    x, pqs = _inputs(S, 2410)
    x2, _ = _inputs(S, 2412)
    y1 = torch.empty((S, 3072), dtype=torch.bfloat16, device="cuda")
    y2, y3 = torch.empty_like(y1), torch.empty_like(y1)
    h = torch.empty((S, 512), dtype=torch.bfloat16, device="cuda")

    def calls():
        h3q.h3q_linear(x, pqs, qkv.handle, 1, 1.0, y=y1, stream=s)
        h3q.h3q_linear(x, pqs, qkv.handle, NONE, 0.0, y=y2, stream=s)
        h3q.h3q_linear_ex(x, pqs, gu.handle, 1, 1.0, h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU, out=h, stream=s)

    with torch.cuda.stream(s):
        calls()  # sizes this stream's workspace
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y1, y2, h)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (y1, y2, h):
            t.zero_()
        with torch.cuda.stream(s):  # eager work on the same workspace between replays
            h3q.h3q_linear(x2, pqs, qkv.handle, 1, 0.5, y=y3, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for got, want in zip((y1, y2, h), ref):
            assert torch.equal(got, want), rep
        say(f"  replay {rep}: bit-identical to the eager calls")


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the refused call enqueued nothing: that is the point
def test_capture_needing_a_larger_workspace_is_refused(projs):
    qkv, _ = projs
    s = torch.cuda.Stream()
    x, pqs = _inputs(512, 2420)
    y = torch.empty((512, 3072), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with pytest.raises(h3q.H3QError) as e:
        with torch.cuda.graph(g, stream=s):
            h3q.h3q_linear(x, pqs, qkv.handle, 1, 1.0, y=y, stream=s)
    assert e.value.code == h3q.H3Q_E_ARG and "capture" in str(e.value)
    torch.cuda.synchronize()
    # the stream is usable afterwards, eagerly
    with torch.cuda.stream(s):
        h3q.h3q_linear(x, pqs, qkv.handle, 1, 1.0, y=y, stream=s)
    torch.cuda.synchronize()


def test_captured_workspace_survives_growth(projs):
    qkv, _ = projs
    s = torch.cuda.Stream()
    x, pqs = _inputs(256, 2430)
    y = torch.empty((256, 3072), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        h3q.h3q_linear(x, pqs, qkv.handle, 1, 1.0, y=y, stream=s)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h3q.h3q_linear(x, pqs, qkv.handle, 1, 1.0, y=y, stream=s)
    torch.cuda.synchronize()
    xb, _ = _inputs(4096, 2432)  # grows this stream's workspace: the captured one must stay allocated
    yb = torch.empty((4096, 3072), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        h3q.h3q_linear(xb, pqs, qkv.handle, 1, 1.0, y=yb, stream=s)
    torch.cuda.synchronize()
    y.zero_()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_two_streams_concurrently(projs):
    qkv, gu = projs
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    xa, pqs = _inputs(777, 2440)
    xb, _ = _inputs(1300, 2442)
    ya = h3q.h3q_linear(xa, pqs, qkv.handle, 1, 1.0)
    hb = h3q.h3q_linear_swiglu(xb, pqs, gu.handle, 1, 0.5)
    torch.cuda.synchronize()
    ya2 = torch.empty_like(ya)
    hb2 = torch.empty_like(hb)
    torch.cuda.synchronize()
    for _ in range(3):  # back to back on two streams, no synchronization in between
        h3q.h3q_linear(xa, pqs, qkv.handle, 1, 1.0, y=ya2, stream=sa)
        h3q.h3q_linear_swiglu(xb, pqs, gu.handle, 1, 0.5, h=hb2, stream=sb)
    torch.cuda.synchronize()
    assert torch.equal(ya, ya2) and torch.equal(hb, hb2)


def test_noalloc_captured_without_a_warm_up_call(projs, monkeypatch):
    """h3q_linear_ex_noalloc under capture with no eager call on the stream first (it needs no
    workspace) and the library's allocator failing throughout: three replays, with eager calls on the
    same fixed scratch between them, equal h3q_linear_ex's results bit for bit (W4A4 included)."""
    qkv, gu = projs
    S = 384
    say(f"no-alloc capture S={S}")
    s = torch.cuda.Stream()
    x, pqs = _inputs(S, 2440)
    x2, _ = _inputs(S, 2442)
    ref = [h3q.h3q_linear_ex(x, pqs, qkv.handle, 1, 1.0),
           h3q.h3q_linear_ex(x, None, qkv.handle, NONE, 0.0),
           h3q.h3q_linear_ex(x, pqs, gu.handle, 1, 1.0, h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU)]
    torch.cuda.synchronize()
    outs = [torch.empty_like(t) for t in ref]
    other = torch.empty_like(ref[0])
    monkeypatch.setenv("H3Q_TEST_FAIL_ALLOC_AFTER", "0")  # any library allocation from here on fails
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h3q.h3q_linear_ex_noalloc(x, pqs, qkv.handle, 1, 1.0, 0, out=outs[0], stream=s)
        h3q.h3q_linear_ex_noalloc(x, None, qkv.handle, NONE, 0.0, 0, out=outs[1], stream=s)
        h3q.h3q_linear_ex_noalloc(x, pqs, gu.handle, 1, 1.0, h3q.H3Q_ACT_NVFP4 | h3q.H3Q_EPI_SWIGLU, out=outs[2],
                                  stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        with torch.cuda.stream(s):  # eager work on the same scratch between replays
            h3q.h3q_linear_ex_noalloc(x2, pqs, qkv.handle, 1, 0.5, h3q.H3Q_ACT_NVFP4, out=other, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), rep
        say(f"  replay {rep}: bit-identical to h3q_linear_ex")
