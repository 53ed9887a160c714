"""The AdaLN modulation curve with the adapter folded in (MiniMax-H3 Turbo CMF card, "What the
conversion did"; MiniMax-H3 Ultra Fast, "Why the pruned transformer matters") against the fp64 oracle:
the per-block [u ; c A silu(e)] table, the interpolated [W_p | B] v(t) + bias apply on a table both
sides share, and the two chained at the full shape (50 blocks of [96768, 24], 1025 samples) on
sampled blocks and rows.

Tolerances (normwise, ||got - ref|| / ||ref||): the table accumulates E products in fp32 with a
hardware exp (relative error per entry about E * 2^-24 of the sum of |terms|), so 1e-5; the apply
interpolates in fp32 and accumulates R = 24 products in fp32, so 1e-5 as well -- both far inside
the 4e-3 bar of the projection, whose bf16 rounding they do not have."""
import numpy as np
import pytest
import torch

import bit_linear_dynamic_amd as h3q
import oracle
from bit_linear_dynamic_amd import synth
from bit_linear_dynamic_amd import workloads as wl
from gpu_helpers import bits, say

pytestmark = pytest.mark.gpu

TOL_CURVE = 1e-5


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def nw(got, ref):
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else got
    return float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))


def curve(c: wl.AdalnCurve, seed: int):
    return synth.adaln_curve_inputs(c.blocks, c.samples, c.emb_dim, c.base_rank, c.lora_rank, c.rows, seed)


@pytest.mark.parametrize("rl,scale", [(16, 1.0), (0, 0.0), (32, -0.5), (5, 2.0)])
def test_adaln_table_parity(rl, scale):
    c = wl.AdalnCurve(blocks=3, samples=33, emb_dim=200, base_rank=8, lora_rank=rl, rows=64)
    say(f"adaln table blocks={c.blocks} samples={c.samples} E={c.emb_dim} rb={c.base_rank} rl={rl} scale={scale}")
    u, emb, A, _, _ = curve(c, 2000 + rl)
    got = h3q.h3q_adaln_table(u.cuda(), emb.cuda(), A.cuda() if rl else None, scale)
    torch.cuda.synchronize()
    ref = oracle.adaln_table(u.numpy(), emb.numpy(), bits(A) if rl else np.zeros((c.blocks, 0, c.emb_dim), np.uint16),
                             scale)
    if not rl:
        ref = ref[:1]
    g = got.cpu().numpy()
    assert np.array_equal(g[:, :, :c.base_rank], np.broadcast_to(u.numpy(), g[:, :, :c.base_rank].shape))
    if rl and scale:
        err = nw(g[:, :, c.base_rank:], ref[:, :, c.base_rank:])
        say(f"  adapter part normwise {err:.3e}")
        assert err <= TOL_CURVE
    elif rl:
        assert not np.any(g[:, :, c.base_rank:])


T_CASES = [0.0, 1.0, 0.5, 0.8125, 1.0 / 32, 0.3, -0.1, 1.3]


@pytest.mark.parametrize("R,rows,T", [(24, 1000, 8), (8, 257, 1), (64, 300, 3)])
def test_adaln_apply_parity(R, rows, T):
    """Apply against the oracle on the same fp32 table (seeded draws), times on and between samples,
    at both ends and clamped outside [0, 1]; ragged row counts."""
    blocks, S = 3, 33
    say(f"adaln apply R={R} rows={rows} T={T}")
    M = synth.normal((blocks, rows, R), 0.1, 2100 + R, dtype=torch.bfloat16)
    bias = synth.normal((blocks, rows), 0.1, 2101 + R)
    table = synth.normal((blocks, S, R), 1.0, 2102 + R)
    t = torch.tensor(T_CASES[:T], dtype=torch.float32)
    for with_bias in (True, False):
        got = h3q.h3q_adaln_apply(M.cuda(), bias.cuda() if with_bias else None, table.cuda(), t.cuda())
        torch.cuda.synchronize()
        ref = oracle.adaln_apply(bits(M), bias.numpy() if with_bias else None, table.numpy().astype(np.float64),
                                 t.numpy())
        err = nw(got, ref)
        say(f"  bias={with_bias}: normwise {err:.3e}")
        assert err <= TOL_CURVE


@pytest.mark.slow
def test_adaln_full_curve_sampled():
    """The full workload (50 blocks, rows 96768, R 24, 1025 samples, E 2688): the GPU table + apply
    against the oracle's table + apply on blocks 0, 17, 49 and a row sample, at two times."""
    c = wl.ADALN
    say(f"adaln full blocks={c.blocks} rows={c.rows} samples={c.samples} E={c.emb_dim}")
    u, emb, A, M, bias = curve(c, 2200)
    t = torch.tensor([0.8125, 0.30078125], dtype=torch.float32)
    table = h3q.h3q_adaln_table(u.cuda(), emb.cuda(), A.cuda(), 1.0)
    out = h3q.h3q_adaln_apply(M.cuda(), bias.cuda(), table, t.cuda())
    torch.cuda.synchronize()
    blks = np.array([0, 17, 49])
    rows = np.unique(np.concatenate([np.arange(256), np.arange(256, c.rows, 97), np.arange(c.rows - 256, c.rows)]))
    Ab = bits(A)[blks]
    ref_table = oracle.adaln_table(u.numpy(), emb.numpy(), Ab, 1.0)
    Mb = bits(M)[blks][:, rows]
    ref = oracle.adaln_apply(Mb, bias.numpy()[blks][:, rows], ref_table, t.numpy())
    got = out.cpu().numpy()[:, blks][:, :, rows]
    err = nw(got, ref)
    say(f"  {len(blks)} blocks x {len(rows)} rows x 2 times: normwise {err:.3e}")
    assert err <= TOL_CURVE


def test_adaln_argument_errors():
    M = torch.zeros((2, 16, 24), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((2, 5, 24), dtype=torch.float32, device="cuda")
    t = torch.zeros(2, dtype=torch.float32, device="cuda")

    def expect(code, fn):
        with pytest.raises(h3q.H3QError) as e:
            fn()
        assert e.value.code == code, e.value

    expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_adaln_apply(M[:, :, :20].contiguous(), None, table[:, :, :20].contiguous(), t))
    expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_adaln_apply(M, None, table, torch.zeros(9, device="cuda")))
    expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_adaln_apply(M, None, table[:, :1].contiguous(), t))
    u = torch.zeros((5, 8), device="cuda")
    emb = torch.zeros((5, 10), device="cuda")
    expect(h3q.H3Q_E_SHAPE, lambda: h3q.h3q_adaln_table(u, emb, torch.zeros((1, 33, 10), dtype=torch.bfloat16,
                                                                               device="cuda"), 1.0))
    expect(h3q.H3Q_E_ARG, lambda: h3q.h3q_adaln_table(u, emb, torch.zeros((1, 4, 10), dtype=torch.bfloat16,
                                                                             device="cuda"), float("inf")))
