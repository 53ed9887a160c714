"""The merged route against the oracle, and merged against dynamic (what never merging buys). The
merged weight (the adapter's update folded in before quantizing: MiniMax-H3 Turbo CMF card, "What the
conversion did") must equal the oracle's bit for bit: its fp32 values, NVFP4 codes, scales and tensor
scale. The dynamic path (FL2VA Turbo, "Implementation") and the merged route are then both compared
with the method's exact output, base + c B (A x) in fp64, on the same inputs."""
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


@pytest.fixture(autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def merged_reference(p: Proj, adapter_id, strength, pqs):
    if adapter_id == NONE:
        return oracle.merged_nvfp4(p.codes, p.scales, p.ts, pqs=pqs)
    A, B, r, alpha = p.adapters[adapter_id]
    return oracle.merged_nvfp4(p.codes, p.scales, p.ts, A, B, r, alpha, strength, pqs)


def merged_f32_reference(p: Proj, adapter_id, strength, pqs, rows=None):
    codes, scales = (p.codes, p.scales) if rows is None else (p.codes[rows], p.scales[rows])
    if adapter_id == NONE:
        return oracle.merge_lora(codes, scales, p.ts, pqs=pqs)
    A, B, r, alpha = p.adapters[adapter_id]
    return oracle.merge_lora(codes, scales, p.ts, A, B if rows is None else B[rows], r, alpha, strength, pqs)


MERGE_CASES = [
    # N, K, rank, alpha, strength, gate_up, with pqs
    (300, 208, 65, 16.0, -1.5, False, True),
    (2 * 200, 512, 128, 128.0, 1.0, True, True),
    (3072, 1024, 384, 384.0, 1.0, False, True),
    (64, 64, 1, 2.0, 0.5, False, False),
]


@pytest.mark.parametrize("N,K,rank,alpha,strength,gate_up,with_pqs", MERGE_CASES)
def test_merge_bit_exact(N, K, rank, alpha, strength, gate_up, with_pqs):
    say(f"merge N={N} K={K} r={rank} alpha={alpha} strength={strength} gate_up={gate_up} pqs={with_pqs}")
    p = Proj(N, K, 1400 + N + K, gate_up=gate_up)
    try:
        p.add_adapter(1, rank, alpha, 1401 + N, 1402 + K)
        pqs = synth.pre_quant_scale(K, 1403) if with_pqs else None
        pq = pqs.numpy() if with_pqs else None
        ck = h3q.h3q_weight_checksum(p.handle)
        for aid, st in ((1, strength), (NONE, 1.0), (1, 0.0)):
            codes, scales, ts, m = h3q.h3q_merge_adapter(p.handle, aid, st, pqs.cuda() if with_pqs else None,
                                                         merged=True)
            torch.cuda.synchronize()
            m_ref = merged_f32_reference(p, aid, st, pq)
            assert np.array_equal(m.cpu().numpy(), m_ref), (aid, st, "merged fp32 weight")
            oc, osc, ots = merged_reference(p, aid, st, pq)
            assert ts.item() == ots, (aid, st)
            assert np.array_equal(scales.cpu().numpy(), osc), (aid, st)
            assert np.array_equal(codes.cpu().numpy(), oc), (aid, st)
            say(f"  adapter={aid} strength={st}: m, codes, scales, ts bit-identical (ts={ots:.6g})")
        assert h3q.h3q_weight_checksum(p.handle) == ck, "the handle's packed weight was modified"
    finally:
        p.free()


def compare_routes(p: Proj, x: torch.Tensor, pqs: torch.Tensor, rows=None, with_delta=True):
    """normwise errors of the dynamic and the merged route against the exact output base + c B (A x)."""
    A, B, r, alpha = p.adapters[1]
    y_dyn = h3q.h3q_linear(x, pqs, p.handle, 1, 1.0)
    codes, scales, ts = h3q.h3q_merge_adapter(p.handle, 1, 1.0, pqs)
    mp = Proj(p.N, p.K, 0, gate_up=p.gate_up, codes=codes.cpu().numpy(), scales=scales.cpu().numpy(),
              ts=float(ts.item()))
    try:
        y_mrg = h3q.h3q_linear(x, pqs, mp.handle, NONE, 0.0)
        torch.cuda.synchronize()
        sel = np.arange(x.shape[0]) if rows is None else rows
        idx = torch.from_numpy(sel).to(x.device)
        xb, pq = bits(x.index_select(0, idx)), pqs.cpu().numpy()
        y_def = oracle.linear(xb, pq, p.codes, p.scales, p.ts, A, B, r, alpha, 1.0)
        y_mrg_ref = oracle.linear(xb, pq, mp.codes, mp.scales, mp.ts)
        e_dyn = normwise(y_dyn.index_select(0, idx), y_def)
        e_mrg = normwise(y_mrg.index_select(0, idx), y_def)
        e_mrg_parity = normwise(y_mrg.index_select(0, idx), y_mrg_ref)
        if with_delta:
            d = y_def - oracle.linear(xb, pq, p.codes, p.scales, p.ts)
            say(f"  adapter term / output = {np.linalg.norm(d) / np.linalg.norm(y_def):.3e}")
        say(f"  error vs exact: dynamic {e_dyn:.3e}, merged {e_mrg:.3e}; merged GPU vs merged oracle "
            f"{e_mrg_parity:.3e}")
        return e_dyn, e_mrg, e_mrg_parity
    finally:
        mp.free()


def test_merged_vs_dynamic_accuracy():
    """One QKV-like projection (3072 x 1024, rank = alpha = 384) at S = 256: the dynamic path stays
    within the parity bar of the exact output; the merged route re-quantizes the adapted weight and
    carries the full NVFP4 rounding of it."""
    N, K, S = 3072, 1024, 256
    say(f"merged vs dynamic N={N} K={K} S={S}")
    p = Proj(N, K, 1500)
    try:
        p.add_adapter(1, 384, 384.0, 1501, 1502)
        x = synth.activation(S, K, 1503).cuda()
        pqs = synth.pre_quant_scale(K, 1504).cuda()
        e_dyn, e_mrg, e_par = compare_routes(p, x, pqs)
        assert e_dyn <= TOL and e_par <= TOL
        assert e_mrg > 4 * e_dyn
    finally:
        p.free()


@pytest.mark.slow
def test_merge_full_qkv():
    """The block's fused QKV projection (18432 x 6144, rank 384): the merged fp32 weight on sampled
    rows bit for bit, and the two routes against the exact output on sampled rows at S = 8192."""
    P, S = wl.QKV, wl.S_MID
    say(f"merge full QKV {P.N}x{P.K}")
    p = Proj(P.N, P.K, synth.seed_of(2, 0, synth.W))
    try:
        p.add_adapter(1, P.rank, P.alpha, synth.seed_of(2, 0, synth.A1), synth.seed_of(2, 0, synth.B1))
        pqs = synth.pre_quant_scale(P.K, synth.seed_of(8, 0, synth.PQS))
        _, _, _, m = h3q.h3q_merge_adapter(p.handle, 1, 1.0, pqs.cuda(), merged=True)
        torch.cuda.synchronize()
        wrows = np.unique(np.concatenate([np.arange(64), np.arange(64, P.N, 997), np.arange(P.N - 64, P.N)]))
        m_ref = merged_f32_reference(p, 1, 1.0, pqs.numpy(), rows=wrows)
        assert np.array_equal(m[torch.from_numpy(wrows).cuda()].cpu().numpy(), m_ref)
        say(f"  merged fp32 weight: {len(wrows)} sampled rows bit-identical")
        del m
        x = synth.activation(S, P.K, synth.seed_of(8, 0, synth.X)).cuda()
        rows = np.unique(np.concatenate([np.arange(32), np.arange(32, S, 512), np.arange(S - 32, S)]))
        e_dyn, e_mrg, e_par = compare_routes(p, x, pqs.cuda(), rows, with_delta=False)
        assert e_dyn <= TOL and e_par <= TOL
    finally:
        p.free()
