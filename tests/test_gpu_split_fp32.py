"""GPU parity of the split-precision fp32 path (LA_F32_SPLIT: every product
as three bf16 MFMAs over hi/lo operand splits) against the fp64 oracle, at the
fp32 tolerance (1e-3, row-normalised).

Each kept product carries about 2^-17 of relative error (the bf16 rounding of
the low terms and the dropped lo.lo term), so outputs land at a few 1e-4 after
the cancellation inside q.S; a plain bf16 evaluation of the same fp32 data
(low terms dropped) lands near 1e-2, which the bound rejects -- checked below
on the oracle itself."""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TIGHT = 1e-3

EDGE = [
    ([1], [0], []),
    ([63], [2], [1, 64]),
    ([64], [3], [63, 65, 1]),
    ([127, 128], [2, 2], [128, 129, 1, 2]),
    ([200, 1, 640], [0, 3, 1], [64, 64, 5, 300]),
]


def _run(q, k, v, plan, ext=None, split=True):
    out, fin = la.scan_packed(q.to(DEV), k.to(DEV), v.to(DEV), plan,
                              ext_state=None if ext is None else ext.to(DEV), split_fp32=split)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 3])
@pytest.mark.parametrize("case", range(len(EDGE)))
def test_split_edge_lengths(case, G, d):
    vl, bc, bl = EDGE[case]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(300 + case), int(so[-1]), 3, d, "f32")
    plan = la.pack(vl, bc, bl, heads=3, block_chunks=G)
    out, fin = _run(q, k, v, plan)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, so, bp)
    eo, ef = oracle.row_rel_err(out, ref_o), oracle.state_rel_err(fin, ref_f)
    print(f"  case {case} G={G} d={d}: out err {eo:.2e} final err {ef:.2e}", flush=True)
    assert eo <= TIGHT and ef <= TIGHT


def test_bound_rejects_a_plain_bf16_evaluation():
    """Inputs rounded to bf16 (what dropping every low term amounts to) miss
    the fp32 bound by a wide margin, so passing it shows the low terms count."""
    vl, bc, bl = EDGE[4]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(304), int(so[-1]), 3, 64, "f32")
    ref, _ = oracle.scan_recurrence(q, k, v, so, bp)
    rounded, _ = oracle.scan_recurrence(*(x.to(torch.bfloat16) for x in (q, k, v)), so, bp)
    assert oracle.row_rel_err(rounded, ref) > 5 * TIGHT


@pytest.mark.parametrize("name", ["view500_br4x32_h2_d64_f32", "view7400_br8x48_h16_d64_f32"])
def test_split_workloads(name):
    w = synth.workload(name)
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    ref_o, ref_f = oracle.scan_recurrence(w.q, w.k, w.v, plan.seg_offsets, plan.branch_parent)
    o_s, f_s = _run(w.q, w.k, w.v, plan, split=True)
    es, fs = oracle.row_rel_err(o_s, ref_o), oracle.state_rel_err(f_s, ref_f)
    print(f"  {name}: split out err {es:.2e} final err {fs:.2e}", flush=True)
    assert es <= TIGHT and fs <= TIGHT


def test_split_workload_and_fp32_mfma_agree():
    w = synth.workload("view500_br4x32_h2_d64_f32")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    ref_o, ref_f = oracle.scan_recurrence(w.q, w.k, w.v, plan.seg_offsets, plan.branch_parent)
    o_s, f_s = _run(w.q, w.k, w.v, plan, split=True)
    o_f, f_f = _run(w.q, w.k, w.v, plan, split=False)
    es, ef = oracle.row_rel_err(o_s, ref_o), oracle.row_rel_err(o_f, ref_o)
    print(f"  split err {es:.2e}  fp32-MFMA err {ef:.2e}", flush=True)
    assert es <= TIGHT and oracle.state_rel_err(f_s, ref_f) <= TIGHT


def test_split_ternary_inputs_are_exact():
    """Values in {-1, 0, 1} split into (x, 0): every product and partial sum
    is an exact integer, so the output equals the oracle bit for bit."""
    vl, bc, bl = [3000, 700], [5, 2], [64, 100, 1, 128, 65, 77, 3]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.ternary_qkv(9, int(so[-1]), 4, 64, "f32")
    plan = la.pack(vl, bc, bl, heads=4, block_chunks=2)
    out, fin = _run(q, k, v, plan)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, so, bp)
    assert torch.equal(out.double(), torch.from_numpy(ref_o))
    assert torch.equal(fin.double(), torch.from_numpy(ref_f))


def test_split_shard_pass_from_external_state():
    vl, bc, bl = [0, 300], [3, 1], [40, 70, 1, 65]
    plan = la.pack(vl, bc, bl, heads=2, block_chunks=2)
    rng = np.random.default_rng(8)
    q, k, v = synth.draw_qkv(rng, plan.info.n_tokens, 2, 64, "f32")
    ext = torch.from_numpy(rng.standard_normal((1, 2, 64, 64)).astype(np.float32))
    out, _ = _run(q, k, v, plan, ext=ext)
    ref_o, _ = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                      ext_state=ext)
    assert oracle.row_rel_err(out, ref_o) <= TIGHT


def test_split_rejects_bf16_inputs():
    plan = la.pack([10], [0], [], heads=1)
    x = torch.zeros((10, 1, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(TypeError):
        la.scan_packed(x, x, x, plan, split_fp32=True)
