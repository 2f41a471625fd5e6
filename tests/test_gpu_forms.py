"""The forms of the scan on the GPU: three launches (block states, prefix
launch, outputs), two launches (the output workgroups sum the block states
they need themselves; a view's last block writes its final state) and, on
the piece path (d = 64, bf16), one launch (each workgroup obtains the prefix
from the workgroups before it in the same launch).

All forms add the block states in the same order, so they must agree bit
for bit, and each must match the fp64 oracle within the tolerance (row-
normalised max relative error 1e-3 for fp32 inputs, 2e-2 for bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}
DEV = "cuda:0"

STRUCTS = [
    # view lengths, branch counts, branch lengths (0 = shard request)
    ([1], [0], []),
    ([64], [3], [63, 65, 1]),
    ([127, 128], [2, 2], [128, 129, 1, 2]),
    ([700, 1, 640], [3, 3, 1], [64, 300, 5, 64, 64, 5, 300]),
    ([0, 900], [2, 2], [200, 70, 129, 1]),
    ([70 * 64], [2], [40 * 64 + 17, 5]),
]


def _pass(case, H, d, dtype):
    vl, bc, bl = STRUCTS[case]
    T = int(np.sum(vl) + np.sum(bl))
    q, k, v = synth.draw_qkv(np.random.default_rng(500 + case), T, H, d, dtype)
    ext = None
    if any(x == 0 for x in vl):
        ext = torch.from_numpy(np.random.default_rng(600 + case).standard_normal(
            (1, H, d, d)).astype(np.float32))
    return vl, bc, bl, q, k, v, ext


def _run(q, k, v, plan, form, ext=None, split=False):
    qd, kd, vd = (x.to(DEV).contiguous() for x in (q, k, v))
    ed = None if ext is None else ext.to(DEV).contiguous()
    out, fin = la.scan_packed(qd, kd, vd, plan, ext_state=ed, form=form, split_fp32=split)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


@pytest.mark.parametrize("dtype,d,split", [("bf16", 64, False), ("bf16", 128, False),
                                           ("f32", 64, False), ("f32", 128, False),
                                           ("f32", 64, True), ("f32", 128, True)])
@pytest.mark.parametrize("G", [1, 3])
@pytest.mark.parametrize("case", range(len(STRUCTS)))
def test_two_and_three_launch_forms_agree(dtype, d, split, G, case):
    vl, bc, bl, q, k, v, ext = _pass(case, 2, d, dtype)
    plan = la.pack(vl, bc, bl, block_chunks=G)
    print(f"case {case} {dtype} d={d} split={split} G={G}: slots={plan.info.n_delta} "
          f"two-launch reads={plan.info.fused_slot_reads}", flush=True)
    o3, f3 = _run(q, k, v, plan, "three", ext, split)
    o2, f2 = _run(q, k, v, plan, "two", ext, split)
    assert torch.equal(o2, o3)
    assert torch.equal(f2, f3)
    if dtype == "bf16" and d == 64:
        o1, f1 = _run(q, k, v, plan, "one", ext, split)
        assert torch.equal(o1, o3) and torch.equal(f1, f3)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                          ext_state=ext)
    eo, ef = oracle.row_rel_err(o2, ref_o), oracle.state_rel_err(f2, ref_f)
    print(f"  out err {eo:.3e}  final err {ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("form", ["two", "three"])
def test_exact_probe_both_forms(form):
    """Integer-valued indexing probe (q = k = e_0, v = one-hot segment code,
    fp32) on a 30-chunk view with branches of 1-3 blocks, one chunk per
    block: outputs and the final state are exact integers in either form."""
    vl, bc, bl = [30 * 64 - 5], [4], [1, 64, 129, 150]
    plan = la.pack(vl, bc, bl, block_chunks=1)
    so, bp = plan.seg_offsets, plan.branch_parent
    H, d = 2, 64
    q, k, v = synth.probe_qkv(so, bp, H, d, 0)
    out, fin = _run(q, k, v, plan, form)
    exp = np.zeros((int(so[-1]), d))
    for s in range(len(bp)):
        a, b = int(so[s]), int(so[s + 1])
        exp[a:b, s % d] += np.arange(1, b - a + 1)
        if bp[s] >= 0:
            exp[a:b, int(bp[s]) % d] += int(so[bp[s] + 1] - so[bp[s]])
    for h in range(H):
        assert np.array_equal(out[:, h].double().numpy(), exp)
    f_exp = np.zeros(d)
    f_exp[0] = int(so[1])
    assert np.array_equal(fin[0, 0, 0].double().numpy(), f_exp)
    assert bool(torch.all(fin[0, :, 1:] == 0))


@pytest.mark.parametrize("name", ["view7400_br8x48_h16_d64_bf16",
                                  "view18000_br256x32-128_h16_d64_bf16"])
def test_workload_forms_agree(name):
    """A benchmark workload in the binding's block configuration, both forms:
    bit-identical outputs and final states, within tolerance of the oracle."""
    w = synth.workload(name)
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    print(f"{name}: G={plan.info.block_chunks} launches(auto)="
          f"{la.scan_launches(plan, w.H, w.d)}", flush=True)
    o3, f3 = _run(w.q, w.k, w.v, plan, "three")
    o2, f2 = _run(w.q, w.k, w.v, plan, "two")
    o1, f1 = _run(w.q, w.k, w.v, plan, "one")
    assert torch.equal(o2, o3) and torch.equal(f2, f3)
    assert torch.equal(o1, o3) and torch.equal(f1, f3)
    ref_o, ref_f = oracle.scan_recurrence(w.q, w.k, w.v, plan.seg_offsets, plan.branch_parent)
    assert oracle.row_rel_err(o2, ref_o) <= TOL["bf16"]
    assert oracle.state_rel_err(f2, ref_f) <= TOL["bf16"]


def test_output_launch_alone_repeats_in_two_launch_form():
    """In the two-launch form the workspace keeps the blocks' own states, so
    the output launch repeated alone after a full pass gives the same out."""
    w = synth.workload("view7400_br8x48_h16_d64_bf16")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    qd, kd, vd = (x.to(DEV) for x in (w.q, w.k, w.v))
    ws = la.new_workspace(plan, w.H, w.d, la.LA_BF16, DEV)
    o1, f1 = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="two")
    o1 = o1.clone()
    o2 = torch.full_like(o1, float("nan"))
    la.scan_packed(qd, kd, vd, plan, out=o2, final_state=f1, workspace=ws,
                   stages=la.STAGE_OUTPUT, form="two")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d", [64, 128])
def test_wide_prefix_launch_agrees(d):
    """Enough segment-heads for the prefix launch to take 4 elements per
    thread (>= 8192 workgroups at one element per thread): 24 views of 150-700
    tokens and 40 branches, some of several blocks, H = 32, one chunk per
    block.  The three-launch form must equal the two-launch form (no prefix
    launch) bit for bit and match the oracle."""
    rng = np.random.default_rng(900 + d)
    vl = rng.integers(150, 700, size=24)
    bc = rng.integers(0, 4, size=24)
    bl = rng.integers(1, 200, size=int(bc.sum()))
    H = 32
    plan = la.pack(vl, bc, bl, heads=H, block_chunks=1)
    assert plan.info.n_scan * H * (d * d // 256) >= 8192
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(rng, T, H, d, "bf16")
    o3, f3 = _run(q, k, v, plan, "three")
    o2, f2 = _run(q, k, v, plan, "two")
    assert torch.equal(o2, o3) and torch.equal(f2, f3)
    if d == 64:
        o1, f1 = _run(q, k, v, plan, "one")
        assert torch.equal(o1, o3) and torch.equal(f1, f3)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent)
    eo, ef = oracle.row_rel_err(o3, ref_o), oracle.state_rel_err(f3, ref_f)
    print(f"  wide prefix d={d}: T={T} scans={plan.info.n_scan} out err {eo:.3e} final err {ef:.3e}",
          flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("form", ["two", "three"])
def test_launches_one_at_a_time_equal_the_full_pass(form):
    """la_scan_packed_stages run launch by launch on one workspace (block
    states, prefix, outputs; the prefix bit does nothing in the two-launch
    form) gives the bits of the full pass, in either form."""
    vl, bc, bl = [900, 300], [3, 2], [70, 129, 1, 64, 200]
    H, d = 2, 64
    plan = la.pack(vl, bc, bl, heads=H, block_chunks=2)
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(np.random.default_rng(77), T, H, d, "bf16")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_full, f_full = la.scan_packed(qd, kd, vd, plan, form=form)
    ws = la.new_workspace(plan, H, d, la.LA_BF16, DEV)
    out = torch.full_like(o_full, float("nan"))
    fin = torch.full_like(f_full, float("nan"))
    for stage in (la.STAGE_STATES, la.STAGE_PREFIX, la.STAGE_OUTPUT):
        la.scan_packed(qd, kd, vd, plan, out=out, final_state=fin, workspace=ws, stages=stage,
                       form=form)
    torch.cuda.synchronize()
    assert torch.equal(out, o_full) and torch.equal(fin, f_full)
