"""The single-launch form of the piece path (d = 64, bf16) on the GPU: its
bounded waits, the state it keeps in the workspace between passes, graph
replays, long look-back chains, and the device-side plan check of every
form.  Results are compared with the three-launch form (bit for bit) and the
fp64 oracle (row-normalised max relative error <= 2e-2)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def _inputs(vl, bc, bl, H, seed, dtype="bf16", d=64):
    plan = la.pack(vl, bc, bl, heads=H)
    q, k, v = synth.draw_qkv(np.random.default_rng(seed), plan.info.n_tokens, H, d, dtype)
    return plan, q, k, v


def _header_words(ws, n):
    torch.cuda.synchronize()
    return ws[:4 * n].view(torch.int32).cpu().tolist()


def test_forced_timeout_exits_and_reports():
    """With every wait made to give up after a few polls (a test aid: the
    flags it polls are treated as never set), every workgroup still reaches
    the end of the kernel, the pass returns, and the workspace reports
    LA_ERR_TIMEOUT.  The counters are reset as after any pass, so the next
    normal pass on the same workspace is correct and reports nothing."""
    plan, q, k, v = _inputs([1500, 300], [3, 2], [48, 1, 100, 70, 129], 4, 11)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ws = la.new_workspace(plan, 4, 64, la.LA_BF16, DEV)
    print("forced timeout pass", flush=True)
    la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one",
                   stages=la.STAGE_ALL | la.DEBUG_FORCE_TIMEOUT)
    st = la.scan_status(ws, clear=True)
    assert st & la.LA_ERR_TIMEOUT
    words = _header_words(ws, 4)
    assert words[2] == 0 and words[3] == 0          # ticket and retire counters reset
    assert la.scan_status(ws) == 0
    out, fin = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
    o3, f3 = la.scan_packed(qd, kd, vd, plan, form="three")
    assert la.scan_status(ws) == 0
    assert torch.equal(out, o3) and torch.equal(fin, f3)


@pytest.mark.parametrize("dtype,form", [("bf16", "one"), ("bf16", "three"), ("f32", "two"),
                                        ("f32", "three")])
def test_device_plan_of_another_pass_is_refused(dtype, form):
    """A device plan uploaded for another pass with the same token count,
    given with this pass's info: the kernels see the plan's hash differ from
    the info's, do no work (outputs keep their sentinel) and record
    LA_ERR_PLAN in the workspace."""
    a = la.pack([100], [2], [10, 20], heads=2)
    b = la.pack([120], [1], [10], heads=2)
    assert a.info.n_tokens == b.info.n_tokens and a.info.plan_hash != b.info.plan_hash
    mixed = la.PassPlan(b.info, b.seg_offsets, b.branch_parent, b.view_ordinal, a.plan)
    q, k, v = synth.draw_qkv(np.random.default_rng(3), b.info.n_tokens, 2, 64, dtype)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    code = la.LA_BF16 if dtype == "bf16" else la.LA_F32
    ws = la.new_workspace(b, 2, 64, code, DEV)
    out = torch.full((b.info.n_tokens, 2, 64), float("nan"), dtype=qd.dtype, device=DEV)
    fin = torch.full((b.info.n_views, 2, 64, 64), float("nan"), device=DEV)
    la.scan_packed(qd, kd, vd, mixed, out=out, final_state=fin, workspace=ws, form=form)
    assert la.scan_status(ws) == la.LA_ERR_PLAN
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(fin).all())
    # the right plan on the same workspace works (after clearing the status)
    la.scan_status(ws, clear=True)
    o, f = la.scan_packed(qd, kd, vd, b, out=out, final_state=fin, workspace=ws, form=form)
    assert la.scan_status(ws) == 0
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, b.seg_offsets, b.branch_parent)
    tol = TOL if dtype == "bf16" else 1e-3
    assert oracle.row_rel_err(o.cpu(), ref_o) <= tol
    assert oracle.state_rel_err(f.cpu(), ref_f) <= tol


def test_repeated_passes_reset_their_state():
    """Passes of different shapes in a row on one workspace: each leaves the
    header counters and the flags at zero, and each equals the three-launch
    form on its own inputs."""
    shapes = [([7400], [8], [48] * 8, 16), ([300, 2000], [2, 1], [5, 600, 64], 4),
              ([7400], [8], [48] * 8, 16), ([64], [1], [1], 2)]
    H_max = 16
    big = [la.pack(vl, bc, bl, heads=H) for vl, bc, bl, H in shapes]
    n = max(la.workspace_size(p, H, 64, la.LA_BF16) for p, (_, _, _, H) in zip(big, shapes))
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    for i, (plan, (vl, bc, bl, H)) in enumerate(zip(big, shapes)):
        q, k, v = synth.draw_qkv(np.random.default_rng(20 + i), plan.info.n_tokens, H, 64,
                                 "bf16")
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        o1, f1 = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
        o3, f3 = la.scan_packed(qd, kd, vd, plan, form="three")
        assert torch.equal(o1, o3) and torch.equal(f1, f3), i
        words = _header_words(ws, 4)
        assert words == [0, 0, 0, 0], (i, words)
        nflag = plan.info.piece_slots * H
        flags = ws[256:256 + 8 * nflag]
        assert int(flags.count_nonzero()) == 0, i
    assert H_max == 16


def test_graph_replays_match_eager():
    """The single launch captured in a HIP graph and replayed several times,
    with eager work and synchronisations between the replays: every replay
    gives the eager result (the form records no memset; it resets its own
    counters and flags)."""
    w = synth.workload("view7400_br8x48_h16_d64_bf16")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    qd, kd, vd = (x.to(DEV) for x in (w.q, w.k, w.v))
    ws = la.new_workspace(plan, w.H, w.d, la.LA_BF16, DEV)
    ref_o, ref_f = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
    ref_o, ref_f = ref_o.clone(), ref_f.clone()
    out = torch.empty_like(ref_o)
    fin = torch.empty_like(ref_f)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        la.scan_packed(qd, kd, vd, plan, out=out, final_state=fin, workspace=ws, form="one",
                       stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        la.scan_packed(qd, kd, vd, plan, out=out, final_state=fin, workspace=ws, form="one",
                       stream=s)
    for r in range(4):
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(fin, ref_f), r
        # eager work between replays (another pass on its own workspace)
        la.scan_packed(qd, kd, vd, plan, form="three")
        torch.cuda.synchronize()
    assert la.scan_status(ws) == 0


@pytest.mark.parametrize("H", [1, 3])
def test_long_chains(H):
    """Views of 40 and 23 blocks (one head, or three): each block's look-back
    walks up to 39 predecessors; a branch of 5 blocks starts from the long
    view's total and looks back along its own chain.  All forms bit-identical,
    oracle within tolerance."""
    vl, bc, bl = [40 * 512 - 7, 23 * 512], [2, 1], [5 * 512 - 100, 30, 64]
    plan, q, k, v = _inputs(vl, bc, bl, H, 31)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, f1 = la.scan_packed(qd, kd, vd, plan, form="one")
    o2, f2 = la.scan_packed(qd, kd, vd, plan, form="two")
    o3, f3 = la.scan_packed(qd, kd, vd, plan, form="three")
    assert torch.equal(o1, o3) and torch.equal(f1, f3)
    assert torch.equal(o2, o3) and torch.equal(f2, f3)
    ref_o, ref_f = oracle.scan_chunked(q, k, v, plan.seg_offsets, plan.branch_parent, 64)
    eo = oracle.row_rel_err(o1.cpu(), ref_o)
    ef = oracle.state_rel_err(f1.cpu(), ref_f)
    print(f"long chains H={H}: blocks={plan.info.piece_blocks} out err {eo:.2e} final {ef:.2e}",
          flush=True)
    assert eo <= TOL and ef <= TOL


def test_single_launch_is_deterministic():
    """Ten single-launch passes of the 7,400-token pass give the same bits:
    the look-back adds predecessors left to right whatever prefix it finds."""
    w = synth.workload("view7400_br8x48_h16_d64_bf16")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    qd, kd, vd = (x.to(DEV) for x in (w.q, w.k, w.v))
    ws = la.new_workspace(plan, w.H, w.d, la.LA_BF16, DEV)
    o0, f0 = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
    o0, f0 = o0.clone(), f0.clone()
    for _ in range(9):
        o, f = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
        assert torch.equal(o, o0) and torch.equal(f, f0)


def test_ordered_tickets_match_index_order():
    """The single launch with the work taken in ticket order (forced; the
    library takes tickets only when the launch does not fit on the device at
    once) gives the bits of the launch that uses the workgroup index, on the
    7,400-token pass (256 workgroups) and on a pass larger than the device."""
    for name in ("view7400_br8x48_h16_d64_bf16", None):
        if name:
            w = synth.workload(name)
            plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
            q, k, v, H = w.q, w.k, w.v, w.H
        else:
            H = 16
            plan, q, k, v = _inputs([20000, 3000], [6, 3], [48, 64, 1, 130, 500, 2, 64, 64, 9],
                                    H, 41)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ws = la.new_workspace(plan, H, 64, la.LA_BF16, DEV)
        print(f"ordered vs index: workgroups={plan.info.piece_items * H}", flush=True)
        o1, f1 = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
        o1, f1 = o1.clone(), f1.clone()
        o2, f2 = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one",
                                stages=la.STAGE_ALL | la.DEBUG_ORDERED)
        o3, f3 = la.scan_packed(qd, kd, vd, plan, form="three")
        assert la.scan_status(ws) == 0
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
        assert torch.equal(o1, o3) and torch.equal(f1, f3)
        assert _header_words(ws, 4) == [0, 0, 0, 0]


def test_packed_short_branches_share_waves():
    """Branches of at most one chunk are packed two to a wave, with seeds
    from different views and from ext_state rows in one wave (the second
    branch reloads its own seed), next to branches of two chunks that take a
    wave alone: all forms bit-identical, oracle within tolerance."""
    vl = [300, 0, 700, 64, 0]
    bc = [3, 2, 4, 2, 2]
    bl = [10, 64, 1, 33, 128, 5, 100, 64, 63, 2, 65, 17, 40]
    H = 3
    plan = la.pack(vl, bc, bl, heads=H)
    P = plan.plan
    oi = int(P[21])
    nbi, ni = plan.info.piece_block_items, plan.info.piece_items
    items = P[oi:oi + 12 * ni].reshape(-1, 12)
    pairs = sum(1 for row in items[nbi:] for w in range(row[1]) if row[3 + 2 * w] != -1)
    assert pairs >= 3
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(np.random.default_rng(57), T, H, 64, "bf16")
    ext = torch.from_numpy(np.random.default_rng(58).standard_normal(
        (plan.info.n_ext, H, 64, 64)).astype(np.float32))
    qd, kd, vd, ed = q.to(DEV), k.to(DEV), v.to(DEV), ext.to(DEV)
    outs = {f: la.scan_packed(qd, kd, vd, plan, ext_state=ed, form=f)
            for f in ("one", "two", "three")}
    for f in ("one", "two"):
        assert torch.equal(outs[f][0], outs["three"][0]), f
        assert torch.equal(outs[f][1], outs["three"][1]), f
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                          ext_state=ext)
    eo = oracle.row_rel_err(outs["one"][0].cpu(), ref_o)
    ef = oracle.state_rel_err(outs["one"][1].cpu(), ref_f)
    print(f"packed short branches: pairs={pairs} out err {eo:.2e} final {ef:.2e}", flush=True)
    assert eo <= TOL and ef <= TOL


def test_alternating_inputs_on_one_workspace():
    """Passes over two different input sets, alternating on one workspace:
    every state slot is rewritten with other values at the same address each
    pass, so a look-back that read a stale cached copy of a slot (from the
    pass before) would change the bits.  Each pass must equal the three-
    launch form on its own inputs."""
    w = synth.workload("view7400_br8x48_h16_d64_bf16")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    sets = []
    for seed in (71, 72):
        q, k, v = synth.draw_qkv(np.random.default_rng(seed), plan.info.n_tokens, w.H, 64,
                                 "bf16")
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        ref = la.scan_packed(qd, kd, vd, plan, form="three")
        sets.append((qd, kd, vd, ref))
    ws = la.new_workspace(plan, w.H, 64, la.LA_BF16, DEV)
    for i in range(8):
        qd, kd, vd, (ro, rf) = sets[i % 2]
        o, f = la.scan_packed(qd, kd, vd, plan, workspace=ws, form="one")
        assert torch.equal(o, ro) and torch.equal(f, rf), i
    assert la.scan_status(ws) == 0
