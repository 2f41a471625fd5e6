"""GPU parity of the HIP scan against the fp64 CPU oracle.

Everything here runs through the C ABI (via the ctypes binding) on an MI355X.
Tolerances, row-normalised max relative error (oracle.metrics): 1e-3 for fp32
inputs, 2e-2 for bf16 inputs.  Integer-valued probes are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import oracle_pool
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}
DEV = "cuda:0"


def _run(q, k, v, plan, ext=None):
    qd, kd, vd = (x.to(DEV).contiguous() for x in (q, k, v))
    ed = None if ext is None else ext.to(DEV).contiguous()
    out, fin = la.scan_packed(qd, kd, vd, plan, ext_state=ed)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


def _dtype_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def _check_full(q, k, v, plan, ext=None, tol=None):
    out, fin = _run(q, k, v, plan, ext)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                          ext_state=ext)
    tol = TOL[_dtype_name(q)] if tol is None else tol
    eo = oracle.row_rel_err(out, ref_o)
    ef = oracle.state_rel_err(fin, ref_f)
    print(f"  out err {eo:.3e}  final err {ef:.3e}  (tol {tol})", flush=True)
    assert eo <= tol
    assert ef <= tol
    return out, fin


@pytest.mark.parametrize("name", [n for n in synth.WORKLOADS if not n.startswith("req32")])
def test_workload_full_parity(name):
    """Workloads 1-4 compared with the full oracle recurrence, in the block
    configuration the benchmark uses (the binding's default)."""
    w = synth.workload(name)
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    print(f"{name}: T={w.n_tokens} G={plan.info.block_chunks} blocks={plan.info.n_blocks}",
          flush=True)
    _check_full(w.q, w.k, w.v, plan)


def _req32_worker(r):
    """Request r of the 32-request pass against the pinned chunked fp64
    evaluator (oracle.scan_chunked, pinned equal to the recurrence): the
    row-normalised error of its output rows and of its view's final state."""
    sh = oracle_pool.SHARED
    a, b = sh["tok"][r]
    so_r, bp_r = sh["tables"][r]
    ref_o, ref_f = oracle.scan_chunked(sh["q"][a:b], sh["k"][a:b], sh["v"][a:b], so_r, bp_r, 64)
    eo = oracle.row_rel_err(sh["out"][a:b], ref_o)
    ef = oracle.state_rel_err(sh["fin"][sh["vrow"][r]][None], ref_f)
    return eo, ef, int(b - a)


def test_workload_req32_full_parity():
    """The 32-request d=128 pass (272,142 tokens, H = 32) at full size, in the
    benchmark's block configuration, compared element by element with the
    fp64 oracle: every output row of every head and every view's final
    state.  The pass is split by request (requests share nothing) and each
    request's error is taken with its own normalisation floor, which is at
    most the whole array's, so the largest per-request error bounds the
    whole-pass error from above."""
    name = "req32_view500-18000_br1-64x24-128_h32_d128_bf16"
    w = synth.workload(name)
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    print(f"{name}: T={w.n_tokens} G={plan.info.block_chunks} blocks={plan.info.n_blocks}",
          flush=True)
    out, fin = _run(w.q, w.k, w.v, plan)
    so, bp = plan.seg_offsets, plan.branch_parent
    tok, tables, vrow = [], [], []
    s = 0
    for r in range(len(w.view_len)):
        nseg = 1 + int(w.branch_count[r])
        a, b = int(so[s]), int(so[s + nseg])
        sub_bp = [-1] + [0] * (nseg - 1)
        assert bp[s] == -1 and all(int(x) == s for x in bp[s + 1:s + nseg])
        tok.append((a, b))
        tables.append((np.asarray(so[s:s + nseg + 1]) - a, np.asarray(sub_bp)))
        vrow.append(int(plan.view_ordinal[s]))
        s += nseg
    assert s == len(bp)
    shared = dict(q=oracle_pool.to_f32(w.q), k=oracle_pool.to_f32(w.k),
                  v=oracle_pool.to_f32(w.v), out=oracle_pool.to_f32(out),
                  fin=fin.numpy(), tok=tok, tables=tables, vrow=vrow)
    res = oracle_pool.run(_req32_worker, list(range(len(tok))), shared)
    eo = max(r[0] for r in res)
    ef = max(r[1] for r in res)
    assert sum(r[2] for r in res) == w.n_tokens
    print(f"  all {w.n_tokens} rows x {w.H} heads: out err {eo:.3e}  final err {ef:.3e} "
          f"({oracle_pool.workers()} workers)", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


def _random_pass(seed, n_req, view_lens, n_br, br_lens, H, d, dtype):
    rng = np.random.default_rng(seed)
    vl = np.asarray(view_lens)
    bc = np.asarray(n_br)
    bl = np.asarray(br_lens)
    T = int(vl.sum() + bl.sum())
    q, k, v = synth.draw_qkv(rng, T, H, d, dtype)
    return vl, bc, bl, q, k, v


EDGE = [
    # view lengths, branch counts, branch lengths
    ([1], [0], []),
    ([63], [2], [1, 64]),
    ([64], [3], [63, 65, 1]),
    ([65], [1], [127]),
    ([127, 128], [2, 2], [128, 129, 1, 2]),
    ([200, 1, 640], [0, 3, 1], [64, 64, 5, 300]),
]


@pytest.mark.parametrize("dtype,d,G", [(dt, d, G) for dt, d in (("f32", 64), ("bf16", 64),
                                                                  ("bf16", 128), ("f32", 128))
                                         for G in (1, 2, 3, 8)] +
                         [("bf16", 128, 16), ("bf16", 128, 64), ("bf16", 64, 16)])
@pytest.mark.parametrize("case", range(len(EDGE)))
def test_edge_lengths(dtype, d, G, case):
    vl, bc, bl = EDGE[case]
    vl, bc, bl, q, k, v = _random_pass(100 + case, 0, vl, bc, bl, 3, d, dtype)
    plan = la.pack(vl, bc, bl, block_chunks=G)
    _check_full(q, k, v, plan)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_segments_in_any_order(dtype):
    """Branches listed before their view, views interleaved."""
    rng = np.random.default_rng(5)
    lens = [37, 150, 300, 20, 90, 3]
    bp = [2, 2, -1, 2, -1, 4]
    so = np.r_[0, np.cumsum(lens)]
    q, k, v = synth.draw_qkv(rng, int(so[-1]), 2, 64, dtype)
    plan = la.plan_segments(so, bp, block_chunks=2)
    _check_full(q, k, v, plan)


@pytest.mark.parametrize("G", [1, 4])
def test_exact_indexing_probe(G):
    """q = k = e_0 and v = one-hot segment code (fp32): every output is an
    integer < 2^24, so the result must equal the closed form bit for bit.  A
    misrouted row, wrong parent, chunk-edge slip or sibling leak breaks it.
    Passes with more segments than d run a second probe on the next digit."""
    name = "view18000_br256x32-128_h16_d64_bf16"
    vl, bc, bl = synth.shapes(name)
    plan = la.pack(vl, bc, bl, block_chunks=G)
    so, bp = plan.seg_offsets, plan.branch_parent
    H, d = 2, 64
    n_seg = len(bp)
    for digit in range(2 if n_seg > d else 1):
        q, k, v = synth.probe_qkv(so, bp, H, d, digit)
        out, fin = _run(q, k, v, plan)
        exp = np.zeros((int(so[-1]), d), dtype=np.float64)
        for s in range(n_seg):
            a, b = int(so[s]), int(so[s + 1])
            code = (s // d ** digit) % d
            exp[a:b, code] += np.arange(1, b - a + 1)
            p = int(bp[s])
            if p >= 0:
                pcode = (p // d ** digit) % d
                exp[a:b, pcode] += int(so[p + 1] - so[p])
        for h in range(H):
            assert np.array_equal(out[:, h].double().numpy(), exp), f"digit {digit} head {h}"
        # final state of the view: row 0 of S holds the code counts
        f_exp = np.zeros((d,))
        f_exp[(0 // d ** digit) % d] = int(so[1])
        assert np.array_equal(fin[0, 0, 0].double().numpy(), f_exp)
        assert bool(torch.all(fin[0, :, 1:] == 0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ternary_inputs_are_exact(dtype):
    """q, k, v in {-1, 0, 1}: every partial sum is an integer below 2^24.  The
    fp32 path must equal the oracle exactly; the bf16 path (state split into
    two bf16 terms, scores exact in bf16) must equal the oracle's value
    rounded to bf16, bit for bit."""
    vl, bc, bl = [3000, 700], [5, 2], [64, 100, 1, 128, 65, 77, 3]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.ternary_qkv(9, int(so[-1]), 4, 64, dtype)
    plan = la.pack(vl, bc, bl, block_chunks=2)
    out, fin = _run(q, k, v, plan)
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, so, bp)
    assert np.abs(ref_o).max() < 2 ** 24
    exp = torch.from_numpy(ref_o).to(q.dtype)
    assert torch.equal(out, exp)
    assert torch.equal(fin.double(), torch.from_numpy(ref_f))


def test_deterministic():
    w = synth.workload("view7400_br8x48_h16_d64_bf16")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    o1, f1 = _run(w.q, w.k, w.v, plan)
    o2, f2 = _run(w.q, w.k, w.v, plan)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_branch_alone_equals_packed(dtype):
    """Section "The Workload": a branch never sees its siblings, so scoring
    {view, one branch} gives that branch's rows of the full pass exactly (the
    view's blocks are identical in both passes)."""
    vl, bc, bl = [1000], [6], [30, 64, 100, 1, 129, 50]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(3), int(so[-1]), 2, 64, dtype)
    plan = la.pack(vl, bc, bl, block_chunks=2)
    out, fin = _run(q, k, v, plan)
    for b in range(6):
        a0, a1 = int(so[1 + b]), int(so[2 + b])
        idx = np.r_[0:1000, a0:a1]
        p1 = la.pack([1000], [1], [bl[b]], block_chunks=2)
        o1, f1 = _run(q[idx], k[idx], v[idx], p1)
        assert torch.equal(o1[1000:], out[a0:a1])
        assert torch.equal(o1[:1000], out[:1000])
        assert torch.equal(f1, fin)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shard_pass_from_exported_state(dtype):
    """Section "Long Requests": view-only pass, export the view state, then
    branch-only shard passes seeded from it reproduce the branch rows of the
    unsharded pass exactly, and match the oracle."""
    name = "view18000_br256x32-128_h16_d64_bf16"
    vl, bc, bl = synth.shapes(name)
    H, d = 4, 64
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(44), int(so[-1]), H, d, dtype)
    full = la.pack(vl, bc, bl, block_chunks=4)
    out, fin = _run(q, k, v, full)
    L = int(vl[0])
    vplan = la.pack(vl, [0], [], block_chunks=4)
    qd, kd, vd = (x[:L].to(DEV).contiguous() for x in (q, k, v))
    _, vfin = la.scan_packed(qd, kd, vd, vplan)
    ext = torch.empty((1, H, d, d), dtype=torch.float32, device=DEV)
    la.export_view_state(vfin, 0, dst=ext[0])
    torch.cuda.synchronize()
    assert torch.equal(ext.cpu(), fin)
    bounds = [0, 64, 128, 192, 256]
    for i in range(4):
        b0, b1 = bounds[i], bounds[i + 1]
        t0, t1 = int(so[1 + b0]), int(so[1 + b1])
        splan = la.pack([0], [b1 - b0], bl[b0:b1], block_chunks=4)
        o, f = _run(q[t0:t1], k[t0:t1], v[t0:t1], splan, ext=ext.cpu())
        assert f.shape[0] == 0
        assert torch.equal(o, out[t0:t1])
    ref = oracle.sample_rows(q, k, v, so, bp, list(range(L, int(so[-1]), 97)))
    assert oracle.row_rel_err(out[L::97], ref) <= TOL[dtype]


def test_q_zero_gives_zero_output_but_states():
    vl, bc, bl = [300], [2], [40, 70]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.draw_qkv(np.random.default_rng(8), int(so[-1]), 2, 64, "bf16")
    q = torch.zeros_like(q)
    plan = la.pack(vl, bc, bl, block_chunks=1)
    out, fin = _run(q, k, v, plan)
    assert torch.all(out == 0)
    _, ref_f = oracle.scan_recurrence(q, k, v, so, bp)
    assert oracle.state_rel_err(fin, ref_f) <= 1e-5


def test_outputs_fully_overwritten():
    """Idempotence: out and final_state are written everywhere, whatever they
    held before."""
    w = synth.workload("view500_br4x32_h2_d64_f32")
    plan = la.pack(w.view_len, w.branch_count, w.branch_len, heads=w.H)
    qd, kd, vd = (x.to(DEV) for x in (w.q, w.k, w.v))
    o1 = torch.full((w.n_tokens, w.H, w.d), float("nan"), device=DEV)
    f1 = torch.full((1, w.H, w.d, w.d), float("nan"), device=DEV)
    la.scan_packed(qd, kd, vd, plan, out=o1, final_state=f1)
    o2, f2 = la.scan_packed(qd, kd, vd, plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype,d,split", [("bf16", 64, False), ("bf16", 128, False),
                                           ("f32", 64, False), ("f32", 64, True)])
def test_long_prefix_chains(dtype, d, split):
    """More than 32 workspace slots in one segment (launch 2 sums them in
    batches of 32): a view of 70 full chunks and a branch of 40 chunks plus a
    ragged tail, one chunk per work block, so the view's chain has 70 slots
    and the branch's 40."""
    H = 2
    vl, bc, bl = [70 * 64], [2], [40 * 64 + 17, 5]
    plan = la.pack(vl, bc, bl, heads=H, block_chunks=1)
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(np.random.default_rng(77 + d), T, H, d, dtype)
    print(f"long chains {dtype} d={d} split={split}: T={T} delta slots={plan.info.n_delta}",
          flush=True)
    out, fin = la.scan_packed(q.to(DEV), k.to(DEV), v.to(DEV), plan, split_fp32=split)
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent)
    eo = oracle.row_rel_err(out.cpu(), ref_o)
    ef = oracle.state_rel_err(fin.cpu(), ref_f)
    print(f"  out err {eo:.3e}  final err {ef:.3e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
