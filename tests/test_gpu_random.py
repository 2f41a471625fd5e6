"""Randomised pass structures on the GPU, against the fp64 oracles: request
counts, view and branch lengths (including 1 and chunk-boundary lengths),
shard requests seeded from external states, block sizes G, dtypes and head
dims drawn from a fixed seed, so every run checks the same 24 + 12 cases.
Each scan case also runs in both forms (two and three launches), which must
agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-3, "bf16": 2e-2}
EDGE_LENS = [1, 2, 63, 64, 65, 127, 128, 129]


def _length(rng, hi):
    return int(rng.choice(EDGE_LENS)) if rng.random() < 0.3 else int(rng.integers(1, hi + 1))


def _structure(rng, shards=True):
    n_req = int(rng.integers(1, 6))
    vl, bc, bl = [], [], []
    for _ in range(n_req):
        shard = shards and rng.random() < 0.2
        vl.append(0 if shard else _length(rng, 700))
        n = int(rng.integers(1 if shard else 0, 6))
        bc.append(n)
        bl += [_length(rng, 200) for _ in range(n)]
    return vl, bc, bl


def _case(i):
    rng = np.random.default_rng(7000 + i)
    vl, bc, bl = _structure(rng)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    d = 64 if rng.random() < 0.7 else 128
    H = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 5, 8]))
    return rng, vl, bc, bl, dtype, d, H, G


@pytest.mark.parametrize("i", range(24))
def test_random_scan(i):
    rng, vl, bc, bl, dtype, d, H, G = _case(i)
    split = dtype == "f32" and rng.random() < 0.5
    plan = la.pack(vl, bc, bl, heads=H, block_chunks=G)
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(rng, T, H, d, dtype)
    n_ext = plan.info.n_ext
    ext = (torch.from_numpy(rng.standard_normal((n_ext, H, d, d)).astype(np.float32))
           if n_ext else None)
    print(f"case {i}: views {vl} branches {bc} T={T} {dtype} d={d} H={H} G={G} "
          f"ext={n_ext} split={split}", flush=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ed = None if ext is None else ext.to(DEV)
    out, fin = la.scan_packed(qd, kd, vd, plan, ext_state=ed, split_fp32=split)
    # every form of the scan (one launch on the piece path; two launches; three
    # with the prefix launch) gives the same bits as the one the library picked
    forms = ("one", "two", "three") if (dtype == "bf16" and d == 64) else ("two", "three")
    for form in forms:
        o_f, f_f = la.scan_packed(qd, kd, vd, plan, ext_state=ed, split_fp32=split, form=form)
        assert torch.equal(o_f, out) and torch.equal(f_f, fin), form
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                          ext_state=ext)
    eo = oracle.row_rel_err(out.cpu(), ref_o)
    ef = oracle.state_rel_err(fin.cpu(), ref_f) if plan.info.n_views else 0.0
    print(f"  out err {eo:.2e} final err {ef:.2e}", flush=True)
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("i", range(4))
def test_random_scan_d128_large_blocks(i):
    """d = 128 at the large block sizes the library picks for long passes
    (G = 16 and 64), random structures with shard requests, all three forms
    equal bit for bit and within tolerance of the oracle."""
    rng = np.random.default_rng(7500 + i)
    vl, bc, bl = _structure(rng)
    vl = [x * 6 if x else 0 for x in vl]          # views long enough for several blocks
    G = (16, 64)[i % 2]
    H = 2
    plan = la.pack(vl, bc, bl, heads=H, block_chunks=G)
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(rng, T, H, 128, "bf16")
    n_ext = plan.info.n_ext
    ext = (torch.from_numpy(rng.standard_normal((n_ext, H, 128, 128)).astype(np.float32))
           if n_ext else None)
    print(f"case {i}: views {vl} branches {bc} T={T} G={G} ext={n_ext}", flush=True)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ed = None if ext is None else ext.to(DEV)
    out, fin = la.scan_packed(qd, kd, vd, plan, ext_state=ed)
    for form in ("two", "three"):
        o_f, f_f = la.scan_packed(qd, kd, vd, plan, ext_state=ed, form=form)
        assert torch.equal(o_f, out) and torch.equal(f_f, fin), form
    torch.cuda.synchronize()
    ref_o, ref_f = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent,
                                          ext_state=ext)
    eo = oracle.row_rel_err(out.cpu(), ref_o)
    ef = oracle.state_rel_err(fin.cpu(), ref_f) if plan.info.n_views else 0.0
    print(f"  out err {eo:.2e} final err {ef:.2e}", flush=True)
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("i", range(12))
def test_random_attention(i):
    rng = np.random.default_rng(8000 + i)
    vl, bc, bl = _structure(rng, shards=False)
    d = 64 if rng.random() < 0.6 else 128
    H = int(rng.integers(1, 4))
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    # one extra shard branch per case, reading an external view
    ext_len = [_length(rng, 300)]
    so = np.concatenate([so, [so[-1] + _length(rng, 150)]])
    bp = np.concatenate([bp, [-2]])
    T = int(so[-1])
    q, k, v = synth.draw_qkv(rng, T, H, d, "bf16")
    ek, ev, _ = synth.draw_qkv(rng, ext_len[0], H, d, "bf16")
    scale = float(rng.uniform(0.3, 3.0))
    print(f"case {i}: views {vl} branches {bc} + shard, T={T} d={d} H={H} scale={scale:.2f}",
          flush=True)
    plan = la.attn_plan(so, bp, ext_len)
    out = la.attn_packed(q.to(DEV), k.to(DEV), v.to(DEV), plan, scale, ext_k=ek.to(DEV),
                         ext_v=ev.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attention_dense(q, k, v, so, bp, scale, ext_kv=[(ek, ev)])
    err = oracle.row_rel_err(out.cpu(), ref)
    print(f"  err {err:.2e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_request_order_does_not_change_results(dtype):
    """Section "Kernels" ("one scan covers every view in a pass"): a request's
    outputs and final state are the same, bit for bit, whatever its position
    in the pass (same block size, so every sum runs in the same order)."""
    rng = np.random.default_rng(77)
    reqs = [(300, [40, 1, 129]), (65, [64]), (0, [70, 3]), (1000, []), (128, [1, 1])]
    H, d, G = 2, 64, 2
    data = []
    for v_len, bls in reqs:
        T = v_len + sum(bls)
        data.append(synth.draw_qkv(rng, T, H, d, dtype))
    ext = torch.from_numpy(rng.standard_normal((1, H, d, d)).astype(np.float32)).to(DEV)

    def run(order):
        vl = [reqs[r][0] for r in order]
        bc = [len(reqs[r][1]) for r in order]
        bl = [x for r in order for x in reqs[r][1]]
        plan = la.pack(vl, bc, bl, heads=H, block_chunks=G)
        q, k, v = (torch.cat([data[r][i] for r in order]).to(DEV) for i in range(3))
        out, fin = la.scan_packed(q, k, v, plan, ext_state=ext)
        torch.cuda.synchronize()
        # per request: its token range and its view row
        res, t, row = {}, 0, 0
        for r in order:
            n = reqs[r][0] + sum(reqs[r][1])
            f = None
            if reqs[r][0] > 0:
                f = fin[row].cpu()
                row += 1
            res[r] = (out[t:t + n].cpu(), f)
            t += n
        return res

    a = run([0, 1, 2, 3, 4])
    b = run([3, 2, 4, 0, 1])
    for r in range(len(reqs)):
        assert torch.equal(a[r][0], b[r][0]), f"request {r} outputs differ"
        if a[r][1] is not None:
            assert torch.equal(a[r][1], b[r][1]), f"request {r} final state differs"
