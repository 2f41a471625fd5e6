"""The view cache holding both the linear-attention state and the K/V of the
softmax layers (section "Long Requests": CUDA nodes cache a view's state and
its softmax K/V so that branch shards skip the view).  A request's branches
are split into shards: the first scores the view and stores its state and
K/V in a ViewStateCache; later shards are branch-only passes whose linear
layer starts from the cached state (ext_state) and whose softmax layer
attends to the cached K/V (pool regions named by attn_plan's ext_start).
Both layers' shard outputs must equal the unsplit pass bit for bit (same
kernels, same key order) and match the fp64 oracles."""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2


def _request(seed, view, n_br, H, d):
    rng = np.random.default_rng(seed)
    lens = rng.integers(20, 151, size=n_br).astype(np.int32)
    T = view + int(lens.sum())
    q, k, v = synth.draw_qkv(rng, T, H, d, "bf16")
    return lens, q, k, v


def _layers(q, k, v, plan, ext_state=None, attn=None, ext_kv=None):
    """Both layer types of one pass: the scan and the softmax attention."""
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, fin = la.scan_packed(qd, kd, vd, plan, ext_state=ext_state)
    if attn is None:
        attn = la.attn_plan(plan.seg_offsets, plan.branch_parent)
    ek, ev = ext_kv if ext_kv is not None else (None, None)
    att = la.attn_packed(qd, kd, vd, attn, 1.0, ext_k=ek, ext_v=ev)
    torch.cuda.synchronize()
    return out.cpu(), fin, att.cpu(), (kd, vd)


@pytest.mark.parametrize("d", [64, 128])
def test_shards_from_cached_state_and_kv(d):
    H, G, view, n_br, shards = 4, 2, 700, 12, 3
    lens, q, k, v = _request(31, view, n_br, H, d)
    off = np.concatenate([[0], np.cumsum(np.concatenate([[view], lens]))])
    plan_u = la.pack([view], [n_br], lens, heads=H, block_chunks=G)
    out_u, fin_u, att_u, _ = _layers(q, k, v, plan_u)

    cache = la.ViewStateCache(3, H, d, DEV, kv_tokens=1024, kv_layers=1)
    parts = np.array_split(np.arange(n_br), shards)
    for s, idx in enumerate(parts):
        b0, b1 = idx[0], idx[-1] + 1
        t0, t1 = off[1 + b0], off[1 + b1]
        if s == 0:
            sel = np.r_[0:view, t0:t1]
            plan = la.pack([view], [len(idx)], lens[b0:b1], heads=H, block_chunks=G)
            out, fin, att, (kd, vd) = _layers(q[sel], k[sel], v[sel], plan)
            row = cache.store(77, fin, 0, kv=[(kd, vd)], view_tok0=0, view_tokens=view)
            torch.cuda.synchronize()
            got_o, got_a = out[view:], att[view:]
            a0 = row * cache.kv_tokens
            assert torch.equal(cache.kv_k[0, a0:a0 + view].cpu(), k[:view])
            assert torch.equal(cache.kv_v[0, a0:a0 + view].cpu(), v[:view])
        else:
            row, first, n = cache.kv_extent(77)
            assert n == view
            plan = la.pack([0], [len(idx)], lens[b0:b1], heads=H, block_chunks=G, ext_row=[row])
            bp_s = np.full(len(idx), -2)
            attn = la.attn_plan(plan.seg_offsets, bp_s, ext_len=[n], ext_start=[first],
                                ext_tokens=cache.kv_pool_tokens)
            got_o, _, got_a, _ = _layers(q[t0:t1], k[t0:t1], v[t0:t1], plan,
                                         ext_state=cache.pool, attn=attn,
                                         ext_kv=(cache.kv_k[0], cache.kv_v[0]))
            ref = oracle.attention_dense(q[t0:t1], k[t0:t1], v[t0:t1], plan.seg_offsets, bp_s,
                                         1.0, ext_kv=[(k[:view], v[:view])])
            err = oracle.row_rel_err(got_a, ref)
            print(f"  d={d} shard {s}: attention oracle err {err:.2e}", flush=True)
            assert err <= TOL
        assert torch.equal(got_o, out_u[t0:t1]), f"shard {s}: linear layer differs"
        assert torch.equal(got_a, att_u[t0:t1]), f"shard {s}: softmax layer differs"
    cache.close()


def test_kv_rows_of_several_views_with_eviction():
    """Three views through a two-row cache: the third evicts the least
    recent, whose K/V extent is then gone; one pass mixes a shard of each
    cached view and a normal request, and its attention matches the oracle
    given each view's own K/V."""
    H, d = 2, 64
    cache = la.ViewStateCache(2, H, d, DEV, kv_tokens=512, kv_layers=1)
    views = {}
    for vid, (seed, L) in {5: (1, 300), 6: (2, 130), 7: (3, 450)}.items():
        q, k, v = synth.draw_qkv(np.random.default_rng(seed), L, H, d, "bf16")
        plan = la.pack([L], [0], [], heads=H, block_chunks=1)
        _, fin, _, (kd, vd) = _layers(q, k, v, plan)
        cache.store(vid, fin, 0, kv=[(kd, vd)], view_tokens=L)
        views[vid] = (k, v, L)
    torch.cuda.synchronize()
    assert cache.kv_extent(5) is None and len(cache) == 2
    e7, e6 = cache.kv_extent(7), cache.kv_extent(6)
    assert e7[2] == 450 and e6[2] == 130 and e7[0] != e6[0]
    # segments: shard branches of view 7, a request (view 90 + branch), shard branch of view 6
    so = np.array([0, 40, 110, 200, 264, 364])
    bp = np.array([-2, -2, -1, 2, -3])
    T = int(so[-1])
    q, k, v = synth.draw_qkv(np.random.default_rng(9), T, H, d, "bf16")
    attn = la.attn_plan(so, bp, ext_len=[e7[2], e6[2]], ext_start=[e7[1], e6[1]],
                        ext_tokens=cache.kv_pool_tokens)
    out = la.attn_packed(q.to(DEV), k.to(DEV), v.to(DEV), attn, 1.0, ext_k=cache.kv_k[0],
                         ext_v=cache.kv_v[0])
    torch.cuda.synchronize()
    ref = oracle.attention_dense(q, k, v, so, bp, 1.0,
                                 ext_kv=[views[7][:2], views[6][:2]])
    err = oracle.row_rel_err(out.cpu(), ref)
    print(f"mixed cached views: err {err:.2e}", flush=True)
    assert err <= TOL
    cache.close()
