"""Branch shards from a cached view state (section "Long Requests" of the
page): a request's branches split into shards, the first shard scores the
view and stores its state in a ViewStateCache, the others run branch-only
passes seeded from the cache pool.  Checked bit for bit against the unsplit
pass (same block size G, so every state is summed in the same order) and
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
import chunked_linear_attention_packed_amd as la

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-3, "bf16": 2e-2}


def _request(seed, view, n_br, H, d, dtype):
    rng = np.random.default_rng(seed)
    lens = rng.integers(20, 151, size=n_br).astype(np.int32)
    T = view + int(lens.sum())
    q, k, v = synth.draw_qkv(rng, T, H, d, dtype)
    return lens, q, k, v


def _scan(q, k, v, plan, ext=None):
    out, fin = la.scan_packed(q.to(DEV), k.to(DEV), v.to(DEV), plan, ext_state=ext)
    torch.cuda.synchronize()
    return out.cpu(), fin


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_shards_from_cache_match_unsplit(dtype, d):
    H, G, view, n_br, shards = 4, 2, 700, 12, 3
    lens, q, k, v = _request(11, view, n_br, H, d, dtype)
    off = np.concatenate([[0], np.cumsum(np.concatenate([[view], lens]))])   # segment offsets
    print(f"shards {dtype} d={d}: view {view}, branches {list(lens)}", flush=True)

    plan_u = la.pack([view], [n_br], lens, heads=H, block_chunks=G)
    out_u, fin_u = _scan(q, k, v, plan_u)

    cache = la.ViewStateCache(4, H, d, DEV)
    parts = np.array_split(np.arange(n_br), shards)
    ref_states = oracle.scan_recurrence(q[:view], k[:view], v[:view], np.array([0, view]),
                                        np.array([-1]))[1]
    for s, idx in enumerate(parts):
        b0, b1 = idx[0], idx[-1] + 1
        t0, t1 = off[1 + b0], off[1 + b1]           # tokens of these branches
        if s == 0:
            sel = np.r_[0:view, t0:t1]
            plan = la.pack([view], [len(idx)], lens[b0:b1], heads=H, block_chunks=G)
            out, fin = _scan(q[sel], k[sel], v[sel], plan)
            row = cache.store(42, fin, 0)
            torch.cuda.synchronize()
            # the cached row is the unsplit pass's view state, bit for bit
            assert torch.equal(cache.pool[row].cpu(), fin_u[0].cpu())
            got = out[view:]
        else:
            row = cache.lookup(42)
            assert row is not None
            plan = la.pack([0], [len(idx)], lens[b0:b1], heads=H, block_chunks=G,
                           ext_row=[row])
            out, _ = _scan(q[t0:t1], k[t0:t1], v[t0:t1], plan, ext=cache.pool)
            got = out
            # and against the oracle, seeded from the oracle's own view state
            ref, _ = oracle.scan_recurrence(q[t0:t1], k[t0:t1], v[t0:t1], plan.seg_offsets,
                                            plan.branch_parent,
                                            ext_state=np.broadcast_to(ref_states[0],
                                                                      (row + 1,) + ref_states[0].shape))
            err = oracle.row_rel_err(out, ref)
            print(f"  shard {s}: oracle err {err:.2e}", flush=True)
            assert err <= TOL[dtype]
        assert torch.equal(got, out_u[t0:t1]), f"shard {s} differs from the unsplit pass"
    cache.close()


def test_cache_eviction_and_rows_from_several_views():
    H, d, G = 2, 64, 1
    cache = la.ViewStateCache(2, H, d, DEV)
    views = {}
    for vid, (seed, L) in {7: (1, 300), 8: (2, 130), 9: (3, 450)}.items():
        rng = np.random.default_rng(seed)
        q, k, v = synth.draw_qkv(rng, L, H, d, "bf16")
        plan = la.pack([L], [0], [], heads=H, block_chunks=G)
        _, fin = _scan(q, k, v, plan)
        row, ev = cache.reserve(vid)
        la.export_view_state(fin, 0, cache.pool[row])
        views[vid] = (fin.clone(), row, ev)
    torch.cuda.synchronize()
    assert views[7][2] is None and views[8][2] is None and views[9][2] == 7
    assert cache.lookup(7) is None and len(cache) == 2
    for vid in (8, 9):
        assert torch.equal(cache.pool[cache.lookup(vid)], views[vid][0][0])
    # one pass: a shard of view 9, a normal request, a shard of view 8
    r8, r9 = cache.lookup(8), cache.lookup(9)
    blen = [40, 70, 5, 64, 100]
    plan = la.pack([0, 90, 0], [2, 1, 2], blen, heads=H, block_chunks=G, ext_row=[r9, 0, r8])
    T = plan.info.n_tokens
    q, k, v = synth.draw_qkv(np.random.default_rng(5), T, H, d, "bf16")
    out, _ = _scan(q, k, v, plan, ext=cache.pool)
    ext = cache.pool.cpu().numpy()
    ref, _ = oracle.scan_recurrence(q, k, v, plan.seg_offsets, plan.branch_parent, ext_state=ext)
    err = oracle.row_rel_err(out, ref)
    print(f"mixed shard pass err {err:.2e}", flush=True)
    assert err <= TOL["bf16"]
    cache.close()
