"""Pins for the CPU oracle: checks against things other than itself.

The oracle follows "Serving 0.88M TPS from Two RTXs and Mac Minis" (sections
"The Workload", "Kernels", "Long Requests").  The page prints no values, so the
pins are: a worked example derived by hand (tests/golden), an O(T^2) explicit
mask evaluation, a chunked evaluation at many chunk sizes, closed forms, and
the structural invariants the page states (branches never see siblings; a
branch shard seeded with the view's cached state equals the unsharded pass;
one scan over the whole pass equals one scan per view).  The last test plants
plausible mistakes in copies of the recurrence and checks that the pins catch
each of them.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_pass(rng, n_req, max_view, max_br, max_blen, H, dk, dv):
    vl = rng.integers(1, max_view, size=n_req, endpoint=True)
    bc = rng.integers(0, max_br, size=n_req, endpoint=True)
    bl = rng.integers(1, max_blen, size=int(bc.sum()), endpoint=True)
    so, bp, vo = oracle.pack_segments(vl, bc, bl)
    T = int(so[-1])
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    return (vl, bc, bl), (so, bp, vo), (q, k, v)


def _hand():
    with open(os.path.join(GOLD, "hand_worked_example.json")) as f:
        return json.load(f)


def _hand_inputs(g):
    q = np.asarray(g["q"], dtype=np.float64)[:, None, :]
    k = np.asarray(g["k"], dtype=np.float64)[:, None, :]
    v = np.asarray(g["v"], dtype=np.float64)[:, None, :]
    return q, k, v


def test_pack_matches_hand_example():
    g = _hand()
    so, bp, vo = oracle.pack_segments(g["view_len"], g["branch_count"], g["branch_len"])
    assert so.tolist() == g["seg_offsets"]
    assert bp.tolist() == g["branch_parent"]
    assert vo.tolist() == g["view_ordinal"]


@pytest.mark.parametrize("fn", ["recurrence", "bruteforce", "chunked1", "chunked2", "chunked64"])
def test_hand_worked_example(fn):
    g = _hand()
    q, k, v = _hand_inputs(g)
    so, bp = g["seg_offsets"], g["branch_parent"]
    if fn == "recurrence":
        out, fin = oracle.scan_recurrence(q, k, v, so, bp)
    elif fn == "bruteforce":
        out, fin = oracle.scan_bruteforce(q, k, v, so, bp)
    else:
        out, fin = oracle.scan_chunked(q, k, v, so, bp, int(fn[7:]))
    assert np.array_equal(out[:, 0, :], np.asarray(g["out"], dtype=np.float64))
    assert np.array_equal(fin[:, 0], np.asarray(g["final_state"], dtype=np.float64))


def test_hand_example_as_shard_pass():
    """Section "Long Requests": branches of a shard pass seeded with the cached
    view state give the same rows as inside the full pass."""
    g = _hand()
    q, k, v = _hand_inputs(g)
    # request 0's branches (tokens 3..5) alone, seeded from view0's state
    so, bp, _ = oracle.pack_segments([0], [2], [2, 1])
    ext = np.asarray(g["final_state"][0], dtype=np.float64)[None, None]
    out, fin = oracle.scan_recurrence(q[3:6], k[3:6], v[3:6], so, bp, ext_state=ext)
    assert fin.shape[0] == 0
    assert np.array_equal(out[:, 0, :], np.asarray(g["out"][3:6], dtype=np.float64))


@pytest.mark.parametrize("seed", range(6))
def test_recurrence_equals_bruteforce(seed):
    rng = np.random.default_rng(seed)
    dk, dv = [(3, 5), (4, 4), (8, 2), (1, 1), (16, 7), (5, 9)][seed]
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 3, 40, 3, 12, 2, dk, dv)
    o1, f1 = oracle.scan_recurrence(q, k, v, so, bp)
    o2, f2 = oracle.scan_bruteforce(q, k, v, so, bp)
    assert oracle.row_rel_err(o1, o2) <= 1e-12
    assert oracle.state_rel_err(f1, f2) <= 1e-12


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 63, 64, 65, 128, 1000])
def test_chunk_size_invariance(chunk):
    rng = np.random.default_rng(7)
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 2, 200, 3, 70, 2, 8, 6)
    o1, f1 = oracle.scan_recurrence(q, k, v, so, bp)
    o2, f2 = oracle.scan_chunked(q, k, v, so, bp, chunk)
    assert oracle.row_rel_err(o2, o1) <= 1e-12
    assert oracle.state_rel_err(f2, f1) <= 1e-12


def test_branch_alone_is_bit_identical():
    """Section "The Workload": branches never attend to each other, so a branch
    scored inside the packed pass equals the pass {its view, that branch}."""
    rng = np.random.default_rng(11)
    (vl, bc, bl), (so, bp, _), (q, k, v) = _rand_pass(rng, 3, 50, 4, 20, 2, 4, 3)
    out, _ = oracle.scan_recurrence(q, k, v, so, bp)
    for s in range(len(bp)):
        p = int(bp[s])
        if p < 0:
            continue
        a, b = int(so[p]), int(so[p + 1])
        c, d = int(so[s]), int(so[s + 1])
        idx = np.r_[a:b, c:d]
        so2, bp2, _ = oracle.pack_segments([b - a], [1], [d - c])
        out2, _ = oracle.scan_recurrence(q[idx], k[idx], v[idx], so2, bp2)
        assert np.array_equal(out2[b - a:], out[c:d])
        assert np.array_equal(out2[:b - a], out[a:b])


def test_shard_pass_is_bit_identical():
    """Section "Long Requests": split the branches into shards, each seeded
    with the view's final state; every shard row equals the unsharded row."""
    rng = np.random.default_rng(12)
    vl, bc = np.array([60]), np.array([9])
    bl = rng.integers(1, 30, size=9, endpoint=True)
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    T = int(so[-1])
    q, k, v = (rng.standard_normal((T, 2, 5)) for _ in range(3))
    full, ffin = oracle.scan_recurrence(q, k, v, so, bp)
    # view-only pass exports the state
    sov, bpv, _ = oracle.pack_segments(vl, [0], [])
    _, vfin = oracle.scan_recurrence(q[:60], k[:60], v[:60], sov, bpv)
    assert np.array_equal(vfin, ffin)
    for lo, hi in [(0, 3), (3, 5), (5, 9)]:
        sos, bps, _ = oracle.pack_segments([0], [hi - lo], bl[lo:hi])
        t0, t1 = int(so[1 + lo]), int(so[1 + hi])
        out, fin = oracle.scan_recurrence(q[t0:t1], k[t0:t1], v[t0:t1], sos, bps,
                                          ext_state=vfin[:1])
        assert np.array_equal(out, full[t0:t1])


def test_one_scan_per_pass_equals_scan_per_view():
    """Section "Kernels" ("One scan per pass"): one scan over the whole packed
    pass equals separate scans of each request; permuting the request order
    permutes the rows and the final states the same way."""
    rng = np.random.default_rng(13)
    (vl, bc, bl), (so, bp, vo), (q, k, v) = _rand_pass(rng, 4, 30, 3, 10, 2, 3, 4)
    out, fin = oracle.scan_recurrence(q, k, v, so, bp)
    views = [s for s in range(len(bp)) if bp[s] == -1]
    ends = views[1:] + [len(bp)]
    boff = np.r_[0, np.cumsum(bc)]
    for r, (s0, s1) in enumerate(zip(views, ends)):
        t0, t1 = int(so[s0]), int(so[s1])
        so_r, bp_r, _ = oracle.pack_segments([vl[r]], [bc[r]], bl[boff[r]:boff[r + 1]])
        o_r, f_r = oracle.scan_recurrence(q[t0:t1], k[t0:t1], v[t0:t1], so_r, bp_r)
        assert np.array_equal(o_r, out[t0:t1])
        assert np.array_equal(f_r[0], fin[r])
    perm = [2, 0, 3, 1]
    toks = []
    for r in perm:
        toks.append(np.arange(int(so[views[r]]), int(so[ends[r]])))
    idx = np.concatenate(toks)
    bl_p = np.concatenate([bl[boff[r]:boff[r + 1]] for r in perm])
    so_p, bp_p, _ = oracle.pack_segments(vl[perm], bc[perm], bl_p)
    out_p, fin_p = oracle.scan_recurrence(q[idx], k[idx], v[idx], so_p, bp_p)
    assert np.array_equal(out_p, out[idx])
    assert np.array_equal(fin_p, fin[perm])


def test_closed_form_all_ones():
    """q = k = v = 1: o_t[j] = d_k * |A(t)| with |A(t)| = pos+1 in a view and
    L_view + pos + 1 in a branch."""
    vl, bc, bl = [7, 3], [2, 1], [4, 1, 5]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    T, H, dk, dv = int(so[-1]), 2, 3, 4
    one = np.ones
    out, fin = oracle.scan_recurrence(one((T, H, dk)), one((T, H, dk)), one((T, H, dv)), so, bp)
    for s in range(len(bp)):
        base = int(so[bp[s] + 1] - so[bp[s]]) if bp[s] >= 0 else 0
        for pos, t in enumerate(range(int(so[s]), int(so[s + 1]))):
            assert np.all(out[t] == dk * (base + pos + 1))
    assert np.all(fin[0] == 7) and np.all(fin[1] == 3)


def test_closed_form_d1_and_zero_q():
    rng = np.random.default_rng(3)
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 2, 20, 2, 6, 1, 1, 1)
    out, fin = oracle.scan_recurrence(q, k, v, so, bp)
    sets = oracle.scan.attend_sets(so, bp)
    for t in range(len(sets)):
        ref = q[t, 0, 0] * sum(k[u, 0, 0] * v[u, 0, 0] for u in sets[t])
        assert abs(out[t, 0, 0] - ref) <= 1e-12 * max(1.0, abs(ref))
    out0, fin0 = oracle.scan_recurrence(np.zeros_like(q), k, v, so, bp)
    assert np.all(out0 == 0)
    assert np.array_equal(fin0, fin)


def test_linearity_in_v():
    rng = np.random.default_rng(4)
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 2, 30, 2, 8, 2, 4, 4)
    o1, f1 = oracle.scan_recurrence(q, k, v, so, bp)
    o2, f2 = oracle.scan_recurrence(q, k, 4.0 * v, so, bp)
    assert np.array_equal(o2, 4.0 * o1) and np.array_equal(f2, 4.0 * f1)


def test_sample_rows_matches_recurrence():
    rng = np.random.default_rng(5)
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 3, 40, 3, 9, 3, 4, 6)
    out, _ = oracle.scan_recurrence(q, k, v, so, bp)
    rows = list(range(0, int(so[-1]), 3))
    smp = oracle.sample_rows(q, k, v, so, bp, rows, heads=[0, 2])
    assert oracle.row_rel_err(smp, out[rows][:, [0, 2]]) <= 1e-12


def test_indexing_probe_expectation():
    """The exact indexing probe (q = k = e_0, v = one-hot segment code): a view
    token at position p gives (p+1) e_view; a branch token gives
    L_view e_view + (p+1) e_branch."""
    import synth
    vl, bc, bl = [5, 3], [2, 2], [2, 4, 1, 3]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    q, k, v = synth.probe_qkv(so, bp, 2, 8)
    out, fin = oracle.scan_recurrence(q, k, v, so, bp)
    for s in range(len(bp)):
        p = int(bp[s])
        for pos, t in enumerate(range(int(so[s]), int(so[s + 1]))):
            exp = np.zeros(8)
            exp[s] += pos + 1
            if p >= 0:
                exp[p] += int(so[p + 1] - so[p])
            assert np.array_equal(out[t, 0], exp) and np.array_equal(out[t, 1], exp)


def test_pack_validation():
    with pytest.raises(ValueError):
        oracle.pack_segments([3], [1], [0])
    with pytest.raises(ValueError):
        oracle.pack_segments([0], [0], [])
    with pytest.raises(ValueError):
        oracle.pack_segments([3, 2], [1], [1])
    with pytest.raises(ValueError):
        oracle.pack_segments([3], [2], [1])
    so, bp, vo = oracle.pack_segments([4, 0, 2], [0, 2, 1], [3, 1, 2])
    assert so.tolist() == [0, 4, 7, 8, 10, 12]
    assert bp.tolist() == [-1, -2, -2, -1, 3]
    assert vo.tolist() == [0, -1, -1, 1, -1]


# ---- planted mistakes: each mutated recurrence must fail at least one pin ----

def _mutant(kind):
    def run(q, k, v, so, bp, ext_state=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        T, H, dk = q.shape
        dv = v.shape[2]
        ords = oracle.view_ordinals(bp)
        out = np.zeros((T, H, dv))
        final = np.zeros((int((np.asarray(bp) == -1).sum()), H, dk, dv))
        S = np.zeros((H, dk, dv))
        last = None
        order = [s for s in range(len(bp)) if bp[s] == -1] + [s for s in range(len(bp)) if bp[s] != -1]
        for s in order:
            p = int(bp[s])
            if kind == "sibling_leak" and p >= 0 and last is not None and bp[last] == p:
                S = S.copy()
            elif kind == "cross_view_leak" and p == -1:
                S = S.copy()
            elif p == -1:
                S = np.zeros((H, dk, dv))
            else:
                S = final[ords[p]].copy()
            for t in range(int(so[s]), int(so[s + 1])):
                if kind == "exclusive":
                    out[t] = np.einsum("hk,hkv->hv", q[t], S)
                if kind == "transposed" and dk == dv:
                    S += v[t][:, :, None] * k[t][:, None, :]
                else:
                    S += k[t][:, :, None] * v[t][:, None, :]
                if kind != "exclusive":
                    out[t] = np.einsum("hk,hkv->hv", q[t], S)
            if p == -1:
                final[ords[s]] = S
            last = s
        return out, final
    return run


@pytest.mark.parametrize("kind", ["exclusive", "sibling_leak", "cross_view_leak", "transposed"])
def test_pins_catch_planted_mistakes(kind):
    g = _hand()
    q, k, v = _hand_inputs(g)
    out, fin = _mutant(kind)(q, k, v, g["seg_offsets"], g["branch_parent"])
    good = np.asarray(g["out"], dtype=np.float64)
    assert not (np.array_equal(out[:, 0], good)
                and np.array_equal(fin[:, 0], np.asarray(g["final_state"], dtype=np.float64)))


def test_view_states_matches_recurrence():
    rng = np.random.default_rng(6)
    _, (so, bp, _), (q, k, v) = _rand_pass(rng, 3, 40, 2, 9, 2, 3, 5)
    _, fin = oracle.scan_recurrence(q, k, v, so, bp)
    views = [s for s in range(len(bp)) if bp[s] == -1]
    st = oracle.view_states(k, v, so, bp, views, heads=[1])
    assert oracle.state_rel_err(st, fin[:, [1]]) <= 1e-12
