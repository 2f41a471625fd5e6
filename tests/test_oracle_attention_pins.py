"""Pins of the tree-masked softmax attention oracle (oracle/attention.py)
against results fixed independently of it:

* a worked example derived by hand (tests/golden/attention_hand_example.json:
  with scale = ln 2 every weight is a power of two, so each output is an exact
  rational; the derivation is in the file);
* a single view with no branches is textbook causal softmax attention: torch's
  scaled_dot_product_attention (float64, CPU) with is_causal=True;
* a branch sees its whole view and itself causally, and nothing else: its rows
  equal the last rows of causal attention over [view tokens; branch tokens];
* q = 0 gives uniform weights: o_t = mean of v over the attend set A(t);
* a shard branch seeded with the view's K/V equals the branch in the full pass;
* per-row evaluation equals the dense one; the FLOP count is a closed form.
Planted mistakes (exclusive diagonal, sibling leak, missing scale) in copies
of the oracle must each fail one of these pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as A

GOLD = os.path.join(os.path.dirname(__file__), "golden", "attention_hand_example.json")


def _hand():
    with open(GOLD) as f:
        g = json.load(f)
    arr = lambda key: np.asarray(g[key], dtype=np.float64)[:, None, :]   # [T, 1, d]
    return g, arr("q"), arr("k"), arr("v")


def test_hand_worked_example():
    g, q, k, v = _hand()
    so, bp, _ = oracle.pack_segments(g["view_len"], g["branch_count"], g["branch_len"])
    assert list(so) == g["seg_offsets"] and list(bp) == g["branch_parent"]
    got = oracle.attention_dense(q, k, v, so, bp, math.log(2.0))
    assert np.allclose(got[:, 0, :], np.asarray(g["out"]), rtol=1e-13, atol=1e-13)
    rows = list(range(len(g["out"])))
    got_r = oracle.attention_rows(q, k, v, so, bp, math.log(2.0), rows)
    assert np.allclose(got_r[:, 0, :], np.asarray(g["out"]), rtol=1e-13, atol=1e-13)


def _rand(rng, T, H, d, dv=None):
    dv = d if dv is None else dv
    return (rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d)),
            rng.standard_normal((T, H, dv)))


def _sdpa_causal(q, k, v, scale):
    """torch causal attention, [T, H, d] float64 in and out."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("T,H,d,dv,scale", [(1, 1, 4, 4, 1.0), (37, 2, 8, 5, 0.3),
                                            (130, 3, 16, 16, 0.25)])
def test_single_view_is_causal_sdpa(T, H, d, dv, scale):
    rng = np.random.default_rng(T)
    q, k, v = _rand(rng, T, H, d, dv)
    got = oracle.attention_dense(q, k, v, [0, T], [-1], scale)
    assert np.allclose(got, _sdpa_causal(q, k, v, scale), rtol=1e-12, atol=1e-12)


def _request(rng, H, d):
    # view 23, branches 7, 1, 12 (one request) + a second request: view 5, branch 3
    vl, bc, bl = [23, 5], [3, 1], [7, 1, 12, 3]
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    T = int(so[-1])
    return so, bp, _rand(rng, T, H, d)


def test_branches_see_their_view_and_themselves_only():
    rng = np.random.default_rng(11)
    so, bp, (q, k, v) = _request(rng, 2, 8)
    scale = 0.4
    got = oracle.attention_dense(q, k, v, so, bp, scale)
    for s in range(len(bp)):
        a, b = int(so[s]), int(so[s + 1])
        p = int(bp[s])
        if p < 0:
            idx = np.arange(a, b)
        else:
            idx = np.r_[so[p]:so[p + 1], a:b]
        ref = _sdpa_causal(q[idx], k[idx], v[idx], scale)[-(b - a):]
        assert np.allclose(got[a:b], ref, rtol=1e-12, atol=1e-12), f"segment {s}"


def test_zero_queries_average_the_attend_set():
    rng = np.random.default_rng(12)
    so, bp, (q, k, v) = _request(rng, 3, 4)
    got = oracle.attention_dense(np.zeros_like(q), k, v, so, bp, 1.0)
    for t, us in enumerate(oracle.scan.attend_sets(so, bp)):
        assert np.allclose(got[t], v[us].mean(axis=0), rtol=1e-13, atol=1e-13)


def test_shard_from_view_kv_equals_full_pass():
    rng = np.random.default_rng(13)
    so, bp, (q, k, v) = _request(rng, 2, 8)
    full = oracle.attention_dense(q, k, v, so, bp, 0.5)
    # branches of request 0 as a shard: parent -2 - 0, view K/V given externally
    a, b = int(so[1]), int(so[4])
    so_s = np.asarray(so[1:5]) - a
    bp_s = np.array([-2, -2, -2])
    ext = [(k[so[0]:so[1]], v[so[0]:so[1]])]
    shard = oracle.attention_dense(q[a:b], k[a:b], v[a:b], so_s, bp_s, 0.5, ext_kv=ext)
    assert np.array_equal(shard, full[a:b])
    with pytest.raises(ValueError):
        oracle.attention_dense(q[a:b], k[a:b], v[a:b], so_s, bp_s, 0.5)


def test_rows_equal_dense():
    rng = np.random.default_rng(14)
    so, bp, (q, k, v) = _request(rng, 2, 8)
    dense = oracle.attention_dense(q, k, v, so, bp, 0.7)
    rows = [0, 5, 22, 23, 29, 30, 43, 44, 48, 50]
    assert np.allclose(oracle.attention_rows(q, k, v, so, bp, 0.7, rows), dense[rows],
                       rtol=1e-12, atol=1e-12)


def test_flop_count():
    so, bp, _ = oracle.pack_segments([23, 5], [3, 1], [7, 1, 12, 3])
    n_pairs = sum(len(us) for us in oracle.scan.attend_sets(so, bp))
    assert oracle.attention_flops(so, bp, H=3, d=8) == 4 * 8 * 3 * n_pairs
    assert oracle.attention_flops([0, 4], [-2], H=1, d=2, ext_len=[10]) == 4 * 2 * (40 + 10)


# ---- planted mistakes: each must fail one pin above --------------------------------

def _planted(kind):
    def f(q, k, v, so, bp, scale, ext_kv=None):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        out = np.zeros_like(v)
        for s in range(len(bp)):
            a, b = int(so[s]), int(so[s + 1])
            p = int(bp[s])
            lo = int(so[p]) if p >= 0 else a
            if kind == "sibling_leak" and p >= 0:
                lo = int(so[p])          # sees everything from its view start: siblings too
            for t in range(a, b):
                if p >= 0 and kind != "sibling_leak":
                    idx = np.r_[so[p]:so[p + 1], a:t + 1]
                else:
                    idx = np.arange(lo, t + 1)
                if kind == "exclusive":
                    idx = idx[:-1] if len(idx) > 1 else idx
                sc = (1.0 if kind == "no_scale" else scale) * np.einsum("uhd,hd->hu", k[idx], q[t])
                w = np.exp(sc - sc.max(axis=1, keepdims=True))
                w /= w.sum(axis=1, keepdims=True)
                out[t] = np.einsum("hu,uhd->hd", w, v[idx])
        return out
    return f


@pytest.mark.parametrize("kind", ["exclusive", "sibling_leak", "no_scale"])
def test_planted_mistakes_fail_the_hand_example(kind):
    g, q, k, v = _hand()
    so, bp, _ = oracle.pack_segments(g["view_len"], g["branch_count"], g["branch_len"])
    bad = _planted(kind)(q, k, v, so, bp, math.log(2.0))
    assert not np.allclose(bad[:, 0, :], np.asarray(g["out"]), rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("kind", ["exclusive", "sibling_leak", "no_scale"])
def test_planted_mistakes_fail(kind):
    rng = np.random.default_rng(15)
    so, bp, (q, k, v) = _request(rng, 2, 8)
    bad = _planted(kind)(q, k, v, so, bp, 0.4)
    caught = False
    for s in range(len(bp)):
        a, b = int(so[s]), int(so[s + 1])
        p = int(bp[s])
        idx = np.arange(a, b) if p < 0 else np.r_[so[p]:so[p + 1], a:b]
        ref = _sdpa_causal(q[idx], k[idx], v[idx], 0.4)[-(b - a):]
        caught |= not np.allclose(bad[a:b], ref, rtol=1e-9, atol=1e-9)
    assert caught
    # and the same planted routine without the mistake passes (the pin is sound)
    assert np.allclose(_planted("none")(q, k, v, so, bp, 0.4),
                       oracle.attention_dense(q, k, v, so, bp, 0.4), rtol=1e-12, atol=1e-12)
