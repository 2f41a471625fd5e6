"""fp64 reference for tree-masked softmax attention over a packed pass.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The page "Serving 0.88M TPS from Two RTXs and Mac Minis"
(section "The Workload") says Span-1 is a hybrid: most layers are linear
attention, a few are softmax attention, and branches attend to their view but
not to each other.  Section "Long Requests" says the view cache holds, besides
the linear-attention state, the K/V of the softmax layers, so a branch shard
attends to its view's cached keys and values.  The page writes no equation;
the reading taken here is standard scaled softmax attention per head over the
same attend set A(t) as the linear layers:

    o_t = sum_{u in A(t)} w_tu v_u,   w_tu = exp(scale * q_t . k_u) / Z_t,
    Z_t = sum_{u in A(t)} exp(scale * q_t . k_u),

where A(t) is the tokens of t's own segment up to and including t, plus every
token of the parent view when t is in a branch.  A shard branch (parent
-2 - e) takes its view's keys and values from an external array (the cached
view K/V of row e) instead of from the pass.

Array conventions as in scan.py: q, k [T, H, d_k]; v [T, H, d_v]; external
views as a list of (k_e [L_e, H, d_k], v_e [L_e, H, d_v]).  Outputs float64.
"""
import numpy as np

from .scan import _f64


def _segment_keys(s, seg_offsets, branch_parent, k, v, ext_kv):
    """Keys and values every token of segment s may see before its own
    segment's tokens: the parent view (packed or external), else nothing."""
    p = int(branch_parent[s])
    if p >= 0:
        a, b = int(seg_offsets[p]), int(seg_offsets[p + 1])
        return k[a:b], v[a:b]
    if p <= -2:
        if ext_kv is None:
            raise ValueError("shard branch but no external view K/V given")
        ek, ev = ext_kv[-p - 2]
        return _f64(ek), _f64(ev)
    return k[:0], v[:0]


def attention_dense(q, k, v, seg_offsets, branch_parent, scale, ext_kv=None):
    """THE attention oracle: for each segment and head, the scores of every
    token against [parent view keys, own segment keys], the causal mask on
    the own part, a softmax over each row (max subtracted), times the values.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dk = q.shape
    dv = v.shape[2]
    seg_offsets = np.asarray(seg_offsets)
    out = np.zeros((T, H, dv))
    for s in range(len(branch_parent)):
        a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
        pk, pv = _segment_keys(s, seg_offsets, branch_parent, k, v, ext_kv)
        keys = np.concatenate([pk, k[a:b]], axis=0)       # [Lp + n, H, dk]
        vals = np.concatenate([pv, v[a:b]], axis=0)
        lp, n = pk.shape[0], b - a
        allowed = np.ones((n, lp + n), dtype=bool)
        allowed[:, lp:] = np.tril(np.ones((n, n), dtype=bool))   # u <= t inside the segment
        for h in range(H):
            sc = scale * (q[a:b, h, :] @ keys[:, h, :].T)
            sc = np.where(allowed, sc, -np.inf)
            w = np.exp(sc - sc.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            out[a:b, h, :] = w @ vals[:, h, :]
    return out


def attention_rows(q, k, v, seg_offsets, branch_parent, scale, rows, ext_kv=None):
    """The same definition for selected tokens only (large passes): returns
    [len(rows), H, d_v]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    seg_offsets = np.asarray(seg_offsets)
    H, dv = q.shape[1], v.shape[2]
    res = np.zeros((len(rows), H, dv))
    seg_of = np.searchsorted(seg_offsets, np.asarray(rows), side="right") - 1
    for i, (t, s) in enumerate(zip(rows, seg_of)):
        a = int(seg_offsets[s])
        pk, pv = _segment_keys(int(s), seg_offsets, branch_parent, k, v, ext_kv)
        keys = np.concatenate([pk, k[a:t + 1]], axis=0)
        vals = np.concatenate([pv, v[a:t + 1]], axis=0)
        for h in range(H):
            sc = scale * (keys[:, h, :] @ q[t, h, :])
            w = np.exp(sc - sc.max())
            res[i, h] = (w / w.sum()) @ vals[:, h, :]
    return res


def attention_flops(seg_offsets, branch_parent, H, d, ext_len=None):
    """Algorithmic FLOPs of a pass: 2 d for the score and 2 d for the
    weighted value per (token, attended key, head)."""
    seg_offsets = np.asarray(seg_offsets)
    total = 0
    for s in range(len(branch_parent)):
        n = int(seg_offsets[s + 1] - seg_offsets[s])
        p = int(branch_parent[s])
        lp = 0
        if p >= 0:
            lp = int(seg_offsets[p + 1] - seg_offsets[p])
        elif p <= -2:
            lp = int(ext_len[-p - 2])
        total += n * lp + n * (n + 1) // 2
    return 4 * d * H * total
