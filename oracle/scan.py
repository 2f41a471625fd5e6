"""fp64 reference evaluations of the packed causal linear-attention scan.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed.  The page "Serving 0.88M TPS from Two RTXs and Mac Minis"
(section "The Workload") says that Span-1 is mostly linear-attention layers,
that a request is one long view and many short branches, and that branches
attend to their view but not to each other.  Section "Kernels" says the layer
is evaluated in 64-token chunks with a few 64x64 matrix products each and that
one scan covers every view of a pass.  The page writes no equation.  The
reading taken here is the plain, unnormalised causal linear attention, per
head, with an fp32/fp64 state of shape d_k x d_v:

    S_t = S_{t-1} + k_t^T v_t        (outer product of row vectors)
    o_t = q_t S_t                    (inclusive: token t sees its own k_t, v_t)

with no feature map, no normaliser and no decay.  A view starts from S = 0.
A branch starts from the final state of its own view (section "Long
Requests": a branch shard needs only the view's cached linear-attention
state), or from an externally supplied state in a shard pass.  A view never
sees a branch and a branch never sees another branch.

Equivalent closed form: o_t = sum over u in A(t) of (q_t . k_u) v_u, where A(t)
is the tokens of t's own segment up to and including t, plus every token of
the parent view when t is in a branch.  The three functions below reach this
result by three independent routes (token recurrence, explicit T x T mask,
chunked blocks), which is what lets them pin one another.

Array conventions: q, k are [T, H, d_k]; v is [T, H, d_v]; segments are given
by seg_offsets[n_seg+1] and branch_parent[n_seg] (see pack.py).  Outputs are
float64: out [T, H, d_v] and final [n_views, H, d_k, d_v].
"""
import numpy as np

from .pack import view_ordinals


def _f64(x):
    if hasattr(x, "detach"):          # a torch tensor: upcast exactly
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _seed_state(p, final, ords, ext_state, H, dk, dv):
    if p == -1:
        return np.zeros((H, dk, dv))
    if p >= 0:
        return final[ords[p]].copy()
    if ext_state is None:
        raise ValueError("branch seeded from external state but ext_state is None")
    return np.array(ext_state[-p - 2], dtype=np.float64)


def scan_recurrence(q, k, v, seg_offsets, branch_parent, ext_state=None):
    """THE oracle: token-by-token recurrence in float64.

    Views are scanned first (each from a zero state, recording its final
    state), then every branch from a copy of its view's final state (or of
    ext_state[-parent-2]).  A branch's own final state is discarded.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    ext = None if ext_state is None else _f64(ext_state)
    T, H, dk = q.shape
    dv = v.shape[2]
    seg_offsets = np.asarray(seg_offsets)
    branch_parent = np.asarray(branch_parent)
    ords = view_ordinals(branch_parent)
    n_views = int((branch_parent == -1).sum())
    out = np.zeros((T, H, dv))
    final = np.zeros((n_views, H, dk, dv))
    order = [s for s in range(len(branch_parent)) if branch_parent[s] == -1]
    order += [s for s in range(len(branch_parent)) if branch_parent[s] != -1]
    for s in order:
        p = int(branch_parent[s])
        S = _seed_state(p, final, ords, ext, H, dk, dv)
        for t in range(int(seg_offsets[s]), int(seg_offsets[s + 1])):
            S += k[t][:, :, None] * v[t][:, None, :]
            out[t] = np.einsum("hk,hkv->hv", q[t], S)
        if p == -1:
            final[ords[s]] = S
    return out, final


def attend_sets(seg_offsets, branch_parent):
    """For every token t, the list of tokens u in A(t) (the closed form)."""
    seg_offsets = np.asarray(seg_offsets)
    T = int(seg_offsets[-1])
    sets = [None] * T
    for s in range(len(branch_parent)):
        a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
        p = int(branch_parent[s])
        base = list(range(int(seg_offsets[p]), int(seg_offsets[p + 1]))) if p >= 0 else []
        for t in range(a, b):
            sets[t] = base + list(range(a, t + 1))
    return sets


def scan_bruteforce(q, k, v, seg_offsets, branch_parent, ext_state=None):
    """O(T^2) evaluation: ((Q K^T) * M) V per head with the explicit mask
    M[t, u] = 1 if u in A(t).  External seeds add q_t . ext.  Final view
    states are sum over the view's tokens of k_u^T v_u.  For small T only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dk = q.shape
    dv = v.shape[2]
    M = np.zeros((T, T))
    for t, us in enumerate(attend_sets(seg_offsets, branch_parent)):
        M[t, us] = 1.0
    out = np.zeros((T, H, dv))
    for h in range(H):
        out[:, h, :] = ((q[:, h, :] @ k[:, h, :].T) * M) @ v[:, h, :]
    branch_parent = np.asarray(branch_parent)
    seg_offsets = np.asarray(seg_offsets)
    if ext_state is not None:
        ext = _f64(ext_state)
        for s in range(len(branch_parent)):
            p = int(branch_parent[s])
            if p <= -2:
                a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
                out[a:b] += np.einsum("thk,hkv->thv", q[a:b], ext[-p - 2])
    views = [s for s in range(len(branch_parent)) if branch_parent[s] == -1]
    final = np.zeros((len(views), H, dk, dv))
    for i, s in enumerate(views):
        a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
        final[i] = np.einsum("uhk,uhv->hkv", k[a:b], v[a:b])
    return out, final


def scan_chunked(q, k, v, seg_offsets, branch_parent, chunk, ext_state=None):
    """Chunked fp64 evaluation, chunks restarting at each segment start.

    Per segment and head: the chunk states K_c^T V_c, their exclusive prefix
    S_in (plus the seed), then O_c = Q_c S_in + tril(Q_c K_c^T) V_c with the
    diagonal included.  Used only to pin that the result does not depend on
    the chunk size (section "Kernels" evaluates the layer in 64-token chunks).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    ext = None if ext_state is None else _f64(ext_state)
    T, H, dk = q.shape
    dv = v.shape[2]
    branch_parent = np.asarray(branch_parent)
    seg_offsets = np.asarray(seg_offsets)
    ords = view_ordinals(branch_parent)
    final = np.zeros((int((branch_parent == -1).sum()), H, dk, dv))
    out = np.zeros((T, H, dv))
    order = [s for s in range(len(branch_parent)) if branch_parent[s] == -1]
    order += [s for s in range(len(branch_parent)) if branch_parent[s] != -1]
    for s in order:
        p = int(branch_parent[s])
        S = _seed_state(p, final, ords, ext, H, dk, dv)
        a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
        for c0 in range(a, b, chunk):
            c1 = min(c0 + chunk, b)
            Qc, Kc, Vc = q[c0:c1], k[c0:c1], v[c0:c1]
            n = c1 - c0
            mask = np.tril(np.ones((n, n)))
            for h in range(H):
                A = (Qc[:, h, :] @ Kc[:, h, :].T) * mask
                out[c0:c1, h, :] = Qc[:, h, :] @ S[h] + A @ Vc[:, h, :]
                S[h] = S[h] + Kc[:, h, :].T @ Vc[:, h, :]
        if p == -1:
            final[ords[s]] = S
    return out, final


def sample_rows(q, k, v, seg_offsets, branch_parent, rows, heads=None, ext_state=None):
    """Closed form for selected tokens: o_t = q_t (sum over u in A(t) of
    k_u^T v_u), in float64, for large passes where the full recurrence is too
    slow.  q, k, v may be torch tensors or arrays of the full pass; only the
    needed rows are upcast.  Returns [len(rows), len(heads), d_v].
    """
    seg_offsets = np.asarray(seg_offsets)
    branch_parent = np.asarray(branch_parent)
    H = q.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    seg_of = np.searchsorted(seg_offsets, np.asarray(rows), side="right") - 1
    res = np.zeros((len(rows), len(heads), v.shape[2]))
    for i, t in enumerate(rows):
        s = int(seg_of[i])
        a = int(seg_offsets[s])
        p = int(branch_parent[s])
        spans = [(a, int(t) + 1)]
        if p >= 0:
            spans.append((int(seg_offsets[p]), int(seg_offsets[p + 1])))
        qt = _f64(q[int(t)])[heads]                      # [h, dk]
        for hi, h in enumerate(heads):
            S = np.zeros((k.shape[2], v.shape[2]))
            for (u0, u1) in spans:
                S += _f64(k[u0:u1, h]).T @ _f64(v[u0:u1, h])
            if p <= -2:
                S += _f64(ext_state[-p - 2, h])
            res[i, hi] = qt[hi] @ S
    return res


def view_states(k, v, seg_offsets, branch_parent, views, heads=None):
    """Final state of selected view segments: sum over the view's tokens of
    k_u^T v_u, float64, [len(views), len(heads), d_k, d_v]."""
    seg_offsets = np.asarray(seg_offsets)
    H = k.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    res = np.zeros((len(views), len(heads), k.shape[2], v.shape[2]))
    for i, s in enumerate(views):
        if int(branch_parent[s]) != -1:
            raise ValueError("segment %d is not a view" % s)
        a, b = int(seg_offsets[s]), int(seg_offsets[s + 1])
        for hi, h in enumerate(heads):
            res[i, hi] = _f64(k[a:b, h]).T @ _f64(v[a:b, h])
    return res
