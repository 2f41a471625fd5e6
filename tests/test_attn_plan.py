"""Host planner of the softmax attention (la_attn_plan): one item per
(segment, 64-token query block), grouped by the view whose keys they read,
groups and items within a group longest key range first; CPU only."""
import numpy as np
import pytest

import oracle
import chunked_linear_attention_packed_amd as la


def _expected(so, bp, ext_len):
    offs = np.concatenate([[0], np.cumsum(ext_len)]) if len(ext_len) else [0]
    items = []
    for s in range(len(bp)):
        a, b, p = int(so[s]), int(so[s + 1]), int(bp[s])
        if p >= 0:
            view = (int(so[p]), int(so[p + 1] - so[p]), la.LA_ATTN_PACKED_VIEW)
        elif p <= -2:
            view = (int(offs[-p - 2]), int(ext_len[-p - 2]), la.LA_ATTN_EXT_VIEW)
        else:
            view = (0, 0, la.LA_ATTN_NO_VIEW)
        # group: the view segment, an external view (after every segment),
        # or the segment itself
        group = p if p >= 0 else (len(bp) - p if p <= -2 else s)
        for q0 in range(a, b, 64):
            nq = min(64, b - q0)
            items.append(((q0, nq, a) + view + (0, 0), view[1] + q0 + nq - a, group))
    longest = {}
    for _, keys, group in items:
        longest[group] = max(longest.get(group, 0), keys)
    # stable: ties keep table order
    items.sort(key=lambda it: (-longest[it[2]], it[2], -it[1]))
    return np.array([it[0] for it in items], dtype=np.int32).reshape(-1, 8)


@pytest.mark.parametrize("vl,bc,bl", [([1], [0], []), ([200], [3], [1, 64, 130]),
                                      ([129, 70], [2, 1], [65, 5, 64]),
                                      ([7400], [8], [48] * 8)])
def test_plan_items(vl, bc, bl):
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    p = la.attn_plan(so, bp)
    assert np.array_equal(p.items, _expected(so, bp, []))
    # every query token is covered exactly once
    cover = np.zeros(int(so[-1]), dtype=int)
    for q0, nq, *_ in p.items:
        cover[q0:q0 + nq] += 1
    assert (cover == 1).all()


def test_plan_external_views():
    so, bp, ext = [0, 30, 130, 200, 201], [-4, -1, 1, -2], [70, 5, 200]
    p = la.attn_plan(so, bp, ext)
    assert np.array_equal(p.items, _expected(so, bp, ext))
    assert p.n_ext_tokens == 275


@pytest.mark.parametrize("so,bp,ext", [([0, 5, 5], [-1, -1], []),       # empty segment
                                       ([1, 5], [-1], []),              # not starting at 0
                                       ([0, 5, 9], [1, -1], []),        # parent after, fine? no: parent must be a view
                                       ([0, 5, 9], [-1, 1], []),        # parent is a branch... itself
                                       ([0, 5], [-3], [4]),             # external view 1 of 1
                                       ([0, 5], [-2], [0])])            # empty external view
def test_plan_rejects_bad_tables(so, bp, ext):
    if bp == [1, -1]:
        # a branch listed before its view is valid
        la.attn_plan(so, bp, ext)
        return
    with pytest.raises(la.LinAttnError):
        la.attn_plan(so, bp, ext)


def test_plan_external_views_at_given_starts():
    """la_attn_plan_ext: external view e at token row ext_start[e] of arrays
    of ext_tokens rows (a K/V cache pool with one region per cache row); the
    items equal the concatenated plan's except for each view's first row."""
    so, bp, ext = [0, 30, 130, 200, 201], [-4, -1, 1, -2], [70, 5, 200]
    starts = [1000, 3000, 0]
    p = la.attn_plan(so, bp, ext, ext_start=starts, ext_tokens=4000)
    want = _expected(so, bp, ext)
    offs = np.concatenate([[0], np.cumsum(ext)])
    for row in want:
        if row[5] == la.LA_ATTN_EXT_VIEW:
            e = int(np.flatnonzero(offs[:-1] == row[3])[0])
            row[3] = starts[e]
    assert np.array_equal(p.items, want)
    assert p.n_ext_tokens == 4000
    # concatenated starts give la_attn_plan's items exactly
    q = la.attn_plan(so, bp, ext, ext_start=offs[:-1], ext_tokens=int(offs[-1]))
    assert np.array_equal(q.items, la.attn_plan(so, bp, ext).items)


@pytest.mark.parametrize("starts,rows", [([1000, 3000, 3801], 4000),   # view 2 past the end
                                         ([-1, 0, 500], 4000),          # negative start
                                         ([0, 0, 0], 199)])             # all past 199 rows
def test_plan_external_starts_checked(starts, rows):
    so, bp, ext = [0, 30, 130, 200, 201], [-4, -1, 1, -2], [70, 5, 200]
    with pytest.raises(la.LinAttnError) as e:
        la.attn_plan(so, bp, ext, ext_start=starts, ext_tokens=rows)
    assert e.value.status == la.LA_ERR_INVALID_ARG
