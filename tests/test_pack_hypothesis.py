"""Property tests (hypothesis) of the host packer and planners against the
oracle's packer and the plan's defining properties, on generated request
shapes, including shard requests and block sizes.  CPU only."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
import chunked_linear_attention_packed_amd as la

requests = st.lists(
    st.tuples(st.integers(0, 700),                                # view length (0: shard)
              st.lists(st.integers(1, 300), min_size=0, max_size=5)),
    min_size=1, max_size=6).filter(lambda rs: all(v > 0 or bl for v, bl in rs))


@settings(max_examples=150, deadline=None)
@given(requests, st.integers(1, 17))
def test_pack_matches_oracle_and_plan_properties(reqs, G):
    vl = [v for v, _ in reqs]
    bc = [len(bl) for _, bl in reqs]
    bl = [x for _, b in reqs for x in b]
    p = la.pack(vl, bc, bl, heads=2, block_chunks=G)
    so, bp, vo = oracle.pack_segments(vl, bc, bl)
    assert np.array_equal(p.seg_offsets, so) and np.array_equal(p.branch_parent, bp)
    info = p.info
    assert info.n_tokens == int(so[-1]) and info.n_segments == len(bp)
    assert info.n_views == sum(1 for v in vl if v > 0)
    assert info.n_ext == sum(1 for v in vl if v == 0)
    # blocks tile every segment exactly, G chunks at most, in whole chunks
    blocks = p.plan[p.plan[8]:p.plan[8] + 8 * info.n_blocks].reshape(-1, 8)
    cover = np.zeros(info.n_tokens, dtype=int)
    for tok0, ntok, sin, dslot, seed, seg, _, _ in blocks:
        assert 1 <= ntok <= 64 * G and tok0 >= so[seg] and tok0 + ntok <= so[seg + 1]
        assert (tok0 - so[seg]) % 64 == 0
        cover[tok0:tok0 + ntok] += 1
        if tok0 == so[seg]:
            assert sin == -1           # a segment's first block needs no prefix
    assert (cover == 1).all()
    # piece path: blocks of at most 8 chunks tile every segment; every block is
    # in exactly one work item, packs hold only one-piece single-block branches
    ob, oi = int(p.plan[20]), int(p.plan[21])
    pblocks = p.plan[ob:ob + 8 * info.piece_blocks].reshape(-1, 8)
    pitems = p.plan[oi:oi + 12 * info.piece_items].reshape(-1, 12)
    cover[:] = 0
    for tok0, ntok, slot, seed, seg, slot0, j, frow in pblocks:
        assert 1 <= ntok <= 512 and tok0 == so[seg] + 512 * j
        cover[tok0:tok0 + ntok] += 1
    assert (cover == 1).all()
    seen = np.zeros(info.piece_blocks, dtype=int)
    for row in pitems:
        kind, n, bs = row[0], row[1], row[2:10]
        members = [b for b in (bs[:1] if kind == 0 else bs[:2 * n]) if b != -1]
        for b in members:
            seen[b] += 1
            if kind == 1:
                tok0, ntok, _, seed, seg = pblocks[b][:5]
                assert seed != -1 and ntok <= 128 and ntok == so[seg + 1] - so[seg]
        if kind == 1:   # a wave holds one branch, or two of at most one chunk
            for w in range(n):
                if bs[2 * w + 1] != -1:
                    assert pblocks[bs[2 * w]][1] <= 64 and pblocks[bs[2 * w + 1]][1] <= 64
    assert (seen == 1).all()
    # attention items cover every query exactly once, in <= 64-token blocks
    ext_len = [11] * info.n_ext
    items = la.attn_plan(so, bp, ext_len).items
    cover[:] = 0
    for q0, nq, seg0, view0, view_len, src, _, _ in items:
        assert 1 <= nq <= 64 and (q0 - seg0) % 64 == 0
        cover[q0:q0 + nq] += 1
    assert (cover == 1).all()
