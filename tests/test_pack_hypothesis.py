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
    blocks = p.plan[16:16 + 8 * info.n_blocks].reshape(-1, 8)
    cover = np.zeros(info.n_tokens, dtype=int)
    for tok0, ntok, sin, dslot, seed, seg, _, _ in blocks:
        assert 1 <= ntok <= 64 * G and tok0 >= so[seg] and tok0 + ntok <= so[seg + 1]
        assert (tok0 - so[seg]) % 64 == 0
        cover[tok0:tok0 + ntok] += 1
        if tok0 == so[seg]:
            assert sin == -1           # a segment's first block needs no prefix
    assert (cover == 1).all()
    # attention items cover every query exactly once, in <= 64-token blocks
    ext_len = [11] * info.n_ext
    items = la.attn_plan(so, bp, ext_len).items
    cover[:] = 0
    for q0, nq, seg0, view0, view_len, src, _, _ in items:
        assert 1 <= nq <= 64 and (q0 - seg0) % 64 == 0
        cover[q0:q0 + nq] += 1
    assert (cover == 1).all()
