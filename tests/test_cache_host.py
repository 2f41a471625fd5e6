"""Host logic of the view-state cache directory (la_cache_*) and of packing
shard requests onto explicit ext_state rows (la_pack_pass_ext).  CPU only:
these calls touch no device memory."""
import numpy as np
import pytest

import oracle
import chunked_linear_attention_packed_amd as la


def test_cache_fills_free_rows_then_evicts_least_recent():
    c = la.ViewStateCache.__new__(la.ViewStateCache)   # directory only, no device pool
    lib = la.load_library()
    import ctypes
    c._lib, c._h = lib, ctypes.c_void_p()
    la._check("la_cache_create", lib.la_cache_create(3, ctypes.byref(c._h)))
    try:
        assert [c.reserve(v) for v in (10, 20, 30)] == [(0, None), (1, None), (2, None)]
        assert len(c) == 3
        assert c.lookup(10) == 0            # 10 becomes most recent: order 10, 30, 20
        assert c.lookup(99) is None
        assert c.reserve(40) == (1, 20)     # evicts 20, the least recently used
        assert c.lookup(20) is None
        assert c.reserve(30) == (2, None)   # already cached: same row, now most recent
        assert c.reserve(50) == (0, 10)     # order was 30, 40, 10 -> evict 10
        c.erase(40)
        assert len(c) == 2 and c.lookup(40) is None
        assert c.reserve(60) == (1, None)   # the erased row is reused before evicting
        c.erase(12345)                      # absent: no-op
        assert len(c) == 3
    finally:
        c.close()


def test_cache_lru_matches_a_reference_model():
    """Random operation sequences against a plain ordered-dict LRU."""
    from collections import OrderedDict
    import ctypes
    lib = la.load_library()
    rng = np.random.default_rng(7)
    for cap in (1, 2, 5):
        h = ctypes.c_void_p()
        la._check("la_cache_create", lib.la_cache_create(cap, ctypes.byref(h)))
        model = OrderedDict()          # id -> row, last = most recent
        free = list(range(cap - 1, -1, -1))   # a stack: row 0 first, freed rows reused first
        try:
            for _ in range(400):
                vid = int(rng.integers(0, 8))
                op = rng.integers(0, 3)
                row = ctypes.c_int32()
                if op == 0:
                    la._check("lookup", lib.la_cache_lookup(h, vid, ctypes.byref(row)))
                    if vid in model:
                        model.move_to_end(vid)
                        assert row.value == model[vid]
                    else:
                        assert row.value == -1
                elif op == 1:
                    ev = ctypes.c_int64()
                    la._check("reserve", lib.la_cache_reserve(h, vid, ctypes.byref(row),
                                                              ctypes.byref(ev)))
                    if vid in model:
                        model.move_to_end(vid)
                        assert (row.value, ev.value) == (model[vid], -1)
                    else:
                        if free:
                            r, e = free.pop(), -1
                        else:
                            e, r = model.popitem(last=False)
                        model[vid] = r
                        assert (row.value, ev.value) == (r, e)
                else:
                    la._check("erase", lib.la_cache_erase(h, vid))
                    if vid in model:
                        free.append(model.pop(vid))
                n = ctypes.c_int32()
                la._check("count", lib.la_cache_count(h, ctypes.byref(n)))
                assert n.value == len(model)
                assert sorted(model.values()) == sorted(set(model.values()))
        finally:
            lib.la_cache_destroy(h)


def test_cache_rejects_bad_arguments():
    import ctypes
    lib = la.load_library()
    h = ctypes.c_void_p()
    assert lib.la_cache_create(0, ctypes.byref(h)) == la.LA_ERR_INVALID_ARG
    assert lib.la_cache_create(4, None) == la.LA_ERR_INVALID_ARG
    la._check("la_cache_create", lib.la_cache_create(4, ctypes.byref(h)))
    row = ctypes.c_int32()
    assert lib.la_cache_lookup(h, -1, ctypes.byref(row)) == la.LA_ERR_INVALID_ARG
    assert lib.la_cache_reserve(h, -5, ctypes.byref(row), None) == la.LA_ERR_INVALID_ARG
    assert lib.la_cache_reserve(h, 5, None, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_cache_lookup(None, 1, ctypes.byref(row)) == la.LA_ERR_INVALID_ARG
    assert lib.la_cache_reserve(h, 5, ctypes.byref(row), None) == la.LA_OK   # evicted_id optional
    assert lib.la_cache_destroy(h) == la.LA_OK
    assert lib.la_cache_destroy(None) == la.LA_ERR_INVALID_ARG


def test_pack_ext_rows_name_the_seed_row():
    vl, bc, bl = [0, 100, 0], [2, 1, 3], [5, 6, 7, 8, 9, 10]
    p = la.pack(vl, bc, bl, heads=2, ext_row=[7, 0, 3])
    assert list(p.branch_parent) == [-9, -9, -1, 2, -5, -5, -5]
    assert p.info.n_ext == 8
    # without ext_row, shard requests take rows 0, 1, ... (la_pack_pass)
    q = la.pack(vl, bc, bl, heads=2)
    assert list(q.branch_parent) == [-2, -2, -1, 2, -3, -3, -3]
    assert q.info.n_ext == 2
    assert np.array_equal(p.seg_offsets, q.seg_offsets)
    # the oracle's own packer agrees on the segment table
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    assert np.array_equal(so, q.seg_offsets) and np.array_equal(bp, q.branch_parent)


@pytest.mark.parametrize("rows", [[-1], [2 ** 30 + 1]])
def test_pack_ext_rejects_bad_rows(rows):
    with pytest.raises(la.LinAttnError):
        la.pack([0], [1], [5], heads=1, ext_row=rows)
    with pytest.raises(ValueError):
        la.pack([0, 0], [1, 1], [5, 5], heads=1, ext_row=[0])


def test_pack_ext_rows_of_view_requests_are_ignored():
    p = la.pack([10, 0], [1, 1], [3, 4], heads=1, ext_row=[-7, 5])
    assert list(p.branch_parent) == [-1, 0, -7]
    assert p.info.n_ext == 6


def test_kv_extents_follow_the_rows():
    """The K/V extent a cache row holds belongs to the view that stored it:
    reserving the row for another view (eviction or a direct reserve) or
    erasing the view forgets it, so a shard never reads another view's K/V."""
    c = la.ViewStateCache.__new__(la.ViewStateCache)   # directory only, no device pool
    lib = la.load_library()
    c._lib = lib
    c._h = la.ctypes.c_void_p()
    assert lib.la_cache_create(2, la.ctypes.byref(c._h)) == la.LA_OK
    c.capacity, c.kv_tokens = 2, 100
    ra, _ = c.reserve(1)
    c._kv_len[ra] = 40                       # as store(..., kv=...) records it
    rb, _ = c.reserve(2)
    c._kv_len[rb] = 70
    assert c.kv_extent(1) == (ra, ra * 100, 40) and c.kv_extent(2) == (rb, rb * 100, 70)
    rc, ev = c.reserve(3)                    # evicts the least recent: view 1
    assert ev == 1 and rc == ra and c.kv_extent(3) is None and c.kv_extent(1) is None
    assert c.kv_extent(2) == (rb, rb * 100, 70)
    c.erase(2)
    assert c.kv_extent(2) is None and rb not in c._kv_len
    c.close()
