"""Host-side tests of the C ABI (no GPU needed): the library loads and exports
every symbol the header declares; la_pack_pass reproduces the oracle's own
packer bit for bit on every workload; malformed shapes are rejected with the
documented status before anything is written; the work plan covers every
token exactly once with consistent state slots."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import chunked_linear_attention_packed_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "linattn.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = la.load_library()
    names = _declared_symbols()
    assert {"la_pack_pass", "la_plan_segments", "la_scan_workspace_size", "la_scan_packed",
            "la_export_view_state", "la_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_pack_matches_oracle_packer(name):
    vl, bc, bl = synth.shapes(name)
    plan = la.pack(vl, bc, bl, heads=synth.WORKLOADS[name][1])
    so, bp, vo = oracle.pack_segments(vl, bc, bl)
    assert np.array_equal(plan.seg_offsets, so)
    assert np.array_equal(plan.branch_parent, bp)
    assert np.array_equal(plan.view_ordinal, vo)
    info = plan.info
    assert info.n_tokens == int(so[-1]) and info.n_segments == len(bp)
    assert info.n_views == int((bp == -1).sum())
    _check_plan(plan, so, bp, vo)


def _fnv1a(words):
    h = 2166136261
    for w in words:
        w &= 0xFFFFFFFF
        for b in range(4):
            h ^= (w >> (8 * b)) & 0xFF
            h = (h * 16777619) & 0xFFFFFFFF
    return h


def _check_piece_tables(plan, so, bp, vo):
    """The piece path's tables against the rules they follow: blocks of 8
    chunks restarting at every segment, a state slot for every view block and
    every branch block but the last, segments' slots contiguous, branches
    whose only block is one piece (<= 128 tokens) packed into items of four
    waves (two branches of <= 64 tokens share a wave, a longer one has a wave
    alone, as few waves as that allows, in branch order), every other block
    one item in block order carrying a copy of its block; and the plan hash
    and info check."""
    info, P = plan.info, plan.plan.astype(np.int64)
    BT, PT = 8 * 64, 2 * 64
    nb_, ni, nbi, nsl, nsc = (int(x) for x in P[15:20])
    assert (nb_, ni, nbi, nsl, nsc) == (info.piece_blocks, info.piece_items,
                                        info.piece_block_items, info.piece_slots,
                                        info.piece_scans)
    ob, oi, osc = (int(x) for x in P[20:23])
    IW = 12
    assert oi == ob + 8 * nb_ and osc == oi + IW * ni and osc + 4 * nsc == info.plan_words
    blocks = P[ob:ob + 8 * nb_].reshape(-1, 8)
    items = P[oi:oi + IW * ni].reshape(-1, IW)
    scans = P[osc:osc + 4 * nsc].reshape(-1, 4)
    # expected blocks, views first then branches, in segment order
    want, slot, view_scan = [], 0, {}
    packed = []
    for pass_ in (0, 1):
        for s in range(len(bp)):
            is_view = bp[s] == -1
            if is_view != (pass_ == 0):
                continue
            n = int(so[s + 1] - so[s])
            nb = -(-n // BT)
            nsl_s = nb if is_view else nb - 1
            seed = -1 if is_view else (int(vo[bp[s]]) if bp[s] >= 0 else int(bp[s]))
            for j in range(nb):
                want.append([int(so[s]) + j * BT, min(BT, n - j * BT),
                             slot + j if j < nsl_s else -1, seed, s,
                             slot if nsl_s > 0 else -1, j,
                             int(vo[s]) if is_view and j == nb - 1 else -1])
                if not is_view and nb == 1 and n <= PT:
                    packed.append(len(want) - 1)
            if is_view:
                view_scan[int(vo[s])] = (slot, nsl_s)
            slot += nsl_s
    assert blocks.tolist() == want and slot == nsl
    kinds = items[:, 0]
    assert np.all(kinds[:nbi] == 0) and np.all(kinds[nbi:] == 1)
    singles = [i for i in range(len(want)) if i not in set(packed)]
    assert items[:nbi, 2].tolist() == singles and np.all(items[:nbi, 1] == 1)
    # a block item carries a copy of its block's 8 words
    assert np.all(items[:nbi, 3] == -1)
    assert items[:nbi, 4:12].tolist() == [want[b] for b in singles]
    assert np.all(items[nbi:, 10:] == 0)
    waves = []
    for r, row in enumerate(items[nbi:]):
        nw = int(row[1])
        assert 1 <= nw <= 4 and (nw == 4 or r == ni - nbi - 1)
        assert np.all(row[2 + 2 * nw:10] == -1)
        waves += [(int(row[2 + 2 * w]), int(row[3 + 2 * w])) for w in range(nw)]
    ntok = {b: want[b][1] for b in packed}
    got = [b for w in waves for b in w if b != -1]
    assert sorted(got) == packed and len(set(got)) == len(got)
    for b0, b1 in waves:
        assert b0 in ntok
        if b1 != -1:   # two short branches, in branch order
            assert ntok[b0] <= 64 and ntok[b1] <= 64 and b0 < b1
    assert [w[0] for w in waves] == sorted(w[0] for w in waves)
    n_short = sum(1 for b in packed if ntok[b] <= 64)
    assert len(waves) == len(packed) - n_short + -(-n_short // 2)
    for v, (first, n) in view_scan.items():
        assert scans[v].tolist() == [first, n, v, int(np.flatnonzero((bp == -1) & (vo == v))[0])]
    ph = P.copy()
    ph[14] = 0
    assert _fnv1a(ph.tolist()) == (int(P[14]) & 0xFFFFFFFF) == (info.plan_hash & 0xFFFFFFFF)
    assert (info.info_check & 0xFFFFFFFF) == la.load_library().la_info_checksum(ctypes.byref(info))


def _check_plan(plan, so, bp, vo):
    """Every token in exactly one block; blocks never cross segments; slots of
    a segment are contiguous, the delta list matches the blocks, and the scan
    list covers views plus branches with >= 2 slots."""
    info, P = plan.info, plan.plan
    G, C = info.block_chunks, info.chunk
    assert P[0] == 0x4C41504E and P[1] == 5
    assert (P[2], P[3], P[4]) == (info.n_blocks, info.n_delta, info.n_scan)
    ob, od, osc = P[8], P[9], P[10]
    blocks = P[ob:ob + 8 * info.n_blocks].reshape(-1, 8)
    deltas = P[od:od + 4 * info.n_delta].reshape(-1, 4)
    scans = P[osc:osc + 4 * info.n_scan].reshape(-1, 4)
    assert osc + 4 * info.n_scan == P[20]
    _check_piece_tables(plan, so, bp, vo)
    cover = np.zeros(info.n_tokens, dtype=np.int64)
    seg_blocks = {}
    fused_reads = 0
    for tok0, ntok, sin, dsl, seed, seg, slot0, frow in blocks:
        assert 1 <= ntok <= G * C
        assert so[seg] <= tok0 and tok0 + ntok <= so[seg + 1]
        cover[tok0:tok0 + ntok] += 1
        seg_blocks.setdefault(seg, []).append((tok0, sin, dsl, seed, slot0, frow))
        p = bp[seg]
        assert seed == (-1 if p == -1 else (vo[p] if p >= 0 else p))
        # two-launch form: own prefix = slots slot0 .. sin; a branch's seed =
        # the slots of its view's scan entry, which sits at index vo[p]
        j = (tok0 - so[seg]) // (G * C)
        if sin >= 0:
            assert slot0 >= 0 and sin - slot0 + 1 == j
        fused_reads += j
        if p >= 0:
            first, n, frow_v, seg_v = scans[vo[p]]
            assert seg_v == p and frow_v == vo[p]
            fused_reads += n
        last = tok0 + ntok == so[seg + 1]
        assert frow == (vo[seg] if (p == -1 and last) else -1)
        if frow >= 0:
            fused_reads += 1
    assert np.all(cover == 1)
    assert info.fused_slot_reads == fused_reads == P[13]
    dl = {int(r[2]): r for r in deltas}
    seen_views = 0
    for seg, bl in seg_blocks.items():
        bl.sort()
        first = None
        for j, (tok0, sin, dsl, seed, slot0, _) in enumerate(bl):
            assert tok0 == so[seg] + j * G * C
            if j == 0:
                assert sin == -1
            else:
                assert sin == bl[j - 1][2]
            if dsl >= 0:
                first = dsl - j if first is None else first
                assert dsl == first + j and dl[dsl][0] == tok0
                assert slot0 == first
        if bp[seg] == -1:
            seen_views += 1
            assert all(b[2] >= 0 for b in bl)
        else:
            assert bl[-1][2] == -1
    assert seen_views == info.n_views
    for first, n, frow, seg in scans:
        if frow >= 0:
            assert bp[seg] == -1 and vo[seg] == frow
        else:
            assert bp[seg] != -1 and n >= 2


@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_plan_random_structures(G):
    rng = np.random.default_rng(G)
    for _ in range(20):
        R = int(rng.integers(1, 6))
        vl = rng.integers(0, 700, size=R)
        bc = rng.integers(0, 5, size=R)
        bc[vl == 0] = np.maximum(bc[vl == 0], 1)
        bl = rng.integers(1, 300, size=int(bc.sum()))
        plan = la.pack(vl, bc, bl, block_chunks=G)
        so, bp, vo = oracle.pack_segments(vl, bc, bl)
        assert np.array_equal(plan.seg_offsets, so) and np.array_equal(plan.branch_parent, bp)
        assert plan.info.n_ext == int((vl == 0).sum())
        _check_plan(plan, so, bp, vo)


def test_plan_segments_any_order():
    # branches listed before their view; two views
    so = [0, 5, 9, 109, 110, 250]
    bp = [2, 2, -1, -1, 3]
    plan = la.plan_segments(so, bp, block_chunks=1)
    assert plan.view_ordinal.tolist() == [-1, -1, 0, 1, -1]
    _check_plan(plan, np.asarray(so), np.asarray(bp), plan.view_ordinal)


@pytest.mark.parametrize("vl,bc,bl", [
    ([3], [1], [0]),            # empty branch
    ([0], [0], []),             # empty request
    ([-1], [1], [2]),           # negative view
    ([3], [-1], []),            # negative count
    ([2**31 - 10], [1], [20]),  # token count overflows int32
])
def test_pack_rejects_bad_shapes(vl, bc, bl):
    with pytest.raises(la.LinAttnError) as e:
        la.pack(vl, bc, bl, block_chunks=1)
    assert e.value.status == la.LA_ERR_INVALID_ARG


@pytest.mark.parametrize("so,bp", [
    ([0, 5, 5], [-1, 0]),       # zero-length segment
    ([0, 5, 9], [-1, 1]),       # parent is a branch (itself)
    ([0, 5, 9], [-1, 7]),       # parent out of range
    ([1, 5, 9], [-1, 0]),       # offsets do not start at 0
    ([0, 5, 9], [0, -1]),       # view's parent points at a view... segment 0 parent 0 is a view? no: 0 -> itself
])
def test_plan_segments_rejects_bad_tables(so, bp):
    with pytest.raises(la.LinAttnError) as e:
        la.plan_segments(so, bp, block_chunks=1)
    assert e.value.status == la.LA_ERR_INVALID_ARG


def test_unsupported_chunk_and_dims():
    lib = la.load_library()
    info = la.PassInfo()
    vl = np.array([10], dtype=np.int32)
    bc = np.array([0], dtype=np.int32)
    st = lib.la_pack_pass(1, vl.ctypes.data_as(la._I32P), bc.ctypes.data_as(la._I32P), None,
                          32, 1, None, None, None, None, ctypes.byref(info))
    assert st == la.LA_ERR_UNSUPPORTED
    plan = la.pack([10], [0], [], block_chunks=1)
    n = ctypes.c_size_t()
    assert lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 96, 96, la.LA_BF16,
                                      ctypes.byref(n)) == la.LA_ERR_UNSUPPORTED
    assert lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 64, 128, la.LA_BF16,
                                      ctypes.byref(n)) == la.LA_ERR_UNSUPPORTED
    assert lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 64, 64, 7,
                                      ctypes.byref(n)) == la.LA_ERR_UNSUPPORTED
    assert lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 64, 64, la.LA_F32,
                                      ctypes.byref(n)) == la.LA_OK
    # a 256-byte header, then one fp32 state per delta block and head
    assert n.value == 256 + plan.info.n_delta * 2 * 64 * 64 * 4
    assert lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 64, 64, la.LA_BF16,
                                      ctypes.byref(n)) == la.LA_OK
    # piece path: header, a flag per slot and head (rounded to 256 bytes), then
    # block states and inclusive prefixes
    nsh = plan.info.piece_slots * 2
    assert n.value == 256 + -(-nsh * 8 // 256) * 256 + 2 * nsh * 64 * 64 * 4


def test_scan_rejects_bad_arguments_before_launch():
    """Host-side validation returns an error without touching the device, so
    it runs without a GPU: NULL pointers, unsupported shapes, a missing or too
    small workspace, missing ext_state for a shard pass."""
    lib = la.load_library()
    plan = la.pack([100], [2], [10, 20], block_chunks=1)
    info = plan.info
    fake = ctypes.c_void_p(4096)   # never dereferenced: every case fails validation first
    need = ctypes.c_size_t()
    lib.la_scan_workspace_size(ctypes.byref(info), 2, 64, 64, la.LA_BF16, ctypes.byref(need))
    args = dict(q=fake, k=fake, v=fake, dtype=la.LA_BF16, H=2, dk=64, dv=64, plan=fake,
                ext=None, n_ext=0, out=fake, fin=fake, ws=fake, wsb=need.value)

    def call(**kw):
        a = dict(args, **kw)
        return lib.la_scan_packed(a["q"], a["k"], a["v"], a["dtype"], a["H"], a["dk"], a["dv"],
                                  ctypes.byref(info), a["plan"], a["ext"], a["n_ext"], a["out"],
                                  a["fin"], a["ws"], a["wsb"], None)
    assert call(q=None) == la.LA_ERR_INVALID_ARG
    assert call(out=None) == la.LA_ERR_INVALID_ARG
    assert call(fin=None) == la.LA_ERR_INVALID_ARG
    assert call(plan=None) == la.LA_ERR_INVALID_ARG
    assert call(H=0) == la.LA_ERR_INVALID_ARG
    assert call(dk=96, dv=96) == la.LA_ERR_UNSUPPORTED
    assert call(dtype=5) == la.LA_ERR_UNSUPPORTED
    assert call(ws=None) == la.LA_ERR_WORKSPACE
    assert call(wsb=need.value - 1) == la.LA_ERR_WORKSPACE
    assert call(q=ctypes.c_void_p(4098)) == la.LA_ERR_INVALID_ARG   # misaligned
    assert call(fin=ctypes.c_void_p(4098)) == la.LA_ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(4100)) == la.LA_ERR_INVALID_ARG
    assert call(plan=ctypes.c_void_p(4097)) == la.LA_ERR_INVALID_ARG
    assert call(dtype=la.LA_F32_SPLIT, dk=96, dv=96) == la.LA_ERR_UNSUPPORTED

    def staged(stages, **kw):
        a = dict(args, **kw)
        return lib.la_scan_packed_stages(stages, a["q"], a["k"], a["v"], a["dtype"], a["H"],
                                         a["dk"], a["dv"], ctypes.byref(info), a["plan"],
                                         a["ext"], a["n_ext"], a["out"], a["fin"], a["ws"],
                                         a["wsb"], None)
    assert staged(la.STAGE_ALL | la.FORM_ONE_LAUNCH | la.FORM_TWO_LAUNCH) == la.LA_ERR_INVALID_ARG
    assert staged(la.FORM_ONE_LAUNCH) == la.LA_ERR_INVALID_ARG        # no stage bit
    assert staged(la.STAGE_ALL | 256) == la.LA_ERR_INVALID_ARG        # unknown bit
    need32 = ctypes.c_size_t()
    lib.la_scan_workspace_size(ctypes.byref(info), 2, 64, 64, la.LA_F32, ctypes.byref(need32))
    # the single-launch form and its timeout aid exist on the piece path only
    assert staged(la.STAGE_ALL | la.FORM_ONE_LAUNCH, dtype=la.LA_F32,
                  wsb=need32.value) == la.LA_ERR_UNSUPPORTED
    assert staged(la.STAGE_ALL | la.DEBUG_FORCE_TIMEOUT, dtype=la.LA_F32,
                  wsb=need32.value) == la.LA_ERR_UNSUPPORTED
    assert staged(la.STAGE_ALL | la.DEBUG_ORDERED, dtype=la.LA_F32,
                  wsb=need32.value) == la.LA_ERR_UNSUPPORTED
    shard = la.pack([0], [2], [10, 20], block_chunks=1)
    st = lib.la_scan_packed(fake, fake, fake, la.LA_BF16, 2, 64, 64, ctypes.byref(shard.info),
                            fake, None, 0, fake, None, fake, 1 << 20, None)
    assert st == la.LA_ERR_INVALID_ARG
    assert lib.la_export_view_state(fake, 3, 2, 2, 64, 64, fake, None) == la.LA_ERR_INVALID_ARG
    assert lib.la_export_view_state(fake, 0, 2, 2, 96, 96, fake, None) == la.LA_ERR_UNSUPPORTED


def test_scan_launches_by_pass_shape():
    """d = 64 with bf16 inputs runs the single-launch piece path.  Otherwise
    the two-launch form is taken while the workspace reads it adds stay small
    (fused_slot_reads x H x d^2 x 4 bytes up to 128 MiB): the 628- and
    7,400-token passes (one view of 15 blocks, 8 one-block branches: 58 MB)
    qualify; the view of 18,000 tokens with 256 branches (each branch reading
    all view slots: 1.25 GB) does not."""
    w7 = synth.shapes("view7400_br8x48_h16_d64_bf16")
    p7 = la.pack(*w7, heads=16)
    nb = -(-7400 // (64 * p7.info.block_chunks))
    assert p7.info.fused_slot_reads == nb * (nb - 1) // 2 + 1 + 8 * nb
    assert la.scan_launches(p7, 16, 64, la.LA_BF16) == 1
    assert la.scan_launches(p7, 16, 128, la.LA_BF16) == 3   # 4x the slot bytes at d 128
    assert la.scan_launches(p7, 16, 64, la.LA_F32) == 2
    w1 = synth.shapes("view500_br4x32_h2_d64_f32")
    assert la.scan_launches(la.pack(*w1, heads=2), 2, 64, la.LA_F32) == 2
    w4 = synth.shapes("view18000_br256x32-128_h16_d64_bf16")
    assert la.scan_launches(la.pack(*w4, heads=16), 16, 64, la.LA_F32_SPLIT) == 3
    # a view of two one-chunk blocks: the second block reads the first slot,
    # and its own to write final_state
    p1 = la.pack([100], [0], [], block_chunks=1)
    assert p1.info.fused_slot_reads == 1 + 1 and la.scan_launches(p1, 1, 64, la.LA_F32) == 2
    with pytest.raises(la.LinAttnError):
        la.scan_launches(p1, 0, 64)
    with pytest.raises(la.LinAttnError):
        la.scan_launches(p1, 1, 96)


@pytest.mark.parametrize("field", ["n_blocks", "n_tokens", "piece_items", "plan_hash",
                                   "n_views"])
def test_edited_pass_info_is_rejected_before_launch(field):
    """A pass info whose fields no longer match its checksum (edited, or
    mixed from two passes) is rejected on the host, without device work."""
    lib = la.load_library()
    plan = la.pack([300, 90], [2, 1], [10, 20, 70], heads=2)
    info = la.PassInfo.from_buffer_copy(plan.info)
    setattr(info, field, getattr(info, field) + 1)
    fake = ctypes.c_void_p(4096)
    need = ctypes.c_size_t()
    lib.la_scan_workspace_size(ctypes.byref(plan.info), 2, 64, 64, la.LA_BF16,
                               ctypes.byref(need))
    st = lib.la_scan_packed(fake, fake, fake, la.LA_BF16, 2, 64, 64, ctypes.byref(info), fake,
                            None, 0, fake, fake, fake, need.value + (1 << 20), None)
    assert st == la.LA_ERR_INVALID_ARG
    assert lib.la_info_checksum(ctypes.byref(info)) != (info.info_check & 0xFFFFFFFF)


def test_block_size_choice_on_the_workloads():
    """The binding's block size: the largest power of two up to 16 chunks that
    keeps >= 300 workgroups, doubled up to 64 while the views alone keep
    >= 2048 workgroups (the choices measured fastest on MI355X)."""
    expect = {"view7400_br8x48_h16_d64_bf16": (16, 8),
              "req4_view500-18000_br8x24-96_h16_d64_bf16": (16, 16),
              "view18000_br256x32-128_h16_d64_bf16": (16, 16),
              "req32_view500-18000_br1-64x24-128_h32_d128_bf16": (32, 64)}
    for name, (H, G) in expect.items():
        assert la.pack(*synth.shapes(name), heads=H).info.block_chunks == G, name
    def table(lens, parents):
        return np.r_[0, np.cumsum(lens)].astype(np.int32), np.asarray(parents, dtype=np.int32)
    # views too short for 2048 long workgroups stay at 16 (4 views of 300 chunks)
    so, bp = table([300 * 64] * 4, [-1] * 4)
    assert la.choose_block_chunks(so, bp, 16) == 16
    so, bp = table([300 * 64] * 64, [-1] * 64)
    assert la.choose_block_chunks(so, bp, 32) == 64
    # branches count towards the 300 workgroups but not towards 2048
    so, bp = table([3 * 64] + [64] * 400, [-1] + [0] * 400)
    assert la.choose_block_chunks(so, bp, 1) == 16
    so, bp = table([3 * 64], [-1])
    assert la.choose_block_chunks(so, bp, 2) == 1
    with pytest.raises(la.LinAttnError):
        la.choose_block_chunks(so, bp, 0)
    so, bp = table([5, 0], [-1, 0])
    with pytest.raises(la.LinAttnError):
        la.choose_block_chunks(so, bp, 2)


def test_stage_and_form_bits_checked_before_any_device_work():
    """la_scan_packed_stages rejects unknown bits, a mask without launches and
    both form bits at once, on the host, before it looks at any pointer; an
    empty pass with valid bits returns LA_OK without touching the device."""
    lib = la.load_library()
    info = la.PassInfo()
    info.chunk = la.CHUNK
    info.info_check = lib.la_info_checksum(ctypes.byref(info))

    def call(stages):
        return lib.la_scan_packed_stages(stages, None, None, None, la.LA_BF16, 1, 64, 64,
                                         ctypes.byref(info), None, None, 0, None, None, None,
                                         0, None)
    assert call(la.STAGE_ALL) == la.LA_OK
    assert call(la.STAGE_ALL | la.FORM_TWO_LAUNCH) == la.LA_OK
    assert call(la.STAGE_OUTPUT | la.FORM_THREE_LAUNCH) == la.LA_OK
    assert call(la.STAGE_ALL | la.FORM_ONE_LAUNCH) == la.LA_OK
    assert call(la.STAGE_ALL | la.FORM_ONE_LAUNCH | la.DEBUG_ORDERED) == la.LA_OK
    for bad in (0, la.FORM_TWO_LAUNCH, la.STAGE_ALL | la.FORM_TWO_LAUNCH | la.FORM_THREE_LAUNCH,
                la.STAGE_ALL | la.FORM_ONE_LAUNCH | la.FORM_THREE_LAUNCH, la.STAGE_ALL | 256,
                -1):
        assert call(bad) == la.LA_ERR_INVALID_ARG, bad


def test_ext_state_overlapping_final_state_rejected():
    """final_state is written while ext_state is read (in the two-launch form
    by the same launch), so overlapping buffers are refused on the host
    before any device work (the pointers here are never dereferenced)."""
    lib = la.load_library()
    p = la.pack([100, 0], [1, 1], [30, 40], heads=2)
    assert p.info.n_views == 1 and p.info.n_ext == 1
    plan = p.plan
    st = 2 * 64 * 64 * 4
    base = 1 << 20                     # fake, aligned, never touched
    fake = ctypes.c_void_p(base)
    for ext in (base, base + st - 16, base - st + 16):
        r = lib.la_scan_packed_stages(la.STAGE_ALL, fake, fake, fake, la.LA_BF16, 2, 64, 64,
                                      ctypes.byref(p.info), fake, ctypes.c_void_p(ext), 1,
                                      fake, ctypes.c_void_p(base), None, 0, None)
        assert r == la.LA_ERR_INVALID_ARG, hex(ext)
    del plan


def test_noalloc_rejects_passes_beyond_its_scratch():
    """la_scan_packed_noalloc checks the pass's workspace against its built-in
    array on the host and returns LA_ERR_TOO_LARGE before any device work (so
    this runs without a GPU)."""
    lib = la.load_library()
    fake = ctypes.c_void_p(16)
    # one view of 2^17 tokens: fp32 in blocks of one chunk (2048 states of
    # 16 KiB per head, 128 MiB at 4 heads); bf16 on the piece path (256
    # blocks, a state and a prefix each, 16 heads: 128 MiB)
    for dtype, H, G in ((la.LA_F32, 4, 1), (la.LA_BF16, 16, 8)):
        plan = la.pack([1 << 17], [0], [], heads=H, block_chunks=G)
        need = la.workspace_size(plan, H, 64, dtype)
        assert need > la.NOALLOC_SCRATCH_BYTES
        st = lib.la_scan_packed_noalloc(fake, fake, fake, dtype, H, 64, 64,
                                        ctypes.byref(plan.info), fake, None, 0, fake, fake,
                                        None)
        assert st == la.LA_ERR_TOO_LARGE
        assert b"scratch" in lib.la_status_string(st)
