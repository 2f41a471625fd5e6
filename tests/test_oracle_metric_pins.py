"""Pins for the error metric and for the oracle's external-state paths.

Every GPU parity verdict is a comparison row_rel_err(out, ref) <= tol (or
state_rel_err for final states), with the error "normalised per output row":
for each row, max_j |o - o*| divided by max_j |o*| of that row, the divisor
floored at 1e-6 times the largest |o*| of the whole array.  The values below
are worked out by hand (in the comments), and copies of the metric with a
plausible mistake planted in them must each miss at least one of them.

The external-state tests pin the branch-shard path of the oracle (section
"Long Requests" of "Serving 0.88M TPS from Two RTXs and Mac Minis": a shard's
branches start from the cached view state): a hand-worked shard pass, and the
three evaluators (recurrence, explicit mask, chunked) agreeing when ext_state
is given.
"""
import numpy as np
import pytest

import oracle
from oracle import metrics

# 3 rows x 4 columns.  Largest |ref| of the array: 2000, so the floor is
# 1e-6 * 2000 = 2e-3.
REF = np.array([[1000.0, -2000.0, 500.0, 0.0],      # row max 2000
                [1e-4, -5e-4, 0.0, 2e-4],            # row max 5e-4 < floor 2e-3
                [1.0, -3.0, 2.0, 0.5]])              # row max 3
ERR = np.array([[2.0, 0.0, -4.0, 0.0],               # row max |err| 4
                [0.0, 1e-5, 0.0, -3e-5],             # 3e-5
                [0.0, 0.03, 0.0, 0.0]])              # 0.03
# per row: 4 / 2000 = 2e-3;  3e-5 / max(5e-4, 2e-3) = 1.5e-2;  0.03 / 3 = 1e-2
ROW_ERRS = [2e-3, 1.5e-2, 1e-2]


def _planted_global_max(out, ref):
    """Mistake: one divisor for the whole array (its largest |ref|)."""
    out, ref = np.asarray(out), np.asarray(ref)
    return float(np.abs(out - ref).max() / np.abs(ref).max())


def _planted_axis0(out, ref):
    """Mistake: maxima taken down the columns instead of along each row."""
    out, ref = np.asarray(out), np.asarray(ref)
    num = np.abs(out - ref).max(axis=0)
    den = np.abs(ref).max(axis=0)
    floor = 1e-6 * float(np.abs(ref).max())
    return float((num / np.maximum(den, floor)).max())


def _planted_no_floor(out, ref):
    """Mistake: the row's own maximum with no floor."""
    out, ref = np.asarray(out), np.asarray(ref)
    return float((np.abs(out - ref).max(axis=-1) / np.abs(ref).max(axis=-1)).max())


def _planted_mean(out, ref):
    """Mistake: mean instead of max over the row's errors."""
    out, ref = np.asarray(out), np.asarray(ref)
    num = np.abs(out - ref).mean(axis=-1)
    den = np.abs(ref).max(axis=-1)
    floor = 1e-6 * float(np.abs(ref).max())
    return float((num / np.maximum(den, floor)).max())


def _check_row_metric(fn):
    """True if fn gives the hand-computed values on every sub-case."""
    cases = [
        ([0, 1, 2], max(ROW_ERRS)),      # 1.5e-2, the floored row
        ([0, 2], 1e-2),                  # row 2 is large only against its own max
        ([0], 2e-3),
        ([0, 1], 1.5e-2),
    ]
    for rows, want in cases:
        got = fn(REF[rows] + ERR[rows], REF[rows])
        if not np.isclose(got, want, rtol=1e-12, atol=0.0):
            return False
    return True


def test_row_rel_err_hand_values():
    # rows 1 and 2 without row 0: the array maximum is 3, the floor 3e-6 no
    # longer binds for row 1, which gives 3e-5 / 5e-4 = 6e-2
    for rows, want in (([0, 1, 2], 1.5e-2), ([0, 2], 1e-2), ([0], 2e-3), ([2], 1e-2),
                       ([1, 2], 6e-2)):
        got = oracle.row_rel_err(REF[rows] + ERR[rows], REF[rows])
        assert np.isclose(got, want, rtol=1e-12, atol=0.0), (rows, got, want)


def test_row_rel_err_floor_uses_whole_array():
    """Row 1 alone: its own maximum 5e-4 is then the array maximum, so the
    floor is 5e-10 and does not bind: 3e-5 / 5e-4 = 6e-2."""
    got = oracle.row_rel_err(REF[[1]] + ERR[[1]], REF[[1]])
    assert np.isclose(got, 6e-2, rtol=1e-12)


def test_row_rel_err_rows_are_last_axis_of_any_rank():
    """[T, H, d] arrays: a row is one (token, head); permuting rows leaves the
    result unchanged, and a 3-D layout gives the 2-D value."""
    ref3 = REF.reshape(3, 1, 4)
    out3 = (REF + ERR).reshape(3, 1, 4)
    assert np.isclose(oracle.row_rel_err(out3, ref3), 1.5e-2, rtol=1e-12)
    perm = [2, 0, 1]
    assert np.isclose(oracle.row_rel_err((REF + ERR)[perm], REF[perm]), 1.5e-2, rtol=1e-12)


def test_row_rel_err_exact_and_zero_reference():
    assert oracle.row_rel_err(REF, REF) == 0.0
    z = np.zeros((2, 3))
    # all-zero reference: the error is reported as the absolute maximum
    assert oracle.row_rel_err(z + np.array([[0, 0.5, 0], [0, 0, 0]]), z) == 0.5
    assert oracle.row_rel_err(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0
    with pytest.raises(ValueError):
        oracle.row_rel_err(np.zeros((2, 3)), np.zeros((3, 2)))


@pytest.mark.parametrize("planted", [_planted_global_max, _planted_axis0, _planted_no_floor,
                                     _planted_mean])
def test_planted_metric_mistakes_are_caught(planted):
    assert _check_row_metric(metrics.row_rel_err)
    assert not _check_row_metric(planted)


# Final states: [n_views, H, d_k, d_v]; the "row" is one (view, head) matrix.
# Two views x two heads of 2 x 2 matrices.  Array maximum 100, floor 1e-4.
ST_REF = np.array([[[[100.0, 0.0], [0.0, 50.0]],        # (0, 0): max 100
                    [[1.0, 2.0], [0.0, 0.0]]],          # (0, 1): max 2
                   [[[0.0, 4.0], [0.0, 0.0]],           # (1, 0): max 4
                    [[1e-6, 0.0], [0.0, 0.0]]]])        # (1, 1): max 1e-6 < floor 1e-4
ST_ERR = np.array([[[[0.5, 0.0], [0.0, 0.0]],           # 0.5 / 100 = 5e-3
                    [[0.0, 0.0], [0.02, 0.0]]],         # 0.02 / 2 = 1e-2
                   [[[0.0, 0.0], [0.0, 0.01]],          # 0.01 / 4 = 2.5e-3
                    [[0.0, 0.0], [0.0, 1e-7]]]])        # 1e-7 / 1e-4 = 1e-3
# maximum over (view, head) matrices: 1e-2


def _state_wrong_flatten(st, ref):
    """Mistake: one row per (view, head, k) -- the last axis only."""
    return metrics.row_rel_err(st, ref)


def _state_per_view(st, ref):
    """Mistake: one row per view (all heads together)."""
    st, ref = np.asarray(st), np.asarray(ref)
    return metrics.row_rel_err(st.reshape(st.shape[0], -1), ref.reshape(ref.shape[0], -1))


def test_state_rel_err_hand_values():
    assert np.isclose(oracle.state_rel_err(ST_REF + ST_ERR, ST_REF), 1e-2, rtol=1e-12)
    # the (1, 1) matrix alone: its own max 1e-6 is the array max, floor 1e-12
    assert np.isclose(oracle.state_rel_err(ST_REF[1:, 1:] + ST_ERR[1:, 1:], ST_REF[1:, 1:]),
                      1e-1, rtol=1e-12)
    # without head 1: max(5e-3, 2.5e-3)
    assert np.isclose(oracle.state_rel_err(ST_REF[:, :1] + ST_ERR[:, :1], ST_REF[:, :1]),
                      5e-3, rtol=1e-12)


@pytest.mark.parametrize("planted", [_state_wrong_flatten, _state_per_view])
def test_planted_state_metric_mistakes_are_caught(planted):
    """(view 0, head 1): per-k rows would give 0.02 / 0 -> floored 0.02 / 1e-4
    = 200; per-view rows 0.02 / 100 = 2e-4 for view 0."""
    want = 1e-2
    assert np.isclose(oracle.state_rel_err(ST_REF + ST_ERR, ST_REF), want, rtol=1e-12)
    assert not np.isclose(planted(ST_REF + ST_ERR, ST_REF), want, rtol=1e-6)


# ---------------------------------------------------------------------------
# External states (shard passes)
# ---------------------------------------------------------------------------
def test_shard_pass_hand_worked():
    """One shard request: a branch of two tokens seeded from an external state
    E (d_k = d_v = 2, one head).  By hand:
        S_0 = E + k_0^T v_0 = [[1, 2], [3, 4]] + [[0, 1], [0, 0]] = [[1, 3], [3, 4]]
        o_0 = q_0 S_0 = [1, 1] S_0 = [4, 7]
        S_1 = S_0 + k_1^T v_1 = [[1, 3], [3, 4]] + [[0, 0], [2, 0]] = [[1, 3], [5, 4]]
        o_1 = q_1 S_1 = [1, -1] S_1 = [-4, -1]
    """
    E = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])             # [n_ext=1, H=1, 2, 2]
    q = np.array([[[1.0, 1.0]], [[1.0, -1.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = np.array([[[0.0, 1.0]], [[2.0, 0.0]]])
    so, bp, _ = oracle.pack_segments([0], [1], [2])
    assert bp.tolist() == [-2]
    want = np.array([[4.0, 7.0], [-4.0, -1.0]])
    for fn in ("recurrence", "bruteforce", "chunked1", "chunked2", "sample"):
        if fn == "recurrence":
            out, fin = oracle.scan_recurrence(q, k, v, so, bp, ext_state=E)
        elif fn == "bruteforce":
            out, fin = oracle.scan_bruteforce(q, k, v, so, bp, ext_state=E)
        elif fn == "sample":
            out = oracle.sample_rows(q, k, v, so, bp, [0, 1], ext_state=E)
            fin = np.zeros((0,))
        else:
            out, fin = oracle.scan_chunked(q, k, v, so, bp, int(fn[7:]), ext_state=E)
        assert np.array_equal(out[:, 0, :], want), fn
        assert fin.shape[0] == 0


def _ext_pass(rng, H, dk, dv):
    """Random pass mixing views, branches of views and shard requests."""
    vl = [int(rng.integers(1, 90)), 0, int(rng.integers(1, 70)), 0]
    bc = [int(rng.integers(0, 4)), int(rng.integers(1, 4)), int(rng.integers(0, 3)),
          int(rng.integers(1, 3))]
    bl = rng.integers(1, 80, size=sum(bc)).tolist()
    so, bp, _ = oracle.pack_segments(vl, bc, bl)
    T = int(so[-1])
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    ext = rng.standard_normal((2, H, dk, dv)) * 3.0
    return so, bp, q, k, v, ext


@pytest.mark.parametrize("seed", range(4))
def test_ext_state_evaluators_agree(seed):
    rng = np.random.default_rng(500 + seed)
    so, bp, q, k, v, ext = _ext_pass(rng, 2, 3, 5)
    assert (np.asarray(bp) <= -2).any()
    ro, rf = oracle.scan_recurrence(q, k, v, so, bp, ext_state=ext)
    bo, bf = oracle.scan_bruteforce(q, k, v, so, bp, ext_state=ext)
    assert oracle.row_rel_err(bo, ro) < 1e-12
    assert oracle.state_rel_err(bf, rf) < 1e-12
    for chunk in (1, 3, 16, 64):
        co, cf = oracle.scan_chunked(q, k, v, so, bp, chunk, ext_state=ext)
        assert oracle.row_rel_err(co, ro) < 1e-12
        assert oracle.state_rel_err(cf, rf) < 1e-12
    rows = np.arange(0, int(so[-1]), 3)
    so_ = np.asarray(so)
    sr = oracle.sample_rows(q, k, v, so_, bp, rows, ext_state=ext)
    assert oracle.row_rel_err(sr, ro[rows]) < 1e-12


def test_ext_state_is_additive():
    """A shard branch's outputs are its zero-seeded outputs plus q_t E: the
    seed enters linearly (closed form with ext)."""
    rng = np.random.default_rng(77)
    so, bp, _ = oracle.pack_segments([0], [2], [5, 9])
    T = int(so[-1])
    q, k, v = (rng.standard_normal((T, 2, 4)) for _ in range(3))
    E = rng.standard_normal((1, 2, 4, 4))
    with_e, _ = oracle.scan_recurrence(q, k, v, so, bp, ext_state=E)
    zero, _ = oracle.scan_recurrence(q, k, v, so, bp, ext_state=np.zeros_like(E))
    want = zero + np.einsum("thk,hkv->thv", q, E[0])
    assert oracle.row_rel_err(with_e, want) < 1e-13
