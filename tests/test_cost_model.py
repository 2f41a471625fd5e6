"""The three-term pass cost model (host arithmetic): recovers known
constants, updates online, and reports residuals."""
import numpy as np
import pytest

from chunked_linear_attention_packed_amd import cost_model as cm


def _shapes(rng, n):
    X = []
    for _ in range(n):
        r = int(rng.integers(1, 9))
        vl = rng.integers(500, 18001, size=r)
        bc = rng.integers(1, 65, size=r)
        X.append(cm.features(vl, bc))
    return np.array(X)


def test_features():
    assert list(cm.features([100, 50], [3, 0])) == [1.0, 150.0, 3.0]
    assert list(cm.features_tokens([100], [5, 6, 7])) == [1.0, 100.0, 18.0]


def test_exact_constants_are_recovered():
    rng = np.random.default_rng(3)
    X = _shapes(rng, 30)
    c = np.array([12.5, 3.1e-3, 0.42])
    r = cm.fit(X, X @ c)
    assert np.allclose(r["c"], c, rtol=1e-9)
    assert r["r2"] == pytest.approx(1.0) and r["rel_max"] < 1e-9


def test_noisy_fit_and_residuals():
    rng = np.random.default_rng(4)
    X = _shapes(rng, 200)
    c = np.array([20.0, 2.0e-3, 0.5])
    t = X @ c * (1 + 0.02 * rng.standard_normal(len(X)))
    r = cm.fit(X, t)
    assert np.allclose(r["c"][1:], c[1:], rtol=0.05)
    assert 0.01 < r["rel_rms"] < 0.04 and r["r2"] > 0.9


def test_online_update_equals_batch_least_squares():
    rng = np.random.default_rng(5)
    X = _shapes(rng, 25)
    t = X @ np.array([5.0, 1e-3, 0.3]) + rng.uniform(0, 3, len(X))
    m = cm.CostModel()
    for x, y in zip(X, t):
        m.update(x, y)
    ref = np.linalg.lstsq(X, t, rcond=None)[0]
    assert np.allclose(m.coefficients(), ref, rtol=1e-8)
    assert m.predict(X[0]) == pytest.approx(float(X[0] @ ref), rel=1e-8)


def test_needs_three_passes():
    m = cm.CostModel()
    m.update([1, 2, 3], 1.0)
    with pytest.raises(ValueError):
        m.coefficients()
    with pytest.raises(ValueError):
        m.update([1, 2, 3, 4], 1.0)
    m4 = cm.CostModel(4)
    for _ in range(3):
        m4.update([1, 2, 3, 4], 1.0)
    with pytest.raises(ValueError):
        m4.coefficients()


def test_structural_features():
    # 7,784 tokens, 16 items x 16 heads on 256 resident workgroups
    assert list(cm.features_structural(7784, 256, 256)) == [1.0, 7784.0, 1.0]
    assert cm.features_structural(100, 257, 256)[2] == 2.0
    assert cm.features_structural(100, 0, 256)[2] == 0.0


def test_structural_constants_are_recovered():
    rng = np.random.default_rng(6)
    X = []
    for _ in range(40):
        T = int(rng.integers(600, 150000))
        items = int(rng.integers(1, 400)) * 16
        X.append(cm.features_structural(T, items, 256))
    X = np.array(X)
    c = np.array([9.0, 2.5e-3, 6.0])
    r = cm.fit(X, X @ c)
    assert np.allclose(r["c"], c, rtol=1e-7) and r["rel_max"] < 1e-9
    m = cm.CostModel(3)
    for x, y in zip(X, X @ c):
        m.update(x, y)
    assert m.predict(X[3]) == pytest.approx(float(X[3] @ c), rel=1e-9)
