"""Three-term pass cost model.

Source: "Serving 0.88M TPS from Two RTXs and Mac Minis", section "Cost
Model": the router predicts how long a pass takes from its shapes only, with
a three-constant model per node, where v_r is a request's view length and b_r
its number of branch rows; nodes measure themselves before joining and keep
refining the constants from measured pass times.  The formula itself did not
survive on the page; the plainest reading with three constants is

    t(pass) = c0 + c1 * sum_r v_r + c2 * sum_r b_r.

`CostModel` keeps the normal equations of that least-squares fit, so each
measured pass updates it in O(1) and the constants can be read at any time.
`features_tokens` gives the variant that counts branch tokens instead of
branch rows, for comparison.

`features_structural` is an extension of ours, not the page's: a pass of
this library is one launch whose time follows the tokens it moves and the
rounds of workgroups the device runs one after another (work items x heads
over the workgroups resident at once), which sums over requests do not see
(a fourth term for the longest view's block chain measured no better).  The
same least-squares machinery fits it.  Host arithmetic only.
"""
import numpy as np

__all__ = ["features", "features_tokens", "features_structural", "CostModel", "fit"]


def features(view_len, branch_count):
    """[1, sum of view lengths, number of branch rows] of one pass."""
    return np.array([1.0, float(np.sum(view_len)), float(np.sum(branch_count))])


def features_tokens(view_len, branch_len):
    """[1, sum of view lengths, sum of branch lengths] of one pass."""
    return np.array([1.0, float(np.sum(view_len)), float(np.sum(branch_len))])


def features_structural(tokens, work_items, resident):
    """[1, tokens of the pass, rounds of workgroups]: rounds =
    ceil(work_items / resident) with work_items the workgroups of the launch
    (items x heads) and resident the workgroups the device holds at once."""
    rounds = -(-int(work_items) // max(int(resident), 1))
    return np.array([1.0, float(tokens), float(rounds)])


class CostModel:
    """Least-squares fit of t = c . x over measured passes, updated one
    measurement at a time (accumulated X^T X and X^T t).  The number of
    constants is the length of the feature vectors (3 unless given)."""

    def __init__(self, n_terms=3):
        self.xtx = np.zeros((n_terms, n_terms))
        self.xtt = np.zeros(n_terms)
        self.n = 0

    def update(self, x, t):
        x = np.asarray(x, dtype=np.float64)
        if x.shape != self.xtt.shape:
            raise ValueError(f"feature vector of length {x.size}, model of {self.xtt.size} terms")
        self.xtx += np.outer(x, x)
        self.xtt += x * float(t)
        self.n += 1

    def coefficients(self):
        """(c0, c1, ...); needs as many passes as terms, with feature
        vectors that span the feature space."""
        k = self.xtt.size
        if self.n < k:
            raise ValueError(f"at least {k} measured passes are needed")
        return np.linalg.solve(self.xtx, self.xtt)

    def predict(self, x):
        return float(np.asarray(x, dtype=np.float64) @ self.coefficients())


def fit(X, t):
    """Fit t ~ X c over rows of X; returns the coefficients and residual
    statistics (relative residuals r_i = (pred_i - t_i) / t_i)."""
    X = np.asarray(X, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    m = CostModel(X.shape[1])
    for x, y in zip(X, t):
        m.update(x, y)
    c = m.coefficients()
    pred = X @ c
    rel = (pred - t) / t
    ss_res = float(np.sum((pred - t) ** 2))
    ss_tot = float(np.sum((t - t.mean()) ** 2))
    return {"c": c.tolist(), "r2": 1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0,
            "rel_rms": float(np.sqrt(np.mean(rel ** 2))), "rel_max": float(np.max(np.abs(rel))),
            "n": int(len(t))}
