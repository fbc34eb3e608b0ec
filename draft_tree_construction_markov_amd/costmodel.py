"""Cost-model tooling for the adaptive build (host side, no GPU work).

The CaDDTree summary ("Method", cost profiling) models the cost of a
speculative round as the drafter's fixed cost plus a verification cost that
grows with the tree size n and the context length l, profiled once per
deployment and required to be convex and increasing in n for the greedy
stop to be optimal.  With C_v(n; l) = c0 + c1 n + c2 n^2 + c_ell l n that
holds exactly when every coefficient is non-negative, so the fit below is a
non-negative least-squares regression on the features (1, n, n^2, l n).

robustness() measures what a wrong cost model costs: every round keeps the
budget that its (perturbed or fitted) model chooses, and the result is the
throughput those budgets reach under the true model, relative to the best
budgets.  It works on throughput curves f(n) = (1 + Phi_n) / D(n) of
best-first-ordered trees, supplied by a callable (the library's
pct_throughput_curve on the GPU, or any other implementation).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

FEATURES = ("c0", "c1", "c2", "c_ell")


@dataclass
class Fit:
    """A fitted verification cost C_v(n; l) = c0 + c1 n + c2 n^2 +
    c_ell l n, with its residual spread on the samples."""
    c0: float
    c1: float
    c2: float
    c_ell: float
    rms: float  # root-mean-square residual of the samples
    max_rel: float  # largest |residual| / sample

    def cost(self, C_d: float) -> dict:
        """The round cost model C(n; l) = C_d + C_v(n; l) in the form the
        library takes."""
        return dict(C_d=float(C_d), c0=self.c0, c1=self.c1, c2=self.c2,
                    c_ell=self.c_ell)


def design(n, ell) -> np.ndarray:
    n = np.asarray(n, np.float64)
    ell = np.asarray(ell, np.float64)
    return np.stack([np.ones_like(n), n, n * n, ell * n], axis=1)


def predict(c: dict | Fit, n, ell) -> np.ndarray:
    if isinstance(c, Fit):
        c = c.cost(0.0)
    return design(n, ell) @ np.array([c["c0"], c["c1"], c["c2"], c["c_ell"]])


def fit(n, ell, latency, weights=None) -> Fit:
    """Non-negative least squares of latency samples (tree size n, context
    length l, measured verification time) on (1, n, n^2, l n).  Columns
    are scaled to unit norm before the solve so that the coefficients of
    very different magnitudes are resolved equally well; `weights`
    (optional) weight the squared residuals (e.g. 1/latency^2 for a
    relative-error fit)."""
    from scipy.optimize import nnls
    X = design(n, ell)
    y = np.asarray(latency, np.float64)
    if X.shape[0] < 1 or X.shape[0] != y.shape[0]:
        raise ValueError("need as many latencies as (n, l) samples")
    if weights is not None:
        w = np.sqrt(np.asarray(weights, np.float64))
        Xw, yw = X * w[:, None], y * w
    else:
        Xw, yw = X, y
    scale = np.linalg.norm(Xw, axis=0)
    scale[scale == 0] = 1.0
    coef, _ = nnls(Xw / scale, yw)
    coef = coef / scale
    res = X @ coef - y
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(y != 0, np.abs(res) / np.abs(y), 0.0)
    return Fit(*(float(c) for c in coef), rms=float(np.sqrt(np.mean(res ** 2))),
               max_rel=float(rel.max()))


def convex_increasing(c: dict | Fit) -> bool:
    """C_v is convex and non-decreasing in n for every l >= 0."""
    if isinstance(c, Fit):
        c = c.cost(0.0)
    return all(c[k] >= 0.0 for k in ("c1", "c2", "c_ell"))


def first_argmax(f: np.ndarray) -> np.ndarray:
    """Per row, the smallest n where f(n) is largest (the greedy stop's
    choice on a unimodal curve)."""
    return np.argmax(f, axis=1)


def perturbed(cost: dict, factors: dict) -> dict:
    """cost with each named coefficient multiplied by its factor."""
    out = dict(cost)
    for k, v in factors.items():
        out[k] = cost[k] * v
    return out


def robustness(curve, true_cost: dict, models: dict) -> dict:
    """For each named cost model, the throughput every round reaches when
    it keeps the budget that model chooses, measured under true_cost.

    curve(cost) -> f [rounds][N+1]: throughput of each prefix length.
    Returns {name: dict(mean_f, rel_loss, mean_budget)}, rel_loss being
    1 - mean_f / (mean of the per-round best f under the true model)."""
    f_true = np.asarray(curve(true_cost), np.float64)
    rows = np.arange(f_true.shape[0])
    best = f_true.max(axis=1).mean()
    out = {}
    for name, c in models.items():
        n_pick = first_argmax(np.asarray(curve(c), np.float64))
        got = f_true[rows, n_pick]
        out[name] = dict(mean_f=float(got.mean()),
                         rel_loss=float(1.0 - got.mean() / best),
                         mean_budget=float(n_pick.mean()))
    return out
