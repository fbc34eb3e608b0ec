"""CPU checks of the cost-model tooling (draft_tree_construction_markov_amd.
costmodel): the non-negative fit recovers a known convex cost, keeps a
concave one convex, and the robustness sweep is zero for the true model and
never better than the per-round best for any other."""
import numpy as np
import pytest

import oracle
import synth
from draft_tree_construction_markov_amd import costmodel as cm

TRUE = dict(C_d=1.0, c0=2.0, c1=0.004, c2=2e-6, c_ell=1e-5)


def _samples(seed, m=400, noise=0.0):
    rng = np.random.default_rng(seed)
    n = rng.integers(1, 1025, size=m)
    ell = np.rint(np.exp(rng.uniform(np.log(512), np.log(32768), size=m)))
    y = cm.predict(TRUE, n, ell)
    if noise:
        y = y * (1.0 + noise * rng.normal(size=m))
    return n, ell, y


def test_fit_recovers_exact_samples():
    n, ell, y = _samples(1)
    f = cm.fit(n, ell, y)
    for k in cm.FEATURES:
        assert abs(getattr(f, k) - TRUE[k]) <= 1e-9 * max(TRUE[k], 1e-6), k
    assert f.max_rel < 1e-9
    assert cm.convex_increasing(f)


def test_fit_with_noise_predicts_within_the_noise():
    n, ell, y = _samples(2, m=2000, noise=0.03)
    f = cm.fit(n, ell, y, weights=1.0 / y ** 2)
    grid_n = np.array([1, 16, 64, 256, 1024])
    for e in (512, 4096, 32768):
        want = cm.predict(TRUE, grid_n, np.full(5, e))
        got = cm.predict(f, grid_n, np.full(5, e))
        assert np.all(np.abs(got / want - 1.0) < 0.02)
    assert cm.convex_increasing(f)


def test_concave_samples_still_give_a_convex_model():
    # latencies that flatten out (sqrt-like) have no convex exact fit: the
    # non-negative regression keeps c2 >= 0 and the slopes >= 0
    n = np.arange(1, 600)
    ell = np.full(n.shape, 1000.0)
    y = 1.0 + 0.2 * np.sqrt(n)
    f = cm.fit(n, ell, y)
    assert cm.convex_increasing(f)
    assert f.c2 >= 0.0
    # an unconstrained quadratic would curve downwards here
    A = np.stack([np.ones_like(n, dtype=float), n, n * n], axis=1)
    free = np.linalg.lstsq(A, y, rcond=None)[0]
    assert free[2] < 0


def _oracle_curves(seed=31, rounds=12, B=6, V=400, n_max=200):
    L, peaked, ctx = synth.adaptive_round(seed, rounds, B, V)
    orders = [oracle.bestfirst(L[q], None, None, 0, n_max)
              for q in range(rounds)]

    def curve(cost):
        return np.stack([oracle.throughput_curve(o["score"], o["n"],
                                                 int(ctx[q]), cost)
                         for q, o in enumerate(orders)])
    return curve, L, ctx


def test_robustness_of_the_true_and_perturbed_models():
    curve, L, ctx = _oracle_curves()
    models = {"true": TRUE,
              "c1x2": cm.perturbed(TRUE, {"c1": 2.0}),
              "c_ell/2": cm.perturbed(TRUE, {"c_ell": 0.5}),
              "all x1.5": cm.perturbed(TRUE, {k: 1.5 for k in cm.FEATURES})}
    res = cm.robustness(curve, TRUE, models)
    assert abs(res["true"]["rel_loss"]) < 1e-12
    for name, r in res.items():
        assert r["rel_loss"] >= -1e-12, name  # never above the best
    # the first non-positive gain of the oracle's stop is the curve's first
    # maximiser under the true model
    f = curve(TRUE)
    for q in range(f.shape[0]):
        o = oracle.adaptive(L[q], 200, int(ctx[q]), TRUE)
        assert o["n_star"] == int(np.argmax(f[q]))


def test_fitted_model_loses_little():
    curve, _, _ = _oracle_curves(seed=37)
    n, ell, y = _samples(5, m=600, noise=0.05)
    f = cm.fit(n, ell, y, weights=1.0 / y ** 2).cost(TRUE["C_d"])
    res = cm.robustness(curve, TRUE, {"fitted": f})
    assert 0.0 <= res["fitted"]["rel_loss"] < 0.01


def test_fit_rejects_mismatched_samples():
    with pytest.raises(ValueError):
        cm.fit([1, 2, 3], [10, 10, 10], [1.0, 2.0])
