"""Pins of the oracle's Markov contraction, log-sum-exp and local top-k
against closed forms and brute force (CPU only)."""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore")


def _rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("bf16", [False, True])
def test_markov_one_hot_selects_a_column(bf16):
    # U[t] = e_j  =>  Markov(t)[v] = W[v][j] exactly.  A transposed or
    # shifted operand reads another element and fails.
    V, r, t, j = 37, 16, 5, 11
    W = _rng(1).normal(size=(V, r)).astype(np.float32)
    U = np.zeros((V, r), np.float32)
    U[t, j] = 1.0
    if bf16:
        U, W = synth.bf16_bits(U), synth.bf16_bits(W)
        want = synth.bf16_to_f32(W)[:, j]
    else:
        want = W[:, j]
    got = oracle.markov_row(U, W, t)
    assert np.array_equal(got, want)


def test_markov_small_integers_exact():
    # Small integers: every product and sum is exact, so the result equals
    # the exact integer dot product computed with Python ints.
    V, r = 29, 24
    rng = _rng(2)
    Ui = rng.integers(-8, 9, size=(V, r))
    Wi = rng.integers(-8, 9, size=(V, r))
    U = synth.bf16_bits(Ui.astype(np.float32))
    W = synth.bf16_bits(Wi.astype(np.float32))
    for t in (0, 7, V - 1):
        got = oracle.markov_row(U, W, t)
        want = [sum(int(Ui[t, j]) * int(Wi[v, j]) for j in range(r))
                for v in range(V)]
        assert np.array_equal(got, np.array(want, np.float32))


def test_markov_rounds_once():
    # Terms chosen so that a running fp32 sum loses the small part but the
    # exact sum rounded once keeps it: 2^24 + 1 + 1 = 2^24 + 2 (representable)
    # while fp32 accumulation gives 2^24.
    V, r = 1, 3
    U = np.array([[2.0 ** 24, 1.0, 1.0]], np.float32)
    W = np.array([[1.0, 1.0, 1.0]], np.float32)
    got = oracle.markov_row(U, W, 0)
    assert got[0] == np.float32(2.0 ** 24 + 2)


@pytest.mark.parametrize("c", [0.0, 3.25, -17.5])
def test_lse_uniform_row(c):
    V = 1000
    lse, tt, tz, g = oracle.row_stats(np.full(V, c, np.float32), None, 4)
    want = c + math.log(V)
    assert abs(lse - want) <= np.spacing(np.float32(abs(want) + 1))
    # exact ties: tokens in ascending order
    assert list(tt) == [0, 1, 2, 3]
    assert g == 0.0


def test_lse_peaked_row():
    # Build a row whose top token has probability 0.95 exactly (in double):
    # then log pi(top) = ln 0.95.
    rng = _rng(3)
    V = 5000
    z = rng.normal(size=V) * 1.5
    a = int(np.argmax(z))
    rest = np.delete(z, a)
    m = rest.max()
    z[a] = math.log(0.95 / 0.05) + m + math.log(np.exp(rest - m).sum())
    z = z.astype(np.float32)
    lse, tt, tz, _ = oracle.row_stats(z, None, 1)
    assert tt[0] == a
    lp = np.float32(tz[0] - np.float32(lse))
    assert abs(float(lp) - math.log(0.95)) < 4e-6


def test_lse_normalises():
    rng = _rng(4)
    for T in (0.5, 1.0, 2.0):
        z = (rng.normal(size=20000) * 3 / T).astype(np.float32)
        lse, _, _, _ = oracle.row_stats(z, None, 1)
        s = np.exp(z.astype(np.float64) - lse).sum()
        assert abs(s - 1.0) < 1e-6 * 20 + 1e-6


def test_topk_matches_full_sort_and_adds_markov_once():
    rng = _rng(5)
    V, k = 3000, 9
    L = (rng.normal(size=V) * 2).astype(np.float32)
    M = (rng.normal(size=V) * 0.1).astype(np.float32)
    # plant exact ties at the top to exercise the token tie-break
    L[[10, 20, 30]] = 9.0
    M[[10, 20, 30]] = 0.0
    lse, tt, tz, g = oracle.row_stats(L, M, k)
    z = (L + M).astype(np.float32)
    order = sorted(range(V), key=lambda v: (-float(z[v]), v))[:k]
    assert list(tt) == order
    assert np.array_equal(tz, z[order])
    assert list(tt[:3]) == [10, 20, 30]
    assert g == 0.0


def test_row_stats_rejects_bad_k():
    with pytest.raises(RuntimeError):
        oracle.row_stats(np.zeros(5, np.float32), None, 6)
