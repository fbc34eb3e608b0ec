"""Pins of the oracle's sampled target tokens (verification with
temperature sampling instead of greedy decoding; CPU only):

- the counter-based generator equals the same published definition
  written independently in synth/;
- the Gumbel-max choice samples softmax(z / T): frequencies over many
  streams match the probabilities, including the temperature's direction;
- a tiny temperature gives the argmax; a huge one a uniform choice;
- verification on sampled targets emits exactly the target's samples along
  the accepted path (so the emitted tokens follow the target's
  distribution), and a tree holding every token accepts to its full depth.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from treecheck import naive_accept, path_tokens


def test_generator_matches_the_published_definition():
    rng = np.random.default_rng(3)
    for _ in range(200):
        seed, stream, idx = (int(x) for x in rng.integers(0, 2 ** 62, 3))
        assert oracle.uniform(seed, stream, idx) == \
            float(synth.uniform(seed, stream, np.array([idx]))[0])


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_frequencies_follow_the_softmax(T):
    z = np.array([1.0, 0.2, -0.5, 2.0, 0.0], np.float32)
    rows = 20000
    out, _ = oracle.sample_targets(np.tile(z, (rows, 1)), T, seed=11)
    p = np.exp(z.astype(np.float64) / T)
    p /= p.sum()
    freq = np.bincount(out, minlength=5) / rows
    sd = np.sqrt(p * (1 - p) / rows)
    assert np.all(np.abs(freq - p) < 5 * sd + 1e-9), (freq, p)


def test_temperature_limits():
    rng = np.random.default_rng(5)
    z = (rng.normal(size=(300, 40)) * 3).astype(np.float32)
    cold, _ = oracle.sample_targets(z, 1e-6, seed=3)
    assert np.array_equal(cold, np.argmax(z, axis=1))
    hot, _ = oracle.sample_targets(np.tile(z[0], (40000, 1)), 1e6, seed=4)
    freq = np.bincount(hot, minlength=40) / 40000
    assert np.all(np.abs(freq - 1 / 40) < 5 * math.sqrt(1 / 40 / 40000))


def test_same_seed_same_sample_other_seed_other_sample():
    rng = np.random.default_rng(6)
    z = rng.normal(size=(64, 500)).astype(np.float32)
    a, _ = oracle.sample_targets(z, 1.0, seed=9)
    b, _ = oracle.sample_targets(z, 1.0, seed=9)
    c, _ = oracle.sample_targets(z, 1.0, seed=10)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    # rows are independent streams: a row's sample depends on its stream
    d, _ = oracle.sample_targets(z[5:6], 1.0, seed=9, stream0=5)
    assert d[0] == a[5]


def test_walk_on_sampled_targets_emits_the_samples():
    rng = np.random.default_rng(7)
    B, V, N = 5, 12, 40
    L = (rng.normal(size=(1, B, V)) * 1.5).astype(np.float32)
    U, W = synth.markov_factors(7, V, 4, False)
    o = oracle.build_tree(L, U, W, np.array([3], np.int32), 3, 6, N)
    n = int(o["n_nodes"][0])
    tgt_logits = (rng.normal(size=(N + 1, V)) * 2).astype(np.float32)
    for seed in range(20):
        y, _ = oracle.sample_targets(tgt_logits, 0.8, seed)
        tau, an, at = oracle.accept(o["tok"][0], o["parent"][0], n, B, y)
        t2, an2, at2 = naive_accept(o["tok"][0], o["parent"][0],
                                    o["depth"][0], n, y, B)
        assert tau == t2 and list(at) == list(at2)
        # the emitted tokens are the target's samples after the root and
        # after each accepted node
        prev = -1
        for d in range(tau):
            assert at[d] == y[prev + 1]
            if d < tau - 1:
                prev = int(an[d])


def test_full_tree_accepts_to_full_depth():
    # every token at every depth is drafted: any sample is a child, so the
    # walk accepts B tokens and the target adds one more
    V, B = 3, 3
    L = np.zeros((1, B, V), np.float32)
    o = oracle.build_tree(L, None, None, np.array([0], np.int32), V, V ** B,
                          V + V ** 2 + V ** 3)
    n = int(o["n_nodes"][0])
    assert n == V + V ** 2 + V ** 3
    rng = np.random.default_rng(8)
    z = rng.normal(size=(n + 1, V)).astype(np.float32)
    y, _ = oracle.sample_targets(z, 1.3, seed=21)
    tau, an, at = oracle.accept(o["tok"][0], o["parent"][0], n, B, y)
    assert tau == B + 1
    assert [len(path_tokens(o["tok"][0], o["parent"][0], int(i)))
            for i in an] == [1, 2, 3]
