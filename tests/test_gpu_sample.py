"""GPU parity of verification with temperature sampling
(pct_verify_sample) against the CPU oracle: the sampled target tokens row
by row (a difference is allowed only where the oracle's best and
second-best Gumbel keys are within 1e-12), then the acceptance walk on
those tokens, with and without the packed mask."""
import numpy as np
import pytest
import torch

import draft_tree_construction_markov_amd as pct
import oracle
import synth
from gpu_util import announce, dev_f32, dev_i32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,B,V,k,beam,N,T,seed", [
    (6, 5, 3000, 4, 8, 48, 0.7, 1),
    (4, 4, 2049, 8, 16, 100, 1.5, 2),    # ragged vocabulary
    (3, 3, 64, 3, 9, 30, 0.05, 3),       # near-greedy temperature
    (2, 3, 5, 3, 6, 20, 1.0, 4),         # five tokens: one short slice
])
def test_sampled_targets_and_walk(batch, B, V, k, beam, N, T, seed):
    rng = np.random.default_rng(seed)
    L = (rng.normal(size=(batch, B, V)) * 2).astype(np.float32)
    U, W = synth.markov_factors(seed, V, 16, False)
    A = rng.integers(0, V, size=batch).astype(np.int32)
    o = oracle.build_tree(L, U, W, A, k, beam, N)
    # target logits after every node: the drafter's next row plus noise
    tl = (rng.normal(size=(batch, N + 1, V)) * 2.5).astype(np.float32)
    masks = np.stack([oracle.mask(o["parent"][q], int(o["n_nodes"][q]), N)
                      for q in range(batch)])
    args = (dev_i32(o["tok"]), dev_i32(o["parent"]), dev_i32(o["depth"]),
            dev_i32(o["n_nodes"]))
    announce("verify sample", dict(batch=batch, N=N, V=V, T=T))
    dtl = dev_f32(tl)
    runs = [pct.verify_sample(*args, dtl, B, T, seed),
            pct.verify_sample(*args, dtl, B, T, seed,
                              mask=torch.from_numpy(masks.view(np.int64))
                              .cuda())]
    torch.cuda.synchronize()
    near = 0
    for sm, tau, an, at in runs:
        sm, tau, an, at = (x.cpu().numpy() for x in (sm, tau, an, at))
        for q in range(batch):
            n = int(o["n_nodes"][q])
            want, gap = oracle.sample_targets(tl[q][:n + 1], T, seed,
                                              stream0=q * (N + 1))
            got = sm[q][:n + 1]
            diff = got != want
            if diff.any():
                assert np.all(gap[diff] < 1e-12), (q, np.nonzero(diff))
                near += 1
                continue
            assert np.all(sm[q][n + 1:] == -1)
            t2, an2, at2 = oracle.accept(o["tok"][q], o["parent"][q], n, B,
                                         np.concatenate(
                                             [want, -np.ones(N - n, np.int32)]))
            assert tau[q] == t2 and list(an[q]) == list(an2) and \
                list(at[q]) == list(at2), q
    assert near == 0
