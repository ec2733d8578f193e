"""CPU pins of the oracle's draft top-k and best-first tree builder (the
step before the verify path: per-depth top-k candidates of the drafter and
the best-first tree built from them).  Checked against a hand-worked tie
fixture, brute-force enumeration of every candidate path on small grids,
numpy's sort and scipy's logsumexp, and structural properties."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp

from mla_tree_verify_parents_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


def test_topk_matches_numpy(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 5000)).astype(np.float32) * 3
    x[1, [10, 20, 4000]] = 50.0                       # ties: lower index first
    x[2, :] = 0.5                                     # all equal: indices 0..K-1
    x[3, 4999] = 99.0                                 # the last entry
    for K in (1, 4, 8, 16):
        ids, lp = orc.draft_topk(x, K)
        for r in range(x.shape[0]):
            order = np.lexsort((np.arange(x.shape[1]), -x[r].astype(np.float64)))[:K]
            assert ids[r].tolist() == order.tolist(), (K, r)
            np.testing.assert_allclose(lp[r], x[r, order].astype(np.float64) - logsumexp(x[r].astype(np.float64)),
                                       rtol=0, atol=1e-12)
    ids, _ = orc.draft_topk(x, 3)
    assert ids[1].tolist() == [10, 20, 4000] and ids[2].tolist() == [0, 1, 2] and ids[3, 0] == 4999


def test_topk_row_stride(orc):
    x = np.random.default_rng(4).standard_normal((5, 300)).astype(np.float32)
    a = orc.draft_topk(x[:, :200], 5)
    b = orc.draft_topk(np.ascontiguousarray(x[:, :200]), 5)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def test_tree_golden_ties(orc):
    for g in json.load(open(os.path.join(GOLDEN, "best_first_ties.json")))["cases"]:
        par, tok, dep = orc.best_first_tree(np.array(g["ids"], np.int32), np.array(g["lp"], np.float32),
                                            g["budget"], g["root"])
        assert par.tolist() == g["parents"] and tok.tolist() == g["tokens"] and dep.tolist() == g["depth"], g["why"]


def _brute_force(ids, lp, budget, root):
    """Every candidate path (ranks r1..rd, d <= D) with its fp32 score summed
    in path order, sorted by score (desc) then depth; the first budget paths
    in that order, numbered in it, form the tree (continuous scores: no ties)."""
    D, K = ids.shape
    paths = []
    for d in range(1, D + 1):
        for ranks in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for j, r in enumerate(ranks):
                s = np.float32(s + lp[j, r])
            paths.append((-float(s), d, ranks))
    paths.sort()
    chosen = [p[2] for p in paths[:budget]]
    index = {(): 0}
    par, tok, dep = [-1], [root], [0]
    for i, ranks in enumerate(chosen, start=1):
        index[ranks] = i
        par.append(index[ranks[:-1]])           # the prefix comes earlier: its score is higher
        tok.append(int(ids[len(ranks) - 1, ranks[-1]]))
        dep.append(len(ranks))
    return par, tok, dep


@pytest.mark.parametrize("D,K,budget", [(1, 3, 3), (2, 2, 6), (3, 2, 14), (3, 3, 20), (2, 3, 12), (3, 3, 39)])
def test_tree_brute_force(orc, D, K, budget):
    rng = np.random.default_rng(D * 10 + K + budget)
    for trial in range(20):
        ids = rng.integers(0, 1000, size=(D, K)).astype(np.int32)
        lp = -np.sort(rng.exponential(1.0, size=(D, K)).astype(np.float32), axis=1)[:, ::-1]
        lp = np.ascontiguousarray(-np.sort(-lp, axis=1))    # descending per depth, all negative
        got = orc.best_first_tree(ids, lp, budget, 7)
        want = _brute_force(ids, lp, budget, 7)
        assert [g.tolist() for g in got] == [list(w) for w in want], (trial, lp)


def test_tree_properties_and_generator(orc):
    """Large random grids: structure, non-increasing scores in node order,
    closure (a node's parent and its lower-ranked sibling are in the tree);
    the input generator's builder gives the same trees."""
    rng = np.random.default_rng(11)
    for trial in range(30):
        D, K = 8, 8
        ids, lp = synth.draft_candidates(rng, D, K, 4096, 3.0)
        root = int(rng.integers(0, 4096))
        par, tok, dep = orc.best_first_tree(ids, lp, 63, root)
        assert par[0] == -1 and tok[0] == root and dep[0] == 0
        score = [np.float32(0.0)]
        rank = [-1]
        for i in range(1, 64):
            assert 0 <= par[i] < i and dep[i] == dep[par[i]] + 1
            r = int(np.where(ids[dep[i] - 1] == tok[i])[0][0])
            rank.append(r)
            score.append(np.float32(score[par[i]] + lp[dep[i] - 1, r]))
            if r > 0:   # the lower-ranked sibling under the same parent came earlier
                assert any(par[j] == par[i] and rank[j] == r - 1 for j in range(1, i))
        assert all(score[i] >= score[i + 1] for i in range(1, 63))
        g = synth.best_first_tree(ids, lp, 63, root)
        assert all((a == b).all() for a, b in zip((par, tok, dep), g))


def test_tree_runs_out(orc):
    ids = np.zeros((2, 2), np.int32)
    lp = np.full((2, 2), -1.0, np.float32)
    with pytest.raises(RuntimeError):
        orc.best_first_tree(ids, lp, 7, 0)            # only 6 candidates exist
    par, _, _ = orc.best_first_tree(ids, lp, 6, 0)
    assert len(par) == 7
