"""GPU parity of the draft step that feeds the verify path: per-depth top-k
of draft logits (ids bit-exact against the fp64 oracle; log-softmax values
within 1e-4 absolute, the fp32 log-sum-exp's error at a 163840-token
vocabulary) and the best-first tree (parents, tokens, depth bit-exact
against the oracle on the same candidate grids)."""
import json
import os

import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LOGP_TOL = 1e-4


@pytest.mark.parametrize("rows,V,K,sigma", [
    (256, 163840, 8, 3.0),   # the verify loop's draft step: 32 requests x 8 depths
    (8, 163840, 4, 3.0),     # the K2-like head share's draft step
    (5, 5000, 16, 1.0),      # one partial chunk
    (3, 16385, 1, 1.0),      # one entry past a chunk
    (4, 16389, 16, 1.0),     # a last chunk with fewer entries than K
    (6, 40000, 8, 2.0),      # two whole chunks and a ragged one
    (7, 100, 5, 1.0),        # one small chunk
])
def test_draft_topk(orc, rows, V, K, sigma):
    rng = np.random.default_rng(rows + V + K)
    x = (rng.standard_normal((rows, V)) * sigma).astype(np.float32)
    x[0, [V // 3, V // 2, V - 1]] = 40.0                      # ties at the top: lower index first
    if rows > 2:
        x[2, :] = 0.25                                         # all equal: indices 0..K-1
    ids, lp = ddt.draft_topk(to_dev(x), K)
    ref_ids, ref_lp = orc.draft_topk(x, K)
    assert (to_host(ids) == ref_ids).all()
    assert np.abs(to_host(lp).astype(np.float64) - ref_lp).max() <= LOGP_TOL


def _bf16_round(x):
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def test_draft_topk_tied_values(orc):
    """Equal values in every amount a chunk's candidate list meets: fewer
    than 64, up to 256, up to 1024 and past 1024 entries tied at the top of
    a chunk (the last falls back to the exact selection over every entry),
    ties across chunks and in the ragged chunk, and logits rounded to bf16
    (many equal values near the top).  Ids bit-exact: equal values by
    ascending index."""
    rng = np.random.default_rng(77)
    rows, V, K = 9, 40000, 16
    x = rng.standard_normal((rows, V)).astype(np.float32)
    for r, count in enumerate([40, 100, 600, 3000]):
        cols = rng.choice(16384, count, replace=False) + 16384   # inside chunk 1
        x[r, cols] = 7.5
    x[4, rng.choice(V, 50, replace=False)] = 6.0                 # ties spread over every chunk
    x[5, 32768 + rng.choice(V - 32768, 20, replace=False)] = 9.0  # ties in the ragged chunk
    x[6] = _bf16_round(x[6] * 3.0)
    x[7] = np.round(x[7] * 2.0) / 2.0                            # few distinct values
    x[8, 16384:32768] = -3.0                                     # a constant chunk beside random ones
    ids, lp = ddt.draft_topk(to_dev(x), K)
    ref_ids, ref_lp = orc.draft_topk(x, K)
    assert (to_host(ids) == ref_ids).all()
    assert np.abs(to_host(lp).astype(np.float64) - ref_lp).max() <= LOGP_TOL


def test_draft_topk_largest_vocabulary(orc):
    """V = 2^20 (the largest vocabulary) and K = 16: 64 chunks per row, so
    the row merge picks the top 16 of 1024 candidates (its widest path)."""
    rng = np.random.default_rng(31)
    rows, V, K = 3, 1 << 20, 16
    x = (rng.standard_normal((rows, V)) * 2.0).astype(np.float32)
    x[1, rng.choice(V, 40, replace=False)] = 12.0     # ties spread over many chunks
    ids, lp = ddt.draft_topk(to_dev(x), K)
    ref_ids, ref_lp = orc.draft_topk(x, K)
    assert (to_host(ids) == ref_ids).all()
    assert np.abs(to_host(lp).astype(np.float64) - ref_lp).max() <= LOGP_TOL


def test_draft_topk_row_view(orc):
    """A column range of a wider array (row stride != V, unaligned start)."""
    rng = np.random.default_rng(9)
    full = rng.standard_normal((6, 9001)).astype(np.float32)
    dx = to_dev(full)[:, 3:8195]
    ids, lp = ddt.draft_topk(dx, 6)
    ref_ids, ref_lp = orc.draft_topk(full[:, 3:8195], 6)
    assert (to_host(ids) == ref_ids).all()
    assert np.abs(to_host(lp).astype(np.float64) - ref_lp).max() <= LOGP_TOL


def _grids(rng, B, D, K, V=4096, sigma=3.0):
    ids = np.empty((B, D, K), np.int32)
    lp = np.empty((B, D, K), np.float32)
    for b in range(B):
        ids[b], lp[b] = synth.draft_candidates(rng, D, K, V, sigma)
    return ids, lp


@pytest.mark.parametrize("B,D,K,budget", [
    (32, 8, 8, 63),     # the verify loop's trees
    (1, 8, 4, 63),      # the K2-like head share's tree
    (4, 4, 8, 127),     # the long-context tree (wide and shallow)
    (3, 3, 3, 39),      # every candidate taken
    (2, 1, 16, 16),     # one level
    (2, 8, 8, 1023),    # the largest tree
    (5, 2, 2, 0),       # root only
    (2, 63, 1, 63),     # one candidate per depth: a chain
    (3, 2, 7, 55),      # two levels, wide
])
def test_best_first_tree(orc, B, D, K, budget):
    rng = np.random.default_rng(B * 1000 + D * 10 + K + budget)
    ids, lp = _grids(rng, B, D, K)
    roots = rng.integers(0, 4096, B).astype(np.int32)
    par, tok, dep = ddt.best_first_tree(to_dev(ids), to_dev(lp), to_dev(roots), budget)
    par, tok, dep = to_host(par), to_host(tok), to_host(dep)
    for b in range(B):
        rp, rt, rd = orc.best_first_tree(ids[b], lp[b], budget, int(roots[b]))
        assert (par[b] == rp).all() and (tok[b] == rt).all() and (dep[b] == rd).all(), b


def test_best_first_tree_ties(orc):
    """Equal scores: the lower depth, then the earlier insertion (the
    hand-worked cases, and grids of equal log-probabilities)."""
    for g in json.load(open(os.path.join(GOLDEN, "best_first_ties.json")))["cases"]:
        ids = np.array(g["ids"], np.int32)[None]
        lp = np.array(g["lp"], np.float32)[None]
        par, tok, dep = ddt.best_first_tree(to_dev(ids), to_dev(lp), to_dev(np.array([g["root"]], np.int32)),
                                            g["budget"])
        assert to_host(par)[0].tolist() == g["parents"] and to_host(tok)[0].tolist() == g["tokens"]
        assert to_host(dep)[0].tolist() == g["depth"], g["why"]
    rng = np.random.default_rng(5)
    for budget in (200, 60):            # the frontier in LDS, and one candidate per lane
        B, D, K = 6, 5, 4
        ids = rng.integers(0, 1000, (B, D, K)).astype(np.int32)
        lp = np.repeat(-np.sort(rng.integers(1, 4, (B, D, 1)), axis=1).astype(np.float32), K, axis=2)  # equal per depth
        lp[:, :, 2:] -= 1.0
        roots = np.arange(B, dtype=np.int32)
        par, tok, dep = ddt.best_first_tree(to_dev(ids), to_dev(np.ascontiguousarray(lp)), to_dev(roots), budget)
        for b in range(B):
            rp, rt, rd = orc.best_first_tree(ids[b], lp[b], budget, int(roots[b]))
            assert (to_host(par)[b] == rp).all() and (to_host(tok)[b] == rt).all()
            assert (to_host(dep)[b] == rd).all(), (budget, b)


def test_draft_step_chain(orc):
    """Top-k on the device feeding the tree builder on the device: the trees
    are valid best-first trees of the device's candidates (structure and
    order checked here; each stage's values are pinned above)."""
    rng = np.random.default_rng(21)
    B, D, K, V = 4, 8, 8, 163840
    x = (rng.standard_normal((B * D, V)) * 3.0).astype(np.float32)
    ids, lp = ddt.draft_topk(to_dev(x), K)
    roots = torch.arange(B, dtype=torch.int32, device="cuda")
    par, tok, dep = ddt.best_first_tree(ids.view(B, D, K), lp.view(B, D, K), roots, 63)
    ids_h, lp_h = to_host(ids).reshape(B, D, K), to_host(lp).reshape(B, D, K)
    par, tok, dep = to_host(par), to_host(tok), to_host(dep)
    ref_ids, _ = orc.draft_topk(x, K)
    assert (ids_h.reshape(-1, K) == ref_ids).all()
    for b in range(B):
        assert par[b, 0] == -1 and tok[b, 0] == b
        score = [np.float32(0)]
        for i in range(1, 64):
            assert 0 <= par[b, i] < i and dep[b, i] == dep[b, par[b, i]] + 1
            r = int(np.where(ids_h[b, dep[b, i] - 1] == tok[b, i])[0][0])
            score.append(np.float32(score[par[b, i]] + lp_h[b, dep[b, i] - 1, r]))
        assert all(score[i] >= score[i + 1] for i in range(1, 63))
