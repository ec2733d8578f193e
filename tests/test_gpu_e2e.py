"""GPU parity of the verify loop (the end-to-end configuration): every step
of `e2e.VerifyLoop` -- the draft stage (device top-k and best-first trees,
checked against the oracle's builder on the same candidates), then
attention, argmax, acceptance, compaction and the length update in one
`ddt_verify_step` call, then the loop's bookkeeping -- against the fp64
oracle run on host copies of the same inputs, with the
host mirror of the cache pool carried from step to step by the oracle's
compaction.  Discrete results and the whole pool must match bit for bit;
attention outputs within relative L2 1e-2 (bf16 inputs)."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import e2e
from tests.helpers import ATTN_TOL, as_f64, rel_l2, to_host

pytestmark = pytest.mark.gpu


def _check_steps(orc, loop, steps, sample_rows=None):
    host_pool = loop.to_logical(to_host(loop.pool))     # the mirror, in the logical layout
    base = loop.kv_base_host
    dl = loop.d_lat
    B, N, H = loop.B, loop.N, loop.H
    accepted = []
    for s in range(steps):
        inp = loop.make_inputs()
        slots = (base[:, None] + inp.prefix_len[:, None] + np.arange(N)[None, :]).reshape(-1)
        host_pool[slots] = to_host(loop.pool[inp.node_rows])     # the step's node latents (inputs)
        if inp.cand_ids is not None:                             # trees built on the device
            for b in range(B):
                tp, tt, _ = orc.best_first_tree(inp.cand_ids[b], inp.cand_lp[b], N - 1, int(inp.roots[b]))
                assert (inp.parents[b] == tp).all() and (inp.draft_ids[b] == tt).all(), (s, b)
        qh = to_host(inp.q)
        logits_h = to_host(inp.logits)
        P = inp.prefix_len.copy()
        ref_out, ref_lse = orc.verify_attn(qh[:, :dl], qh[:, dl:], host_pool[:, :dl], host_pool[:, dl:], base, P,
                                           inp.parents, H=H, scale=loop.scale, rows=sample_rows)
        t_ref = orc.argmax(logits_h).reshape(B, N)
        oa, op, ot = orc.greedy_accept(t_ref, inp.draft_ids, inp.parents)
        opl, _ = orc.compact_kv(host_pool[:, :dl], host_pool[:, dl:], base, P, op, oa)

        res = loop.run_step(inp)
        out = as_f64(to_host(res.out))
        lse = to_host(res.lse)
        if sample_rows is not None:
            out, lse = out[sample_rows], lse[sample_rows]
        e_out, e_lse = rel_l2(out, ref_out), rel_l2(lse, ref_lse)
        assert e_out <= ATTN_TOL["bf16"] and e_lse <= ATTN_TOL["bf16"], (s, e_out, e_lse)
        assert (to_host(res.idx).reshape(B, N) == t_ref).all(), s
        assert (to_host(res.accept_len) == oa).all() and (to_host(res.path) == op).all(), s
        assert (to_host(res.tokens) == ot).all(), s
        dev_pool = loop.to_logical(to_host(loop.pool))
        assert (dev_pool.view(np.uint8) == host_pool.view(np.uint8)).all(), s
        acc = loop.advance(res)
        assert (loop.P_host == opl).all(), s
        assert (loop.roots == ot[np.arange(B), oa]).all(), s          # the bonus token is the next root
        accepted.append(acc)
        print(f"step {s}: P {P[:4].tolist()}.. accepted {acc[:8].tolist()}.. attn rel_l2 {e_out:.2e}", flush=True)
    return np.array(accepted)


def test_loop_small_every_row(orc):
    """A small loop (4 requests, 16 nodes, vocabulary 3000) over 12 steps,
    every query row against the oracle at every step; the cache grows by
    accept_len + 1 per step and the next root is the bonus token."""
    loop = e2e.VerifyLoop(B=4, H=2, N=16, prefix_range=(30, 300), steps=12, vocab=3000, K=4, D=4, seed=7)
    P0 = loop.P_host.copy()
    acc = _check_steps(orc, loop, 12)
    assert (loop.P_host == P0 + (acc + 1).sum(axis=0)).all()
    assert acc.max() >= 2                                           # the planted targets accept paths


def test_loop_end_to_end_shape(orc):
    """The end-to-end configuration's shape (32 requests, 8 heads, 64 nodes,
    prefix U[2048, 65536], vocabulary 163840, top-8 best-first trees) for
    two steps: discrete results and the pool exact, attention on a seeded
    sample of 64 query rows."""
    loop = e2e.VerifyLoop()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(loop.B * loop.N * loop.H, 64, replace=False))
    _check_steps(orc, loop, 2, sample_rows=rows)


@pytest.mark.parametrize("page_size", [32, 256])
def test_loop_paged_every_row(orc, page_size):
    """The small loop on a paged cache: pages handed out from a shuffled
    free list as the requests grow; attention, acceptance and compaction go
    through the block table, checked every step against the oracle on the
    logical cache (the whole cache, bit for bit)."""
    loop = e2e.VerifyLoop(B=4, H=2, N=16, prefix_range=(30, 300), steps=12, vocab=3000, K=4, D=4, seed=7,
                          page_size=page_size)
    P0 = loop.P_host.copy()
    acc = _check_steps(orc, loop, 12)
    assert (loop.P_host == P0 + (acc + 1).sum(axis=0)).all()


def test_loop_host_trees(orc):
    """The loop with its trees built on the host (torch top-k, host builder)."""
    loop = e2e.VerifyLoop(B=3, H=2, N=16, prefix_range=(30, 300), steps=4, vocab=3000, K=4, D=4, seed=9,
                          device_draft=False)
    _check_steps(orc, loop, 4)
