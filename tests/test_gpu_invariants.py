"""Invariants of the tree-verify attention on the GPU (no oracle involved):

* the result does not depend on how the keys are cut into splits, beyond
  rounding (each split takes its own softmax reference, so the bf16
  probabilities round differently);
* permuting the heads of every node permutes the output rows, bit for bit
  (a row's arithmetic does not depend on where it sits in a row tile);
* relabelling the tree nodes by another topological order (node latents
  and queries moving with their nodes) permutes the output rows, up to
  rounding (the tree keys then sit in other slots and other tiles).

The pages define the attention per (node, head) row over the committed
prefix and the node's ancestors ("The Architecture of Pragmatic Ambition",
section "The Decision Architecture"): nothing in that definition depends
on the split-KV decomposition, the head order or the node numbering."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, rel_l2, to_host

pytestmark = pytest.mark.gpu


def run(w: synth.Workload, kv_chunk=0):
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask, H=w.H,
                               scale=w.scale, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    return synth.bf16_bits_to_f32(to_host(out)).astype(np.float64), to_host(lse).astype(np.float64)


def close(out_a, lse_a, out_b, lse_b, what):
    assert np.isfinite(out_a).all() and np.isfinite(out_b).all(), what
    assert rel_l2(out_a, out_b) < 5e-3, (what, rel_l2(out_a, out_b))
    rows = np.linalg.norm(out_a - out_b, axis=1) / np.maximum(np.linalg.norm(out_b, axis=1), 1e-30)
    assert rows.max() < 2e-2, (what, float(rows.max()))
    assert np.abs(lse_a - lse_b).max() < 5e-3, (what, float(np.abs(lse_a - lse_b).max()))


def test_split_count_independence():
    w = synth.workload(3, B=3, H=8, N=32, prefix_range=(500, 6000))
    ref_out, ref_lse = run(w, kv_chunk=1 << 20)  # one split per request: no merge
    for kv_chunk in (0, 32, 96, 256, 1024):
        out, lse = run(w, kv_chunk)
        close(out, lse, ref_out, ref_lse, f"kv_chunk {kv_chunk}")


def test_head_permutation_equivariance():
    w = synth.workload(3, B=3, H=8, N=32, prefix_range=(300, 5000))
    out, lse = run(w)
    rng = np.random.default_rng(11)
    sigma = np.stack([rng.permutation(w.H) for _ in range(w.B * w.N)])  # per node: new head of old head h
    base = (np.arange(w.B * w.N) * w.H)[:, None]
    src = (base + np.arange(w.H)[None, :]).reshape(-1)
    dst = (base + sigma).reshape(-1)
    wp = synth.Workload(**{**w.__dict__})
    wp.q = np.empty_like(w.q)
    wp.q[dst] = w.q[src]
    out_p, lse_p = run(wp)
    assert np.array_equal(out_p[dst], out[src]) and np.array_equal(lse_p[dst], lse[src])


def linear_extension(rng, parents):
    """A random topological numbering of a tree: new index of every old node."""
    N = parents.shape[0]
    children = [[] for _ in range(N)]
    for i in range(1, N):
        children[parents[i]].append(i)
    pi = np.empty(N, np.int64)
    pi[0] = 0
    ready = list(children[0])
    for k in range(1, N):
        j = ready.pop(int(rng.integers(len(ready))))
        pi[j] = k
        ready.extend(children[j])
    return pi


def test_node_relabelling_equivariance():
    w = synth.workload(3, B=3, H=8, N=32, prefix_range=(300, 5000))
    out, lse = run(w)
    rng = np.random.default_rng(12)
    wp = synth.Workload(**{**w.__dict__})
    wp.parents = np.empty_like(w.parents)
    wp.q = np.empty_like(w.q)
    wp.pool = w.pool.copy()
    src_rows, dst_rows = [], []
    for b in range(w.B):
        pi = linear_extension(rng, w.parents[b])
        assert sorted(pi) == list(range(w.N))
        wp.parents[b, 0] = -1
        wp.parents[b, pi[1:]] = pi[w.parents[b, 1:]]
        assert (wp.parents[b, 1:] < np.arange(1, w.N)).all()
        slot0 = int(w.kv_base[b]) + int(w.prefix_len[b])
        wp.pool[slot0 + pi] = w.pool[slot0 + np.arange(w.N)]        # node latents move with their nodes
        for h in range(w.H):
            src_rows.append((b * w.N + np.arange(w.N)) * w.H + h)
            dst_rows.append((b * w.N + pi) * w.H + h)
    src, dst = np.concatenate(src_rows), np.concatenate(dst_rows)
    wp.q[dst] = w.q[src]
    out_p, lse_p = run(wp)
    close(out_p[dst], lse_p[dst], out[src], lse[src], "relabelled")
