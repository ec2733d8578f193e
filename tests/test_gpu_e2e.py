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
from tests.helpers import check_attn, to_host

pytestmark = pytest.mark.gpu


def _touched_rows(loop, P):
    """Logical pool rows of slots P .. P+N-1 of every request (what a step writes)."""
    return (loop.kv_base_host[:, None] + P[:, None] + np.arange(loop.N)[None, :]).reshape(-1)


def _check_steps(orc, loop, steps, sample_rows=None, full_pool_every_step=True, rows_per_step=None):
    """Run `steps` loop iterations, each against the oracle on host copies of
    its inputs.  Discrete outputs are compared bit for bit every step, and
    so are the cache rows the step writes (slots P .. P+N-1 of every
    request); the whole pool every step, or once at the end.  Attention:
    every row, the fixed `sample_rows`, or `rows_per_step` rows drawn
    afresh each step (seeded)."""
    host_pool = loop.to_logical(to_host(loop.pool))     # the mirror, in the logical layout
    base = loop.kv_base_host
    dl = loop.d_lat
    B, N, H = loop.B, loop.N, loop.H
    accepted = []
    pick = np.random.default_rng(99)
    for s in range(steps):
        if rows_per_step is not None:
            sample_rows = np.sort(pick.choice(B * N * H, rows_per_step, replace=False))
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
        out = to_host(res.out)
        lse = to_host(res.lse)
        if sample_rows is not None:
            out, lse = out[sample_rows], lse[sample_rows]
        e = check_attn(out, lse, ref_out, ref_lse, "bf16", f"step {s}")
        assert (to_host(res.idx).reshape(B, N) == t_ref).all(), s
        assert (to_host(res.accept_len) == oa).all() and (to_host(res.path) == op).all(), s
        assert (to_host(res.tokens) == ot).all(), s
        if full_pool_every_step:
            dev_pool = loop.to_logical(to_host(loop.pool))
            assert (dev_pool.view(np.uint8) == host_pool.view(np.uint8)).all(), s
        else:
            r = _touched_rows(loop, P)
            got = to_host(loop.pool[torch.from_numpy(_pool_rows(loop, P)).to(loop.device)])
            assert (got.view(np.uint8) == host_pool[r].view(np.uint8)).all(), s
        acc = loop.advance(res)
        assert (loop.P_host == opl).all(), s
        assert (loop.roots == ot[np.arange(B), oa]).all(), s          # the bonus token is the next root
        accepted.append(acc)
        print(f"step {s}: P {P[:4].tolist()}.. accepted {acc[:8].tolist()}.. attn rel_l2 {e[0]:.2e} "
              f"max row {e[2]:.2e}", flush=True)
    if not full_pool_every_step:
        dev_pool = loop.to_logical(to_host(loop.pool))
        assert (dev_pool.view(np.uint8) == host_pool.view(np.uint8)).all()
    return np.array(accepted)


def _pool_rows(loop, P):
    """Physical pool rows of slots P .. P+N-1 of every request."""
    return np.concatenate([loop.rows_of(b, P[b] + np.arange(loop.N)) for b in range(loop.B)])


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


def test_loop_end_to_end_100_steps(orc):
    """The end-to-end configuration over its whole run: 100 steps at full
    shape (32 requests, 8 heads, 64 nodes, prefix U[2048, 65536] growing by
    accept_len + 1 per step, vocabulary 163840, device top-8 and best-first
    trees).  Every step: trees, argmax ids, acceptance, tokens, lengths and
    the cache rows the step wrote, bit for bit; attention on 64 query rows
    drawn afresh each step.  The whole pool once, at the end."""
    loop = e2e.VerifyLoop()
    P0 = loop.P_host.copy()
    acc = _check_steps(orc, loop, 100, full_pool_every_step=False, rows_per_step=64)
    assert (loop.P_host == P0 + (acc + 1).sum(axis=0)).all()
    assert acc.mean() > 0.5                                         # the planted targets accept drafts


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


# ------------------------------------------------ greedy-exact invariant ----
# "The Architecture of Pragmatic Ambition", section "The Reframing: MVP as
# Architecture Validation": speculative decoding must emit exactly the tokens
# plain autoregressive greedy decoding emits.  The target model is replaced
# by a hash: the target's greedy token after a sequence is a fixed function
# of the whole sequence, so both decoders can be run side by side.

_HASH_MUL, _HASH_MOD = 1_000_003, (1 << 61) - 1


def _extend(h: int, tok: int) -> int:
    """Rolling hash of a token sequence, extended by one token."""
    return (h * _HASH_MUL + tok + 1) % _HASH_MOD


def _seq_hash(seq) -> int:
    h = 0
    for t in seq:
        h = _extend(h, int(t))
    return h


def _latents(pos: np.ndarray, tok: np.ndarray, width: int) -> np.ndarray:
    """Closed-form cache latent of token `tok` at position `pos`: bf16 bits
    of values in [-2, 2) from a counter hash of (pos, tok, column)."""
    from mla_tree_verify_parents_amd import synth
    x = (pos.astype(np.uint64)[:, None] * np.uint64(0x9E3779B97F4A7C15)
         ^ tok.astype(np.uint64)[:, None] * np.uint64(0xC2B2AE3D27D4EB4F)
         ^ np.arange(width, dtype=np.uint64)[None, :] * np.uint64(0x165667B19E3779F9))
    x ^= x >> np.uint64(29)
    x *= np.uint64(0xBF58476D1CE4E5B9)
    x ^= x >> np.uint64(32)
    u = (x >> np.uint64(40)).astype(np.float64) / float(1 << 24)
    return synth.to_bf16_bits((4.0 * u - 2.0).astype(np.float32))


def test_loop_greedy_exact_hash_target(orc):
    """The device step (ddt_verify_step: attention, argmax, acceptance,
    compaction, length update) in a loop whose target logits come from a
    hash of the committed sequence plus the path to each node: over 24
    steps every request emits exactly the autoregressive greedy sequence,
    the committed lengths advance by accept_len + 1, and after every step
    cache slot s holds the closed-form latent of (s, committed token s)."""
    from mla_tree_verify_parents_amd import ddt, synth
    from tests.helpers import to_dev

    B, H, N, V, steps = 4, 2, 16, 64, 24
    dl, dr = 512, 64
    scale = 1.0 / np.sqrt(dl + dr)
    rng = np.random.default_rng(2024)
    P = rng.integers(40, 200, size=B).astype(np.int32)
    cap = P.astype(np.int64) + N * (steps + 1)
    base = np.concatenate([[32], 32 + np.cumsum(cap + 32)[:-1]]).astype(np.int64)
    pool = np.full((int(base[-1] + cap[-1] + 32), dl + dr), synth.BF16_NAN, np.uint16)
    # committed tokens c_0 .. c_P: slots s < P hold latent(s, c_s); c_P is the next root
    committed = [list(rng.integers(0, V, size=int(P[b]) + 1)) for b in range(B)]
    for b in range(B):
        s = np.arange(P[b])
        pool[base[b] + s] = _latents(s, np.array(committed[b][: P[b]]), dl + dr)
    dpool = to_dev(pool)
    dbase, dP = to_dev(base), to_dev(P)
    emitted_total = 0
    for step in range(steps):
        parents = synth.random_parents(rng, B, N)
        draft = np.zeros((B, N), np.int32)
        target = np.zeros((B, N), np.int32)
        depth = np.zeros((B, N), np.int64)
        for b in range(B):
            h = [0] * N
            h[0] = _seq_hash(committed[b])                     # the root: the last committed token
            draft[b, 0] = committed[b][-1]
            for i in range(1, N):
                par = parents[b, i]
                depth[b, i] = depth[b, par] + 1
                # most drafts guess the target's next token after their parent
                draft[b, i] = h[par] % V if rng.random() < 0.7 else rng.integers(0, V)
                h[i] = _extend(h[par], int(draft[b, i]))
            target[b] = [x % V for x in h]
        # logits: noise in [0, 1) plus 10 on the target token (argmax = target)
        logits = rng.random((B * N, V), dtype=np.float32)
        logits[np.arange(B * N), target.reshape(-1)] += 10.0
        # node latents at slots P + i: latent(P + depth(i), draft token)
        for b in range(B):
            rows = base[b] + P[b] + np.arange(N)
            dpool[torch.from_numpy(rows).cuda()] = to_dev(_latents(P[b] + depth[b], draft[b], dl + dr))
        q = to_dev(synth.normal(rng, (B * N * H, dl + dr), "bf16"))
        out, lse, idx, acc, path, tok, npl = ddt.verify_step(
            q[:, :dl], q[:, dl:], dpool[:, :dl], dpool[:, dl:], dbase, P, None, to_dev(logits), to_dev(draft),
            to_dev(parents), dP, H=H, scale=scale)
        torch.cuda.synchronize()
        acc_h, tok_h, npl_h = to_host(acc), to_host(tok), to_host(npl)
        assert (to_host(idx).reshape(B, N) == target).all(), step
        for b in range(B):
            k = int(acc_h[b])
            got = [int(t) for t in tok_h[b, : k + 1]]
            # autoregressive greedy from the same committed sequence
            seq, want = list(committed[b]), []
            for _ in range(k + 1):
                t = _seq_hash(seq) % V
                want.append(t)
                seq.append(t)
            assert got == want, (step, b, got, want)
            assert (tok_h[b, k + 1:] == -1).all()
            committed[b].extend(got)
            assert npl_h[b] == P[b] + k + 1 == len(committed[b]) - 1
            emitted_total += k + 1
        P = npl_h.astype(np.int32)
        # slot s < P holds latent(s, c_s): the compacted path landed in order
        host = to_host(dpool)
        for b in range(B):
            s = np.arange(P[b])
            want_lat = _latents(s, np.array(committed[b][: P[b]]), dl + dr)
            assert (host[base[b] + s] == want_lat).all(), (step, b)
    assert emitted_total > 2 * steps * B                   # drafts were accepted, not just bonus tokens
    print(f"greedy-exact: {emitted_total} tokens over {steps} steps x {B} requests")
