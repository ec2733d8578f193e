"""Pins for the fp64 oracle: each test checks the oracle against something
other than itself -- closed forms, brute force, library routines (torch CPU
fp64 attention, numpy argmax), the absorbed/explicit MLA identity, and
hand-worked fixtures under tests/golden/.  CPU only."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_parent_arrays(N):
    """Every valid parent array of an N-node tree (parents[i] in [0, i))."""
    for tail in itertools.product(*[range(i) for i in range(1, N)]):
        yield np.array((-1,) + tail, np.int32)


def closure_ancestors(par):
    """Ancestor-or-self relation as the reflexive-transitive closure of the
    child->parent adjacency matrix, by repeated boolean squaring."""
    N = len(par)
    A = np.eye(N, dtype=bool)
    for i in range(1, N):
        A[i, par[i]] = True
    while True:
        A2 = (A.astype(np.int64) @ A.astype(np.int64)) > 0
        if (A2 == A).all():
            return A
        A = A2


def mask_to_bool(mask, N):
    """[N, W] uint64 words -> [N, N] bool, bit j of row i."""
    out = np.zeros((N, N), bool)
    for i in range(N):
        for j in range(N):
            out[i, j] = (int(mask[i, j // 64]) >> (j % 64)) & 1
    return out


# ----------------------------------------------------------------- mask ----

def test_mask_golden_tree7(orc):
    g = json.load(open(os.path.join(GOLDEN, "tree7.json")))
    mask, depth, err = orc.build_mask(np.array([g["parents"]], np.int32))
    assert err[0] == 0
    assert [int(x) for x in mask[0, :, 0]] == g["mask_word0"]
    assert depth[0].tolist() == g["depth"]
    for i, anc in enumerate(g["ancestors_incl_self"]):
        assert sorted(np.nonzero(mask_to_bool(mask[0], 7)[i])[0].tolist()) == anc


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 130, 1024])
def test_mask_chain_is_causal(orc, N):
    par = np.arange(-1, N - 1, dtype=np.int32)[None]
    mask, depth, err = orc.build_mask(par)
    assert err[0] == 0
    assert (mask_to_bool(mask[0], N) == np.tril(np.ones((N, N), bool))).all()
    assert (depth[0] == np.arange(N)).all()


@pytest.mark.parametrize("N", [2, 9, 100])
def test_mask_star(orc, N):
    par = np.zeros((1, N), np.int32)
    par[0, 0] = -1
    mask, depth, _ = orc.build_mask(par)
    expect = np.eye(N, dtype=bool)
    expect[:, 0] = True
    assert (mask_to_bool(mask[0], N) == expect).all()
    assert depth[0, 0] == 0 and (depth[0, 1:] == 1).all()


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7])
def test_mask_all_trees_vs_closure(orc, N):
    pars = np.stack(list(all_parent_arrays(N)))
    mask, depth, err = orc.build_mask(pars)
    assert (err == 0).all()
    for b in range(pars.shape[0]):
        m = mask_to_bool(mask[b], N)
        assert (m == closure_ancestors(pars[b])).all()
        assert (m.sum(1) == depth[b] + 1).all()


def test_mask_all_trees_n8_recurrence(orc):
    """N=8: all 5040 trees; mask[i] == mask[parent(i)] | e_i and popcount = depth+1."""
    pars = np.stack(list(all_parent_arrays(8)))
    mask, depth, err = orc.build_mask(pars)
    assert (err == 0).all()
    w = mask[:, :, 0]
    for i in range(1, 8):
        parent_word = w[np.arange(len(pars)), pars[:, i]]
        assert (w[:, i] == (parent_word | np.uint64(1 << i))).all()
    pop = np.array([[bin(int(x)).count("1") for x in row] for row in w])
    assert (pop == depth + 1).all()


def test_mask_random_large_vs_closure(orc):
    rng = np.random.default_rng(7)
    pars = synth.random_parents(rng, 3, 200)
    mask, depth, err = orc.build_mask(pars)
    for b in range(3):
        assert (mask_to_bool(mask[b], 200) == closure_ancestors(pars[b])).all()


@pytest.mark.parametrize("bad", [[0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, -1, 0], [-1, 0, 5]])
def test_mask_invalid_tree(orc, bad):
    par = np.array([[-1, 0, 1], bad], np.int32)
    mask, depth, err = orc.build_mask(par)
    assert err.tolist() == [0, 1]
    assert (mask[1] == 0).all() and (depth[1] == -1).all()
    assert (mask[0, :, 0] == np.array([1, 3, 7], np.uint64)).all()


# ------------------------------------------------------------ attention ----

def _sdpa_reference(q, k, v, vis, scale):
    """torch CPU fp64 scaled_dot_product_attention with a boolean mask.
    q [R, D], k/v [T, *], vis [R, T] bool -> out [R, Dv]."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    m = torch.from_numpy(vis)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0, 0].numpy()


def _f64(a):
    a = np.asarray(a)
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _small_case(rng, B, H, N, P, dl, dr, dtype="f32", parents=None):
    Ps = np.full(B, P, np.int32) if np.isscalar(P) else np.asarray(P, np.int32)
    pool, base, _ = synth.make_pool(rng, Ps, N, dl + dr, dtype)
    q = synth.normal(rng, (B * N * H, dl + dr), dtype)
    if parents is None:
        parents = synth.random_parents(rng, B, N)
    return pool, base, Ps, q, parents


def _oracle_attn(orc, pool, base, Ps, q, parents, H, dl, scale, **kw):
    return orc.verify_attn(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], base, Ps, parents,
                           H=H, scale=scale, **kw)


@pytest.mark.parametrize("P,N", [(0, 6), (5, 1), (37, 9), (100, 40)])
def test_attn_chain_equals_causal_sdpa(orc, P, N):
    """A chain-shaped tree is causal attention over P+N keys (SDPA, fp64)."""
    rng = np.random.default_rng(11)
    H, dl, dr = 3, 32, 8
    par = np.arange(-1, N - 1, dtype=np.int32)[None]
    pool, base, Ps, q, _ = _small_case(rng, 1, H, N, P, dl, dr, parents=par)
    scale = 0.2
    out, lse = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, scale)
    T = P + N
    kv = _f64(pool[base[0]: base[0] + T])
    causal = np.tril(np.ones((T, T), bool))[P:]          # rows of the N tree nodes
    for h in range(H):
        qh = _f64(q[h::H])                               # rows i*H + h
        ref = _sdpa_reference(qh, kv, kv[:, :dl], causal, scale)
        np.testing.assert_allclose(out[h::H], ref, rtol=1e-11, atol=1e-12)


def test_attn_budget0_is_decode(orc):
    """N = 1 (budget 0): one query row per head over the P+1 keys, all visible."""
    rng = np.random.default_rng(12)
    H, dl, dr, P = 4, 64, 16, 77
    pool, base, Ps, q, par = _small_case(rng, 2, H, 1, P, dl, dr)
    out, lse = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.1)
    for b in range(2):
        kv = _f64(pool[base[b]: base[b] + P + 1])
        qb = _f64(q[b * H:(b + 1) * H])
        ref = _sdpa_reference(qb, kv, kv[:, :dl], np.ones((H, P + 1), bool), 0.1)
        np.testing.assert_allclose(out[b * H:(b + 1) * H], ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attn_random_tree_vs_sdpa(orc, dtype):
    """General trees: SDPA with the visibility built from the parent closure."""
    rng = np.random.default_rng(13)
    B, H, N, dl, dr = 3, 2, 17, 64, 16
    pool, base, Ps, q, par = _small_case(rng, B, H, N, [0, 31, 64], dl, dr, dtype)
    out, lse = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 1 / np.sqrt(80))
    for b in range(B):
        P = int(Ps[b])
        anc = closure_ancestors(par[b])
        vis = np.concatenate([np.ones((N, P), bool), anc], axis=1)
        kv = _f64(pool[base[b]: base[b] + P + N])
        for h in range(H):
            rows = [(b * N + i) * H + h for i in range(N)]
            ref = _sdpa_reference(_f64(q[rows]), kv, kv[:, :dl], vis, 1 / np.sqrt(80))
            np.testing.assert_allclose(out[rows], ref, rtol=1e-11, atol=1e-12)


def test_attn_absorbed_equals_explicit_mha(orc):
    """q_nope.(c_kv W_UK) == (W_UK q_nope).c_kv and softmax(.)(c_kv W_UV) ==
    (softmax(.) c_kv) W_UV: the absorbed latent attention reproduces
    explicit per-head MHA with up-projected keys and values, out and lse.
    Integer W_UK and q_nope keep q_lat exact in fp32."""
    rng = np.random.default_rng(14)
    B, H, N, P, dl, dr, dn, dv = 1, 3, 6, 20, 64, 16, 16, 16
    par = np.array([[-1, 0, 0, 1, 3, 2]], np.int32)
    pool, base, Ps, _, _ = _small_case(rng, B, H, N, P, dl, dr, parents=par)
    W_UK = rng.integers(-2, 3, size=(H, dl, dn)).astype(np.float64)
    W_UV = rng.standard_normal((H, dl, dv))
    q_nope = rng.integers(-2, 3, size=(N, H, dn)).astype(np.float64)
    q_pe = rng.standard_normal((N, H, dr)).astype(np.float32)
    q_lat = np.einsum("hld,ihd->ihl", W_UK, q_nope)            # [N, H, dl], integers
    q = np.concatenate([q_lat.astype(np.float32), q_pe], axis=2).reshape(N * H, dl + dr)
    scale = 0.01
    out, lse = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, scale)
    T = P + N
    kv = _f64(pool[base[0]: base[0] + T])
    ckv, kpe = kv[:, :dl], kv[:, dl:]
    anc = closure_ancestors(par[0])
    for i in range(N):
        vis = np.concatenate([np.ones(P, bool), anc[i]])
        for h in range(H):
            k_nope = ckv @ W_UK[h]                               # [T, dn]
            v = ckv @ W_UV[h]                                    # [T, dv]
            s = scale * (k_nope @ q_nope[i, h] + kpe @ q_pe[i, h].astype(np.float64))
            s = torch.from_numpy(s[vis])
            w = torch.softmax(s, 0).numpy()
            ref = w @ v[vis]
            np.testing.assert_allclose(out[i * H + h] @ W_UV[h], ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[i * H + h], torch.logsumexp(s, 0).item(), rtol=1e-12)


def test_attn_zero_query_closed_form(orc):
    """q = 0: every visible score is 0, out = mean of the visible c_kv rows and lse = ln|V|."""
    rng = np.random.default_rng(15)
    B, H, N, dl, dr = 2, 2, 12, 64, 16
    pool, base, Ps, q, par = _small_case(rng, B, H, N, [9, 50], dl, dr)
    q[:] = 0
    out, lse = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.3)
    for b in range(B):
        P = int(Ps[b])
        anc = closure_ancestors(par[b])
        ckv = _f64(pool[base[b]: base[b] + P + N, :dl])
        for i in range(N):
            vis = np.concatenate([np.ones(P, bool), anc[i]])
            for h in range(H):
                r = (b * N + i) * H + h
                np.testing.assert_allclose(out[r], ckv[vis].mean(0), rtol=1e-12, atol=1e-14)
                assert abs(lse[r] - np.log(vis.sum())) < 1e-12


def test_attn_constant_values(orc):
    """All latent rows equal to one vector v (any rope keys): out = v."""
    rng = np.random.default_rng(16)
    H, N, dl, dr, P = 2, 7, 64, 16, 30
    pool, base, Ps, q, par = _small_case(rng, 1, H, N, P, dl, dr)
    v = rng.standard_normal(dl).astype(np.float32)
    pool[base[0]: base[0] + P + N, :dl] = v
    out, _ = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v.astype(np.float64), out.shape), rtol=1e-12)


def test_attn_weights_sum_to_one_and_row_sampling(orc):
    rng = np.random.default_rng(17)
    B, H, N, dl, dr = 2, 4, 16, 64, 16
    pool, base, Ps, q, par = _small_case(rng, B, H, N, [200, 3], dl, dr, "bf16")
    out, lse, ws = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.125, with_wsum=True)
    assert np.abs(ws - 1).max() < 1e-12
    rows = np.array([0, 5, 77, B * N * H - 1], np.int64)
    o2, l2 = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.125, rows=rows)
    assert (o2 == out[rows]).all() and (l2 == lse[rows]).all()


def test_attn_bf16_equals_exact_f32_widening(orc):
    """bf16 inputs are widened exactly: the same values given as fp32 give identical results."""
    rng = np.random.default_rng(18)
    H, N, dl, dr = 2, 5, 64, 16
    pool, base, Ps, q, par = _small_case(rng, 1, H, N, 40, dl, dr, "bf16")
    out_b, lse_b = _oracle_attn(orc, pool, base, Ps, q, par, H, dl, 0.2)
    out_f, lse_f = _oracle_attn(orc, synth.bf16_bits_to_f32(pool), base, Ps,
                                synth.bf16_bits_to_f32(q), par, H, dl, 0.2)
    assert (out_b == out_f).all() and (lse_b == lse_f).all()


def test_attn_rejects_invalid_tree(orc):
    rng = np.random.default_rng(19)
    pool, base, Ps, q, par = _small_case(rng, 1, 1, 3, 4, 64, 16)
    par[0, 2] = 2
    with pytest.raises(RuntimeError):
        _oracle_attn(orc, pool, base, Ps, q, par, 1, 64, 0.1)


# --------------------------------------------------------------- argmax ----

def test_argmax_matches_numpy(orc):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((37, 1000)).astype(np.float32)
    x[3, [5, 900]] = 50.0                       # tie: first index wins
    x[4, :] = 0.0                               # all equal -> 0
    x[5, 7] = np.nan                            # NaN wins (numpy convention)
    x[6, [2, 9]] = np.nan                       # first NaN
    x[7, :] = -np.inf
    x[8, 10] = np.inf
    x[9, :] = -1.0
    x[9, 4] = -0.0
    x[9, 6] = 0.0                               # -0 == +0: first of the two
    np.testing.assert_array_equal(orc.argmax(x), np.argmax(x, axis=1))


def test_argmax_bf16_and_strided(orc):
    rng = np.random.default_rng(22)
    big = rng.standard_normal((16, 300)).astype(np.float32)
    xb = synth.to_bf16_bits(big)                # many exact ties after rounding
    np.testing.assert_array_equal(orc.argmax(xb), np.argmax(synth.bf16_bits_to_f32(xb), axis=1))
    view = big[:, 10:250]
    np.testing.assert_array_equal(orc.argmax(view), np.argmax(view, axis=1))


# --------------------------------------------------------------- accept ----

def test_accept_golden_tree7(orc):
    g = json.load(open(os.path.join(GOLDEN, "tree7.json")))
    par = np.array([g["parents"]], np.int32)
    for c in g["accept_cases"]:
        acc, path, tok = orc.greedy_accept(np.array([c["target"]]), np.array([c["draft"]]), par)
        assert acc[0] == c["accept_len"], c["why"]
        assert path[0].tolist() == c["path"], c["why"]
        assert tok[0].tolist() == c["tokens"], c["why"]


def _check_accept(par, draft, t, acc, path, tok):
    """The returned path is valid, maximal and lowest-numbered at every step."""
    N = len(par)
    n = acc + 1
    p = path[:n].tolist()
    assert p[0] == 0 and (path[n:] == -1).all()
    for a, c in zip(p, p[1:]):
        assert par[c] == a and draft[c] == t[a]
        lower = [k for k in range(1, c) if par[k] == a and draft[k] == t[a]]
        assert not lower
    last = p[-1]
    assert not [k for k in range(1, N) if par[k] == last and draft[k] == t[last]]
    assert tok[:n].tolist() == [int(draft[c]) for c in p[1:]] + [int(t[last])]
    assert (tok[n:] == -1).all()


def _all_valid_paths(par, draft, t):
    """Brute force: every root-to-node path whose every step matches."""
    N = len(par)
    out = []
    for node in range(N):
        chain = [node]
        while chain[-1] != 0:
            chain.append(int(par[chain[-1]]))
        chain = chain[::-1]
        if all(draft[c] == t[a] for a, c in zip(chain, chain[1:])):
            out.append(chain)
    return out


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5])
def test_accept_exhaustive_vocab2(orc, N):
    """Every tree with N <= 5 nodes x every draft pattern x every target
    pattern over a 2-token vocabulary, batched."""
    cases = []
    for par in all_parent_arrays(N):
        for dr in itertools.product((0, 1), repeat=N - 1):
            for tt in itertools.product((0, 1), repeat=N):
                cases.append((par, np.array((5,) + dr, np.int32), np.array(tt, np.int32)))
    pars = np.stack([c[0] for c in cases])
    drafts = np.stack([c[1] for c in cases])
    ts = np.stack([c[2] for c in cases])
    acc, path, tok = orc.greedy_accept(ts, drafts, pars)
    for b, (par, dr, tt) in enumerate(cases):
        _check_accept(par, dr, tt, int(acc[b]), path[b], tok[b])
        valid = _all_valid_paths(par, dr, tt)
        assert path[b, : acc[b] + 1].tolist() in valid
        # when siblings never share a token the greedy path is the longest valid path
        sib_distinct = all(len({int(dr[k]) for k in range(1, N) if par[k] == a}) ==
                           sum(1 for k in range(1, N) if par[k] == a) for a in range(N))
        if sib_distinct:
            assert acc[b] + 1 == max(len(v) for v in valid)


def test_accept_random_large(orc):
    rng = np.random.default_rng(23)
    B, N = 64, 64
    par = synth.random_parents(rng, B, N)
    draft = rng.integers(0, 3, size=(B, N)).astype(np.int32)
    t = synth.planted_targets(rng, par, draft, 3, 0.7)
    acc, path, tok = orc.greedy_accept(t, draft, par)
    for b in range(B):
        _check_accept(par[b], draft[b], t[b], int(acc[b]), path[b], tok[b])


def test_speculative_equals_autoregressive_greedy(orc):
    """Greedy-exact invariant ('The Architecture of Pragmatic Ambition',
    section 'The Reframing'): with a deterministic target whose next token
    is a hash of the whole committed sequence, repeated draft-tree
    verification + greedy acceptance emits exactly the autoregressive greedy
    sequence, whatever the drafts are."""
    V = 5

    def next_tok(seq):
        h = 0
        for x in seq:
            h = (h * 1000003 + x + 1) % 2147483647
        return (h >> 3) % V

    prompt = [1, 2, 3]
    ar = list(prompt)
    for _ in range(60):
        ar.append(next_tok(ar))
    rng = np.random.default_rng(24)
    seq = list(prompt)
    steps = 0
    while len(seq) < len(ar):
        N = int(rng.integers(1, 12))
        par = synth.random_parents(rng, 1, N)[0]
        draft = rng.integers(0, V, size=N).astype(np.int32)
        draft[0] = seq[-1]
        # target token after node c = next_tok(committed + tokens on the path to c)
        t = np.zeros(N, np.int32)
        for c in range(N):
            chain = [c]
            while chain[-1] != 0:
                chain.append(int(par[chain[-1]]))
            toks = [int(draft[x]) for x in chain[::-1][1:]]
            t[c] = next_tok(seq + toks)
        acc, path, tok = orc.greedy_accept(t[None], draft[None], par[None])
        seq.extend(tok[0, : acc[0] + 1].tolist())
        steps += 1
    assert seq[: len(ar)] == ar
    assert steps < len(ar) - len(prompt)    # some drafts were accepted


# ----------------------------------------------------------- compaction ----

def _tagged_pool(rows, dl, dr, dtype):
    """Row r holds r // 256 in even columns and r % 256 in odd columns: small
    integers, exact in fp32 and bf16, so every row carries a distinct tag."""
    r = np.arange(rows)
    v = np.where(np.arange(dl + dr)[None, :] % 2 == 0, (r // 256)[:, None], (r % 256)[:, None])
    v = v.astype(np.float32)
    return v if dtype == "f32" else synth.to_bf16_bits(v)


def _tag(row, dtype):
    """Decode the tag of one row; -1 if the columns disagree."""
    v = row.astype(np.float64) if dtype == "f32" else synth.bf16_bits_to_f32(row).astype(np.float64)
    hi, lo = v[0::2], v[1::2]
    if (hi != hi[0]).any() or (lo != lo[0]).any():
        return -1
    return int(hi[0] * 256 + lo[0])


def test_compact_golden(orc):
    g = json.load(open(os.path.join(GOLDEN, "tree7.json")))["compact_case"]
    pool = _tagged_pool(40, 8, 4, "f32")
    new_pl, src = orc.compact_kv(pool[:, :8], pool[:, 8:], np.array([10]), np.array([g["prefix_len"]]),
                                 np.array([g["path"]]), np.array([g["accept_len"]]))
    assert new_pl[0] == g["new_prefix_len"]
    assert src[0].tolist() == g["src_slot"]
    P = g["prefix_len"]
    for j, s in enumerate(g["new_slot_sources"]):
        assert _tag(pool[10 + P + j], "f32") == 10 + s


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compact_tagged_rows(orc, dtype):
    """Tagged rows: after compaction slot P+j holds old slot P+path[j]
    (c_kv and k_pe), rows below P and from P+k+1 on are unchanged, and the
    length is P+k+1.  Covers the aliasing path [0,1,2,...] and sparse paths."""
    N, dl, dr = 12, 16, 8
    paths = [[0], [0, 1, 2, 3], [0, 5, 9], [0, 1, 4, 5, 11], list(range(12)), [0, 11]]
    B = len(paths)
    P = np.array([3, 0, 20, 7, 1, 50], np.int32)
    base = np.array([2 + 80 * b for b in range(B)], np.int64)
    pool = _tagged_pool(80 * B + 4, dl, dr, dtype)
    before = pool.copy()
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b, p in enumerate(paths):
        path[b, : len(p)] = p
        acc[b] = len(p) - 1
    new_pl, src = orc.compact_kv(pool[:, :dl], pool[:, dl:], base, P, path, acc)
    assert (new_pl == P + acc + 1).all()
    for b, p in enumerate(paths):
        for j in range(N):
            r = base[b] + P[b] + j
            if j < len(p):
                assert _tag(pool[r], dtype) == base[b] + P[b] + p[j]
                assert src[b, j] == P[b] + p[j]
            else:
                assert (pool[r] == before[r]).all() and src[b, j] == -1
        lo = base[b]
        assert (pool[lo: lo + P[b]] == before[lo: lo + P[b]]).all()


def test_compact_separate_strides(orc):
    """c_kv and k_pe in two arrays with different row strides."""
    rng = np.random.default_rng(25)
    ckv = rng.standard_normal((30, 24)).astype(np.float32)[:, :16]
    kpe = rng.standard_normal((30, 8)).astype(np.float32)
    c0, k0 = ckv.copy(), kpe.copy()
    path = np.array([[0, 2, 3, -1]], np.int32)
    new_pl, src = orc.compact_kv(ckv, kpe, np.array([4]), np.array([5]), path, np.array([2]))
    assert new_pl[0] == 8
    for j, s in enumerate([0, 2, 3]):
        assert (ckv[9 + j] == c0[9 + s]).all() and (kpe[9 + j] == k0[9 + s]).all()
