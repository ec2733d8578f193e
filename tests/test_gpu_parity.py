"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Discrete outputs (mask, depth, argmax, accept, paths,
tokens, compacted rows, lengths) must match bit for bit; attention outputs
within relative L2 1e-5 (fp32 inputs) / 1e-2 (bf16 inputs, fp32 accumulate)."""
import itertools

import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, as_f64, check_attn, oracle_attn, to_dev, to_host

pytestmark = pytest.mark.gpu


def all_parent_arrays(N):
    for tail in itertools.product(*[range(i) for i in range(1, N)]):
        yield np.array((-1,) + tail, np.int32)


# ----------------------------------------------------------------- mask ----

def _mask_check(orc, pars):
    m, d, e = ddt.build_mask(to_dev(pars))
    torch.cuda.synchronize()
    om, od, oe = orc.build_mask(pars)
    assert (to_host(m).view(np.uint64) == om).all()
    assert (to_host(d) == od).all()
    assert (to_host(e) == oe).all()


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8])
def test_mask_every_tree(orc, N):
    _mask_check(orc, np.stack(list(all_parent_arrays(N))))


@pytest.mark.parametrize("N", [63, 64, 65, 130, 1024])
def test_mask_random_chain_star(orc, N):
    rng = np.random.default_rng(N)
    pars = synth.random_parents(rng, 5, N)
    pars[3] = np.arange(-1, N - 1)
    pars[4] = 0
    pars[4, 0] = -1
    _mask_check(orc, pars)


def test_mask_invalid_trees(orc):
    pars = np.array([[-1, 0, 1, 2], [0, 0, 1, 2], [-1, 1, 0, 0], [-1, 0, 3, 1], [-1, -1, 0, 1]], np.int32)
    _mask_check(orc, pars)


# --------------------------------------------------------------- accept ----

@pytest.mark.parametrize("N", [1, 2, 3, 4, 5])
def test_accept_exhaustive_vocab2(orc, N):
    cases = [(p, (5,) + d, t) for p in all_parent_arrays(N)
             for d in itertools.product((0, 1), repeat=N - 1)
             for t in itertools.product((0, 1), repeat=N)]
    par = np.stack([c[0] for c in cases])
    dr = np.array([c[1] for c in cases], np.int32)
    tt = np.array([c[2] for c in cases], np.int32)
    acc, path, tok = ddt.greedy_accept(to_dev(tt), to_dev(dr), to_dev(par))
    oa, op, ot = orc.greedy_accept(tt, dr, par)
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()


@pytest.mark.parametrize("N,V", [(64, 3), (200, 2), (1024, 2), (1024, 100)])
def test_accept_random(orc, N, V):
    rng = np.random.default_rng(N + V)
    B = 16
    par = synth.random_parents(rng, B, N)
    par[0] = np.arange(-1, N - 1)               # a chain: the walk can go N-1 deep
    dr = rng.integers(0, V, size=(B, N)).astype(np.int32)
    t = synth.planted_targets(rng, par, dr, V, 0.8)
    t[0, :-1] = dr[0, 1:]
    acc, path, tok = ddt.greedy_accept(to_dev(t), to_dev(dr), to_dev(par))
    oa, op, ot = orc.greedy_accept(t, dr, par)
    assert oa[0] == N - 1
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()


# --------------------------------------------------------------- argmax ----

def test_argmax_workspace_reuse(orc):
    """One workspace across calls: each call must leave it ready for the next."""
    rows, V = 64, 163840
    ws = torch.zeros((ddt.argmax_workspace_bytes(rows, V),), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(7)
    for k in range(3):
        x = rng.standard_normal((rows, V)).astype(np.float32)
        x[np.arange(rows), rng.integers(0, V, rows)] += 10.0 + k
        got = to_host(ddt.argmax(to_dev(x), workspace=ws))
        assert (got == orc.argmax(x)).all(), k
    assert int(ws.sum().item()) == 0


@pytest.mark.parametrize("rows,V", [(64, 163840), (3, 1), (5, 1000), (2100, 4099), (2048, 4096), (1, 300001)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax(orc, rows, V, dtype):
    rng = np.random.default_rng(rows * 7 + V)
    x = rng.standard_normal((rows, V)).astype(np.float32)
    if V > 10 and rows > 4:
        x[0, [3, V - 2]] = 40.0                     # tie -> lower index
        x[1, :] = -3.0                              # all equal -> 0
        x[2, V // 2] = np.nan                       # NaN wins
        x[3, [V // 3, V - 1]] = np.nan              # first NaN wins
        x[4, :] = -1.0
        x[4, [5, 9]] = [-0.0, 0.0]                  # -0 == +0 -> index 5
    if V > 200 and rows > 6:
        x[5, :] = -np.inf                           # all -inf -> index 0
        x[6, :] = 0.0
        x[6, 150] = 1e-39                           # a positive denormal is the maximum
    if dtype == "bf16":
        x = synth.to_bf16_bits(np.nan_to_num(x, nan=0.0))
        x[2 % rows, V // 2] = synth.BF16_NAN
    got = to_host(ddt.argmax(to_dev(x)))
    assert (got == orc.argmax(x)).all()


def test_argmax_unaligned_view(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, 5003)).astype(np.float32)
    dev = to_dev(x)[:, 1:4999]                      # not 16-byte aligned rows
    got = to_host(ddt.argmax(dev))
    assert (got == orc.argmax(x[:, 1:4999])).all()


# ------------------------------------------------------------ compaction ----

def _tagged(rows, width, dtype):
    r = np.arange(rows)
    v = np.where(np.arange(width)[None, :] % 2 == 0, (r // 256)[:, None], (r % 256)[:, None]).astype(np.float32)
    return v if dtype == "f32" else synth.to_bf16_bits(v)


@pytest.mark.parametrize("dtype,dl,dr", [("bf16", 512, 64), ("f32", 64, 16), ("bf16", 6, 2)])
def test_compact(orc, dtype, dl, dr):
    N = 40
    paths = [[0], [0, 1, 2, 3], [0, 5, 9], [0, 1, 4, 5, 39], list(range(40)), [0, 39], [0, 2, 3, 4, 5, 6, 7]]
    B = len(paths)
    P = np.array([3, 0, 20, 700, 1, 50, 9], np.int32)
    cap = 800
    base = np.array([5 + (cap + 3) * b for b in range(B)], np.int64)
    pool = _tagged(int(base[-1]) + cap + 5, dl + dr, dtype)
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b, p in enumerate(paths):
        path[b, : len(p)] = p
        acc[b] = len(p) - 1
    dpool = to_dev(pool)
    dpl = to_dev(P)
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    ddt.compact_kv(dpool[:, :dl], dpool[:, dl:], to_dev(base), dpl, to_dev(path), to_dev(acc), src)
    opool = pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], base, P, path, acc)
    assert (to_host(dpl) == opl).all()
    assert (to_host(src) == osrc).all()
    assert (to_host(dpool) == opool).all()


def test_compact_separate_arrays_and_invalid(orc):
    rng = np.random.default_rng(3)
    ckv = rng.standard_normal((300, 64)).astype(np.float32)
    kpe = rng.standard_normal((300, 16)).astype(np.float32)
    P = np.array([10, 20, 30], np.int32)
    base = np.array([0, 100, 200], np.int64)
    path = np.array([[0, 2, 5, -1, -1, -1], [0, 1, 1, -1, -1, -1], [0, 3, -1, -1, -1, -1]], np.int32)
    acc = np.array([2, 2, 7], np.int32)             # request 1: path not increasing, request 2: bad length
    dc, dk = to_dev(ckv), to_dev(kpe)
    dpl = to_dev(P)
    src = torch.empty((3, 6), dtype=torch.int32, device="cuda")
    ddt.compact_kv(dc, dk, to_dev(base), dpl, to_dev(path), to_dev(acc), src)
    c2, k2 = ckv.copy(), kpe.copy()
    orc.compact_kv(c2[0:100], k2[0:100], base[:1], P[:1], path[:1], acc[:1])
    assert (to_host(dc) == c2).all() and (to_host(dk) == k2).all()
    assert to_host(dpl).tolist() == [13, 20, 30]
    s = to_host(src)
    assert s[0].tolist() == [10, 12, 15, -1, -1, -1] and (s[1:] == -1).all()


@pytest.mark.parametrize("dtype,dl,dr,N", [("bf16", 512, 64, 64), ("f32", 64, 16, 40), ("bf16", 512, 64, 1024)])
def test_accept_compact_fused(orc, dtype, dl, dr, N):
    """ddt_accept_compact == greedy acceptance then compaction (oracle), on
    random and chain trees (a full chain moves every row onto itself)."""
    rng = np.random.default_rng(N + dl)
    B, V = 6, 3
    par = synth.random_parents(rng, B, N)
    par[0] = np.arange(-1, N - 1)
    dr_ = rng.integers(0, V, size=(B, N)).astype(np.int32)
    t = synth.planted_targets(rng, par, dr_, V, 0.8)
    t[0, :-1] = dr_[0, 1:]                         # request 0 accepts its whole chain
    P = rng.integers(0, 300, B).astype(np.int32)
    cap = 300 + N + 8
    base = np.array([3 + cap * b for b in range(B)], np.int64)
    pool = _tagged(int(base[-1]) + cap, dl + dr, dtype)
    dpool, dpl = to_dev(pool), to_dev(P)
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    acc, path, tok = ddt.accept_compact(to_dev(t), to_dev(dr_), to_dev(par), dpool[:, :dl], dpool[:, dl:],
                                        to_dev(base), dpl, src_slot=src)
    oa, op, ot = orc.greedy_accept(t, dr_, par)
    opool = pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], base, P, op, oa)
    assert oa[0] == N - 1
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(dpl) == opl).all() and (to_host(src) == osrc).all()
    assert (to_host(dpool) == opool).all()


# ------------------------------------------------------------- attention ----

def _attn_gpu(dw: DevWorkload, kv_chunk=0):
    w = dw.w
    mask, _, err = ddt.build_mask(dw.parents)
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask,
                               H=w.H, scale=w.scale, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert (to_host(err) == 0).all()
    return to_host(out), to_host(lse)


def _attn_check(orc, w, kv_chunks=(0,), rows=None):
    dw = DevWorkload(w)
    ref_out, ref_lse = oracle_attn(orc, w, rows=rows)
    results = []
    for ch in kv_chunks:
        out, lse = _attn_gpu(dw, ch)
        o = as_f64(out)
        if rows is not None:
            o, lse = o[rows], lse[rows]
        e = check_attn(o, lse, ref_out, ref_lse, w.dtype, f"{w.name} kv_chunk={ch}")
        print(f"{w.name} kv_chunk={ch}: rel_l2 out {e[0]:.3e} lse {e[1]:.3e}, max row {e[2]:.3e}, "
              f"max lse error {e[3]:.3f} of its bound")
        results.append(o)
    return results


@pytest.mark.parametrize("cfg,over,logit_shape,ldt,kv_chunk", [
    (2, dict(), (64, 163840), "f32", 0),                       # the K2-like head share, split keys
    (2, dict(), (64, 163840), "bf16", 1 << 20),                # one split per request
    (1, dict(), (2100, 4099), "f32", 0),                       # fp32 attention; argmax rows unchunked
    (3, dict(B=3, prefix_range=(100, 3000)), (96, 50001), "bf16", 224),
    (2, dict(), (9, 40000), "f32", 0),                         # streamed rows: NaN, -inf, signed zeros
    (2, dict(), (9, 70016), "bf16", 0),
])
def test_attn_argmax_fused(orc, cfg, over, logit_shape, ldt, kv_chunk):
    """verify_attn_argmax == verify_attn (against the oracle) and argmax
    (against the oracle) from one launch; the argmax workspace is reused."""
    w = synth.workload(cfg, with_logits=False, **over) if cfg == 2 else synth.workload(cfg, **over)
    dw = DevWorkload(w)
    rng = np.random.default_rng(sum(logit_shape))
    x = rng.standard_normal(logit_shape).astype(np.float32)
    x[np.arange(logit_shape[0]), rng.integers(0, logit_shape[1], logit_shape[0])] += 8.0
    x[0, [5, logit_shape[1] - 3]] = 50.0                        # tie -> lower index
    if logit_shape[0] == 9:
        V = logit_shape[1]
        x[1] = -np.inf                                          # every value -inf: index 0
        x[2, [100, V // 2]] = [99.0, np.nan]                    # NaN above every number
        x[3] = -1.0
        x[3, [V // 3, V // 3 + 1, V - 7]] = [-0.0, 0.0, 0.0]    # -0 == +0: the first zero
        x[4, V - 1] = 1e30                                      # last element of the row
        x[5, 7] = np.inf
        x[6, [V - 5, V - 2]] = [np.nan, np.nan]                 # NaN in a row's final stage
    if ldt == "bf16":
        x = synth.to_bf16_bits(x)
    logits = to_dev(x)
    mask, _, _ = ddt.build_mask(dw.parents)
    ref_out, ref_lse = oracle_attn(orc, w)
    ref_idx = orc.argmax(x)
    ws = torch.zeros((max(ddt.argmax_workspace_bytes(*logit_shape), 16),), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        out, lse, idx = ddt.verify_attn_argmax(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len,
                                               mask, logits, H=w.H, scale=w.scale, kv_chunk=kv_chunk,
                                               argmax_workspace=ws)
        assert (to_host(idx) == ref_idx).all(), rep
        check_attn(to_host(out), to_host(lse), ref_out, ref_lse, w.dtype, f"rep {rep}")
    assert int(ws.sum().item()) == 0


@pytest.mark.parametrize("with_mask", [True, False], ids=["mask", "in_kernel_mask"])
@pytest.mark.parametrize("cfg,over,V,ldt,kv_chunk", [
    (2, dict(), None, "f32", 0),                                  # the K2-like head share, its own logits
    (1, dict(B=3, H=3, N=5, prefix=61), 4096, "f32", 0),          # fp32 attention
    (3, dict(B=3, prefix_range=(100, 3000)), None, "bf16", 224),  # ragged prefixes, full vocabulary
    (3, dict(B=2, prefix_range=(0, 40)), 1000, "f32", 0),         # no split: the merge launch only accepts
    (1, dict(B=2, H=1, N=128, prefix=70), 500, "f32", 0),         # two mask words, one row per node
    (1, dict(B=2, H=2, N=100, prefix=9, chain=True), 500, "f32", 32),  # chains: deepest trees
])
def test_verify_step(orc, cfg, over, V, ldt, kv_chunk, with_mask):
    """ddt_verify_step == attention and argmax, then greedy acceptance on the
    argmax ids and compaction with the length update (all against the
    oracle); the committed lengths are read from one array and the advanced
    ones written to another.  Without a mask the attention derives the
    ancestor bits from the parents itself."""
    over = dict(over)
    chain = over.pop("chain", False)
    w = synth.workload(cfg, **over)
    if chain:
        w.parents[:] = np.arange(-1, w.N - 1, dtype=np.int32)
    rng = np.random.default_rng(17 + cfg)
    if w.logits is not None:
        x = w.logits
    else:
        V = w.vocab if V is None else V
        t = synth.planted_targets(rng, w.parents, w.draft_ids % V, V, 0.8)
        w.draft_ids = w.draft_ids % V
        x = synth.target_logits(rng, t.reshape(-1), V)
        if ldt == "bf16":
            x = synth.to_bf16_bits(x)
    dw = DevWorkload(w)
    B, N = w.B, w.N
    ref_out, ref_lse = oracle_attn(orc, w)        # attention reads the cache before compaction
    t_ref = orc.argmax(x).reshape(B, N)
    oa, op, ot = orc.greedy_accept(t_ref, w.draft_ids, w.parents)
    opool = w.pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :w.d_lat], opool[:, w.d_lat:], w.kv_base, w.prefix_len, op, oa)
    mask = ddt.build_mask(dw.parents)[0] if with_mask else None
    new_pl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    out, lse, idx, acc, path, tok, npl = ddt.verify_step(
        dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask, to_dev(x), dw.draft,
        dw.parents, dw.prefix_dev, H=w.H, scale=w.scale, new_prefix_len=new_pl, src_slot=src, kv_chunk=kv_chunk)
    assert (to_host(idx).reshape(B, N) == t_ref).all()
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, w.dtype)
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(npl) == opl).all() and (to_host(dw.prefix_dev) == w.prefix_len).all()
    assert (to_host(src) == osrc).all()
    got = np.ascontiguousarray(to_host(dw.pool))
    assert got.dtype == opool.dtype and (got.view(np.uint8) == opool.view(np.uint8)).all()  # bits: the pool holds NaN
    print(f"{w.name} B={B} N={N}: accepted {oa.tolist()}")


def test_verify_step_invalid_tree_without_mask():
    """An invalid tree gives its rows no tree keys without a mask exactly as
    build_mask's all-zero mask does (same kernel, same bits: bit-exact);
    the valid request beside it is unaffected."""
    w = synth.workload(3, B=2, N=40, prefix_range=(50, 400))
    w.parents[1, 9] = 12                                  # parent after its child: invalid
    V = 700
    rng = np.random.default_rng(5)
    w.draft_ids = w.draft_ids % V
    x = synth.target_logits(rng, synth.planted_targets(rng, w.parents, w.draft_ids, V, 0.8).reshape(-1), V)
    res = []
    for with_mask in (True, False):
        dw = DevWorkload(w)
        mask, _, err = ddt.build_mask(dw.parents)
        assert to_host(err).tolist() == [0, 1]
        r = ddt.verify_step(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len,
                            mask if with_mask else None, to_dev(x), dw.draft, dw.parents, dw.prefix_dev,
                            H=w.H, scale=w.scale, new_prefix_len=torch.empty_like(dw.prefix_dev))
        res.append([to_host(t) for t in r] + [to_host(dw.pool)])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_attn_config1_tiny_fp32(orc):
    _attn_check(orc, synth.workload(1), kv_chunks=(0, 32, 64))


def test_attn_config2_k2_head_share(orc):
    w = synth.workload(2, with_logits=False)
    _attn_check(orc, w, kv_chunks=(0, 32, 224, 4160))


def test_attn_config3_ragged_small(orc):
    w = synth.workload(3, B=5, prefix_range=(0, 3000))
    _attn_check(orc, w, kv_chunks=(0, 96, 1 << 20))


@pytest.mark.parametrize("cfg,over", [
    (1, dict(prefix=0)),                    # no prefix: only tree keys
    (1, dict(N=1, prefix=5)),               # budget 0: single-token decode
    (1, dict(H=3, N=5, prefix=61)),         # 15 rows: partial row tiles, ragged key tail
    (1, dict(H=1, N=1024, prefix=3)),       # maximum node count
    (3, dict(B=3, N=1, prefix_range=(0, 40))),
    (3, dict(B=2, H=1, N=1024, prefix_range=(31, 33))),
    (2, dict(H=3, N=7, prefix=1, with_logits=False)),
    (3, dict(B=128, N=4, prefix_range=(0, 300))),   # the maximum batch, ragged prefixes
])
def test_attn_edge_cases(orc, cfg, over):
    _attn_check(orc, synth.workload(cfg, **over), kv_chunks=(0, 32))


def test_attn_chain_tree_is_causal(orc):
    """Chain tree through the whole path: equal to the oracle, which is pinned to causal SDPA."""
    w = synth.workload(3, B=2, N=64, prefix_range=(100, 500))
    w.parents[:] = np.arange(-1, 63)
    _attn_check(orc, w, kv_chunks=(0, 64))


def test_attn_config3_full_every_row(orc):
    """The batched ragged configuration at full shape (16 requests, prefixes
    U[1024, 32768]): every one of the 4096 query rows against the oracle."""
    w = synth.workload(3)
    _attn_check(orc, w)


def test_attn_config4_full_sampled(orc):
    """The long-context configuration (4 x 131072 keys, 64 heads, 128 nodes):
    several rounds of workgroups dealt in units of row tiles across the
    XCDs, tiles touched into L2 before their loads; 336 sampled rows (1 %
    of the 32768), each within the per-row bound."""
    w = synth.workload(4)
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(w.rows, 336, replace=False))
    _attn_check(orc, w, rows=rows)


@pytest.mark.parametrize("fused", [True, False], ids=["verify_step", "attn_then_accept_compact"])
def test_config3_full_shape_step(orc, fused):
    """Configuration 3 at full shape (16 requests, prefixes U[1024, 32768],
    8 heads, 32 nodes, random trees), attention followed by greedy
    acceptance and compaction of the accepted path: acceptance, paths,
    tokens, lengths and the whole cache pool bit for bit against the
    oracle, attention on every row.  fused: one
    ddt_verify_step with the target ids as the argmax of planted target
    logits over the 163840-token vocabulary; else ddt_verify_attn and
    ddt_accept_compact on the target ids directly (the benchmark's form)."""
    w = synth.workload(3)
    B, N, dl = w.B, w.N, w.d_lat
    rng = np.random.default_rng(33)
    ref_out, ref_lse = oracle_attn(orc, w)
    if fused:
        x = synth.target_logits(rng, w.target_ids.reshape(-1), w.vocab)
        t_ref = orc.argmax(x).reshape(B, N)
        assert (t_ref == w.target_ids).all()
    else:
        t_ref = w.target_ids
    oa, op, ot = orc.greedy_accept(t_ref, w.draft_ids, w.parents)
    opool = w.pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], w.kv_base, w.prefix_len, op, oa)
    dw = DevWorkload(w)
    new_pl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    if fused:
        out, lse, idx, acc, path, tok, npl = ddt.verify_step(
            dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, None, to_dev(x), dw.draft,
            dw.parents, dw.prefix_dev, H=w.H, scale=w.scale, new_prefix_len=new_pl, src_slot=src)
        assert (to_host(idx).reshape(B, N) == t_ref).all()
    else:
        mask = ddt.build_mask(dw.parents)[0]
        out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask,
                                   H=w.H, scale=w.scale)
        acc, path, tok = ddt.accept_compact(dw.target, dw.draft, dw.parents, dw.ckv(), dw.kpe(), dw.kv_base,
                                            dw.prefix_dev, src_slot=src, new_prefix_len=new_pl)
    torch.cuda.synchronize()
    e = check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16")
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(new_pl) == opl).all() and (to_host(src) == osrc).all()
    assert (to_host(dw.prefix_dev) == w.prefix_len).all()
    got = np.ascontiguousarray(to_host(dw.pool))
    assert (got.view(np.uint8) == opool.view(np.uint8)).all()
    print(f"config3 full shape ({'fused' if fused else 'attn + accept_compact'}): accepted {oa.tolist()}, "
          f"rel_l2 {e[0]:.2e}, max row {e[2]:.2e}")


@pytest.mark.parametrize("cfg,over", [
    (3, dict(B=2, H=64, N=128, prefix_range=(20000, 45000))),  # whole-chunk splits in rounds, then shorter last splits
    (4, dict(B=3, H=16, N=96, prefix=9000)),                   # row tiles not a multiple of the unit
])
def test_attn_multi_round_sampled(orc, cfg, over):
    """Launches of several rounds: whole-chunk work items dealt to the XCDs
    in units of row tiles, the shorter last splits after them."""
    w = synth.workload(cfg, **over)
    rng = np.random.default_rng(w.B * 7 + w.N)
    rows = np.sort(rng.choice(w.rows, 64, replace=False))
    _attn_check(orc, w, rows=rows)


@pytest.mark.parametrize("factor", [100.0, 1e4])
def test_attn_large_score_range(orc, factor):
    """Some cache rows far into each request scaled up so their scores exceed
    the first tiles' by many orders of magnitude: the kernel's fixed softmax
    reference must be abandoned (second pass) without losing accuracy."""
    w = synth.workload(3, B=3, prefix_range=(600, 2000))
    rng = np.random.default_rng(int(factor))
    for b in range(w.B):
        rows = w.kv_base[b] + rng.choice(np.arange(300, int(w.prefix_len[b])), 3, replace=False)
        big = synth.bf16_bits_to_f32(w.pool[rows]) * np.float32(factor)
        w.pool[rows] = synth.to_bf16_bits(big)
    _attn_check(orc, w, kv_chunks=(0, 256, 1 << 20))
