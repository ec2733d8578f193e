"""Paged latent cache on the GPU: the verify attention and the whole verify
step (attention, argmax, acceptance, compaction through the block table)
with each request's slots in pages of a shared pool.

Pages are assigned by a random permutation, so requests interleave and no
request's pages are in order; every pool row no table entry names holds
NaN, so a wrong row lookup shows in the outputs.  The logical cache of
request b (slot t -> row table[b][t // ps] * ps + t % ps) is rebuilt on the
host for the oracle.  Paged attention must equal the contiguous launch bit
for bit (same plan, same arithmetic, other addresses) and match the oracle
to the bf16 bar; acceptance, compacted rows and lengths are bit-exact."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, check_attn, oracle_attn, to_dev, to_host

pytestmark = pytest.mark.gpu


def to_paged(w, ps, rng, spare=3):
    """Physical pool and block table holding w's logical cache in pages of ps rows."""
    T = w.prefix_len.astype(np.int64) + w.N
    npg = (T + ps - 1) // ps
    total = int(npg.sum()) + spare
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((w.B, int(npg.max())), np.int32)
    k = 0
    for b in range(w.B):
        table[b, : npg[b]] = perm[k: k + npg[b]]
        k += npg[b]
    nan = synth.BF16_NAN if w.dtype == "bf16" else synth.F32_NAN
    phys = np.full((total * ps, w.pool.shape[1]), nan, dtype=w.pool.dtype)
    for b in range(w.B):
        t = np.arange(T[b])
        phys[table[b, t // ps].astype(np.int64) * ps + t % ps] = w.pool[w.kv_base[b] + t]
    return phys, table


def from_paged(phys, table, ps, w):
    """w.pool with each request's logical rows [0, P+N) read back through the table."""
    pool = w.pool.copy()
    for b in range(w.B):
        t = np.arange(int(w.prefix_len[b]) + w.N)
        pool[w.kv_base[b] + t] = phys[table[b, t // ps].astype(np.int64) * ps + t % ps]
    return pool


@pytest.mark.parametrize("ps,prefix_range,kv_chunk,N", [
    (32, (100, 3000), 0, 32),
    (64, (100, 3000), 0, 32),
    (512, (100, 3000), 0, 32),
    (32, (25000, 32000), 0, 32),      # splits of ~1000 pages: the page-window ring wraps many times
    (64, (100, 3000), 1 << 20, 32),   # an explicit chunk of 2^20 keys: one split per request
    (64, (100, 1500), 256, 300),      # a large tree: splits end at each work item's last node
])
def test_paged_attention_equals_contiguous(orc, ps, prefix_range, kv_chunk, N):
    """The paged launch has the contiguous launch's plan and arithmetic, so
    the two are bit-identical, and both match the oracle."""
    w = synth.workload(3, B=2 if prefix_range[0] > 20000 or N > 128 else 4, N=N, prefix_range=prefix_range)
    rng = np.random.default_rng(ps)
    phys, table = to_paged(w, ps, rng)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    out_c, lse_c = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask,
                                   H=w.H, scale=w.scale, kv_chunk=kv_chunk)
    pd, td = to_dev(phys), to_dev(table)
    dl = w.d_lat
    out_p, lse_p = ddt.verify_attn(dw.q_lat(), dw.q_pe(), pd[:, :dl], pd[:, dl:], None, w.prefix_len, mask,
                                   H=w.H, scale=w.scale, pages=(td, ps), kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(lse_c, lse_p)
    ref_out, ref_lse = oracle_attn(orc, w)
    check_attn(to_host(out_p), to_host(lse_p), ref_out, ref_lse, "bf16")


@pytest.mark.parametrize("ps,kv_chunk", [(32, 0), (32, 1 << 20), (32, 4096), (64, 1 << 20)])
def test_paged_attention_second_pass(orc, ps, kv_chunk):
    """Scores far above the first tiles' late in each split force the second
    pass after the page-window ring has moved on: the pass refills the
    first windows, and the result is bit-identical to the contiguous launch
    and matches the oracle."""
    w = synth.workload(3, B=3, prefix_range=(6000, 9000))
    rng = np.random.default_rng(1000 + ps)
    for b in range(w.B):
        P = int(w.prefix_len[b])
        rows = w.kv_base[b] + rng.choice(np.arange(P - 1500, P), 3, replace=False)
        big = synth.bf16_bits_to_f32(w.pool[rows]) * np.float32(1e4)
        w.pool[rows] = synth.to_bf16_bits(big)
    phys, table = to_paged(w, ps, rng)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    out_c, lse_c = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask,
                                   H=w.H, scale=w.scale, kv_chunk=kv_chunk)
    pd, td = to_dev(phys), to_dev(table)
    dl = w.d_lat
    out_p, lse_p = ddt.verify_attn(dw.q_lat(), dw.q_pe(), pd[:, :dl], pd[:, dl:], None, w.prefix_len, mask,
                                   H=w.H, scale=w.scale, pages=(td, ps), kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out_c.view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(lse_c, lse_p)
    ref_out, ref_lse = oracle_attn(orc, w)
    check_attn(to_host(out_p), to_host(lse_p), ref_out, ref_lse, "bf16")


@pytest.mark.parametrize("ps,with_mask", [(32, False), (128, True), (64, False)])
def test_paged_verify_step(orc, ps, with_mask):
    """The whole step on a paged cache: attention + argmax, then acceptance
    and compaction of the accepted path's latents through the table."""
    w = synth.workload(3, B=5, prefix_range=(0, 2000))
    rng = np.random.default_rng(100 + ps)
    V = 3000
    w.draft_ids = w.draft_ids % V
    t = synth.planted_targets(rng, w.parents, w.draft_ids, V, 0.8)
    x = synth.target_logits(rng, t.reshape(-1), V)
    phys, table = to_paged(w, ps, rng)
    B, N, dl = w.B, w.N, w.d_lat

    ref_out, ref_lse = oracle_attn(orc, w)
    t_ref = orc.argmax(x).reshape(B, N)
    oa, op, ot = orc.greedy_accept(t_ref, w.draft_ids, w.parents)
    opool = w.pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], w.kv_base, w.prefix_len, op, oa)

    pd, td = to_dev(phys), to_dev(table)
    parents, draft = to_dev(w.parents), to_dev(w.draft_ids)
    prefix = to_dev(w.prefix_len)
    q = to_dev(w.q)
    mask = ddt.build_mask(parents)[0] if with_mask else None
    new_pl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    out, lse, idx, acc, path, tok, npl = ddt.verify_step(
        q[:, :dl], q[:, dl:], pd[:, :dl], pd[:, dl:], None, w.prefix_len, mask, to_dev(x), draft, parents, prefix,
        H=w.H, scale=w.scale, new_prefix_len=new_pl, src_slot=src, pages=(td, ps))
    torch.cuda.synchronize()
    assert (to_host(idx).reshape(B, N) == t_ref).all()
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16")
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(npl) == opl).all() and (to_host(src) == osrc).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    got = from_paged(got_phys, table, ps, w)
    assert (got.view(np.uint8) == opool.view(np.uint8)).all()       # bits: gaps hold NaN
    # rows no table entry names are untouched
    named = np.zeros(got_phys.shape[0], bool)
    for b in range(B):
        tt = np.arange(int(w.prefix_len[b]) + N)
        named[table[b, tt // ps].astype(np.int64) * ps + tt % ps] = True
    assert (got_phys[~named].view(np.uint8) == phys[~named].view(np.uint8)).all()
    print(f"paged ps={ps}: accepted {oa.tolist()}")


@pytest.mark.parametrize("ps,extra", [(32, 200), (64, 1000)])
def test_paged_verify_step_device_lengths(orc, ps, extra):
    """The fused step on a paged cache with the committed lengths read on
    the device: the host passes bounds `extra` keys above them, the table
    rows run that far with NaN pages past each request's keys, and the
    results (attention, acceptance, compaction through the table, lengths)
    equal the oracle's on the actual lengths."""
    w = synth.workload(3, B=4, prefix_range=(0, 2500))
    rng = np.random.default_rng(300 + ps)
    V = 2000
    w.draft_ids = w.draft_ids % V
    t = synth.planted_targets(rng, w.parents, w.draft_ids, V, 0.8)
    x = synth.target_logits(rng, t.reshape(-1), V)
    phys, table = to_paged(w, ps, rng)
    B, N, dl = w.B, w.N, w.d_lat
    npg = (w.prefix_len.astype(np.int64) + N + ps - 1) // ps
    named = set()
    for b in range(B):
        named |= set(table[b, : npg[b]].tolist())
    free = np.array(sorted(set(range(phys.shape[0] // ps)) - named), np.int32)  # NaN pages no request owns
    assert len(free) > 0
    bound = w.prefix_len.astype(np.int64) + extra
    cols = int(((bound + N + ps - 1) // ps).max())
    wide = np.empty((B, cols), np.int32)
    for b in range(B):
        wide[b, : npg[b]] = table[b, : npg[b]]
        wide[b, npg[b]:] = free[np.arange(cols - npg[b]) % len(free)]
    ref_out, ref_lse = oracle_attn(orc, w)
    t_ref = orc.argmax(x).reshape(B, N)
    oa, op, ot = orc.greedy_accept(t_ref, w.draft_ids, w.parents)
    opool = w.pool.copy()
    opl, _ = orc.compact_kv(opool[:, :dl], opool[:, dl:], w.kv_base, w.prefix_len, op, oa)
    pd, td = to_dev(phys), to_dev(wide)
    prefix = to_dev(w.prefix_len)
    q = to_dev(w.q)
    out, lse, idx, acc, path, tok, npl = ddt.verify_step(
        q[:, :dl], q[:, dl:], pd[:, :dl], pd[:, dl:], None, bound, None, to_dev(x), to_dev(w.draft_ids),
        to_dev(w.parents), prefix, H=w.H, scale=w.scale, pages=(td, ps), device_lengths=True, kv_chunk=256)
    torch.cuda.synchronize()
    assert (to_host(idx).reshape(B, N) == t_ref).all()
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16")
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(prefix) == opl).all()
    got = from_paged(np.ascontiguousarray(to_host(pd)), wide, ps, w)
    assert (got.view(np.uint8) == opool.view(np.uint8)).all()


@pytest.mark.parametrize("ps,cfg", [(1, 3), (32, 1), (256, 3)])
def test_paged_compact_kv(orc, ps, cfg):
    """Standalone compaction through a block table (ddt_compact_kv_paged):
    the accepted path's latents land at logical slots P.. of each request,
    bit for bit as the oracle's compaction of the logical cache; rows no
    table entry names are untouched."""
    w = synth.workload(3, B=6, prefix_range=(0, 900)) if cfg == 3 else synth.workload(1, B=6, N=8, prefix=45)
    rng = np.random.default_rng(7 + ps)
    B, N, dl = w.B, w.N, w.d_lat
    w.draft_ids = w.draft_ids % 50
    t = synth.planted_targets(rng, w.parents, w.draft_ids, 50, 0.85)
    oa, op, _ = orc.greedy_accept(t, w.draft_ids, w.parents)
    oa[1] = 0                                                   # a request that accepts only the root
    op[1, 1:] = -1
    phys, table = to_paged(w, ps, rng)
    opool = w.pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], w.kv_base, w.prefix_len, op, oa)

    pd, td = to_dev(phys), to_dev(table)
    dpl = to_dev(w.prefix_len)
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    ddt.compact_kv(pd[:, :dl], pd[:, dl:], None, dpl, to_dev(op), to_dev(oa), src, pages=(td, ps))
    torch.cuda.synchronize()
    assert (to_host(dpl) == opl).all() and (to_host(src) == osrc).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    got = from_paged(got_phys, table, ps, w)
    assert (got.view(np.uint8) == opool.view(np.uint8)).all()
    named = np.zeros(got_phys.shape[0], bool)
    for b in range(B):
        tt = np.arange(int(w.prefix_len[b]) + N)
        named[table[b, tt // ps].astype(np.int64) * ps + tt % ps] = True
    assert (got_phys[~named].view(np.uint8) == phys[~named].view(np.uint8)).all()


def _spare_page(table, w, ps, n_pages):
    """A page of the pool that no request's table row names."""
    T = w.prefix_len.astype(np.int64) + w.N
    owned = set()
    for b in range(w.B):
        owned.update(table[b, : (T[b] + ps - 1) // ps].tolist())
    return min(set(range(n_pages)) - owned)


def _padded_table(table, pad_rows, spare_page):
    """A device copy of `table` with pad_rows extra rows naming spare_page,
    and the [B, bt_ld] view of its first rows: slots past a request's row
    then still read valid table entries that name a valid page."""
    B, L = table.shape
    full = np.full((B + pad_rows, L), spare_page, np.int32)
    full[:B] = table
    d = to_dev(full)
    return d, d[:B]


def _oracle_compact_some(orc, pool, dl, kv_base, P, path, acc, keep):
    """The oracle's compaction of the requests in `keep` only (in place on
    pool); the others keep their length and report src_slot -1."""
    B, N = path.shape
    keep = np.asarray(keep)
    opl = np.array(P, np.int32, copy=True)
    osrc = np.full((B, N), -1, np.int32)
    if len(keep):
        pl, src = orc.compact_kv(pool[:, :dl], pool[:, dl:], kv_base[keep], P[keep], path[keep], acc[keep])
        opl[keep], osrc[keep] = pl, src
    return opl, osrc


def test_paged_compact_unmappable_left_untouched(orc):
    """ddt_compact_kv_paged with device lengths whose accepted slots run past
    the request's table row (a stale or oversized length): those requests
    are left untouched (src_slot -1, length unchanged, no row written),
    the others compacted as the oracle does."""
    w = synth.workload(3, B=3, N=8, prefix_range=(40, 90))
    ps, B, N, dl = 32, 3, 8, 512
    rng = np.random.default_rng(11)
    phys, table = to_paged(w, ps, rng, spare=2)
    spare = _spare_page(table, w, ps, phys.shape[0] // ps)
    L = table.shape[1]
    path = np.full((B, N), -1, np.int32)
    path[:, :3] = [0, 1, 3]
    acc = np.full(B, 2, np.int32)
    P_dev = w.prefix_len.copy()
    P_dev[1] = L * ps - 2                               # slot P+3 is past row 1 (would read row 2's entries)
    P_dev[2] = L * ps - 1                               # the last request: past the table itself
    opool = w.pool.copy()
    opl, osrc = _oracle_compact_some(orc, opool, dl, w.kv_base, w.prefix_len, path, acc, [0])
    pd = to_dev(phys)
    td_full, td = _padded_table(table, 2, spare)
    dpl = to_dev(P_dev)
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    ddt.compact_kv(pd[:, :dl], pd[:, dl:], None, dpl, to_dev(path), to_dev(acc), src, pages=(td, ps))
    torch.cuda.synchronize()
    got_pl = to_host(dpl)
    assert got_pl[0] == opl[0] and got_pl[1] == P_dev[1] and got_pl[2] == P_dev[2]
    s = to_host(src)
    assert (s[0] == osrc[0]).all() and (s[1:] == -1).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    assert (from_paged(got_phys, table, ps, w).view(np.uint8) == opool.view(np.uint8)).all()
    sp = slice(spare * ps, (spare + 1) * ps)
    assert (got_phys[sp].view(np.uint8) == phys[sp].view(np.uint8)).all()


def test_accept_compact_negative_length_left_untouched(orc):
    """ddt_accept_compact with a negative committed length on the device:
    acceptance outputs as usual, no row moved, new length = old length."""
    w = synth.workload(3, B=3, N=16, prefix_range=(40, 90))
    rng = np.random.default_rng(12)
    V = 4
    w.draft_ids = w.draft_ids % V
    t = synth.planted_targets(rng, w.parents, w.draft_ids, V, 0.9)
    oa, op, ot = orc.greedy_accept(t, w.draft_ids, w.parents)
    B, N, dl = w.B, w.N, w.d_lat
    P_dev = w.prefix_len.copy()
    P_dev[1] = -int(N)                      # kv_base >= 32 + ...: even a broken guard stays in the pool
    assert int(w.kv_base[1]) - N >= 0
    opool = w.pool.copy()
    opl, osrc = _oracle_compact_some(orc, opool, dl, w.kv_base, w.prefix_len, op, oa, [0, 2])
    dw = DevWorkload(w)
    dpl = to_dev(P_dev)
    npl = torch.full((B,), 99, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    acc, path, tok = ddt.accept_compact(to_dev(t), dw.draft, dw.parents, dw.ckv(), dw.kpe(), dw.kv_base, dpl,
                                        src_slot=src, new_prefix_len=npl)
    torch.cuda.synchronize()
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    got = to_host(npl)
    assert got[1] == P_dev[1] and got[0] == opl[0] and got[2] == opl[2]
    s = to_host(src)
    assert (s[1] == -1).all() and (s[0] == osrc[0]).all() and (s[2] == osrc[2]).all()
    assert (to_host(dw.pool).view(np.uint8) == opool.view(np.uint8)).all()


def test_paged_verify_step_unmappable_length(orc):
    """The paged verify step with a device length past the table row for
    one request (the host length, which plans the attention, is valid):
    that request's acceptance is reported and its cache left as it was."""
    w = synth.workload(3, B=3, prefix_range=(100, 600))
    ps = 32
    rng = np.random.default_rng(13)
    V = 3000
    w.draft_ids = w.draft_ids % V
    t = synth.planted_targets(rng, w.parents, w.draft_ids, V, 0.8)
    x = synth.target_logits(rng, t.reshape(-1), V)
    phys, table = to_paged(w, ps, rng, spare=2)
    spare = _spare_page(table, w, ps, phys.shape[0] // ps)
    B, N, dl = w.B, w.N, w.d_lat
    L = table.shape[1]
    t_ref = orc.argmax(x).reshape(B, N)
    oa, op, ot = orc.greedy_accept(t_ref, w.draft_ids, w.parents)
    P_dev = w.prefix_len.copy()
    P_dev[2] = L * ps                                   # every slot P.. is past the last request's row
    opool = w.pool.copy()
    opl, osrc = _oracle_compact_some(orc, opool, dl, w.kv_base, w.prefix_len, op, oa, [0, 1])
    pd = to_dev(phys)
    td_full, td = _padded_table(table, 2 + N // ps, spare)
    q = to_dev(w.q)
    parents, draft = to_dev(w.parents), to_dev(w.draft_ids)
    dpl = to_dev(P_dev)
    npl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    _, _, idx, acc, path, tok, _ = ddt.verify_step(
        q[:, :dl], q[:, dl:], pd[:, :dl], pd[:, dl:], None, w.prefix_len, None, to_dev(x), draft, parents, dpl,
        H=w.H, scale=w.scale, new_prefix_len=npl, src_slot=src, pages=(td, ps))
    torch.cuda.synchronize()
    assert (to_host(idx).reshape(B, N) == t_ref).all()
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    got = to_host(npl)
    assert got[2] == P_dev[2] and (got[:2] == opl[:2]).all()
    s = to_host(src)
    assert (s[2] == -1).all() and (s[:2] == osrc[:2]).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    assert (from_paged(got_phys, table, ps, w).view(np.uint8) == opool.view(np.uint8)).all()
    sp = slice(spare * ps, (spare + 1) * ps)
    assert (got_phys[sp].view(np.uint8) == phys[sp].view(np.uint8)).all()


@pytest.mark.parametrize("ps,cfg", [(1, 3), (32, 1), (128, 3)])
def test_paged_accept_compact(orc, ps, cfg):
    """Acceptance and compaction in one launch through a block table
    (ddt_accept_compact_paged): acceptance outputs, advanced lengths and
    source slots bit-exact against the oracle's acceptance and compaction of
    the logical cache, the compacted rows bit for bit, rows no table entry
    names untouched, and the committed lengths left as they were."""
    w = synth.workload(3, B=6, prefix_range=(0, 900)) if cfg == 3 else synth.workload(1, B=6, N=8, prefix=45)
    rng = np.random.default_rng(31 + ps)
    B, N, dl = w.B, w.N, w.d_lat
    w.draft_ids = w.draft_ids % 50
    t = synth.planted_targets(rng, w.parents, w.draft_ids, 50, 0.85)
    oa, op, ot = orc.greedy_accept(t, w.draft_ids, w.parents)
    phys, table = to_paged(w, ps, rng)
    opool = w.pool.copy()
    opl, osrc = orc.compact_kv(opool[:, :dl], opool[:, dl:], w.kv_base, w.prefix_len, op, oa)

    pd, td = to_dev(phys), to_dev(table)
    dpl = to_dev(w.prefix_len)
    npl = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    acc, path, tok = ddt.accept_compact(to_dev(t), to_dev(w.draft_ids), to_dev(w.parents), pd[:, :dl], pd[:, dl:],
                                        None, dpl, src_slot=src, new_prefix_len=npl, pages=(td, ps))
    torch.cuda.synchronize()
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(npl) == opl).all() and (to_host(src) == osrc).all()
    assert (to_host(dpl) == w.prefix_len).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    assert (from_paged(got_phys, table, ps, w).view(np.uint8) == opool.view(np.uint8)).all()
    named = np.zeros(got_phys.shape[0], bool)
    for b in range(B):
        tt = np.arange(int(w.prefix_len[b]) + N)
        named[table[b, tt // ps].astype(np.int64) * ps + tt % ps] = True
    assert (got_phys[~named].view(np.uint8) == phys[~named].view(np.uint8)).all()


def test_paged_accept_compact_unmappable_left_untouched(orc):
    """ddt_accept_compact_paged with committed lengths whose accepted slots
    run past the request's table row: those requests still get their
    acceptance outputs, with new length = old length, src_slot -1 and no
    row written; the others are compacted as the oracle does."""
    w = synth.workload(3, B=3, N=8, prefix_range=(40, 90))
    ps, B, N, dl = 32, 3, 8, 512
    rng = np.random.default_rng(13)
    w.draft_ids = w.draft_ids % 20
    t = synth.planted_targets(rng, w.parents, w.draft_ids, 20, 0.9)
    oa, op, ot = orc.greedy_accept(t, w.draft_ids, w.parents)
    phys, table = to_paged(w, ps, rng, spare=2)
    spare = _spare_page(table, w, ps, phys.shape[0] // ps)
    L = table.shape[1]
    P_dev = w.prefix_len.copy()
    P_dev[1] = L * ps - 1                               # the path's slots run past row 1 (unless only the root)
    P_dev[2] = L * ps + 5                               # past the table itself
    mappable = [0] + [b for b in (1, 2) if int(P_dev[b]) + int(op[b, oa[b]]) < L * ps]
    opool = w.pool.copy()
    opl, osrc = _oracle_compact_some(orc, opool, dl, w.kv_base, w.prefix_len, op, oa, [0])
    opl[1:], osrc[1:] = P_dev[1:], -1
    pd = to_dev(phys)
    _, td = _padded_table(table, 2, spare)
    npl = torch.empty((B,), dtype=torch.int32, device="cuda")
    src = torch.empty((B, N), dtype=torch.int32, device="cuda")
    acc, path, tok = ddt.accept_compact(to_dev(t), to_dev(w.draft_ids), to_dev(w.parents), pd[:, :dl], pd[:, dl:],
                                        None, to_dev(P_dev), src_slot=src, new_prefix_len=npl, pages=(td, ps))
    torch.cuda.synchronize()
    assert mappable == [0], mappable                   # the case exercises two unmappable requests
    assert (to_host(acc) == oa).all() and (to_host(path) == op).all() and (to_host(tok) == ot).all()
    assert (to_host(npl) == opl).all() and (to_host(src) == osrc).all()
    got_phys = np.ascontiguousarray(to_host(pd))
    assert (from_paged(got_phys, table, ps, w).view(np.uint8) == opool.view(np.uint8)).all()
    sp = slice(spare * ps, (spare + 1) * ps)
    assert (got_phys[sp].view(np.uint8) == phys[sp].view(np.uint8)).all()
