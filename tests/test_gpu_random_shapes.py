"""Seeded random shapes through the verify attention, against the oracle.

Each case draws a batch (1-24 requests), a head count that need not fill a
64-row tile (1, 2, 3, 5, 8 or 16), a tree size (1-128 nodes, random
parents), ragged prefix lengths (0-6000), a key chunk (automatic or forced
to a few tiles), and, for some cases, a paged cache (pages of 32 or 128
rows in random order, unused pool rows NaN) and device-resident lengths
below the host bounds.  The work plan (ddt_verify_plan) of every case must
cover each (request, split, row tile) once, and the outputs must meet the
bf16 bars on every row (all rows when the case is small, a seeded sample
otherwise)."""
import numpy as np
import pytest

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, check_attn, oracle_attn, to_dev, to_host

pytestmark = pytest.mark.gpu


def paged_copy(w, ps, rng):
    T = w.prefix_len.astype(np.int64) + w.N
    npg = (T + ps - 1) // ps
    total = int(npg.sum()) + 2
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((w.B, int(npg.max())), np.int32)
    phys = np.full((total * ps, w.pool.shape[1]), synth.BF16_NAN, dtype=w.pool.dtype)
    k = 0
    for b in range(w.B):
        table[b, : npg[b]] = perm[k: k + npg[b]]
        k += npg[b]
        t = np.arange(T[b])
        phys[table[b, t // ps].astype(np.int64) * ps + t % ps] = w.pool[w.kv_base[b] + t]
    return phys, table


@pytest.mark.parametrize("seed", range(24))
def test_random_shape(orc, seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 25))
    H = int(rng.choice([1, 2, 3, 5, 8, 16]))
    N = int(rng.choice([1, 2, 7, 31, 33, 64, 100, 128]))
    lo = int(rng.integers(0, 3000))
    hi = lo + int(rng.integers(1, 3000))
    kv_chunk = int(rng.choice([0, 0, 32, 96, 1000]))
    ps = int(rng.choice([0, 0, 32, 128]))
    device_lengths = bool(rng.integers(0, 2))
    w = synth.workload(3, seed=7000 + seed, B=B, H=H, N=N, prefix_range=(lo, hi))
    what = f"B={B} H={H} N={N} prefix=[{lo},{hi}) kv_chunk={kv_chunk} pages={ps} device_lengths={device_lengths}"
    print(what, flush=True)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    dl = w.d_lat
    bound = w.prefix_len.astype(np.int64) + (int(rng.integers(0, 200)) if device_lengths else 0)
    kw = dict(H=H, scale=w.scale, kv_chunk=kv_chunk, prefix_len_dev=dw.prefix_dev if device_lengths else None)
    if ps:
        phys, table = paged_copy(w, ps, rng)
        if device_lengths:  # the table row must cover the bounds
            need = int(((bound + N + ps - 1) // ps).max())
            table = np.pad(table, ((0, 0), (0, max(0, need - table.shape[1]))), constant_values=int(table.max()))
        pd, td = to_dev(phys), to_dev(table)
        ckv, kpe, kv_base, pages = pd[:, :dl], pd[:, dl:], None, (td, ps)
    else:
        ckv, kpe, kv_base, pages = dw.ckv(), dw.kpe(), dw.kv_base, None
    desc = ddt.attn_desc(dw.q_lat(), dw.q_pe(), ckv, kpe, B=B, H=H, N=N, scale=w.scale, kv_chunk=kv_chunk,
                         pages=pages)
    nb, chunk, nsplit, items = ddt.verify_plan(desc, bound)
    rt_n = -(-H * N // 64)
    got = {(int(b), int(s), int(r)) for _, b, s, r, _, _ in items}
    assert len(got) == len(items) == int(nsplit.sum()) * rt_n, what
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), ckv, kpe, kv_base, bound, mask, pages=pages, **kw)
    rows = None if w.rows * int(w.keys().sum()) < 4e7 else np.sort(rng.choice(w.rows, 256, replace=False))
    ref_out, ref_lse = oracle_attn(orc, w, rows=rows)
    o, l = to_host(out), to_host(lse)
    if rows is not None:
        o, l = o[rows], l[rows]
    check_attn(o, l, ref_out, ref_lse, "bf16", what)
