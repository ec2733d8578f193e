"""The split-KV work plan of the verify attention, on the host
(ddt_verify_plan: no device work).  Each request's keys [0, P_b + N) are cut
into splits of `chunk` keys and each split into row tiles of 64 query rows;
the launch's workgroups must cover every (request, split, row tile) exactly
once (a duplicate would add a partial twice in the merge, a gap would drop
keys), with only padding workgroups left over.  The checks also pin the
dispatch properties the kernel relies on for speed: row tiles of one split
dealt to one XCD together, XCD loads within a unit of each other, a
one-round launch giving each XCD a contiguous run of items, large trees
dealt last row tile first, and a paged cache planned exactly like a
contiguous one."""
import math

import numpy as np
import pytest

from mla_tree_verify_parents_amd import ddt

KT, XCDS, UNIT = 32, 8, 8


def desc(B, H, N, kv_chunk=0, paged=0):
    d = ddt.AttnDesc(B, H, N, 512, 64, ddt.DDT_BF16, 0.04, kv_chunk, 576, 576, 576, 576)
    if paged:
        d.block_table, d.bt_ld, d.page_size = 1 << 20, 1 << 20, paged  # host checks only: never dereferenced
    return d


def check_plan(B, H, N, P, kv_chunk=0):
    d = desc(B, H, N, kv_chunk)
    nb, chunk, nsplit, items = ddt.verify_plan(d, P)
    T = P.astype(np.int64) + N
    rt_n = math.ceil(H * N / 64)
    assert chunk > 0 and chunk % KT == 0
    if kv_chunk > 0:
        assert chunk == math.ceil(kv_chunk / KT) * KT
    blk, b, s, r, k0, k1 = (items[:, i].astype(np.int64) for i in range(6))
    assert ((blk >= 0) & (blk < nb)).all() and ((b >= 0) & (b < B)).all() and ((r >= 0) & (r < rt_n)).all()
    assert ((s >= 0) & (s < nsplit[b])).all()
    # every (request, split, row tile) exactly once: item k of the
    # (request, split, row tile) order is row tile r of split s of request b
    first = np.concatenate([[0], np.cumsum(nsplit.astype(np.int64) * rt_n)])
    key = first[b] + s * rt_n + r
    assert len(key) == first[-1] and (np.sort(key) == np.arange(first[-1])).all()
    # the splits of a request cut its keys [0, T_b) into consecutive,
    # non-empty, tile-aligned ranges in split order
    o = np.argsort(key)
    kb, ke, bb, ss = k0[o], k1[o], b[o], s[o]
    assert (kb % KT == 0).all() and (ke > kb).all()
    assert (kb[ss == 0] == 0).all()
    nxt = (bb[rt_n:] == bb[:-rt_n]) if len(kb) > rt_n else np.zeros(0, bool)
    assert (kb[rt_n:][nxt] == ke[:-rt_n][nxt]).all()
    last = ss == nsplit[bb] - 1
    assert (ke[last] == T[bb[last]]).all()
    assert len(blk) == len(np.unique(blk))                            # one work item per workgroup
    assert (k0 == s * chunk).all() and (k1 == np.minimum((s + 1) * chunk, T[b])).all()
    n = len(key)
    xcd = blk % XCDS
    if n <= 256:
        # one round: XCD x runs a contiguous range of items in (request, split, row tile) order
        for x in range(XCDS):
            ks = np.sort(key[xcd == x])
            assert len(ks) == 0 or (ks == np.arange(ks[0], ks[0] + len(ks))).all()
    else:
        counts = np.bincount(xcd, minlength=XCDS)
        assert counts.max() - counts.min() <= 2 * UNIT
        # a unit (up to 8 row tiles of one split) shares one XCD's L2; at most
        # the last n_units % 8 units are dealt row tile by row tile
        unit_rows = min(UNIT, rt_n)
        rr = r if N <= 128 else rt_n - 1 - r          # large trees: the split's row tiles go last first
        grp = first[b] // rt_n + s
        unit = grp * rt_n + rr // unit_rows
        spread = {}
        for u, x in zip(unit.tolist(), xcd.tolist()):
            spread.setdefault(u, set()).add(x)
        assert sum(len(v) > 1 for v in spread.values()) < XCDS
        # within a split, row tiles are dealt in that order: a later one never
        # starts in an earlier round of the deal (longest work items first for
        # large trees, whose later rows see more keys)
        pos = blk // XCDS // unit_rows
        o = np.lexsort((rr, grp))
        g, p = grp[o], pos[o]
        same = g[1:] == g[:-1]
        assert (p[1:][same] >= p[:-1][same]).all()
    return nb, chunk, nsplit, items


@pytest.mark.parametrize("seed", range(60))
def test_plan_covers_every_item_once(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 3, 4, 7, 16, 32, 64, 128]))
    H = int(rng.choice([1, 2, 8, 16, 64]))
    N = int(rng.choice([1, 8, 31, 64, 128, 300, 1024]))
    while H * N > 8192 or (B > 16 and H * N > 1024):
        H //= 2
    H = max(H, 1)
    hi = int(rng.choice([64, 4096, 40000, 140000]))
    P = rng.integers(0, hi, B).astype(np.int32)
    kv_chunk = int(rng.choice([0, 0, 0, 32, 100, 4096, 1 << 20]))
    check_plan(B, H, N, P, kv_chunk)


@pytest.mark.parametrize("B,H,N,P,kv_chunk", [
    (1, 8, 64, [4096], 0),                              # the K2-like head share
    (4, 64, 128, [131072] * 4, 0),                      # long context, all heads
    (16, 8, 32, list(range(1024, 32769, 2048)), 0),     # batched ragged
    (32, 8, 64, list(range(2048, 65537, 2048)), 0),     # the verify loop's batch
    (8, 8, 1024, [1024 * c for c in range(8)], 0),      # an 8192-token prompt in 1024-token chunks
    (1, 1, 1, [0], 0),                                  # one row, one key
    (128, 2, 3, [0] * 128, 0),                          # many tiny requests
    (3, 8, 64, [10, 5000, 70000], 32),                  # one tile per split
])
def test_plan_named_shapes(B, H, N, P, kv_chunk):
    check_plan(B, H, N, np.array(P, np.int32), kv_chunk)


def test_plan_single_split_for_equal_long_requests():
    """Four equal 131 k-key requests with 128 row tiles each fill the CUs in
    two rounds without splitting: no partial outputs and no merge."""
    nb, chunk, nsplit, items = check_plan(4, 64, 128, np.full(4, 131072, np.int32))
    assert (nsplit == 1).all() and nb == 512


def test_paged_plan_equals_contiguous():
    rng = np.random.default_rng(7)
    for _ in range(10):
        B = int(rng.integers(1, 40))
        P = rng.integers(0, 100000, B).astype(np.int32)
        a = ddt.verify_plan(desc(B, 8, 64), P)
        b = ddt.verify_plan(desc(B, 8, 64, paged=64), P)
        assert a[:2] == b[:2] and (a[2] == b[2]).all() and (a[3] == b[3]).all()


def test_plan_validation():
    P = np.array([100, 200], np.int32)
    with pytest.raises(ValueError):
        ddt.verify_plan(desc(2, 8, 64), np.array([100], np.int32))        # one length for two requests
    with pytest.raises(ValueError):
        ddt.verify_plan(desc(2, 8, 64), np.array([100, 1 << 33], np.int64))  # past int32
    with pytest.raises(ddt.DdtError):
        ddt.verify_plan(desc(2, 8, 2000), P)            # more nodes than the limit
    with pytest.raises(ddt.DdtError):
        ddt.verify_plan(desc(2, 8, 64), np.array([100, -1], np.int32))
