"""Causal prefill through the verify attention, on the GPU.

A chain-shaped tree's ancestor mask is the causal mask, so a prompt is
prefilled in chunks of up to 1024 tokens, chunk c a request at committed
length P0 + c*chunk; the full chunks go into one batched verify-attention
call (mla_tree_verify_parents_amd.prefill).
The chunked result is compared with the oracle's attention over the whole
prompt as ONE chain (unchunked), on sampled rows that include every chunk's
first and last tokens; the bf16 bar (rel-L2 <= 1e-2 on out and lse).  The
mask builder is checked bit-exactly on chains and deep trees up to the
maximum node count."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from mla_tree_verify_parents_amd.prefill import ChunkedPrefill
from tests.helpers import as_f64, check_attn, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [65, 200, 1024])
def test_mask_chains_and_deep_trees(orc, N):
    rng = np.random.default_rng(N)
    par = synth.random_parents(rng, 6, N)
    par[0] = np.arange(-1, N - 1)                                            # chain: causal
    par[1, 1:] = 0                                                           # star
    for b in (2, 3):                                                         # deep: parent among the last 3
        par[b, 1:] = [rng.integers(max(0, i - 3), i) for i in range(1, N)]
    par[4, 1:] = np.arange(N - 1) // 2                                       # binary heap order
    m, d, e = ddt.build_mask(to_dev(par))
    om, od, oe = orc.build_mask(par)
    assert (to_host(m).view(np.uint64) == om).all()
    assert (to_host(d) == od).all() and (to_host(e) == oe).all()


def _prompt(seed, T, P0, H=8):
    rng = np.random.default_rng(seed)
    dl, dr = 512, 64
    pool, base, _ = synth.make_pool(rng, np.array([P0], np.int32), T, dl + dr, "bf16")
    q = synth.normal(rng, (T * H, dl + dr), "bf16")
    return pool, base, q, dl, dr, 1.0 / np.sqrt(dl + dr)


@pytest.mark.parametrize("T,P0,chunk", [
    (700, 50, 256),      # three chunks, a ragged last one
    (2100, 1500, 1024),  # full-size chunks over a committed prefix
    (64, 0, 1024),       # one chunk, empty prefix: plain causal attention
    (4096, 0, 1024),     # four full chunks in one call, nothing left over
    (200 * 32 + 5, 7, 32),  # more full chunks than one call takes (128), then a 5-token chunk
])
def test_chunked_prefill_equals_unchunked_oracle(orc, T, P0, chunk):
    H = 8
    pool, base, q, dl, dr, scale = _prompt(T + P0, T, P0, H)
    pd, qd = to_dev(pool), to_dev(q)
    pf = ChunkedPrefill(H, scale, chunk=chunk)
    out, lse = pf.run(qd[:, :dl], qd[:, dl:], pd[:, :dl], pd[:, dl:], to_dev(base), P0)
    torch.cuda.synchronize()

    rng = np.random.default_rng(T)
    toks = set(rng.choice(T, size=min(T, 24), replace=False).tolist())
    ch = pf.chunks(T, P0)
    for t0, n, _ in ch[:3] + ch[-3:]:                 # first and last tokens of the outer chunks
        toks |= {t0, t0 + n - 1}
    rows = np.array(sorted(t * H + h for t in toks for h in (0, H - 1)), np.int64)
    chain = np.arange(-1, T - 1, dtype=np.int32)[None]
    ref_out, ref_lse = orc.verify_attn(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], base,
                                       np.array([P0], np.int32), chain, H=H, scale=scale, rows=rows)
    o = as_f64(to_host(out))[rows]
    l_ = to_host(lse).astype(np.float64)[rows]
    check_attn(o, l_, ref_out, ref_lse, "bf16")
