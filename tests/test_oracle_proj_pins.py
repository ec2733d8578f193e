"""Pins for the oracle's per-head projection (q_lat = q_nope @ W_UK[h],
o = out_lat @ W_UV[h]): permutation and rank-one weights with closed-form
results, and the chain projection -> absorbed attention -> projection
against explicit per-head MHA computed by torch's fp64 attention on
up-projected keys and values.  CPU only."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import synth
from test_oracle_pins import _f64, _sdpa_reference, _small_case, closure_ancestors


def test_proj_permutation_weights(orc):
    """W[h][k][n] = 1 iff n = pi_h(k) sends x[k] to column pi_h(k).  The
    permutations differ per head and are not involutions, so a transposed
    weight (pi_h^-1) or a wrong head index gives a different result."""
    rng = np.random.default_rng(21)
    M, H, K = 5, 3, 12
    perms = [rng.permutation(K) for _ in range(H)]
    for p in perms:
        assert (p[p] != np.arange(K)).any()
    W = np.zeros((H, K, K), np.float32)
    for h, p in enumerate(perms):
        W[h, np.arange(K), p] = 1.0
    x = rng.standard_normal((M * H, K)).astype(np.float32)
    y = orc.head_proj(x, W)
    for r in range(M * H):
        expect = np.empty(K)
        expect[perms[r % H]] = x[r]
        np.testing.assert_array_equal(y[r], expect)


def test_proj_rank_one_weights(orc):
    """W[h] = a_h b_h^T gives y[r] = (x[r] . a_h) b_h; x is a strided view
    of wider bf16 rows."""
    rng = np.random.default_rng(22)
    M, H, K, n_out = 7, 4, 32, 48
    a = rng.integers(-3, 4, size=(H, K)).astype(np.float64)
    b = rng.integers(-3, 4, size=(H, n_out)).astype(np.float64)
    W = np.einsum("hk,hn->hkn", a, b).astype(np.float32)       # small integers: exact
    wide = synth.to_bf16_bits(rng.integers(-4, 5, size=(M * H, K + 16)).astype(np.float32))
    x = wide[:, 8:8 + K]
    y = orc.head_proj(x, W)
    xf = _f64(x)
    for r in range(M * H):
        h = r % H
        np.testing.assert_array_equal(y[r], (xf[r] @ a[h]) * b[h])


def test_proj_rejects_bad_arguments(orc):
    with pytest.raises(AssertionError):
        orc.head_proj(np.zeros((6, 4), np.float32), np.zeros((4, 5, 3), np.float32))   # K mismatch
    with pytest.raises(AssertionError):
        orc.head_proj(np.zeros((7, 5), np.float32), np.zeros((2, 5, 3), np.float32))   # rows not M*H


def test_proj_absorbed_chain_equals_explicit_mha(orc):
    """q_lat = q_nope @ w_kc[h] (oracle projection), the oracle's absorbed
    tree-verify attention, then o = out_lat @ w_vc[h] (oracle projection)
    equals per-head MHA with keys [w_kc[h] c_kv | k_pe] and values
    c_kv @ w_vc[h], on the tree's visibility, from torch's fp64 attention.
    w_kc is [d_nope, d_lat] and w_vc [d_lat, d_v] ([in, out]); d_nope,
    d_lat and d_v all differ, so a transposed weight cannot pass.  Integer
    q_nope and w_kc keep q_lat exact in the fp32 attention input."""
    rng = np.random.default_rng(23)
    B, H, N, P, dl, dr, dn, dv = 1, 3, 7, 25, 64, 16, 24, 40
    par = np.array([[-1, 0, 1, 0, 3, 1, 5]], np.int32)
    pool, base, Ps, _, _ = _small_case(rng, B, H, N, P, dl, dr, parents=par)
    w_kc = rng.integers(-2, 3, size=(H, dn, dl)).astype(np.float32)
    w_vc = rng.standard_normal((H, dl, dv))
    q_nope = rng.integers(-2, 3, size=(N * H, dn)).astype(np.float32)
    q_pe = rng.standard_normal((N * H, dr)).astype(np.float32)
    q_lat = orc.head_proj(q_nope, w_kc)
    assert (q_lat == np.round(q_lat)).all() and np.abs(q_lat).max() < 2 ** 24
    q = np.concatenate([q_lat.astype(np.float32), q_pe], axis=1)
    scale = 0.01
    out_lat, lse = orc.verify_attn(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], base, Ps, par,
                                   H=H, scale=scale)
    o = orc.head_proj(out_lat, w_vc)

    T = P + N
    kv = _f64(pool[base[0]: base[0] + T])
    ckv, kpe = kv[:, :dl], kv[:, dl:]
    anc = closure_ancestors(par[0])
    for i in range(N):
        vis = np.concatenate([np.ones(P, bool), anc[i]])[None, :]
        for h in range(H):
            r = i * H + h
            k = np.concatenate([ckv @ w_kc[h].astype(np.float64).T, kpe], axis=1)     # [T, dn+dr]
            v = ckv @ w_vc[h]                                                          # [T, dv]
            qr = np.concatenate([q_nope[r].astype(np.float64), q_pe[r].astype(np.float64)])[None, :]
            ref = _sdpa_reference(qr, k, v, vis, scale)[0]
            np.testing.assert_allclose(o[r], ref, rtol=1e-10, atol=1e-12)
            s = torch.from_numpy(scale * (k[vis[0]] @ qr[0]))
            np.testing.assert_allclose(lse[r], torch.logsumexp(s, 0).item(), rtol=1e-12)
