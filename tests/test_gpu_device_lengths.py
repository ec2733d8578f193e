"""Device-resident committed lengths (ddt_attn_desc.prefix_len_dev): the
attention is planned for host upper bounds of the lengths and reads each
request's actual length from device memory when it runs.  Every pool row
past a request's actual keys holds NaN (and so does every page past them),
so a read past them shows in the outputs; the results are checked against
the oracle on the actual lengths.  A graph of three consecutive verify
steps, with the host holding only bounds that grow by N per step, must
reproduce three eager steps run with exact lengths."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, check_attn, oracle_attn, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("extra,kv_chunk", [
    (0, 0),        # bounds equal to the lengths
    (64, 0),       # one step of growth
    (3000, 256),   # whole key splits past every request's keys (empty partials)
    (5000, 0),     # a plan made for much longer requests
])
def test_verify_attn_device_lengths(orc, extra, kv_chunk):
    w = synth.workload(3, B=4, N=32, prefix_range=(300, 4000), extra_rows=extra)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    bound = w.prefix_len.astype(np.int64) + extra
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, bound, mask, H=w.H,
                               scale=w.scale, kv_chunk=kv_chunk, prefix_len_dev=dw.prefix_dev)
    ref_out, ref_lse = oracle_attn(orc, w)
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16", f"extra {extra}")


def test_verify_attn_device_lengths_fp32(orc):
    """The fp32 instance (MFMA 32x32x2 f32, the tiny configuration's
    shapes) reads device lengths the same way."""
    w = synth.workload(1, B=3, prefix_range=(10, 300), extra_rows=500)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    bound = w.prefix_len.astype(np.int64) + 400
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, bound, mask, H=w.H,
                               scale=w.scale, kv_chunk=64, prefix_len_dev=dw.prefix_dev)
    ref_out, ref_lse = oracle_attn(orc, w)
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "f32")


def test_verify_attn_device_lengths_clamped(orc):
    """A device length above its bound is taken as the bound; a negative
    one as 0 (the request then sees its N tree keys only)."""
    w = synth.workload(3, B=4, N=32, prefix_range=(300, 2000), extra_rows=200)
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    bound = w.prefix_len.copy()
    bound[3] = 0                                          # request 3: bound 0 ...
    dev_len = w.prefix_len.astype(np.int32).copy()
    dev_len[1] += 150                                     # ... request 1 asks past its bound
    dev_len[2] = -7
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, bound, mask, H=w.H,
                               scale=w.scale, kv_chunk=256, prefix_len_dev=to_dev(dev_len))
    ref = synth.Workload(**{**w.__dict__})
    ref.prefix_len = np.minimum(np.maximum(dev_len, 0), bound).astype(w.prefix_len.dtype)
    ref_out, ref_lse = oracle_attn(orc, ref)
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16")


@pytest.mark.parametrize("ps,extra,prefix_range,kv_chunk", [
    (64, 1000, (200, 3000), 512),
    (32, 3000, (4000, 9000), 1 << 20),   # one split of up to 375 pages: the page-window ring wraps
])
def test_paged_verify_attn_device_lengths(orc, ps, extra, prefix_range, kv_chunk):
    """Pages past each request's keys (inside its table row for the
    bounds) are NaN pages: none of them may be read."""
    w = synth.workload(3, B=3, N=32, prefix_range=prefix_range)
    rng = np.random.default_rng(5)
    T = w.prefix_len.astype(np.int64) + w.N
    bound = w.prefix_len.astype(np.int64) + extra
    npg, npg_b = (T + ps - 1) // ps, (bound + w.N + ps - 1) // ps
    nan_pages = 4
    total = int(npg.sum()) + nan_pages
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((w.B, int(npg_b.max())), np.int32)
    phys = np.full((total * ps, w.pool.shape[1]), synth.BF16_NAN, dtype=w.pool.dtype)
    k = 0
    for b in range(w.B):
        table[b, : npg[b]] = perm[k: k + npg[b]]
        k += npg[b]
        table[b, npg[b]:] = perm[total - 1 - (np.arange(table.shape[1] - npg[b]) % nan_pages)]
        t = np.arange(T[b])
        phys[table[b, t // ps].astype(np.int64) * ps + t % ps] = w.pool[w.kv_base[b] + t]
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    pd, td = to_dev(phys), to_dev(table)
    dl = w.d_lat
    out, lse = ddt.verify_attn(dw.q_lat(), dw.q_pe(), pd[:, :dl], pd[:, dl:], None, bound, mask, H=w.H,
                               scale=w.scale, pages=(td, ps), kv_chunk=kv_chunk, prefix_len_dev=dw.prefix_dev)
    ref_out, ref_lse = oracle_attn(orc, w)
    check_attn(to_host(out), to_host(lse), ref_out, ref_lse, "bf16")


def test_verify_steps_device_lengths_graph():
    """Three verify steps captured in one graph with device lengths (host
    bounds P0 + s*N) equal three eager steps with exact host lengths:
    acceptance, tokens, lengths and the compacted cache bit for bit, the
    attention to the bf16 bar.  Before each step its tree's latents go to
    slots P..P+N-1 at the device lengths (a torch scatter, captured too)."""
    B, H, N, steps, V = 4, 8, 16, 3, 4096
    w = synth.workload(3, B=B, H=H, N=N, prefix_range=(200, 1500), extra_rows=steps * N)
    rng = np.random.default_rng(17)
    dl = w.d_lat
    dev = torch.device("cuda")
    kvb = to_dev(w.kv_base)
    qs, pars, drafts, logs, lats = [], [], [], [], []
    for s in range(steps):
        parents = synth.random_parents(rng, B, N)
        draft = rng.integers(0, V, size=(B, N)).astype(np.int32)
        target = synth.planted_targets(rng, parents, draft, V, 0.7)
        qs.append(to_dev(synth.normal(rng, (B * N * H, w.q.shape[1]), "bf16")))
        lats.append(to_dev(synth.normal(rng, (B * N, w.pool.shape[1]), "bf16")))
        pars.append(to_dev(parents))
        drafts.append(to_dev(draft))
        logs.append(to_dev(synth.target_logits(rng, target.reshape(-1), V)))
    pool0 = to_dev(w.pool)
    bound_last = w.prefix_len.astype(np.int64) + (steps - 1) * N
    desc = ddt.attn_desc(qs[0][:, :dl], qs[0][:, dl:], pool0[:, :dl], pool0[:, dl:], B=B, H=H, N=N, scale=w.scale,
                         kv_chunk=256)
    ws = torch.empty((max(1, ddt.verify_workspace_bytes(desc, bound_last)),), dtype=torch.uint8, device=dev)
    am_ws = torch.zeros((max(16, ddt.argmax_workspace_bytes(B * N, V)),), dtype=torch.uint8, device=dev)

    node = torch.arange(N, dtype=torch.int64, device=dev)

    def place_nodes(pool, prefix, s):
        rows = (kvb + prefix.long()).unsqueeze(1) + node  # slots P_b .. P_b + N - 1
        pool.index_copy_(0, rows.reshape(-1), lats[s])

    def outputs():
        return [dict(out=torch.empty((B * N * H, dl), dtype=torch.bfloat16, device=dev),
                     lse=torch.empty((B * N * H,), dtype=torch.float32, device=dev),
                     idx=torch.empty((B * N,), dtype=torch.int32, device=dev),
                     accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                     path=torch.empty((B, N), dtype=torch.int32, device=dev),
                     tokens=torch.empty((B, N), dtype=torch.int32, device=dev)) for _ in range(steps)]

    # eager, exact host lengths read back after every step
    pool = pool0.clone()
    prefix = to_dev(w.prefix_len)
    ref = outputs()
    P = w.prefix_len.copy()
    for s in range(steps):
        place_nodes(pool, prefix, s)
        ddt.verify_step(qs[s][:, :dl], qs[s][:, dl:], pool[:, :dl], pool[:, dl:], kvb, P, None, logs[s], drafts[s],
                        pars[s], prefix, H=H, scale=w.scale, workspace=ws, argmax_workspace=am_ws, kv_chunk=256,
                        **ref[s])
        P = to_host(prefix).astype(w.prefix_len.dtype)
    ref_pool, ref_prefix = pool.clone(), prefix.clone()
    assert int(ref_prefix.sum()) > int(w.prefix_len.sum()) + B * steps  # some drafts accepted

    # captured: the host knows only bounds
    pool.copy_(pool0)
    prefix.copy_(to_dev(w.prefix_len))
    got = outputs()

    def run():
        for s in range(steps):
            bound = w.prefix_len.astype(np.int64) + s * N
            place_nodes(pool, prefix, s)
            ddt.verify_step(qs[s][:, :dl], qs[s][:, dl:], pool[:, :dl], pool[:, dl:], kvb, bound, None, logs[s],
                            drafts[s], pars[s], prefix, H=H, scale=w.scale, workspace=ws, argmax_workspace=am_ws,
                            kv_chunk=256, device_lengths=True, **got[s])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(2):
        pool.copy_(pool0)
        prefix.copy_(to_dev(w.prefix_len))
        for o in got:
            for v in o.values():
                v.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for s in range(steps):
            for k in ("idx", "accept_len", "path", "tokens"):
                assert torch.equal(got[s][k], ref[s][k]), (rep, s, k)
            a, r = got[s]["out"].float(), ref[s]["out"].float()
            assert torch.isfinite(a).all()
            assert float((a - r).norm() / r.norm()) < 5e-3, (rep, s)
            assert float((got[s]["lse"] - ref[s]["lse"]).abs().max()) < 1e-3, (rep, s)
        assert torch.equal(prefix, ref_prefix), rep
        assert torch.equal(pool.view(torch.int16), ref_pool.view(torch.int16)), rep
