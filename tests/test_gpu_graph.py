"""Graph replays of the fused verify step.  The benchmark times the step as
HIP graph replays, so every replay must give the eager result: the argmax
workspace clears itself after each call (no memset node is recorded), the
split partials are rewritten before they are read, and the lengths are read
from one array and written to another.  Between replays the program does
its own eager work (the cache is restored, outputs are poisoned); each
replay is compared with the eager step bit for bit (the kernels are
deterministic)."""
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("with_mask", [False, True])
def test_verify_step_graph_replays(with_mask):
    w = synth.workload(2, B=3, N=16, prefix=700, vocab=5000)
    dl, B, N, H = w.d_lat, w.B, w.N, w.H
    pool, q = to_dev(w.pool), to_dev(w.q)
    parents, draft, kvb = to_dev(w.parents), to_dev(w.draft_ids), to_dev(w.kv_base)
    prefix = to_dev(w.prefix_len)
    logits = to_dev(w.logits)
    dev = pool.device
    mask = ddt.build_mask(parents)[0] if with_mask else None
    am_ws = torch.zeros((max(16, ddt.argmax_workspace_bytes(B * N, w.vocab)),), dtype=torch.uint8, device=dev)
    desc = ddt.attn_desc(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], B=B, H=H, N=N, scale=w.scale,
                         kv_chunk=256)
    ws = torch.empty((max(1, ddt.verify_workspace_bytes(desc, w.prefix_len)),), dtype=torch.uint8, device=dev)
    outs = dict(out=torch.empty((B * N * H, dl), dtype=torch.bfloat16, device=dev),
                lse=torch.empty((B * N * H,), dtype=torch.float32, device=dev),
                idx=torch.empty((B * N,), dtype=torch.int32, device=dev),
                accept_len=torch.empty((B,), dtype=torch.int32, device=dev),
                path=torch.empty((B, N), dtype=torch.int32, device=dev),
                tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                new_prefix_len=torch.empty((B,), dtype=torch.int32, device=dev))

    def step():
        ddt.verify_step(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], kvb, w.prefix_len, mask, logits, draft,
                        parents, prefix, H=H, scale=w.scale, workspace=ws, argmax_workspace=am_ws, kv_chunk=256,
                        **outs)

    pool0 = pool.clone()
    step()                                   # eager
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref_pool = pool.clone()
    assert int(ref["accept_len"].max()) >= 1   # compaction moves rows

    pool.copy_(pool0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                               # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        pool.copy_(pool0)
        for v in outs.values():
            v.view(torch.uint8).fill_(0xA5)  # poison every output
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), ref[k].view(torch.uint8)), (rep, k)
        assert torch.equal(pool.view(torch.int16), ref_pool.view(torch.int16)), rep
        assert torch.equal(prefix.cpu(), torch.from_numpy(w.prefix_len)), rep
