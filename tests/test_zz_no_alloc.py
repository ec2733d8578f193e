"""The allocation-free verify attention (ddt_verify_attn_noalloc) through
the C ABI against ddt_verify_attn: two calls in a row on one device, the
second with a smaller input, each bit-identical to ddt_verify_attn's
output on the same inputs (same plan, same kernels; the split partials
live in the library's scratch instead of a workspace) and within the
oracle's bar; a call whose partials exceed the scratch is refused."""
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import DevWorkload, check_attn, oracle_attn, to_host

pytestmark = pytest.mark.gpu


def _launch(dw, mask, kv_chunk, noalloc):
    w = dw.w
    out = torch.empty((w.rows, w.d_lat), dtype=dw.q.dtype, device="cuda")
    lse = torch.empty((w.rows,), dtype=torch.float32, device="cuda")
    args = (dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask)
    if noalloc:
        ddt.verify_attn_noalloc(*args, H=w.H, scale=w.scale, out=out, lse=lse, kv_chunk=kv_chunk)
    else:
        ddt.verify_attn(*args, H=w.H, scale=w.scale, out=out, lse=lse, kv_chunk=kv_chunk)
    return out, lse


def test_noalloc_equals_verify_attn_two_calls(orc):
    cases = [(synth.workload(2, with_logits=False), 256),                  # 17 splits x 8 row tiles
             (synth.workload(3, B=3, N=16, prefix_range=(300, 1200)), 96)]  # smaller, still split
    devs = []
    for w, ch in cases:
        dw = DevWorkload(w)
        mask = ddt.build_mask(dw.parents)[0]
        d = ddt.attn_desc(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), B=w.B, H=w.H, N=w.N, scale=w.scale,
                          kv_chunk=ch)
        need = ddt.verify_workspace_bytes(d, w.prefix_len)
        assert 0 < need <= ddt.noalloc_scratch_bytes(), need      # the partials go through the scratch
        devs.append((w, dw, mask, ch, need))
    refs = [_launch(dw, mask, ch, False) for w, dw, mask, ch, _ in devs]
    torch.cuda.synchronize()
    # the two allocation-free calls back to back: the second, smaller one
    # runs on the scratch the first left behind
    gots = [_launch(dw, mask, ch, True) for w, dw, mask, ch, _ in devs]
    torch.cuda.synchronize()
    for (w, dw, mask, ch, need), (ro, rl), (go, gl) in zip(devs, refs, gots):
        assert torch.equal(go.view(torch.int16), ro.view(torch.int16)), w.name
        assert torch.equal(gl, rl), w.name
        ref_out, ref_lse = oracle_attn(orc, w)
        e = check_attn(to_host(go), to_host(gl), ref_out, ref_lse, w.dtype, w.name)
        print(f"{w.name}: partials {need} bytes in the scratch; rel_l2 {e[0]:.2e}, max row {e[2]:.2e}")


def test_noalloc_refuses_partials_beyond_the_scratch():
    """A plan whose partials exceed the scratch is refused (DDT_EWORKSPACE)
    before anything is launched."""
    w = synth.workload(3, B=32, N=64, prefix_range=(1024, 1024))
    dw = DevWorkload(w)
    mask = ddt.build_mask(dw.parents)[0]
    d = ddt.attn_desc(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), B=w.B, H=w.H, N=w.N, scale=w.scale, kv_chunk=256)
    assert ddt.verify_workspace_bytes(d, w.prefix_len) > ddt.noalloc_scratch_bytes()
    out = torch.empty((w.rows, w.d_lat), dtype=dw.q.dtype, device="cuda")
    lse = torch.empty((w.rows,), dtype=torch.float32, device="cuda")
    with pytest.raises(ddt.DdtError, match="EWORKSPACE"):
        ddt.verify_attn_noalloc(dw.q_lat(), dw.q_pe(), dw.ckv(), dw.kpe(), dw.kv_base, w.prefix_len, mask,
                                H=w.H, scale=w.scale, out=out, lse=lse, kv_chunk=256)
