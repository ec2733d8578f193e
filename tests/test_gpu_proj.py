"""GPU parity of the per-head projections around the absorbed attention
(ddt_proj_pack_weight + ddt_head_proj) against the fp64 oracle, and of the
whole chain q_nope -> q_lat -> tree-verify attention -> o against the
oracle's chain.

Shapes whose 64-row x 128-column grid would leave CUs idle run the
split-reduction variant (small M), the others the row-tile variant; both
are covered.  Bar: rel-L2 <= 1e-2 over the output (bf16 inputs, fp32 accumulation), and
per element |y - ref| <= 2^-8 |ref| + 2^-16 sum_k |x_k W_kn| (the bf16
rounding of the result plus the fp32 summation)."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt, synth
from tests.helpers import ATTN_TOL, as_f64, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu
TOL = ATTN_TOL["bf16"]


def _weights(rng, H, K, n_out):
    return synth.to_bf16_bits((rng.standard_normal((H, K, n_out)) / np.sqrt(K)).astype(np.float32))


def _check(orc, x_bits, w_bits, y_bits):
    ref = orc.head_proj(x_bits, w_bits)
    bound = orc.head_proj(np.abs(as_f64(x_bits)), np.abs(as_f64(w_bits)))
    y = as_f64(y_bits)
    assert rel_l2(y, ref) <= TOL, rel_l2(y, ref)
    err = np.abs(y - ref)
    lim = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * bound
    assert (err <= lim).all(), float((err - lim).max())


@pytest.mark.parametrize("M,H,K,n_out", [
    (64, 8, 128, 512),     # q_nope -> q_lat, the K2-like head share (64 tree nodes)
    (2048, 8, 128, 512),   # 32 requests x 64 nodes
    (64, 8, 512, 128),     # out_lat -> o
    (2048, 8, 512, 128),
    (512, 64, 128, 512),   # all 64 heads, 4 requests x 128 nodes
    (1, 8, 128, 512),      # one token
    (100, 3, 64, 96),      # ragged token tile, a column block of 96
    (70, 2, 256, 32),      # one 32-column tile
    (6000, 3, 64, 96),     # enough rows for the 128-column workgroups, with a partial column block
    (0, 8, 128, 512),      # nothing to do
])
def test_head_proj(orc, M, H, K, n_out):
    rng = np.random.default_rng(M * 7 + H * 3 + K + n_out)
    x = synth.normal(rng, (M * H, K), "bf16")
    w = _weights(rng, H, K, n_out)
    wp = ddt.proj_pack_weight(to_dev(w))
    y = ddt.head_proj(to_dev(x), wp, H)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M * H, n_out)
    if M:
        _check(orc, x, w, to_host(y))


def test_head_proj_strided_into_query_rows(orc):
    """x is a column range of wider rows; y is written into the first 512
    columns of 576-wide q_lat|q_pe rows, leaving the q_pe columns and
    every other byte as they were."""
    rng = np.random.default_rng(5)
    M, H, K, n_out, wide = 37, 8, 128, 512, 576
    xw = synth.normal(rng, (M * H, K + 64), "bf16")
    w = _weights(rng, H, K, n_out)
    q = synth.normal(rng, (M * H, wide), "bf16")
    xd, qd = to_dev(xw), to_dev(q)
    wp = ddt.proj_pack_weight(to_dev(w))
    ddt.head_proj(xd[:, 32:32 + K], wp, H, y=qd[:, :n_out])
    torch.cuda.synchronize()
    qh = to_host(qd)
    assert (qh[:, n_out:] == q[:, n_out:]).all()
    _check(orc, xw[:, 32:32 + K], w, qh[:, :n_out])


def test_head_proj_argument_errors():
    dev = torch.device("cuda")
    x = torch.zeros((16, 128), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((2, 128, 512), dtype=torch.bfloat16, device=dev)
    wp = ddt.proj_pack_weight(w)
    with pytest.raises(ddt.DdtError):      # K not built in
        ddt.proj_pack_weight(torch.zeros((2, 96, 512), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ddt.DdtError):      # n_out not a multiple of 32
        ddt.proj_pack_weight(torch.zeros((2, 128, 500), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ddt.DdtError):      # row stride not a multiple of 8 elements
        big = torch.zeros((16 * 131,), dtype=torch.bfloat16, device=dev)
        ddt.head_proj(big.as_strided((16, 128), (131, 1)), wp, 2)
    L = ddt.lib()
    rc = L.ddt_head_proj(x.data_ptr(), 128, wp.data_ptr(), 8, 2, 128, 512, ddt.DDT_BF16, None, 512, None)
    assert rc == ddt.DDT_EINVAL                                  # null output
    y = torch.empty((16, 512), dtype=torch.bfloat16, device=dev)
    rc = L.ddt_head_proj(x.data_ptr(), 128, wp.data_ptr(), 8, 2, 128, 512, ddt.DDT_F32, y.data_ptr(), 512, None)
    assert rc == ddt.DDT_EUNSUPPORTED                            # fp32: not built in


def test_absorbed_chain_on_gpu(orc):
    """q_lat = q_nope @ w_kc[h] written into the query rows, the verify
    attention, then o = out_lat @ w_vc[h], all on the GPU, against the
    oracle's chain (projection, attention, projection in fp64)."""
    rng = np.random.default_rng(77)
    w = synth.workload(2, B=2, N=16, prefix=300, vocab=4096)
    H, N, B, dl = w.H, w.N, w.B, w.d_lat
    dn, dv = 128, 128
    q_nope = synth.normal(rng, (B * N * H, dn), "bf16")
    w_kc = _weights(rng, H, dn, dl)
    w_vc = _weights(rng, H, dl, dv)

    q = to_dev(w.q)                                    # q_pe columns from the workload
    ddt.head_proj(to_dev(q_nope), ddt.proj_pack_weight(to_dev(w_kc)), H, y=q[:, :dl])
    pool = to_dev(w.pool)
    mask, _, _ = ddt.build_mask(to_dev(w.parents))
    out, lse = ddt.verify_attn(q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:], to_dev(w.kv_base), w.prefix_len,
                               mask, H=H, scale=w.scale)
    o = ddt.head_proj(out, ddt.proj_pack_weight(to_dev(w_vc)), H)
    torch.cuda.synchronize()

    q_lat_ref = orc.head_proj(q_nope, w_kc)
    out_ref, lse_ref = _oracle_attn_f64_q(orc, w, q_lat_ref)
    o_ref = orc.head_proj(out_ref, w_vc)
    assert rel_l2(as_f64(to_host(o)), o_ref) <= TOL
    assert rel_l2(to_host(lse).astype(np.float64), lse_ref) <= TOL


def _oracle_attn_f64_q(orc, w, q_lat_ref):
    """The oracle's attention on fp64 projected queries: the verify oracle
    takes fp32/bf16 inputs, so the queries go in as fp32 (a relative change
    of 2^-24, far below the bf16 bar) and the cache as its bf16 values
    widened to fp32 exactly."""
    q_lat = q_lat_ref.astype(np.float32)
    q_pe = synth.bf16_bits_to_f32(w.q_pe())
    ckv = synth.bf16_bits_to_f32(np.ascontiguousarray(w.ckv()))
    kpe = synth.bf16_bits_to_f32(np.ascontiguousarray(w.kpe()))
    return orc.verify_attn(q_lat, np.ascontiguousarray(q_pe), ckv, kpe, w.kv_base, w.prefix_len, w.parents,
                           H=w.H, scale=w.scale)
