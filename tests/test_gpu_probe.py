"""The roofline probes (include/ddt_probe.h) compute what they claim, so the
rates bench.py derives from them count real work: the MFMA loop's folded
sums against a closed form on small-integer operands (exact in fp32), the
streaming read's XOR fold and the streaming copy's bytes."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt

pytestmark = pytest.mark.gpu


def test_mfma_probe_sums():
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    vals = rng.integers(-2, 3, size=ddt.PROBE_MFMA_OPERANDS).astype(np.float32)
    ops = torch.from_numpy(vals).to(dev).to(torch.bfloat16)
    blocks, iters = 3, 5
    sink, clk = ddt.probe_mfma_bf16(ops, blocks, iters)
    torch.cuda.synchronize()
    # fragment k of A (B) for lane l holds k-values 8*(l // 32) .. +7 of row
    # (column) l % 32; the sum of all 32x32 products of A_k B_m is then
    # sum over the two k-halves h and e of colsum(A_k)[h, e] * rowsum(B_m)[h, e]
    a = vals[: 4 * 512].reshape(4, 2, 32, 8)   # [frag, half, row, e]
    b = vals[4 * 512:].reshape(4, 2, 32, 8)
    sa, sb = a.sum(axis=2), b.sum(axis=2)      # [frag, half, e]
    per_wave = sum(float((sa[k] * sb[(k + c) % 4]).sum()) for k in range(4) for c in range(4)) * iters
    got = sink.cpu().numpy().astype(np.float64).sum()
    assert got == per_wave * blocks * 4
    c = clk.cpu().numpy()
    assert (c > 0).all()


def test_read_and_copy_probes():
    dev = torch.device("cuda:0")
    n = (1 << 20) + 48  # not a multiple of the grid stride: exercises the tail
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=dev, generator=g)
    blocks = 7
    sink = ddt.probe_read(src, blocks)
    torch.cuda.synchronize()
    fold = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert fold == want
    dst = torch.zeros_like(src)
    ddt.probe_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
