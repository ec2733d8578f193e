"""The Python binding refuses tensors that are too small for what the
library reads or writes through them.  The C ABI takes bare pointers and
cannot check sizes, so these checks run before any launch (no kernel runs
in the refused calls)."""
import numpy as np
import pytest
import torch

from mla_tree_verify_parents_amd import ddt

pytestmark = pytest.mark.gpu

B, N, H = 3, 8, 2


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def chain_parents():
    return torch.tensor([[-1] + list(range(N - 1))] * B, dtype=torch.int32, device="cuda")


def test_acceptance_sizes():
    par, ok = chain_parents(), i32(B, N)
    with pytest.raises(ValueError, match="target_ids"):
        ddt.greedy_accept(i32(B * N - 1), ok, par)
    with pytest.raises(ValueError, match="draft_ids"):
        ddt.greedy_accept(ok, i32(B, N - 1), par)
    with pytest.raises(ValueError, match="accept_len"):
        ddt.greedy_accept(ok, ok, par, accept_len=i32(B - 1))
    with pytest.raises(ValueError, match="path"):
        ddt.greedy_accept(ok, ok, par, path=i32(B, N - 1))
    with pytest.raises(ValueError, match="tokens"):
        ddt.greedy_accept(ok, ok, par, tokens=i32(B * N))


def test_mask_sizes():
    par = chain_parents()
    with pytest.raises(ValueError, match="mask"):
        ddt.build_mask(par, mask=torch.zeros((B, N - 1, 1), dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError, match="depth"):
        ddt.build_mask(par, depth=i32(B, N - 1))
    with pytest.raises(ValueError, match="tree_err"):
        ddt.build_mask(par, tree_err=i32(B - 1))
    with pytest.raises(ValueError, match="parents"):
        ddt.build_mask(i32(B * N))


def test_compaction_sizes():
    pool = torch.zeros((200, 576), dtype=torch.bfloat16, device="cuda")
    ckv, kpe = pool[:, :512], pool[:, 512:]
    kvb = torch.zeros((B,), dtype=torch.int64, device="cuda")
    par, ok = chain_parents(), i32(B, N)
    acc, P = i32(B), i32(B)
    with pytest.raises(ValueError, match="prefix_len"):
        ddt.compact_kv(ckv, kpe, kvb, i32(B - 1), ok, acc)
    with pytest.raises(ValueError, match="accept_len"):
        ddt.compact_kv(ckv, kpe, kvb, P, ok, i32(B - 1))
    with pytest.raises(ValueError, match="kv_base"):
        ddt.compact_kv(ckv, kpe, kvb[:B - 1], P, ok, acc)
    with pytest.raises(ValueError, match="new_prefix_len"):
        ddt.accept_compact(ok, ok, par, ckv, kpe, kvb, P, new_prefix_len=i32(B - 1))
    with pytest.raises(ValueError, match="kv_base"):
        ddt.accept_compact(ok, ok, par, ckv, kpe, kvb[:1], P)
    with pytest.raises(ValueError, match="target_ids"):
        ddt.accept_compact(i32(B, N - 1), ok, par, ckv, kpe, kvb, P)


def test_attention_sizes():
    rows = B * N * H
    q = torch.zeros((rows, 576), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((400, 576), dtype=torch.bfloat16, device="cuda")
    kvb = torch.tensor([0, 100, 200], dtype=torch.int64, device="cuda")
    P = np.array([10, 20, 30], np.int32)
    mask = ddt.build_mask(chain_parents())[0]
    args = (q[:, :512], q[:, 512:], pool[:, :512], pool[:, 512:])
    scale = 1 / 24
    with pytest.raises(ValueError, match="out"):
        ddt.verify_attn(*args, kvb, P, mask, H=H, scale=scale,
                        out=torch.empty((rows - 1, 512), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="lse"):
        ddt.verify_attn(*args, kvb, P, mask, H=H, scale=scale,
                        lse=torch.empty((rows - 1,), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="kv_base"):
        ddt.verify_attn(*args, kvb[:2], P, mask, H=H, scale=scale)
    with pytest.raises(ValueError, match="mask"):
        ddt.verify_attn(*args, kvb, P, mask[:, :, :0], H=H, scale=scale)
    logits = torch.zeros((B * N, 1000), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="idx"):
        ddt.verify_attn_argmax(*args, kvb, P, mask, logits, H=H, scale=scale, idx=i32(B * N - 1))
    with pytest.raises(ValueError, match="prefix_len"):
        ddt.verify_step(*args, kvb, P, None, logits, i32(B, N), chain_parents(), i32(B - 1), H=H, scale=scale)


def test_scan_sizes():
    logits = torch.zeros((4, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="idx"):
        ddt.argmax(logits, idx=i32(3))
    with pytest.raises(ValueError, match="ids"):
        ddt.draft_topk(logits, 8, ids=i32(4, 7))
    ids = i32(B, 2, 4)
    lp = torch.zeros((B, 2, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="parents"):
        ddt.best_first_tree(ids, lp, i32(B), 5, parents=i32(B, 5))
