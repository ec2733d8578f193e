"""Shared helpers for the GPU parity tests: moving synthetic workloads onto the
device, running the oracle on the same inputs, and error metrics."""
from __future__ import annotations

import numpy as np
import torch

from mla_tree_verify_parents_amd import synth


def to_dev(a: np.ndarray, dev="cuda"):
    """numpy -> torch on `dev`; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t: torch.Tensor) -> np.ndarray:
    """torch -> numpy; bf16 becomes uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


class DevWorkload:
    """Device copies of one synthetic workload."""

    def __init__(self, w: synth.Workload):
        self.w = w
        self.pool = to_dev(w.pool)
        self.q = to_dev(w.q)
        self.parents = to_dev(w.parents)
        self.draft = to_dev(w.draft_ids)
        self.kv_base = to_dev(w.kv_base)
        self.prefix_dev = to_dev(w.prefix_len)
        self.target = None if w.target_ids is None else to_dev(w.target_ids)
        self.logits = None if w.logits is None else to_dev(w.logits)

    def q_lat(self):
        return self.q[:, : self.w.d_lat]

    def q_pe(self):
        return self.q[:, self.w.d_lat:]

    def ckv(self):
        return self.pool[:, : self.w.d_lat]

    def kpe(self):
        return self.pool[:, self.w.d_lat:]


def oracle_attn(orc, w: synth.Workload, rows=None):
    return orc.verify_attn(w.q_lat(), w.q_pe(), w.ckv(), w.kpe(), w.kv_base, w.prefix_len, w.parents,
                           H=w.H, scale=w.scale, rows=rows)


ATTN_TOL = {"f32": 1e-5, "bf16": 1e-2}
