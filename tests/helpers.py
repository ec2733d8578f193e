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


# Whole-tensor relative L2 of out and of lse: the tolerance the method's
# statement fixes (fp32 inputs 1e-5; bf16 inputs with fp32 accumulation 1e-2).
ATTN_TOL = {"f32": 1e-5, "bf16": 1e-2}
# Every row's relative L2 error of out.  On the bf16 path each probability
# and each stored output element is rounded to nearest even in bf16 (unit
# roundoff u = 2^-8, independent errors), so a row's relative L2 error is a
# few times u/sqrt(3) ~ 2.3e-3 whatever the row's key count; 2e-2 leaves a
# wide margin yet fails one wrong 32-column tile of a row (~0.25).  fp32
# inputs: fp32 probabilities and outputs, row errors ~1e-6.
ROW_TOL = {"f32": 2e-5, "bf16": 2e-2}
# Largest lse error, LSE_ABS_TOL + LSE_REL_TOL * |lse|.  lse = m + ln(sum
# of probabilities) with the probabilities rounded to bf16 before they are
# summed, so the sum is off by at most a factor 1 +- u: |error| <=
# ln(1 + 2^-8) ~ 3.9e-3.  The scores themselves are fp32 sums of 576
# products, whose rounding is relative to their size (~sqrt(576) * 2^-24 ~
# 1.4e-6 of |s|, more where terms cancel): that part scales with |lse|,
# which reaches ~1e4 on rows with huge scores.  fp32 inputs: probabilities
# in fp32.
LSE_ABS_TOL = {"f32": 1e-4, "bf16": 5e-3}
LSE_REL_TOL = 1e-5


def attn_errors(out, lse, ref_out, ref_lse, dtype):
    """(rel-L2 of out, rel-L2 of lse, largest per-row rel-L2 of out, largest
    lse error as a fraction of its bound LSE_ABS_TOL + LSE_REL_TOL * |lse|)."""
    o = as_f64(out) if out.dtype == np.uint16 else np.asarray(out, np.float64)
    o = o.reshape(ref_out.shape)
    lse = np.asarray(lse, np.float64).reshape(ref_lse.shape)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "non-finite attention output"
    row = np.linalg.norm(o - ref_out, axis=1) / np.maximum(np.linalg.norm(ref_out, axis=1), 1e-300)
    lse_frac = np.abs(lse - ref_lse) / (LSE_ABS_TOL[dtype] + LSE_REL_TOL * np.abs(ref_lse))
    return rel_l2(o, ref_out), rel_l2(lse, ref_lse), float(row.max()), float(lse_frac.max())


def check_attn(out, lse, ref_out, ref_lse, dtype, what=""):
    """Attention outputs against the oracle: whole-tensor rel-L2 of out and
    lse within ATTN_TOL, every row of out within ROW_TOL, every lse within
    LSE_ABS_TOL + LSE_REL_TOL * |lse|.  out: host array (bf16 bits or
    float), rows as ref_out."""
    e = attn_errors(out, lse, ref_out, ref_lse, dtype)
    ok = e[0] <= ATTN_TOL[dtype] and e[1] <= ATTN_TOL[dtype] and e[2] <= ROW_TOL[dtype] and e[3] <= 1.0
    assert ok, (what, "rel_l2 out %.3e lse %.3e, max row %.3e, max lse error %.3f of its bound" % e)
    return e
