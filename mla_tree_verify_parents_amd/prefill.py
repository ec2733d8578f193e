"""Chunked causal prefill through the verify attention.

"The Architecture of Pragmatic Ambition", section "The Decision
Architecture": prefill, decode and tree verification share one absorbed
attention and differ only in the mask -- causal for prefill, the tree's
ancestor relation for verification.  A chain-shaped tree (node i's parent is
i-1) has exactly the causal mask, so a prefill chunk of N <= 1024 tokens
placed at cache rows P .. P+N-1 is one ``ddt_verify_attn`` call with a chain
tree at committed length P, and a prompt of any length is a sequence of
such calls with P advancing by the chunk length.

This module is host orchestration only (chain masks built once per chunk
length by ``ddt_build_mask``, one workspace, one library call per chunk); the
arithmetic is the library's.  One sequence per call: the verify attention
takes one query row stride for all requests, and a chunk's rows are
contiguous only within one sequence.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ddt


class ChunkedPrefill:
    """Causal attention of T prompt tokens over a request's latent cache.

    The caller has written the latents c_kv | k_pe of the prompt's tokens at
    cache rows kv_base + P0 .. kv_base + P0 + T - 1 (the model's forward would
    write each chunk's rows before its attention) and passes the absorbed
    queries of the prompt, row t*H + h for token t and head h.
    """

    def __init__(self, H: int, scale: float, chunk: int = 1024, device="cuda"):
        if not 1 <= chunk <= ddt.MAX_NODES:
            raise ValueError(f"chunk must be in [1, {ddt.MAX_NODES}]")
        self.H, self.scale, self.chunk = H, float(scale), chunk
        self.device = torch.device(device)
        self._masks = {}
        self._ws = None

    def mask(self, n: int) -> torch.Tensor:
        """Ancestor mask of an n-node chain (the causal mask), built once."""
        m = self._masks.get(n)
        if m is None:
            par = torch.arange(-1, n - 1, dtype=torch.int32, device=self.device).view(1, n)
            m, _, err = ddt.build_mask(par)
            self._masks[n] = m
        return m

    def chunks(self, T: int, P0: int):
        """(first token, tokens, committed length) of each chunk."""
        out, done = [], 0
        while done < T:
            n = min(self.chunk, T - done)
            out.append((done, n, P0 + done))
            done += n
        return out

    def workspace(self, q_lat, q_pe, ckv, kpe, T: int, P0: int) -> torch.Tensor:
        need = 1
        for _, n, P in self.chunks(T, P0):
            d = ddt.attn_desc(q_lat[: n * self.H], q_pe[: n * self.H], ckv, kpe, B=1, H=self.H, N=n,
                              scale=self.scale)
            need = max(need, ddt.verify_workspace_bytes(d, np.array([P], np.int32)))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty((need,), dtype=torch.uint8, device=self.device)
        return self._ws

    def run(self, q_lat, q_pe, ckv, kpe, kv_base, P0: int, out=None, lse=None, stream=None):
        """q_lat [T*H, d_lat], q_pe [T*H, d_rope] row views; ckv/kpe views of
        the cache pool; kv_base [1] int64 (device).  Returns (out [T*H,
        d_lat], lse [T*H]); rows of chunk c are written by its call."""
        H = self.H
        if q_lat.shape[0] % H:
            raise ValueError("q rows must be T*H")
        T = q_lat.shape[0] // H
        if out is None:
            out = torch.empty((T * H, q_lat.shape[1]), dtype=q_lat.dtype, device=q_lat.device)
        if lse is None:
            lse = torch.empty((T * H,), dtype=torch.float32, device=q_lat.device)
        ws = self.workspace(q_lat, q_pe, ckv, kpe, T, P0)
        for t0, n, P in self.chunks(T, P0):
            r0, r1 = t0 * H, (t0 + n) * H
            ddt.verify_attn(q_lat[r0:r1], q_pe[r0:r1], ckv, kpe, kv_base, np.array([P], np.int32), self.mask(n),
                            H=H, scale=self.scale, out=out[r0:r1], lse=lse[r0:r1], workspace=ws, stream=stream)
        return out, lse
