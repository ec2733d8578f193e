"""Chunked causal prefill through the verify attention.

"The Architecture of Pragmatic Ambition", section "The Decision
Architecture": prefill, decode and tree verification share one absorbed
attention and differ only in the mask -- causal for prefill, the tree's
ancestor relation for verification.  A chain-shaped tree (node i's parent is
i-1) has exactly the causal mask, so a prefill chunk of N <= 1024 tokens
placed at cache rows P .. P+N-1 is a chain tree at committed length P.

Within one layer every latent of the prompt exists before the layer's
attention runs, so the chunks do not depend on each other: chunk c is one
request of a batched ``ddt_verify_attn`` call whose requests all share the
prompt's cache region (the same kv_base), with committed length P0 + c*chunk.
The query rows of the requests, request-major, are exactly the prompt's
token-major rows, so one call covers every full chunk (and the library's
work plan balances their ragged key ranges over the CUs); a shorter last
chunk is a second call.

This module is host orchestration only (chain masks built once per shape by
``ddt_build_mask``, one workspace, at most two library calls); the
arithmetic is the library's.  One prompt per call.
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

    def mask(self, n: int, reqs: int = 1) -> torch.Tensor:
        """Ancestor masks of `reqs` n-node chains (the causal mask), built once."""
        m = self._masks.get((n, reqs))
        if m is None:
            par = torch.arange(-1, n - 1, dtype=torch.int32, device=self.device).view(1, n).repeat(reqs, 1)
            m, _, err = ddt.build_mask(par.contiguous())
            self._masks[(n, reqs)] = m
        return m

    def calls(self, T: int, P0: int):
        """(first token, chunks, tokens per chunk) of each library call: the
        full chunks together (up to MAX_BATCH per call), then the shorter
        last chunk."""
        full, rest = divmod(T, self.chunk)
        out = []
        for c0 in range(0, full, ddt.MAX_BATCH):          # at most MAX_BATCH requests per call
            out.append((c0 * self.chunk, min(ddt.MAX_BATCH, full - c0), self.chunk))
        if rest:
            out.append((full * self.chunk, 1, rest))
        return out

    def chunks(self, T: int, P0: int):
        """(first token, tokens, committed length) of each chunk."""
        out, done = [], 0
        while done < T:
            n = min(self.chunk, T - done)
            out.append((done, n, P0 + done))
            done += n
        return out

    def _prefix(self, t0: int, reqs: int, n: int, P0: int) -> np.ndarray:
        return (P0 + t0 + n * np.arange(reqs)).astype(np.int32)

    def workspace(self, q_lat, q_pe, ckv, kpe, T: int, P0: int) -> torch.Tensor:
        need = 1
        for t0, reqs, n in self.calls(T, P0):
            rows = reqs * n * self.H
            d = ddt.attn_desc(q_lat[:rows], q_pe[:rows], ckv, kpe, B=reqs, H=self.H, N=n, scale=self.scale)
            need = max(need, ddt.verify_workspace_bytes(d, self._prefix(t0, reqs, n, P0)))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty((need,), dtype=torch.uint8, device=self.device)
        return self._ws

    def run(self, q_lat, q_pe, ckv, kpe, kv_base, P0: int, out=None, lse=None, stream=None):
        """q_lat [T*H, d_lat], q_pe [T*H, d_rope] row views; ckv/kpe views of
        the cache pool; kv_base [1] int64 (device).  Returns (out [T*H,
        d_lat], lse [T*H])."""
        H = self.H
        if q_lat.shape[0] % H:
            raise ValueError("q rows must be T*H")
        T = q_lat.shape[0] // H
        if out is None:
            out = torch.empty((T * H, q_lat.shape[1]), dtype=q_lat.dtype, device=q_lat.device)
        if lse is None:
            lse = torch.empty((T * H,), dtype=torch.float32, device=q_lat.device)
        ws = self.workspace(q_lat, q_pe, ckv, kpe, T, P0)
        for t0, reqs, n in self.calls(T, P0):
            r0, r1 = t0 * H, (t0 + reqs * n) * H
            base = kv_base.expand(reqs).contiguous() if reqs > 1 else kv_base
            ddt.verify_attn(q_lat[r0:r1], q_pe[r0:r1], ckv, kpe, base, self._prefix(t0, reqs, n, P0),
                            self.mask(n, reqs), H=H, scale=self.scale, out=out[r0:r1], lse=lse[r0:r1], workspace=ws,
                            stream=stream)
        return out, lse
