"""The verify loop over many steps: the end-to-end configuration.

A DDTree decode loop repeats one verify step per iteration ("The
Architectural Keystone: Writing the Model Header ...", section "The
Reasoning That Preceded the Header": the root of the next tree is the last
committed token, placed at the next free cache slot; after acceptance the
accepted path is compacted and the cache length advances).  This module
keeps the loop's state and bookkeeping:

* per request: the committed length P (device array, advanced in place by
  the step's compaction, mirrored on the host for the attention's work
  plan) and the root token of the next tree (the bonus token of the last
  step: the target's prediction after the deepest accepted node);
* one cache pool with room for the growth of every step: contiguous (each
  request owns a fixed range of rows), or paged (page_size > 0: the pool is
  pages of page_size rows, each request's block table row lists its pages,
  and pages are taken from a shuffled free list as the request grows --
  the table edits that go with compaction in a paged cache).

Each iteration draws its inputs (synthetic, seeded; untimed) and runs the
hot path through the C ABI with one `ddt.verify_step` call.  Inputs per
step, as the end-to-end configuration lays them out:

* draft logits N(0, sigma^2) over the vocabulary, per request and depth; per
  depth the top-K tokens and their log-probabilities, and the best-first
  draft tree of N nodes from those candidates rooted at the request's root
  token -- on the device by the library (`ddt_draft_topk`,
  `ddt_best_first_tree`; the loop's draft stage, timed on its own), or on
  the host (torch top-k and `synth.best_first_tree`) with device_draft=False;
* the node latents c_kv | k_pe (N(0,1), bf16) written at cache slots
  P .. P+N-1, and the absorbed queries q_lat | q_pe (N(0,1), bf16);
* target logits N(0,1) with +10 on a planted token per node: with
  probability alpha the node's first child's draft token, otherwise a
  uniform random token (`synth.planted_targets`).

The module holds none of the step's arithmetic (mask, attention, argmax,
acceptance, compaction are the library's); it only draws inputs and moves
the loop state forward.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import ddt, synth

BOOST = 10.0


@dataclass
class StepInputs:
    step: int
    parents: np.ndarray      # [B, N] int32 (host)
    draft_ids: np.ndarray    # [B, N] int32 (host); [:, 0] is the root token
    targets: np.ndarray      # [B, N] int32 planted target tokens (host)
    prefix_len: np.ndarray   # [B] int32 committed lengths P of this step (host)
    node_rows: torch.Tensor  # [B*N] int64 pool rows of the tree nodes (device)
    q: torch.Tensor          # [B*N*H, d_lat + d_rope] bf16 (device)
    logits: torch.Tensor     # [B*N, vocab] fp32 (device)
    parents_dev: torch.Tensor
    draft_dev: torch.Tensor
    roots: np.ndarray = None         # [B] root tokens of the trees (host)
    cand_ids: np.ndarray = None      # [B, D, K] draft candidates (host copies; device draft stage only)
    cand_lp: np.ndarray = None       # [B, D, K] fp32 log-probabilities
    draft_ms: float = 0.0            # device time of the draft stage (top-k + trees)

    def visible_pairs(self, H: int) -> int:
        """Visible (query row, key) pairs of the step: prefix plus ancestors and self."""
        B, N = self.parents.shape
        total = 0
        for b in range(B):
            d = np.zeros(N, np.int64)
            for i in range(1, N):
                d[i] = d[self.parents[b, i]] + 1
            total += int(self.prefix_len[b]) * N + int((d + 1).sum())
        return total * H


@dataclass
class StepResult:
    out: torch.Tensor
    lse: torch.Tensor
    idx: torch.Tensor
    accept_len: torch.Tensor
    path: torch.Tensor
    tokens: torch.Tensor


class VerifyLoop:
    """State of B requests across verify steps, on `device`."""

    def __init__(self, B=32, H=8, N=64, prefix_range=(2048, 65536), steps=100, vocab=synth.K2_VOCAB, K=8,
                 D=8, sigma=3.0, alpha=0.6, d_lat=512, d_rope=64, seed=1005, device="cuda", gap=32, page_size=0,
                 device_draft=True):
        self.B, self.H, self.N, self.steps = B, H, N, steps
        self.vocab, self.K, self.D, self.sigma, self.alpha = vocab, K, D, sigma, alpha
        self.d_lat, self.d_rope = d_lat, d_rope
        self.scale = 1.0 / float(np.sqrt(d_lat + d_rope))
        self.device = torch.device(device)
        self.seed = seed
        self.rng = np.random.default_rng(seed)
        lo, hi = prefix_range
        P0 = self.rng.integers(lo, hi + 1, size=B).astype(np.int32)
        # each step grows a request by at most N rows (root + accepted drafts)
        cap = P0.astype(np.int64) + N + steps * N
        base = np.zeros(B, np.int64)
        off = gap
        for b in range(B):
            base[b] = off
            off += int(cap[b]) + gap
        self.capacity = cap
        self.kv_base_host = base          # the logical (contiguous) layout: the pool's rows unless paged
        self.logical_rows = int(off)
        self.P_host = P0.copy()
        self.roots = self.rng.integers(0, vocab, size=B).astype(np.int32)
        dev = self.device
        g = self._gen(-1)
        d_qk = d_lat + d_rope
        self.page_size = page_size
        if page_size:
            if page_size < 32 or page_size & (page_size - 1):
                raise ValueError("page_size must be a power of two >= 32")
            per_req = (cap + page_size - 1) // page_size
            n_pages = int(per_req.sum())
            self.free_pages = list(self.rng.permutation(n_pages).astype(np.int32))
            self.table_host = np.zeros((B, int(per_req.max())), np.int32)
            self.n_pages = np.zeros(B, np.int64)
            self.table_dev = torch.zeros((B, int(per_req.max())), dtype=torch.int32, device=dev)
            pool_rows = n_pages * page_size
        else:
            pool_rows = int(off)
        # rows past a request's keys (and the gaps, and pages not yet handed
        # out) hold NaN, so a read past the keys would show in the outputs
        self.pool = torch.full((pool_rows, d_qk), float("nan"), dtype=torch.bfloat16, device=dev)
        if page_size:
            self._ensure_slots(P0.astype(np.int64))
        for b in range(B):
            rows = int(P0[b])
            if rows:
                r = torch.from_numpy(self.rows_of(b, np.arange(rows))).to(dev)
                self.pool[r] = torch.randn((rows, d_qk), generator=g, device=dev, dtype=torch.float32).to(
                    torch.bfloat16)
        self.kv_base = torch.from_numpy(base).to(dev)
        self.prefix_dev = torch.from_numpy(P0.copy()).to(dev)
        rows = B * N * H
        self.out = torch.empty((rows, d_lat), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((rows,), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B * N,), dtype=torch.int32, device=dev)
        self.acc = torch.empty((B,), dtype=torch.int32, device=dev)
        self.path = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.tok = torch.empty((B, N), dtype=torch.int32, device=dev)
        n = ddt.argmax_workspace_bytes(B * N, vocab)
        self.am_ws = torch.zeros((max(n, 16),), dtype=torch.uint8, device=dev)   # zero before first use
        self.ws = torch.empty((1,), dtype=torch.uint8, device=dev)
        self.logits = torch.empty((B * N, vocab), dtype=torch.float32, device=dev)
        self.q = torch.empty((rows, d_qk), dtype=torch.bfloat16, device=dev)
        self.device_draft = device_draft
        if device_draft:
            self.cand_ids = torch.empty((B * D, K), dtype=torch.int32, device=dev)
            self.cand_lp = torch.empty((B * D, K), dtype=torch.float32, device=dev)
            self.topk_ws = torch.empty((max(16, ddt.draft_topk_workspace_bytes(B * D, vocab, K)),),
                                       dtype=torch.uint8, device=dev)
            self.tree_out = [torch.empty((B, N), dtype=torch.int32, device=dev) for _ in range(3)]
        self.step_no = 0

    # ------------------------------------------------------------- cache ----
    def rows_of(self, b: int, t: np.ndarray) -> np.ndarray:
        """Pool rows of request b's cache slots t."""
        t = np.asarray(t, np.int64)
        if not self.page_size:
            return self.kv_base_host[b] + t
        ps = self.page_size
        return self.table_host[b, t // ps].astype(np.int64) * ps + t % ps

    def _ensure_slots(self, T: np.ndarray):
        """Paged: hand out pages until request b has at least T[b] slots."""
        grew = False
        for b in range(self.B):
            while self.n_pages[b] * self.page_size < T[b]:
                if not self.free_pages:
                    raise RuntimeError("cache capacity exceeded")
                self.table_host[b, self.n_pages[b]] = self.free_pages.pop()
                self.n_pages[b] += 1
                grew = True
        if grew:
            self.table_dev.copy_(torch.from_numpy(self.table_host))

    def to_logical(self, pool_host: np.ndarray) -> np.ndarray:
        """A host copy of the pool in the logical layout (request b's slot t
        at row kv_base_host[b] + t; slots without a page are NaN)."""
        if not self.page_size:
            return pool_host
        out = np.full((self.logical_rows, pool_host.shape[1]), pool_host.dtype.type(0x7FC0), pool_host.dtype)
        for b in range(self.B):
            t = np.arange(int(self.n_pages[b]) * self.page_size)
            out[self.kv_base_host[b] + t] = pool_host[self.rows_of(b, t)]
        return out

    def pages(self):
        return (self.table_dev, self.page_size) if self.page_size else None

    # ------------------------------------------------------------ inputs ----
    def _gen(self, step: int) -> torch.Generator:
        g = torch.Generator(device=self.device)
        g.manual_seed(self.seed * 1_000_003 + step + 1)
        return g

    def ckv(self):
        return self.pool[:, : self.d_lat]

    def kpe(self):
        return self.pool[:, self.d_lat:]

    def make_inputs(self) -> StepInputs:
        """Draw step `step_no`'s inputs and write its node latents into the pool."""
        B, N, H, V, K, D = self.B, self.N, self.H, self.vocab, self.K, self.D
        dev = self.device
        g = self._gen(self.step_no)
        # per request and depth: top-K of N(0, sigma^2) draft logits and their log-softmax
        x = torch.randn((B, D, V), generator=g, device=dev, dtype=torch.float32) * self.sigma
        roots = self.roots.copy()
        cand_ids = cand_lp = None
        draft_ms = 0.0
        if self.device_draft:
            # the draft stage on the device: top-K per (request, depth), then the trees
            roots_dev = torch.from_numpy(roots).to(dev)
            stream = torch.cuda.current_stream(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ddt.draft_topk(x.view(B * D, V), K, self.cand_ids, self.cand_lp, self.topk_ws)
            par_d, tok_d, _ = ddt.best_first_tree(self.cand_ids.view(B, D, K), self.cand_lp.view(B, D, K), roots_dev,
                                                  N - 1, *self.tree_out)
            e1.record(stream)
            parents, draft = par_d.cpu().numpy(), tok_d.cpu().numpy()   # (synchronises)
            draft_ms = e0.elapsed_time(e1)
            cand_ids = self.cand_ids.view(B, D, K).cpu().numpy()
            cand_lp = self.cand_lp.view(B, D, K).cpu().numpy()
        else:
            top = torch.topk(x, K, dim=-1)
            lp = (top.values - torch.logsumexp(x, dim=-1, keepdim=True)).cpu().numpy()
            ids = top.indices.to(torch.int32).cpu().numpy()
            parents = np.empty((B, N), np.int32)
            draft = np.empty((B, N), np.int32)
            for b in range(B):
                parents[b], draft[b], _ = synth.best_first_tree(ids[b], lp[b], N - 1, int(roots[b]))
        del x
        targets = synth.planted_targets(self.rng, parents, draft, V, self.alpha)
        # node latents at slots P .. P+N-1 and the queries
        P = self.P_host.copy()
        if np.any(P.astype(np.int64) + N > self.capacity):
            raise RuntimeError("cache capacity exceeded")
        if self.page_size:
            self._ensure_slots(P.astype(np.int64) + N)
        node_rows = torch.from_numpy(np.concatenate([self.rows_of(b, P[b] + np.arange(N)) for b in range(B)])).to(dev)
        d_qk = self.d_lat + self.d_rope
        lat = torch.randn((B * N, d_qk), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        self.pool.index_copy_(0, node_rows, lat)
        self.q.copy_(torch.randn(self.q.shape, generator=g, device=dev, dtype=torch.float32))
        # target logits: N(0,1) noise, +BOOST on each node's planted token
        self.logits.normal_(generator=g)
        rows = torch.arange(B * N, device=dev)
        self.logits[rows, torch.from_numpy(targets.reshape(-1).astype(np.int64)).to(dev)] += BOOST
        return StepInputs(self.step_no, parents, draft, targets, P, node_rows, self.q, self.logits,
                          torch.from_numpy(parents).to(dev), torch.from_numpy(draft).to(dev), roots, cand_ids, cand_lp,
                          draft_ms)

    # -------------------------------------------------------------- step ----
    def workspace_for(self, P: np.ndarray):
        desc = ddt.attn_desc(self.q[:, : self.d_lat], self.q[:, self.d_lat:], self.ckv(), self.kpe(), B=self.B,
                             H=self.H, N=self.N, scale=self.scale, pages=self.pages())
        need = ddt.verify_workspace_bytes(desc, P)
        if need > self.ws.numel():
            self.ws = torch.empty((need,), dtype=torch.uint8, device=self.device)
        return self.ws

    def run_step(self, inp: StepInputs, stream=None) -> StepResult:
        """The hot path of one step: ancestor bits, attention, argmax,
        acceptance, compaction and the length update (prefix_dev in place)."""
        ws = self.workspace_for(inp.prefix_len)
        dl = self.d_lat
        mask = None
        if self.N > 128:
            mask = ddt.build_mask(inp.parents_dev, stream=stream)[0]
        kv_base = None if self.page_size else self.kv_base
        ddt.verify_step(inp.q[:, :dl], inp.q[:, dl:], self.ckv(), self.kpe(), kv_base, inp.prefix_len, mask,
                        inp.logits, inp.draft_dev, inp.parents_dev, self.prefix_dev, H=self.H, scale=self.scale,
                        out=self.out, lse=self.lse, workspace=ws, idx=self.idx, argmax_workspace=self.am_ws,
                        accept_len=self.acc, path=self.path, tokens=self.tok, pages=self.pages(), stream=stream)
        return StepResult(self.out, self.lse, self.idx, self.acc, self.path, self.tok)

    def advance(self, res: StepResult):
        """Loop bookkeeping after a step: the bonus token (the target's token
        after the deepest accepted node) is the next root, and the host copy
        of the committed lengths follows the device's."""
        acc = res.accept_len.cpu().numpy()
        tok = res.tokens.cpu().numpy()
        P = self.prefix_dev.cpu().numpy()
        self.roots = tok[np.arange(self.B), acc].astype(np.int32)
        self.P_host = P.astype(np.int32)
        self.step_no += 1
        return acc
