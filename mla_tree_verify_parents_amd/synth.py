"""Seeded synthetic workloads for the tree-verify hot path.

This module only draws inputs: random latents and queries, draft trees and
target tokens.  It holds none of the arithmetic of the verify step (no mask,
attention, argmax, acceptance or compaction) and is the only code that both
the HIP path's tests and the oracle consume.  One step before the verify
path does live here: `best_first_tree` grows the input trees of the
best-first configurations.  It is input generation only; the device builder
(ddt_best_first_tree) is checked against the oracle's own builder, never
against this one.

Shapes follow the Kimi-K2 style MLA attention the pages target: a latent
cache row is c_kv (kv_lora_rank wide) followed by the decoupled rope key
k_pe; queries are the absorbed q_lat followed by q_pe.  Draft trees are
either uniform random trees (node i's parent uniform in [0, i)) or best-first
trees grown from per-depth top-k draft candidates, the tree shape DDTree
builds ("The Architecture of Pragmatic Ambition", section "The Knowledge
Architecture": a best-first tree from the drafter's per-depth top-k).
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32(np.nan)
K2_VOCAB = 163840


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) samples stored as fp32 or as bf16 bits, drawn in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = x if dtype == "f32" else to_bf16_bits(x)
    return out.reshape(shape)


def random_parents(rng: np.random.Generator, B: int, N: int) -> np.ndarray:
    """parents[b][0] = -1 and parents[b][i] uniform in [0, i)."""
    p = np.empty((B, N), np.int32)
    p[:, 0] = -1
    for i in range(1, N):
        p[:, i] = rng.integers(0, i, size=B)
    return p


def topk_desc(x: np.ndarray, k: int):
    """Indices of the k largest entries, ordered by (value desc, index asc)."""
    part = np.argpartition(-x, k - 1)[:k]
    order = np.lexsort((part, -x[part]))
    return part[order]


def draft_candidates(rng: np.random.Generator, D: int, K: int, V: int, sigma: float):
    """Per-depth top-K draft candidates from seeded N(0, sigma^2) draft logits.

    Returns (ids [D, K] int32, logp [D, K] float32) with logp the log-softmax
    of the candidates' logits over the full vocabulary, in descending order.
    """
    ids = np.empty((D, K), np.int32)
    lp = np.empty((D, K), np.float32)
    for d in range(D):
        x = rng.standard_normal(V).astype(np.float64) * sigma
        top = topk_desc(x, K)
        mx = x.max()
        lse = mx + np.log(np.exp(x - mx).sum())
        ids[d] = top
        lp[d] = (x[top] - lse).astype(np.float32)
    return ids, lp


def best_first_tree(ids: np.ndarray, lp: np.ndarray, budget: int, root_token: int = 0):
    """Grow a draft tree of budget+1 nodes best first.

    A node at depth d >= 1 with rank r carries token ids[d-1][r]; its score is
    its parent's score plus lp[d-1][r] (fp32, added along the path).  The
    frontier starts with (depth 1, rank 0) under the root.  Popping a
    candidate appends it as the next node and pushes its first child
    (depth d+1, rank 0) and its next sibling (depth d, rank r+1).  Ties go by
    (score desc, depth asc, push order).  Nodes are numbered in pop order, so
    parents[i] < i.
    """
    D, K = ids.shape
    parents = [-1]
    tokens = [int(root_token)]
    depth = [0]
    score = [np.float32(0.0)]
    heap = []
    push = 0

    def add(parent, d, r):
        nonlocal push
        s = np.float32(score[parent] + lp[d - 1][r])
        heapq.heappush(heap, (-float(s), d, push, parent, r, s))
        push += 1

    if D > 0 and K > 0 and budget > 0:
        add(0, 1, 0)
    while heap and len(parents) < budget + 1:
        _, d, _, parent, r, s = heapq.heappop(heap)
        node = len(parents)
        parents.append(parent)
        tokens.append(int(ids[d - 1][r]))
        depth.append(d)
        score.append(s)
        if d < D:
            add(node, d + 1, 0)
        if r + 1 < K:
            add(parent, d, r + 1)
    n = len(parents)
    if n < budget + 1:
        raise ValueError(f"candidate grid too small for budget {budget}: {n - 1} drafts")
    return (np.array(parents, np.int32), np.array(tokens, np.int32), np.array(depth, np.int32))


def first_child(parents: np.ndarray) -> np.ndarray:
    """Lowest-numbered child of every node (-1 for leaves); parents [N]."""
    N = parents.shape[0]
    fc = np.full(N, -1, np.int32)
    for k in range(N - 1, 0, -1):
        fc[parents[k]] = k
    return fc


def planted_targets(rng, parents, draft_ids, vocab: int, alpha: float) -> np.ndarray:
    """Target greedy tokens: with probability alpha a node's target token is
    its first child's draft token (so that child is accepted), otherwise a
    uniform random token.  parents/draft_ids [B, N]."""
    B, N = parents.shape
    t = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
    for b in range(B):
        fc = first_child(parents[b])
        hit = rng.random(N) < alpha
        for c in range(N):
            if hit[c] and fc[c] >= 0:
                t[b, c] = draft_ids[b, fc[c]]
    return t


def target_logits(rng, t: np.ndarray, vocab: int, boost: float = 10.0) -> np.ndarray:
    """fp32 logits [rows, vocab] = N(0,1) noise plus `boost` on token t[row]."""
    rows = t.shape[0]
    x = rng.standard_normal((rows, vocab), dtype=np.float32)
    x[np.arange(rows), t] += np.float32(boost)
    return x


@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d_lat: int
    d_rope: int
    dtype: str                 # "f32" or "bf16"
    scale: float
    prefix_len: np.ndarray     # [B] int32, committed cache length before the root
    kv_base: np.ndarray        # [B] int64, first pool row of request b
    capacity: np.ndarray       # [B] int64, pool rows reserved for request b
    pool: np.ndarray           # [rows, d_lat + d_rope] cache pool (c_kv | k_pe)
    q: np.ndarray              # [B*N*H, d_lat + d_rope] queries (q_lat | q_pe)
    parents: np.ndarray        # [B, N] int32
    draft_ids: np.ndarray      # [B, N] int32 (entry 0: last committed token)
    target_ids: Optional[np.ndarray] = None  # [B, N] int32 when given directly
    logits: Optional[np.ndarray] = None      # [B*N, vocab] fp32 when argmax is on the path
    vocab: int = K2_VOCAB
    meta: dict = field(default_factory=dict)

    @property
    def d_qk(self):
        return self.d_lat + self.d_rope

    @property
    def rows(self):
        return self.B * self.N * self.H

    def q_lat(self):
        return self.q[:, : self.d_lat]

    def q_pe(self):
        return self.q[:, self.d_lat:]

    def ckv(self, pool=None):
        p = self.pool if pool is None else pool
        return p[:, : self.d_lat]

    def kpe(self, pool=None):
        p = self.pool if pool is None else pool
        return p[:, self.d_lat:]

    def keys(self) -> np.ndarray:
        return self.prefix_len.astype(np.int64) + self.N

    def visible_pairs(self) -> int:
        """Number of visible (query row, key) pairs: prefix plus ancestors."""
        depth_sum = 0
        for b in range(self.B):
            d = np.zeros(self.N, np.int64)
            for i in range(1, self.N):
                d[i] = d[self.parents[b, i]] + 1
            depth_sum += int(self.prefix_len[b]) * self.N + int((d + 1).sum())
        return depth_sum * self.H


def make_pool(rng, prefix_len, N, d_qk, dtype, extra_rows=0, gap=32):
    """Cache pool with one region per request.  Rows [0, P_b + N) of a region
    hold N(0,1) latents; the remaining reserved rows and the gaps between
    regions hold NaN so any read past a request's keys shows up."""
    B = len(prefix_len)
    cap = np.array([int(p) + N + extra_rows for p in prefix_len], np.int64)
    base = np.zeros(B, np.int64)
    off = gap
    for b in range(B):
        base[b] = off
        off += cap[b] + gap
    total = int(off)
    nan = F32_NAN if dtype == "f32" else BF16_NAN
    pool = np.full((total, d_qk), nan, dtype=np.float32 if dtype == "f32" else np.uint16)
    for b in range(B):
        T = int(prefix_len[b]) + N
        pool[base[b]: base[b] + T] = normal(rng, (T, d_qk), dtype)
    return pool, base, cap


def workload(cfg: int, seed: Optional[int] = None, **over) -> Workload:
    """Build one of the five configurations (1..5) with its default seed 1000+cfg.

    Keyword overrides (B, H, N, prefix, ...) shrink a configuration for tests.
    """
    seed = 1000 + cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    if cfg == 1:
        B, H, N, dl, dr, dt = 1, 2, 8, 64, 16, "f32"
        B, H, N = over.get("B", B), over.get("H", H), over.get("N", N)
        P = np.full(B, over.get("prefix", 32), np.int32)
        vocab = 64
        parents = random_parents(rng, B, N)
        draft = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
        target = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
        logits = None
    elif cfg in (2, 4):
        if cfg == 2:
            B, H, N, K, D, sigma = 1, 8, 64, 4, 8, 3.0
            prefix = 4096
        else:
            B, H, N, K, D, sigma = 4, 64, 128, 8, 4, 1.0
            prefix = 131072
        dl, dr, dt = 512, 64, "bf16"
        B, H, N = over.get("B", B), over.get("H", H), over.get("N", N)
        P = np.full(B, over.get("prefix", prefix), np.int32)
        vocab = over.get("vocab", K2_VOCAB)
        parents = np.empty((B, N), np.int32)
        draft = np.empty((B, N), np.int32)
        for b in range(B):
            ids, lp = draft_candidates(rng, D, K, vocab, sigma)
            root = int(rng.integers(0, vocab))
            parents[b], draft[b], _ = best_first_tree(ids, lp, N - 1, root)
        target = planted_targets(rng, parents, draft, vocab, 0.6)
        logits = None
        if cfg == 2 and over.get("with_logits", True):
            logits = target_logits(rng, target.reshape(-1), vocab)
            target = None
    elif cfg == 3:
        B, H, N, dl, dr, dt = 16, 8, 32, 512, 64, "bf16"
        B, H, N = over.get("B", B), over.get("H", H), over.get("N", N)
        lo, hi = over.get("prefix_range", (1024, 32768))
        P = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        vocab = K2_VOCAB
        parents = random_parents(rng, B, N)
        draft = rng.integers(0, vocab, size=(B, N)).astype(np.int32)
        target = planted_targets(rng, parents, draft, vocab, 0.6)
        logits = None
    else:
        raise ValueError(f"unknown configuration {cfg}")
    pool, base, cap = make_pool(rng, P, N, dl + dr, dt, extra_rows=over.get("extra_rows", 0))
    q = normal(rng, (B * N * H, dl + dr), dt)
    return Workload(name=f"config{cfg}", B=B, H=H, N=N, d_lat=dl, d_rope=dr, dtype=dt,
                    scale=1.0 / float(np.sqrt(dl + dr)), prefix_len=P, kv_base=base,
                    capacity=cap, pool=pool, q=q, parents=parents, draft_ids=draft,
                    target_ids=target, logits=logits, vocab=vocab, meta={"seed": seed})
