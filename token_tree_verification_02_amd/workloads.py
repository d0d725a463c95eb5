"""Seeded synthetic inputs for tree attention and greedy tree verification.

This module only *produces inputs*: tree topologies, KV caches in the
library's layouts, queries, logits, draft tokens and planted edits.  It
computes nothing that the method computes (no scores, no softmax, no argmax,
no accept walk), so the CPU oracle and the HIP path can both consume what it
returns without sharing any of the method's arithmetic.

Randomness is counter-keyed: every stream (tree, lengths, Q, K, ...) and every
chunk inside a stream draws from ``SeedSequence(seed, spawn_key=(stream,
chunk))`` with PCG64, so the arrays are identical whatever the thread count.
Floating-point draws are made in float32 and rounded to bfloat16
round-to-nearest-even where the workload is bf16.

Layouts (last dimension contiguous, matching ``include/tree_verify.h``):
  q, k_tree, v_tree     [B][n][H][D]
  k_cache, v_cache contiguous    [B][Hkv][Lmax][D]
  k_cache, v_cache paged         [num_blocks][Hkv][16][D]
  block_table           [B][max_blocks]  int32, -1 where unused
  logits                [B][n][V]
Cache slots past a sequence's prefix length hold NaN, so a kernel that reads
them shows it in its output.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

PAGE = 16
BF16_NAN = np.uint16(0x7FC0)
F16_NAN = np.uint16(0x7E00)
F32_NAN = np.float32(np.nan)

# stream ids for the counter-keyed generator
_S_TREE, _S_LEN, _S_PERM, _S_Q, _S_K, _S_V, _S_KT, _S_VT, _S_LOGIT, _S_TOK, _S_PLANT, _S_VAR = range(12)
_S_SSM, _S_UNIF = range(12, 14)
_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str          # "f32", "bf16" or "f16" (q, k, v, out and logits share it)
    L_lo: int           # prefix length range, inclusive
    L_hi: int
    paged: bool
    tree: str           # "expand:<k1,k2,...>", "merge", "random", "frontier"
    n: int              # tree nodes including the root
    max_depth: int
    vocab: int          # 0 = no verification on this workload
    logit_sigma: float
    Lmax: int = 0       # contiguous cache capacity (0 = L_hi)
    kv: str = ""        # "" : the cache has `dtype`; "fp8": OCP E4M3 codes times a per-tensor scale

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def capacity(self) -> int:
        """Contiguous cache capacity in tokens (a multiple of 16)."""
        c = self.Lmax or self.L_hi
        return (c + PAGE - 1) // PAGE * PAGE


CONFIGS = {
    1: Config(1, "tiny_fp32", 1, 4, 4, 64, "f32", 128, 128, False, "expand:2,2", 7, 2, 1000, 1.0),
    2: Config(2, "llama7b_layer", 8, 32, 32, 128, "bf16", 1024, 1024, False,
              "expand:1,1,3,1,1,1,1,1", 21, 8, 32000, 2.0),
    3: Config(3, "merge_trees", 16, 64, 8, 128, "bf16", 2048, 2048, False, "merge", 64, 8, 32000, 2.0),
    4: Config(4, "long_ragged_paged", 32, 64, 8, 128, "bf16", 8192, 32768, True, "random", 32, 6, 0, 2.0),
    5: Config(5, "wide_trees", 64, 32, 8, 128, "bf16", 512, 8192, False, "frontier", 128, 12, 128000, 2.0,
              Lmax=8192),
}


def config(index: int, **overrides) -> Config:
    """The numbered workload, optionally with fields overridden (smaller B, L, ...)."""
    c = CONFIGS[index]
    return replace(c, **overrides) if overrides else c


# ----------------------------------------------------------------------------- rng helpers
def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, chunk))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); returns the raw uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


FP8_NAN = np.uint8(0x7F)


def _fp8_table():
    """Non-negative finite E4M3 values (codes 0..126) in increasing order."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def fp8_encode(x: np.ndarray) -> np.ndarray:
    """float -> nearest OCP E4M3 code (saturating at 448), as uint8."""
    tab = _fp8_table()
    y = np.abs(np.asarray(x, np.float64))
    mid = (tab[1:] + tab[:-1]) / 2
    code = np.searchsorted(mid, np.minimum(y, 448.0), side="left").astype(np.uint8)
    return np.where(np.asarray(x) < 0, code | 0x80, code).astype(np.uint8)


def is16(dtype: str) -> bool:
    """16-bit types are stored as raw uint16 bit patterns."""
    return dtype in ("bf16", "f16")


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values (raw bits for 16-bit types) -> float32 (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float32)
    return a


def _normal(seed: int, stream: int, count: int, sigma: float, dtype: str) -> np.ndarray:
    """count N(0, sigma^2) draws, chunked and threaded; raw uint16 bits (16-bit types) or float32."""
    out = np.empty(count, dtype=np.uint16 if is16(dtype) else np.float32)
    nchunks = (count + _CHUNK - 1) // _CHUNK

    def job(c):
        lo = c * _CHUNK
        hi = min(count, lo + _CHUNK)
        x = _rng(seed, stream, c).standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[lo:hi] = _store(x, dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            job(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(job, range(nchunks)))
    return out


def _nan(dtype: str):
    return BF16_NAN if dtype == "bf16" else (F16_NAN if dtype == "f16" else F32_NAN)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)     # round to nearest even
    return x


# ----------------------------------------------------------------------------- trees
def expansion_tree(ks) -> tuple[np.ndarray, np.ndarray]:
    """Expansion config <k1..km>: every node at depth i-1 gets k_i children, BFS order."""
    parent, depth = [-1], [0]
    level = [0]
    for d, k in enumerate(ks, start=1):
        nxt = []
        for p in level:
            for _ in range(k):
                parent.append(p)
                depth.append(d)
                nxt.append(len(parent) - 1)
        level = nxt
    return np.array(parent, np.int32), np.array(depth, np.int32)


def _bfs_relabel(parent: list[int]) -> np.ndarray:
    """Relabel a parent list (parent index < child index not required) into BFS order."""
    n = len(parent)
    children = [[] for _ in range(n)]
    for v in range(1, n):
        children[parent[v]].append(v)
    order, head = [0], 0
    while head < len(order):
        order.extend(children[order[head]])
        head += 1
    new = {old: i for i, old in enumerate(order)}
    out = np.empty(n, np.int32)
    for old in order:
        out[new[old]] = -1 if old == 0 else new[parent[old]]
    return out


def merge_tree(rng: np.random.Generator, n: int, max_depth: int, drafts: int = 3, alphabet: int = 4):
    """Trie-merge of several drafts under a shared root.

    Each draft is a chain of length U{1..max_depth} whose tokens come from a small
    per-depth alphabet, so drafts share prefixes and merge.  Further drafts start
    at random nodes of depth < max_depth, round-robin over the draft sources,
    until exactly n nodes exist.  Returns BFS-ordered parent array.
    """
    parent, depth = [-1], [0]
    trie = {}
    first = True
    src = 0
    while len(parent) < n:
        if first or src < drafts:
            start = 0
        else:
            cands = [v for v in range(len(parent)) if depth[v] < max_depth]
            start = cands[rng.integers(len(cands))]
        length = int(rng.integers(1, max_depth - depth[start] + 1))
        cur = start
        for _ in range(length):
            if len(parent) >= n:
                break
            tok = int(rng.integers(alphabet))
            key = (cur, tok)
            if key not in trie:
                trie[key] = len(parent)
                parent.append(cur)
                depth.append(depth[cur] + 1)
            cur = trie[key]
        first = False
        src += 1
    return _bfs_relabel(parent)


def random_tree(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """Node u picks its parent uniformly among earlier nodes of depth < max_depth."""
    parent, depth = [-1], [0]
    for _ in range(1, n):
        cands = [v for v in range(len(parent)) if depth[v] < max_depth]
        p = cands[rng.integers(len(cands))]
        parent.append(p)
        depth.append(depth[p] + 1)
    return np.array(parent, np.int32)


def frontier_tree(rng: np.random.Generator, n: int, max_depth: int, bmin: int = 1, bmax: int = 5):
    """Repeatedly give a random childless node of depth < max_depth U{bmin..bmax} children.

    Nodes are numbered in creation order (a valid topological order that is not BFS).
    A draw whose frontier runs out before n nodes is redrawn; if 1000 draws all
    fall short (n out of reach at this depth), ValueError.
    """
    for _ in range(1000):
        parent, depth, nchild = [-1], [0], [0]
        while len(parent) < n:
            front = [v for v in range(len(parent)) if nchild[v] == 0 and depth[v] < max_depth]
            if not front:
                break
            p = front[rng.integers(len(front))]
            for _ in range(int(rng.integers(bmin, bmax + 1))):
                if len(parent) >= n:
                    break
                parent.append(p)
                depth.append(depth[p] + 1)
                nchild.append(0)
                nchild[p] += 1
        if len(parent) == n:
            return np.array(parent, np.int32)
    raise ValueError(f"frontier tree: {n} nodes not reached within depth {max_depth} in 1000 draws")


def depths_of(parent: np.ndarray) -> np.ndarray:
    """Depth of each node (root 0) for a parent array in topological order."""
    d = np.zeros(len(parent), np.int32)
    for v in range(1, len(parent)):
        d[v] = d[parent[v]] + 1
    return d


def make_tree(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    if cfg.tree.startswith("expand:"):
        return expansion_tree([int(k) for k in cfg.tree[7:].split(",")])[0]
    if cfg.tree == "merge":
        return merge_tree(rng, cfg.n, cfg.max_depth)
    if cfg.tree == "random":
        return random_tree(rng, cfg.n, cfg.max_depth)
    if cfg.tree == "frontier":
        return frontier_tree(rng, cfg.n, cfg.max_depth)
    if cfg.tree == "chain":
        return np.arange(-1, cfg.n - 1, dtype=np.int32)
    raise ValueError(cfg.tree)


def children_lists(parent: np.ndarray) -> list[list[int]]:
    ch = [[] for _ in range(len(parent))]
    for v in range(1, len(parent)):
        ch[parent[v]].append(v)
    return ch


# ----------------------------------------------------------------------------- workload
def make(cfg: Config, seed: int | None = None, *, variant: str = "plain", plant: bool = True,
         poison: bool = True, with_logits: bool = True, room: int = 0, kv_scale: float | None = None) -> dict:
    """Seeded inputs for one workload.

    variant:
      "plain"    Q, K, V, K_tree, V_tree ~ N(0,1).
      "balanced" Q and K_tree share a component a_b*e (e = first basis vector) so the
                 tree keys carry a large share of each row's softmax mass: a wrong mask
                 bit or a dropped prefix moves the output by far more than the bf16
                 tolerance.  a_b solves a^2 = sqrt(D)*(ln(L_b/|S|) + (a^2 + D/16)/(2D)).
      "needle"   one dominant prefix key at j = L_b - 1 (pins the prefix end).
      "ramp"     prefix scores rising by about 0.2 per key (Q and the prefix keys share
                 a first component that grows with the position): every 64-key tile
                 raises the row maximum far past any rescale threshold of an online
                 softmax.  "ramp_down": falling instead, so after the first tile every
                 tile's terms sit far below the running maximum.  16- or 32-bit caches.
    plant: planted accept paths, duplicate sibling tokens and logit ties (needs vocab).
    room: cache capacity kept free after each prefix, in tokens (NaN-filled), for
          committing accepted tokens; paged sequences get blocks for L_b + room tokens.
    kv_scale: with an fp8 cache, the scale of both K and V (default: per tensor,
          max |x| / 440).
    """
    seed = cfg.index if seed is None else seed
    dt = cfg.dtype
    B, n, Hq, Hkv, D = cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.D
    trng = _rng(seed, _S_TREE)
    parent = np.stack([make_tree(cfg, trng) for _ in range(B)]).astype(np.int32)
    depth = np.stack([depths_of(p) for p in parent]).astype(np.int32)

    lrng = _rng(seed, _S_LEN)
    if cfg.L_lo == cfg.L_hi:
        prefix_len = np.full(B, cfg.L_lo, np.int32)
    else:
        prefix_len = lrng.integers(cfg.L_lo, cfg.L_hi + 1, size=B).astype(np.int32)

    out = dict(cfg=cfg, seed=seed, variant=variant, parent=parent, depth=depth, prefix_len=prefix_len)

    # ---- queries and tree keys/values
    q = _normal(seed, _S_Q, B * n * Hq * D, 1.0, "f32").reshape(B, n, Hq, D)
    kt = _normal(seed, _S_KT, B * n * Hkv * D, 1.0, "f32").reshape(B, n, Hkv, D)
    vt = _normal(seed, _S_VT, B * n * Hkv * D, 1.0, "f32").reshape(B, n, Hkv, D)

    # ---- prefix cache
    tot_valid = int(prefix_len.sum())
    fp8 = cfg.kv == "fp8"
    kvals = _normal(seed, _S_K, tot_valid * Hkv * D, 1.0, "f32" if fp8 else dt)
    vvals = _normal(seed, _S_V, tot_valid * Hkv * D, 1.0, "f32" if fp8 else dt)
    if fp8:   # per-tensor scales: the largest magnitude maps near the top code (or a given scale)
        k_scale = kv_scale or max(float(np.abs(kvals).max()) / 440.0, 1e-30) if tot_valid else (kv_scale or 1.0)
        v_scale = kv_scale or max(float(np.abs(vvals).max()) / 440.0, 1e-30) if tot_valid else (kv_scale or 1.0)
        kvals = fp8_encode(kvals / k_scale)
        vvals = fp8_encode(vvals / v_scale)
        out.update(k_scale=np.float32(k_scale), v_scale=np.float32(v_scale))
    offs = np.concatenate([[0], np.cumsum(prefix_len.astype(np.int64))])
    edt = np.uint8 if fp8 else (np.uint16 if is16(dt) else np.float32)
    cnan = FP8_NAN if fp8 else _nan(dt)
    if cfg.paged:
        nblk = (prefix_len + room + PAGE - 1) // PAGE
        total_blocks = int(nblk.sum())
        max_blocks = (cfg.L_hi + room + PAGE - 1) // PAGE
        perm = _rng(seed, _S_PERM).permutation(total_blocks).astype(np.int32)
        bt = np.full((B, max_blocks), -1, np.int32)
        k_cache = np.full((total_blocks, Hkv, PAGE, D), cnan, edt)
        v_cache = np.full((total_blocks, Hkv, PAGE, D), cnan, edt)
        bo = 0
        for b in range(B):
            L = int(prefix_len[b])
            ids = perm[bo:bo + nblk[b]]
            bt[b, :nblk[b]] = ids
            bo += nblk[b]
            kv = kvals[offs[b] * Hkv * D:offs[b + 1] * Hkv * D].reshape(L, Hkv, D)
            vv = vvals[offs[b] * Hkv * D:offs[b + 1] * Hkv * D].reshape(L, Hkv, D)
            full = L // PAGE
            if full:
                k_cache[ids[:full]] = kv[:full * PAGE].reshape(full, PAGE, Hkv, D).transpose(0, 2, 1, 3)
                v_cache[ids[:full]] = vv[:full * PAGE].reshape(full, PAGE, Hkv, D).transpose(0, 2, 1, 3)
            rem = L - full * PAGE
            if rem:
                blk = ids[full]
                k_cache[blk, :, :rem, :] = kv[full * PAGE:].transpose(1, 0, 2)
                v_cache[blk, :, :rem, :] = vv[full * PAGE:].transpose(1, 0, 2)
        out.update(block_table=bt, max_blocks=max_blocks, num_blocks=total_blocks, Lmax=0)
    else:
        Lmax = max(cfg.capacity, (cfg.L_hi + room + PAGE - 1) // PAGE * PAGE)
        k_cache = np.full((B, Hkv, Lmax, D), cnan, edt)
        v_cache = np.full((B, Hkv, Lmax, D), cnan, edt)
        for b in range(B):
            L = int(prefix_len[b])
            kv = kvals[offs[b] * Hkv * D:offs[b + 1] * Hkv * D].reshape(L, Hkv, D)
            vv = vvals[offs[b] * Hkv * D:offs[b + 1] * Hkv * D].reshape(L, Hkv, D)
            k_cache[b, :, :L, :] = kv.transpose(1, 0, 2)
            v_cache[b, :, :L, :] = vv.transpose(1, 0, 2)
        out.update(block_table=None, max_blocks=0, num_blocks=0, Lmax=Lmax)
    del kvals, vvals
    if not poison:
        for c in (k_cache, v_cache):
            c[(c & 0x7F) == 0x7F if fp8 else np.isnan(to_f32(c, dt))] = 0

    # ---- variants (input shaping only)
    if variant == "balanced":
        vr = _rng(seed, _S_VAR)
        for b in range(B):
            L = int(prefix_len[b])
            s_mean = float((depth[b] + 1).mean())
            a2 = float(D) / 4
            for _ in range(60):
                a2 = math.sqrt(D) * (math.log(max(L, 1) / s_mean) + (a2 + D / 16) / (2 * D)) if L > 0 else 4.0
                a2 = max(a2, 1.0)
            a = math.sqrt(a2)
            q[b] = 0.25 * vr.standard_normal(q[b].shape).astype(np.float32)
            q[b, ..., 0] += a
            kt[b] = 0.25 * vr.standard_normal(kt[b].shape).astype(np.float32)
            kt[b, ..., 0] += a
    elif variant == "needle":
        for b in range(B):
            L = int(prefix_len[b])
            q[b] *= 0.5
            q[b, ..., 0] += 4.0
            if L == 0:
                continue
            kappa = (math.log(L) + 2.0) * math.sqrt(D) / 4.0
            j = L - 1
            row = np.zeros(D, np.float32)
            row[0] = kappa
            val = fp8_encode(row / out["k_scale"]) if fp8 else _store(row, dt)
            if cfg.paged:
                blk = out["block_table"][b, j // PAGE]
                k_cache[blk, :, j % PAGE, :] = val
            else:
                k_cache[b, :, j, :] = val
    elif variant in ("ramp", "ramp_down"):
        if fp8:
            raise ValueError("the ramp variants take a 16- or 32-bit cache")
        step = 0.2 * math.sqrt(D) / 4.0  # with q[..., 0] = 4: a score step of 0.2
        for b in range(B):
            L = int(prefix_len[b])
            q[b, ..., 0] = 4.0
            if L == 0:
                continue
            pos = np.arange(L) if variant == "ramp" else (L - 1 - np.arange(L))
            col = np.repeat((pos * step).astype(np.float32)[:, None], Hkv, axis=1)  # [L][Hkv]
            if cfg.paged:
                j = np.arange(L)
                k_cache[out["block_table"][b, j // PAGE], :, j % PAGE, 0] = _store(col, dt)
            else:
                k_cache[b, :, :L, 0] = _store(col.T, dt)
    elif variant != "plain":
        raise ValueError(variant)

    out.update(q=_store(q, dt), k_tree=_store(kt, dt), v_tree=_store(vt, dt), k_cache=k_cache, v_cache=v_cache)

    # ---- verification inputs
    if cfg.vocab and with_logits:
        V = cfg.vocab
        logits = _normal(seed, _S_LOGIT, B * n * V, cfg.logit_sigma, dt).reshape(B, n, V)
        tok_rng = _rng(seed, _S_TOK)
        tokens = np.zeros((B, n), np.int32)
        for b in range(B):
            for p, ch in enumerate(children_lists(parent[b])):
                if ch:  # distinct sibling tokens
                    tokens[b, ch] = tok_rng.choice(V, size=len(ch), replace=False)
        plan = []
        if plant:
            plan = _plant(cfg, parent, tokens, logits, _rng(seed, _S_PLANT))
        out.update(logits=logits, tokens=tokens, planted=plan)
    return out


def make_stochastic(cfg: Config, seed: int | None = None, *, ssm_noise: float = 1.0, w: dict | None = None) -> dict:
    """Inputs of stochastic verification for a workload with a vocabulary.

    LLM logits ~ N(0, logit_sigma) per node (as for greedy verification).  The SSM
    logits of node c are its parent's LLM logits plus N(0, ssm_noise) noise, so
    the draft distributions resemble the LLM's and acceptance is common but not
    certain.  Each draft token is drawn from its SSM row's softmax by inverse CDF
    with a uniform of its own, as a sampling draft model would.  Uniforms given
    to the verifier are multiples of 2^-24 in [0, 1), exact in float32 and
    float64.  Sequences are generated in parallel, each from its own stream.
    Returns the workload dict with ssm_logits, tokens, u_accept, u_sample added.
    """
    from concurrent.futures import ThreadPoolExecutor

    seed = cfg.index if seed is None else seed
    w = make(cfg, seed, plant=False) if w is None else w
    B, n, V, dt = cfg.B, cfg.n, cfg.vocab, cfg.dtype
    edt = np.uint16 if is16(dt) else np.float32
    ssm_st = np.empty((B, n, V), edt)
    tokens = np.zeros((B, n), np.int32)

    def one(b):
        rng = _rng(seed, _S_SSM, b)
        llm = to_f32(w["logits"][b], dt)
        par = np.maximum(w["parent"][b], 0)
        row = llm[par] + rng.standard_normal((n, V), dtype=np.float32) * np.float32(ssm_noise)
        row[0] = 0.0                                 # the root has no draft distribution
        ssm_st[b] = _store(row, dt)
        rf = to_f32(ssm_st[b], dt)
        e = np.exp((rf - rf.max(axis=1, keepdims=True)).astype(np.float64))
        cdf = np.cumsum(e, axis=1)
        u = rng.random(n) * cdf[:, -1]
        tokens[b] = [min(int(np.searchsorted(cdf[v], u[v], side="right")), V - 1) for v in range(n)]

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(one, range(B)))
    tokens[:, 0] = 0
    urng = _rng(seed, _S_UNIF)
    u_acc = (urng.integers(0, 1 << 24, size=(B, n)) / float(1 << 24)).astype(np.float32)
    u_smp = (urng.integers(0, 1 << 24, size=(B, n)) / float(1 << 24)).astype(np.float32)
    out = dict(w)
    out.update(ssm_logits=ssm_st, tokens=tokens, u_accept=u_acc, u_sample=u_smp)
    return out


def _plant(cfg: Config, parent, tokens, logits, rng) -> list:
    """Plant accept paths, duplicate sibling tokens and logit ties.

    Only inputs are edited: a planted edge (p -> c) sets logits[p][t] to a value no
    random draw reaches and tokens[c] = t.  What the method then accepts is left to
    the oracle and the kernels.
    """
    big = 32.0 if cfg.dtype == "bf16" else 16.0   # beyond any draw, exact in the stored type
    V = cfg.vocab
    bigv = _store(np.array([big], np.float32), cfg.dtype)[0]
    records = []
    for b in range(cfg.B):
        ch = children_lists(parent[b])
        # a random root->leaf path, followed to a random stopping depth
        path = [0]
        while ch[path[-1]]:
            path.append(ch[path[-1]][rng.integers(len(ch[path[-1]]))])
        stop = int(rng.integers(1, len(path))) if len(path) > 1 else 0
        rec = dict(b=b, path=path[:stop + 1], dup=None, tie=None)
        for i in range(1, stop + 1):
            p, c = path[i - 1], path[i]
            t = int(tokens[b, c])
            logits[b, p, t] = bigv
            # equal-valued decoy at a higher vocab index: the lower one must win
            if t + 1 < V and rng.random() < 0.5:
                logits[b, p, min(V - 1, t + 1 + int(rng.integers(V - t - 1)))] = bigv
        # duplicate sibling token on the path (lowest node index must win)
        for i in range(1, stop + 1):
            sib = [s for s in ch[path[i - 1]] if s != path[i]]
            if sib and rng.random() < 0.6:
                s = sib[rng.integers(len(sib))]
                tokens[b, s] = tokens[b, path[i]]
                rec["dup"] = (path[i], s)
                break
        # a tie at the stopping node where the lower index is not a draft token
        end = path[stop]
        if ch[end] and rng.random() < 0.5:
            c = ch[end][0]
            t = int(tokens[b, c])
            if t > 0:
                lo = int(rng.integers(t))
                logits[b, end, lo] = bigv
                logits[b, end, t] = bigv
                rec["tie"] = (end, lo, t)
        records.append(rec)
    return records


def reference_bytes(w: dict) -> dict:
    """Algorithmic byte and flop counts of one pass over this workload."""
    cfg = w["cfg"]
    es = 2 if is16(cfg.dtype) else 4
    L = w["prefix_len"].astype(np.int64)
    n, Hq, Hkv, D, B = cfg.n, cfg.Hq, cfg.Hkv, cfg.D, cfg.B
    kv_prefix = int(L.sum()) * Hkv * D * 2 * (1 if cfg.kv == "fp8" else es)
    kv_tree = B * n * Hkv * D * 2 * es
    q_o = 2 * B * n * Hq * D * es
    masks = B * n * ((n + 63) // 64) * 8
    s_sum = int((w["depth"] + 1).sum())
    flops_prefix = 4 * n * Hq * D * int(L.sum())
    flops_tree = 4 * Hq * D * s_sum
    logits = B * n * cfg.vocab * es if cfg.vocab else 0
    return dict(attn_bytes=kv_prefix + kv_tree + q_o + masks, prefix_kv_bytes=kv_prefix,
                attn_flops=flops_prefix + flops_tree, verify_bytes=logits, ancestor_pairs=s_sum)
