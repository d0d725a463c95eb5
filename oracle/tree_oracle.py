"""CPU oracle for tree attention and greedy token-tree verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

It is the plain definition of what the hot path computes, in float64 NumPy,
from the stored input values (bf16 -> float64 and fp32 -> float64 are exact):

* tree_build: S_u, the set of tokens on the path from the root to node u
  (both ends included), found by walking u's parent chain, written as a
  per-node ancestor bitmask; position id = prefix length + depth.
  (SpecInfer explainer, section on the token-tree structure, where S_u is
  defined; section on kernel fusion, item on the precomputed topology mask.)
* tree_attention: for each node u and query head h,
  softmax(Q_u K^T / sqrt(d_k)) V over the keys of the shared prefix plus
  exactly the nodes of S_u, as ONE softmax over that union.
  (Same explainer, the attention equation of the token-tree section; the
  contributions list says the mask is consistent with KV-cache reuse, so the
  cached prefix is attended too.)
* verify_greedy: per-node argmax of the logits (lowest index on ties), then
  the walk from the root that accepts a child whose draft token equals the
  argmax at its parent (lowest node index among equal draft tokens), stopping
  at the first node with no such child; the argmax there is the bonus token.
  (Explainer: greedy verification is named in the tree-verification section;
  the accept-up-to-first-mismatch-plus-one-target-token rule is the sequence
  case on the speculative-decoding explainer, technical mechanism section, and
  on the speculative-decoding operations guide's diagram, applied per branch.)
* verify_stochastic: multi-step speculative sampling over the tree.  At the
  current node the LLM distribution p (softmax of its logits) is compared with
  each child c in node-id order: c's draft token x was drawn from q_c (softmax
  of c's SSM logits) and is accepted with probability min(1, p(x)/q_c(x)),
  i.e. iff u_c * q_c(x) < p(x) for c's uniform u_c in [0, 1); on rejection p
  becomes the normalised residual max(0, p - q_c) and the next child is tried
  against it.  An accepted child becomes the current node.  When every child
  is rejected (or there is none) one token is drawn from p by inverse CDF with
  the node's second uniform: the smallest y whose cumulative mass exceeds it.
  (Explainer, tree-verification section: the acceptance probability and the
  normalised residual equations, and the statement that the scheme samples
  exactly from the LLM's distribution.)  The uniforms are inputs.
* topk_lowest, expand_topk: the expansion-based construction step: each
  frontier node gets as children the k tokens of its SSM logits row with the
  largest values (ties to the lower token id), numbered after the existing
  nodes in (frontier order, rank) order.  (Explainer, multi-draft section: one
  SSM proposes its top-k tokens at each step and the tree grows in depth,
  configuration <k1, ..., km>.)
* merge_drafts: the merge-based construction: each draft token sequence is
  inserted from the root, reusing the child with the same token where one
  exists and creating one otherwise, drafts in order; node ids follow
  creation.  (Explainer, multi-draft section: the outputs of several SSMs are
  merged into one token tree, as in its figure.)
* commit_kv: the keys and values of the accepted root path become ordinary
  prefix tokens: path node t goes to cache position L_b + t, so the cache
  again holds one linear sequence and the next step attends it like any
  prefix.  (Explainer, kernel-fusion section, item on depth-first traversal
  keeping the tree consistent with the existing KV cache; "practical
  applications" section on PagedAttention's block-wise KV memory, which gives
  the paged layout.)

Layouts are those of include/tree_verify.h.  No blocking, fusion or reordering
is done beyond vectorising the prefix scores of all rows of a KV head, which
every node attends identically.
"""
from __future__ import annotations

import numpy as np

TV_OK = 0
TV_EINVAL = 1
TV_ETOPOLOGY = 2
PAGE = 16


# ----------------------------------------------------------------------------- values
def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64.  bf16 and f16 arrays are raw uint16 bit patterns."""
    if dtype == "bf16":
        return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "fp8":
        return fp8_e4m3_value(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def fp8_e4m3_value(codes) -> np.ndarray:
    """Values of OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal; S.1111.111 is NaN; no infinities)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def cache_values(w: dict, which: str, rows) -> np.ndarray:
    """float64 values of cache rows: the stored element type, or fp8 codes times the
    cache's scale when the cache is fp8."""
    if w["cfg"].kv == "fp8":
        return fp8_e4m3_value(rows) * float(w["k_scale" if which == "k" else "v_scale"])
    return to_f64(rows, w["cfg"].dtype)


# ----------------------------------------------------------------------------- topology
def validate_tree(parent: np.ndarray, depth: np.ndarray) -> bool:
    """Single root at node 0, every other node's parent precedes it, depths agree."""
    n = len(parent)
    if n < 1 or parent[0] != -1 or depth[0] != 0:
        return False
    for u in range(1, n):
        p = int(parent[u])
        if not (0 <= p < u):
            return False
        if depth[u] != depth[p] + 1:
            return False
    return True


def ancestors(parent: np.ndarray, u: int) -> list[int]:
    """S_u: node u and every node on its parent chain up to the root."""
    out = []
    v = u
    while v != -1:
        out.append(v)
        v = int(parent[v])
    return out


def tree_build(parent: np.ndarray, depth: np.ndarray, prefix_len: np.ndarray):
    """(mask [B][n][W] uint64, pos [B][n] int32, status [B] int32).

    Bit v of word v>>6 (least significant bit first) of mask[b][u] is set iff
    v is in S_u.  Rows of a sequence whose topology is invalid are left zero and
    its status is TV_ETOPOLOGY.
    """
    parent = np.asarray(parent)
    B, n = parent.shape
    W = (n + 63) // 64
    mask = np.zeros((B, n, W), np.uint64)
    pos = np.zeros((B, n), np.int32)
    status = np.zeros(B, np.int32)
    for b in range(B):
        if not validate_tree(parent[b], depth[b]):
            status[b] = TV_ETOPOLOGY
            continue
        for u in range(n):
            for v in ancestors(parent[b], u):
                mask[b, u, v >> 6] |= np.uint64(1) << np.uint64(v & 63)
            pos[b, u] = int(prefix_len[b]) + int(depth[b, u])
    return mask, pos, status


# ----------------------------------------------------------------------------- prefix gather
def gather_prefix(k_cache, v_cache, b: int, g: int, L: int, *, paged: bool, block_table=None):
    """Keys and values of prefix tokens 0..L-1 of sequence b, KV head g, as [L][D] arrays.

    contiguous: K, V [B][Hkv][Lmax][D]
    paged:      token j lives in block block_table[b][j // 16], slot j % 16;
                K, V [blocks][Hkv][16][D]
    """
    if not paged:
        return k_cache[b, g, :L, :], v_cache[b, g, :L, :]
    j = np.arange(L)
    blk = np.asarray(block_table)[b, j // PAGE]
    slot = j % PAGE
    return k_cache[blk, g, slot, :], v_cache[blk, g, slot, :]


# ----------------------------------------------------------------------------- attention
def tree_attention(w: dict, seqs=None, kv_heads=None, scale: float | None = None):
    """Tree attention of workload dict ``w`` (see workloads.make) in float64.

    Returns (O [B][n][Hq][D], lse [B][n][Hq]) as float64; entries of sequences or
    KV heads not selected are NaN.
    """
    cfg = w["cfg"]
    dt = cfg.dtype
    B, n, Hq, Hkv, D = cfg.B, cfg.n, cfg.Hq, cfg.Hkv, cfg.D
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    seqs = range(B) if seqs is None else seqs
    kv_heads = range(Hkv) if kv_heads is None else kv_heads
    O = np.full((B, n, Hq, D), np.nan)
    LSE = np.full((B, n, Hq), np.nan)
    parent = w["parent"]
    for b in seqs:
        L = int(w["prefix_len"][b])
        # A[u][v] = 1 iff tree node v is in S_u (parent-chain walk)
        A = np.zeros((n, n), bool)
        for u in range(n):
            A[u, ancestors(parent[b], u)] = True
        for g in kv_heads:
            Kp, Vp = gather_prefix(w["k_cache"], w["v_cache"], b, g, L, paged=cfg.paged,
                                   block_table=w.get("block_table"))
            Kp, Vp = cache_values(w, "k", Kp), cache_values(w, "v", Vp)
            Kt = to_f64(w["k_tree"][b, :, g, :], dt)            # [n][D]
            Vt = to_f64(w["v_tree"][b, :, g, :], dt)
            heads = range(g * G, (g + 1) * G)
            Q = to_f64(w["q"][b][:, heads, :], dt)              # [n][G][D]
            Qr = Q.reshape(n * G, D)
            s_pre = (Qr @ Kp.T) * scale                         # every node sees the whole prefix
            s_tree = (Qr @ Kt.T) * scale
            s_tree = np.where(np.repeat(A, G, axis=0), s_tree, -np.inf)
            s = np.concatenate([s_pre, s_tree], axis=1)         # one softmax over prefix U S_u
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            o = (p @ np.concatenate([Vp, Vt], axis=0)) / l
            O[b][:, heads, :] = o.reshape(n, G, D)
            LSE[b][:, heads] = (m + np.log(l)).reshape(n, G)
    return O, LSE


# ----------------------------------------------------------------------------- verification
def argmax_lowest(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Index of the largest value of each row; ties go to the lowest index.

    Values are compared as numbers (-0 equals +0).  NaN inputs are out of contract.
    """
    shp = logits.shape
    rows = logits.reshape(-1, shp[-1])
    out = np.empty(rows.shape[0], np.int64)
    for r0 in range(0, rows.shape[0], 64):
        x = to_f64(rows[r0:r0 + 64], dtype)
        m = x.max(axis=1, keepdims=True)
        hit = x == m
        out[r0:r0 + 64] = hit.argmax(axis=1)   # first True = lowest index
    return out.reshape(shp[:-1]).astype(np.int32)


def accept_walk(am: np.ndarray, tokens: np.ndarray, parent: np.ndarray):
    """Greedy walk of one sequence: (path list of node ids, root first; bonus token)."""
    n = len(parent)
    path = [0]
    cur = 0
    while True:
        hits = [v for v in range(n) if parent[v] == cur and tokens[v] == am[cur]]
        if not hits:
            break
        cur = min(hits)
        path.append(cur)
    return path, int(am[cur])


def verify_greedy(logits: np.ndarray, tokens: np.ndarray, parent: np.ndarray, dtype: str):
    """(argmax [B][n], path [B][n] -1 padded, path_len [B], bonus [B]) as int32."""
    B, n = tokens.shape
    am = argmax_lowest(logits, dtype)
    path = np.full((B, n), -1, np.int32)
    plen = np.zeros(B, np.int32)
    bonus = np.zeros(B, np.int32)
    for b in range(B):
        p, bo = accept_walk(am[b], tokens[b], parent[b])
        path[b, :len(p)] = p
        plen[b] = len(p)
        bonus[b] = bo
    return am, path, plen, bonus


def softmax64(row: np.ndarray, dtype: str) -> np.ndarray:
    """softmax of one stored logits row, in float64 (-inf logits get probability 0)."""
    x = to_f64(row, dtype)
    m = x.max()
    e = np.exp(x - m)
    return e / e.sum()


def mss_accepts(u: float, q: np.ndarray, p: np.ndarray, x: int):
    """The acceptance test of draft token x: (accepted?, lhs, rhs) with accepted = lhs < rhs.

    u < min(1, p(x)/q(x)) written without the division: u * q(x) < p(x), which
    also covers q(x) == 0 (accepted iff p(x) > 0).
    """
    lhs, rhs = u * q[x], p[x]
    return lhs < rhs, lhs, rhs


def mss_residual(p: np.ndarray, q: np.ndarray):
    """The distribution after a rejection: norm(max(0, p - q)); p itself if that is all zero.
    Returns (new p, residual mass)."""
    r = np.maximum(0.0, p - q)
    tot = r.sum()
    return (r / tot if tot > 0 else p), tot


def mss_draw(p: np.ndarray, u: float):
    """Inverse-CDF draw: the smallest y with cdf(y) > u (the last y with p(y) > 0 if
    rounding leaves u >= cdf(V-1)).  Returns (y, cdf(y-1), cdf(y))."""
    cdf = np.cumsum(p)
    hit = np.nonzero(cdf > u)[0]
    y = int(hit[0]) if len(hit) else int(np.nonzero(p > 0)[0][-1])
    return y, (cdf[y - 1] if y > 0 else 0.0), cdf[y]


def mss_walk(logits, ssm_logits, tokens, parent, u_acc, u_smp, dtype):
    """Stochastic verification of one sequence's tree.

    logits, ssm_logits [n][V] stored values; tokens, parent, u_acc, u_smp [n].
    Returns (path, bonus, decisions): path = accepted node ids, root first;
    bonus = the token drawn at the last node; decisions = every comparison the
    walk made, as (lhs, rhs) pairs of a test lhs < rhs (a residual mass appears
    as (0, mass)), for callers that need to know how close each decision was.
    """
    n = len(parent)
    cur, path, decisions = 0, [0], []
    while True:
        p = softmax64(logits[cur], dtype)
        moved = False
        for c in [v for v in range(n) if parent[v] == cur]:     # children in node-id order
            q = softmax64(ssm_logits[c], dtype)
            ok, lhs, rhs = mss_accepts(float(u_acc[c]), q, p, int(tokens[c]))
            decisions.append((lhs, rhs))
            if ok:
                cur = c
                path.append(c)
                moved = True
                break
            p, tot = mss_residual(p, q)
            decisions.append((0.0, tot))
        if not moved:
            break
    u = float(u_smp[cur])
    bonus, lo, hi = mss_draw(p, u)
    decisions.append((lo, u))                   # the draw: cdf(y-1) <= u < cdf(y)
    decisions.append((u, hi))
    return path, bonus, decisions


def verify_stochastic(logits, ssm_logits, tokens, parent, u_acc, u_smp, dtype):
    """Batched mss_walk: (path [B][n] -1 padded, path_len [B], bonus [B], status [B], decisions
    list per sequence).  A sequence whose parent array is not topological with root 0, or
    with a draft token outside [0, V), gets status TV_EINVAL, path_len 0 and bonus -1."""
    B, n = tokens.shape
    V = logits.shape[-1]
    path = np.full((B, n), -1, np.int32)
    plen = np.zeros(B, np.int32)
    bonus = np.full(B, -1, np.int32)
    status = np.full(B, TV_OK, np.int32)
    dec = []
    for b in range(B):
        par, tok = parent[b], tokens[b]
        if par[0] != -1 or any(not (0 <= par[v] < v) or not (0 <= tok[v] < V) for v in range(1, n)):
            status[b] = TV_EINVAL                 # not a tree in topological order, or a token outside the vocab
            dec.append([])
            continue
        p, bo, d = mss_walk(logits[b], ssm_logits[b], tokens[b], parent[b], u_acc[b], u_smp[b], dtype)
        path[b, :len(p)] = p
        plen[b] = len(p)
        bonus[b] = bo
        dec.append(d)
    return path, plen, bonus, status, dec


# ----------------------------------------------------------------------------- tree construction
def topk_lowest(row: np.ndarray, k: int, dtype: str):
    """The k largest entries of one row, largest first, ties to the lower index:
    (indices, values) as int32 / float64."""
    x = to_f64(row, dtype)
    order = np.lexsort((np.arange(len(x)), -x))   # primary key: value descending; then index ascending
    sel = order[:k]
    return sel.astype(np.int32), x[sel]


def expand_topk(parent, depth, tokens, n_cur, frontier, ssm_logits, k: int, n_max: int, dtype: str):
    """One expansion step for a batch.

    parent, depth, tokens [B][n_max] (entries u < n_cur[b] hold the tree);
    frontier [B][F] node ids (-1 = unused slot); ssm_logits [B][F][V].
    Frontier entry f (the r-th valid one) gets children n_cur + r*k + j, j < k,
    with the j-th largest token of its row.  A sequence with a frontier id
    outside [0, n_cur), or n_cur outside [1, n_max], or more than n_max nodes
    after the step, is left unchanged with status TV_EINVAL.
    Returns (parent, depth, tokens, scores, n_new, status); scores [B][n_max]
    holds the chosen logits at the new nodes (NaN elsewhere).
    """
    parent, depth, tokens = parent.copy(), depth.copy(), tokens.copy()
    B, F = frontier.shape
    scores = np.full(parent.shape, np.nan)
    n_new = np.asarray(n_cur, np.int32).copy()
    status = np.full(B, TV_OK, np.int32)
    for b in range(B):
        nc = int(n_cur[b])
        valid = [f for f in range(F) if frontier[b][f] >= 0]
        if not (1 <= nc <= n_max) or any(frontier[b][f] >= nc for f in valid) or nc + len(valid) * k > n_max:
            status[b] = TV_EINVAL
            continue
        for r, f in enumerate(valid):
            p = int(frontier[b][f])
            idx, val = topk_lowest(ssm_logits[b][f], k, dtype)
            for j in range(k):
                u = nc + r * k + j
                parent[b][u] = p
                depth[b][u] = depth[b][p] + 1
                tokens[b][u] = idx[j]
                scores[b][u] = val[j]
        n_new[b] = nc + len(valid) * k
    return parent, depth, tokens, scores, n_new, status


def merge_drafts(drafts, draft_len, root_token, n_max: int):
    """Merge draft token sequences into one token tree per sequence (a trie).

    drafts [B][M][Ld] int32, draft_len [B][M]; root_token [B] (the token of node 0).
    Returns (parent, depth, tokens [B][n_max] with -1 past the tree, n [B],
    node_of [B][M][Ld] = node id of each draft position (-1 past its length),
    status [B]).  A sequence with a length outside [0, Ld], or needing more than
    n_max nodes, gets status TV_EINVAL, n = 0 and -1 everywhere.
    """
    B, M, Ld = drafts.shape
    parent = np.full((B, n_max), -1, np.int32)
    depth = np.full((B, n_max), -1, np.int32)
    tokens = np.full((B, n_max), -1, np.int32)
    node_of = np.full((B, M, Ld), -1, np.int32)
    n = np.zeros(B, np.int32)
    status = np.full(B, TV_OK, np.int32)
    for b in range(B):
        if any(not (0 <= draft_len[b][m] <= Ld) for m in range(M)):
            status[b] = TV_EINVAL
            continue
        par, dep, tok = [-1], [0], [int(root_token[b])]
        child = {}                                # (parent node, token) -> node
        where = np.full((M, Ld), -1, np.int32)
        for m in range(M):
            cur = 0
            for d in range(int(draft_len[b][m])):
                key = (cur, int(drafts[b][m][d]))
                if key not in child:
                    child[key] = len(par)
                    par.append(cur)
                    dep.append(d + 1)
                    tok.append(key[1])
                cur = child[key]
                where[m][d] = cur
        if len(par) > n_max:
            status[b] = TV_EINVAL
            continue
        n[b] = len(par)
        parent[b, :n[b]] = par
        depth[b, :n[b]] = dep
        tokens[b, :n[b]] = tok
        node_of[b] = where
    return parent, depth, tokens, n, node_of, status


# ----------------------------------------------------------------------------- KV commit
def cache_index(w: dict, b: int, j: int):
    """Index of token j of sequence b in a cache array: selects its [Hkv][D] rows."""
    if w["cfg"].paged:
        return (int(w["block_table"][b][j // PAGE]), slice(None), j % PAGE)
    return (b, slice(None), j)


def commit_kv(w: dict, path: np.ndarray, path_len: np.ndarray):
    """Append the accepted path's tree keys/values to each sequence's cache.

    Sequence b with prefix length L and P = path_len[b] accepted nodes gets
    k_tree[b][path[b][t]] (all KV heads) at cache position L + t for t < P;
    its new length is L + P.  A sequence is rejected as a whole (status
    TV_EINVAL, cache untouched, new length L) if P is outside [0, n], a path
    entry t < P is outside [0, n), L + P exceeds the capacity, or (paged) a
    block id covering positions L..L+P-1 is outside [0, num_blocks).

    Returns (k_cache, v_cache, new_len [B], status [B]); the caches are copies.
    """
    cfg = w["cfg"]
    B, n = cfg.B, cfg.n
    kc, vc = w["k_cache"].copy(), w["v_cache"].copy()
    plen = np.asarray(w["prefix_len"])
    new_len = plen.astype(np.int32).copy()
    status = np.full(B, TV_OK, np.int32)
    if cfg.paged:
        bt = np.asarray(w["block_table"])
        cap = w["max_blocks"] * PAGE
    else:
        cap = w["Lmax"]
    for b in range(B):
        L, P = int(plen[b]), int(path_len[b])
        ok = 0 <= L and 0 <= P <= n and L + P <= cap
        ok = ok and all(0 <= int(path[b][t]) < n for t in range(P))
        if ok and cfg.paged:
            ok = all(0 <= int(bt[b, j // PAGE]) < w["num_blocks"] for j in range(L, L + P))
        if not ok:
            status[b] = TV_EINVAL
            continue
        for t in range(P):
            at = cache_index(w, b, L + t)
            kc[at] = w["k_tree"][b, int(path[b][t])]
            vc[at] = w["v_tree"][b, int(path[b][t])]
        new_len[b] = L + P
    return kc, vc, new_len, status
