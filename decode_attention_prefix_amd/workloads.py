"""Seeded synthetic inputs for shared-prefix decode attention.

This module builds radix trees, request paths, bf16 Q/K/V values and the
paged KV pools that both the HIP path and the CPU oracle read.  It holds no
attention arithmetic: no dot products, no softmax, no merge.  Its only
numeric work is drawing N(0,1) values and rounding them to bfloat16
(round-to-nearest-even on the bit pattern).

The setting follows the Capillary Kernels project page (abstract, first
paragraph): several decode requests share context prefixes through a
radix-tree KV cache, so one tree node's KV serves every request whose
root-to-leaf path passes through it.  The pages name no dataset for this
path; the five shapes below are synthetic stand-ins with the head counts of
one Llama-3-8B-like layer (32 q / 8 KV heads, head_dim 128) and one
70B-like layer (64 q / 8 KV heads).

Paged layout (shared with the kernels and the oracle as a data format,
implemented independently by each):

* page size P = 16 tokens; every node starts on a fresh page and owns
  ceil(tokens / 16) pages; the last page of a node may be partial.
* K pool, bf16 bits, shape [pool_pages][Hkv][D/8][P][8]: token slot t,
  dim d of one (page, KV head) block sits at ((d // 8) * P + t) * 8 + d % 8.
  Sixteen tokens' 16-byte pieces of one 8-dim chunk are contiguous.
* V pool, bf16 bits, shape [pool_pages][Hkv][D][P]: element (t, d) of a
  block sits at d * P + t, i.e. tokens are contiguous for each dim.
* Q, bf16 bits, shape [R][Hq][D].
* Slots past a node's last valid token, and pool pages owned by no node,
  hold ``tail_fill`` (NaN by default, so an unmasked read shows up).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

PAGE = 16
BF16_NAN = np.uint16(0x7FC0)

__all__ = [
    "PAGE", "Tree", "Workload", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "tree_from_lengths", "make_config", "make_random_tree", "make_workload",
    "control_workload", "CONFIG_NAMES", "tree_stats", "free_pages", "grow_tree",
    "write_new_tokens", "ROW_KINDS", "make_rows",
]

CONFIG_NAMES = {
    0: "tiny: root 256 shared by 4 requests, 4 x 64-token suffixes, 8q/2kv, D=64",
    1: "shared system prompt: 4096-token root, 64 suffixes U[256,1024], 32q/8kv, D=128",
    2: "two-level tree: 8192 root, 8 x 2048 children, 16 leaves each U[256,2048], 32q/8kv, D=128",
    3: "long shared doc: 32768 root, 32 suffixes U[1024,4096], 64q/8kv, D=128",
    4: "random radix tree: depth 1-4, branching U[1,8], lengths geometric mean 1024 (min 16), 256 leaves, 32q/8kv, D=128",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Tree:
    """Host description of a paged radix tree plus the requests' paths.

    parent[i] < i for every non-root node (roots have -1); a request's path
    lists node ids from a root down to the node where its context ends.
    """
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    parent: np.ndarray          # int32 [N]
    num_tokens: np.ndarray      # int32 [N]
    page_offsets: np.ndarray    # int64 [N+1]
    page_ids: np.ndarray        # int32 [total pages]
    path_offsets: np.ndarray    # int32 [R+1]
    path_nodes: np.ndarray      # int32 [sum of path lengths]
    num_pool_pages: int
    sm_scale: float
    page_size: int = PAGE

    @property
    def num_nodes(self) -> int:
        return int(self.parent.shape[0])

    @property
    def num_requests(self) -> int:
        return int(self.path_offsets.shape[0] - 1)

    def path(self, r: int) -> np.ndarray:
        return self.path_nodes[self.path_offsets[r]:self.path_offsets[r + 1]]

    def context_len(self, r: int) -> int:
        return int(self.num_tokens[self.path(r)].sum())


@dataclass
class Workload:
    tree: Tree
    q: np.ndarray               # uint16 [R][Hq][D]
    k_pool: np.ndarray          # uint16 [pool][Hkv][D/8][P][8]
    v_pool: np.ndarray          # uint16 [pool][Hkv][D][P]
    k_tokens: Optional[np.ndarray] = None   # uint16 [sum tokens][Hkv][D], node order
    v_tokens: Optional[np.ndarray] = None
    token_offsets: Optional[np.ndarray] = None  # int64 [N+1] into *_tokens
    meta: dict = field(default_factory=dict)


def tree_from_lengths(num_tokens: Sequence[int], parent: Sequence[int],
                      paths: Sequence[Sequence[int]], num_q_heads: int,
                      num_kv_heads: int, head_dim: int,
                      sm_scale: Optional[float] = None,
                      page_perm_rng: Optional[np.random.Generator] = None,
                      extra_pool_pages: int = 0) -> Tree:
    """Give each node ceil(len/16) pages; optionally permute physical pages."""
    nt = np.asarray(num_tokens, dtype=np.int32)
    par = np.asarray(parent, dtype=np.int32)
    npg = (nt.astype(np.int64) + PAGE - 1) // PAGE
    offs = np.zeros(nt.shape[0] + 1, dtype=np.int64)
    np.cumsum(npg, out=offs[1:])
    total = int(offs[-1])
    pool = total + int(extra_pool_pages)
    if page_perm_rng is not None:
        ids = page_perm_rng.permutation(pool)[:total].astype(np.int32)
    else:
        ids = np.arange(total, dtype=np.int32)
    poffs = np.zeros(len(paths) + 1, dtype=np.int32)
    np.cumsum([len(p) for p in paths], out=poffs[1:])
    pn = np.asarray([n for p in paths for n in p], dtype=np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / float(np.sqrt(head_dim))
    return Tree(num_q_heads, num_kv_heads, head_dim, par, nt, offs, ids,
                poffs, pn, pool, float(sm_scale))


def _config_shape(cfg: int, rng: np.random.Generator):
    """Return (num_tokens, parent, paths, Hq, Hkv, D) for one of the five shapes."""
    if cfg == 0:
        nt = [256] + [64] * 4
        par = [-1] + [0] * 4
        paths = [[0, i] for i in range(1, 5)]
        return nt, par, paths, 8, 2, 64
    if cfg == 1:
        suf = rng.integers(256, 1024, size=64, endpoint=True)
        nt = [4096] + [int(x) for x in suf]
        par = [-1] + [0] * 64
        paths = [[0, i] for i in range(1, 65)]
        return nt, par, paths, 32, 8, 128
    if cfg == 2:
        nt, par, paths = [8192], [-1], []
        kids = []
        for _ in range(8):
            kids.append(len(nt)); nt.append(2048); par.append(0)
        suf = rng.integers(256, 2048, size=128, endpoint=True)
        for ci, c in enumerate(kids):
            for j in range(16):
                nid = len(nt); nt.append(int(suf[ci * 16 + j])); par.append(c)
                paths.append([0, c, nid])
        return nt, par, paths, 32, 8, 128
    if cfg == 3:
        suf = rng.integers(1024, 4096, size=32, endpoint=True)
        nt = [32768] + [int(x) for x in suf]
        par = [-1] + [0] * 32
        paths = [[0, i] for i in range(1, 33)]
        return nt, par, paths, 64, 8, 128
    if cfg == 4:
        return (*_random_radix(rng, leaves=256), 32, 8, 128)
    raise ValueError(f"unknown config {cfg}")


def _random_radix(rng: np.random.Generator, leaves: int, max_depth: int = 4,
                  max_branch: int = 8, mean_len: int = 1024, min_len: int = 16):
    """Random radix tree: an empty sentinel root, then top-level subtrees.

    Each top-level subtree draws a depth in 1..max_depth; a node at that
    depth is a leaf (one request ends there); any other node draws a
    branching factor in 1..max_branch and creates its children while fewer
    than ``leaves`` leaves exist (the first child always).  Node lengths are
    max(min_len, Geometric(p = 1/mean_len)).
    """
    nt, par, paths = [0], [-1], []

    def grow(depth, dmax, parent_id, prefix):
        length = max(min_len, int(rng.geometric(1.0 / mean_len)))
        nid = len(nt); nt.append(length); par.append(parent_id)
        path = prefix + [nid]
        if depth == dmax:
            paths.append(path)
            return
        b = int(rng.integers(1, max_branch, endpoint=True))
        for i in range(b):
            if i > 0 and len(paths) >= leaves:
                break
            grow(depth + 1, dmax, nid, path)

    while len(paths) < leaves:
        dmax = int(rng.integers(1, max_depth, endpoint=True))
        grow(1, dmax, 0, [0])
    return nt, par, paths


def make_random_tree(rng: np.random.Generator, num_requests: int, max_depth: int,
                     max_len: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, min_len: int = 1, internal_end_prob: float = 0.0,
                     empty_root: bool = False):
    """Small random trees for tests: arbitrary lengths (not page multiples),
    requests that may end at internal nodes, optional empty sentinel root."""
    nt, par, paths = [], [], []
    if empty_root:
        nt.append(0); par.append(-1)
    while len(paths) < num_requests:
        # walk down from a root, creating or reusing nodes
        cur = 0 if empty_root else -1
        path = [0] if empty_root else []
        depth = int(rng.integers(1, max_depth, endpoint=True))
        for d in range(depth):
            kids = [i for i in range(len(nt)) if par[i] == cur]
            if kids and rng.random() < 0.6:
                nid = int(kids[rng.integers(0, len(kids))])
            else:
                nid = len(nt); nt.append(int(rng.integers(min_len, max_len, endpoint=True)))
                par.append(cur)
            path.append(nid)
            cur = nid
            if d < depth - 1 and rng.random() < internal_end_prob:
                break
        if sum(nt[n] for n in path) == 0:
            continue
        paths.append(path)
    return nt, par, paths


def make_workload(num_tokens, parent, paths, num_q_heads, num_kv_heads, head_dim,
                  rng: np.random.Generator, sm_scale: Optional[float] = None,
                  permute_pages: bool = True, tail_fill: str = "nan",
                  extra_pool_pages: int = 0, keep_tokens: bool = True,
                  q_values=None, k_values=None, v_values=None) -> Workload:
    """Draw Q, then K, then V (N(0,1) rounded to bf16) and pack the pools.

    ``k_values``/``v_values`` (float arrays [sum tokens][Hkv][D] in node order)
    and ``q_values`` ([R][Hq][D]) override the random draws, for hand-made
    cases; they are rounded to bf16 all the same.
    """
    perm_rng = rng if permute_pages else None
    tree = tree_from_lengths(num_tokens, parent, paths, num_q_heads, num_kv_heads,
                             head_dim, sm_scale, perm_rng, extra_pool_pages)
    R, Hq, Hkv, D = tree.num_requests, num_q_heads, num_kv_heads, head_dim
    total_tok = int(tree.num_tokens.astype(np.int64).sum())
    if q_values is None:
        q_values = rng.standard_normal((R, Hq, D), dtype=np.float32)
    q = f32_to_bf16_bits(np.asarray(q_values, dtype=np.float32).reshape(R, Hq, D))
    if k_values is None:
        k_values = rng.standard_normal((total_tok, Hkv, D), dtype=np.float32)
    kt = f32_to_bf16_bits(np.asarray(k_values, dtype=np.float32).reshape(total_tok, Hkv, D))
    del k_values
    if v_values is None:
        v_values = rng.standard_normal((total_tok, Hkv, D), dtype=np.float32)
    vt = f32_to_bf16_bits(np.asarray(v_values, dtype=np.float32).reshape(total_tok, Hkv, D))
    del v_values
    tok_offs = np.zeros(tree.num_nodes + 1, dtype=np.int64)
    np.cumsum(tree.num_tokens.astype(np.int64), out=tok_offs[1:])
    k_pool, v_pool = pack_pools(tree, kt, vt, tok_offs, tail_fill)
    w = Workload(tree, q, k_pool, v_pool)
    if keep_tokens:
        w.k_tokens, w.v_tokens, w.token_offsets = kt, vt, tok_offs
    return w


def pack_pools(tree: Tree, kt: np.ndarray, vt: np.ndarray, tok_offs: np.ndarray,
               tail_fill: str = "nan"):
    """Scatter per-token K/V (node order) into the paged pool layouts."""
    Hkv, D, P = tree.num_kv_heads, tree.head_dim, PAGE
    fill = BF16_NAN if tail_fill == "nan" else np.uint16(0)
    total_pages = int(tree.page_offsets[-1])
    # token -> (global page index, slot) for every token, node by node
    nt = tree.num_tokens.astype(np.int64)
    tok_node = np.repeat(np.arange(tree.num_nodes), nt)
    tok_in_node = np.arange(int(nt.sum()), dtype=np.int64) - np.repeat(tok_offs[:-1], nt)
    gpage = tree.page_offsets[tok_node] + tok_in_node // P
    slot = tok_in_node % P
    # staging in logical page order: [total_pages][P][Hkv][D]
    stage_k = np.full((total_pages, P, Hkv, D), fill, dtype=np.uint16)
    stage_v = np.full((total_pages, P, Hkv, D), fill, dtype=np.uint16)
    stage_k[gpage, slot] = kt
    stage_v[gpage, slot] = vt
    k_pool = np.full((tree.num_pool_pages, Hkv, D // 8, P, 8), fill, dtype=np.uint16)
    v_pool = np.full((tree.num_pool_pages, Hkv, D, P), fill, dtype=np.uint16)
    phys = tree.page_ids.astype(np.int64)
    # [pg][P][Hkv][D] -> [pg][Hkv][D/8][P][8]
    k_pool[phys] = stage_k.reshape(total_pages, P, Hkv, D // 8, 8).transpose(0, 2, 3, 1, 4)
    del stage_k
    # [pg][P][Hkv][D] -> [pg][Hkv][D][P]
    v_pool[phys] = stage_v.transpose(0, 2, 3, 1)
    return k_pool, v_pool


def make_config(cfg: int, seed: int = 0, tail_fill: str = "nan",
                keep_tokens: bool = True, permute_pages: bool = True,
                extra_pool_pages: int = 0, heads_divisor: int = 1) -> Workload:
    """The five seeded shapes.  RNG = default_rng([seed, cfg]); draw order:
    tree structure, then Q, then K, then V; physical pages are a permutation.
    ``extra_pool_pages`` free pages (filled like unused slots) are appended to
    the pools afterwards, for decode steps that grow the tree; the draws do
    not depend on it.  ``heads_divisor`` = N keeps 1/N of the query and KV
    heads (same tree): one GPU's share when the heads are split over N GPUs."""
    rng = np.random.default_rng([seed, cfg])
    nt, par, paths, Hq, Hkv, D = _config_shape(cfg, rng)
    if heads_divisor != 1:
        if Hkv % heads_divisor:
            raise ValueError(f"{Hkv} KV heads do not split {heads_divisor} ways")
        Hq, Hkv = Hq // heads_divisor, Hkv // heads_divisor
    w = make_workload(nt, par, paths, Hq, Hkv, D, rng, permute_pages=permute_pages,
                      tail_fill=tail_fill, keep_tokens=keep_tokens)
    if extra_pool_pages > 0:
        fill = BF16_NAN if tail_fill == "nan" else np.uint16(0)
        n = int(extra_pool_pages)
        w.k_pool = np.concatenate([w.k_pool, np.full((n,) + w.k_pool.shape[1:], fill, np.uint16)])
        w.v_pool = np.concatenate([w.v_pool, np.full((n,) + w.v_pool.shape[1:], fill, np.uint16)])
        w.tree.num_pool_pages += n
    w.meta.update(config=cfg, seed=seed, name=CONFIG_NAMES[cfg])
    return w


def control_workload(w: Workload, tail_fill: str = "nan", seed: int = 0) -> Workload:
    """The unshared control batch: every request gets a private single-node
    copy of its flattened root-to-leaf context, in distinct physical pages,
    with identical values (so the attention result is identical)."""
    t = w.tree
    assert w.k_tokens is not None, "control batch needs the per-token arrays"
    R = t.num_requests
    nt, ks, vs = [], [], []
    for r in range(R):
        idx = np.concatenate([np.arange(w.token_offsets[n], w.token_offsets[n + 1])
                              for n in t.path(r)])
        nt.append(int(idx.shape[0]))
        ks.append(w.k_tokens[idx]); vs.append(w.v_tokens[idx])
    kt = np.concatenate(ks); vt = np.concatenate(vs)
    del ks, vs
    rng = np.random.default_rng([seed, 1000])
    tree = tree_from_lengths(nt, [-1] * R, [[r] for r in range(R)], t.num_q_heads,
                             t.num_kv_heads, t.head_dim, t.sm_scale, rng)
    tok_offs = np.zeros(R + 1, dtype=np.int64)
    np.cumsum(np.asarray(nt, dtype=np.int64), out=tok_offs[1:])
    k_pool, v_pool = pack_pools(tree, kt, vt, tok_offs, tail_fill)
    out = Workload(tree, w.q, k_pool, v_pool, kt, vt, tok_offs)
    out.meta.update(w.meta); out.meta["control"] = True
    return out


def tree_stats(t: Tree) -> dict:
    """Byte and FLOP counts of one decode step over the tree (no arithmetic on values)."""
    b_tok = 2 * t.num_kv_heads * t.head_dim * 2          # K+V bytes per token, all KV heads
    unique_tok = int(t.num_tokens.astype(np.int64).sum())
    ctx = np.asarray([t.context_len(r) for r in range(t.num_requests)], dtype=np.int64)
    return {
        "num_nodes": t.num_nodes,
        "num_requests": t.num_requests,
        "unique_tokens": unique_tok,
        "unique_kv_bytes": unique_tok * b_tok,
        "unshared_kv_bytes": int(ctx.sum()) * b_tok,
        "q_bytes": t.num_requests * t.num_q_heads * t.head_dim * 2,
        "out_bytes": t.num_requests * t.num_q_heads * t.head_dim * 2,
        "useful_flop": int(4 * t.head_dim * t.num_q_heads * int(ctx.sum())),
        "request_heads": t.num_requests * t.num_q_heads,
        "sum_context": int(ctx.sum()),
    }


# --------------------------------------------------------------- decode growth

def free_pages(tree: Tree) -> np.ndarray:
    """Pool pages that no node holds, ascending."""
    used = np.zeros(int(tree.num_pool_pages), dtype=bool)
    used[tree.page_ids.astype(np.int64)] = True
    return np.flatnonzero(~used).astype(np.int32)


def grow_tree(tree: Tree, active=None, new_pages=None):
    """The tree after one decode step: every active request gains one token at
    the end of its context.

    Rule: when a request's path ends at a leaf that no other request's path
    passes through, the leaf takes the token, in the next slot of its last
    page or, when that page is full (or the leaf has no page), in page
    ``new_pages[r]``; otherwise a new one-token child of the end node, holding
    page ``new_pages[r]``, becomes the request's leaf (new ids in request
    order).  Returns ``(new_tree, dest)`` with dest[r] = (page << 4) | slot,
    -1 for an inactive request.  Pure bookkeeping on the description."""
    N, R = tree.num_nodes, tree.num_requests
    act = np.ones(R, dtype=bool) if active is None else np.asarray(active, dtype=bool)
    ntok = [int(x) for x in tree.num_tokens]
    parent = [int(x) for x in tree.parent]
    pages = [list(tree.page_ids[tree.page_offsets[n]:tree.page_offsets[n + 1]]) for n in range(N)]
    paths = [list(tree.path(r)) for r in range(R)]
    passing = np.zeros(N, dtype=np.int64)
    for p in paths:
        passing[p] += 1
    has_child = np.zeros(N, dtype=bool)
    for c in range(N):
        if parent[c] >= 0:
            has_child[parent[c]] = True
    dest = np.full(R, -1, dtype=np.int32)
    for r in range(R):
        if not act[r]:
            continue
        n = paths[r][-1]
        if not has_child[n] and passing[n] == 1:
            if ntok[n] % PAGE == 0:
                pages[n].append(int(new_pages[r]))
            dest[r] = (int(pages[n][ntok[n] // PAGE]) << 4) | (ntok[n] % PAGE)
            ntok[n] += 1
        else:
            parent.append(n)
            ntok.append(1)
            pages.append([int(new_pages[r])])
            paths[r].append(len(parent) - 1)
            dest[r] = int(new_pages[r]) << 4
    offs = np.zeros(len(pages) + 1, dtype=np.int64)
    np.cumsum([len(p) for p in pages], out=offs[1:])
    ids = np.asarray([pg for p in pages for pg in p], dtype=np.int32)
    poffs = np.zeros(R + 1, dtype=np.int32)
    np.cumsum([len(p) for p in paths], out=poffs[1:])
    pn = np.asarray([n for p in paths for n in p], dtype=np.int32)
    new = Tree(tree.num_q_heads, tree.num_kv_heads, tree.head_dim,
               np.asarray(parent, dtype=np.int32), np.asarray(ntok, dtype=np.int32), offs, ids,
               poffs, pn, tree.num_pool_pages, tree.sm_scale, tree.page_size)
    return new, dest


def write_new_tokens(k_pool: np.ndarray, v_pool: np.ndarray, dest: np.ndarray,
                     k_new: np.ndarray, v_new: np.ndarray) -> None:
    """Store token i's K/V bits ([n][Hkv][D] each) at page dest[i] >> 4, slot
    dest[i] & 15 of the host pools (in place); negative entries are skipped."""
    for i, e in enumerate(np.asarray(dest)):
        if e < 0:
            continue
        pg, slot = int(e) >> 4, int(e) & 15
        Hkv, D = k_new.shape[1], k_new.shape[2]
        k_pool[pg, :, :, slot, :] = k_new[i].reshape(Hkv, D // 8, 8)
        v_pool[pg, :, :, slot] = v_new[i]


# ------------------------------------------------- wide-row reduction inputs

# rows per workload as in the CREDIT summary's evaluation (section V.A):
# 2048 for LayerNorm, 4096 for the others; widths 4K..64K
ROW_KINDS = {"softmax": 4096, "layernorm": 2048}


def make_rows(kind: str, width: int, rows: Optional[int] = None, seed: int = 0):
    """Seeded FP32 inputs of one row workload: x [rows][width] ~ N(0, 1);
    LayerNorm also gets per-column gamma ~ 1 + 0.1 N(0, 1) and beta ~
    0.1 N(0, 1).  RNG = default_rng([seed, 7, width, kind index]); draw
    order x, gamma, beta.  Returns (x, gamma, beta), the last two None for
    softmax."""
    if kind not in ROW_KINDS:
        raise ValueError(f"unknown row workload {kind}")
    rows = ROW_KINDS[kind] if rows is None else int(rows)
    rng = np.random.default_rng([seed, 7, int(width), list(ROW_KINDS).index(kind)])
    x = rng.standard_normal((rows, int(width)), dtype=np.float32)
    if kind != "layernorm":
        return x, None, None
    gamma = (1.0 + 0.1 * rng.standard_normal(int(width))).astype(np.float32)
    beta = (0.1 * rng.standard_normal(int(width))).astype(np.float32)
    return x, gamma, beta
