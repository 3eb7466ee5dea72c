"""Page tables and pools for decode steps whose requests share several
prefixes (seeded synthetic inputs; no attention arithmetic here).

A prefix cache that matches exact, block-aligned prefixes hands two requests
the same physical page exactly when their content up to and including that
block is the same.  ``tables_from_blocks`` builds page tables with that
property from per-block content labels; ``make_grouped_batch`` draws a whole
batch (queries, K/V values, paged pool) in which groups of requests sit on
shared prefixes of their own.

What ``make_grouped_batch`` draws, in order (one ``default_rng(seed)``):

1. the assignment of requests to groups (a permutation of the requests; the
   first n_0 go to group 0, the next n_1 to group 1, ...; the rest share
   nothing);
2. per-request own-token counts (integers, uniform and inclusive);
3. queries ``q[B][H_q][d]`` ~ N(0, 1) in fp32;
4. keys ~ N(0, 1): every group's prefix tokens in group order, then request
   0's own tokens, request 1's, ...;
5. values, in the same order;
6. the cast to the stored dtype (as ``synth``: bf16 round-to-nearest-even;
   fp8 e4m3 with a per-KV-head scale amax / 448);
7. a random permutation of the pool's physical pages.

Only whole pages of a prefix are shared; its tail (prefix length mod page
size) is copied into each member's own pages.  Unused slots hold NaN (fp8:
the NaN code), as in ``synth``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from .synth import _BITS_DTYPE, _TORCH_DTYPE, _cast, _fp8_scale


def token_blocks(tokens, p):
    """Cut a list of token labels into blocks of p (the last may be short)."""
    return [tuple(tokens[j:j + p]) for j in range(0, len(tokens), p)]


def tables_from_blocks(requests, p, seed=0, scramble=True):
    """Page tables for requests given as lists of per-block contents.

    A physical page is shared exactly when the content up to and including
    its block is the same.  Page numbers are scrambled by a permutation drawn
    from ``default_rng(seed)``; with ``scramble=False`` they are handed out in
    order of first use (a request's new pages then follow one another, the
    contiguous placement of a prefix).  Returns (page_indptr, page_indices),
    int64.
    """
    ids = {}
    tables = []
    for blocks in requests:
        tables.append([ids.setdefault(tuple(blocks[:j + 1]), len(ids)) for j in range(len(blocks))])
    perm = (np.random.default_rng(seed).permutation(max(1, len(ids))) if scramble
            else np.arange(max(1, len(ids))))
    page_indptr = np.zeros(len(requests) + 1, np.int64)
    for b, t in enumerate(tables):
        page_indptr[b + 1] = page_indptr[b] + len(t)
    page_indices = np.array([perm[x] for t in tables for x in t], np.int64)
    return page_indptr, page_indices


def random_group_tables(rng, p, max_batch=8):
    """Requests drawn from a few system prompts of random lengths (in
    tokens), some continued by one of two shared follow-ups (nested sharing),
    each followed by its own tokens; some requests have no prompt.  Returns
    (per-request block lists, token counts)."""
    n_prompts = int(rng.integers(0, 4))
    prompts = [int(rng.integers(0, 5 * p)) for _ in range(n_prompts)]
    follow = [[int(rng.integers(1, 3 * p)) for _ in range(2)] for _ in range(n_prompts)]
    B = int(rng.integers(0, max_batch + 1))
    reqs, lens = [], []
    for b in range(B):
        k = int(rng.integers(-1, n_prompts)) if n_prompts else -1
        toks = []
        if k >= 0:
            toks = [f"s{k}"] * prompts[k]
            j = int(rng.integers(-1, 2))
            if j >= 0:
                toks += [f"f{k}.{j}"] * follow[k][j]
        toks += [f"o{b}"] * int(rng.integers(0, 3 * p))
        reqs.append(token_blocks(toks, p))
        lens.append(len(toks))
    return reqs, lens


@dataclass
class GroupedBatch:
    """One decode step with several shared prefixes, in a paged pool.

    ``group_of[b]`` is the prefix group request b was drawn on (-1: none);
    ``seq_lens[b]`` counts its prefix tokens plus its own tokens.
    """

    B: int
    H_q: int
    H_kv: int
    d: int
    q_dtype: str
    kv_dtype: str
    page_size: int
    group_of: np.ndarray          # int64 [B]
    prefix_lens: list             # tokens of each group's prefix
    seq_lens: np.ndarray          # int32 [B]
    q: torch.Tensor               # [B, H_q, d] (cpu)
    prefix_k: list                # per group [P_g, H_kv, d] stored dtype (cpu)
    prefix_v: list
    own_k: torch.Tensor           # [sum own, H_kv, d]
    own_v: torch.Tensor
    own_offsets: np.ndarray       # int64 [B+1]
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    num_pages: int = 0
    page_indptr: np.ndarray = field(default=None)
    page_indices: np.ndarray = field(default=None)
    k_pool: torch.Tensor = field(default=None)
    v_pool: torch.Tensor = field(default=None)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def logical_kv(self, b: int):
        """Stored K, V of request b in logical order: its prefix ++ own."""
        lo, hi = int(self.own_offsets[b]), int(self.own_offsets[b + 1])
        g = int(self.group_of[b])
        if g < 0:
            return self.own_k[lo:hi], self.own_v[lo:hi]
        return (torch.cat([self.prefix_k[g], self.own_k[lo:hi]], 0),
                torch.cat([self.prefix_v[g], self.own_v[lo:hi]], 0))

    def bits(self, t: torch.Tensor, dtype: str) -> np.ndarray:
        return t.contiguous().view(_BITS_DTYPE[dtype]).numpy()


def make_grouped_batch(*, seed, B, H_q, H_kv, d, groups, own_len, q_dtype="bf16", kv_dtype="bf16",
                       page_size=16, perm="random", pool_factor=1, device=None) -> GroupedBatch:
    """Draw a batch in which ``groups = [(members, prefix_tokens), ...]``
    requests sit on prefixes of their own (see the module docstring)."""
    assert H_q % H_kv == 0 and sum(n for n, _ in groups) <= B
    rng = np.random.default_rng(seed)
    order = rng.permutation(B)
    group_of = np.full(B, -1, np.int64)
    at = 0
    for g, (n, _) in enumerate(groups):
        group_of[order[at:at + n]] = g
        at += n
    lo, hi = own_len
    own = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    own_offsets = np.zeros(B + 1, np.int64)
    np.cumsum(own, out=own_offsets[1:])
    prefix_lens = [int(P) for _, P in groups]
    seq_lens = np.array([own[b] + (prefix_lens[group_of[b]] if group_of[b] >= 0 else 0) for b in range(B)],
                        np.int32)
    q32 = rng.standard_normal((B, H_q, d), dtype=np.float32)
    n_pre = sum(prefix_lens)
    T = n_pre + int(own_offsets[-1])
    k32 = rng.standard_normal((T, H_kv, d), dtype=np.float32)
    v32 = rng.standard_normal((T, H_kv, d), dtype=np.float32)
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_scale, v_scale = _fp8_scale(k32), _fp8_scale(v32)
    q = _cast(q32, q_dtype)
    k_all = _cast(k32, kv_dtype, k_scale)
    v_all = _cast(v32, kv_dtype, v_scale)
    del k32, v32
    cut = np.cumsum([0] + prefix_lens)
    prefix_k = [k_all[cut[g]:cut[g + 1]] for g in range(len(groups))]
    prefix_v = [v_all[cut[g]:cut[g + 1]] for g in range(len(groups))]
    own_k, own_v = k_all[n_pre:], v_all[n_pre:]

    # Pages: each group's whole prefix pages once, then every request's own
    # pages (its prefix tail, if any, and its own tokens).
    p = int(page_size)
    shared = [P // p for P in prefix_lens]
    own_store = np.array([int(seq_lens[b]) - (shared[group_of[b]] * p if group_of[b] >= 0 else 0)
                          for b in range(B)], np.int64)
    own_pages = (own_store + p - 1) // p
    live = sum(shared) + int(own_pages.sum())
    pool_pages = max(1, live * pool_factor)
    pages = rng.permutation(pool_pages).astype(np.int64) if perm == "random" else np.arange(pool_pages)
    cursor = 0
    shared_pages = []
    for n in shared:
        shared_pages.append(pages[cursor:cursor + n])
        cursor += n
    page_indptr = np.zeros(B + 1, np.int64)
    tables = []
    for b in range(B):
        mine = pages[cursor:cursor + own_pages[b]]
        cursor += int(own_pages[b])
        g = int(group_of[b])
        tables.append(np.concatenate([shared_pages[g], mine]) if g >= 0 else mine)
        page_indptr[b + 1] = page_indptr[b] + len(tables[-1])
    page_indices = np.concatenate(tables) if tables else np.zeros(0, np.int64)

    dev = torch.device(device) if device else torch.device("cpu")
    H = H_kv
    dt = _TORCH_DTYPE[kv_dtype]
    out = GroupedBatch(B=B, H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=p,
                       group_of=group_of, prefix_lens=prefix_lens, seq_lens=seq_lens, q=q, prefix_k=prefix_k,
                       prefix_v=prefix_v, own_k=own_k, own_v=own_v, own_offsets=own_offsets, k_scale=k_scale,
                       v_scale=v_scale)
    pools = []
    for which in ("k", "v"):
        pool = torch.empty((pool_pages, p, H, d), dtype=dt, device=dev)
        if kv_dtype == "fp8":
            pool.view(torch.uint8).fill_(0x7F)
        else:
            pool.fill_(float("nan"))
        for g in range(len(groups)):
            if shared[g]:
                src = (prefix_k if which == "k" else prefix_v)[g][: shared[g] * p].to(dev)
                pool[torch.from_numpy(shared_pages[g]).to(dev)] = src.reshape(shared[g], p, H, d)
        for b in range(B):
            n = int(own_pages[b])
            if n == 0:
                continue
            k, v = out.logical_kv(b)
            g = int(group_of[b])
            seq = (k if which == "k" else v)[(shared[g] * p if g >= 0 else 0):].to(dev)
            buf = torch.empty((n * p, H, d), dtype=dt, device=dev)
            if kv_dtype == "fp8":
                buf.view(torch.uint8).fill_(0x7F)
            else:
                buf.fill_(float("nan"))
            buf[: seq.shape[0]] = seq
            first = int(page_indptr[b]) + (shared[g] if g >= 0 else 0)
            pool[torch.from_numpy(page_indices[first:first + n]).to(dev)] = buf.view(n, p, H, d)
        pools.append(pool.view(pool_pages * p, H, d))
    out.num_pages = pool_pages
    out.page_indptr = page_indptr.astype(np.int32)
    out.page_indices = page_indices.astype(np.int32)
    out.k_pool, out.v_pool = pools
    return out


# Several prompts live in one step (the pages' "two system prompts, two
# trees" case, at the Llama-3.1-8B layer shape): 256 requests, four prompts of
# 4096, 2048, 1024 and 512 tokens with 48 requests each, 64 requests on no
# prompt, own tokens U{64..512}, bf16, page size 16.
GROUP_CONFIGS = {
    "groups4": dict(B=256, H_q=32, H_kv=8, d=128, groups=[(48, 4096), (48, 2048), (48, 1024), (48, 512)],
                    own_len=(64, 512), q_dtype="bf16", kv_dtype="bf16", page_size=16),
}
GROUP_CONFIG_SEED = {"groups4": 1006}


def make_group_config(name: str, **overrides) -> GroupedBatch:
    kw = dict(GROUP_CONFIGS[name])
    kw.update(overrides)
    kw.setdefault("seed", GROUP_CONFIG_SEED[name])
    return make_grouped_batch(**kw)


@dataclass
class TreeBatch:
    """One decode step whose requests share runs of tokens as a tree.

    Request b's logical tokens are ``tokens[b]`` (indices into the value
    tables ``k_all``, ``v_all``): the tokens of the tree nodes on its path,
    root first, then its own.
    """

    B: int
    H_q: int
    H_kv: int
    d: int
    q_dtype: str
    kv_dtype: str
    page_size: int
    tokens: list                  # per request: int64 array of token ids
    seq_lens: np.ndarray          # int32 [B]
    q: torch.Tensor
    k_all: torch.Tensor           # [tokens, H_kv, d] stored dtype (cpu)
    v_all: torch.Tensor
    node_members: list            # per tree node: its requests
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    num_pages: int = 0
    page_indptr: np.ndarray = field(default=None)
    page_indices: np.ndarray = field(default=None)
    k_pool: torch.Tensor = field(default=None)
    v_pool: torch.Tensor = field(default=None)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    def logical_kv(self, b: int):
        idx = torch.from_numpy(self.tokens[b])
        return self.k_all[idx], self.v_all[idx]

    def bits(self, t: torch.Tensor, dtype: str) -> np.ndarray:
        return t.contiguous().view(_BITS_DTYPE[dtype]).numpy()


def make_tree_batch(*, seed, B, H_q, H_kv, d, tree, own_len, q_dtype="bf16", kv_dtype="bf16", page_size=16,
                    pool_factor=1, device=None) -> TreeBatch:
    """Draw a batch whose requests share token runs along a tree.

    ``tree = [(members, tokens, parent), ...]``, parents before children:
    node i takes ``members`` requests from its parent's (from all requests
    for a root), disjoint from its earlier siblings' (and from earlier
    roots'), and adds ``tokens`` tokens.  Pages are content addressed, as a
    prefix cache that matches exact block-aligned prefixes would lay them
    out: two requests share a physical page exactly when their token
    sequences agree up to the end of that page.

    Draw order (one ``default_rng(seed)``): node memberships, own lengths
    (integers, uniform inclusive), Q, K then V for the node tokens in node
    order followed by each request's own tokens, the cast, the page
    permutation.
    """
    assert H_q % H_kv == 0
    rng = np.random.default_rng(seed)
    taken_root = set()
    taken_child = {}
    members_of = []
    for n, _, parent in tree:
        if parent < 0:
            free = [b for b in range(B) if b not in taken_root]
        else:
            used = taken_child.setdefault(parent, set())
            free = [b for b in members_of[parent] if b not in used]
        assert len(free) >= n, "tree does not fit the batch"
        pick = sorted(int(x) for x in rng.permutation(free)[:n])
        (taken_root if parent < 0 else taken_child[parent]).update(pick)
        members_of.append(pick)
    lo, hi = own_len
    own = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    q32 = rng.standard_normal((B, H_q, d), dtype=np.float32)
    node_off = np.cumsum([0] + [T for _, T, _ in tree])
    own_off = node_off[-1] + np.concatenate([[0], np.cumsum(own)])
    T_all = int(own_off[-1])
    k32 = rng.standard_normal((T_all, H_kv, d), dtype=np.float32)
    v32 = rng.standard_normal((T_all, H_kv, d), dtype=np.float32)
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_scale, v_scale = _fp8_scale(k32), _fp8_scale(v32)
    q = _cast(q32, q_dtype)
    k_all = _cast(k32, kv_dtype, k_scale)
    v_all = _cast(v32, kv_dtype, v_scale)
    del k32, v32
    # each request's token ids: its path's node tokens, then its own
    path = [[] for _ in range(B)]
    for i, (n, T, parent) in enumerate(tree):
        for b in members_of[i]:
            path[b].append(i)
    tokens = []
    for b in range(B):
        parts = [np.arange(node_off[i], node_off[i + 1]) for i in path[b]]
        parts.append(np.arange(own_off[b], own_off[b + 1]))
        tokens.append(np.concatenate(parts).astype(np.int64))
    seq_lens = np.array([len(t) for t in tokens], np.int32)
    # content-addressed pages: (previous page, this block's token ids)
    p = int(page_size)
    page_id, page_tokens, tables = {}, [], []
    for b in range(B):
        prev, tab = -1, []
        for j in range(0, len(tokens[b]), p):
            key = (prev, tuple(tokens[b][j:j + p]))
            if key not in page_id:
                page_id[key] = len(page_tokens)
                page_tokens.append(tokens[b][j:j + p])
            prev = page_id[key]
            tab.append(prev)
        tables.append(tab)
    live = max(1, len(page_tokens))
    pool_pages = live * pool_factor
    perm = rng.permutation(pool_pages).astype(np.int64)
    page_indptr = np.zeros(B + 1, np.int64)
    for b in range(B):
        page_indptr[b + 1] = page_indptr[b] + len(tables[b])
    page_indices = np.array([perm[x] for t in tables for x in t], np.int64)

    dev = torch.device(device) if device else torch.device("cpu")
    dt = _TORCH_DTYPE[kv_dtype]
    out = TreeBatch(B=B, H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=p, tokens=tokens,
                    seq_lens=seq_lens, q=q, k_all=k_all, v_all=v_all, node_members=members_of, k_scale=k_scale,
                    v_scale=v_scale)
    pools = []
    for src in (k_all, v_all):
        pool = torch.empty((pool_pages, p, H_kv, d), dtype=dt)
        if kv_dtype == "fp8":
            pool.view(torch.uint8).fill_(0x7F)
        else:
            pool.fill_(float("nan"))
        for i, ids in enumerate(page_tokens):
            pool[int(perm[i]), :len(ids)] = src[torch.from_numpy(np.asarray(ids, np.int64))]
        pools.append(pool.view(pool_pages * p, H_kv, d).to(dev))
    out.num_pages = pool_pages
    out.page_indptr = page_indptr.astype(np.int32)
    out.page_indices = page_indices.astype(np.int32)
    out.k_pool, out.v_pool = pools
    return out


# A system prompt under several conversations (nested sharing, the radix
# tree of a prefix cache), at the Llama-3.1-8B layer shape: 256 requests, a
# 2048-token prompt shared by 192 of them, four conversations of 48 requests
# each sharing 1024 more tokens, 64 requests on nothing, own tokens
# U{64..512}, bf16, page size 16.
TREE_CONFIGS = {
    "tree4": dict(B=256, H_q=32, H_kv=8, d=128, tree=[(192, 2048, -1)] + [(48, 1024, 0)] * 4,
                  own_len=(64, 512), q_dtype="bf16", kv_dtype="bf16", page_size=16),
}
TREE_CONFIG_SEED = {"tree4": 1007}


def make_tree_config(name: str, **overrides) -> TreeBatch:
    kw = dict(TREE_CONFIGS[name])
    kw.update(overrides)
    kw.setdefault("seed", TREE_CONFIG_SEED[name])
    return make_tree_batch(**kw)
