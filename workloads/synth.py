"""Seeded synthetic decode batches laid out in a paged KV pool.

What is drawn, and in which order (one ``numpy.random.default_rng(seed)``):

1. per-request own-token counts (integers, uniform and inclusive);
2. queries ``q[B][H_q][d]`` ~ N(0, 1) in fp32;
3. keys for every logical token ~ N(0, 1) in fp32: the shared-prefix tokens
   first, then request 0's own tokens, request 1's, ...;
4. values, in the same order;
5. the cast to the stored dtype (bf16 by round-to-nearest-even through torch;
   fp8 e4m3 by a per-KV-head scale ``amax / 448``, clamp to +-448, torch cast);
6. a random permutation of the physical pages of the pool.

The shared prefix (if any) is stored either once in physical pages that every
request's page table points at ("shared"), or as a private copy in each
request's own pages ("unique").  Only whole pages are shared; a prefix tail
that does not fill a page lives in each request's own pages.

Slots of the pool that no request uses hold a poison value (NaN, or the fp8
NaN code 0x7F) so that a gather from a wrong slot cannot go unnoticed.

The pool is filled page by page: logical page ``j`` of a request is copied
whole into the physical page its page table names.  Nothing here turns a page
table into per-token indices or evaluates attention.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0

_TORCH_DTYPE = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
    "fp8": torch.float8_e4m3fn,
}

_BITS_DTYPE = {"f32": torch.int32, "bf16": torch.int16, "fp8": torch.uint8}


@dataclass
class DecodeBatch:
    """One decode step's inputs: queries plus a paged K/V pool.

    ``seq_lens[b]`` counts every KV token request ``b`` attends: the shared
    prefix (``prefix_len`` tokens) followed by its own tokens.
    """

    B: int
    H_q: int
    H_kv: int
    d: int
    q_dtype: str
    kv_dtype: str
    page_size: int
    prefix_len: int
    layout: str
    seq_lens: np.ndarray  # int32 [B]
    q: torch.Tensor  # [B, H_q, d] in q dtype (cpu)
    k_tokens: torch.Tensor  # [prefix_len + sum(own), H_kv, d] stored dtype (cpu)
    v_tokens: torch.Tensor
    own_offsets: np.ndarray  # int64 [B+1], offsets of own tokens after the prefix
    k_scale: Optional[np.ndarray]  # float32 [H_kv] (fp8 only)
    v_scale: Optional[np.ndarray]
    num_pages: int = 0
    page_indptr: np.ndarray = field(default=None)  # int32 [B+1]
    page_indices: np.ndarray = field(default=None)  # int32 [sum pages]
    k_pool: torch.Tensor = field(default=None)  # [num_pages*p, H_kv, d]
    v_pool: torch.Tensor = field(default=None)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    def logical_kv(self, b: int):
        """Stored K, V of request ``b`` in logical order: prefix ++ own."""
        P = self.prefix_len
        lo = P + int(self.own_offsets[b])
        hi = P + int(self.own_offsets[b + 1])
        k = torch.cat([self.k_tokens[:P], self.k_tokens[lo:hi]], dim=0)
        v = torch.cat([self.v_tokens[:P], self.v_tokens[lo:hi]], dim=0)
        return k, v

    def bits(self, t: torch.Tensor, dtype: str) -> np.ndarray:
        """Raw stored bits of a tensor as a numpy integer array."""
        return t.contiguous().view(_BITS_DTYPE[dtype]).numpy()


def _cast(x32: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None) -> torch.Tensor:
    t = torch.from_numpy(x32)
    if dtype == "f32":
        return t.clone()
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp8":
        s = torch.from_numpy(scale.astype(np.float32)).view(1, -1, 1)
        return (t / s).clamp_(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    raise ValueError(dtype)


def _fp8_scale(x32: np.ndarray) -> np.ndarray:
    """Per-KV-head scale amax/448 over all live tokens; never zero."""
    amax = np.abs(x32).max(axis=(0, 2)) if x32.shape[0] else np.zeros(x32.shape[1], np.float32)
    amax = np.where(amax > 0, amax, 1.0).astype(np.float32)
    return (amax / np.float32(FP8_MAX)).astype(np.float32)


def _poison(dtype: str) -> torch.Tensor:
    if dtype == "fp8":
        return torch.tensor([0x7F], dtype=torch.uint8).view(torch.float8_e4m3fn)[0]
    return torch.tensor(float("nan"), dtype=_TORCH_DTYPE[dtype])


def make_decode_batch(
    *,
    seed: int,
    B: int,
    H_q: int,
    H_kv: int,
    d: int,
    own_len: tuple,
    prefix_len: int = 0,
    q_dtype: str = "bf16",
    kv_dtype: str = "bf16",
    page_size: int = 16,
    layout: str = "shared",
    pool_pages: Optional[int] = None,
    pool_factor: int = 1,
    perm: str = "random",
    perm_seed: Optional[int] = None,
    device: Optional[str] = None,
    own_lens: Optional[list] = None,
) -> DecodeBatch:
    """Draw one batch and lay it out in a paged pool.

    ``own_len`` is ``(lo, hi)``: each request's own token count is drawn
    uniformly from the integers ``lo..hi`` inclusive.  ``pool_pages`` fixes the
    pool size in pages; otherwise the pool holds ``pool_factor`` times the live
    pages.  ``perm`` is ``"random"`` or ``"identity"`` (pages in allocation
    order: the contiguous control).  ``own_lens`` fixes every request's own
    token count instead (the draw still happens, keeping the stream aligned).
    """
    assert H_q % H_kv == 0 and layout in ("shared", "unique")
    rng = np.random.default_rng(seed)
    lo, hi = own_len
    own = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    if own_lens is not None:
        own = np.asarray(own_lens, np.int64)
        assert own.shape == (B,)
    own_offsets = np.zeros(B + 1, np.int64)
    np.cumsum(own, out=own_offsets[1:])
    seq_lens = (own + prefix_len).astype(np.int32)
    q32 = rng.standard_normal((B, H_q, d), dtype=np.float32)
    T = prefix_len + int(own_offsets[-1])
    k32 = rng.standard_normal((T, H_kv, d), dtype=np.float32)
    v32 = rng.standard_normal((T, H_kv, d), dtype=np.float32)
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_scale, v_scale = _fp8_scale(k32), _fp8_scale(v32)
    q = _cast(q32, q_dtype)
    k_tokens = _cast(k32, kv_dtype, k_scale)
    v_tokens = _cast(v32, kv_dtype, v_scale)
    del k32, v32
    batch = DecodeBatch(
        B=B, H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype,
        page_size=page_size, prefix_len=prefix_len, layout=layout,
        seq_lens=seq_lens, q=q, k_tokens=k_tokens, v_tokens=v_tokens,
        own_offsets=own_offsets, k_scale=k_scale, v_scale=v_scale,
    )
    return relayout(batch, page_size=page_size, rng=rng if perm_seed is None else None,
                    seed=perm_seed, layout=layout, pool_pages=pool_pages,
                    pool_factor=pool_factor, perm=perm, device=device)


def relayout(
    batch: DecodeBatch,
    *,
    page_size: int,
    seed: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
    layout: Optional[str] = None,
    pool_pages: Optional[int] = None,
    pool_factor: int = 1,
    perm: str = "random",
    device: Optional[str] = None,
    prefix_first_page: int = 0,
) -> DecodeBatch:
    """Place the same logical tokens into a fresh pool.

    Draws a new page permutation (from ``rng``, else ``default_rng(seed)``) and
    returns a copy of ``batch`` with a new page table and pool.  With
    ``perm="prefix_first"`` the shared prefix's whole pages are stored in
    order as one run starting at page ``prefix_first_page``, every other page
    randomly placed around it.
    """
    layout = layout or batch.layout
    p = int(page_size)
    P = batch.prefix_len
    B = batch.B
    n_shared = P // p if (layout == "shared" and B > 0) else 0
    # tokens each request stores in its own pages
    own_store = batch.seq_lens.astype(np.int64) - n_shared * p
    own_pages = (own_store + p - 1) // p
    live_pages = n_shared + int(own_pages.sum())
    if pool_pages is None:
        pool_pages = max(1, live_pages * pool_factor)
    if pool_pages < live_pages:
        raise ValueError(f"pool of {pool_pages} pages cannot hold {live_pages} live pages")
    if rng is None:
        rng = np.random.default_rng(seed)
    if perm == "random":
        order = rng.permutation(pool_pages).astype(np.int64)
    elif perm == "identity":
        order = np.arange(pool_pages, dtype=np.int64)
    elif perm == "prefix_first":
        # the shared prefix in consecutive pages, in order (stored
        # contiguously) from prefix_first_page; every other page randomly
        # placed around it
        f0 = int(prefix_first_page)
        if not 0 <= f0 <= pool_pages - n_shared:
            raise ValueError("prefix run does not fit in the pool")
        rest = np.concatenate([np.arange(f0), np.arange(f0 + n_shared, pool_pages)])
        order = np.concatenate([np.arange(f0, f0 + n_shared), rng.permutation(rest)]).astype(np.int64)
    else:
        raise ValueError(perm)
    shared_pages = order[:n_shared]
    cursor = n_shared
    page_indptr = np.zeros(B + 1, np.int64)
    tables = []
    for b in range(B):
        mine = order[cursor:cursor + own_pages[b]]
        cursor += int(own_pages[b])
        tables.append(np.concatenate([shared_pages, mine]))
        page_indptr[b + 1] = page_indptr[b] + len(tables[-1])
    page_indices = (np.concatenate(tables) if tables else np.zeros(0, np.int64))

    dev = torch.device(device) if device else torch.device("cpu")
    H, d = batch.H_kv, batch.d
    dt = _TORCH_DTYPE[batch.kv_dtype]
    pools = []
    for src in (batch.k_tokens, batch.v_tokens):
        pool = torch.empty((pool_pages, p, H, d), dtype=dt, device=dev)
        if batch.kv_dtype == "fp8":
            pool.view(torch.uint8).fill_(0x7F)
        else:
            pool.fill_(float("nan"))
        src_dev = src.to(dev)
        if n_shared:
            pool[torch.from_numpy(shared_pages).to(dev)] = src_dev[: n_shared * p].reshape(n_shared, p, H, d)
        for b in range(B):
            if own_pages[b] == 0:
                continue
            lo = P + int(batch.own_offsets[b])
            hi = P + int(batch.own_offsets[b + 1])
            parts = []
            if P - n_shared * p > 0:
                parts.append(src_dev[n_shared * p: P])
            parts.append(src_dev[lo:hi])
            seq = torch.cat(parts, dim=0) if len(parts) > 1 else parts[0]
            n = int(own_pages[b])
            buf = torch.empty((n * p, H, d), dtype=dt, device=dev)
            if batch.kv_dtype == "fp8":
                buf.view(torch.uint8).fill_(0x7F)
            else:
                buf.fill_(float("nan"))
            buf[: seq.shape[0]] = seq
            first = int(page_indptr[b]) + n_shared
            dst = torch.from_numpy(page_indices[first:first + n]).to(dev)
            pool[dst] = buf.view(n, p, H, d)
        pools.append(pool.view(pool_pages * p, H, d))
    out = DecodeBatch(**{k: getattr(batch, k) for k in (
        "B", "H_q", "H_kv", "d", "q_dtype", "kv_dtype", "prefix_len", "seq_lens",
        "q", "k_tokens", "v_tokens", "own_offsets", "k_scale", "v_scale")},
        page_size=p, layout=layout)
    out.num_pages = pool_pages
    out.page_indptr = page_indptr.astype(np.int32)
    out.page_indices = page_indices.astype(np.int32)
    out.k_pool, out.v_pool = pools
    return out


# The five workloads.  Seeds follow 1000 + k; page re-layouts of the same
# logical values use 2000 + k.
CONFIGS = {
    "c1": dict(B=4, H_q=8, H_kv=2, d=64, own_len=(64, 256), q_dtype="f32", kv_dtype="f32",
               page_size=16, pool_pages=128),
    "c2": dict(B=32, H_q=32, H_kv=8, d=128, own_len=(4096, 4096), q_dtype="bf16",
               kv_dtype="bf16", page_size=128),
    "c3": dict(B=256, H_q=32, H_kv=8, d=128, own_len=(64, 512), prefix_len=4096,
               q_dtype="bf16", kv_dtype="bf16", page_size=16),
    "c4": dict(B=512, H_q=32, H_kv=8, d=128, own_len=(256, 1024), prefix_len=512,
               q_dtype="bf16", kv_dtype="bf16", page_size=16),
    "c5": dict(B=16, H_q=64, H_kv=8, d=128, own_len=(16384, 16384), q_dtype="bf16",
               kv_dtype="fp8", page_size=16, pool_factor=2),
}

# The shared-prefix workload with an fp8 cache: the same shapes, K/V stored
# as e4m3 codes with per-KV-head scales (its own seed).
CONFIGS["c3_fp8"] = dict(CONFIGS["c3"], kv_dtype="fp8")

CONFIG_SEED = {"c1": 1001, "c2": 1002, "c3": 1003, "c4": 1004, "c5": 1005, "c3_fp8": 1013}
RELAYOUT_SEED = {"c1": 2001, "c2": 2002, "c3": 2003, "c4": 2004, "c5": 2005, "c3_fp8": 2013}


def make_config(name: str, **overrides) -> DecodeBatch:
    """Build one of the named workloads, with optional overrides."""
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    kw.setdefault("seed", CONFIG_SEED[name])
    return make_decode_batch(**kw)
