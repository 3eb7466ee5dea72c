"""Page table -> token-flat indices (test oracle).

"The 25% Page-Size Slowdown That Wasn't", section "Four meanings of page
size": a serving backend either passes per-page metadata or expands it into
per-token indices, and in the studied decode path the per-token list has one
entry per (request, cached token) -- length B x L -- at every page size
(section "When source beats intuition").  Each sequence owns logical pages
that map onto physical storage; token t of a request sits in its logical page
floor(t / p) at offset t mod p, so its physical slot is

    slot(b, t) = page_indices[page_indptr[b] + floor(t / p)] * p + (t mod p)

A request with L tokens must own exactly ceil(L / p) pages (no page past its
last token; "Track C · Document 10", block-size paragraph: the last page may
be partly filled).
"""
import numpy as np


class LoweringError(ValueError):
    pass


def _check(page_size, page_indptr, seq_lens):
    if page_size < 1:
        raise LoweringError("page_size must be >= 1")
    B = len(seq_lens)
    if len(page_indptr) != B + 1 or page_indptr[0] != 0:
        raise LoweringError("page_indptr must have B+1 entries starting at 0")
    for b in range(B):
        n = int(page_indptr[b + 1]) - int(page_indptr[b])
        L = int(seq_lens[b])
        if n < 0 or L < 0:
            raise LoweringError("negative length")
        if n != (L + page_size - 1) // page_size:
            raise LoweringError(f"request {b}: {L} tokens need {(L + page_size - 1) // page_size} pages, got {n}")


def lower_page_table_bruteforce(page_size, page_indptr, page_indices, seq_lens):
    """Pure-Python loops; for small cases."""
    _check(page_size, page_indptr, seq_lens)
    kv_indptr = [0]
    kv_indices = []
    for b in range(len(seq_lens)):
        first = int(page_indptr[b])
        for t in range(int(seq_lens[b])):
            page = int(page_indices[first + t // page_size])
            kv_indices.append(page * page_size + t % page_size)
        kv_indptr.append(len(kv_indices))
    return kv_indptr, kv_indices


def lower_page_table(page_size, page_indptr, page_indices, seq_lens):
    """Same formula, one numpy expression per request; returns int64 arrays."""
    _check(page_size, page_indptr, seq_lens)
    page_indices = np.asarray(page_indices, np.int64)
    B = len(seq_lens)
    kv_indptr = np.zeros(B + 1, np.int64)
    parts = []
    for b in range(B):
        L = int(seq_lens[b])
        t = np.arange(L, dtype=np.int64)
        pages = page_indices[int(page_indptr[b]) + t // page_size]
        parts.append(pages * page_size + t % page_size)
        kv_indptr[b + 1] = kv_indptr[b] + L
    kv_indices = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return kv_indptr, kv_indices


def shared_prefix_pages(prefix_tokens: int, page_size: int):
    """Block-aligned prefix matching ("Track C · Document 10", block-size
    paragraph): only whole pages are shared.  Returns (shared pages, tokens
    left unshared)."""
    return prefix_tokens // page_size, prefix_tokens % page_size
