"""Prefix groups of one decode step, found in its page tables (test oracle,
integers only).

Prefix matching is exact and aligned to blocks, counted from the start of a
sequence ("Track C · Document 10 · Shrinking the footprint", block-size
paragraph and the table of prompt-layout mistakes: content that differs at
the top shares nothing; two system prompts make two separate trees).  A
prefix cache keeps what it matched as a radix tree keyed on shared
beginnings (same document, the comparison of engines; "GraniKV: asymmetric
KV cache paging for shared-prefix agents", the prefix placement flow, in
which the tree creates a node).  Each shared run is read once for all the
requests on it ("GraniKV", section 2), and each gets its own dispatcher
decision from its own realized batch (section 3: M_eff = realized batch x
GQA group).

Readings taken here (the pages give no procedure):

1. Only whole pages are shared: request b holds floor(L_b / p) full pages; a
   partly filled last page is its own.
2. Requests whose first full page is the same physical page are the members
   of one root group.
3. A group's run is the longest stretch of pages, from where its parent's
   run ends (the start of the sequence for a root), that every member holds
   in full and that is the same for all members.  Members that hold the
   page right after the run and agree on it form a child group (if there are
   two or more of them), recursively: the groups are the nodes of the radix
   tree of the requests' page lists that are shared by two or more requests.
4. A group of one request is no group.
5. Each group is planned as the step it would be on its own over its own
   run (``planner.plan`` over its members, with the run's tokens as the
   declared prefix): the gate, the DENSE / CASCADE choice and forced paths
   are that rule's.  Groups that come out PAGED are dissolved: their run is
   read by each member in the paged pass; their children are still planned.
6. Groups are numbered depth first, parents before children, siblings (and
   roots) in the order of their first member; members are listed in request
   order.  Each request's suffix is its tokens outside the runs of the kept
   groups on its path, in logical order.
"""
import numpy as np

from . import lowering, planner


def detect_prefix_groups(page_size, page_indptr, page_indices, seq_lens):
    """Groups of requests that share runs of whole pages, as a tree.

    Returns a list of dicts ``{"members", "start_pages", "shared_pages",
    "parent"}`` in depth-first order: the group's run is pages
    [start_pages, shared_pages) of each member's page list; ``parent`` is the
    index of the enclosing group (-1 for a root).
    """
    p = int(page_size)
    B = len(seq_lens)
    full = [int(seq_lens[b]) // p for b in range(B)]
    table = [list(int(x) for x in page_indices[int(page_indptr[b]):int(page_indptr[b + 1])]) for b in range(B)]
    out = []

    def split(members, at):
        """Members that hold page `at` in full, grouped by it, in order of
        first member; only groups of two or more."""
        by_page, order = {}, []
        for b in members:
            if full[b] <= at:
                continue
            pg = table[b][at]
            if pg not in by_page:
                by_page[pg] = []
                order.append(pg)
            by_page[pg].append(b)
        return [by_page[pg] for pg in order if len(by_page[pg]) >= 2]

    def visit(members, start, parent):
        end = min(full[b] for b in members)
        first = table[members[0]]
        for b in members[1:]:
            j = start
            while j < end and table[b][j] == first[j]:
                j += 1
            end = j
        me = len(out)
        out.append({"members": list(members), "start_pages": start, "shared_pages": end, "parent": parent})
        for child in split(members, end):
            visit(child, end, me)

    for root in split(range(B), 0):
        visit(root, 0, -1)
    return out


def plan_groups(*, H_q, H_kv, d, q_dtype, kv_dtype, page_size, page_indptr, page_indices, seq_lens,
                force_path, t_dense, gate_ratio, launch_bytes, prefix_placement=1):
    """The kept groups, each planned on its own run (the single-prefix rule
    without its cached-prefix allowance: this library's reading, measured).

    Returns ``(groups, path_of)``: ``groups`` lists the kept groups in
    depth-first order as dicts with ``members``, ``start_tokens``,
    ``prefix_tokens`` (the run's tokens), ``parent`` (index of the nearest
    kept ancestor, -1 if none), ``path``, ``m_eff`` and ``prefix_base``;
    ``path_of[b]`` lists the indices of the kept groups request b belongs
    to, outermost first.

    ``prefix_base`` (prefix placement, "GraniKV" section 1): with placement
    enabled, a run whose whole pages are consecutive physical pages is one
    stretch of consecutive slots, read as base + offset from the slot of its
    first token; otherwise -1.
    """
    p = int(page_size)
    B = len(seq_lens)
    kept, path_of = [], [[] for _ in range(B)]
    detected = detect_prefix_groups(page_size, page_indptr, page_indices, seq_lens)
    kept_at = {}  # detected index -> kept index (parents come before children)
    for i, g in enumerate(detected):
        members = g["members"]
        start, run = g["start_pages"] * p, (g["shared_pages"] - g["start_pages"]) * p
        dec = planner.plan(B=len(members), H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype,
                           page_size=page_size, seq_lens=[int(seq_lens[b]) - start for b in members],
                           shared_prefix_len=run, force_path=force_path, t_dense=t_dense,
                           gate_ratio=gate_ratio, launch_bytes=launch_bytes)
        if dec["path"] == planner.PAGED:
            continue
        a = g["parent"]  # nearest kept ancestor
        while a >= 0 and a not in kept_at:
            a = detected[a]["parent"]
        kept_at[i] = len(kept)
        for b in members:
            path_of[b].append(len(kept))
        pages = [int(x) for x in page_indices[int(page_indptr[members[0]]):int(page_indptr[members[0] + 1])]]
        run_pages = pages[g["start_pages"]:g["shared_pages"]]
        consecutive = all(run_pages[j + 1] == run_pages[j] + 1 for j in range(len(run_pages) - 1))
        base = run_pages[0] * p if (prefix_placement and consecutive) else -1
        kept.append({"members": list(members), "start_tokens": start, "prefix_tokens": dec["prefix_tokens"],
                     "parent": kept_at[a] if a >= 0 else -1, "path": dec["path"], "m_eff": dec["m_eff"],
                     "prefix_base": base})
    return kept, path_of


def lower_groups(page_size, page_indptr, page_indices, seq_lens, groups, path_of):
    """Token-flat indices of a grouped step.

    Returns ``(suffix_indptr, suffix_indices, prefix_indptr, prefix_indices)``:
    request b's suffix is its logical tokens outside the runs of its kept
    groups, in order; group g's prefix is the run's tokens
    [start_tokens, start_tokens + prefix_tokens) of its first member (the
    same slots for every member, by construction).
    """
    kv_indptr, kv_indices = lowering.lower_page_table(page_size, page_indptr, page_indices, seq_lens)
    B = len(seq_lens)
    suf_ptr = np.zeros(B + 1, np.int64)
    parts = []
    for b in range(B):
        mine = kv_indices[int(kv_indptr[b]):int(kv_indptr[b + 1])]
        keep = np.ones(len(mine), bool)
        for gi in path_of[b]:
            g = groups[gi]
            keep[g["start_tokens"]:g["start_tokens"] + g["prefix_tokens"]] = False
        parts.append(mine[keep])
        suf_ptr[b + 1] = suf_ptr[b] + len(parts[-1])
    pre_ptr = np.zeros(len(groups) + 1, np.int64)
    pre = []
    for i, g in enumerate(groups):
        b0 = g["members"][0]
        lo = int(kv_indptr[b0]) + g["start_tokens"]
        pre.append(kv_indices[lo:lo + g["prefix_tokens"]])
        pre_ptr[i + 1] = pre_ptr[i] + len(pre[-1])
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return suf_ptr, cat(parts), pre_ptr, cat(pre)
