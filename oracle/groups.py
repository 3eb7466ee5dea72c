"""Prefix groups of one decode step, found in its page tables (test oracle,
integers only).

Prefix matching is exact and aligned to blocks, counted from the start of a
sequence ("Track C · Document 10 · Shrinking the footprint", block-size
paragraph and the table of prompt-layout mistakes: content that differs at
the top shares nothing; two system prompts make two separate trees).  Several
such trees can be live in one decode step; each shared run is read once for
all the requests on it ("GraniKV: asymmetric KV cache paging for
shared-prefix agents", section 2) and each gets its own dispatcher decision
from its own realized batch (section 3: M_eff = realized batch x GQA group).

Readings taken here (the pages give no procedure):

1. Only whole pages are shared: request b holds floor(L_b / p) full pages; a
   partly filled last page is its own.
2. Requests whose first full page is the same physical page form one group
   (one level: a group is the set of requests on one tree's root page).
3. The group's shared pages are the longest leading run of page numbers that
   every member holds in full and that is the same for all members.
4. A group of one request is no group.
5. Each group is planned as the step it would be on its own (``planner.plan``
   over the members, with the group's shared tokens as the declared prefix):
   the gate, the DENSE / CASCADE choice and forced paths are that rule's.
   Groups that come out PAGED are dissolved: their members read every token
   in the paged pass.
6. Groups are numbered in the order of their first member; members are listed
   in request order.  Each request's suffix is its tokens after its kept
   group's shared tokens (all of its tokens if it is in no kept group).
"""
import numpy as np

from . import lowering, planner


def detect_prefix_groups(page_size, page_indptr, page_indices, seq_lens):
    """Groups of requests that share leading whole pages.

    Returns a list of dicts ``{"members": [b, ...], "shared_pages": k}``, in
    the order of each group's first member; only groups of two or more.
    """
    p = int(page_size)
    B = len(seq_lens)
    full = [int(seq_lens[b]) // p for b in range(B)]
    table = [list(int(x) for x in page_indices[int(page_indptr[b]):int(page_indptr[b + 1])]) for b in range(B)]
    by_root = {}
    order = []
    for b in range(B):
        if full[b] == 0:
            continue
        root = table[b][0]
        if root not in by_root:
            by_root[root] = []
            order.append(root)
        by_root[root].append(b)
    groups = []
    for root in order:
        members = by_root[root]
        if len(members) < 2:
            continue
        k = min(full[b] for b in members)
        first = table[members[0]]
        for b in members[1:]:
            j = 0
            while j < k and table[b][j] == first[j]:
                j += 1
            k = j
        groups.append({"members": members, "shared_pages": k})
    return groups


def plan_groups(*, H_q, H_kv, d, q_dtype, kv_dtype, page_size, page_indptr, page_indices, seq_lens,
                force_path, t_dense, gate_ratio, launch_bytes):
    """The kept groups, each planned on its own.

    Returns ``(groups, group_of)``: ``groups`` lists the kept groups as dicts
    with ``members``, ``shared_pages``, ``prefix_tokens`` (= shared_pages x p),
    ``path`` and ``m_eff``; ``group_of[b]`` is the index of request b's kept
    group or -1.
    """
    B = len(seq_lens)
    kept = []
    group_of = [-1] * B
    for g in detect_prefix_groups(page_size, page_indptr, page_indices, seq_lens):
        members = g["members"]
        dec = planner.plan(B=len(members), H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype,
                           page_size=page_size, seq_lens=[int(seq_lens[b]) for b in members],
                           shared_prefix_len=g["shared_pages"] * int(page_size), force_path=force_path,
                           t_dense=t_dense, gate_ratio=gate_ratio, launch_bytes=launch_bytes)
        if dec["path"] == planner.PAGED:
            continue
        for b in members:
            group_of[b] = len(kept)
        kept.append({"members": list(members), "shared_pages": g["shared_pages"],
                     "prefix_tokens": dec["prefix_tokens"], "path": dec["path"], "m_eff": dec["m_eff"]})
    return kept, group_of


def lower_groups(page_size, page_indptr, page_indices, seq_lens, groups, group_of):
    """Token-flat indices of a grouped step.

    Returns ``(suffix_indptr, suffix_indices, prefix_indptr, prefix_indices)``:
    request b's suffix is its logical tokens [P, L_b) with P its kept group's
    shared tokens (0 if none); group g's prefix is the first P_g tokens of its
    first member (the same slots for every member, by construction).
    """
    kv_indptr, kv_indices = lowering.lower_page_table(page_size, page_indptr, page_indices, seq_lens)
    B = len(seq_lens)
    suf_ptr = np.zeros(B + 1, np.int64)
    parts = []
    for b in range(B):
        skip = groups[group_of[b]]["prefix_tokens"] if group_of[b] >= 0 else 0
        parts.append(kv_indices[int(kv_indptr[b]) + skip:int(kv_indptr[b + 1])])
        suf_ptr[b + 1] = suf_ptr[b] + len(parts[-1])
    pre_ptr = np.zeros(len(groups) + 1, np.int64)
    pre = []
    for i, g in enumerate(groups):
        b0 = g["members"][0]
        pre.append(kv_indices[int(kv_indptr[b0]):int(kv_indptr[b0]) + g["prefix_tokens"]])
        pre_ptr[i + 1] = pre_ptr[i] + len(pre[-1])
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return suf_ptr, cat(parts), pre_ptr, cat(pre)
