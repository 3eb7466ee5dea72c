"""The synthetic pools hold each request's logical tokens where the oracle's
lowering of its page table says they are (CPU)."""
import numpy as np
import pytest
import torch

from oracle import lowering as ol
from workloads import make_decode_batch, relayout


def _gathered_matches_logical(batch):
    kv_indptr, kv_indices = ol.lower_page_table(batch.page_size, batch.page_indptr,
                                                batch.page_indices, batch.seq_lens)
    idx = torch.from_numpy(kv_indices)
    for b in range(batch.B):
        k, v = batch.logical_kv(b)
        sl = idx[kv_indptr[b]:kv_indptr[b + 1]]
        assert torch.equal(batch.k_pool[sl].view(torch.uint8), k.contiguous().view(torch.uint8))
        assert torch.equal(batch.v_pool[sl].view(torch.uint8), v.contiguous().view(torch.uint8))
    return kv_indices


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("layout", ["shared", "unique"])
@pytest.mark.parametrize("p", [1, 5, 16])
def test_pool_holds_logical_tokens(kv, layout, p):
    q = "f32" if kv == "f32" else "bf16"
    b = make_decode_batch(seed=5, B=5, H_q=8, H_kv=2, d=64, own_len=(0, 40), prefix_len=37,
                          q_dtype=q, kv_dtype=kv, page_size=p, layout=layout, pool_factor=2)
    kv_indices = _gathered_matches_logical(b)
    if layout == "shared" and p <= 37:
        # every request's first floor(P/p) pages are the same physical pages
        n = 37 // p
        first = b.page_indices[b.page_indptr[0]:b.page_indptr[0] + n]
        for r in range(b.B):
            assert np.array_equal(b.page_indices[b.page_indptr[r]:b.page_indptr[r] + n], first)
    else:
        assert len(np.unique(kv_indices)) == len(kv_indices)


def test_relayout_keeps_values_and_moves_pages():
    b = make_decode_batch(seed=9, B=4, H_q=8, H_kv=2, d=64, own_len=(64, 256),
                          q_dtype="f32", kv_dtype="f32", page_size=16, pool_pages=128)
    b1 = relayout(b, page_size=1, seed=2001, pool_pages=2048)
    _gathered_matches_logical(b)
    _gathered_matches_logical(b1)
    assert b1.k_tokens is b.k_tokens and b1.num_slots == 2048 and b.num_slots == 2048


def test_fp8_codes_finite_and_scaled():
    b = make_decode_batch(seed=1, B=3, H_q=16, H_kv=2, d=128, own_len=(100, 200),
                          q_dtype="bf16", kv_dtype="fp8", page_size=16, pool_factor=2)
    codes = b.k_tokens.view(torch.uint8)
    assert not ((codes & 0x7F) == 0x7F).any()
    # the largest magnitude of each head reaches the top code (448)
    mags = (codes & 0x7F).view(-1, 2, 128)
    assert (mags.amax(dim=(0, 2)) == 0x7E).all()
    assert b.k_scale.shape == (2,) and (b.k_scale > 0).all()


def test_unused_slots_are_poison():
    b = make_decode_batch(seed=2, B=2, H_q=4, H_kv=1, d=64, own_len=(3, 3), q_dtype="f32",
                          kv_dtype="f32", page_size=16, pool_pages=8)
    used = set()
    kv_indptr, kv_indices = ol.lower_page_table(16, b.page_indptr, b.page_indices, b.seq_lens)
    used.update(kv_indices.tolist())
    unused = [s for s in range(b.num_slots) if s not in used]
    assert torch.isnan(b.k_pool[unused]).all()


# ------------------------------------------------------------ grouped batches --

from workloads import make_grouped_batch  # noqa: E402
from oracle import groups as og  # noqa: E402


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("p", [1, 4, 16])
def test_grouped_pool_holds_logical_tokens_and_the_groups(kv, p):
    groups = [(4, 37), (3, 16), (2, 5)]
    b = make_grouped_batch(seed=9, B=12, H_q=8, H_kv=2, d=64, groups=groups, own_len=(0, 30), page_size=p,
                           kv_dtype=kv, pool_factor=2)
    _gathered_matches_logical(b)
    # the requests drawn on a prefix share exactly its whole pages, so the
    # oracle's grouping finds the drawn groups (a prefix shorter than one
    # page shares nothing)
    found = {tuple(g["members"]): g["shared_pages"] for g in
             og.detect_prefix_groups(p, b.page_indptr, b.page_indices, b.seq_lens)}
    want = {}
    for g, (n, P) in enumerate(groups):
        members = tuple(int(x) for x in np.flatnonzero(b.group_of == g))
        assert len(members) == n
        if P // p >= 1:
            want[members] = P // p
    # own tokens never share a page, but a whole-page prefix run can be
    # followed by nothing else in common
    assert found == want, (found, want)


def test_grouped_unused_slots_are_poison():
    b = make_grouped_batch(seed=3, B=6, H_q=8, H_kv=2, d=64, groups=[(3, 20)], own_len=(1, 9), page_size=4,
                           kv_dtype="bf16", pool_factor=3)
    kv_indptr, kv_indices = ol.lower_page_table(b.page_size, b.page_indptr, b.page_indices, b.seq_lens)
    used = np.zeros(b.k_pool.shape[0], bool)
    used[kv_indices] = True
    assert torch.isnan(b.k_pool[torch.from_numpy(~used)].float()).all()


from workloads import make_tree_batch  # noqa: E402


@pytest.mark.parametrize("p", [1, 5, 16])
def test_tree_pool_holds_logical_tokens_and_the_tree(p):
    tree = [(9, 40, -1), (4, 21, 0), (3, 16, 0), (2, 9, 1), (3, 33, -1)]
    b = make_tree_batch(seed=4, B=14, H_q=8, H_kv=2, d=64, tree=tree, own_len=(0, 20), page_size=p,
                        kv_dtype="bf16", pool_factor=2)
    _gathered_matches_logical(b)
    # every drawn node whose members share at least one whole page more than
    # its parent's is a group of the oracle's tree with exactly those members
    found = {tuple(g["members"]) for g in og.detect_prefix_groups(p, b.page_indptr, b.page_indices, b.seq_lens)}
    cum = {}
    for i, (n, T, parent) in enumerate(tree):
        cum[i] = T + (cum[parent] if parent >= 0 else 0)
        base = cum[parent] if parent >= 0 else 0
        if cum[i] // p > base // p:
            assert tuple(b.node_members[i]) in found, (i, b.node_members[i], found)
