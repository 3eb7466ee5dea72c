"""The checked library (libpkv_checked.so) on the GPU, through the C ABI.

It runs the same kernels as libpkv.so, so every step it lets through must
give the release library's bits; and a step whose index arrays do not
describe the planned batch or reach outside the pool is refused with
EINVAL / ERANGE before anything is launched (its outputs stay untouched).

Each refused array reaches at most one page past the pool the call declares,
and the pools here are allocated one page (or more) larger than declared, so
even a check that let such an array through could not send a kernel outside
device memory.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _imports():
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_decode_batch, make_grouped_batch
    return pkv, DeviceBatch, make_decode_batch, make_grouped_batch


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _slack_pool(pkv, db, extra_pages=1):
    """db's pool copied into tensors extra_pages pages longer than the pool
    the returned pkv_pool declares."""
    n = db.k_pool.shape[0]
    extra = extra_pages * db.page_size
    k = torch.zeros((n + extra,) + tuple(db.k_pool.shape[1:]), dtype=db.k_pool.dtype, device=db.device)
    v = torch.zeros_like(k)
    k[:n] = db.k_pool
    v[:n] = db.v_pool
    return pkv.make_pool(k[:n], v[:n], db.page_size, db.k_scale, db.v_scale), (k, v)


def _sentinel(t):
    return t.fill_(7.0)


def _refused(pkv, fn, status, what):
    with pytest.raises(pkv.PkvError) as e:
        fn()
    assert e.value.name == status, f"{what}: {e.value}"


def _batches(make_decode_batch):
    # a paged step (requests cut by chunk edges, an empty request) and a
    # shared-prefix step
    paged = make_decode_batch(seed=71, B=6, H_q=8, H_kv=2, d=128, own_len=(0, 700), page_size=16, pool_factor=2)
    casc = make_decode_batch(seed=72, B=24, H_q=32, H_kv=8, d=128, own_len=(20, 200), prefix_len=256,
                             page_size=16, pool_factor=2)
    return paged, casc


def test_checked_library_gives_the_release_bits():
    pkv, DeviceBatch, make_decode_batch, make_grouped_batch = _imports()
    paged, casc = _batches(make_decode_batch)
    grouped = make_grouped_batch(seed=73, B=24, H_q=32, H_kv=8, d=128, groups=[(8, 700), (5, 300)],
                                 own_len=(0, 150), page_size=16)
    runs = []
    db = DeviceBatch.from_batch(paged)
    runs.append(("paged", db, lambda: db.plan(force_path=0, tuning=dict(target_workgroups=64)),
                 lambda plan: db.paged(plan)))
    runs.append(("paged, page table", db, lambda: db.plan(force_path=0, tuning=dict(target_workgroups=64)),
                 lambda plan: db.paged_pages(plan)))
    dc = DeviceBatch.from_batch(casc)
    for force in (1, 2):
        runs.append((f"cascade step force={force}", dc,
                     lambda force=force: dc.plan(shared_prefix_len=casc.prefix_len, force_path=force),
                     lambda plan: dc.step(plan)))
    runs.append(("prefix pass", dc, lambda: dc.plan(shared_prefix_len=casc.prefix_len, force_path=2),
                 lambda plan: dc.prefix(plan)))
    runs.append(("no-alloc step", dc, lambda: dc.plan(shared_prefix_len=casc.prefix_len, force_path=2),
                 lambda plan: _noalloc(pkv, dc, plan)))
    dg = DeviceBatch.from_batch(grouped)
    runs.append(("grouped step", dg, lambda: dg.plan_grouped(tuning=dict(gate_ratio=0)),
                 lambda plan: dg.step_grouped(plan, dg.metadata(plan))))
    for what, d, make_plan, run in runs:
        say(f"checked vs release: {what}")
        plan = make_plan()
        o, lse = run(plan)
        torch.cuda.synchronize()
        with pkv.checked_library():
            plan_c = make_plan()
            assert plan_c.info == plan.info
            o_c, lse_c = run(plan_c)
        torch.cuda.synchronize()
        assert same_bits(o, o_c) and same_bits(lse, lse_c), what


def _noalloc(pkv, db, plan):
    o, lse = db.new_out(), db.new_lse()
    pkv.pkv_decode_step_noalloc(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, db.sm_scale, o, lse)
    return o, lse


def test_checked_library_refuses_bad_index_arrays():
    pkv, DeviceBatch, make_decode_batch, make_grouped_batch = _imports()
    paged, casc = _batches(make_decode_batch)
    db = DeviceBatch.from_batch(paged)
    db.pool, keep = _slack_pool(pkv, db)
    n_slots, p = db.pool.num_slots, db.page_size
    first = next(b for b in range(db.B) if db.seq_lens_host[b] > 0)  # a request with tokens
    o, lse = _sentinel(db.new_out()), _sentinel(db.new_lse())
    with pkv.checked_library():
        plan = db.plan(force_path=0, tuning=dict(target_workgroups=64))
        ws = db.workspace(plan)
        say("checked: a valid step passes")
        db.paged(plan, db.new_out(), None, db.new_lse(), ws)
        torch.cuda.synchronize()
        # a slot one past the pool (inside the allocation)
        ix = db.kv_indices.clone()
        ix[int(db.kv_indptr_host[first]) + int(db.seq_lens_host[first]) // 2] = n_slots
        say("checked: slot past the pool")
        _refused(pkv, lambda: pkv.pkv_paged_decode_attn(plan, db.q, db.pool, db.kv_indptr, ix, db.sm_scale, o, None,
                                                        lse, ws), "ERANGE", "slot past the pool")
        _refused(pkv, lambda: pkv.pkv_decode_step(plan, db.q, db.pool, db.kv_indptr, ix, db.sm_scale, o, lse, ws),
                 "ERANGE", "decode step, slot past the pool")
        # a request boundary moved by one (the total unchanged)
        ip = db.kv_indptr.clone()
        ip[1] += 1
        say("checked: kv_indptr not the planned one")
        _refused(pkv, lambda: pkv.pkv_paged_decode_attn(plan, db.q, db.pool, ip, db.kv_indices, db.sm_scale, o,
                                                        None, lse, ws), "EINVAL", "moved boundary")
        # the page-table entry: a page one past the pool, a request one page short
        pages = db.page_indices.clone()
        pages[int(db.page_indptr_host[first])] = n_slots // p
        say("checked: page past the pool")
        _refused(pkv, lambda: pkv.pkv_paged_decode_attn_pages(plan, db.q, db.pool, db.kv_indptr, db.page_indptr,
                                                              pages, db.sm_scale, o, None, lse, ws),
                 "ERANGE", "page past the pool")
        pptr = db.page_indptr.clone()
        pptr[first + 1:] -= 1
        say("checked: page list one short")
        _refused(pkv, lambda: pkv.pkv_paged_decode_attn_pages(plan, db.q, db.pool, db.kv_indptr, pptr,
                                                              db.page_indices, db.sm_scale, o, None, lse, ws),
                 "ERANGE", "page list one short")
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all()), "a refused call wrote its outputs"

    dc = DeviceBatch.from_batch(casc)
    dc.pool, keep2 = _slack_pool(pkv, dc)
    n_slots = dc.pool.num_slots
    o, lse = _sentinel(dc.new_out()), _sentinel(dc.new_lse())
    o_p = _sentinel(dc.new_out(torch.float32))
    with pkv.checked_library():
        plan = dc.plan(shared_prefix_len=casc.prefix_len, force_path=2)
        assert plan.info["prefix_base"] == -1  # the prefix pass reads its slots by index
        ws = dc.workspace(plan)
        pre = dc.prefix_indices(plan).clone()
        pre[5] = n_slots
        say("checked: prefix slot past the pool")
        _refused(pkv, lambda: pkv.pkv_cascade_prefix_attn(plan, dc.q, dc.pool, pre, plan.info["prefix_tokens"],
                                                          dc.sm_scale, o_p, lse, ws), "ERANGE", "prefix slot")
        ix = dc.kv_indices.clone()
        ix[7] = n_slots  # a prefix position of request 0
        _refused(pkv, lambda: pkv.pkv_decode_step(plan, dc.q, dc.pool, dc.kv_indptr, ix, dc.sm_scale, o, lse, ws),
                 "ERANGE", "cascade step, prefix slot")
        _refused(pkv, lambda: pkv.pkv_decode_step_noalloc(plan, dc.q, dc.pool, dc.kv_indptr, ix, dc.sm_scale, o,
                                                          lse), "ERANGE", "no-alloc step, prefix slot")
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all()) and bool((o_p == 7.0).all()), \
        "a refused call wrote its outputs"

    grouped = make_grouped_batch(seed=74, B=16, H_q=32, H_kv=8, d=128, groups=[(6, 500)], own_len=(1, 100),
                                 page_size=16)
    dg = DeviceBatch.from_batch(grouped)
    dg.pool, keep3 = _slack_pool(pkv, dg)
    o, lse = _sentinel(dg.new_out()), _sentinel(dg.new_lse())
    with pkv.checked_library():
        plan = dg.plan_grouped(tuning=dict(gate_ratio=0))
        assert plan.info["num_groups"] == 1
        meta = dg.metadata(plan)
        block = pkv.split_metadata(pkv.pkv_plan_metadata(plan), dg.B, plan.info["num_groups"])
        n_suffix = len(block["suffix_indices"])
        assert n_suffix > 0
        bad = meta.clone()
        bad[dg.B + 1 + n_suffix // 2] = dg.pool.num_slots  # a suffix slot past the pool
        say("checked: grouped metadata not the planned block")
        _refused(pkv, lambda: dg.step_grouped(plan, bad, o, lse), "EINVAL", "grouped metadata")
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all()), "a refused call wrote its outputs"
    del keep, keep2, keep3
