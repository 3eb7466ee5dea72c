"""pkv_decode_step_noalloc (the decode step whose workspace is the library's
own device scratch array, for callers that cannot allocate) against
pkv_decode_step with a caller workspace, through the C ABI: the same kernels
run, so results must be bitwise equal, and both within tolerance of the
oracle.  Two calls in a row, the second with a smaller input, so the second
reuses scratch that still holds the first call's partial states."""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check_oracle(kv_dtype, o, lse, o_ref, lse_ref, what):
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), what
    assert np.abs(o - o_ref).max() <= 2e-2, what
    assert (np.abs(lse[fin] - lse_ref[fin]).max() if fin.any() else 0.0) <= 2e-2, what


def _run_both(pkv, DeviceBatch, ob, batch, shared_prefix, force_path, what, tuning=None):
    db = DeviceBatch.from_batch(batch)
    plan = db.plan(shared_prefix_len=shared_prefix, force_path=force_path, tuning=tuning)
    assert 0 < plan.info["workspace_bytes"] <= pkv.NOALLOC_SCRATCH_BYTES, plan.info
    say(f"{what}: plan {plan.info['path_name']} workspace {plan.info['workspace_bytes']} B")
    o_ref, lse_ref = ob.batch_reference(batch)
    o_n, l_n = db.new_out(), db.new_lse()
    o_n.fill_(float("nan"))
    l_n.fill_(float("nan"))
    say(f"{what}: pkv_decode_step_noalloc")
    pkv.pkv_decode_step_noalloc(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, db.sm_scale, o_n, l_n)
    torch.cuda.synchronize()
    say(f"{what}: pkv_decode_step with a workspace")
    ws = db.workspace(plan)
    ws.fill_(0xFF)
    o_w, l_w = db.step(plan, ws=ws)
    torch.cuda.synchronize()
    assert _same_bits(o_n, o_w) and _same_bits(l_n, l_w), f"{what}: no-alloc step differs from the workspace step"
    _check_oracle(batch.kv_dtype, o_n, l_n, o_ref, lse_ref, what)
    return plan


def test_noalloc_matches_workspace_step_two_calls_second_smaller():
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from oracle import batch as ob
    from workloads import make_decode_batch
    big = make_decode_batch(seed=71, B=96, H_q=32, H_kv=8, d=128, own_len=(64, 512), prefix_len=2048,
                            page_size=16)
    p1 = _run_both(pkv, DeviceBatch, ob, big, 2048, -1, "first call, B=96 shared prefix")
    small = make_decode_batch(seed=72, B=7, H_q=32, H_kv=8, d=128, own_len=(30, 300), prefix_len=256,
                              page_size=16)
    p2 = _run_both(pkv, DeviceBatch, ob, small, 256, 2, "second call, B=7 shared prefix")
    assert p2.info["workspace_bytes"] < p1.info["workspace_bytes"]


def test_noalloc_paged_and_fp8_steps():
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from oracle import batch as ob
    from workloads import make_decode_batch
    b = make_decode_batch(seed=73, B=4, H_q=32, H_kv=8, d=128, own_len=(3000, 4096), page_size=1)
    plan = _run_both(pkv, DeviceBatch, ob, b, 0, -1, "paged bf16, requests split over chunks")
    assert plan.info["num_splits"] > 1
    f = make_decode_batch(seed=74, B=3, H_q=64, H_kv=8, d=128, own_len=(500, 2000), page_size=16, kv_dtype="fp8",
                          pool_factor=2)
    _run_both(pkv, DeviceBatch, ob, f, 0, -1, "paged fp8, smaller")


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_decode_batch
    b = make_decode_batch(seed=75, B=32, H_q=32, H_kv=8, d=128, own_len=(4096, 4096), page_size=128)
    db = DeviceBatch.from_batch(b)
    plan = db.plan(tuning=dict(min_split_tokens=16, target_workgroups=1 << 20))
    assert plan.info["workspace_bytes"] > pkv.NOALLOC_SCRATCH_BYTES
    o = db.new_out()
    o.fill_(1.0)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_step_noalloc(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, db.sm_scale, o)
    assert e.value.name == "EWORKSPACE"
    torch.cuda.synchronize()
    assert bool((o == 1.0).all()), "a refused call wrote its output"
