"""GPU parity of the HIP path against the float64 oracle (MI355X, gfx950).

Tolerances (fixed before any kernel ran):
* fp32 K/V: per output row max|o - o_ref| <= 1e-5 * max|o_ref row|, and
  |lse - lse_ref| <= 1e-5 * max(1, |lse_ref|);
* bf16 / fp8 K/V: elementwise |o - o_ref| <= 2e-2 and |lse - lse_ref| <= 2e-2.
Indexing and planning are bit exact (tested on the CPU).  The paged path
orders its arithmetic by logical token position, so its output must also be
bitwise identical across page size, page permutation and prefix layout.

Sizes: small cases the oracle finishes in seconds that still span several
work items and ragged tails; the full workloads at the launch configuration
the bench times, checked on sampled requests.
"""
import math
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
    from oracle import batch as ob
    from oracle import attention as oa
    from workloads import make_config, make_decode_batch, relayout
    return pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout


def check_close(kv_dtype, o, lse, o_ref, lse_ref, what):
    o = o.detach().float().cpu().double().numpy().reshape(o_ref.shape)
    lse = lse.detach().float().cpu().double().numpy().reshape(lse_ref.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf pattern differs"
    if kv_dtype == "f32":
        err_o = np.abs(o - o_ref).max(axis=-1)
        bound = 1e-5 * np.maximum(np.abs(o_ref).max(axis=-1), 1e-30)
        assert (err_o <= bound).all(), f"{what}: o rel err {(err_o / bound).max() * 1e-5:.3g}"
        err_l = np.abs(lse[fin] - lse_ref[fin])   # only finite entries: no inf - inf
        assert (err_l <= 1e-5 * np.maximum(1, np.abs(lse_ref[fin]))).all(), f"{what}: lse err {err_l.max():.3g}"
    else:
        err_o = np.abs(o - o_ref).max()
        err_l = np.abs(lse[fin] - lse_ref[fin]).max() if fin.any() else 0.0
        assert err_o <= 2e-2, f"{what}: o err {err_o:.4g}"
        assert err_l <= 2e-2, f"{what}: lse err {err_l:.4g}"
    assert not np.isnan(o).any(), f"{what}: NaN in output"


def run_paged(DeviceBatch, batch, tuning=None, want_f32=False):
    db = DeviceBatch.from_batch(batch)
    plan = db.plan(force_path=0, tuning=tuning)
    o, lse = db.paged(plan, want_f32=want_f32)
    torch.cuda.synchronize()
    return o, lse, plan


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def spread_requests(batch, plan, n=32):
    """n requests spread over the batch, half of them (where there are that
    many) requests that the plan's paged pass cuts at chunk edges (their
    partial states go through the combine), half whole ones."""
    P = plan.info["prefix_tokens"]
    C = plan.info["split_tokens"]
    own = np.asarray(batch.seq_lens, np.int64) - P
    start = np.concatenate([[0], np.cumsum(own)[:-1]])
    cut = [b for b in range(batch.B) if own[b] > 0 and (start[b] + own[b] - 1) // C != start[b] // C]
    whole = [b for b in range(batch.B) if b not in set(cut)]
    pick = lambda xs, k: [xs[i] for i in np.linspace(0, len(xs) - 1, min(k, len(xs))).astype(int)] if xs else []
    reqs = sorted(set(pick(cut, n // 2)) | set(pick(whole, n - min(n // 2, len(cut)))) | {0, batch.B - 1})
    return reqs, sum(1 for b in reqs if b in set(cut))


# ----------------------------------------------------------------- c1 ------

def test_c1_tiny_fp32_page16_and_page1():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b16 = make_config("c1")
    b1 = relayout(b16, page_size=1, seed=2001, pool_pages=2048)
    o_ref, lse_ref = ob.batch_reference(b16)
    say("c1 p=16 paged_decode_attn")
    o16, l16, plan = run_paged(DeviceBatch, b16)
    check_close("f32", o16, l16, o_ref, lse_ref, "c1 p=16")
    say("c1 p=1 paged_decode_attn")
    o1, l1, _ = run_paged(DeviceBatch, b1)
    check_close("f32", o1, l1, o_ref, lse_ref, "c1 p=1")
    assert same_bits(o16, o1) and same_bits(l16, l1), "page size changed the bits"
    # many small splits: the split-K reduction path at fp32 precision
    say("c1 p=16 forced splits")
    os_, ls_, plan_s = run_paged(DeviceBatch, b16, tuning=dict(min_split_tokens=64, target_workgroups=4096))
    assert plan_s.info["num_splits"] > 1
    check_close("f32", os_, ls_, o_ref, lse_ref, "c1 split")


# ----------------------------------------------------------------- c2 ------

def test_c2_shape_small_all_layouts():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    base = make_config("c2", B=3, own_len=(4096, 4096), page_size=128)
    o_ref, lse_ref = ob.batch_reference(base)
    outs = []
    for p, perm in ((128, "random"), (1, "random"), (1, "identity"), (16, "random")):
        b = relayout(base, page_size=p, seed=2002, perm=perm)
        say(f"c2-small p={p} {perm}")
        o, lse, plan = run_paged(DeviceBatch, b)
        check_close("bf16", o, lse, o_ref, lse_ref, f"c2 small p={p} {perm}")
        outs.append((o, lse))
    for o, lse in outs[1:]:
        assert same_bits(outs[0][0], o) and same_bits(outs[0][1], lse)


def test_c2_full_sampled_page1_vs_page128():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b128 = make_config("c2")
    b1 = relayout(b128, page_size=1, seed=2002)
    say("c2 full: oracle over every request")
    o_ref, lse_ref = ob.batch_reference(b128)
    say("c2 full p=128")
    o128, l128, plan = run_paged(DeviceBatch, b128)
    assert plan.info["num_splits"] > 1
    check_close("bf16", o128, l128, o_ref, lse_ref, "c2 p=128")
    del b128
    say("c2 full p=1")
    o1, l1, _ = run_paged(DeviceBatch, b1)
    assert same_bits(o128, o1) and same_bits(l128, l1), "page 1 vs 128 differ"


# ----------------------------------------------------------------- c5 ------

def test_c5_fp8_small():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c5", B=3, own_len=(1000, 3000))
    o_ref, lse_ref = ob.batch_reference(b)
    say("c5-small fp8")
    o, lse, plan = run_paged(DeviceBatch, b)
    check_close("fp8", o, lse, o_ref, lse_ref, "c5 small")
    b2 = relayout(b, page_size=1, seed=2005, pool_factor=2)
    say("c5-small fp8 p=1")
    o2, l2, _ = run_paged(DeviceBatch, b2)
    assert same_bits(o, o2) and same_bits(lse, l2)


def test_c5_full_every_request():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c5")
    say("c5 full: oracle over every request")
    o_ref, lse_ref = ob.batch_reference(b)
    say("c5 full fp8")
    o, lse, plan = run_paged(DeviceBatch, b)
    assert plan.info["num_splits"] > 1
    check_close("fp8", o, lse, o_ref, lse_ref, "c5 full")


# --------------------------------------------------------- shared prefix ---

def _cascade_paths(DeviceBatch, batch, ob, reqs=None):
    db = DeviceBatch.from_batch(batch)
    P = batch.prefix_len
    res = {}
    for force in (0, 1, 2):
        plan = db.plan(shared_prefix_len=P, force_path=force)
        say(f"decode_step force={force} B={batch.B} P={P} layout={batch.layout}")
        o, lse = db.step(plan)
        torch.cuda.synchronize()
        res[force] = (o, lse, plan)
    return db, res


def test_cascade_small_all_paths_and_layouts():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    for B, P, own in ((24, 512, (0, 100)), (5, 1000, (1, 3)), (3, 40, (30, 70))):
        shared = make_decode_batch(seed=31 + B, B=B, H_q=32, H_kv=8, d=128, own_len=own, prefix_len=P,
                                   page_size=16, layout="shared")
        o_ref, lse_ref = ob.batch_reference(shared)
        db, res = _cascade_paths(DeviceBatch, shared, ob)
        for force, (o, lse, plan) in res.items():
            check_close("bf16", o, lse, o_ref, lse_ref, f"B={B} P={P} path={force}")
        # the prefix pass alone, against the oracle over the first tokens
        plan = res[2][2]
        n = plan.info["prefix_tokens"]
        say(f"cascade_prefix_attn B={B} n={n}")
        o_p, lse_p = db.prefix(plan)
        torch.cuda.synchronize()
        op_ref, lp_ref = ob.prefix_reference(shared, n)
        check_close("bf16", o_p, lse_p, op_ref, lp_ref, f"prefix B={B}")
        # paged over unique copies of the prefix, planned alike (the same
        # declared prefix length): same bits as over shared pages
        unique = relayout(shared, page_size=16, seed=77, layout="unique")
        say(f"paged unique B={B}")
        du = DeviceBatch.from_batch(unique)
        ou, lu = du.paged(du.plan(shared_prefix_len=P, force_path=0))
        torch.cuda.synchronize()
        assert same_bits(ou, res[0][0]) and same_bits(lu, res[0][1]), "layout changed the bits"


def _full_prefix_case(name):
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config(name)
    db = DeviceBatch.from_batch(b)
    plan = db.plan(shared_prefix_len=b.prefix_len)
    reqs, n_cut = spread_requests(b, plan)
    assert len(reqs) >= 32 and n_cut >= 8, (len(reqs), n_cut)
    say(f"{name} full: oracle over {len(reqs)} requests ({n_cut} cut by chunk edges)")
    o_ref, lse_ref = ob.batch_reference(b, requests=reqs)
    say(f"{name} full plan={plan.info['path_name']} decode_step")
    o, lse = db.step(plan)
    torch.cuda.synchronize()
    check_close("bf16", o[reqs], lse[reqs], o_ref, lse_ref, f"{name} {plan.info['path_name']}")
    outs = {plan.info["path"]: (o, lse)}
    for force in (0, 1, 2):
        if force in outs:
            continue
        p2 = db.plan(shared_prefix_len=b.prefix_len, force_path=force)
        say(f"{name} full forced {p2.info['path_name']}")
        o2, l2 = db.step(p2)
        torch.cuda.synchronize()
        check_close("bf16", o2[reqs], l2[reqs], o_ref, lse_ref, f"{name} {p2.info['path_name']}")
        outs[force] = (o2, l2)
    return plan


def test_c3_full_sampled():
    plan = _full_prefix_case("c3")
    assert plan.info["m_eff"] == 1024


def test_c4_full_sampled():
    plan = _full_prefix_case("c4")
    assert plan.info["m_eff"] == 2048


# ------------------------------------------------------------ edge cases ---

@pytest.mark.parametrize("case", [
    dict(B=6, H_q=16, H_kv=2, d=128, own_len=(0, 3), q_dtype="bf16", kv_dtype="bf16", page_size=1),
    dict(B=4, H_q=3, H_kv=3, d=128, own_len=(1, 900), q_dtype="bf16", kv_dtype="bf16", page_size=7),
    dict(B=5, H_q=8, H_kv=8, d=64, own_len=(100, 1500), q_dtype="bf16", kv_dtype="bf16", page_size=16),
    dict(B=3, H_q=16, H_kv=8, d=128, own_len=(2000, 2100), q_dtype="bf16", kv_dtype="bf16", page_size=32),
    dict(B=2, H_q=64, H_kv=8, d=64, own_len=(300, 700), q_dtype="bf16", kv_dtype="fp8", page_size=16),
    dict(B=3, H_q=12, H_kv=6, d=128, own_len=(50, 400), q_dtype="bf16", kv_dtype="fp8", page_size=8),
    dict(B=2, H_q=4, H_kv=1, d=64, own_len=(1, 700), q_dtype="f32", kv_dtype="f32", page_size=3),
    dict(B=3, H_q=16, H_kv=2, d=128, own_len=(100, 900), q_dtype="f32", kv_dtype="f32", page_size=16),
    dict(B=1, H_q=32, H_kv=4, d=128, own_len=(1, 1), q_dtype="bf16", kv_dtype="bf16", page_size=16),
])
@pytest.mark.parametrize("splits", ["one", "many", "balanced"])
def test_edge_shapes(case, splits):
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_decode_batch(seed=sum(case["own_len"]) + case["H_q"], pool_factor=2, **case)
    tuning = {"one": dict(min_split_tokens=2048, target_workgroups=1),
              "many": dict(min_split_tokens=16, target_workgroups=100000),
              "balanced": dict(min_split_tokens=16, target_workgroups=7)}[splits]
    o_ref, lse_ref = ob.batch_reference(b)
    say(f"edge {case} splits={splits}")
    o, lse, plan = run_paged(DeviceBatch, b, tuning=tuning)
    check_close(case["kv_dtype"], o, lse, o_ref, lse_ref, f"edge {case} {splits}")
    if case["kv_dtype"] != "f32":
        of, lf, _ = run_paged(DeviceBatch, b, tuning=tuning, want_f32=True)
        check_close(case["kv_dtype"], of, lf, o_ref, lse_ref, f"edge f32-out {case}")


@pytest.mark.parametrize("chunk", [16, 256, 2048])
def test_chunkings_agree_with_oracle_and_repeat_bitwise(chunk):
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c2", B=5, own_len=(1, 5000), page_size=16)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    plan = db.plan(tuning=dict(min_split_tokens=chunk, target_workgroups=10**8))
    assert plan.info["split_tokens"] == chunk
    ws = db.workspace(plan)
    if ws is not None:
        ws.fill_(0xFF)  # the workspace needs no initial contents (0xFFFFFFFF is a NaN)
    say(f"chunk={chunk}")
    o1, l1 = db.step(plan, ws=ws)
    o2, l2 = db.step(plan, ws=ws)
    torch.cuda.synchronize()
    check_close("bf16", o1, l1, o_ref, lse_ref, f"chunk={chunk}")
    assert same_bits(o1, o2) and same_bits(l1, l2)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_request_bins_and_chunks_agree_with_oracle(kv):
    """The same batches on bins of whole requests and on chunks of the flat
    sequence (segment_tokens 0), a plain paged step and a cascade step, both
    against the oracle; the binned step repeats bitwise, also with a workspace
    of garbage, and does not depend on the page size."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    for P, force in ((0, 0), (256, 2), (256, 1)):
        # 400 requests of up to 300 positions: every one fits a chunk, so the planner may bin
        b = make_decode_batch(seed=31 + P + force, B=400, H_q=32, H_kv=8, d=128,
                              own_len=(1, 300) if kv == "bf16" else (100, 300), prefix_len=P, kv_dtype=kv,
                              page_size=16)
        o_ref, lse_ref = ob.batch_reference(b)
        db = DeviceBatch.from_batch(b)
        binned = db.plan(shared_prefix_len=P, force_path=force)
        chunked = db.plan(shared_prefix_len=P, force_path=force, tuning=dict(segment_tokens=0))
        assert binned.info["request_bins"] > 0 and chunked.info["request_bins"] == 0, (P, force)
        say(f"bins {kv} P={P} force={force}: {binned.info['request_bins']} bins")
        ws = db.workspace(binned)
        if ws is not None:
            ws.fill_(0xFF)
        o1, l1 = db.step(binned, ws=ws)
        o2, l2 = db.step(binned, ws=ws)
        oc, lc = db.step(chunked)
        torch.cuda.synchronize()
        check_close(kv, o1, l1, o_ref, lse_ref, f"bins {kv} P={P} force={force}")
        check_close(kv, oc, lc, o_ref, lse_ref, f"chunks {kv} P={P} force={force}")
        assert same_bits(o1, o2) and same_bits(l1, l2)
        # the bins depend on the lengths only: a page size of 1 gives the same bits
        b1 = relayout(b, page_size=1, seed=4001)
        d1 = DeviceBatch.from_batch(b1)
        p1 = d1.plan(shared_prefix_len=P, force_path=force)
        assert p1.info["request_bins"] == binned.info["request_bins"]
        o3, l3 = d1.step(p1)
        torch.cuda.synchronize()
        if P == 0:
            assert same_bits(o1, o3) and same_bits(l1, l3), f"bins {kv}: page size changed the bits"
        else:
            check_close(kv, o3, l3, o_ref, lse_ref, f"bins p=1 {kv} P={P} force={force}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_request_bins_at_their_limits(kv):
    """1,024 short requests, the most the kernel arguments carry, run on bins;
    1,025 fall back to chunks (requests cut at chunk edges and combined);
    both against the oracle on requests spread over the batch."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    for B, binned in ((1024, True), (1025, False)):
        b = make_decode_batch(seed=41 + B, B=B, H_q=32, H_kv=8, d=128, own_len=(20, 200), kv_dtype=kv, page_size=16)
        db = DeviceBatch.from_batch(b)
        plan = db.plan()
        assert (plan.info["request_bins"] > 0) == binned, (B, plan.info)
        reqs, n_cut = spread_requests(b, plan)
        assert binned or n_cut >= 8, n_cut
        say(f"bins limit {kv} B={B}: {plan.info['request_bins']} bins, {len(reqs)} requests checked ({n_cut} cut)")
        o, lse = db.step(plan)
        torch.cuda.synchronize()
        o_ref, lse_ref = ob.batch_reference(b, requests=reqs)
        check_close(kv, o[reqs], lse[reqs], o_ref, lse_ref, f"bins limit {kv} B={B}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_narrow_head_blocks_and_long_chunks(kv):
    """Work items of 1 and 2 KV heads (several tokens per wave-wide load) and
    whole-request chunks of 4096 positions with no combine step."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_decode_batch(seed=21, B=6, H_q=32, H_kv=8, d=128, own_len=(1, 4096), q_dtype="bf16", kv_dtype=kv,
                          page_size=16)
    o_ref, lse_ref = ob.batch_reference(b)
    for tune in (dict(max_heads_per_item=1), dict(max_heads_per_item=2, min_split_tokens=16, target_workgroups=4096),
                 dict(max_heads_per_item=1, min_split_tokens=4096, target_workgroups=1)):
        say(f"narrow heads {kv} {tune}")
        o, lse, plan = run_paged(DeviceBatch, b, tuning=tune)
        assert plan.info["heads_per_item"] == tune["max_heads_per_item"]
        check_close(kv, o, lse, o_ref, lse_ref, f"{kv} {tune}")
        if tune.get("min_split_tokens") == 4096:
            assert plan.info["split_tokens"] == 4096 and plan.info["num_splits"] <= 2


def test_page_table_reads_match_token_flat_bitwise():
    """pkv_paged_decode_attn_pages (the kernel reads the page table) against
    pkv_paged_decode_attn over the lowered indices: same bits, and the oracle."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    c1 = make_config("c1")
    c2 = make_config("c2", B=3, own_len=(1, 3000))
    cases = [("c1 p16", c1), ("c1 p1", relayout(c1, page_size=1, seed=2001, pool_pages=2048)),
             ("c2 p128", c2), ("c2 p7", relayout(c2, page_size=7, seed=2002)),
             ("c5 p16", make_config("c5", B=2, own_len=(1, 3000))),
             ("empty", make_decode_batch(seed=8, B=6, H_q=32, H_kv=8, d=128, own_len=(0, 0),
                                         own_lens=[0, 700, 0, 1, 17, 0], page_size=16))]
    for name, b in cases:
        o_ref, lse_ref = ob.batch_reference(b)
        db = DeviceBatch.from_batch(b)
        for tune in (None, dict(min_split_tokens=16, target_workgroups=100000), dict(max_heads_per_item=1)):
            plan = db.plan(force_path=0, tuning=tune)
            say(f"page table {name} {tune}")
            o1, l1 = db.paged(plan)
            o2, l2 = db.paged_pages(plan)
            torch.cuda.synchronize()
            assert same_bits(o1, o2) and same_bits(l1, l2), f"{name} {tune}: page-table read differs"
            check_close(b.kv_dtype, o2, l2, o_ref, lse_ref, f"page table {name}")
    # the suffix pass of a cascade plan, fp32 state out
    c = make_config("c3", B=16, own_len=(0, 200))
    dc = DeviceBatch.from_batch(c)
    plan = dc.plan(shared_prefix_len=c.prefix_len, force_path=2)
    o1, l1 = dc.paged(plan, want_f32=True)
    o2, l2 = dc.paged_pages(plan, want_f32=True)
    torch.cuda.synchronize()
    assert same_bits(o1, o2) and same_bits(l1, l2)


def test_empty_and_tiny_requests_across_chunks():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    lens = [0, 1500, 0, 63, 64, 65, 0, 1000]
    b = make_decode_batch(seed=8, B=8, H_q=32, H_kv=8, d=128, own_len=(0, 0), own_lens=lens, page_size=16)
    o_ref, lse_ref = ob.batch_reference(b)
    for tune in (dict(min_split_tokens=64, target_workgroups=100000), dict(min_split_tokens=2048)):
        say(f"empty requests {tune}")
        o, lse, plan = run_paged(DeviceBatch, b, tuning=tune)
        check_close("bf16", o, lse, o_ref, lse_ref, f"empty requests {tune}")
        assert torch.isinf(lse[0]).all() and not o[0].float().abs().sum()
    # many one-to-three-token requests share each chunk, empty ones between
    lens = [int(x) for x in np.random.default_rng(3).integers(0, 4, size=300)]
    t = make_decode_batch(seed=10, B=300, H_q=16, H_kv=4, d=64, own_len=(0, 0), own_lens=lens, q_dtype="f32",
                          kv_dtype="f32", page_size=1)
    o_ref, lse_ref = ob.batch_reference(t)
    for tune in (dict(min_split_tokens=16, target_workgroups=100000), dict(min_split_tokens=2048)):
        say(f"tiny requests {tune}")
        o, lse, plan = run_paged(DeviceBatch, t, tuning=tune)
        check_close("f32", o, lse, o_ref, lse_ref, f"tiny requests {tune}")
    # a shared prefix whose suffixes are partly empty, on every path
    lens = [0, 1500, 0, 63, 64, 65, 0, 1000]
    c = make_decode_batch(seed=9, B=8, H_q=32, H_kv=8, d=128, own_len=(0, 0), prefix_len=256, own_lens=lens,
                          page_size=16)
    o_ref, lse_ref = ob.batch_reference(c)
    db = DeviceBatch.from_batch(c)
    for force in (0, 1, 2):
        plan = db.plan(shared_prefix_len=256, force_path=force, tuning=dict(min_split_tokens=64,
                                                                            target_workgroups=100000))
        say(f"empty suffixes force={force}")
        o, lse = db.step(plan)
        torch.cuda.synchronize()
        check_close("bf16", o, lse, o_ref, lse_ref, f"empty suffixes path {force}")


def test_fused_cascade_launch_matches_separate_launches():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    cases = [make_config("c3", B=64, own_len=(0, 300)),
             make_decode_batch(seed=12, B=37, H_q=16, H_kv=2, d=64, own_len=(0, 700), prefix_len=320,
                               page_size=16),
             make_decode_batch(seed=13, B=5, H_q=64, H_kv=8, d=128, own_len=(1, 3000), prefix_len=2048,
                               page_size=16)]
    for b in cases:
        o_ref, lse_ref = ob.batch_reference(b)
        db = DeviceBatch.from_batch(b)
        outs = []
        for fuse in (0, 1):
            for tune in (dict(), dict(min_split_tokens=16, target_workgroups=100000, prefix_target_workgroups=4096,
                                      min_prefix_split_tokens=64)):
                t = dict(tune, fuse_cascade=fuse)
                plan = db.plan(shared_prefix_len=b.prefix_len, force_path=2, tuning=t)
                say(f"fused cascade B={b.B} G={b.H_q // b.H_kv} d={b.d} {t}")
                o, lse = db.step(plan)
                torch.cuda.synchronize()
                check_close("bf16", o, lse, o_ref, lse_ref, f"fuse={fuse} {tune}")
                o2, lse2 = db.step(plan)
                torch.cuda.synchronize()
                assert same_bits(o, o2) and same_bits(lse, lse2), f"fuse={fuse} {tune} not repeatable"
                outs.append((o, lse))
        # The fused kernel runs the same two bodies, but compiled into another
        # kernel its floating-point contractions may differ: compare closely,
        # not bitwise.
        for a_, b_ in ((outs[0], outs[2]), (outs[1], outs[3])):
            assert (a_[0].float() - b_[0].float()).abs().max().item() <= 8e-3
            assert (a_[1] - b_[1]).abs().max().item() <= 1e-4


def test_concurrent_prefix_pass_matches_single_stream():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c3", B=64, own_len=(0, 300))
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    outs = []
    for conc in (0, 1):
        for force in (1, 2):
            plan = db.plan(shared_prefix_len=b.prefix_len, force_path=force,
                           tuning=dict(concurrent_prefix=conc, fuse_cascade=0))
            say(f"concurrent_prefix={conc} force={force}")
            o, lse = db.step(plan)
            torch.cuda.synchronize()
            check_close("bf16", o, lse, o_ref, lse_ref, f"conc={conc} path={force}")
            outs.append((o, lse))
    assert same_bits(outs[0][0], outs[2][0]) and same_bits(outs[1][0], outs[3][0])
    # on a non-default caller stream, with work queued ahead of the step
    side = torch.cuda.Stream()
    plan = db.plan(shared_prefix_len=b.prefix_len, force_path=2, tuning=dict(concurrent_prefix=1, fuse_cascade=0))
    with torch.cuda.stream(side):
        q_saved = db.q.clone()
        db.q.mul_(1.0)  # queued work the step must wait for
        o, lse = db.step(plan, stream=side)
    torch.cuda.synchronize()
    assert same_bits(o, outs[3][0]) and same_bits(lse, outs[3][1])
    assert torch.equal(q_saved, db.q)


def test_run_twice_bitwise_identical():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c3", B=40, own_len=(10, 300))
    db = DeviceBatch.from_batch(b)
    for force in (0, 1, 2):
        plan = db.plan(shared_prefix_len=b.prefix_len, force_path=force)
        say(f"determinism force={force}")
        o1, l1 = db.step(plan)
        o2, l2 = db.step(plan)
        torch.cuda.synchronize()
        assert same_bits(o1, o2) and same_bits(l1, l2), f"path {force} not reproducible"


def test_merge_states_vs_oracle():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    rng = np.random.default_rng(3)
    for d in (64, 128):
        rows = 1000
        o_a, o_b = rng.standard_normal((rows, d)), rng.standard_normal((rows, d))
        la, lb = rng.normal(0, 5, rows), rng.normal(0, 5, rows)
        la[::7] = -np.inf
        lb[::11] = -np.inf
        o_ref, l_ref = oa.merge_states(o_a, la, o_b, lb)
        t = lambda x: torch.tensor(x, dtype=torch.float32, device="cuda")
        lse_out = torch.empty(rows, dtype=torch.float32, device="cuda")
        say(f"merge_states d={d} f32")
        o = DeviceBatch.merge(t(o_a), t(la), t(o_b), t(lb), torch.float32, lse_out)
        torch.cuda.synchronize()
        check_close("f32", o, lse_out, o_ref, l_ref, f"merge d={d}")
        say(f"merge_states d={d} bf16")
        ob16 = DeviceBatch.merge(t(o_a), t(la), t(o_b), t(lb), torch.bfloat16)
        torch.cuda.synchronize()
        assert np.abs(ob16.float().cpu().numpy() - o_ref).max() <= 2e-2


def test_abi_rejects_bad_arguments_without_launching():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c1")
    db = DeviceBatch.from_batch(b)
    plan = db.plan(tuning=dict(min_split_tokens=64, target_workgroups=4096))
    assert plan.info["workspace_bytes"] > 0
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_paged_decode_attn(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, 0.125, o=db.new_out(),
                                  workspace=None)
    assert e.value.name == "EWORKSPACE"
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_paged_decode_attn(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, 0.125,
                                  workspace=db.workspace(plan))
    assert e.value.name == "EINVAL"
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_cascade_prefix_attn(plan, db.q.bfloat16(), db.pool, db.kv_indices, 0, 0.125,
                                    db.new_out(torch.float32), db.new_lse())
    assert e.value.name == "EINVAL"   # a PAGED plan has no prefix pass
    # the binding checks sizes and dtypes against the plan before any call
    for kw in (dict(o=db.new_out()[:2]), dict(o=db.new_out(), lse=db.new_lse()[:1]),
               dict(o=db.new_out(torch.bfloat16)), dict(o_f32=db.new_out(torch.float32)[1:])):
        with pytest.raises(ValueError):
            pkv.pkv_paged_decode_attn(plan, db.q, db.pool, db.kv_indptr, db.kv_indices, 0.125,
                                      workspace=db.workspace(plan), **kw)
    with pytest.raises(ValueError):
        pkv.pkv_paged_decode_attn(plan, db.q, db.pool, db.kv_indptr[:-1], db.kv_indices, 0.125,
                                  o=db.new_out(), workspace=db.workspace(plan))
    with pytest.raises(pkv.PkvError) as e:   # page-table form: missing page table
        pkv._check(pkv._lib.pkv_paged_decode_attn_pages(plan.handle, db.q.data_ptr(), pkv.ctypes.byref(db.pool),
                                                        db.kv_indptr.data_ptr(), None, None, 0.125,
                                                        db.new_out().data_ptr(), None, None,
                                                        db.workspace(plan).data_ptr(), plan.info["workspace_bytes"],
                                                        None), "pages")
    assert e.value.name == "EINVAL"
    with pytest.raises(ValueError):
        pkv.pkv_paged_decode_attn(plan, db.q.cpu(), db.pool, db.kv_indptr, db.kv_indices, 0.125,
                                  o=db.new_out(), workspace=db.workspace(plan))


# ------------------------------------------------------------ prefix groups --

def _grouped_imports():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    from workloads import make_grouped_batch
    return pkv, DeviceBatch, ob, make_grouped_batch


def _garbage_workspace(db, plan):
    ws = db.workspace(plan)
    if ws is not None:
        ws.fill_(0xFF)  # NaN bytes: nothing may rely on a cleared workspace
    return ws


def _grouped_run(db, plan, ws=None):
    meta = db.metadata(plan)
    say(f"grouped step B={db.B} groups={plan.info['num_groups']} path={plan.info['path_name']}")
    o, lse = db.step_grouped(plan, meta, ws=_garbage_workspace(db, plan) if ws is None else ws)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("force", [-1, 0, 1, 2])
def test_grouped_step_small_vs_oracle(force):
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    # three prefixes (one with a tail that does not fill a page), loners, and
    # requests with no tokens of their own or none at all
    b = make_grouped_batch(seed=501, B=24, H_q=32, H_kv=8, d=128, groups=[(8, 1000), (5, 300), (2, 64)],
                           own_len=(0, 200), page_size=16)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    plan = db.plan_grouped(force_path=force, tuning=dict(gate_ratio=0))
    assert plan.info["num_groups"] == (0 if force == 0 else 3)
    o, lse = _grouped_run(db, plan)
    check_close("bf16", o, lse, o_ref, lse_ref, f"grouped force={force}")
    o2, lse2 = _grouped_run(db, plan)
    assert same_bits(o, o2) and same_bits(lse, lse2), "grouped step not repeatable"


def test_grouped_step_dense_and_tiled_groups_in_one_step():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    b = make_grouped_batch(seed=502, B=40, H_q=16, H_kv=4, d=128, groups=[(20, 700), (6, 129), (3, 2048)],
                           own_len=(1, 300), page_size=8)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    # M_eff = 80, 24, 12: the first DENSE, the other two tiled
    plan = db.plan_grouped(tuning=dict(gate_ratio=0, t_dense=64, prefix_target_workgroups=97))
    assert plan.info["num_groups"] == 3 and plan.info["path_name"] == "DENSE"
    o, lse = _grouped_run(db, plan)
    check_close("bf16", o, lse, o_ref, lse_ref, "grouped dense+tiled")


def test_grouped_step_without_groups_is_the_paged_step_bitwise():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    for kv in ("bf16", "fp8"):
        # fp8 K/V at head_dim 64 has no prefix kernel: its groups are dissolved
        b = make_grouped_batch(seed=503, B=12, H_q=32 if kv == "bf16" else 64, H_kv=8, d=128 if kv == "bf16" else 64,
                               groups=[(4, 512)] if kv == "fp8" else [], own_len=(0, 900), page_size=16, kv_dtype=kv)
        o_ref, lse_ref = ob.batch_reference(b)
        db = DeviceBatch.from_batch(b)
        plan = db.plan_grouped()
        assert plan.info["num_groups"] == 0 and plan.info["path_name"] == "PAGED"
        o, lse = _grouped_run(db, plan)
        check_close(kv, o, lse, o_ref, lse_ref, f"grouped no-groups {kv}")
        ref_plan = db.plan(force_path=0)
        say(f"paged reference {kv}")
        o2, lse2 = db.step(ref_plan)
        torch.cuda.synchronize()
        assert same_bits(o, o2) and same_bits(lse, lse2), "grouped PAGED step differs from the paged step"


def test_grouped_step_full_size_sampled():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    # Llama-3.1-8B layer shape: 256 requests, four prompts of 4096 .. 512
    # tokens (48 requests each) and 64 requests on no prompt
    b = make_grouped_batch(seed=504, B=256, H_q=32, H_kv=8, d=128,
                           groups=[(48, 4096), (48, 2048), (48, 1024), (48, 512)], own_len=(64, 512), page_size=16)
    reqs = [int(np.flatnonzero(b.group_of == g)[i]) for g in range(4) for i in (0, -1)]
    reqs += [int(x) for x in np.flatnonzero(b.group_of < 0)[:2]]
    o_ref, lse_ref = ob.batch_reference(b, requests=reqs)
    db = DeviceBatch.from_batch(b)
    plan = db.plan_grouped()
    assert plan.info["num_groups"] == 4 and plan.info["path_name"] == "DENSE"
    o, lse = _grouped_run(db, plan)
    check_close("bf16", o[reqs], lse[reqs], o_ref, lse_ref, "grouped full")


def test_grouped_fused_launch_matches_separate_launches():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    # prefix-heavy: the all-DENSE grouped step takes the fused launch
    b = make_grouped_batch(seed=505, B=40, H_q=32, H_kv=8, d=128, groups=[(16, 2048), (12, 1024), (6, 700)],
                           own_len=(0, 96), page_size=16)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    outs = []
    for fuse in (12, 0):
        plan = db.plan_grouped(tuning=dict(fuse_cascade=fuse, gate_ratio=0))  # keep every group
        assert plan.info["num_groups"] == 3 and plan.info["path_name"] == "DENSE"
        o, lse = _grouped_run(db, plan)
        check_close("bf16", o, lse, o_ref, lse_ref, f"grouped fuse={fuse}")
        o2, lse2 = _grouped_run(db, plan)
        assert same_bits(o, o2) and same_bits(lse, lse2), f"fuse={fuse} not repeatable"
        outs.append((o.float(), lse))
    # the two launches order the same arithmetic the same way up to the
    # chunking of the suffix, so they agree far inside the tolerance
    assert (outs[0][0] - outs[1][0]).abs().max().item() <= 8e-3
    fin = torch.isfinite(outs[0][1])
    assert torch.equal(fin, torch.isfinite(outs[1][1]))
    assert (outs[0][1][fin] - outs[1][1][fin]).abs().max().item() <= 1e-4



# ------------------------------------------------------- fp8 shared prefix --

def test_cascade_fp8_small_all_paths():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    for B, P, own in ((24, 512, (0, 100)), (5, 1000, (1, 3)), (70, 300, (20, 60))):
        b = make_decode_batch(seed=41 + B, B=B, H_q=32, H_kv=8, d=128, own_len=own, prefix_len=P, page_size=16,
                              kv_dtype="fp8", pool_factor=2)
        o_ref, lse_ref = ob.batch_reference(b)
        db, res = _cascade_paths(DeviceBatch, b, ob)
        for force, (o, lse, plan) in res.items():
            check_close("fp8", o, lse, o_ref, lse_ref, f"fp8 B={B} P={P} path={force}")
        plan = res[2][2]
        n = plan.info["prefix_tokens"]
        say(f"fp8 cascade_prefix_attn B={B} n={n}")
        o_p, lse_p = db.prefix(plan)
        torch.cuda.synchronize()
        op_ref, lp_ref = ob.prefix_reference(b, n)
        check_close("fp8", o_p, lse_p, op_ref, lp_ref, f"fp8 prefix B={B}")
        # prefix tiles of 1 and of several ranges, tiled and dense
        for force in (1, 2):
            plan = db.plan(shared_prefix_len=P, force_path=force,
                           tuning=dict(prefix_target_workgroups=4096, min_prefix_split_tokens=64))
            say(f"fp8 many ranges force={force} splits={plan.info['prefix_splits']}")
            o, lse = db.step(plan)
            torch.cuda.synchronize()
            check_close("fp8", o, lse, o_ref, lse_ref, f"fp8 ranges B={B} force={force}")


def test_c3_fp8_full_sampled():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_config("c3", kv_dtype="fp8")
    db = DeviceBatch.from_batch(b)
    plan = db.plan(shared_prefix_len=b.prefix_len)
    assert plan.info["path_name"] == "DENSE"
    reqs, n_cut = spread_requests(b, plan)
    assert len(reqs) >= 32 and n_cut >= 8, (len(reqs), n_cut)
    say(f"c3 fp8 full: oracle over {len(reqs)} requests ({n_cut} cut by chunk edges)")
    o_ref, lse_ref = ob.batch_reference(b, requests=reqs)
    say("c3 fp8 full decode_step")
    o, lse = db.step(plan)
    torch.cuda.synchronize()
    check_close("fp8", o[reqs], lse[reqs], o_ref, lse_ref, "c3 fp8 DENSE")


def test_grouped_step_fp8():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    b = make_grouped_batch(seed=506, B=30, H_q=64, H_kv=8, d=128, groups=[(9, 1500), (6, 400), (3, 77)],
                           own_len=(0, 150), page_size=16, kv_dtype="fp8")
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    for t_dense in (1, 40):  # every group DENSE; the small groups tiled
        plan = db.plan_grouped(tuning=dict(gate_ratio=0, t_dense=t_dense))
        assert plan.info["num_groups"] == 3
        o, lse = _grouped_run(db, plan)
        check_close("fp8", o, lse, o_ref, lse_ref, f"grouped fp8 t_dense={t_dense}")


def test_fp8_fused_cascade_launch_matches_separate_launches():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_decode_batch(seed=47, B=48, H_q=32, H_kv=8, d=128, own_len=(1, 64), prefix_len=1536, page_size=16,
                          kv_dtype="fp8")
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    outs = []
    for fuse in (12, 0):
        plan = db.plan(shared_prefix_len=b.prefix_len, force_path=2, tuning=dict(fuse_cascade=fuse))
        say(f"fp8 DENSE fuse={fuse}")
        o, lse = db.step(plan)
        torch.cuda.synchronize()
        check_close("fp8", o, lse, o_ref, lse_ref, f"fp8 fuse={fuse}")
        o2, lse2 = db.step(plan)
        torch.cuda.synchronize()
        assert same_bits(o, o2) and same_bits(lse, lse2), f"fp8 fuse={fuse} not repeatable"
        outs.append((o.float(), lse))
    assert (outs[0][0] - outs[1][0]).abs().max().item() <= 8e-3
    assert (outs[0][1] - outs[1][1]).abs().max().item() <= 1e-4


# ------------------------------------------------------------- maximum sizes --

def test_pool_larger_than_4gib_addresses_rows_past_4gib():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    # 196,608 pages of 16 slots x 8 KV heads x 128 bf16: 6.4 GB per K (and V)
    # pool; the few live pages are scattered through all of it, so most row
    # offsets are beyond 4 GiB
    b = make_decode_batch(seed=61, B=3, H_q=32, H_kv=8, d=128, own_len=(200, 700), page_size=16,
                          pool_pages=196608, device="cuda")
    top = int(b.page_indices.max()) * 16 * 8 * 128 * 2
    assert top > (1 << 32), top
    o_ref, lse_ref = ob.batch_reference(b)
    for tune in (None, dict(min_split_tokens=16, target_workgroups=100000)):
        say(f"big pool tune={tune}")
        o, lse, _ = run_paged(DeviceBatch, b, tuning=tune)
        check_close("bf16", o, lse, o_ref, lse_ref, f"big pool {tune}")
    del b
    torch.cuda.empty_cache()


def test_one_long_request_in_thousands_of_chunks():
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    b = make_decode_batch(seed=62, B=1, H_q=8, H_kv=2, d=128, own_len=(100_000, 100_000), page_size=16,
                          device="cuda")
    o_ref, lse_ref = ob.batch_reference(b)
    say("long request, 16-token chunks")
    o, lse, plan = run_paged(DeviceBatch, b, tuning=dict(min_split_tokens=16, target_workgroups=10**8))
    assert plan.info["num_splits"] == 6250
    check_close("bf16", o, lse, o_ref, lse_ref, "long request, many chunks")


# --------------------------------------------------------- nested prefixes --

@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_nested_prefix_groups_vs_oracle(kv):
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    from workloads import make_tree_batch
    # a system prompt under two conversations (one with a longer shared
    # branch), a second prompt, and loners; runs cross page boundaries
    tree = [(14, 700, -1), (6, 300, 0), (5, 250, 0), (3, 120, 1), (4, 333, -1)]
    b = make_tree_batch(seed=507, B=24, H_q=32, H_kv=8, d=128, tree=tree, own_len=(0, 90), page_size=16,
                        kv_dtype=kv)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    for t in (dict(gate_ratio=0), dict(gate_ratio=0, t_dense=40), dict(gate_ratio=0, fuse_cascade=0)):
        plan = db.plan_grouped(tuning=t)
        meta = pkv.split_metadata(pkv.pkv_plan_metadata(plan), b.B, plan.info["num_groups"])
        assert plan.info["num_groups"] == 5 and (meta["group_parent"] >= 0).sum() == 3
        o, lse = _grouped_run(db, plan)
        check_close(kv, o, lse, o_ref, lse_ref, f"nested {kv} {t}")


def test_nested_prefix_groups_full_size_sampled():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    from workloads import make_tree_config
    # Llama-3.1-8B layer shape: a 2048-token system prompt under four
    # conversations of 48 requests (1024 more shared tokens each), 64 loners
    b = make_tree_config("tree4")
    inner = set(int(x) for m in b.node_members for x in m)
    reqs = [int(b.node_members[k][i]) for k in range(1, 5) for i in (0, -1)]
    reqs += [x for x in range(b.B) if x not in inner][:2]
    o_ref, lse_ref = ob.batch_reference(b, requests=reqs)
    db = DeviceBatch.from_batch(b)
    plan = db.plan_grouped()
    meta = pkv.split_metadata(pkv.pkv_plan_metadata(plan), b.B, plan.info["num_groups"])
    assert plan.info["num_groups"] == 5 and plan.info["path_name"] == "DENSE"
    assert list(meta["group_parent"]) == [-1, 0, 0, 0, 0]
    o, lse = _grouped_run(db, plan)
    check_close("bf16", o[reqs], lse[reqs], o_ref, lse_ref, "nested full")


# ------------------------------------------------------ randomized sweep --

@pytest.mark.parametrize("case", range(64))
def test_random_shapes_vs_oracle(case):
    """Seeded random mixes of dtype, head_dim, GQA group, KV heads, page size,
    batch and lengths (empty requests included), shared prefix, forced path
    and tuning (work-item target and geometry, bins, gate, fused launch, side
    stream), every request checked against the oracle."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    rng = np.random.default_rng(9000 + case)
    kv = str(rng.choice(["f32", "bf16", "fp8"], p=[0.2, 0.5, 0.3]))
    q = "f32" if kv == "f32" else "bf16"
    d = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    H_kv = int(rng.choice([1, 2, 3, 4, 8]))
    p = int(rng.choice([1, 3, 8, 16, 64]))
    B = int(rng.integers(1, 33))
    lo = int(rng.integers(0, 40))
    hi = lo + int(rng.integers(0, 600))
    P = int(rng.integers(1, 700)) if rng.random() < 0.7 else 0
    prefix_ok = q == "bf16" and (kv == "bf16" or d == 128) and P >= p and B >= 1
    force = int(rng.choice([-1, 0, 1, 2])) if prefix_ok else int(rng.choice([-1, 0]))
    tune = dict(target_workgroups=int(rng.choice([64, 256, 512, 1024])),
                min_split_tokens=int(rng.choice([16, 64, 256])), gate_ratio=int(rng.choice([0, 3])),
                fuse_cascade=int(rng.choice([0, 1, 12])), t_dense=int(rng.choice([1, 64, 4096])),
                segment_tokens=int(rng.choice([0, 32, 128])), max_heads_per_item=int(rng.choice([0, 0, 1, 2])),
                cached_prefix_bytes=int(rng.choice([0, 2 << 20])), concurrent_prefix=int(rng.choice([0, 0, 1])))
    layout = str(rng.choice(["shared", "unique"])) if P else "shared"
    b = make_decode_batch(seed=9000 + case, B=B, H_q=G * H_kv, H_kv=H_kv, d=d, own_len=(lo, hi), prefix_len=P,
                          q_dtype=q, kv_dtype=kv, page_size=p, layout=layout)
    what = f"case {case}: {kv} d={d} G={G} H_kv={H_kv} p={p} B={B} L=P{P}+U{{{lo}..{hi}}} force={force} {tune}"
    say(what)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    plan = db.plan(shared_prefix_len=P, force_path=force, tuning=tune)
    o, lse = db.step(plan, ws=_garbage_workspace(db, plan))
    torch.cuda.synchronize()
    check_close(kv, o, lse, o_ref, lse_ref, what + f" path={plan.info['path_name']}")


@pytest.mark.parametrize("case", range(24))
def test_random_prefix_trees_vs_oracle(case):
    """Seeded random trees of shared runs (roots with nested children, loners,
    runs crossing page boundaries) planned from the page table."""
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    from workloads import make_tree_batch
    rng = np.random.default_rng(9100 + case)
    kv = str(rng.choice(["bf16", "fp8"]))
    d = 128 if kv == "fp8" else int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    H_kv = int(rng.choice([1, 2, 4, 8]))
    p = int(rng.choice([4, 16, 32]))
    B = int(rng.integers(6, 40))
    tree, free = [], B
    for _ in range(int(rng.integers(1, 4))):          # roots
        n = int(rng.integers(2, max(3, free // 2 + 1)))
        if n > free:
            break
        free -= n
        r = len(tree)
        tree.append((n, int(rng.integers(1, 600)), -1))
        left = n
        for _ in range(int(rng.integers(0, 3))):      # children of this root
            m = int(rng.integers(2, max(3, left // 2 + 1)))
            if m > left:
                break
            left -= m
            tree.append((m, int(rng.integers(1, 300)), r))
    tune = dict(gate_ratio=int(rng.choice([0, 0, 0, 3])), t_dense=int(rng.choice([1, 16, 4096])),
                fuse_cascade=int(rng.choice([0, 1, 12])), segment_tokens=int(rng.choice([0, 32])),
                max_heads_per_item=int(rng.choice([0, 1, 2])))
    b = make_tree_batch(seed=9100 + case, B=B, H_q=G * H_kv, H_kv=H_kv, d=d, tree=tree,
                        own_len=(0, int(rng.integers(1, 200))), page_size=p, kv_dtype=kv)
    what = f"tree case {case}: {kv} d={d} G={G} H_kv={H_kv} p={p} B={B} tree={tree} {tune}"
    say(what)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    plan = db.plan_grouped(tuning=tune)
    o, lse = _grouped_run(db, plan)
    check_close(kv, o, lse, o_ref, lse_ref, what + f" groups={plan.info['num_groups']} path={plan.info['path_name']}")


# ------------------------------------------------------- prefix placement --

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_contiguous_prefix_read_as_base_plus_offset(kv_dtype):
    """A shared prefix stored as one run of consecutive slots ("GraniKV",
    section 1, asymmetric placement): the plan finds the run from the host
    indices and the prefix pass reads slots base + t with no index staging.
    Same bits as the slot-by-slot read of the same pool, on every prefix
    path (tiled, DENSE fused and separate) and for the prefix pass alone;
    within tolerance of the oracle."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    P = 1000
    b0 = make_decode_batch(seed=81, B=40, H_q=32, H_kv=8, d=128, own_len=(1, 300), prefix_len=P, page_size=16,
                           kv_dtype=kv_dtype, pool_factor=2)
    b = relayout(b0, page_size=16, seed=82, layout="shared", perm="prefix_first", pool_factor=2,
                 prefix_first_page=37)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    for force, tune in ((1, None), (2, None), (2, dict(fuse_cascade=0)), (2, dict(fuse_cascade=1)),
                        (2, dict(prefix_target_workgroups=4096, min_prefix_split_tokens=64))):
        strided = db.plan(shared_prefix_len=P, force_path=force, tuning=tune)
        gathered = db.plan(shared_prefix_len=P, force_path=force, tuning=tune, host_indices=False)
        assert strided.info["prefix_base"] == 37 * 16 and strided.info["contiguous_prefixes"] == 1
        assert gathered.info["prefix_base"] == -1 and gathered.info["contiguous_prefixes"] == 0
        say(f"contiguous prefix {kv_dtype} force={force} tune={tune}: base + offset, then slot by slot")
        o1, l1 = db.step(strided)
        o2, l2 = db.step(gathered)
        torch.cuda.synchronize()
        check_close(kv_dtype, o1, l1, o_ref, lse_ref, f"contiguous prefix {kv_dtype} force={force}")
        assert same_bits(o1, o2) and same_bits(l1, l2), f"placement changed the bits ({kv_dtype}, {force}, {tune})"
    say(f"contiguous prefix {kv_dtype}: prefix pass alone")
    strided = db.plan(shared_prefix_len=P, force_path=2)
    gathered = db.plan(shared_prefix_len=P, force_path=2, host_indices=False)
    p1, q1 = db.prefix(strided)
    p2, q2 = db.prefix(gathered)
    torch.cuda.synchronize()
    n = strided.info["prefix_tokens"]
    op_ref, lp_ref = ob.prefix_reference(b, n)
    check_close(kv_dtype, p1, q1, op_ref, lp_ref, f"contiguous prefix pass {kv_dtype}")
    assert same_bits(p1, p2) and same_bits(q1, q2)
    # the scattered layout of the same tokens: no run, read slot by slot
    assert DeviceBatch.from_batch(b0).plan(shared_prefix_len=P, force_path=2).info["prefix_base"] == -1


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_grouped_contiguous_runs_read_as_base_plus_offset(kv_dtype):
    """Several prefixes each stored in consecutive pages: every kept group's
    run is read as base + offset (the planner finds it in the page table);
    same bits as with placement switched off, for DENSE (fused) and tiled
    groups; within tolerance of the oracle."""
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    b = make_grouped_batch(seed=84, B=40, H_q=32, H_kv=8, d=128, groups=[(12, 700), (9, 300), (5, 64)],
                           own_len=(0, 120), page_size=16, perm="identity", kv_dtype=kv_dtype)
    o_ref, lse_ref = ob.batch_reference(b)
    db = DeviceBatch.from_batch(b)
    for t_dense in (1, 40):
        on = db.plan_grouped(tuning=dict(gate_ratio=0, t_dense=t_dense))
        off = db.plan_grouped(tuning=dict(gate_ratio=0, t_dense=t_dense, prefix_placement=0))
        assert on.info["num_groups"] == 3 and on.info["contiguous_prefixes"] == 3
        assert off.info["contiguous_prefixes"] == 0
        meta = pkv.split_metadata(pkv.pkv_plan_metadata(on), b.B, 3)
        assert (meta["group_prefix_base"] >= 0).all()
        o1, l1 = _grouped_run(db, on)
        o2, l2 = _grouped_run(db, off)
        check_close(kv_dtype, o1, l1, o_ref, lse_ref, f"grouped contiguous {kv_dtype} t_dense={t_dense}")
        assert same_bits(o1, o2) and same_bits(l1, l2), f"placement changed the bits ({kv_dtype}, {t_dense})"


def _capture(fn):
    """fn captured into a graph on a side stream of default priority, after
    one warm-up call there (the library allocates nothing and sets no
    memory: its launches are the whole graph)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(g, o, lse, o_ref, lse_ref, what, replays=4):
    for r in range(replays):
        # eager work and a synchronisation between replays: the outputs are
        # overwritten, so each replay has to write all of them again
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(o, o_ref) and same_bits(lse, lse_ref), f"{what}: replay {r} differs from the eager step"


@pytest.mark.parametrize("case", ["paged_split", "paged_fp8_bins", "cascade_fused", "cascade_separate"])
def test_graph_replays_match_the_eager_step(case):
    """A decode step captured into a HIP graph (as a serving loop would)
    replays to the eager step's bits, replay after replay."""
    pkv, DeviceBatch, ob, oa, make_config, make_decode_batch, relayout = _imports()
    if case == "paged_split":
        b = make_decode_batch(seed=91, B=6, H_q=32, H_kv=8, d=128, own_len=(1500, 3000), q_dtype="bf16",
                              kv_dtype="bf16", page_size=16)
        P, tune = 0, dict(target_workgroups=64)
    elif case == "paged_fp8_bins":
        b = make_decode_batch(seed=92, B=300, H_q=64, H_kv=8, d=128, own_len=(50, 400), q_dtype="bf16",
                              kv_dtype="fp8", page_size=16)
        P, tune = 0, {}
    else:
        b = make_decode_batch(seed=93, B=64, H_q=32, H_kv=8, d=128, own_len=(1, 64), prefix_len=1024,
                              q_dtype="bf16", kv_dtype="bf16", page_size=16)
        P, tune = 1024, dict(gate_ratio=0, fuse_cascade=12 if case == "cascade_fused" else 0)
    db = DeviceBatch.from_batch(b)
    plan = db.plan(shared_prefix_len=P, tuning=tune)
    if case == "paged_split":
        assert plan.info["num_splits"] > 1
    if case == "paged_fp8_bins":
        assert plan.info["request_bins"] > 0
    if P:
        assert plan.info["path_name"] == "DENSE"
    say(f"graph {case}: path={plan.info['path_name']} splits={plan.info['num_splits']}")
    ws = db.workspace(plan)
    o, lse = db.new_out(), db.new_lse()
    db.step(plan, o, lse, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    reqs = list(range(0, b.B, max(1, b.B // 6)))
    o64, lse64 = ob.batch_reference(b, requests=reqs)
    check_close(b.kv_dtype, o_ref[reqs], lse_ref[reqs], o64, lse64, f"graph {case} eager")
    g = _capture(lambda: db.step(plan, o, lse, ws))
    _replays_match(g, o, lse, o_ref, lse_ref, f"graph {case}")


def test_graph_replays_match_the_eager_grouped_step():
    pkv, DeviceBatch, ob, make_grouped_batch = _grouped_imports()
    b = make_grouped_batch(seed=94, B=40, H_q=32, H_kv=8, d=128, groups=[(16, 1024), (12, 512)], own_len=(0, 96),
                           page_size=16)
    db = DeviceBatch.from_batch(b)
    plan = db.plan_grouped(tuning=dict(gate_ratio=0))
    assert plan.info["num_groups"] == 2
    meta = db.metadata(plan)
    ws = db.workspace(plan)
    o, lse = db.new_out(), db.new_lse()
    db.step_grouped(plan, meta, o, lse, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    g = _capture(lambda: db.step_grouped(plan, meta, o, lse, ws))
    _replays_match(g, o, lse, o_ref, lse_ref, "graph grouped")
