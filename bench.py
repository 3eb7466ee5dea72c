"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs c1,c2,...,tree4]

A step is one whole decode-attention step of one layer as the planner chose
it (pkv_decode_step: the paged pass, or prefix pass + suffix pass + merge),
with every input already resident in HBM.  Only kernels are inside the timed
region: planning, page-table lowering and uploads happen once before it, and
the same inputs are reused every step (warm caches, no admission ramp).

The headline line is the Llama-3.1-8B-shaped layer (B=32, 32 query / 8 KV
heads, head_dim 128, 4096 tokens each, bf16, token-flat indices at page size
1): ``value`` is its algorithmic HBM throughput in GB/s.  The other workloads
(tiny fp32, shared-prefix cascade, short prefix, long-context fp8, several
prompts in one step, prompts nested as a tree) are reported under ``extra``.  Prints one JSON line on stdout.
"""
import argparse
import itertools
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
BYTES = {"f32": 4, "bf16": 2, "fp8": 1}


def algorithmic_bytes(batch, path, prefix_tokens=0):
    """Bytes the method must move for one step (not re-reads, not split partials)."""
    B, Hq, Hkv, d = batch.B, batch.H_q, batch.H_kv, batch.d
    bkv = 2 * BYTES[batch.kv_dtype]
    bq = BYTES[batch.q_dtype]
    rows = B * Hq
    L = [int(x) for x in batch.seq_lens]
    if path == "PAGED":
        tot = sum(L)
        n = tot * Hkv * d * bkv + 4 * tot + 4 * (B + 1) + rows * d * 2 * bq + 4 * rows
        if batch.kv_dtype == "fp8":
            n += 8 * Hkv
        return n
    P = prefix_tokens
    S = sum(x - P for x in L)
    return (P * Hkv * d * bkv + 4 * P + S * Hkv * d * bkv + 4 * S + 2 * rows * d * bq + 4 * rows * (d + 1) * 4
            + rows * d * bq)


WINDOWS = 7             # timed windows of --steps steps per leg
STABLE_TOL = 0.01       # warm until two consecutive windows agree this closely
MIN_WARM_S = 0.25       # ... after at least this much warming (a leg on a freshly laid out pool drifts
                        # slowly: consecutive short windows can agree while it is still 3-5 % slow)
MAX_WARM_S = 3.0        # ... or until this much warming has passed


def time_windows(fn, steps, warmup, windows=WINDOWS):
    """`warmup` untimed calls; then windows of `steps` back-to-back calls, each
    between two events on the launch stream, for at least MIN_WARM_S and until
    two consecutive windows agree within STABLE_TOL (a steady clock and warm
    caches; at most MAX_WARM_S of such warming); then `windows` timed
    windows.  Returns the
    median, min and max ms per step over the timed windows, the warm-up
    windows it took and the total number of calls."""
    import statistics
    import torch
    stream = torch.cuda.current_stream()
    calls = 0
    for _ in range(warmup):
        fn()
        calls += 1

    def window():
        nonlocal calls
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        end.synchronize()
        calls += steps
        return start.elapsed_time(end) / steps

    t0 = time.perf_counter()
    warm = [window()]
    while True:
        warm.append(window())
        a, b = warm[-2], warm[-1]
        if abs(a - b) <= STABLE_TOL * min(a, b) and time.perf_counter() - t0 >= MIN_WARM_S:
            stable = True
            break
        if time.perf_counter() - t0 > MAX_WARM_S:
            stable = False
            break
    vals = [window() for _ in range(windows)]
    return dict(ms=statistics.median(vals), ms_min=min(vals), ms_max=max(vals), windows=windows,
                warm_windows=len(warm), warm_stable=stable, calls=calls)


def time_steps(fn, steps, warmup):
    """Median ms per step (see time_windows)."""
    return time_windows(fn, steps, warmup)["ms"]


# Peaks of one MI355X (vendor figures): HBM3E bandwidth, dense bf16 MFMA, and
# fp32 vector ALU (256 CUs x 4 SIMDs x 2.4 GHz x 64 flops per SIMD-cycle).
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_VALU_F32_TFLOPS = 157.3


def roofline(us, hbm_bytes, mfma_flops=0, valu_flops=0, note=None):
    """Floors of a step at the chip's peaks: HBM bytes / 8 TB/s, MFMA flops /
    2.5 PFLOP/s (bf16 dense), vector-ALU flops / 157.3 TFLOP/s; the step's
    roofline is the largest of them and frac = that floor / measured time."""
    fl = dict(hbm_us=hbm_bytes / (PEAK_HBM_GBS * 1e3), mfma_us=mfma_flops / (PEAK_MFMA_BF16_TFLOPS * 1e6),
              valu_us=valu_flops / (PEAK_VALU_F32_TFLOPS * 1e6))
    bound = max(fl, key=fl.get)
    floor = fl[bound]
    out = dict(bound={"hbm_us": "hbm", "mfma_us": "mfma", "valu_us": "alu"}[bound], floor_us=floor,
               frac=floor / us if us > 0 else None, floors_us=fl)
    if note:
        out["note"] = note
    return out


def leg(t, nbytes, **roof):
    """One timed leg: median (min, max) us per step, GB/s of the algorithmic
    bytes at the median, and the roofline at the median."""
    us = t["ms"] * 1e3
    note = roof.pop("note", None)
    return dict(us_per_step=us, us_min=t["ms_min"] * 1e3, us_max=t["ms_max"] * 1e3, windows=t["windows"],
                warm_windows=t["warm_windows"], warm_stable=t["warm_stable"], algorithmic_bytes=nbytes,
                gbs=nbytes / us / 1e3, roofline=roofline(us, nbytes, note=note, **roof))


def valu_flops(tokens, batch):
    """Vector-ALU flops of attending `tokens` (token, request) positions: one
    multiply-add (2 flops) per query-head element for each of q.k and p.v."""
    return 4 * tokens * batch.H_q * batch.d


def mfma_flops(m_eff, prefix_tokens, batch):
    """Matrix-core flops of the prefix contraction: S = Q K^T and O = P V for
    M_eff query rows per KV head over the prefix."""
    return 4 * m_eff * prefix_tokens * batch.d * batch.H_kv


def bench_paged_config(name, steps, warmup, **overrides):
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_config
    b = make_config(name, device="cuda", **overrides)
    db = DeviceBatch.from_batch(b)
    plan = db.plan()
    o, lse, ws = db.new_out(), db.new_lse(), db.workspace(plan)
    t = time_windows(lambda: db.step(plan, o, lse, ws), steps, warmup)
    nbytes = algorithmic_bytes(b, plan.info["path_name"])
    tokens = int(sum(int(x) for x in b.seq_lens))
    rec = dict(workload=name, page_size=b.page_size, path=plan.info["path_name"],
               **leg(t, nbytes, valu_flops=valu_flops(tokens, b)), num_splits=plan.info["num_splits"],
               split_tokens=plan.info["split_tokens"], work_items=plan.info["num_work_items"])
    rec["pct_peak"] = 100.0 * rec["gbs"] / PEAK_HBM_GBS
    issue = valu_issue_floor(name)
    if issue:
        rec["roofline"]["valu_issue"] = issue
    return rec, b, db, plan


COUNTERS_FILE = os.path.join(ROOT, "profiles", "paged_split_kernel.c2_c5.counters.json")


def valu_issue_floor(name):
    """Vector-instruction issue floor of a workload's paged kernel from the
    committed counter summary: wave64 VALU instructions per step (median per
    dispatch), at one instruction per 4 cycles on each of the 1,024 SIMDs at
    2.4 GHz.  None if the summary does not cover the workload."""
    try:
        rec = json.load(open(COUNTERS_FILE))
        n = rec["workloads"][name]["counters_median_per_dispatch"]["SQ_INSTS_VALU"]
    except (OSError, ValueError, KeyError):
        return None
    return dict(valu_insts_per_step=n, floor_us=n * 4 / (1024 * 2.4e3),
                counters_source_matches=rec.get("source_sha256") == kernel_source_hash())


def add_ceiling(rec, ceiling):
    rec["pct_read_ceiling"] = 100.0 * rec["gbs"] / ceiling
    return rec


# legs of a shared-prefix workload: label, forced path, tuning
PREFIX_LEGS = (("paged_shared", 0, None), ("cascade", 1, None), ("dense", 2, None),
               ("dense_separate", 2, dict(fuse_cascade=0)), ("planned", -1, None))

SHARED_PAGES_NOTE = ("requested bytes: every request re-reads the shared pages, which mostly hit in L2 / "
                     "Infinity Cache, so this floor understates the step and frac can exceed 1")


def prefix_leg(b, plan, t):
    """A shared-prefix leg's record with its floors: HBM over the path's
    algorithmic bytes, MFMA over the prefix contraction, vector ALU over the
    paged pass's positions."""
    path = plan.info["path_name"]
    P = plan.info["prefix_tokens"]
    nbytes = algorithmic_bytes(b, path, P)
    tokens = int(sum(int(x) for x in b.seq_lens)) - (b.B * P if path != "PAGED" else 0)
    return dict(path=path, **leg(t, nbytes, valu_flops=valu_flops(tokens, b),
                                 mfma_flops=mfma_flops(plan.info["m_eff"], P, b) if path != "PAGED" else 0))


def bench_prefix_config(name, steps, warmup, legs=None, oracle=False):
    """PAGED over unique prefix copies, PAGED over shared pages, each prefix
    path (DENSE also as two launches), and the planner's choice."""
    import torch
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_config, relayout
    from workloads.synth import RELAYOUT_SEED
    b = make_config(name, device="cuda")
    P = b.prefix_len
    out = dict(workload=name, B=b.B, prefix=P)
    db = DeviceBatch.from_batch(b)
    o, lse = db.new_out(), db.new_lse()
    for label, force, tune in PREFIX_LEGS:
        if legs and label not in legs:
            continue
        plan = db.plan(shared_prefix_len=P, force_path=force, tuning=tune)
        ws = db.workspace(plan)
        t = time_windows(lambda: db.step(plan, o, lse, ws), steps, warmup)
        out[label] = prefix_leg(b, plan, t)
        if label == "paged_shared":
            out[label]["roofline"]["note"] = SHARED_PAGES_NOTE
        del ws
    del db
    torch.cuda.empty_cache()
    if not legs or "planned_contiguous_prefix" in legs or "contiguous_prefix_gathered" in legs:
        # the prefix stored contiguously ("GraniKV", section 1, asymmetric
        # placement): the planner, shown the host indices, reads it as base
        # + offset; the same pool planned without them reads it slot by slot
        c = relayout(b, page_size=b.page_size, seed=RELAYOUT_SEED[name] + 1000, layout="shared", perm="prefix_first",
                     device="cuda")
        dc = DeviceBatch.from_batch(c)
        for label, host in (("planned_contiguous_prefix", True), ("contiguous_prefix_gathered", False)):
            if legs and label not in legs:
                continue
            plan = dc.plan(shared_prefix_len=P, host_indices=host)
            ws = dc.workspace(plan)
            t = time_windows(lambda: dc.step(plan, o, lse, ws), steps, warmup)
            out[label] = prefix_leg(c, plan, t)
            out[label]["prefix_base"] = plan.info["prefix_base"]
            del ws
        del dc, c
        torch.cuda.empty_cache()
    if not legs or "paged_unique" in legs:
        u = relayout(b, page_size=b.page_size, seed=RELAYOUT_SEED[name], layout="unique", device="cuda")
        du = DeviceBatch.from_batch(u)
        plan = du.plan(force_path=0)
        ws = du.workspace(plan)
        t = time_windows(lambda: du.step(plan, o, lse, ws), steps, warmup)
        out["paged_unique"] = prefix_leg(u, plan, t)
        out["paged_unique"]["pct_peak"] = 100 * out["paged_unique"]["gbs"] / PEAK_HBM_GBS
        del du, u, ws
    if oracle:
        n, runs = ORACLE_SAMPLE[name]
        out["oracle"] = oracle_sample(b, list(range(n)), runs)
        if "planned" in out:
            out["oracle"]["gpu_speedup"] = out["oracle"]["ms_per_step"] / (out["planned"]["us_per_step"] / 1e3)
    del b
    torch.cuda.empty_cache()
    if "planned" in out and "paged_unique" in out:
        out["speedup_vs_paged_unique"] = out["paged_unique"]["us_per_step"] / out["planned"]["us_per_step"]
    if "planned" in out and "paged_shared" in out:
        out["speedup_vs_paged_shared"] = out["paged_shared"]["us_per_step"] / out["planned"]["us_per_step"]
    return out


def grouped_algorithmic_bytes(batch, plan_meta, group_rows):
    """Bytes a grouped step must move: each kept group's prefix once, every
    request's own tokens, the queries twice (both passes), one partial state
    per (kept group, member row) (written and read as fp32 (o, m, l)), the
    output.  ``group_rows`` counts a row once per kept group on its path."""
    bkv = BYTES[batch.kv_dtype] * 2
    bq = BYTES[batch.q_dtype]
    Hkv, d, rows = batch.H_kv, batch.d, batch.B * batch.H_q
    n_pre = int(plan_meta["prefix_indptr"][-1])
    n_suf = int(plan_meta["suffix_indptr"][-1])
    return ((n_pre + n_suf) * (Hkv * d * bkv + 4) + 2 * rows * d * bq + 4 * group_rows * (d + 1) * 4
            + rows * d * bq)


def grouped_mfma_flops(batch, plan_meta):
    """Matrix-core flops of a grouped step: each kept group's members' rows
    over its own run."""
    gp, pp = plan_meta["group_indptr"], plan_meta["prefix_indptr"]
    return sum(4 * int(gp[i + 1] - gp[i]) * batch.G * int(pp[i + 1] - pp[i]) * batch.d * batch.H_kv
               for i in range(len(gp) - 1))


def bench_groups_config(name, steps, warmup):
    """Several prompts in one step (side by side, or nested as a tree):
    PAGED over the shared pages, every group forced to the tiled cascade,
    and the planner's choice."""
    import numpy as np
    import torch
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_group_config, make_tree_config
    if name.startswith("tree"):
        b = make_tree_config(name, device="cuda")
        out = dict(workload=name, B=b.B, tree_node_requests=[len(m) for m in b.node_members])
    else:
        b = make_group_config(name, device="cuda")
        out = dict(workload=name, B=b.B, groups=[[int(n), int(P)] for n, P in
                                                 zip(np.bincount(b.group_of[b.group_of >= 0]), b.prefix_lens)])
    db = DeviceBatch.from_batch(b)
    o, lse = db.new_out(), db.new_lse()
    plan = db.plan(force_path=0)
    ws = db.workspace(plan)
    t = time_windows(lambda: db.step(plan, o, lse, ws), steps, warmup)
    tokens = int(sum(int(x) for x in b.seq_lens))
    out["paged_shared"] = dict(path="PAGED", **leg(t, algorithmic_bytes(b, "PAGED"), valu_flops=valu_flops(tokens, b),
                                                   note=SHARED_PAGES_NOTE))
    del ws
    for label, force in (("grouped_cascade", 1), ("grouped_planned", -1)):
        plan = db.plan_grouped(force_path=force)
        meta = db.metadata(plan)
        ws = db.workspace(plan)
        t = time_windows(lambda: db.step_grouped(plan, meta, o, lse, ws), steps, warmup)
        m = pkv.split_metadata(pkv.pkv_plan_metadata(plan), b.B, plan.info["num_groups"])
        nb = grouped_algorithmic_bytes(b, m, len(m["group_members"]) * b.H_q)
        out[label] = dict(path=plan.info["path_name"], num_groups=plan.info["num_groups"],
                          **leg(t, nb, mfma_flops=grouped_mfma_flops(b, m),
                                valu_flops=valu_flops(int(m["suffix_indptr"][-1]), b)))
        del ws, meta
    out["speedup_vs_paged_shared"] = out["paged_shared"]["us_per_step"] / out["grouped_planned"]["us_per_step"]
    del db, b
    torch.cuda.empty_cache()
    if not name.startswith("tree"):
        # every prompt's whole pages stored in consecutive pages ("GraniKV",
        # section 1): each group's run read as base + offset, against the
        # same pool with placement switched off
        c = make_group_config(name, device="cuda", perm="identity")
        dc = DeviceBatch.from_batch(c)
        for label, placement in (("grouped_planned_contiguous", 1), ("grouped_contiguous_gathered", 0)):
            plan = dc.plan_grouped(tuning=dict(prefix_placement=placement))
            meta = dc.metadata(plan)
            ws = dc.workspace(plan)
            t = time_windows(lambda: dc.step_grouped(plan, meta, o, lse, ws), steps, warmup)
            m = pkv.split_metadata(pkv.pkv_plan_metadata(plan), c.B, plan.info["num_groups"])
            nb = grouped_algorithmic_bytes(c, m, len(m["group_members"]) * c.H_q)
            out[label] = dict(path=plan.info["path_name"], num_groups=plan.info["num_groups"],
                              contiguous_prefixes=plan.info["contiguous_prefixes"],
                              **leg(t, nb, mfma_flops=grouped_mfma_flops(c, m),
                                    valu_flops=valu_flops(int(m["suffix_indptr"][-1]), c)))
            del ws, meta
        del dc, c
        torch.cuda.empty_cache()
    return out


SWEEP_B = (1, 2, 4, 16, 64, 256, 512)
SWEEP_G = (1, 4, 8)
SWEEP_P = (256, 1024, 4096)
SWEEP_DTYPES = ("bf16", "fp8")


def dispatch_sweep(out_path, steps=10, warmup=3):
    """The dispatcher's refit grid ("GraniKV", section 3: the dense
    threshold is a per-GPU constant): B x G x P x K/V dtype, 8 KV heads,
    d = 128, own tokens U{64..512}, page size 16.  Every cell times PAGED
    over the shared prefix pages and over per-request copies, the tiled
    cascade and DENSE (forced), and the planner's own choice; then replays
    the planner over a grid of candidate constants (t_dense, gate_ratio,
    launch_bytes) against the measured times, and writes every cell and
    the replay to out_path (JSON)."""
    import numpy as np
    import torch
    import paged_kv_cache_201_amd as pkv
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_decode_batch, relayout
    log = lambda m: print(m, file=sys.stderr, flush=True)  # noqa: E731
    cells = []
    t_start = time.perf_counter()
    seed = 5000
    for kv, P, G, B in itertools.product(SWEEP_DTYPES, SWEEP_P, SWEEP_G, SWEEP_B):
        seed += 1
        b = make_decode_batch(seed=seed, B=B, H_q=8 * G, H_kv=8, d=128, own_len=(64, 512), prefix_len=P,
                              page_size=16, kv_dtype=kv, device="cuda")
        db = DeviceBatch.from_batch(b)
        o, lse = db.new_out(), db.new_lse()
        cell = dict(B=B, G=G, P=P, kv_dtype=kv, m_eff=B * G, us={})
        for label, force in (("paged_shared", 0), ("cascade", 1), ("dense", 2), ("planned", -1)):
            if force > 0 and B < 2:
                continue  # nothing to share
            plan = db.plan(shared_prefix_len=P, force_path=force)
            ws = db.workspace(plan)
            cell["us"][label] = time_windows(lambda: db.step(plan, o, lse, ws), steps, warmup, windows=3)["ms"] * 1e3
            if force == -1:
                cell["planned_path"] = plan.info["path_name"]
            del ws
        del db
        u = relayout(b, page_size=16, seed=seed, layout="unique", device="cuda")
        du = DeviceBatch.from_batch(u)
        plan = du.plan(force_path=0)
        ws = du.workspace(plan)
        cell["us"]["paged_unique"] = time_windows(lambda: du.step(plan, o, lse, ws), steps, warmup,
                                                  windows=3)["ms"] * 1e3
        del du, u, ws, b, o, lse
        torch.cuda.empty_cache()
        choices = {k: v for k, v in cell["us"].items() if k in ("paged_shared", "cascade", "dense")}
        cell["fastest"] = min(choices, key=choices.get)
        cell["planned_over_fastest"] = cell["us"]["planned"] / choices[cell["fastest"]]
        cells.append(cell)
        log(f"sweep {len(cells)}: {kv} P={P} G={G} B={B} planned {cell['planned_path']} "
            f"{cell['us']['planned']:.1f} us, fastest {cell['fastest']} {choices[cell['fastest']]:.1f} us "
            f"({time.perf_counter() - t_start:.0f} s)")

    replay = replay_sweep(cells)
    defaults = pkv.pkv_tuning_defaults()
    planned = [c["planned_over_fastest"] for c in cells]
    planned_multi = [c["planned_over_fastest"] for c in cells if c["B"] >= 2]
    rec = dict(
        what="forced-path sweep of the dispatcher: us per step of each path, the planner's choice and its ratio "
             "to the fastest path on the shared-page layout; paged_unique = PAGED over per-request prefix copies",
        grid=dict(B=SWEEP_B, G=SWEEP_G, P=SWEEP_P, kv_dtype=SWEEP_DTYPES, H_kv=8, d=128, own_tokens="U{64..512}",
                  page_size=16, steps=steps, windows=3),
        defaults_when_measured={k: defaults[k] for k in DISPATCH_CONSTANTS},
        planned_mean_ratio=float(np.mean(planned)), planned_worst_ratio=float(np.max(planned)),
        planned_mean_ratio_b_ge_2=float(np.mean(planned_multi)),
        planned_worst_ratio_b_ge_2=float(np.max(planned_multi)),
        replay_best=replay[:10], cells=cells, source_sha256=kernel_source_hash(),
        command=f"python bench.py --dispatch-sweep {out_path}")
    write_sweep_json(out_path, rec)
    return rec


REPLAY_T_DENSE = (1, 64, 256, 1024)
REPLAY_RATIO = (1, 2, 3, 4, 5, 6, 8)
REPLAY_LAUNCH_MB = (0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 15, 20, 30)
REPLAY_CACHED_MIB = (0, 64, 96, 128, 192)  # cached_reread_bytes in MiB (0: no allowance)


# the planner constants a dispatcher sweep depends on
DISPATCH_CONSTANTS = ("t_dense", "gate_ratio", "launch_bytes", "fuse_cascade", "cached_prefix_bytes",
                      "cached_reread_bytes")


def write_sweep_json(path, rec):
    """The sweep record with one line per cell (a short, diffable file)."""
    head = {k: v for k, v in rec.items() if k != "cells"}
    lines = json.dumps(head, indent=1)[:-2] + ',\n "cells": [\n'
    lines += ",\n".join("  " + json.dumps(c, separators=(",", ":")) for c in rec.get("cells", []))
    with open(path, "w") as f:
        f.write(lines + "\n ]\n}\n")


def replay_sweep(cells):
    """The planner (the library's own, host only) replayed over a grid of
    candidate dispatcher constants against the measured times of a sweep:
    for each candidate, the path it picks in every cell is looked up among
    the timed paths, and its ratio to the cell's fastest path is averaged
    and maximised.  Sorted best first (worst ratio over cells with two or
    more requests, then the mean)."""
    import numpy as np
    import paged_kv_cache_201_amd as pkv
    leg_of = {"PAGED": "paged_shared", "CASCADE": "cascade", "DENSE": "dense"}

    def decide(cell, tuning):
        Bc, Gc, Pc = cell["B"], cell["G"], cell["P"]
        indptr = np.arange(Bc + 1, dtype=np.int32) * (Pc + 288)
        pl = pkv.pkv_plan_create(batch=Bc, num_q_heads=8 * Gc, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                                 kv_dtype=cell["kv_dtype"], page_size=16, kv_indptr=indptr, shared_prefix_len=Pc,
                                 tuning=tuning)
        return pl.info["path_name"]

    replay = []
    for t_dense, ratio, launch, cached in itertools.product(REPLAY_T_DENSE, REPLAY_RATIO, REPLAY_LAUNCH_MB,
                                                            REPLAY_CACHED_MIB):
        tune = dict(t_dense=t_dense, gate_ratio=ratio, launch_bytes=launch * 10**6, cached_reread_bytes=cached << 20)
        ratios = []
        for cell in cells:
            path = decide(cell, tune)
            t = cell["us"].get(leg_of[path], cell["us"]["paged_shared"])
            best = min(v for k, v in cell["us"].items() if k in ("paged_shared", "cascade", "dense"))
            ratios.append(t / best)
        multi = [r for r, c in zip(ratios, cells) if c["B"] >= 2]
        replay.append(dict(tuning=tune, mean_ratio=float(np.mean(ratios)), worst_ratio=float(np.max(ratios)),
                           mean_ratio_b_ge_2=float(np.mean(multi)), worst_ratio_b_ge_2=float(np.max(multi))))
    replay.sort(key=lambda r: (round(r["worst_ratio_b_ge_2"], 3), r["mean_ratio_b_ge_2"]))
    return replay


def clock_probe(name, steps):
    """`steps` decode steps of one workload back to back from a cold start
    (right after the inputs are uploaded, no warm-up), one event pair per
    step on the launch stream.  For a counter run (GRBM_GUI_ACTIVE with a
    kernel trace) that sets each dispatch's busy cycles against its
    duration: the effective clock, cold and warm."""
    import torch
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_config
    b = make_config(name, device="cuda")
    db = DeviceBatch.from_batch(b)
    plan = db.plan()
    o, lse, ws = db.new_out(), db.new_lse(), db.workspace(plan)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        db.step(plan, o, lse, ws)
        e1.record(stream)
    torch.cuda.synchronize()
    return dict(workload=name, path=plan.info["path_name"], steps=steps,
                us=[e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])


def write_clock_summary(name, run_json, prof_dir, command):
    """profiles/paged_split_kernel.<name>_clock.md: per-dispatch duration and
    effective clock (GRBM_GUI_ACTIVE, summed over the 8 XCDs, divided by 8
    and by the dispatch's duration) of the paged kernel in a cold-start
    clock-probe run, by dispatch index."""
    import csv
    import glob
    import statistics
    rec = json.loads(open(run_json).read().strip().splitlines()[-1])
    cycles, dur = {}, {}
    for f in glob.glob(os.path.join(prof_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == "GRBM_GUI_ACTIVE" and "paged_split_kernel" in r["Kernel_Name"]:
                cycles[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    for f in glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "paged_split_kernel" in r["Kernel_Name"]:
                dur[int(r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    ids = sorted(set(cycles) & set(dur))
    rows = [(i, dur[d], cycles[d] / 8 / dur[d]) for i, d in enumerate(ids)]  # MHz = cycles / us
    lines = [f"# Effective clock of the paged kernel, {name} ({rec.get('path')}), cold start", "", "Command:", "",
             "```", command, "```", "",
             "Each decode step of the workload back to back from a cold start (no warm-up). Per dispatch of "
             "`paged_split_kernel`: duration from the kernel trace, and effective clock = GRBM_GUI_ACTIVE "
             "(summed over the 8 XCDs) / 8 / duration. (The run's own event-timed steps are not shown: the "
             "counter collection serialises the dispatches.)",
             "", "| dispatches | kernel us (median) | kernel us (min..max) | clock MHz (median) | clock MHz (min..max) |",
             "|---|---|---|---|---|"]
    for lo, hi in ((0, 1), (1, 5), (5, 20), (20, 50), (50, 100), (100, 200), (200, len(rows))):
        part = rows[lo:hi]
        if not part:
            continue
        du = [r[1] for r in part]
        mh = [r[2] for r in part]
        lines.append(f"| {lo}..{hi - 1} | {statistics.median(du):.1f} | {min(du):.1f}..{max(du):.1f} | "
                     f"{statistics.median(mh):.0f} | {min(mh):.0f}..{max(mh):.0f} |")
    lines.append("")
    lines.append(f"Source sha256 of the profiled library: `{rec.get('source_sha256')}`")
    path = os.path.join(ROOT, "profiles", f"paged_split_kernel.{name}_clock.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def page_control(steps, warmup):
    """Page size as a control ("The 25% Page-Size Slowdown That Wasn't",
    section "A backend where pages really do reach the kernel"): the paged
    pass reading the page table (page-aware) and reading token-flat indices,
    at page sizes 16, 64 and 128, on distinct K/V (16 requests of 8192 own
    tokens: the DRAM-bound regime) and on a shared prefix (32 requests on
    the same 8192 tokens in shared physical pages: the reuse regime).  Each
    leg records how many paged-pass dispatches it issued, in the order
    listed, so that counter runs can attribute dispatches to legs."""
    import torch
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_decode_batch, relayout
    legs = []
    cases = (("distinct", dict(seed=1007, B=16, own_len=(8192, 8192), prefix_len=0)),
             ("shared", dict(seed=1008, B=32, own_len=(0, 0), prefix_len=8192)))
    for case, kw in cases:
        base = make_decode_batch(H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="bf16", page_size=16,
                                 layout="shared", device="cuda", **kw)
        for p in (16, 64, 128):
            b = base if p == 16 else relayout(base, page_size=p, seed=2007, layout="shared", device="cuda")
            db = DeviceBatch.from_batch(b)
            # the shared case declares its prefix (the pass re-reads it from L2)
            plan = db.plan(shared_prefix_len=b.prefix_len, force_path=0)
            o, lse, ws = db.new_out(), db.new_lse(), db.workspace(plan)
            for mode in ("page_table", "token_flat"):
                fn = ((lambda: db.paged_pages(plan, o=o, lse=lse, ws=ws)) if mode == "page_table"
                      else (lambda: db.paged(plan, o=o, lse=lse, ws=ws)))
                t = time_windows(fn, steps, warmup)
                ms = t["ms"]
                nb = algorithmic_bytes(b, "PAGED")
                legs.append(dict(case=case, page_size=p, mode=mode, us_per_step=ms * 1e3,
                                 requested_gbs=nb / (ms * 1e-3) / 1e9, dispatches=t["calls"],
                                 page_entries=int(b.page_indptr[-1]), tokens=int(b.seq_lens.sum())))
            del db, o, lse, ws
            if b is not base:
                del b
            torch.cuda.empty_cache()
        del base
        torch.cuda.empty_cache()
    return legs


def write_page_control(run_json, vmem_dir, tcc_dir, commands):
    """profiles/paged_split_kernel.page_size_control.md from one timing run
    and two counter runs of --page-control."""
    import statistics
    rec = json.loads(open(run_json).read().strip().splitlines()[-1])
    legs = rec["page_control"]

    def per_leg(d, counter):
        # the counter run's own legs (its stdout, saved next to its output
        # folder) say how many dispatches each leg issued
        import csv
        import glob
        run_legs = json.loads(open(d.rstrip("/") + ".json").read().strip().splitlines()[-1])["page_control"]
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter and "paged_split_kernel" in r["Kernel_Name"]:
                    rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        rows.sort()
        vals, at = [], 0
        for leg in run_legs:
            chunk = [v for _, v in rows[at:at + leg["dispatches"]]]
            at += leg["dispatches"]
            vals.append(statistics.median(chunk) if chunk else None)
        return vals

    vmem = per_leg(vmem_dir, "SQ_INSTS_VMEM_RD")
    hit = per_leg(tcc_dir, "TCC_HIT_sum")
    miss = per_leg(tcc_dir, "TCC_MISS_sum")
    lines = ["# Page size as a control: paged_split_kernel, page-table reads vs token-flat indices", "",
             "Commands:", "", "```"] + [commands[k] for k in ("time", "vmem", "tcc", "summary")] + ["```", "",
             "Distinct: 16 requests x 8192 own tokens (537 MB of K/V per step, DRAM-bound). Shared: 32 requests "
             "on one 8192-token prefix in shared physical pages (the same 16.8 MB re-read by every request). "
             "Same plan at every page size (work is cut by logical position). `vmem_rd` = vector-memory read "
             "instructions per dispatch (`SQ_INSTS_VMEM_RD`), `L2 hit` = TCC_HIT / (TCC_HIT + TCC_MISS).", "",
             "| case | page size | reads | page entries | us/step | requested GB/s | vmem_rd per dispatch | L2 hit |",
             "|---|---|---|---|---|---|---|---|"]
    for leg, v, h, m in zip(legs, vmem, hit, miss):
        rate = f"{100 * h / (h + m):.1f} %" if h is not None and m is not None and h + m > 0 else "-"
        lines.append(f"| {leg['case']} | {leg['page_size']} | {leg['mode']} | "
                     f"{leg['page_entries'] if leg['mode'] == 'page_table' else leg['tokens']} | "
                     f"{leg['us_per_step']:.1f} | {leg['requested_gbs']:.0f} | "
                     f"{v:.0f} | {rate} |" if v is not None else
                     f"| {leg['case']} | {leg['page_size']} | {leg['mode']} | - | {leg['us_per_step']:.1f} | "
                     f"{leg['requested_gbs']:.0f} | - | {rate} |")
    lines.append("")
    lines.append(f"Source sha256 of the profiled library: `{rec.get('source_sha256')}`")
    path = os.path.join(ROOT, "profiles", "paged_split_kernel.page_size_control.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def read_ceiling(steps=20, warmup=5, nbytes=4 << 30):
    """Streaming-read bandwidth of this GPU (GB/s), through the library's read
    probe: by default over 4 GiB, far more than the 256 MB Infinity Cache;
    with ``nbytes`` set to a step's byte count, what one contiguous read of
    that size reaches (launch ramp and tail included)."""
    import torch
    import paged_kv_cache_201_amd as pkv
    n = nbytes // 16 * 16
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    if nbytes == 4 << 30:
        # filled by the library's write probe: a write of known size for the
        # write-traffic counter's calibration
        pkv.pkv_stream_write_probe(buf, 0x01010101, 1024)
    best = None
    for wgs in (512, 1024, 2048):
        out = torch.empty(wgs, dtype=torch.int32, device="cuda")
        ms = time_steps(lambda: pkv.pkv_stream_read_probe(buf, out, wgs), steps, warmup)
        gbs = n / (ms * 1e-3) / 1e9
        best = max(best or 0, gbs)
    del buf
    torch.cuda.empty_cache()
    return best


# ------------------------------------------------------------ profiles --

CSRC = os.path.join(ROOT, "paged_kv_cache_201_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "paged_split_kernel.llama_layer_p1.traffic.json")


def kernel_source_hash():
    """sha256 over the library sources and headers: counters taken before a
    change of any of them no longer describe the kernels."""
    import hashlib
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(d)):
            if name.endswith((".h", ".hip", ".cpp")):
                h.update(name.encode())
                h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def _short(name):
    name = name.replace("void ", "")
    return name.split("(")[0]


def summarize_trace(prof_dir):
    """Markdown table of kernel durations from a rocprofv3 --kernel-trace csv run."""
    import csv
    import glob
    import statistics
    rows = []
    for f in glob.glob(os.path.join(prof_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    agg = {}
    for r in rows:
        n = _short(r["Kernel_Name"])
        wg = int(r["Workgroup_Size_X"])
        key = (n, int(r["Grid_Size_X"]) // wg, int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]), wg)
        agg.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | workgroups (x,y,z) | threads | calls | mean us | median us | min us |",
           "|---|---|---|---|---|---|---|"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{k[0]}` | {k[1]},{k[2]},{k[3]} | {k[4]} | {len(v)} | {statistics.mean(v):.1f} | "
                   f"{statistics.median(v):.1f} | {min(v):.1f} |")
    return "\n".join(out), agg


PLANNED_TRACE_CONFIGS = "c2,c2p128,c5,c1,c3,c4,c3_fp8,groups4,tree4"
PLANNED_TRACE_STEPS, PLANNED_TRACE_WARMUP = 60, 200


def trace_planned(name, steps, warmup):
    """The planner's step of one workload, nothing else (for a kernel trace):
    warmup steps, then steps steps.  c2p128 is the Llama layer at page size
    128 (c2 itself at page size 1, as in the headline)."""
    import torch
    from paged_kv_cache_201_amd.step import DeviceBatch
    from workloads import make_config
    if name in ("groups4", "tree4"):
        from workloads import make_group_config, make_tree_config
        b = (make_tree_config if name.startswith("tree") else make_group_config)(name, device="cuda")
        db = DeviceBatch.from_batch(b)
        plan = db.plan_grouped()
        meta, ws = db.metadata(plan), db.workspace(plan)
        run = lambda: db.step_grouped(plan, meta, o, lse, ws)
    else:
        over = dict(page_size=1) if name == "c2" else {}
        b = make_config("c2" if name == "c2p128" else name, device="cuda", **over)
        db = DeviceBatch.from_batch(b)
        plan = db.plan(shared_prefix_len=b.prefix_len)
        ws = db.workspace(plan)
        run = lambda: db.step(plan, o, lse, ws)
    o, lse = db.new_out(), db.new_lse()
    for _ in range(warmup + steps):
        run()
    torch.cuda.synchronize()
    return dict(workload=name, path=plan.info["path_name"], steps=steps, warmup=warmup)


def write_planned_traces(parent, configs, command):
    """profiles/kernels.planned_steps.trace.md: for each workload, the
    library's kernels in its planned step (one kernel-trace run per workload
    under parent/<workload>), medians over the second half of each kernel's
    calls (the steady state after the warm-up)."""
    import csv
    import glob
    import statistics
    out = [f"# Kernel durations of each workload's planned step\n",
           "One `rocprofv3 --kernel-trace` run per workload, each running only the planner's step "
           f"({PLANNED_TRACE_WARMUP} warm-up steps, then {PLANNED_TRACE_STEPS}); library kernels only; "
           "median, mean and minimum over the second half of each kernel's calls.\n",
           "Command (per workload W):\n", f"```\n{command}\n```\n"]
    for name in configs.split(","):
        agg = {}
        for f in glob.glob(os.path.join(parent, name, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if "pkv::" not in r["Kernel_Name"]:
                    continue
                wg = int(r["Workgroup_Size_X"])
                key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // wg, int(r["Grid_Size_Y"]), wg)
                agg.setdefault(key, []).append((int(r["Start_Timestamp"]),
                                                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        out.append(f"## {name}\n")
        if not agg:
            out.append("(no trace)\n")
            continue
        out.append("| kernel | workgroups (x,y) | threads | calls | median us | mean us | min us |")
        out.append("|---|---|---|---|---|---|---|")
        total = 0.0
        for k, v in sorted(agg.items(), key=lambda kv: kv[1][0][0]):
            d = [x for _, x in sorted(v)][len(v) // 2:]
            total += statistics.median(d)
            out.append(f"| `{k[0]}` | {k[1]},{k[2]} | {k[3]} | {len(v)} | {statistics.median(d):.1f} | "
                       f"{statistics.mean(d):.1f} | {min(d):.1f} |")
        out.append(f"\nSum of kernel medians: {total:.1f} us per step.\n")
    out.append(f"Source sha256 of the profiled library: `{kernel_source_hash()}`\n")
    path = os.path.join(ROOT, "profiles", "kernels.planned_steps.trace.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    return path


def write_trace_summary(trace_dir, name, title, command):
    """profiles/kernels.<name>.trace.md from one rocprofv3 --kernel-trace run."""
    table, _ = summarize_trace(trace_dir)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = os.path.join(ROOT, "profiles", f"kernels.{name}.trace.md")
    with open(path, "w") as f:
        f.write(f"# Kernel durations, {title}\n\nCommand:\n\n```\n{command}\n```\n\n{table}\n")
    return path


def pmc_per_dispatch(prof_dir, counter):
    """{(kernel, grid size): [counter value per dispatch]} from a rocprofv3 --pmc csv run."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(prof_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
            out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def write_profile_summaries(trace_dir, fetch_dir, write_dir, commands):
    """Turn the rocprofv3 output of the three profiling runs of the headline
    workload into the committed summaries under profiles/."""
    table, agg = summarize_trace(trace_dir)
    # the sources the profiled run was built from (its bench line), else these
    try:
        sha = json.loads(open(trace_dir.rstrip("/") + ".json").read().strip().splitlines()[-1])["source_sha256"]
    except (OSError, ValueError, KeyError, IndexError):
        sha = kernel_source_hash()
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "kernels.llama_layer.trace.md"), "w") as f:
        f.write("# Kernel durations, Llama-3.1-8B decode layer (B=32, 4096 tokens, bf16), page size 1 and 128\n\n")
        f.write("Command:\n\n```\n" + commands["trace"] + "\n```\n\n")
        f.write("Every dispatch of the run, grouped by kernel and grid (the streaming-read probe is the "
                "read-ceiling measurement; `paged_split_kernel` + `split_reduce_kernel` are one decode step).\n\n")
        f.write(table + "\n")
        f.write(f"\nSource sha256 of the profiled library: `{sha}`\n")
    fetch = pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = pmc_per_dispatch(write_dir, "WRITE_SIZE")
    med = lambda v: sorted(v)[len(v) // 2]
    # calibration: the read probe reads its 4 GiB buffer once (smaller probe
    # reads of a step's size are left out); the write probe writes it once
    probe = [v for (k, _), vs in fetch.items() if "stream_read_kernel" in k for v in vs]
    probe = [v for v in probe if v > 0.5 * max(probe)]
    fills = [max(vs) for (k, _), vs in write.items() if "stream_write_kernel" in k]
    nbytes = 4 << 30
    fetch_scale = nbytes / (med(probe) * 1024)
    write_scale = nbytes / (max(fills) * 1024)
    kernels = {}
    for (k, grid), vs in fetch.items():
        if "paged_split_kernel" in k or "split_reduce_kernel" in k:
            w = write.get((k, grid), [0.0])
            kernels[f"{k} grid={grid}"] = dict(dispatches=len(vs), fetch_kib_median=med(vs),
                                               write_kib_median=med(w),
                                               bytes=med(vs) * 1024 * fetch_scale + med(w) * 1024 * write_scale)
    rec = dict(workload="Llama-3.1-8B decode layer, B=32, 4096 tokens, bf16, page size 1 and 128 (same plan)",
               commands=commands, source_sha256=sha, fetch_scale=fetch_scale,
               write_scale=write_scale,
               calibration="FETCH_SIZE of the streaming-read probe over 4 GiB; WRITE_SIZE of the streaming-write "
                           "probe filling the same 4 GiB buffer",
               kernels=kernels, traffic_bytes_per_step=sum(v["bytes"] for v in kernels.values()))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def write_prefix_traffic(name, unique_dir, separate_dir, commands):
    """Prefix-traffic reduction of a shared-prefix workload from two FETCH_SIZE
    runs: PAGED over per-request prefix copies, and the cascade step run as
    separate launches (so that the prefix pass has its own dispatches)."""
    import statistics
    from workloads import make_config
    b = make_config(name)
    P, B = b.prefix_len, b.B
    prefix_bytes = P * b.H_kv * b.d * 2 * BYTES[b.kv_dtype]
    res = {}
    for label, d in (("paged_unique", unique_dir), ("cascade_separate", separate_dir)):
        fetch = pmc_per_dispatch(d, "FETCH_SIZE")
        probe = [v for (k, _), vs in fetch.items() if "stream_read_kernel" in k for v in vs]
        scale = (4 << 30) / (statistics.median(probe) * 1024)
        per = {}
        for (k, grid), vs in fetch.items():
            if k.startswith("pkv::") and "stream_read" not in k:
                per[f"{k} grid={grid}"] = statistics.median(vs) * 1024 * scale
        res[label] = dict(fetch_scale=scale, bytes_per_dispatch=per)
    pre = [v for k, v in res["cascade_separate"]["bytes_per_dispatch"].items() if "prefix_attn_kernel" in k]
    uniq = sum(v for k, v in res["paged_unique"]["bytes_per_dispatch"].items() if "paged_split_kernel" in k)
    casc = sum(res["cascade_separate"]["bytes_per_dispatch"].values())
    try:
        sha = json.loads(open(separate_dir.rstrip("/") + ".json").read().strip().splitlines()[-1])["source_sha256"]
    except (OSError, ValueError, KeyError, IndexError):
        sha = kernel_source_hash()
    rec = dict(workload=f"{name}: B={B} requests sharing a {P}-token prefix, {b.H_q}/{b.H_kv} heads, d={b.d}, "
                        f"{b.kv_dtype}, page size {b.page_size}",
               commands=commands, source_sha256=sha, prefix_bytes=prefix_bytes,
               per_request_prefix_bytes_total=B * prefix_bytes,
               prefix_pass_fetch_bytes=sum(pre),
               reduction_vs_per_request_reads=B * prefix_bytes / sum(pre) if pre else None,
               paged_unique_fetch_bytes=uniq, cascade_step_fetch_bytes=casc,
               saved_over_prefix_bytes=(uniq - casc) / prefix_bytes, runs=res)
    path = os.path.join(ROOT, "profiles", f"prefix_attn_kernel.{name}_shared_prefix.traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


PREFIX_MFMA_COUNTERS = "MfmaUtil MfmaFlopsBF16 SQ_INSTS_MFMA SQ_INSTS_VALU SQ_BUSY_CYCLES"
PREFIX_LDS_COUNTERS = "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_WAVE_CYCLES GRBM_GUI_ACTIVE"


def write_prefix_counters(name, mfma_dir, lds_dir, commands):
    """MFMA utilisation, MFMA flops and LDS / wait counters of a shared-prefix
    workload's prefix pass (run as its own launch), per dispatch."""
    import statistics
    from workloads import make_config
    b = make_config(name)
    flops = 4 * b.B * b.G * b.prefix_len * b.d * b.H_kv
    med = {}
    for d, names in ((mfma_dir, PREFIX_MFMA_COUNTERS), (lds_dir, PREFIX_LDS_COUNTERS)):
        for c in names.split():
            vals = [v for (k, _), vs in pmc_per_dispatch(d, c).items() if "prefix_attn" in k for v in vs]
            med[c] = statistics.median(vals) if vals else None
    try:
        sha = json.loads(open(mfma_dir.rstrip("/") + ".json").read().strip().splitlines()[-1])["source_sha256"]
    except (OSError, ValueError, KeyError, IndexError):
        sha = kernel_source_hash()
    ratio = lambda x, y: (x / y) if (x is not None and y) else None  # noqa: E731
    rec = dict(workload=f"{name}: prefix pass of B={b.B} requests over a {b.prefix_len}-token prefix, "
                        f"M_eff={b.B * b.G}, {b.H_kv} KV heads, d={b.d}, {b.kv_dtype}",
               commands=commands, source_sha256=sha, algorithmic_flops=flops, counters_median_per_dispatch=med,
               mfma_util_pct=med.get("MfmaUtil"),
               mfma_flops_over_algorithmic=ratio(med.get("MfmaFlopsBF16"), flops),
               lds_bank_conflict_over_lds_active=ratio(med.get("SQ_LDS_BANK_CONFLICT"), med.get("SQ_LDS_IDX_ACTIVE")),
               wait_over_wave_cycles=ratio(med.get("SQ_WAIT_ANY"), med.get("SQ_WAVE_CYCLES")),
               active_inst_over_wave_cycles=ratio(med.get("SQ_ACTIVE_INST_ANY"), med.get("SQ_WAVE_CYCLES")))
    path = os.path.join(ROOT, "profiles", f"prefix_attn_kernel.{name}_shared_prefix.counters.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


PAGED_VALU_COUNTERS = ("SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_THREAD_CYCLES_VALU SQ_WAVE_CYCLES SQ_BUSY_CYCLES "
                       "SQ_WAIT_ANY SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE")
# the paged kernel of each workload in a `--configs c2,c5` run (kernel name, grid size)
# the paged kernel of each workload in the counter run: the bf16 and the fp8
# instantiation (KV template argument 1 and 2) with the most dispatches
PAGED_COUNTER_KERNELS = {"c2": "pkv::paged_split_kernel<1,", "c5": "pkv::paged_split_kernel<2,"}


def write_paged_counters(valu_dir, fetch_dir, commands):
    """Vector-ALU and wait counters of the paged kernel on the Llama layer
    (bf16, G = 4) and the long fp8 workload (G = 8), per dispatch; and a
    repeat of the headline FETCH_SIZE pass, against the committed traffic
    summary (byte-count drift between two profiles of the same step)."""
    import statistics
    from workloads import make_config
    out = {}
    per_counter = {c: pmc_per_dispatch(valu_dir, c) for c in PAGED_VALU_COUNTERS.split()}
    for name, prefix in PAGED_COUNTER_KERNELS.items():
        b = make_config(name)
        tokens = int(sum(int(x) for x in b.seq_lens))
        cands = {k: len(v) for k, v in per_counter["SQ_INSTS_VALU"].items() if k[0].startswith(prefix)}
        key = max(cands, key=cands.get) if cands else (prefix, 0)
        med = {}
        for c in PAGED_VALU_COUNTERS.split():
            vals = per_counter[c].get(key, [])
            med[c] = statistics.median(vals) if vals else None
        ratio = lambda x, y: (x / y) if (x is not None and y) else None  # noqa: E731
        out[name] = dict(kernel=f"{key[0]} grid={key[1]}", tokens=tokens, kv_heads=b.H_kv, group=b.G,
                         kv_dtype=b.kv_dtype, counters_median_per_dispatch=med,
                         valu_insts_per_token_and_kv_head=ratio(med["SQ_INSTS_VALU"], tokens * b.H_kv),
                         active_valu_over_wave_cycles=ratio(med["SQ_ACTIVE_INST_VALU"], med["SQ_WAVE_CYCLES"]),
                         wait_over_wave_cycles=ratio(med["SQ_WAIT_ANY"], med["SQ_WAVE_CYCLES"]),
                         active_inst_over_wave_cycles=ratio(med["SQ_ACTIVE_INST_ANY"], med["SQ_WAVE_CYCLES"]),
                         valu_lane_use=ratio(med["SQ_THREAD_CYCLES_VALU"],
                                             None if med["SQ_ACTIVE_INST_VALU"] is None
                                             else 64 * med["SQ_ACTIVE_INST_VALU"]))
    # FETCH_SIZE repeat of the headline step against the committed summary
    prev = json.load(open(TRAFFIC_FILE))
    fetch = pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    repeat = {}
    for (k, grid), vs in fetch.items():
        label = f"{k} grid={grid}"
        if label in prev["kernels"]:
            now = statistics.median(vs)
            was = prev["kernels"][label]["fetch_kib_median"]
            repeat[label] = dict(fetch_kib_median=now, committed_fetch_kib_median=was, drift=(now - was) / was,
                                 dispatches=len(vs))
    rec = dict(commands=commands, source_sha256=kernel_source_hash(), workloads=out,
               fetch_repeat_of_committed_traffic=repeat)
    path = os.path.join(ROOT, "profiles", "paged_split_kernel.c2_c5.counters.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def measured_traffic():
    """Scaled HBM bytes per decode step of the headline workload from the
    committed counter summary, or None when the sources changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_step")


def host_timing(reps=21):
    """Median host time (us) of page-table lowering (page sizes 1 and 16) and
    planning through the C ABI, at 64 .. 2,097,152 tokens over 32 requests."""
    import ctypes
    import numpy as np
    import paged_kv_cache_201_amd as pkv
    lib = pkv._lib
    i32p = ctypes.POINTER(ctypes.c_int32)
    out = {}
    for n, p in itertools.product((64, 1024, 16384, 262144, 2097152), (1, 16)):
        B = 32
        lens = np.full(B, n // B, np.int32)
        npg = (lens + p - 1) // p
        page_indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
        pages = np.random.default_rng(n).permutation(int(npg.sum())).astype(np.int32)
        kv_indptr = np.zeros(B + 1, np.int32)
        kv_indices = np.zeros(n, np.int32)
        args = (B, p, page_indptr.ctypes.data_as(i32p), pages.ctypes.data_as(i32p), lens.ctypes.data_as(i32p),
                kv_indptr.ctypes.data_as(i32p), kv_indices.ctypes.data_as(i32p), ctypes.c_int64(n))
        tl = []
        for _ in range(reps):
            t = time.perf_counter_ns()
            st = lib.pkv_lower_page_table(*args)
            tl.append((time.perf_counter_ns() - t) / 1e3)
            assert st == 0
        prob = pkv.pkv_problem(B, 32, 8, 128, pkv.DTYPE_CODES["bf16"], pkv.DTYPE_CODES["bf16"], p,
                               kv_indptr.ctypes.data_as(i32p), 0, -1)
        tp = []
        for _ in range(reps):
            h = ctypes.c_void_p()
            t = time.perf_counter_ns()
            st = lib.pkv_plan_create(ctypes.byref(prob), None, ctypes.byref(h))
            tp.append((time.perf_counter_ns() - t) / 1e3)
            assert st == 0
            lib.pkv_plan_destroy(h)
        out[f"{n}_p{p}"] = dict(lower_us=sorted(tl)[reps // 2], plan_us=sorted(tp)[reps // 2])
    return out


def cpu_baseline(batch, min_seconds=10.0, max_steps=200):
    """The oracle, as it stands, on the same workload on the host cores: whole
    steps back to back until at least min_seconds of CPU work (a bounded
    sample).  Returns (seconds per step, threads, steps, seconds)."""
    from oracle import batch as ob
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    t = time.perf_counter()
    n = 0
    while True:
        ob.batch_reference(batch)
        n += 1
        if n >= max_steps or time.perf_counter() - t >= min_seconds:
            break
    total = time.perf_counter() - t
    return total / n, threads, n, total


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), else what platform says."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def oracle_sample(batch, requests, runs=1):
    """The oracle on a bounded sample of one workload's requests, on the host
    cores: gathering each request's contiguous K/V (stored values widened to
    float64) timed apart from the attention itself; the median of `runs`
    passes, scaled from the sample to the whole step."""
    import statistics
    from oracle import attention as oa
    from oracle import batch as ob
    gather, attend = [], []
    for _ in range(runs):
        tg = ta = 0.0
        for b in requests:
            t0 = time.perf_counter()
            q, k, v = ob.request_inputs(batch, b)
            t1 = time.perf_counter()
            oa.decode_attention(q, k, v, ob.default_scale(batch.d))
            t2 = time.perf_counter()
            tg += t1 - t0
            ta += t2 - t1
        gather.append(tg)
        attend.append(ta)
    scale = batch.B / len(requests)
    g, a = statistics.median(gather) * scale, statistics.median(attend) * scale
    return dict(ms_per_step=(g + a) * 1e3, gather_ms=g * 1e3, attention_ms=a * 1e3, runs=runs,
                sample=f"{len(requests)} of {batch.B} requests (first ones), scaled by {scale:g}",
                kind="oracle")


# requests the per-workload oracle timing samples, and passes (bounded: a few
# seconds each on the host)
ORACLE_SAMPLE = {"c1": (None, 5), "c3": (8, 1), "c4": (16, 1), "c5": (2, 1), "c3_fp8": (8, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--configs", default="c1,c2,c3,c4,c5,c3_fp8,groups4,tree4")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", metavar="CONFIG:LEG[,LEG]",
                    help="time only these legs of one shared-prefix workload (e.g. c3:paged_unique) and exit; "
                         "for profiling one leg at a time")
    ap.add_argument("--summarize-prefix-traffic", nargs=3, metavar=("CONFIG", "UNIQUE_DIR", "SEPARATE_DIR"),
                    help="write the prefix-traffic summary from two FETCH_SIZE runs (see --only) and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "CONFIGS"),
                    help="write profiles/kernels.<configs>.trace.md from a kernel-trace run of --configs CONFIGS")
    ap.add_argument("--trace-planned", metavar="CONFIG",
                    help="run only the planned step of one workload (warm-up, then steps) and exit; for a "
                         "kernel-trace run per workload")
    ap.add_argument("--summarize-planned-traces", nargs=2, metavar=("PARENT_DIR", "CONFIGS"),
                    help="write profiles/kernels.planned_steps.trace.md from PARENT_DIR/<config> kernel traces "
                         "of --trace-planned runs and exit")
    ap.add_argument("--dispatch-sweep", metavar="OUT_JSON",
                    help="run the dispatcher's forced-path refit grid, write it to OUT_JSON and exit")
    ap.add_argument("--replay-sweep", metavar="SWEEP_JSON",
                    help="replay the planner over candidate dispatcher constants against a sweep's measured times "
                         "(host only, no GPU); rewrites the file's replay and exits")
    ap.add_argument("--clock-probe", metavar="CONFIG",
                    help="run --steps decode steps of one workload from a cold start, one event pair each, print "
                         "them and exit (for a GRBM_GUI_ACTIVE counter run)")
    ap.add_argument("--summarize-clock", nargs=3, metavar=("CONFIG", "RUN_JSON", "PROF_DIR"),
                    help="write profiles/paged_split_kernel.<CONFIG>_clock.md from a clock-probe counter run")
    ap.add_argument("--page-control", action="store_true",
                    help="time the page-size control (page-table vs token-flat reads, distinct vs shared K/V) "
                         "and exit")
    ap.add_argument("--summarize-page-control", nargs=3, metavar=("RUN_JSON", "VMEM_DIR", "TCC_DIR"),
                    help="write the page-size control summary from a --page-control run and two counter runs")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 output of the headline workload and exit")
    ap.add_argument("--summarize-paged-counters", nargs=2, metavar=("VALU_DIR", "FETCH_DIR"),
                    help="write the paged kernel's vector-ALU counter summary (Llama layer and long fp8) and the "
                         "repeat of the headline FETCH_SIZE pass from two counter runs and exit")
    ap.add_argument("--summarize-prefix-counters", nargs=3, metavar=("CONFIG", "MFMA_DIR", "LDS_DIR"),
                    help="write the prefix pass's MFMA/LDS counter summary from two counter runs of "
                         "--only CONFIG:dense_separate and exit")
    args = ap.parse_args()
    if args.replay_sweep:
        rec = json.load(open(args.replay_sweep))
        replay = replay_sweep(rec["cells"])
        rec["replay_best"] = replay[:12]
        rec["replay_grid"] = dict(t_dense=REPLAY_T_DENSE, gate_ratio=REPLAY_RATIO, launch_mb=REPLAY_LAUNCH_MB,
                                   cached_reread_mib=REPLAY_CACHED_MIB)
        rec["replay_command"] = f"python bench.py --replay-sweep {args.replay_sweep}"
        import paged_kv_cache_201_amd as pkv
        if "defaults" in rec:
            rec["defaults_when_measured"] = rec.pop("defaults")
        cur = pkv.pkv_tuning_defaults()
        rec["defaults_now"] = {k: cur[k] for k in DISPATCH_CONSTANTS}
        write_sweep_json(args.replay_sweep, rec)
        print(json.dumps(replay[:5], indent=1))
        return
    if args.summarize_clock:
        name, r, d = args.summarize_clock
        cmd = (f"cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc "
               f"GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d {d} -o run -- python bench.py --clock-probe "
               f"{name} --steps 300 > {r}")
        print(write_clock_summary(name, r, d, cmd))
        return
    if args.summarize_paged_counters:
        v, f = args.summarize_paged_counters
        prof = "cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc"
        cmds = dict(valu=f"{prof} {PAGED_VALU_COUNTERS} --output-format csv -d {v} -o run -- python bench.py "
                         "--configs c2,c5 --steps 10 --warmup 2 --no-cpu",
                    fetch=f"{prof} FETCH_SIZE --output-format csv -d {f} -o run -- python bench.py --configs c2 "
                          "--steps 20 --warmup 5 --no-cpu",
                    summary=f"python bench.py --summarize-paged-counters {v} {f}")
        rec = write_paged_counters(v, f, cmds)
        print(json.dumps({k: v for k, v in rec.items() if k != "commands"}, indent=1))
        return
    if args.summarize_prefix_counters:
        name, m, l = args.summarize_prefix_counters
        prof = "cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc"
        run = f"-o run -- python bench.py --only {name}:dense_separate --steps 10 --warmup 2"
        cmds = dict(mfma=f"{prof} {PREFIX_MFMA_COUNTERS} --output-format csv -d {m} {run}",
                    lds=f"{prof} {PREFIX_LDS_COUNTERS} --output-format csv -d {l} {run}",
                    summary=f"python bench.py --summarize-prefix-counters {name} {m} {l}")
        rec = write_prefix_counters(name, m, l, cmds)
        print(json.dumps({k: v for k, v in rec.items() if k != "commands"}, indent=1))
        return
    if args.summarize_prefix_traffic:
        name, u, c = args.summarize_prefix_traffic
        prof = "cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE"
        cmds = dict(paged_unique=f"{prof} --output-format csv -d {u} -o run -- python bench.py --only {name}:paged_unique "
                                 "--steps 10 --warmup 2",
                    cascade_separate=f"{prof} --output-format csv -d {c} -o run -- python bench.py --only "
                                     f"{name}:dense_separate --steps 10 --warmup 2",
                    summary=f"python bench.py --summarize-prefix-traffic {name} {u} {c}")
        rec = write_prefix_traffic(name, u, c, cmds)
        print(json.dumps({k: v for k, v in rec.items() if k != "runs"}, indent=1))
        return
    if args.summarize_planned_traces:
        d, configs = args.summarize_planned_traces
        cmd = ("cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && timeout -k 10 180 rocprofv3 --kernel-trace "
               f"--output-format csv -d {d}/W -o run -- python bench.py --trace-planned W\n"
               f"python bench.py --summarize-planned-traces {d} {configs}")
        print(write_planned_traces(d, configs, cmd))
        return
    if args.summarize_trace:
        d, configs = args.summarize_trace
        cmd = ("cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && rocprofv3 --kernel-trace --stats "
               f"--output-format csv -d {d} -o run -- python bench.py --configs {configs} --steps 20 --warmup 20 --no-cpu")
        title = (f"workloads {configs} (each leg of the shared-prefix workloads, then the long fp8 workload; "
                 "the Llama layer at page size 1 and 128 runs first in every bench run)")
        print(write_trace_summary(d, configs.replace(",", "_"), title, cmd))
        return
    if args.summarize_profiles:
        t, f, w = args.summarize_profiles
        prof = "cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && "
        run = "-- python bench.py --configs c2 --steps 20 --warmup 5 --no-cpu"
        cmds = dict(trace=f"{prof}rocprofv3 --kernel-trace --stats --output-format csv -d {t} -o run {run}",
                    fetch=f"{prof}timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {f} -o run {run}",
                    write=f"{prof}timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {w} -o run {run}",
                    summary=f"python bench.py --summarize-profiles {t} {f} {w}")
        rec = write_profile_summaries(t, f, w, cmds)
        print(json.dumps(rec["kernels"], indent=1))
        return
    if args.summarize_page_control:
        r, v, t = args.summarize_page_control
        prof = "cd /tmp && export TMPDIR=/tmp && cd $GRAFT_REPO_ROOT && "
        run = "-- python bench.py --page-control --steps 5 --warmup 2"
        cmds = dict(time=f"python bench.py --page-control > {r}",
                    vmem=f"{prof}timeout -s KILL 120 rocprofv3 --pmc SQ_INSTS_VMEM_RD --output-format csv -d {v} "
                         f"-o run {run} > {v}.json",
                    tcc=f"{prof}timeout -s KILL 120 rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv "
                        f"-d {t} -o run {run} > {t}.json",
                    summary=f"python bench.py --summarize-page-control {r} {v} {t}")
        print(write_page_control(r, v, t, cmds))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the decode step shards by request or KV head with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if args.trace_planned:
        rec = trace_planned(args.trace_planned, PLANNED_TRACE_STEPS, PLANNED_TRACE_WARMUP)
        rec["source_sha256"] = kernel_source_hash()
        print(json.dumps(rec), flush=True)
        return
    if args.clock_probe:
        rec = clock_probe(args.clock_probe, args.steps)
        rec["source_sha256"] = kernel_source_hash()
        print(json.dumps(rec), flush=True)
        return
    if args.dispatch_sweep:
        rec = dispatch_sweep(args.dispatch_sweep)
        print(json.dumps({k: v for k, v in rec.items() if k != "cells"}), flush=True)
        return
    if args.page_control:
        legs = page_control(args.steps, args.warmup)
        print(json.dumps(dict(page_control=legs, steps=args.steps, warmup=args.warmup,
                              source_sha256=kernel_source_hash())), flush=True)
        return
    if args.only:
        name, legs = args.only.split(":")
        read_ceiling(steps=1, warmup=0)  # a known 4 GiB read, to scale FETCH_SIZE by
        rec = bench_prefix_config(name, args.steps, args.warmup, legs=legs.split(","))
        rec["source_sha256"] = kernel_source_hash()
        print(json.dumps(rec), flush=True)
        return
    wanted = args.configs.split(",")
    extra = {}
    log = lambda m: print(m, file=sys.stderr, flush=True)
    log("streaming-read ceiling")
    ceiling = read_ceiling()
    extra["read_ceiling_gbs"] = ceiling
    log(f"read ceiling {ceiling:.0f} GB/s")

    # headline: Llama-3.1-8B layer, page size 1 (token-flat scatter) and 128
    log("bench c2 p=1")
    rec1, b1, db1, plan1 = bench_paged_config("c2", args.steps, args.warmup, page_size=1)
    add_ceiling(rec1, ceiling)
    log(json.dumps(rec1))
    # the same number of bytes as one contiguous streaming read
    same = read_ceiling(nbytes=rec1["algorithmic_bytes"])
    log(f"read of the step's {rec1['algorithmic_bytes'] / 1e6:.1f} MB as one stream: {same:.0f} GB/s")
    del db1
    torch.cuda.empty_cache()
    log("bench c2 p=128")
    rec128, b128, db128, plan128 = bench_paged_config("c2", args.steps, args.warmup)
    add_ceiling(rec128, ceiling)
    log(json.dumps(rec128))
    # the same step with the kernel reading the page table (1,024 page entries
    # instead of 131,072 token indices)
    o, lse, ws = db128.new_out(), db128.new_lse(), db128.workspace(plan128)
    t = time_windows(lambda: db128.paged_pages(plan128, o=o, lse=lse, ws=ws), args.steps, args.warmup)
    nb = rec128["algorithmic_bytes"] - 4 * 32 * 4096 + 4 * 32 * (4096 // 128)
    extra["c2_page128_page_table"] = leg(t, nb, valu_flops=valu_flops(32 * 4096, b128))
    log(json.dumps(extra["c2_page128_page_table"]))
    del o, lse, ws
    del db128, b128
    torch.cuda.empty_cache()
    extra["c2_page128"] = rec128
    for name in wanted:
        if name in ("c1", "c5"):
            log(f"bench {name}")
            r, bb, db, _ = bench_paged_config(name, args.steps, args.warmup)
            extra[name] = add_ceiling(r, ceiling)
            del db
            torch.cuda.empty_cache()
            if not args.no_cpu:
                n, runs = ORACLE_SAMPLE[name]
                r["oracle"] = oracle_sample(bb, list(range(n or bb.B)), runs)
                r["oracle"]["gpu_speedup"] = r["oracle"]["ms_per_step"] / (r["us_per_step"] / 1e3)
            log(json.dumps(r))
            del bb
        elif name in ("c3", "c4", "c3_fp8"):
            log(f"bench {name}")
            extra[name] = bench_prefix_config(name, args.steps, args.warmup, oracle=not args.no_cpu)
            log(json.dumps(extra[name]))
        elif name in ("groups4", "tree4"):
            log(f"bench {name}")
            extra[name] = bench_groups_config(name, args.steps, args.warmup)
            log(json.dumps(extra[name]))

    extra["host_us"] = host_timing()
    log(f"host timing {json.dumps(extra['host_us'])}")

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle) on c2")
        dt, threads, n_steps, total = cpu_baseline(b1)
        nbytes = rec1["algorithmic_bytes"]
        cpu = dict(value=nbytes / dt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                   sample=f"the whole Llama-layer step (B=32, 4096 tokens, bf16 widened to fp64) {n_steps} times "
                          f"back to back, {total:.1f} s: {dt:.2f} s per step",
                   cpu_model=cpu_model(), cpu_count=os.cpu_count())

    ms = rec1["us_per_step"] / 1e3
    line = {
        "metric": "decode-attn HBM GB/s (algorithmic bytes / step time), Llama-3.1-8B layer, page size 1",
        "value": rec1["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": rec1["us_per_step"],
        "us_min": rec1["us_min"],
        "us_max": rec1["us_max"],
        "timing": f"median of {rec1['windows']} windows of {args.steps} steps each, after {args.warmup} warm-up "
                  f"steps and {rec1['warm_windows']} warm-up windows (at least {MIN_WARM_S:g} s, until two "
                  f"windows agree within {100 * STABLE_TOL:g} %)",
        "pct_peak": rec1["pct_peak"],
        "pct_read_ceiling": rec1["pct_read_ceiling"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q, token-flat indices over a randomly permuted pool)",
        "config": {"workload": "Llama-3.1-8B decode layer: B=32, 32 q / 8 kv heads, head_dim 128, 4096 tokens "
                               "per request, bf16, kv_indices of length 131072, page size 1",
                   "global_batch": 32, "seq_len": 4096, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": rec1["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": rec1["gbs"] / PEAK_HBM_GBS, "traffic": measured_traffic(),
                     "kernel": "paged decode step: paged_split_kernel + split_reduce_kernel, timed together "
                               "(events cannot split one library call)",
                     "read_ceiling_gbs": ceiling,
                     # one contiguous streaming read of exactly the step's bytes
                     "read_ceiling_same_bytes_gbs": same,
                     "frac_of_same_bytes_read": rec1["gbs"] / same},
        "cpu_baseline": cpu,
        "source_sha256": kernel_source_hash(),
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
