"""Pins of the test oracle against facts that do not come from the oracle.

Each check is a function taking the oracle routine under test, so that the
same check also runs against deliberately broken copies of the oracle (the
``test_mutant_*`` cases at the bottom): a plausible mistake must fail at
least one pin.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import lowering as ol
from oracle import planner as op
from oracle import values as ov

RNG = np.random.default_rng(7)


# ---------------------------------------------------------------- values ---

def check_fp8_table(decode_one):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = np.array([decode_one(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_fp8_all_codes_match_torch():
    check_fp8_table(ov.fp8_e4m3_value)
    assert np.array_equal(ov.FP8_E4M3_TABLE[:0x7F], [ov.fp8_e4m3_value(c) for c in range(0x7F)])


def test_bf16_widening_matches_torch():
    bits = RNG.integers(0, 1 << 16, size=20000, dtype=np.int64).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = ov.bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


F32_SPECIAL_BITS = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x00800000, 0x3F800000,
                             0xBF800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001],
                            np.uint32)


def check_f32_widening(widen):
    """The tiny workload stores fp32 values; its bits must reach float64 as a
    bit-view, not as integers.  Torch's own reinterpretation of the same bits
    is the reference: random patterns plus signed zeros, subnormals, the
    largest finite value, infinities and NaNs."""
    bits = np.concatenate([RNG.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32),
                           F32_SPECIAL_BITS])
    stored = bits.view(np.int32)  # the dtype the workloads keep fp32 bits in
    ref = torch.from_numpy(stored.copy()).view(torch.float32).to(torch.float64).numpy()
    got = widen(stored)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))  # -0.0 stays negative


def test_f32_widening_matches_torch():
    check_f32_widening(ov.f32_bits_to_f64)
    # and through the dtype switch the batch code uses
    check_f32_widening(lambda b: ov.stored_to_f64(b, "f32"))


def check_default_scale(default_scale):
    """The Llama-layer workload states its softmax scale, 1/sqrt(128); the
    reading taken for the other workloads is 1/sqrt(d) (tiny: d = 64 -> 1/8)."""
    s = default_scale(128)
    assert abs(s * s * 128 - 1) < 1e-15 and s > 0
    assert default_scale(64) == 0.125


def test_default_scale_is_the_stated_one():
    from oracle import batch as ob
    check_default_scale(ob.default_scale)


def _small_batch(kv_dtype, q_dtype, seed=5, **kw):
    from workloads import make_decode_batch
    args = dict(seed=seed, B=3, H_q=8, H_kv=2, d=16, own_len=(1, 9), prefix_len=5, q_dtype=q_dtype,
                kv_dtype=kv_dtype, page_size=4)
    args.update(kw)
    return make_decode_batch(**args)


def _torch_widened(batch, b):
    """Request b's stored query, keys and values widened by torch's own
    conversions (fp8: torch's float8_e4m3fn decode times the head's scale)."""
    k, v = batch.logical_kv(b)
    q = batch.q[b].to(torch.float64).numpy()
    k, v = k.to(torch.float64).numpy(), v.to(torch.float64).numpy()
    if batch.kv_dtype == "fp8":
        k = k * np.asarray(batch.k_scale, np.float64)[None, :, None]
        v = v * np.asarray(batch.v_scale, np.float64)[None, :, None]
    return q, k, v


def check_request_inputs(request_inputs):
    """K is widened with the K scales and V with the V scales: an fp8 batch
    whose V scales are made unlike its K scales (x3 on every head) must give
    torch's decode of each times its own scale; bf16 and fp32 batches
    likewise, and a token range selects those logical tokens."""
    for kv, qd in (("fp8", "bf16"), ("bf16", "bf16"), ("f32", "f32")):
        batch = _small_batch(kv, qd)
        if kv == "fp8":
            batch.v_scale = (np.asarray(batch.v_scale, np.float32) * np.float32(3.0)).astype(np.float32)
            assert not np.allclose(batch.k_scale, batch.v_scale)
        for b in range(batch.B):
            q, k, v = request_inputs(batch, b)
            tq, tk, tv = _torch_widened(batch, b)
            assert np.array_equal(q, tq) and np.array_equal(k, tk) and np.array_equal(v, tv), (kv, b)
            L = int(batch.seq_lens[b])
            q2, k2, v2 = request_inputs(batch, b, (2, L - 1))
            assert np.array_equal(k2, tk[2:L - 1]) and np.array_equal(v2, tv[2:L - 1]), (kv, b)


def test_request_inputs_widen_k_and_v_with_their_own_scales():
    from oracle import batch as ob
    check_request_inputs(ob.request_inputs)


def check_batch_reference(batch_reference, prefix_reference):
    """A whole batch against torch's SDPA in float64 on torch-widened inputs
    (scale 1/sqrt(d)), the suffix form (tokens from token_start on) and the
    prefix form (the first tokens)."""
    for kv, qd in (("fp8", "bf16"), ("bf16", "bf16"), ("f32", "f32")):
        batch = _small_batch(kv, qd, seed=9)
        if kv == "fp8":
            batch.v_scale = (np.asarray(batch.v_scale, np.float32) * np.float32(0.5)).astype(np.float32)
        G, d = batch.G, batch.d

        def sdpa(q, k, v):
            qt = torch.from_numpy(q)[None, :, None, :]
            kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
            o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=d ** -0.5)[0, :, 0]
            lse = torch.logsumexp((qt @ kt.transpose(-1, -2))[0, :, 0] * d ** -0.5, dim=-1)
            return o.numpy(), lse.numpy()

        o, lse = batch_reference(batch)
        o_s, lse_s = batch_reference(batch, token_start=3)
        o_p, lse_p = prefix_reference(batch, 4)
        for b in range(batch.B):
            q, k, v = _torch_widened(batch, b)
            for got, (lo, hi) in (((o[b], lse[b]), (0, len(k))), ((o_s[b], lse_s[b]), (3, len(k))),
                                  ((o_p[b], lse_p[b]), (0, 4))):
                ro, rl = sdpa(q, k[lo:hi], v[lo:hi])
                assert np.allclose(got[0], ro, rtol=0, atol=1e-12), (kv, b, lo, hi)
                assert np.allclose(got[1], rl, rtol=0, atol=1e-12), (kv, b, lo, hi)


def test_batch_reference_matches_sdpa_on_torch_widened_inputs():
    from oracle import batch as ob
    check_batch_reference(ob.batch_reference, ob.prefix_reference)


def test_fp8_scale_applies_per_head():
    bits = np.array([[[0x38, 0x40], [0x38, 0x40]]], np.uint8)  # 1.0, 2.0 per head
    x = ov.stored_to_f64(bits, "fp8", np.array([0.5, 3.0], np.float32))
    assert np.array_equal(x, [[[0.5, 1.0], [3.0, 6.0]]])


# ------------------------------------------------------------- attention ---

def _rand(*shape):
    return RNG.standard_normal(shape)


def check_closed_forms(attn):
    # one token: softmax weight 1 -> o = V_0, lse = s_0
    q, k, v = _rand(8, 16), _rand(1, 2, 16), _rand(1, 2, 16)
    o, lse = attn(q, k, v, 0.25)
    for h in range(8):
        g = h // 4
        assert np.allclose(o[h], v[0, g], rtol=0, atol=1e-14)
        assert np.isclose(lse[h], 0.25 * q[h] @ k[0, g], rtol=0, atol=1e-13)
    # zero query: uniform weights -> mean of V, lse = ln L
    L = 37
    q0, k, v = np.zeros((4, 8)), _rand(L, 1, 8), _rand(L, 1, 8)
    o, lse = attn(q0, k, v, 1.0)
    assert np.allclose(o, v[:, 0].mean(0), atol=1e-14)
    assert np.allclose(lse, math.log(L), atol=1e-14)
    # two tokens: logistic weights
    q, k, v = _rand(2, 4), _rand(2, 2, 4), _rand(2, 2, 4)
    o, lse = attn(q, k, v, 0.5)
    for h in range(2):
        s0, s1 = 0.5 * q[h] @ k[0, h], 0.5 * q[h] @ k[1, h]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(o[h], w0 * v[0, h] + (1 - w0) * v[1, h], atol=1e-14)
        assert np.isclose(lse[h], math.log(math.exp(s0) + math.exp(s1)), atol=1e-13)
    # identical keys: uniform weights whatever the query
    k1 = np.repeat(_rand(1, 1, 8), 9, axis=0)
    v = _rand(9, 1, 8)
    o, lse = attn(_rand(2, 8), k1, v, 0.3)
    assert np.allclose(o, v[:, 0].mean(0), atol=1e-13)
    # empty: zeros and -inf
    o, lse = attn(_rand(4, 8), np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), 1.0)
    assert not o.any() and np.all(lse == -np.inf)


def test_attention_closed_forms():
    check_closed_forms(oa.decode_attention)


def check_against_sdpa(attn, cases=12):
    """torch's scaled_dot_product_attention on CPU in float64, K/V heads
    repeated so that query head h reads KV head h // G."""
    for _ in range(cases):
        H_kv = int(RNG.choice([1, 2, 4]))
        G = int(RNG.choice([1, 2, 4, 8]))
        d = int(RNG.choice([1, 4, 64, 128]))
        L = int(RNG.integers(1, 300))
        scale = float(RNG.uniform(0.05, 1.0))
        q, k, v = _rand(H_kv * G, d), _rand(L, H_kv, d), _rand(L, H_kv, d)
        o, lse = attn(q, k, v, scale)
        qt = torch.from_numpy(q)[None, :, None, :]                       # 1,H,1,d
        kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)[None]  # 1,H,L,d
        vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, :, 0]
        scores = (qt @ kt.transpose(-1, -2))[0, :, 0] * scale
        lse_ref = torch.logsumexp(scores, dim=-1)
        assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12), (H_kv, G, d, L)
        assert np.allclose(lse, lse_ref.numpy(), rtol=0, atol=1e-11), (H_kv, G, d, L)


def test_attention_matches_sdpa_fp64():
    check_against_sdpa(oa.decode_attention)


def _brute(q, k, v, scale):
    H_q, d = len(q), len(q[0])
    L, H_kv = len(k), len(k[0]) if len(k) else 1
    G = H_q // H_kv
    o, lse = [], []
    for h in range(H_q):
        g = h // G
        s = [scale * sum(q[h][i] * k[j][g][i] for i in range(d)) for j in range(L)]
        z = sum(math.exp(x) for x in s)
        o.append([sum(math.exp(s[j]) * v[j][g][i] for j in range(L)) / z for i in range(d)])
        lse.append(math.log(z))
    return o, lse


def check_against_bruteforce(attn):
    for _ in range(30):
        H_kv = int(RNG.integers(1, 3))
        G = int(RNG.integers(1, 4))
        d = int(RNG.integers(1, 5))
        L = int(RNG.integers(1, 9))
        q, k, v = _rand(H_kv * G, d), _rand(L, H_kv, d), _rand(L, H_kv, d)
        o, lse = attn(q, k, v, 0.7)
        ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7)
        assert np.allclose(o, ob, atol=1e-13) and np.allclose(lse, lb, atol=1e-13)


def test_attention_matches_bruteforce():
    check_against_bruteforce(oa.decode_attention)


# ----------------------------------------------------------------- merge ---

def check_split_invariance(merge, attn=oa.decode_attention):
    q, k, v = _rand(8, 16), _rand(23, 2, 16), _rand(23, 2, 16)
    o_full, lse_full = attn(q, k, v, 0.3)
    for c in range(0, 24):
        oa_, la = attn(q, k[:c], v[:c], 0.3)
        ob, lb = attn(q, k[c:], v[c:], 0.3)
        o, lse = merge(oa_, la, ob, lb)
        assert np.allclose(o, o_full, atol=1e-13), c
        assert np.allclose(lse, lse_full, atol=1e-13), c
        assert np.allclose(lse, np.logaddexp(la, lb), atol=1e-13)


def test_merge_split_at_every_point():
    check_split_invariance(oa.merge_states)


def test_merge_algebra():
    rows, d = 6, 5
    sa = (_rand(rows, d), _rand(rows))
    sb = (_rand(rows, d), _rand(rows))
    sc = (_rand(rows, d), _rand(rows))
    ab = oa.merge_states(*sa, *sb)
    ba = oa.merge_states(*sb, *sa)
    assert np.allclose(ab[0], ba[0], atol=1e-14) and np.allclose(ab[1], ba[1], atol=1e-14)
    left = oa.merge_states(*ab, *sc)
    right = oa.merge_states(*sa, *oa.merge_states(*sb, *sc))
    assert np.allclose(left[0], right[0], atol=1e-13) and np.allclose(left[1], right[1], atol=1e-13)
    empty = (np.zeros((rows, d)), np.full(rows, -np.inf))
    o, lse = oa.merge_states(*sa, *empty)
    assert np.array_equal(o, sa[0]) and np.array_equal(lse, sa[1])
    o, lse = oa.merge_states(*empty, *empty)
    assert not o.any() and np.all(lse == -np.inf) and not np.isnan(o).any()


def test_cascade_equals_full():
    q, kp, vp = _rand(32, 64), _rand(40, 8, 64), _rand(40, 8, 64)
    ks, vs = _rand(9, 8, 64), _rand(9, 8, 64)
    o, lse = oa.cascade_attention(q, kp, vp, ks, vs, 0.125)
    of, lf = oa.decode_attention(q, np.concatenate([kp, ks]), np.concatenate([vp, vs]), 0.125)
    assert np.allclose(o, of, atol=1e-13) and np.allclose(lse, lf, atol=1e-13)
    o2, l2 = oa.split_attention(q, np.concatenate([kp, ks]), np.concatenate([vp, vs]), 0.125, [3, 17, 40])
    assert np.allclose(o2, of, atol=1e-13) and np.allclose(l2, lf, atol=1e-13)


# -------------------------------------------------------------- lowering ---

def _random_table(rng, B, p, lmax, pool_extra=5):
    lens = rng.integers(0, lmax + 1, size=B)
    npages = [(int(L) + p - 1) // p for L in lens]
    pool = sum(npages) + pool_extra
    perm = rng.permutation(pool)
    indptr = np.concatenate([[0], np.cumsum(npages)])
    return lens, indptr, perm[: indptr[-1]], pool


def check_lowering(lower):
    rng = np.random.default_rng(3)
    for p in (1, 2, 3, 16, 128):
        lens, indptr, pages, pool = _random_table(rng, 7, p, 300)
        kv_indptr, kv_indices = lower(p, indptr, pages, lens)
        kv_indptr, kv_indices = np.asarray(kv_indptr), np.asarray(kv_indices)
        assert kv_indptr[-1] == lens.sum() and len(kv_indices) == lens.sum()
        # inverse gather: a pool holding each slot's own id, read through the
        # indices, returns the indices; and every slot sits in its page
        slot_ids = np.arange(pool * p)
        assert np.array_equal(slot_ids[kv_indices], kv_indices)
        for b in range(len(lens)):
            mine = kv_indices[kv_indptr[b]:kv_indptr[b + 1]]
            assert len(set(mine.tolist())) == len(mine)
            own = pages[indptr[b]:indptr[b + 1]]
            assert set((mine // p).tolist()) <= set(own.tolist())
            # logical order: token t is at offset t mod p of logical page t // p
            t = np.arange(len(mine))
            assert np.array_equal(mine % p, t % p)
            assert np.array_equal(mine // p, own[t // p])


def test_lowering_bruteforce_and_numpy_agree_and_hold_invariants():
    check_lowering(ol.lower_page_table_bruteforce)
    check_lowering(ol.lower_page_table)
    rng = np.random.default_rng(11)
    for p in (1, 16, 64):
        lens, indptr, pages, _ = _random_table(rng, 9, p, 200)
        a = ol.lower_page_table_bruteforce(p, indptr, pages, lens)
        b = ol.lower_page_table(p, indptr, pages, lens)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lowering_rejects_wrong_page_counts():
    with pytest.raises(ol.LoweringError):
        ol.lower_page_table(16, [0, 2], [3, 4], [16])      # trailing empty page
    with pytest.raises(ol.LoweringError):
        ol.lower_page_table(16, [0, 1], [3], [17])         # one page short
    with pytest.raises(ol.LoweringError):
        ol.lower_page_table(0, [0, 0], [], [0])


def test_index_length_is_batch_times_context(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "index_length.json")))
    B, L = g["batch"], g["context_tokens"]
    for p in g["page_sizes"]:
        n = (L + p - 1) // p
        indptr = np.arange(B + 1) * n
        pages = np.random.default_rng(p).permutation(B * n)
        kv_indptr, kv_indices = ol.lower_page_table(p, indptr, pages, [L] * B)
        assert len(kv_indices) == g["index_length"] and kv_indptr[-1] == g["index_length"]


def test_block_aligned_prefix_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "prefix_block_alignment.json")))
    assert ol.shared_prefix_pages(g["prefix_tokens"], g["block_size"]) == (g["shared_blocks"], g["unshared_tokens"])


def test_worst_case_internal_waste_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "block_internal_waste.json")))
    p = g["block_size"]
    waste = [((L + p - 1) // p) * p - L for L in range(1, 10 * p)]
    assert max(waste) == g["worst_case_unused_slots"]


# --------------------------------------------------------------- planner ---

TUNE = dict(t_dense=1024, gate_ratio=1, launch_bytes=0)


def _plan(B, G, P, p=16, H_kv=8, d=128, L=None, **kw):
    args = dict(B=B, H_q=H_kv * G, H_kv=H_kv, d=d, q_dtype="bf16", kv_dtype="bf16",
                page_size=p, seq_lens=[L if L is not None else P + 100] * B,
                shared_prefix_len=P, force_path=-1, **TUNE)
    args.update(kw)
    return op.plan(**args)


def check_cached_gate(plan_fn):
    """Pins of the cached-prefix allowance, worked out by hand."""
    def pl(B, G, P, p=16, H_kv=8, d=128, L=None, **kw):
        args = dict(B=B, H_q=H_kv * G, H_kv=H_kv, d=d, q_dtype="bf16", kv_dtype="bf16",
                    page_size=p, seq_lens=[L if L is not None else P + 100] * B,
                    shared_prefix_len=P, force_path=-1, **TUNE)
        args.update(kw)
        return plan_fn(**args)

    # the cached-prefix allowance (constants as the gfx950 defaults: R = 3,
    # launch term 5,000,000 B, prefixes of at most 2 MiB stored re-read from
    # L2 below 128 MiB of saved reads), values worked out by hand:
    cached = dict(t_dense=1, gate_ratio=3, launch_bytes=5_000_000, cached_prefix_bytes=2 << 20,
                  cached_reread_bytes=128 << 20)
    # 64 requests, G = 1, P = 256 bf16: stores 256*8*128*2*2 = 1,048,576 B;
    # saves 63*256*8*128*4 = 66,060,288 B against 3*(4*512*129*4 + 5e6) =
    # 18,170,304 -> DENSE by the byte rule, PAGED with the allowance
    assert pl(64, 1, 256, **cached)["path"] == "PAGED"
    assert pl(64, 1, 256, **dict(cached, cached_prefix_bytes=0))["path"] == "DENSE"
    assert pl(64, 1, 256, **dict(cached, cached_prefix_bytes=(1 << 20) - 1))["path"] == "DENSE"
    # 256 requests: saves 267,386,880 B, above the allowance -> DENSE
    assert pl(256, 1, 256, **cached)["path"] == "DENSE"
    # 16 requests over 1,024 tokens: fp8 stores exactly 2 MiB (PAGED: saves
    # 62,914,560 B, counted at 2 bytes a value), bf16 stores 4 MiB (the byte
    # rule: 62,914,560 >= 3*(4*128*129*4 + 5e6) = 15,792,384 -> DENSE)
    assert pl(16, 1, 1024, kv_dtype="fp8", **cached)["path"] == "PAGED"
    assert pl(16, 1, 1024, kv_dtype="bf16", **cached)["path"] == "DENSE"
    # gate_ratio 0 turns the whole gate off, the allowance included
    assert pl(64, 1, 256, **dict(cached, gate_ratio=0))["path"] == "DENSE"
    # ... and a step whose DENSE form would fuse keeps the byte rule: 32
    # requests, G = 4, P = 512 (2 MiB stored), 8 own tokens each: saves
    # 31*512*8*128*4 = 65,011,712 B (under the allowance, over 3*(4*1024*129*4
    # + 5e6) = 21,340,608); prefix flops 4*128*512*128*8 = 268,435,456 >= 12 *
    # 256*8*128*4 = 12,582,912 -> fuses -> DENSE; 2,000 own tokens each
    # (suffix 262,144,000 B) or fuse_cascade = 0 -> PAGED
    fused = dict(cached, fuse_cascade=12)
    assert pl(32, 4, 512, L=520, **fused)["path"] == "DENSE"
    assert pl(32, 4, 512, L=2512, **fused)["path"] == "PAGED"
    assert pl(32, 4, 512, L=520, **dict(fused, fuse_cascade=0))["path"] == "PAGED"


def test_planner_cached_prefix_allowance():
    check_cached_gate(op.plan)


# Plausible mistakes in the allowance, each emulated through the oracle's
# own arguments: the stored bytes counted at the gate's 2 bytes per fp8
# value, a strict bound, and the fused-step guard left out.
def _mut_cached_rule_bytes(**kw):
    kw = dict(kw)
    if kw.get("kv_dtype") == "fp8":
        kw["cached_prefix_bytes"] = kw.get("cached_prefix_bytes", 0) // 2
    return op.plan(**kw)


def _mut_cached_strict(**kw):
    kw = dict(kw)
    kw["cached_prefix_bytes"] = max(0, kw.get("cached_prefix_bytes", 0) - 1)
    return op.plan(**kw)


def _mut_cached_no_fuse_guard(**kw):
    kw = dict(kw)
    kw["fuse_cascade"] = 0
    return op.plan(**kw)


@pytest.mark.parametrize("mutant", [_mut_cached_rule_bytes, _mut_cached_strict, _mut_cached_no_fuse_guard])
def test_mutant_cached_allowance_caught(mutant):
    with pytest.raises(AssertionError):
        check_cached_gate(mutant)


def test_dispatcher_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "dispatcher.json")))
    for c in g["cases"]:
        r = _plan(c["batch"], c["group"], 4096, t_dense=g["a100_threshold"])
        assert r["m_eff"] == c["m_eff"] and r["path"] == c["path"], c


def test_planner_gate_and_alignment():
    assert _plan(256, 4, 4096)["path"] == "DENSE"                   # c3 shape
    assert _plan(512, 4, 512)["path"] == "DENSE"                    # c4 shape
    r = _plan(256, 4, 2003)
    assert r["shared_pages"] == 125 and r["prefix_tokens"] == 2000
    assert _plan(1, 4, 4096)["path"] == "PAGED"                      # nothing to share
    r = _plan(256, 4, 15)
    assert r["path"] == "PAGED" and r["shared_pages"] == 0          # no whole page
    assert _plan(256, 4, 0)["path"] == "PAGED"
    # the gate: a huge launch cost keeps short prefixes on the paged path
    # B=4, P=16: saves 3*16*8*128*4 = 196,608 B of prefix reads but adds
    # 16*128*129 = 264,192 B of partial-state traffic -> stays paged
    assert _plan(4, 4, 16, launch_bytes=0)["path"] == "PAGED"
    assert _plan(4, 4, 256, launch_bytes=0)["path"] == "CASCADE"
    assert _plan(4, 4, 256, launch_bytes=10**12)["path"] == "PAGED"
    # fp8 K/V: a prefix kernel at d = 128; none at d = 64, where forcing a
    # prefix path is refused
    assert _plan(256, 4, 4096, kv_dtype="fp8")["path"] == "DENSE"     # M_eff = 1024 at the A100 threshold
    assert _plan(256, 4, 4096, d=64, kv_dtype="fp8")["path"] == "PAGED"
    with pytest.raises(op.PlanError) as e:
        _plan(256, 4, 4096, d=64, kv_dtype="fp8", force_path=2)
    assert e.value.code == "EUNSUPPORTED"
    # the gate counts an fp8 value at bf16's 2 bytes: 3 requests on 64 pages
    # save 8.4 MB either way, against a 5.2 MB overhead (launch term 5 MB,
    # R = 1) and not against a 9.2 MB one
    for kv in ("bf16", "fp8"):
        assert _plan(3, 4, 1024, launch_bytes=5 * 10**6, kv_dtype=kv)["path"] == "CASCADE"
        assert _plan(3, 4, 1024, launch_bytes=9 * 10**6, kv_dtype=kv)["path"] == "PAGED"
    with pytest.raises(op.PlanError) as e:
        _plan(256, 4, 8, force_path=1)
    assert e.value.code == "EINVAL"
    r = _plan(256, 4, 4096, force_path=0)
    assert r["path"] == "PAGED" and r["prefix_tokens"] == 0 and r["shared_pages"] == 256


def check_prefix_placement(plan_fn):
    """Prefix placement: a prefix whose slots are one ascending run is read
    from its first slot; any break in the run, a PAGED plan, placement
    switched off or no slots shown give -1; only the prefix pass's whole
    pages matter (the tail of a 2,003-token prefix is not part of the run)."""
    def run(slots, P=64, B=8, **kw):
        return plan_fn(B=B, H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="bf16", page_size=16,
                       seq_lens=[P + 50] * B, shared_prefix_len=P, force_path=kw.pop("force_path", 2),
                       prefix_slots=slots, **TUNE, **kw)["prefix_base"]
    assert run(list(range(40, 104))) == 40
    assert run(list(range(0, 64))) == 0
    broken = list(range(40, 104))
    broken[63] = 7
    assert run(broken) == -1
    broken = list(range(40, 104))
    broken[1] = 40
    assert run(broken) == -1
    assert run(list(range(100, 36, -1))) == -1                    # descending is not a run
    assert run(list(range(40, 104)), force_path=0) == -1           # PAGED reads no prefix
    assert run(list(range(40, 104)), prefix_placement=0) == -1
    assert run(None) == -1
    tail = list(range(500, 2500)) + [9, 8, 7]                       # 125 whole pages + 3 tail tokens
    assert run(tail, P=2003) == 500


def test_prefix_placement_rule():
    check_prefix_placement(op.plan)


def test_planner_rejects():
    for kw, code in [(dict(H_q=30), "EINVAL"), (dict(d=96), "EUNSUPPORTED"),
                     (dict(q_dtype="f32"), "EUNSUPPORTED"), (dict(force_path=3), "EINVAL"),
                     (dict(L=10), "EINVAL")]:
        with pytest.raises(op.PlanError) as e:
            _plan(8, 4, 64, **kw)
        assert e.value.code == code, kw
    with pytest.raises(op.PlanError) as e:
        _plan(8, 16, 64, H_kv=2)                     # G = 16 not built
    assert e.value.code == "EUNSUPPORTED"


# ------------------------------------------------ planted mistakes (CPU) ---
# Each mutant is a copy of an oracle routine with one plausible mistake.  The
# pins above must reject every one of them.

def _mut_head_map(q, k, v, s):          # h % H_kv instead of h // G
    H_q, d = q.shape
    L, H_kv, _ = k.shape
    o, lse = np.zeros((H_q, d)), np.full(H_q, -np.inf)
    for h in range(H_q):
        g = h % H_kv
        sc = s * (k[:, g] @ q[h]); m = sc.max(); e = np.exp(sc - m)
        o[h] = e @ v[:, g] / e.sum(); lse[h] = m + np.log(e.sum())
    return o, lse


def _mut_lse_unscaled(q, k, v, s):      # lse of the raw dot products
    o, lse = oa.decode_attention(q, k, v, s)
    if k.shape[0]:
        o2, l2 = oa.decode_attention(q, k, v, 1.0)
        lse = l2
    return o, lse


def _mut_no_normalise(q, k, v, s):      # forgets the division by l
    o, lse = oa.decode_attention(q, k, v, s)
    if k.shape[0]:
        H_q = q.shape[0]
        G = H_q // k.shape[1]
        for h in range(H_q):
            sc = s * (k[:, h // G] @ q[h])
            o[h] *= np.exp(sc - sc.max()).sum()
    return o, lse


def _mut_transposed_pv(q, k, v, s):     # uses K where V belongs
    return oa.decode_attention(q, k, k, s)


def _mut_merge_swapped(o_a, lse_a, o_b, lse_b):   # weights crossed over
    M = np.maximum(lse_a, lse_b)
    wa, wb = np.exp(lse_a - M)[:, None], np.exp(lse_b - M)[:, None]
    return (wb * o_a + wa * o_b) / (wa + wb), M + np.log(wa + wb)[:, 0]


def _mut_merge_no_max(o_a, lse_a, o_b, lse_b):    # drops lse_b's weight term
    o, lse = oa.merge_states(o_a, lse_a, o_b, lse_b)
    return o, np.maximum(lse_a, lse_b)


def _mut_fp8_bias8(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return float("nan")
    sign = -1.0 if s else 1.0
    return sign * ((m / 8) * 2.0 ** -7 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8))


def _mut_lower_swapped(p, indptr, pages, lens):   # offset and page swapped
    kv_indptr, kv = [0], []
    for b in range(len(lens)):
        for t in range(int(lens[b])):
            kv.append(int(pages[int(indptr[b]) + t % p]) * p + t // p if t % p < indptr[b + 1] - indptr[b] else 0)
        kv_indptr.append(len(kv))
    return kv_indptr, kv


def _mut_lower_offbyone(p, indptr, pages, lens):  # skips page 0's first slot
    kv_indptr, kv = ol.lower_page_table(p, indptr, pages, lens)
    return kv_indptr, kv + (kv % p == 0)


@pytest.mark.parametrize("mutant", [_mut_head_map, _mut_transposed_pv])
def test_mutant_attention_caught_by_sdpa(mutant):
    with pytest.raises(AssertionError):
        check_against_sdpa(mutant, cases=8)


@pytest.mark.parametrize("mutant", [_mut_lse_unscaled, _mut_no_normalise, _mut_transposed_pv])
def test_mutant_attention_caught_by_closed_forms(mutant):
    with pytest.raises(AssertionError):
        check_closed_forms(mutant)


@pytest.mark.parametrize("mutant", [_mut_merge_swapped, _mut_merge_no_max])
def test_mutant_merge_caught(mutant):
    with pytest.raises(AssertionError):
        check_split_invariance(mutant)


def test_mutant_fp8_caught():
    with pytest.raises(AssertionError):
        check_fp8_table(_mut_fp8_bias8)


def _mut_f32_astype(bits):              # converts the integers instead of viewing the bits
    return np.asarray(bits).astype(np.float64)


def _mut_scale_over_d(d):               # 1/d instead of 1/sqrt(d)
    return 1.0 / d


def _mut_request_inputs_swapped(batch, b, token_range=None):   # V widened with the K scales
    from oracle import batch as ob
    q, k, v = ob.request_inputs(batch, b, token_range)
    if batch.kv_dtype == "fp8":
        k = k / np.asarray(batch.k_scale, np.float64)[None, :, None] * np.asarray(batch.v_scale, np.float64)[None, :, None]
        v = v / np.asarray(batch.v_scale, np.float64)[None, :, None] * np.asarray(batch.k_scale, np.float64)[None, :, None]
    return q, k, v


def _mut_request_inputs_range(batch, b, token_range=None):     # token range one late
    from oracle import batch as ob
    if token_range is not None:
        token_range = (token_range[0] + 1, token_range[1] + 1)
    return ob.request_inputs(batch, b, token_range)


def _mut_batch_reference_scale(batch, sm_scale=None, requests=None, token_start=0):   # scale 1/d
    from oracle import batch as ob
    return ob.batch_reference(batch, 1.0 / batch.d if sm_scale is None else sm_scale, requests, token_start)


def _mut_prefix_reference_short(batch, prefix_tokens, sm_scale=None, requests=None):  # drops the last prefix token
    from oracle import batch as ob
    return ob.prefix_reference(batch, prefix_tokens - 1, sm_scale, requests)


def test_mutant_f32_widening_caught():
    with pytest.raises(AssertionError):
        check_f32_widening(_mut_f32_astype)


def test_mutant_default_scale_caught():
    with pytest.raises(AssertionError):
        check_default_scale(_mut_scale_over_d)


@pytest.mark.parametrize("mutant", [_mut_request_inputs_swapped, _mut_request_inputs_range])
def test_mutant_request_inputs_caught(mutant):
    with pytest.raises(AssertionError):
        check_request_inputs(mutant)


@pytest.mark.parametrize("mutants", [("scale", _mut_batch_reference_scale, None),
                                     ("prefix", None, _mut_prefix_reference_short)])
def test_mutant_batch_reference_caught(mutants):
    from oracle import batch as ob
    _, br, pr = mutants
    with pytest.raises(AssertionError):
        check_batch_reference(br or ob.batch_reference, pr or ob.prefix_reference)


def _mut_placement_first_only(**kw):    # takes the first slot without checking the run
    out = op.plan(**kw)
    if out["path"] != "PAGED" and kw.get("prefix_slots") is not None and kw.get("prefix_placement", 1):
        out["prefix_base"] = int(kw["prefix_slots"][0])
    return out


def _mut_placement_ignores_switch(**kw):  # ignores prefix_placement = 0
    kw = dict(kw)
    kw["prefix_placement"] = 1
    return op.plan(**kw)


@pytest.mark.parametrize("mutant", [_mut_placement_first_only, _mut_placement_ignores_switch])
def test_mutant_prefix_placement_caught(mutant):
    with pytest.raises(AssertionError):
        check_prefix_placement(mutant)


@pytest.mark.parametrize("mutant", [_mut_lower_swapped, _mut_lower_offbyone])
def test_mutant_lowering_caught(mutant):
    with pytest.raises((AssertionError, IndexError)):
        check_lowering(mutant)


# ---------------------------------------------------------- prefix groups ---

from oracle import groups as og  # noqa: E402


from workloads.groups import random_group_tables as _random_group_tables  # noqa: E402
from workloads.groups import tables_from_blocks  # noqa: E402
from workloads.groups import token_blocks as _token_blocks  # noqa: E402


def golden_group_case(c, p):
    if "requests" in c:
        reqs = c["requests"]
        lens = [p * len(r) for r in reqs]
        return reqs, lens
    P = c["prefix_tokens"]
    reqs, lens = [], []
    for b, n in enumerate(c["own_tokens"]):
        toks = ["P"] * P + [f"own{b}"] * n
        reqs.append(_token_blocks(toks, p))
        lens.append(len(toks))
    return reqs, lens


def check_group_golden(detect, golden_dir):
    g = json.load(open(os.path.join(golden_dir, "prefix_groups.json")))
    p = g["block_size"]
    for c in g["cases"]:
        reqs, lens = golden_group_case(c, p)
        for seed in (0, 1):
            ptr, pages = tables_from_blocks(reqs, p, seed)
            got = [{"members": g["members"], "shared_pages": g["shared_pages"]} for g in detect(p, ptr, pages, lens)]
            want = [{"members": x["members"], "shared_pages": x["shared_blocks"]} for x in c["groups"]]
            assert got == want, (c["name"], got)


def test_prefix_groups_golden(golden_dir):
    check_group_golden(og.detect_prefix_groups, golden_dir)


def _groups_bruteforce(p, ptr, pages, lens):
    """The tree from its definition by prefixes: for every request b and
    page count k, the set of requests whose first k whole pages are b's;
    each distinct such set with two or more members is a group, its run
    ending at the largest k that gives the set and starting at the largest k
    that gives a strictly larger set (0 if none).  Returned as a set of
    (members, start, end, parent members)."""
    B = len(lens)
    tab = [list(pages[ptr[b]:ptr[b + 1]]) for b in range(B)]
    full = [lens[b] // p for b in range(B)]
    sets = {}
    for b in range(B):
        for k in range(1, full[b] + 1):
            S = tuple(c for c in range(B) if full[c] >= k and tab[c][:k] == tab[b][:k])
            if len(S) >= 2:
                lo, hi = sets.get(S, (k, k))
                sets[S] = (min(lo, k), max(hi, k))
    out = set()
    for S, (lo, hi) in sets.items():
        parents = [T for T in sets if set(S) < set(T)]
        parent = min(parents, key=len) if parents else None
        out.add((S, lo - 1, hi, parent))
    return out


def _as_tree(groups):
    return {(tuple(g["members"]), g["start_pages"], g["shared_pages"],
             tuple(groups[g["parent"]]["members"]) if g["parent"] >= 0 else None) for g in groups}


def test_prefix_groups_match_bruteforce():
    check_groups_bruteforce(og.detect_prefix_groups)
    # the random tables do exercise groups, including ones whose members
    # share runs of different lengths
    rng = np.random.default_rng(7)
    n_groups = 0
    for it in range(400):
        p = int(rng.choice([1, 2, 4, 16]))
        reqs, lens = _random_group_tables(rng, p)
        ptr, pages = tables_from_blocks(reqs, p, it)
        n_groups += len(og.detect_prefix_groups(p, ptr, pages, lens))
    assert n_groups > 100


def test_plan_groups_is_the_single_prefix_rule_per_group():
    # Two groups of 200 and 2 requests on 4096-token prompts, one loner:
    # the large group passes the gate, the small one does not (A100 constants).
    p = 16
    reqs = [["A%d" % j for j in range(256)] + ["a%d" % b] for b in range(200)]
    reqs += [["B%d" % j for j in range(256)] + ["b%d" % b] for b in range(2)]
    reqs += [["C"]]
    lens = [p * len(r) for r in reqs]
    ptr, pages = tables_from_blocks(reqs, p)
    tune = dict(t_dense=1024, gate_ratio=3, launch_bytes=10_000_000)
    kept, path_of = og.plan_groups(H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="bf16", page_size=p,
                                   page_indptr=ptr, page_indices=pages, seq_lens=lens, force_path=-1, **tune)
    one = op.plan(B=200, H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="bf16", page_size=p,
                  seq_lens=lens[:200], shared_prefix_len=4096, force_path=-1, **tune)
    assert len(kept) == 1 and kept[0]["members"] == list(range(200))
    assert kept[0]["path"] == one["path"] == "CASCADE" and kept[0]["m_eff"] == 800
    assert kept[0]["prefix_tokens"] == 4096 and path_of[:200] == [[0]] * 200 and path_of[200:] == [[]] * 3
    # forced: every group takes the forced prefix path, the loner stays alone
    kept, _ = og.plan_groups(H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="bf16", page_size=p,
                             page_indptr=ptr, page_indices=pages, seq_lens=lens, force_path=2, **tune)
    assert [g["path"] for g in kept] == ["DENSE", "DENSE"] and [len(g["members"]) for g in kept] == [200, 2]
    # fp8 K/V at d = 64 has no prefix kernel: nothing is kept unless forced,
    # which is refused; at d = 128 the group is kept (half the bytes saved)
    kept, _ = og.plan_groups(H_q=32, H_kv=8, d=64, q_dtype="bf16", kv_dtype="fp8", page_size=p,
                             page_indptr=ptr, page_indices=pages, seq_lens=lens, force_path=-1, **tune)
    assert kept == []
    with pytest.raises(op.PlanError):
        og.plan_groups(H_q=32, H_kv=8, d=64, q_dtype="bf16", kv_dtype="fp8", page_size=p, page_indptr=ptr,
                       page_indices=pages, seq_lens=lens, force_path=1, **tune)
    kept, _ = og.plan_groups(H_q=32, H_kv=8, d=128, q_dtype="bf16", kv_dtype="fp8", page_size=p,
                             page_indptr=ptr, page_indices=pages, seq_lens=lens, force_path=-1, **tune)
    assert [len(g["members"]) for g in kept] == [200]


def test_lower_groups_partitions_every_request():
    rng = np.random.default_rng(11)
    n_nested = 0
    for it in range(200):
        p = int(rng.choice([1, 4, 16]))
        reqs, lens = _random_group_tables(rng, p)
        ptr, pages = tables_from_blocks(reqs, p, it)
        kept, path_of = og.plan_groups(H_q=8, H_kv=2, d=64, q_dtype="bf16", kv_dtype="bf16", page_size=p,
                                       page_indptr=ptr, page_indices=pages, seq_lens=lens,
                                       force_path=int(rng.choice([-1, 1, 2])), t_dense=8, gate_ratio=0,
                                       launch_bytes=0)
        suf_ptr, suf, pre_ptr, pre = og.lower_groups(p, ptr, pages, lens, kept, path_of)
        kv_ptr, kv = ol.lower_page_table(p, ptr, pages, lens)
        for b in range(len(lens)):
            full = list(kv[kv_ptr[b]:kv_ptr[b + 1]])
            covered = np.zeros(len(full), bool)
            for gi in path_of[b]:
                g = kept[gi]
                assert b in g["members"]
                run = list(pre[pre_ptr[gi]:pre_ptr[gi + 1]])
                lo = g["start_tokens"]
                assert len(run) % p == 0 and len(run) > 0 and lo % p == 0
                assert run == full[lo:lo + len(run)]          # the run is b's tokens there
                assert not covered[lo:lo + len(run)].any()    # runs on a path do not overlap
                covered[lo:lo + len(run)] = True
            assert list(suf[suf_ptr[b]:suf_ptr[b + 1]]) == [x for x, c in zip(full, covered) if not c]
            n_nested += len(path_of[b]) > 1
    assert n_nested > 0


def _mut_groups_max_run(p, ptr, pages, lens):
    """Takes the longest run any member shares with the first member instead
    of the run all members share."""
    out = og.detect_prefix_groups(p, ptr, pages, lens)
    B = len(lens)
    tab = [list(pages[ptr[b]:ptr[b + 1]]) for b in range(B)]
    for g in out:
        m0, best = g["members"][0], 0
        for c in g["members"][1:]:
            k = 0
            while k < min(lens[m0], lens[c]) // p and tab[c][k] == tab[m0][k]:
                k += 1
            best = max(best, k)
        g["shared_pages"] = best
    return out


def _mut_groups_partial_page(p, ptr, pages, lens):
    """Counts a partly filled last page as shareable."""
    return og.detect_prefix_groups(p, ptr, pages, [((x + p - 1) // p) * p for x in lens])


def _mut_groups_pairwise_first(p, ptr, pages, lens):
    """Shared run measured against the first member only, with the wrong
    member: the last one's full-page count is ignored."""
    out = og.detect_prefix_groups(p, ptr, pages, lens)
    for g in out:
        g["shared_pages"] = min(lens[g["members"][0]] // p, g["shared_pages"] + 1)
    return out


def check_groups_bruteforce(detect, n=400):
    rng = np.random.default_rng(7)
    for it in range(n):
        p = int(rng.choice([1, 2, 4, 16]))
        reqs, lens = _random_group_tables(rng, p)
        ptr, pages = tables_from_blocks(reqs, p, it)
        assert _as_tree(detect(p, ptr, pages, lens)) == _groups_bruteforce(p, ptr, pages, lens)


def check_group_placement(plan_groups):
    """Each kept group's prefix_base against the lowered token-level slots of
    its first member: the run's slots must be first, first + 1, ... for a
    base to be set, and then base = first (tables with pages handed out in
    order, where many runs are contiguous, and scrambled ones)."""
    rng = np.random.default_rng(11)
    n_set = n_unset = 0
    for it in range(200):
        p = int(rng.choice([1, 2, 4, 16]))
        reqs, lens = _random_group_tables(rng, p, max_batch=10)
        ptr, pages = tables_from_blocks(reqs, p, it, scramble=bool(it % 2))
        for placement in (1, 0):
            kept, _ = plan_groups(H_q=8, H_kv=2, d=64, q_dtype="bf16", kv_dtype="bf16", page_size=p,
                                  page_indptr=ptr, page_indices=pages, seq_lens=lens, force_path=-1,
                                  t_dense=4, gate_ratio=0, launch_bytes=0, prefix_placement=placement)
            kv_indptr, kv = ol.lower_page_table(p, ptr, pages, lens)
            for g in kept:
                lo = int(kv_indptr[g["members"][0]]) + g["start_tokens"]
                slots = [int(x) for x in kv[lo:lo + g["prefix_tokens"]]]
                is_run = slots == list(range(slots[0], slots[0] + len(slots)))
                want = slots[0] if (placement and is_run) else -1
                assert g["prefix_base"] == want, (it, g, slots[:4])
                n_set += want >= 0
                n_unset += want < 0
    assert n_set > 50 and n_unset > 50


def test_group_placement_matches_token_level_slots():
    check_group_placement(og.plan_groups)


def _mut_groups_placement_next_page(**kw):   # base from the page after the run's first
    kept, path_of = og.plan_groups(**kw)
    p = kw["page_size"]
    for g in kept:
        if g["prefix_base"] >= 0:
            g["prefix_base"] += p
    return kept, path_of


def test_mutant_group_placement_caught():
    with pytest.raises(AssertionError):
        check_group_placement(_mut_groups_placement_next_page)


@pytest.mark.parametrize("mutant", [_mut_groups_max_run, _mut_groups_partial_page, _mut_groups_pairwise_first])
def test_mutant_groups_caught(mutant, golden_dir):
    caught = 0
    for check in (lambda: check_group_golden(mutant, golden_dir), lambda: check_groups_bruteforce(mutant)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1
