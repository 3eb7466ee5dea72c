"""Decode attention, LSE merge and the cascade split (test oracle, float64).

Decode attention ("The 25% Page-Size Slowdown That Wasn't", section "Four
meanings of page size"; "Track C · Document 10", PagedAttention Q&A): each
request has one new query token whose heads attend over every cached K/V
token of that request.  Paging only changes where the cached rows live, so
the result is the ordinary softmax attention over the request's tokens taken
in logical order, written out here directly.

Grouped-query attention ("GraniKV", section 3: M_eff counts queries per KV
head): with G = H_q / H_kv, query head h reads KV head floor(h / G).  The
pages do not fix the head map; consecutive query heads sharing a KV head is
the reading taken.

For one request with L tokens, query head h, KV head g = h // G and scale
sigma:

    s_j   = sigma * <q_h, K_j,g>
    m     = max_j s_j
    l     = sum_j exp(s_j - m)
    o_h   = sum_j exp(s_j - m) * V_j,g / l
    lse_h = m + ln l                       (natural log, sigma included)

An empty token set gives o = 0 and lse = -inf.

Merge of two partial states over disjoint token sets A and B (not on the
pages; it follows from the definition above, and is what lets a shared prefix
be read once and combined with each request's own suffix, "GraniKV" sections
2-3):

    M = max(lse_a, lse_b)
    w_a = exp(lse_a - M),  w_b = exp(lse_b - M)
    o   = (w_a o_a + w_b o_b) / (w_a + w_b)
    lse = M + ln(w_a + w_b)

with (0, -inf) when both sides are empty.
"""
import numpy as np


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """One request.  q: [H_q, d]; k, v: [L, H_kv, d] (float64).

    Returns (o [H_q, d], lse [H_q]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    H_q, d = q.shape
    L, H_kv, _ = k.shape
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    o = np.zeros((H_q, d), np.float64)
    lse = np.full(H_q, -np.inf, np.float64)
    if L == 0:
        return o, lse
    for h in range(H_q):
        g = h // G
        s = sm_scale * (k[:, g, :] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[h] = (e @ v[:, g, :]) / l
        lse[h] = m + np.log(l)
    return o, lse


def merge_states(o_a, lse_a, o_b, lse_b):
    """Combine two partial states row by row.  o: [rows, d]; lse: [rows]."""
    o_a = np.asarray(o_a, np.float64)
    o_b = np.asarray(o_b, np.float64)
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    rows = lse_a.shape[0]
    o = np.zeros_like(o_a)
    lse = np.full(rows, -np.inf)
    for r in range(rows):
        M = max(lse_a[r], lse_b[r])
        if M == -np.inf:
            continue
        wa = np.exp(lse_a[r] - M)
        wb = np.exp(lse_b[r] - M)
        o[r] = (wa * o_a[r] + wb * o_b[r]) / (wa + wb)
        lse[r] = M + np.log(wa + wb)
    return o, lse


def split_attention(q, k, v, sm_scale, cuts):
    """Attention computed over consecutive token ranges and merged left to right.

    ``cuts`` are split points 0 < c_1 < ... < L; used to check that splitting
    the token axis and merging returns the full result.
    """
    L = k.shape[0]
    edges = [0] + list(cuts) + [L]
    o, lse = decode_attention(q, k[0:0], v[0:0], sm_scale)
    for a, b in zip(edges[:-1], edges[1:]):
        o2, lse2 = decode_attention(q, k[a:b], v[a:b], sm_scale)
        o, lse = merge_states(o, lse, o2, lse2)
    return o, lse


def cascade_attention(q, k_prefix, v_prefix, k_suffix, v_suffix, sm_scale):
    """Prefix read once, suffix per request, merged: equals attention over
    prefix ++ suffix."""
    o_p, lse_p = decode_attention(q, k_prefix, v_prefix, sm_scale)
    o_s, lse_s = decode_attention(q, k_suffix, v_suffix, sm_scale)
    return merge_states(o_p, lse_p, o_s, lse_s)
