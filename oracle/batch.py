"""Run the oracle over a synthetic decode batch (test oracle).

Works from the batch's logical token values (stored bits, widened exactly to
float64) and never reads the paged pool or any index list.
"""
import math

import numpy as np

from .attention import decode_attention
from .values import stored_to_f64


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d)."""
    return 1.0 / math.sqrt(d)


def _q64(batch, b):
    return stored_to_f64(batch.bits(batch.q[b], batch.q_dtype), batch.q_dtype)


def _kv64(batch, t, which):
    scale = None
    if batch.kv_dtype == "fp8":
        scale = batch.k_scale if which == "k" else batch.v_scale
    return stored_to_f64(batch.bits(t, batch.kv_dtype), batch.kv_dtype, scale)


def request_inputs(batch, b, token_range=None):
    """Request ``b``'s query and contiguous K, V over its logical tokens
    ``token_range = (lo, hi)`` (default: all of them), stored values widened
    exactly to float64: (q [H_q, d], k [L, H_kv, d], v [L, H_kv, d])."""
    k, v = batch.logical_kv(b)
    if token_range is not None:
        lo, hi = token_range
        k, v = k[lo:hi], v[lo:hi]
    return _q64(batch, b), _kv64(batch, k, "k"), _kv64(batch, v, "v")


def request_reference(batch, b, sm_scale=None, token_range=None):
    """(o [H_q, d], lse [H_q]) of request ``b`` over its logical tokens
    ``token_range = (lo, hi)`` (default: all of them)."""
    sm_scale = default_scale(batch.d) if sm_scale is None else sm_scale
    return decode_attention(*request_inputs(batch, b, token_range), sm_scale)


def batch_reference(batch, sm_scale=None, requests=None, token_start=0):
    """Oracle output for the chosen requests (default: all).

    ``token_start`` skips each request's first tokens (the suffix of a
    cascade).  Returns (o [n, H_q, d], lse [n, H_q]) in float64.
    """
    reqs = range(batch.B) if requests is None else list(requests)
    o = np.zeros((len(reqs), batch.H_q, batch.d))
    lse = np.zeros((len(reqs), batch.H_q))
    for i, b in enumerate(reqs):
        rng = (token_start, int(batch.seq_lens[b])) if token_start else None
        o[i], lse[i] = request_reference(batch, b, sm_scale, rng)
    return o, lse


def prefix_reference(batch, prefix_tokens, sm_scale=None, requests=None):
    """Every request's queries over the first ``prefix_tokens`` tokens."""
    reqs = range(batch.B) if requests is None else list(requests)
    o = np.zeros((len(reqs), batch.H_q, batch.d))
    lse = np.zeros((len(reqs), batch.H_q))
    for i, b in enumerate(reqs):
        o[i], lse[i] = request_reference(batch, b, sm_scale, (0, prefix_tokens))
    return o, lse
