"""Test oracle for batched paged decode attention (TEST INFRASTRUCTURE ONLY).

A plain, slow, CPU-only float64 statement of what the GPU library computes,
written from the pages' description of the method and from the definition of
softmax attention.  It is used only by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``; the
library itself never imports, links or calls it, and the two share no code.

Contents and what each part follows:

* ``values``    -- widening of stored bf16 / fp8-e4m3 / fp32 values to float64
                   (fp8 KV cache: "Track C · Document 10 · Shrinking the
                   footprint", section on the fp8 cache).
* ``attention`` -- decode attention over one request's contiguous K/V, the LSE
                   merge of two partial softmax states, and the cascade
                   (prefix ++ suffix) check.  The pages state that paging leaves
                   the attention result unchanged ("Track C · Document 10",
                   PagedAttention Q&A), so the oracle is the plain definition
                   over contiguous K/V and never sees pages.
* ``lowering``  -- page table -> token-flat ``kv_indices``
                   ("The 25% Page-Size Slowdown That Wasn't", section "Four
                   meanings of page size" and "When source beats intuition").
* ``planner``   -- the per-step dispatcher on M_eff = realized batch x GQA
                   group ("GraniKV: asymmetric KV cache paging for
                   shared-prefix agents", section 3 "Per-step dispatcher").
* ``groups``    -- several shared prefixes in one step: groups of requests on
                   the same leading whole pages, each planned on its own
                   ("Track C · Document 10", block-size paragraph and the
                   table of prompt-layout mistakes; "GraniKV", sections 2-3).
* ``batch``     -- runs the above over a whole synthetic batch.

Pins (tests/test_oracle.py, each with planted mistakes that it rejects):
widening against torch's own bit reinterpretation and fp8 decode (all 256
codes, random fp32 and bf16 patterns with zeros, subnormals, infinities and
NaNs); the default softmax scale against the Llama layer's stated 1/sqrt(128);
a request's inputs against torch-widened values with unlike K and V scales;
attention against torch's SDPA in float64, brute force and closed forms; the
merge against splits at every point; the batch and prefix references against
SDPA on torch-widened inputs; lowering, planner and groups against brute force
and the pages' worked examples.

Parity unpinned: none of the functions here.  The planner's tuning constants
are inputs; whether their gfx950 values are the right ones is a measurement,
not an oracle question.
"""
from . import values, attention, lowering, planner, groups, batch  # noqa: F401
