"""Per-step path choice (test oracle, integers only).

"GraniKV: asymmetric KV cache paging for shared-prefix agents", section 3
"Per-step dispatcher": M_eff is the realized batch times the GQA group size
(queries per KV head).  At or above a threshold the shared prefix goes to a
dense matmul kernel, below it to a tiled cascade loop; the threshold was
fitted on one GPU and must be refitted on another.  Section 5 reports that
short prefixes regress, without giving a rule; the gate below is this
library's reading, with its constants passed in.

Prefix matching is block aligned ("Track C · Document 10", block-size
paragraph), so only floor(P / p) whole pages are shared and the tail of the
prefix is treated as part of every request's own suffix.

Rule, in order (all arithmetic in Python integers):

1. forced path (force_path >= 0): taken as is, after the capability checks;
2. no declared prefix, fewer than two requests, no whole shared page, or a
   dtype pair the prefix kernels do not handle -> PAGED;
3. saved    = (n_shared - 1) * prefix_tokens * H_kv * d * (b_k + b_v)
   overhead = 4 * rows * (d + 1) * 4 + launch_bytes
   allowed  = gate_ratio * overhead, raised to cached_reread_bytes when
              gate_ratio > 0 and the prefix's stored K and V (prefix_tokens *
              H_kv * d * 2 * the stored value's bytes) take at most
              cached_prefix_bytes > 0
   (the allowance only where the DENSE step would not take the fused launch:
   fuse_cascade = 0, or 4 * M_eff * prefix_tokens * d * H_kv <
   fuse_cascade * (sum of L_b - prefix_tokens) * H_kv * d * (b_k + b_v))
   saved < allowed -> PAGED;  (b_k, b_v: an fp8 value counts as 2 bytes, the
   bf16 width: the library's fp8 paged pass is bound by the vector ALU, so its
   tokens cost about the time of bf16 tokens; measured.  A small prefix stays
   cached while every request re-reads it, so its re-reads cost little; also
   measured)
4. M_eff >= t_dense -> DENSE, else CASCADE.

Prefix placement ("GraniKV", section 1, asymmetric paging: the shared prefix
is placed contiguously when its radix node is created, so that the dense
kernel reads it as a plain strided operand).  Reading taken: on a CASCADE or
DENSE plan, when the planner is shown the prefix's slots and placement is
enabled, a prefix whose slots are first, first + 1, ..., first + P' - 1 (P'
= prefix_tokens) is read as base + offset with base = first; otherwise (or
on PAGED) base = -1 and the prefix is read slot by slot.  The result is the
same either way; only the addressing differs.

Problem checks mirror what the library accepts: d in {64, 128}; (q, kv)
dtype in {(f32, f32), (bf16, bf16), (bf16, fp8)}; G in {1, 2, 4, 8}; the
prefix kernels take bf16 queries over bf16 K/V, or over fp8 K/V at d = 128.
"""
PAGED, CASCADE, DENSE = "PAGED", "CASCADE", "DENSE"
PATH_NAMES = (PAGED, CASCADE, DENSE)

BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
SUPPORTED_DTYPES = {("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8")}
PREFIX_DTYPES = {("bf16", "bf16"), ("bf16", "fp8")}


def prefix_capable(q_dtype, kv_dtype, d):
    """Whether a prefix kernel exists for this pair (fp8 K/V: d = 128 only)."""
    return (q_dtype, kv_dtype) in PREFIX_DTYPES and (kv_dtype != "fp8" or d == 128)


class PlanError(ValueError):
    def __init__(self, code, msg=""):
        super().__init__(f"{code}: {msg}")
        self.code = code  # "EINVAL" or "EUNSUPPORTED"


def plan(*, B, H_q, H_kv, d, q_dtype, kv_dtype, page_size, seq_lens,
         shared_prefix_len, force_path, t_dense, gate_ratio, launch_bytes, prefix_slots=None,
         prefix_placement=1, cached_prefix_bytes=0, cached_reread_bytes=0, fuse_cascade=0):
    """Returns dict(path, m_eff, shared_pages, prefix_tokens, prefix_base).

    ``prefix_slots`` (optional): the slots of the first request's first
    tokens, at least ``prefix_tokens`` of them; ``prefix_base`` follows the
    placement rule above.
    """
    out = _plan_path(B=B, H_q=H_q, H_kv=H_kv, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=page_size,
                     seq_lens=seq_lens, shared_prefix_len=shared_prefix_len, force_path=force_path,
                     t_dense=t_dense, gate_ratio=gate_ratio, launch_bytes=launch_bytes,
                     cached_prefix_bytes=cached_prefix_bytes, cached_reread_bytes=cached_reread_bytes,
                     fuse_cascade=fuse_cascade)
    out["prefix_base"] = -1
    n = out["prefix_tokens"]
    if out["path"] != PAGED and prefix_placement and prefix_slots is not None and n > 0:
        first = int(prefix_slots[0])
        if first >= 0 and all(int(prefix_slots[t]) == first + t for t in range(n)):
            out["prefix_base"] = first
    return out


def _plan_path(*, B, H_q, H_kv, d, q_dtype, kv_dtype, page_size, seq_lens,
               shared_prefix_len, force_path, t_dense, gate_ratio, launch_bytes,
               cached_prefix_bytes=0, cached_reread_bytes=0, fuse_cascade=0):
    """Returns dict(path, m_eff, shared_pages, prefix_tokens).

    ``shared_pages`` is floor(P / p) whenever a prefix is declared;
    ``prefix_tokens`` is the number of tokens the prefix pass covers: the
    shared whole pages on CASCADE / DENSE, and 0 on PAGED (the paged pass then
    attends every token).
    """
    if B < 0 or H_kv < 1 or H_q < 1 or page_size < 1 or d < 1:
        raise PlanError("EINVAL", "non-positive size")
    if H_q % H_kv:
        raise PlanError("EINVAL", "H_q not a multiple of H_kv")
    if len(seq_lens) != B or any(int(x) < 0 for x in seq_lens):
        raise PlanError("EINVAL", "bad sequence lengths")
    if shared_prefix_len < 0 or (B and shared_prefix_len > min(int(x) for x in seq_lens)):
        raise PlanError("EINVAL", "prefix longer than a request")
    if force_path not in (-1, 0, 1, 2):
        raise PlanError("EINVAL", "bad force_path")
    G = H_q // H_kv
    if d not in (64, 128) or (q_dtype, kv_dtype) not in SUPPORTED_DTYPES or G not in (1, 2, 4, 8):
        raise PlanError("EUNSUPPORTED", "shape or dtype")
    n_shared = B if shared_prefix_len > 0 else 0
    shared_pages = shared_prefix_len // page_size if n_shared else 0
    prefix_tokens = shared_pages * page_size
    m_eff = B * G
    capable = prefix_capable(q_dtype, kv_dtype, d)
    out = dict(m_eff=m_eff, shared_pages=shared_pages, prefix_tokens=prefix_tokens)
    if force_path >= 0:
        path = PATH_NAMES[force_path]
        if path != PAGED:
            if not capable:
                raise PlanError("EUNSUPPORTED", "prefix path for this dtype")
            if prefix_tokens == 0:
                raise PlanError("EINVAL", "no whole shared page")
        else:
            out["prefix_tokens"] = 0
        out["path"] = path
        return out
    if not capable or n_shared < 2 or shared_pages == 0:
        out.update(path=PAGED, prefix_tokens=0)
        return out
    rows = B * H_q
    gate_bytes = 2 if kv_dtype == "fp8" else BYTES[kv_dtype]
    saved = (n_shared - 1) * prefix_tokens * H_kv * d * (gate_bytes * 2)
    overhead = 4 * rows * (d + 1) * 4 + launch_bytes
    allowed = gate_ratio * overhead
    stored = prefix_tokens * H_kv * d * 2 * BYTES[kv_dtype]
    suffix = sum(int(x) - prefix_tokens for x in seq_lens)
    fuses = fuse_cascade > 0 and 4 * m_eff * prefix_tokens * d * H_kv >= fuse_cascade * suffix * H_kv * d * gate_bytes * 2
    if gate_ratio > 0 and cached_prefix_bytes > 0 and stored <= cached_prefix_bytes and not fuses:
        allowed = max(allowed, cached_reread_bytes)
    if saved < allowed:
        out.update(path=PAGED, prefix_tokens=0)
    elif m_eff >= t_dense:
        out["path"] = DENSE
    else:
        out["path"] = CASCADE
    return out
