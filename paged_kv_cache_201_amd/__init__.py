"""Python binding of libpkv.so (batched paged decode attention for gfx950).

Argument marshalling only: every function here has the name of the C entry
point it calls, converts torch tensors / numpy arrays to pointers, and raises
``PkvError`` when the library returns a non-OK status.  All device work runs
in the library's HIP kernels; there is no fallback path.  Importing this
package fails if ``libpkv.so`` has not been built
(``python paged_kv_cache_201_amd/build.py``).

Device tensors must be contiguous and on a CUDA (HIP) device; this is checked
before any pointer is passed, so a host pointer never reaches a kernel.
"""
import contextlib
import ctypes
import os

import numpy as np
# torch before the library: libpkv.so needs libamdhip64.so.7, and torch ships a
# HIP runtime of its own under that soname.  Loaded first, the library would
# map the system runtime and torch a second one, so torch's streams and
# allocations and this library's kernels would live in different runtimes;
# loaded second, it binds to the runtime torch already holds.
import torch  # noqa: F401

_LIB_PATH =os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python paged_kv_cache_201_amd/build.py`")
_lib = ctypes.CDLL(_LIB_PATH)

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_ERANGE, PKV_EHIP, PKV_ENOMEM = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "ERANGE", -5: "EHIP",
                -6: "ENOMEM"}
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"f32": PKV_F32, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3}
PKV_PATH_PAGED, PKV_PATH_CASCADE, PKV_PATH_DENSE = 0, 1, 2
PATH_NAMES = {0: "PAGED", 1: "CASCADE", 2: "DENSE"}

_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p


class PkvError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({_lib.pkv_status_string(status).decode()})")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class pkv_pool(ctypes.Structure):
    _fields_ = [("k", _vp), ("v", _vp), ("k_scale", _vp), ("v_scale", _vp), ("num_slots", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


class pkv_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("kv_indptr", _i32p), ("shared_prefix_len", ctypes.c_int32),
                ("force_path", ctypes.c_int32), ("kv_indices", _i32p)]


class pkv_tuning(ctypes.Structure):
    _fields_ = [("t_dense", ctypes.c_int32), ("gate_ratio", ctypes.c_int32), ("launch_bytes", ctypes.c_int64),
                ("target_workgroups", ctypes.c_int32), ("min_split_tokens", ctypes.c_int32),
                ("concurrent_prefix", ctypes.c_int32), ("fuse_cascade", ctypes.c_int32),
                ("prefix_target_workgroups", ctypes.c_int32), ("min_prefix_split_tokens", ctypes.c_int32),
                ("max_heads_per_item", ctypes.c_int32), ("prefix_placement", ctypes.c_int32),
                ("segment_tokens", ctypes.c_int32), ("cached_prefix_bytes", ctypes.c_int64),
                ("cached_reread_bytes", ctypes.c_int64)]


class pkv_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("m_eff", ctypes.c_int32), ("shared_pages", ctypes.c_int32),
                ("prefix_tokens", ctypes.c_int32), ("split_tokens", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("heads_per_item", ctypes.c_int32), ("prefix_splits", ctypes.c_int32),
                ("num_work_items", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("num_groups", ctypes.c_int32), ("metadata_ints", ctypes.c_int64),
                ("prefix_base", ctypes.c_int32), ("contiguous_prefixes", ctypes.c_int32),
                ("request_bins", ctypes.c_int32)]


_SIGS = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_tuning_defaults": (None, [ctypes.POINTER(pkv_tuning)]),
    "pkv_lower_page_table": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p,
                                              ctypes.c_int64]),
    "pkv_validate_indices": (ctypes.c_int32, [_i32p, _i32p, ctypes.c_int32, ctypes.c_int64]),
    "pkv_plan_create": (ctypes.c_int32, [ctypes.POINTER(pkv_problem), ctypes.POINTER(pkv_tuning),
                                         ctypes.POINTER(_vp)]),
    "pkv_plan_create_grouped": (ctypes.c_int32, [ctypes.POINTER(pkv_problem), ctypes.POINTER(pkv_tuning),
                                                 _i32p, _i32p, _i32p, ctypes.POINTER(_vp)]),
    "pkv_plan_metadata": (ctypes.c_int32, [_vp, _i32p, ctypes.c_int64]),
    "pkv_plan_request_bins": (ctypes.c_int32, [_vp, _i32p, ctypes.c_int64]),
    "pkv_plan_get_info": (ctypes.c_int32, [_vp, ctypes.POINTER(pkv_plan_info)]),
    "pkv_plan_destroy": (None, [_vp]),
    "pkv_paged_decode_attn": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, _vp, ctypes.c_float, _vp,
                                               _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "pkv_paged_decode_attn_pages": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, _vp, _vp,
                                                     ctypes.c_float, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "pkv_cascade_prefix_attn": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, ctypes.c_int32,
                                                 ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "pkv_merge_states": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                          _vp, _vp]),
    "pkv_decode_step": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, _vp, ctypes.c_float, _vp, _vp,
                                         _vp, ctypes.c_size_t, _vp]),
    "pkv_decode_step_noalloc": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, _vp, ctypes.c_float,
                                                 _vp, _vp, _vp]),
    "pkv_decode_step_grouped": (ctypes.c_int32, [_vp, _vp, ctypes.POINTER(pkv_pool), _vp, ctypes.c_float, _vp,
                                                 _vp, _vp, ctypes.c_size_t, _vp]),
    "pkv_stream_read_probe": (ctypes.c_int32, [_vp, ctypes.c_int64, _vp, ctypes.c_int32, _vp]),
    "pkv_stream_write_probe": (ctypes.c_int32, [_vp, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32, _vp]),
}


def _bind(lib):
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_bind(_lib)

EXPORTS = tuple(_SIGS)
LIB_PATH = _LIB_PATH
CHECKED_LIB_PATH = os.path.join(os.path.dirname(_LIB_PATH), "libpkv_checked.so")
_checked_lib = None


@contextlib.contextmanager
def checked_library():
    """Route the calls made inside the block (plans included) to
    libpkv_checked.so: the same kernels and entry points, which before any
    launch wait for the caller's stream and check the step's index arrays
    against the plan and the pool (PKV_EINVAL / PKV_ERANGE instead of a
    launch).  For tests and debugging; not thread-safe."""
    global _lib, _checked_lib
    if _checked_lib is None:
        if not os.path.exists(CHECKED_LIB_PATH):
            raise ImportError(f"{CHECKED_LIB_PATH} is not built; run `python paged_kv_cache_201_amd/build.py`")
        _checked_lib = _bind(ctypes.CDLL(CHECKED_LIB_PATH))
    prev, _lib = _lib, _checked_lib
    try:
        yield _lib
    finally:
        _lib = prev


def _check(status, where):
    if status != PKV_OK:
        raise PkvError(status, where)


def _host_i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(_i32p)


def _dev(t, name, dtypes=None, allow_none=False):
    """Device pointer of a contiguous CUDA tensor (None -> NULL if allowed)."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t.data_ptr()


def _torch_of_code(code):
    import torch
    return {PKV_F32: torch.float32, PKV_BF16: torch.bfloat16}[code]


def _check_sizes(plan, **tensors):
    """Sizes and dtypes of the step's tensors against the plan's problem,
    before any pointer reaches the library (which trusts them)."""
    import torch
    pr = plan.problem
    B, H_q, d = pr["batch"], pr["num_q_heads"], pr["head_dim"]
    qd = _torch_of_code(DTYPE_CODES.get(pr["q_dtype"], pr["q_dtype"]))
    want = {"q": (B * H_q * d, (qd,)), "o": (B * H_q * d, (qd,)), "o_f32": (B * H_q * d, (torch.float32,)),
            "o_p": (B * H_q * d, (torch.float32,)), "lse": (B * H_q, (torch.float32,)),
            "lse_p": (B * H_q, (torch.float32,)), "kv_indptr": (B + 1, (torch.int32,)),
            "page_indptr": (B + 1, (torch.int32,)),
            "metadata": (plan.info.get("metadata_ints", 0), (torch.int32,))}
    for name, t in tensors.items():
        if t is None:
            continue
        n, dtypes = want[name]
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}; the plan needs {dtypes[0]}")
        if (t.numel() < n) if name == "metadata" else (t.numel() != n):
            raise ValueError(f"{name} has {t.numel()} elements; the plan needs {n}")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _torch_dtype_code(t):
    import torch
    return {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16, torch.float8_e4m3fn: PKV_FP8_E4M3,
            torch.uint8: PKV_FP8_E4M3}[t.dtype]


def pkv_status_string(status: int) -> str:
    return _lib.pkv_status_string(status).decode()


def pkv_version() -> str:
    return _lib.pkv_version().decode()


def pkv_tuning_defaults() -> dict:
    t = pkv_tuning()
    _lib.pkv_tuning_defaults(ctypes.byref(t))
    return {name: getattr(t, name) for name, _ in pkv_tuning._fields_}


def pkv_lower_page_table(page_size, page_indptr, page_indices, seq_lens):
    """Host lowering; returns (kv_indptr, kv_indices) as int32 numpy arrays."""
    pi, pi_p = _host_i32(page_indptr)
    pg, pg_p = _host_i32(page_indices if len(page_indices) else np.zeros(1, np.int32))
    sl, sl_p = _host_i32(seq_lens)
    B = len(sl)
    cap = int(max(0, sl.astype(np.int64).sum()))
    kv_indptr = np.zeros(B + 1, np.int32)
    kv_indices = np.zeros(max(cap, 1), np.int32)
    st = _lib.pkv_lower_page_table(B, page_size, pi_p, pg_p, sl_p, kv_indptr.ctypes.data_as(_i32p),
                                   kv_indices.ctypes.data_as(_i32p), cap)
    _check(st, "pkv_lower_page_table")
    return kv_indptr, kv_indices[:cap]


def pkv_validate_indices(kv_indptr, kv_indices, num_slots):
    ip, ip_p = _host_i32(kv_indptr)
    ix, ix_p = _host_i32(kv_indices if len(kv_indices) else np.zeros(1, np.int32))
    _check(_lib.pkv_validate_indices(ip_p, ix_p, len(ip) - 1, int(num_slots)), "pkv_validate_indices")


class Plan:
    """Owns one pkv_plan handle."""

    def __init__(self, handle, problem):
        self.handle = handle
        self.problem = problem
        self._lib = _lib  # the library that made the plan destroys it
        info = pkv_plan_info()
        _check(_lib.pkv_plan_get_info(handle, ctypes.byref(info)), "pkv_plan_get_info")
        self.info = {name: getattr(info, name) for name, _ in pkv_plan_info._fields_}
        self.info["path_name"] = PATH_NAMES[self.info["path"]]

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        lib = getattr(self, "_lib", None)
        if h and lib is not None:  # the library may already be gone at interpreter exit
            lib.pkv_plan_destroy(h)


def pkv_plan_create(*, batch, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype, page_size, kv_indptr,
                    shared_prefix_len=0, force_path=-1, tuning=None, kv_indices=None) -> Plan:
    """Plan one step.  q_dtype/kv_dtype: "f32", "bf16" or "fp8" (or the codes).
    kv_indices (host, optional) lets the planner find a contiguously placed
    prefix."""
    ip, ip_p = _host_i32(kv_indptr)
    ix_p = None
    if kv_indices is not None:
        ix, ix_p = _host_i32(kv_indices if len(kv_indices) else np.zeros(1, np.int32))
        if len(kv_indices) < int(ip[-1]) if len(ip) else False:
            raise ValueError("kv_indices is shorter than kv_indptr[B]")
    pr = pkv_problem(batch, num_q_heads, num_kv_heads, head_dim, DTYPE_CODES.get(q_dtype, q_dtype),
                     DTYPE_CODES.get(kv_dtype, kv_dtype), page_size, ip_p, shared_prefix_len, force_path, ix_p)
    tp = None
    if tuning is not None:
        d = pkv_tuning_defaults()
        d.update(tuning)
        tp = ctypes.byref(pkv_tuning(**d))
    h = _vp()
    _check(_lib.pkv_plan_create(ctypes.byref(pr), tp, ctypes.byref(h)), "pkv_plan_create")
    return Plan(h.value, dict(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                              q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=page_size,
                              shared_prefix_len=shared_prefix_len, force_path=force_path))


def pkv_plan_create_grouped(*, batch, num_q_heads, num_kv_heads, head_dim, q_dtype, kv_dtype, page_size,
                            page_indptr, page_indices, seq_lens, force_path=-1, tuning=None) -> Plan:
    """Plan a step whose requests may share several prefixes, found in the
    page table (host arrays)."""
    ptr, ptr_p = _host_i32(page_indptr)
    pages, pages_p = _host_i32(page_indices if len(page_indices) else np.zeros(1, np.int32))
    lens, lens_p = _host_i32(seq_lens if len(seq_lens) else np.zeros(1, np.int32))
    pr = pkv_problem(batch, num_q_heads, num_kv_heads, head_dim, DTYPE_CODES.get(q_dtype, q_dtype),
                     DTYPE_CODES.get(kv_dtype, kv_dtype), page_size, None, 0, force_path)
    tp = None
    if tuning is not None:
        d = pkv_tuning_defaults()
        d.update(tuning)
        tp = ctypes.byref(pkv_tuning(**d))
    h = _vp()
    _check(_lib.pkv_plan_create_grouped(ctypes.byref(pr), tp, ptr_p, pages_p, lens_p, ctypes.byref(h)),
           "pkv_plan_create_grouped")
    return Plan(h.value, dict(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                              q_dtype=q_dtype, kv_dtype=kv_dtype, page_size=page_size, force_path=force_path,
                              grouped=True))


def pkv_plan_metadata(plan: Plan):
    """The grouped plan's metadata block as a numpy int32 array."""
    n = plan.info["metadata_ints"]
    out = np.zeros(max(n, 1), np.int32)
    _check(_lib.pkv_plan_metadata(plan.handle, out.ctypes.data_as(_i32p), n), "pkv_plan_metadata")
    return out[:n]


def pkv_plan_request_bins(plan: Plan):
    """(bin_start [W+1], requests [B]) of a plan whose paged pass runs on bins
    of whole requests (plan.info["request_bins"] = W > 0)."""
    W, B = plan.info["request_bins"], plan.problem["batch"]
    out = np.zeros(W + 1 + B, np.int32)
    _check(_lib.pkv_plan_request_bins(plan.handle, out.ctypes.data_as(_i32p), len(out)), "pkv_plan_request_bins")
    return out[:W + 1], out[W + 1:]


def split_metadata(block, batch, num_groups):
    """Views of the public arrays of a metadata block, by name."""
    out, off = {}, 0
    for name, n in (("suffix_indptr", batch + 1), ("suffix_indices", None), ("group_indptr", num_groups + 1),
                    ("group_members", None), ("prefix_indptr", num_groups + 1), ("prefix_indices", None),
                    ("group_parent", num_groups), ("group_prefix_base", num_groups)):
        if n is None:
            ptr = out[{"suffix_indices": "suffix_indptr", "group_members": "group_indptr",
                       "prefix_indices": "prefix_indptr"}[name]]
            n = int(ptr[-1])
        out[name] = block[off:off + n]
        off += n
    return out


def pkv_plan_get_info(plan: Plan) -> dict:
    return dict(plan.info)


def make_pool(k, v, page_size, k_scale=None, v_scale=None):
    """pkv_pool describing torch tensors k, v of shape [num_slots, H_kv, d]."""
    import torch
    kv_dtype = _torch_dtype_code(k)
    scales = (torch.float32,)
    pool = pkv_pool(_dev(k, "k"), _dev(v, "v"), _dev(k_scale, "k_scale", scales, allow_none=True),
                    _dev(v_scale, "v_scale", scales, allow_none=True), k.shape[0], page_size, k.shape[1],
                    k.shape[2], kv_dtype)
    pool._keep = (k, v, k_scale, v_scale)
    return pool


def _ws(workspace, plan):
    need = plan.info["workspace_bytes"]
    if workspace is None:
        return None, 0
    import torch
    ptr = _dev(workspace, "workspace")
    return ptr, workspace.numel() * workspace.element_size()


def pkv_paged_decode_attn(plan, q, pool, kv_indptr, kv_indices, sm_scale, o=None, o_f32=None, lse=None,
                          workspace=None, stream=None):
    import torch
    _check_sizes(plan, q=q, o=o, o_f32=o_f32, lse=lse, kv_indptr=kv_indptr)
    ws, wsb = _ws(workspace, plan)
    st = _lib.pkv_paged_decode_attn(plan.handle, _dev(q, "q"), ctypes.byref(pool),
                                    _dev(kv_indptr, "kv_indptr", (torch.int32,)),
                                    _dev(kv_indices, "kv_indices", (torch.int32,)), float(sm_scale),
                                    _dev(o, "o", allow_none=True), _dev(o_f32, "o_f32", (torch.float32,), True),
                                    _dev(lse, "lse", (torch.float32,), True), ws, wsb, _stream(stream))
    _check(st, "pkv_paged_decode_attn")


def pkv_paged_decode_attn_pages(plan, q, pool, kv_indptr, page_indptr, page_indices, sm_scale, o=None, o_f32=None,
                                lse=None, workspace=None, stream=None):
    import torch
    _check_sizes(plan, q=q, o=o, o_f32=o_f32, lse=lse, kv_indptr=kv_indptr, page_indptr=page_indptr)
    ws, wsb = _ws(workspace, plan)
    i32 = (torch.int32,)
    st = _lib.pkv_paged_decode_attn_pages(plan.handle, _dev(q, "q"), ctypes.byref(pool),
                                          _dev(kv_indptr, "kv_indptr", i32), _dev(page_indptr, "page_indptr", i32),
                                          _dev(page_indices, "page_indices", i32), float(sm_scale),
                                          _dev(o, "o", allow_none=True), _dev(o_f32, "o_f32", (torch.float32,), True),
                                          _dev(lse, "lse", (torch.float32,), True), ws, wsb, _stream(stream))
    _check(st, "pkv_paged_decode_attn_pages")


def pkv_cascade_prefix_attn(plan, q, pool, prefix_indices, prefix_len, sm_scale, o_p, lse_p, workspace=None,
                            stream=None):
    import torch
    _check_sizes(plan, o_p=o_p, lse_p=lse_p)   # q: bf16, checked below
    if q is not None and q.numel() != o_p.numel():
        raise ValueError(f"q has {q.numel()} elements; the plan needs {o_p.numel()}")
    if prefix_indices is not None and prefix_indices.numel() < int(prefix_len):
        raise ValueError(f"prefix_indices has {prefix_indices.numel()} entries; prefix_len is {prefix_len}")
    ws, wsb = _ws(workspace, plan)
    st = _lib.pkv_cascade_prefix_attn(plan.handle, _dev(q, "q", (torch.bfloat16,)), ctypes.byref(pool),
                                      _dev(prefix_indices, "prefix_indices", (torch.int32,)), int(prefix_len),
                                      float(sm_scale), _dev(o_p, "o_p", (torch.float32,)),
                                      _dev(lse_p, "lse_p", (torch.float32,)), ws, wsb, _stream(stream))
    _check(st, "pkv_cascade_prefix_attn")


def pkv_merge_states(o_a, lse_a, o_b, lse_b, o_out, lse_out=None, stream=None):
    import torch
    f32 = (torch.float32,)
    rows = lse_a.numel()
    d = o_a.shape[-1]
    for name, t, n in (("lse_b", lse_b, rows), ("o_a", o_a, rows * d), ("o_b", o_b, rows * d),
                       ("o_out", o_out, rows * d), ("lse_out", lse_out, rows)):
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements; {n} expected for {rows} rows of {d}")
    st = _lib.pkv_merge_states(rows, d, _dev(o_a, "o_a", f32), _dev(lse_a, "lse_a", f32), _dev(o_b, "o_b", f32),
                               _dev(lse_b, "lse_b", f32), _dev(o_out, "o_out", (torch.float32, torch.bfloat16)),
                               _torch_dtype_code(o_out), _dev(lse_out, "lse_out", f32, True), _stream(stream))
    _check(st, "pkv_merge_states")


def pkv_decode_step(plan, q, pool, kv_indptr, kv_indices, sm_scale, o, lse=None, workspace=None, stream=None):
    import torch
    _check_sizes(plan, q=q, o=o, lse=lse, kv_indptr=kv_indptr)
    ws, wsb = _ws(workspace, plan)
    st = _lib.pkv_decode_step(plan.handle, _dev(q, "q"), ctypes.byref(pool),
                              _dev(kv_indptr, "kv_indptr", (torch.int32,)),
                              _dev(kv_indices, "kv_indices", (torch.int32,)), float(sm_scale), _dev(o, "o"),
                              _dev(lse, "lse", (torch.float32,), True), ws, wsb, _stream(stream))
    _check(st, "pkv_decode_step")


NOALLOC_SCRATCH_BYTES = 64 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def pkv_decode_step_noalloc(plan, q, pool, kv_indptr, kv_indices, sm_scale, o, lse=None, stream=None):
    """pkv_decode_step with the library's device scratch as workspace."""
    import torch
    _check_sizes(plan, q=q, o=o, lse=lse, kv_indptr=kv_indptr)
    st = _lib.pkv_decode_step_noalloc(plan.handle, _dev(q, "q"), ctypes.byref(pool),
                                      _dev(kv_indptr, "kv_indptr", (torch.int32,)),
                                      _dev(kv_indices, "kv_indices", (torch.int32,)), float(sm_scale), _dev(o, "o"),
                                      _dev(lse, "lse", (torch.float32,), True), _stream(stream))
    _check(st, "pkv_decode_step_noalloc")


def pkv_decode_step_grouped(plan, q, pool, metadata, sm_scale, o, lse=None, workspace=None, stream=None):
    import torch
    _check_sizes(plan, q=q, o=o, lse=lse, metadata=metadata)
    ws, wsb = _ws(workspace, plan)
    st = _lib.pkv_decode_step_grouped(plan.handle, _dev(q, "q"), ctypes.byref(pool),
                                      _dev(metadata, "metadata", (torch.int32,)), float(sm_scale), _dev(o, "o"),
                                      _dev(lse, "lse", (torch.float32,), True), ws, wsb, _stream(stream))
    _check(st, "pkv_decode_step_grouped")


def pkv_stream_write_probe(buf, value, num_workgroups, stream=None):
    """Write all of ``buf`` (a CUDA tensor) once with the 32-bit ``value``."""
    _check(_lib.pkv_stream_write_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(), int(value) & 0xFFFFFFFF,
                                       int(num_workgroups), _stream(stream)), "pkv_stream_write_probe")


def pkv_stream_read_probe(buf, out, num_workgroups, stream=None):
    """Read all of ``buf`` (a CUDA tensor) once; ``out`` holds num_workgroups int32."""
    import torch
    _check(_lib.pkv_stream_read_probe(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                      _dev(out, "out", (torch.int32,)), int(num_workgroups), _stream(stream)),
           "pkv_stream_read_probe")


def workspace_for(plan, device="cuda"):
    """A uint8 workspace tensor of the plan's size (None if 0)."""
    import torch
    n = plan.info["workspace_bytes"]
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device) if n else None
