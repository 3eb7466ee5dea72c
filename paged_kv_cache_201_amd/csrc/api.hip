// C ABI entry points that enqueue device work: argument checks, workspace
// carving, and kernel launches on the caller's stream.  No allocation, no
// synchronisation.
//
// Built a second time with PKV_CHECKED=1 into libpkv_checked.so (the same
// kernels and entry points): there, before any launch, a call that takes
// device index arrays waits for the caller's stream, copies to the host what
// its kernels would read of those arrays and checks it against the plan and
// the pool (the checks are in host.cpp).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "kernels.h"
#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
hipError_t launch_paged_split_f32(const pkv_plan& p, const PagedArgs& a, hipStream_t s);
hipError_t launch_paged_split_bf16(const pkv_plan& p, const PagedArgs& a, hipStream_t s);
hipError_t launch_paged_split_fp8(const pkv_plan& p, const PagedArgs& a, hipStream_t s);

hipError_t launch_paged_split(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    switch (p.kv_dtype) {
        case PKV_F32: return launch_paged_split_f32(p, a, s);
        case PKV_BF16: return launch_paged_split_bf16(p, a, s);
        case PKV_FP8_E4M3: return launch_paged_split_fp8(p, a, s);
        default: return hipErrorInvalidValue;
    }
}
}  // namespace pkv

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The kernels take row maxima of unscaled scores and scale them afterwards,
// which needs a positive scale (a NaN or infinite one has no softmax either).
bool scale_ok(float sm_scale) { return sm_scale > 0.f && sm_scale < INFINITY; }

pkv_status check_pool(const pkv_plan* pl, const pkv_pool* pool) {
    if (!pool || !pool->k || !pool->v) return PKV_EINVAL;
    if (pool->kv_dtype != pl->kv_dtype || pool->num_kv_heads != pl->H_kv ||
        pool->head_dim != pl->D || pool->page_size != pl->page_size)
        return PKV_EINVAL;
    if (pool->num_slots < 0 || pool->num_slots % pool->page_size) return PKV_EINVAL;
    if (pl->kv_dtype == PKV_FP8_E4M3 && (!pool->k_scale || !pool->v_scale)) return PKV_EINVAL;
    return PKV_OK;
}

pkv_status check_workspace(const pkv_plan* pl, const void* ws, size_t ws_bytes) {
    if (pl->workspace_bytes == 0) return PKV_OK;
    if (!ws || (int64_t)ws_bytes < pl->workspace_bytes) return PKV_EWORKSPACE;
    return PKV_OK;
}

template <typename T>
T* ws_at(void* ws, int64_t off) {
    return off < 0 ? nullptr : reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_EHIP; }

// Per-device side stream and fork/join events for running the prefix pass
// concurrently with the suffix pass.  Created on first use, default
// priority, kept until the process ends.  The mutex also serialises the
// record/wait sequence so that two host threads never interleave their use
// of the shared events.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::unordered_map<int, SideStream> g_side;

hipError_t side_stream_locked(SideStream** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    SideStream& ss = g_side[dev];
    if (!ss.stream) {
        if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    }
    *out = &ss;
    return hipSuccess;
}

// The paged pass over tokens [plan.prefix_tokens, L_b) of every request.
pkv::PagedArgs paged_args(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* kv_indptr,
                          const int32_t* kv_indices, float sm_scale) {
    pkv::PagedArgs a{};
    a.q = q;
    a.k = pool->k;
    a.v = pool->v;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.kv_indptr = kv_indptr;
    a.kv_indices = kv_indices;
    a.B = pl->B;
    a.H_kv = pl->H_kv;
    a.token_offset = pl->prefix_tokens;
    a.chunk_tokens = pl->split_tokens;
    a.total_tokens = pl->paged_tokens;
    a.max_parts = pl->num_splits;
    a.scale_log2 = sm_scale * kLog2e;
    a.out_dtype = pl->q_dtype;
    a.request_bins = pl->request_bins;
    a.bin_max_tokens = pl->bin_max_tokens;
    if (pl->request_bins > 0) {
        std::copy(pl->bin_start.begin(), pl->bin_start.end(), a.bin_start);
        std::copy(pl->bin_req.begin(), pl->bin_req.end(), a.bin_req);
    }
    return a;
}

// The combine of a paged pass: chunk partials of every request (and, for a
// cascade step, the prefix ranges before them).
pkv::SplitReduceArgs chunk_reduce_args(const pkv_plan* pl, const pkv::PagedArgs& a) {
    pkv::SplitReduceArgs r{};
    r.B = pl->B;
    r.H_q = pl->H_q;
    r.D = pl->D;
    r.part_acc = a.part_acc;
    r.part_ml = a.part_ml;
    r.max_parts = pl->num_splits;
    r.kv_indptr = a.kv_indptr;
    r.token_offset = a.token_offset;
    r.chunk_tokens = a.chunk_tokens;
    r.whole_requests = pl->request_bins > 0;
    r.out_dtype = pl->q_dtype;
    return r;
}

pkv_status run_paged_args(const pkv_plan* pl, pkv::PagedArgs a, void* o, float* o_f32, float* lse, void* ws,
                          hipStream_t stream) {
    a.o = o;
    a.o_f32 = o_f32;
    a.lse = lse;
    a.part_acc = ws_at<float>(ws, pl->ws_paged_acc);
    a.part_ml = ws_at<float>(ws, pl->ws_paged_ml);
    if (pl->num_chunks > 0 && pkv::launch_paged_split(*pl, a, stream) != hipSuccess) return PKV_EHIP;
    if (!pl->needs_reduce) return PKV_OK;
    pkv::SplitReduceArgs r = chunk_reduce_args(pl, a);
    r.skip_whole = 1;
    r.o = o;
    r.o_f32 = o_f32;
    r.lse = lse;
    return hip_status(pkv::launch_split_reduce(r, stream));
}

pkv_status run_paged(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* kv_indptr,
                     const int32_t* kv_indices, float sm_scale, void* o, float* o_f32, float* lse,
                     void* ws, hipStream_t stream) {
    return run_paged_args(pl, paged_args(pl, q, pool, kv_indptr, kv_indices, sm_scale), o, o_f32, lse, ws, stream);
}

pkv::PrefixArgs prefix_args(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* prefix_indices,
                            float sm_scale) {
    pkv::PrefixArgs a{};
    a.q = q;
    a.k = pool->k;
    a.v = pool->v;
    a.kv_dtype = pl->kv_dtype;
    a.k_scale = pool->k_scale;
    a.v_scale = pool->v_scale;
    a.prefix_indices = prefix_indices;
    a.prefix_base = pl->prefix_base;
    a.B = pl->B;
    a.H_kv = pl->H_kv;
    a.G = pl->G;
    a.D = pl->D;
    a.prefix_len = pl->prefix_tokens;
    a.split_tokens = pl->prefix_split_tokens;
    a.num_splits = pl->prefix_splits;
    a.row_tiles = (pl->m_eff + pl->prefix_rows_per_wg - 1) / pl->prefix_rows_per_wg;
    a.scale_log2 = sm_scale * kLog2e;
    return a;
}

pkv_status run_prefix(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* prefix_indices,
                      float sm_scale, float* o_p, float* lse_p, void* ws, hipStream_t stream) {
    pkv::PrefixArgs a = prefix_args(pl, q, pool, prefix_indices, sm_scale);
    if (pl->prefix_splits == 1) {
        a.o = o_p;
        a.lse = lse_p;
        return hip_status(pkv::launch_prefix_attn(a, pl->prefix_rows_per_wg, stream));
    }
    a.part_acc = ws_at<float>(ws, pl->ws_prefix_acc);
    a.part_ml = ws_at<float>(ws, pl->ws_prefix_ml);
    hipError_t e = pkv::launch_prefix_attn(a, pl->prefix_rows_per_wg, stream);
    if (e != hipSuccess) return PKV_EHIP;
    pkv::SplitReduceArgs r{};
    r.B = pl->B;
    r.H_q = pl->H_q;
    r.D = pl->D;
    r.pre_acc = a.part_acc;
    r.pre_ml = a.part_ml;
    r.pre_splits = pl->prefix_splits;
    r.o = nullptr;
    r.out_dtype = PKV_F32;
    r.o_f32 = o_p;
    r.lse = lse_p;
    return hip_status(pkv::launch_split_reduce(r, stream));
}

// One decode step as the plan chose it, with the workspace at ws (checked
// by the caller).  side_stream: the prefix pass may run on the library's
// side stream when the plan asks for it.
pkv_status run_decode_step(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* kv_indptr,
                           const int32_t* kv_indices, float sm_scale, void* o, float* lse, void* ws, hipStream_t s,
                           bool side_stream) {
    if (pl->path == PKV_PATH_PAGED)
        return run_paged(pl, q, pool, kv_indptr, kv_indices, sm_scale, o, nullptr, lse, ws, s);
    // Cascade: both passes leave partial states in the workspace, and one
    // kernel combines the prefix ranges and then the suffix chunks of every
    // row into the output.
    pkv::PrefixArgs pa = prefix_args(pl, q, pool, kv_indices + pl->indptr0, sm_scale);
    pa.part_acc = ws_at<float>(ws, pl->ws_prefix_acc);
    pa.part_ml = ws_at<float>(ws, pl->ws_prefix_ml);
    pa.force_partial = 1;
    pkv::PagedArgs sa = paged_args(pl, q, pool, kv_indptr, kv_indices, sm_scale);
    sa.part_acc = ws_at<float>(ws, pl->ws_paged_acc);
    sa.part_ml = ws_at<float>(ws, pl->ws_paged_ml);
    sa.force_partial = 1;
    if (pl->fuse_cascade) {
        if (pkv::launch_cascade_fused(*pl, pa, sa, s) != hipSuccess) return PKV_EHIP;
    } else if (side_stream) {
        std::lock_guard<std::mutex> lock(g_side_mu);
        SideStream* ss = nullptr;
        if (side_stream_locked(&ss) != hipSuccess) return PKV_EHIP;
        // fork: the side stream starts after everything already on `s`
        if (hipEventRecord(ss->fork, s) != hipSuccess) return PKV_EHIP;
        if (hipStreamWaitEvent(ss->stream, ss->fork, 0) != hipSuccess) return PKV_EHIP;
        if (pkv::launch_prefix_attn(pa, pl->prefix_rows_per_wg, ss->stream) != hipSuccess) return PKV_EHIP;
        if (pl->num_chunks > 0 && pkv::launch_paged_split(*pl, sa, s) != hipSuccess) return PKV_EHIP;
        // join: the combine on `s` waits for the prefix pass
        if (hipEventRecord(ss->join, ss->stream) != hipSuccess) return PKV_EHIP;
        if (hipStreamWaitEvent(s, ss->join, 0) != hipSuccess) return PKV_EHIP;
    } else {
        if (pkv::launch_prefix_attn(pa, pl->prefix_rows_per_wg, s) != hipSuccess) return PKV_EHIP;
        if (pl->num_chunks > 0 && pkv::launch_paged_split(*pl, sa, s) != hipSuccess) return PKV_EHIP;
    }
    pkv::SplitReduceArgs r = chunk_reduce_args(pl, sa);
    r.pre_acc = pa.part_acc;
    r.pre_ml = pa.part_ml;
    r.pre_splits = pl->prefix_splits;
    r.o = o;
    r.lse = lse;
    return hip_status(pkv::launch_split_reduce(r, s));
}

#ifndef PKV_CHECKED
#define PKV_CHECKED 0
#endif

#if PKV_CHECKED
// Host copy of n ints of device memory (after the stream sync below).
pkv_status fetch(const int32_t* dev, int64_t n, std::vector<int32_t>* out) {
    out->assign((size_t)n, 0);
    if (n == 0) return PKV_OK;
    if (!dev) return PKV_EINVAL;
    return hip_status(hipMemcpy(out->data(), dev, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost));
}

// The work already queued on the caller's stream may write the arrays.
pkv_status sync(hipStream_t s) { return hip_status(hipStreamSynchronize(s)); }

// Token-flat steps: kv_indptr as planned, every slot of
// kv_indices[kv_indptr[0] .. kv_indptr[B]) in the pool, and (with_prefix) the
// prefix pass's slots, the first prefix_tokens of them.
pkv_status checked_flat(const pkv_plan* pl, const pkv_pool* pool, const int32_t* kv_indptr,
                        const int32_t* kv_indices, bool with_prefix, hipStream_t s) try {
    pkv_status st = sync(s);
    std::vector<int32_t> ip, ix;
    if (st == PKV_OK) st = fetch(kv_indptr, pl->B + 1, &ip);
    if (st == PKV_OK) st = pkv::check_step_indptr(*pl, ip.data());
    if (st != PKV_OK) return st;
    const int64_t n = (int64_t)ip[pl->B] - ip[0];
    if (n > 0 && kv_indices) {
        if ((st = fetch(kv_indices + ip[0], n, &ix)) != PKV_OK) return st;
        if ((st = pkv::check_slots(ix.data(), n, pool->num_slots)) != PKV_OK) return st;
    }
    if (with_prefix && pl->path != PKV_PATH_PAGED && pl->prefix_tokens > 0) {
        if ((int64_t)ix.size() < pl->prefix_tokens) return PKV_EINVAL;
        st = pkv::check_prefix_slots(*pl, ix.data(), pool->num_slots);
    }
    return st;
} catch (const std::bad_alloc&) {
    return PKV_ENOMEM;
}

// Page-table steps: kv_indptr as planned, enough pages per request, and
// every page the kernel reads in the pool.
pkv_status checked_pages(const pkv_plan* pl, const pkv_pool* pool, const int32_t* kv_indptr,
                         const int32_t* page_indptr, const int32_t* page_indices, hipStream_t s) try {
    pkv_status st = sync(s);
    std::vector<int32_t> ip, pp, pages;
    if (st == PKV_OK) st = fetch(kv_indptr, pl->B + 1, &ip);
    if (st == PKV_OK) st = pkv::check_step_indptr(*pl, ip.data());
    if (st == PKV_OK) st = fetch(page_indptr, pl->B + 1, &pp);
    int64_t lo = 0, hi = 0;
    if (st == PKV_OK) st = pkv::check_page_indptr(*pl, pp.data(), &lo, &hi);
    if (st != PKV_OK || hi <= lo) return st;
    if ((st = fetch(page_indices + lo, hi - lo, &pages)) != PKV_OK) return st;
    return pkv::check_slots(pages.data(), hi - lo, pool->num_slots / pl->page_size);
} catch (const std::bad_alloc&) {
    return PKV_ENOMEM;
}

// The prefix pass alone: its prefix_tokens slots.
pkv_status checked_prefix(const pkv_plan* pl, const pkv_pool* pool, const int32_t* prefix_indices,
                          hipStream_t s) try {
    pkv_status st = sync(s);
    std::vector<int32_t> px;
    if (st == PKV_OK) st = fetch(prefix_indices, pl->prefix_tokens, &px);
    if (st == PKV_OK) st = pkv::check_prefix_slots(*pl, px.data(), pool->num_slots);
    return st;
} catch (const std::bad_alloc&) {
    return PKV_ENOMEM;
}

// Grouped steps: the metadata block as planned, its slots in the pool.
pkv_status checked_grouped(const pkv_plan* pl, const pkv_pool* pool, const int32_t* meta, hipStream_t s) try {
    pkv_status st = sync(s);
    std::vector<int32_t> m;
    if (st == PKV_OK) st = fetch(meta, (int64_t)pl->meta.size(), &m);
    if (st == PKV_OK) st = pkv::check_group_metadata(*pl, m.data(), pool->num_slots);
    return st;
} catch (const std::bad_alloc&) {
    return PKV_ENOMEM;
}
#endif

// Workspace of pkv_decode_step_noalloc, for callers that cannot allocate:
// a fixed array in device memory, one copy per GPU the library runs on,
// held until the process ends.  In host code `scratch` names only a
// host-side stand-in; its device address on the current GPU is taken once
// per device with hipGetSymbolAddress and kept in g_scratch, and only that
// address is ever handed to a kernel.  No part of it needs clearing: the
// kernels write every partial state before the combine reads it.
__device__ __align__(256) static unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch;

hipError_t device_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        it = g_scratch.emplace(dev, p).first;
    }
    *out = it->second;
    return hipSuccess;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_decode_attn(const pkv_plan* pl, const void* q, const pkv_pool* pool,
                                 const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale,
                                 void* o, float* o_f32, float* lse, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (!pl || pl->grouped) return PKV_EINVAL;
    if (!o && !o_f32) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    st = check_workspace(pl, ws, ws_bytes);
    if (st != PKV_OK) return st;
    if (pl->B == 0) return PKV_OK;
    if (!q || !kv_indptr || (pl->paged_tokens > 0 && !kv_indices)) return PKV_EINVAL;
#if PKV_CHECKED
    st = checked_flat(pl, pool, kv_indptr, kv_indices, false, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    return run_paged(pl, q, pool, kv_indptr, kv_indices, sm_scale, o, o_f32, lse, ws,
                     static_cast<hipStream_t>(stream));
}

pkv_status pkv_paged_decode_attn_pages(const pkv_plan* pl, const void* q, const pkv_pool* pool,
                                       const int32_t* kv_indptr, const int32_t* page_indptr,
                                       const int32_t* page_indices, float sm_scale, void* o, float* o_f32,
                                       float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!pl || pl->grouped) return PKV_EINVAL;
    if (!o && !o_f32) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    st = check_workspace(pl, ws, ws_bytes);
    if (st != PKV_OK) return st;
    if (pl->B == 0) return PKV_OK;
    if (!q || !kv_indptr || !page_indptr || (pl->paged_tokens > 0 && !page_indices)) return PKV_EINVAL;
#if PKV_CHECKED
    st = checked_pages(pl, pool, kv_indptr, page_indptr, page_indices, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    pkv::PagedArgs a = paged_args(pl, q, pool, kv_indptr, nullptr, sm_scale);
    a.page_indptr = page_indptr;
    a.page_indices = page_indices;
    a.page_size = pl->page_size;
    return run_paged_args(pl, a, o, o_f32, lse, ws, static_cast<hipStream_t>(stream));
}

pkv_status pkv_cascade_prefix_attn(const pkv_plan* pl, const void* q, const pkv_pool* pool,
                                   const int32_t* prefix_indices, int32_t prefix_len, float sm_scale,
                                   float* o_p, float* lse_p, void* ws, size_t ws_bytes, void* stream) {
    if (!pl || pl->grouped) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    if (pl->path == PKV_PATH_PAGED) return PKV_EINVAL;
    if (prefix_len != pl->prefix_tokens) return PKV_EINVAL;
    if (!q || !prefix_indices || !o_p || !lse_p) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    st = check_workspace(pl, ws, ws_bytes);
    if (st != PKV_OK) return st;
#if PKV_CHECKED
    st = checked_prefix(pl, pool, prefix_indices, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    return run_prefix(pl, q, pool, prefix_indices, sm_scale, o_p, lse_p, ws,
                      static_cast<hipStream_t>(stream));
}

pkv_status pkv_merge_states(int32_t rows, int32_t head_dim, const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b, void* o_out, int32_t out_dtype,
                            float* lse_out, void* stream) {
    if (rows < 0 || (head_dim != 64 && head_dim != 128)) return PKV_EINVAL;
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) return PKV_EUNSUPPORTED;
    if (rows == 0) return PKV_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o_out) return PKV_EINVAL;
    return hip_status(pkv::launch_merge_states(rows, head_dim, o_a, lse_a, o_b, lse_b, o_out, out_dtype,
                                               lse_out, static_cast<hipStream_t>(stream)));
}

pkv_status pkv_decode_step(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* kv_indptr,
                           const int32_t* kv_indices, float sm_scale, void* o, float* lse, void* ws,
                           size_t ws_bytes, void* stream) {
    if (!pl || !o) return PKV_EINVAL;
    if (pl->grouped) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    st = check_workspace(pl, ws, ws_bytes);
    if (st != PKV_OK) return st;
    if (pl->B == 0) return PKV_OK;
    if (!q || !kv_indptr || !kv_indices) return PKV_EINVAL;
#if PKV_CHECKED
    st = checked_flat(pl, pool, kv_indptr, kv_indices, true, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    return run_decode_step(pl, q, pool, kv_indptr, kv_indices, sm_scale, o, lse, ws, static_cast<hipStream_t>(stream),
                           pl->concurrent_prefix != 0);
}

pkv_status pkv_decode_step_noalloc(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* kv_indptr,
                                   const int32_t* kv_indices, float sm_scale, void* o, float* lse, void* stream) {
    if (!pl || !o) return PKV_EINVAL;
    if (pl->grouped) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    if (pl->workspace_bytes > (int64_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_EWORKSPACE;
    if (pl->B == 0) return PKV_OK;
    if (!q || !kv_indptr || !kv_indices) return PKV_EINVAL;
#if PKV_CHECKED
    st = checked_flat(pl, pool, kv_indptr, kv_indices, true, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    void* ws = nullptr;
    if (pl->workspace_bytes > 0 && device_scratch(&ws) != hipSuccess) return PKV_EHIP;
    // one stream: the side stream of concurrent_prefix would be created here
    return run_decode_step(pl, q, pool, kv_indptr, kv_indices, sm_scale, o, lse, ws, static_cast<hipStream_t>(stream),
                           false);
}

pkv_status pkv_decode_step_grouped(const pkv_plan* pl, const void* q, const pkv_pool* pool, const int32_t* meta,
                                   float sm_scale, void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!pl || !o || !pl->grouped) return PKV_EINVAL;
    if (!scale_ok(sm_scale)) return PKV_EINVAL;
    pkv_status st = check_pool(pl, pool);
    if (st != PKV_OK) return st;
    st = check_workspace(pl, ws, ws_bytes);
    if (st != PKV_OK) return st;
    if (pl->B == 0) return PKV_OK;
    if (!q || !meta) return PKV_EINVAL;
#if PKV_CHECKED
    st = checked_grouped(pl, pool, meta, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) return st;
#endif
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t* suffix_indptr = meta + pl->meta_suffix_indptr;
    const int32_t* suffix_indices = meta + pl->meta_suffix_indices;
    pkv::PagedArgs sa = paged_args(pl, q, pool, suffix_indptr, suffix_indices, sm_scale);
    sa.token_offset = 0;
    if (pl->num_groups == 0) {
        // no shared prefix anywhere: a plain paged step over every token
        return run_paged_args(pl, sa, o, nullptr, lse, ws, s);
    }
    // Prefix pass: items of the DENSE groups, then of the CASCADE groups,
    // each set in one launch; partial states per (request, range).
    pkv::PrefixArgs pa{};
    pa.q = q;
    pa.k = pool->k;
    pa.v = pool->v;
    pa.kv_dtype = pl->kv_dtype;
    pa.k_scale = pool->k_scale;
    pa.v_scale = pool->v_scale;
    pa.prefix_indices = meta + pl->meta_prefix_indices;
    pa.prefix_base = -1;  // each group's own placement is in the group table
    pa.B = pl->B;
    pa.H_kv = pl->H_kv;
    pa.G = pl->G;
    pa.D = pl->D;
    pa.num_splits = pl->prefix_splits;
    pa.scale_log2 = sm_scale * kLog2e;
    pa.part_acc = ws_at<float>(ws, pl->ws_prefix_acc);
    pa.part_ml = ws_at<float>(ws, pl->ws_prefix_ml);
    pa.force_partial = 1;
    pa.groups = meta + pl->meta_desc;
    pa.members = meta + pl->meta_members;
    pa.num_groups = pl->num_groups;
    pa.item_base = 0;
    pa.num_items = pl->dense_items;
    sa.part_acc = ws_at<float>(ws, pl->ws_paged_acc);
    sa.part_ml = ws_at<float>(ws, pl->ws_paged_ml);
    sa.force_partial = 1;
    if (pl->fuse_cascade) {
        // every group DENSE: prefix items and suffix chunks in one launch
        if (pkv::launch_cascade_fused(*pl, pa, sa, s) != hipSuccess) return PKV_EHIP;
    } else {
        if (pl->dense_items > 0 && pkv::launch_prefix_attn(pa, pkv::kDenseRowsPerWg, s) != hipSuccess)
            return PKV_EHIP;
        pa.item_base = pl->dense_items;
        pa.num_items = pl->tiled_items;
        if (pl->tiled_items > 0 && pkv::launch_prefix_attn(pa, pkv::kTiledRowsPerWg, s) != hipSuccess)
            return PKV_EHIP;
        // suffix pass
        if (pl->num_chunks > 0 && pkv::launch_paged_split(*pl, sa, s) != hipSuccess) return PKV_EHIP;
    }
    // the combine of each row's prefix ranges (its group's count) and
    // suffix chunks
    pkv::SplitReduceArgs r = chunk_reduce_args(pl, sa);
    r.pre_acc = pa.part_acc;
    r.pre_ml = pa.part_ml;
    r.pre_splits = pl->prefix_splits;
    r.pre_count = meta + pl->meta_pre_count;
    r.o = o;
    r.lse = lse;
    return hip_status(pkv::launch_split_reduce(r, s));
}

}  // extern "C"
