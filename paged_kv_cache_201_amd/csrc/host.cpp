// Host half of the library: status strings, page-table lowering, index
// validation and the per-step planner.  Plain C++17, no device code, so it
// also builds and runs without a GPU.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t dtype_bytes(int32_t dt) {
    switch (dt) {
        case PKV_F32: return 4;
        case PKV_BF16: return 2;
        case PKV_FP8_E4M3: return 1;
        default: return 0;
    }
}

bool dtype_pair_supported(int32_t q, int32_t kv) {
    return (q == PKV_F32 && kv == PKV_F32) || (q == PKV_BF16 && kv == PKV_BF16) ||
           (q == PKV_BF16 && kv == PKV_FP8_E4M3);
}

// The prefix kernels run bf16 MFMA: bf16 queries over bf16 K/V.
bool prefix_pair_supported(int32_t q, int32_t kv) { return q == PKV_BF16 && kv == PKV_BF16; }

bool group_supported(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

}  // namespace

namespace pkv {

bool paged_geometry(int32_t kv_dtype, int32_t head_dim, int32_t group, int32_t num_kv_heads, int32_t max_heads,
                    PagedGeometry* out) {
    if (head_dim != 64 && head_dim != 128) return false;
    if (!group_supported(group) || num_kv_heads < 1) return false;
    int32_t epl;
    switch (kv_dtype) {
        case PKV_F32: epl = 4; break;        // 16-byte loads
        case PKV_BF16: epl = 8; break;       // 16-byte loads
        case PKV_FP8_E4M3: epl = 8; break;   // 8-byte loads
        default: return false;
    }
    const int32_t lph = head_dim / epl;
    const int32_t rs = 64 / lph;
    // One head slot per lane (measured faster than two on every workload):
    // a wave-wide load covers RS rows, one token's RS heads, or TPI tokens of
    // fewer heads when the head count or max_heads calls for it.
    const auto allowed = [&](int32_t hb) { return max_heads <= 0 || hb <= max_heads; };
    if (num_kv_heads % rs == 0 && allowed(rs)) {
        *out = PagedGeometry{epl, lph, rs, 1, 1, rs};
        return true;
    }
    for (int32_t hb = rs / 2; hb >= 1; hb /= 2) {
        if (num_kv_heads % hb == 0 && allowed(hb)) {
            *out = PagedGeometry{epl, lph, rs, 1, rs / hb, hb};
            return true;
        }
    }
    return false;
}

}  // namespace pkv

extern "C" {

const char* pkv_status_string(int32_t status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_EINVAL: return "invalid argument";
        case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
        case PKV_EWORKSPACE: return "workspace missing or too small";
        case PKV_ERANGE: return "index or length out of range";
        case PKV_EHIP: return "HIP error";
        case PKV_ENOMEM: return "out of host memory";
        default: return "unknown status";
    }
}

const char* pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

void pkv_tuning_defaults(pkv_tuning* out) {
    if (!out) return;
    // Dispatcher constants refitted on MI355X from a forced-path sweep over
    // B in {1..512}, G in {1,2,4,8}, P in {256..8192}, suffixes U{64..512}:
    // DENSE (with its fused launch) was never slower than the tiled path by
    // more than noise at any M_eff, so every cascade step goes DENSE; the
    // PAGED gate with R = 3 and a 10 MB launch term picks a path within 15 %
    // of the fastest in every cell (0.6 % on average).
    out->t_dense = 1;
    out->gate_ratio = 3;
    out->launch_bytes = 10LL * 1000 * 1000;
    out->target_workgroups = 512;   // two workgroups per CU
    out->min_split_tokens = 64;
    out->concurrent_prefix = 0;  // measured: overlap with the suffix pass does not shorten the step
    out->fuse_cascade = 12;  // MFMA flops per suffix byte: fused on c3 (57), separate on c4 (3)
    out->prefix_target_workgroups = 256;
    out->min_prefix_split_tokens = 64;
    out->max_heads_per_item = 0;
}

pkv_status pkv_lower_page_table(int32_t batch, int32_t page_size, const int32_t* page_indptr,
                                const int32_t* page_indices, const int32_t* seq_lens,
                                int32_t* kv_indptr_out, int32_t* kv_indices_out,
                                int64_t kv_indices_capacity) {
    if (batch < 0 || page_size < 1) return PKV_EINVAL;
    if (!page_indptr || !seq_lens || !kv_indptr_out) return PKV_EINVAL;
    if (page_indptr[0] != 0) return PKV_EINVAL;
    int64_t total = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t n = (int64_t)page_indptr[b + 1] - page_indptr[b];
        const int64_t L = seq_lens[b];
        if (n < 0 || L < 0) return PKV_EINVAL;
        if (n != ceil_div(L, page_size)) return PKV_ERANGE;
        if (n > 0 && !page_indices) return PKV_EINVAL;
        int32_t lo = INT32_MAX, hi = 0;
        const int32_t* pages = page_indices + page_indptr[b];
        for (int64_t j = 0; j < n; ++j) {
            lo = std::min(lo, pages[j]);
            hi = std::max(hi, pages[j]);
        }
        if (n > 0 && (lo < 0 || (int64_t)hi * page_size + (page_size - 1) > INT32_MAX)) return PKV_ERANGE;
        total += L;
    }
    if (total > INT32_MAX || total > kv_indices_capacity) return PKV_ERANGE;
    if (total > 0 && !kv_indices_out) return PKV_EINVAL;
    int64_t pos = 0;
    kv_indptr_out[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int32_t* pages = page_indices + page_indptr[b];
        const int32_t L = seq_lens[b];
        if (page_size == 1) {  // one token per page: the slots are the pages
            std::memcpy(kv_indices_out + pos, pages, (size_t)L * sizeof(int32_t));
            pos += L;
            kv_indptr_out[b + 1] = (int32_t)pos;
            continue;
        }
        // page by page: slots page*p .. page*p + (tokens on that page) - 1
        for (int32_t t0 = 0, j = 0; t0 < L; t0 += page_size, ++j) {
            const int32_t base = pages[j] * page_size;
            const int32_t cnt = std::min(page_size, L - t0);
            int32_t* dst = kv_indices_out + pos;
            for (int32_t i = 0; i < cnt; ++i) dst[i] = base + i;
            pos += cnt;
        }
        kv_indptr_out[b + 1] = (int32_t)pos;
    }
    return PKV_OK;
}

pkv_status pkv_validate_indices(const int32_t* kv_indptr, const int32_t* kv_indices, int32_t batch,
                                int64_t num_slots) {
    if (batch < 0 || !kv_indptr) return PKV_EINVAL;
    if (kv_indptr[0] != 0) return PKV_EINVAL;
    for (int32_t b = 0; b < batch; ++b)
        if (kv_indptr[b + 1] < kv_indptr[b]) return PKV_EINVAL;
    const int64_t n = kv_indptr[batch];
    if (n > 0 && !kv_indices) return PKV_EINVAL;
    for (int64_t i = 0; i < n; ++i)
        if (kv_indices[i] < 0 || kv_indices[i] >= num_slots) return PKV_ERANGE;
    return PKV_OK;
}

pkv_status pkv_plan_create(const pkv_problem* pr, const pkv_tuning* tuning, pkv_plan** out) {
    if (!pr || !out) return PKV_EINVAL;
    pkv_tuning tu;
    if (tuning) {
        tu = *tuning;
    } else {
        pkv_tuning_defaults(&tu);
    }
    if (tu.t_dense < 1 || tu.gate_ratio < 0 || tu.launch_bytes < 0 || tu.target_workgroups < 1 ||
        tu.min_split_tokens < 1 ||
        tu.concurrent_prefix < 0 || tu.concurrent_prefix > 1 || tu.fuse_cascade < 0 ||
        tu.prefix_target_workgroups < 1 ||
        tu.min_prefix_split_tokens < 1 || tu.max_heads_per_item < 0)
        return PKV_EINVAL;

    // Checks, in the same order as the planner's reference statement.
    const int32_t B = pr->batch, H_q = pr->num_q_heads, H_kv = pr->num_kv_heads;
    const int32_t D = pr->head_dim, p = pr->page_size;
    if (B < 0 || H_kv < 1 || H_q < 1 || p < 1 || D < 1) return PKV_EINVAL;
    if (H_q % H_kv) return PKV_EINVAL;
    if (B > 0 && !pr->kv_indptr) return PKV_EINVAL;
    int64_t min_len = INT64_MAX, max_len = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t L = (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b];
        if (L < 0) return PKV_EINVAL;
        min_len = std::min(min_len, L);
        max_len = std::max(max_len, L);
    }
    if (B > 0 && pr->kv_indptr[0] < 0) return PKV_EINVAL;
    const int32_t P = pr->shared_prefix_len;
    if (P < 0 || (B > 0 && P > min_len)) return PKV_EINVAL;
    if (pr->force_path < -1 || pr->force_path > 2) return PKV_EINVAL;
    const int32_t G = H_q / H_kv;
    if ((D != 64 && D != 128) || !dtype_pair_supported(pr->q_dtype, pr->kv_dtype) ||
        !group_supported(G))
        return PKV_EUNSUPPORTED;
    pkv::PagedGeometry geo;
    if (!pkv::paged_geometry(pr->kv_dtype, D, G, H_kv, tu.max_heads_per_item, &geo)) return PKV_EUNSUPPORTED;

    // Path choice.
    const int64_t n_shared = P > 0 ? B : 0;
    const int64_t shared_pages = n_shared ? P / p : 0;
    int64_t prefix_tokens = shared_pages * p;
    const int64_t m_eff = (int64_t)B * G;
    const bool capable = prefix_pair_supported(pr->q_dtype, pr->kv_dtype);
    int32_t path;
    if (pr->force_path >= 0) {
        path = pr->force_path;
        if (path != PKV_PATH_PAGED) {
            if (!capable) return PKV_EUNSUPPORTED;
            if (prefix_tokens == 0) return PKV_EINVAL;
        }
    } else if (!capable || n_shared < 2 || shared_pages == 0) {
        path = PKV_PATH_PAGED;
    } else {
        const int64_t rows = (int64_t)B * H_q;
        const int64_t kv_bytes = 2LL * dtype_bytes(pr->kv_dtype);
        const int64_t saved = (n_shared - 1) * prefix_tokens * H_kv * D * kv_bytes;
        const int64_t overhead = 4 * rows * (D + 1) * 4 + tu.launch_bytes;
        if (saved < (int64_t)tu.gate_ratio * overhead)
            path = PKV_PATH_PAGED;
        else if (m_eff >= tu.t_dense)
            path = PKV_PATH_DENSE;
        else
            path = PKV_PATH_CASCADE;
    }
    if (path == PKV_PATH_PAGED) prefix_tokens = 0;
    if (m_eff > INT32_MAX) return PKV_EUNSUPPORTED;

    pkv_plan* pl = new (std::nothrow) pkv_plan;
    if (!pl) return PKV_ENOMEM;
    std::memset(pl, 0, sizeof(*pl));
    pl->B = B;
    pl->H_q = H_q;
    pl->H_kv = H_kv;
    pl->D = D;
    pl->G = G;
    pl->q_dtype = pr->q_dtype;
    pl->kv_dtype = pr->kv_dtype;
    pl->page_size = p;
    pl->indptr0 = B > 0 ? pr->kv_indptr[0] : 0;
    pl->prefix_len = P;
    pl->path = path;
    pl->m_eff = (int32_t)m_eff;
    pl->shared_pages = (int32_t)shared_pages;
    pl->prefix_tokens = (int32_t)prefix_tokens;
    pl->geo = geo;
    pl->head_blocks = H_kv / geo.hb;
    pl->concurrent_prefix = tu.concurrent_prefix;
    pl->fuse_cascade = tu.fuse_cascade && path == PKV_PATH_DENSE;

    // Prefix pass: M_eff query rows per KV head in tiles, the prefix cut into
    // ranges so that the grid fills the GPU.
    pl->prefix_rows_per_wg = path == PKV_PATH_DENSE ? pkv::kDenseRowsPerWg : pkv::kTiledRowsPerWg;
    pl->prefix_split_tokens = 0;
    pl->prefix_splits = 0;
    if (path != PKV_PATH_PAGED) {
        const int64_t tiles = (int64_t)H_kv * ceil_div(m_eff, pl->prefix_rows_per_wg);
        const int64_t want = std::max<int64_t>(1, ceil_div(tu.prefix_target_workgroups, tiles));
        int64_t ps = align_up(ceil_div(prefix_tokens, want), pkv::kPrefixTokenQuantum);
        ps = std::max<int64_t>(ps, align_up(tu.min_prefix_split_tokens, pkv::kPrefixTokenQuantum));
        ps = std::min<int64_t>(ps, pkv::kMaxPrefixSplitTokens);
        pl->prefix_split_tokens = (int32_t)ps;
        pl->prefix_splits = (int32_t)ceil_div(prefix_tokens, ps);
    }
    // Workgroups of the prefix pass (a multiple of 8 for the XCD placement).
    const int64_t prefix_wgs =
        pl->prefix_splits ? align_up((int64_t)H_kv * ceil_div(m_eff, pl->prefix_rows_per_wg) * pl->prefix_splits, 8)
                          : 0;

    // Paged pass: the attended positions [prefix_tokens, L_b) of all
    // requests, request after request, form one flat sequence that is cut
    // into equal chunks, one workgroup per (chunk, head block).
    int64_t total = 0;
    bool any_empty = false;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t n = (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b] - prefix_tokens;
        total += n;
        any_empty |= n == 0;
    }
    pl->paged_tokens = total;
    // One launch runs both passes of a DENSE step when the prefix pass is
    // heavy enough to hide suffix streaming under it and its items take at
    // most half of the workgroup slots; the suffix chunks then fill the rest.
    if (pl->fuse_cascade) {
        const int64_t prefix_flops = 4 * m_eff * prefix_tokens * D * H_kv;
        const int64_t suffix_bytes = total * H_kv * D * 2 * dtype_bytes(pr->kv_dtype);
        if (2 * prefix_wgs > tu.target_workgroups || prefix_flops < (int64_t)tu.fuse_cascade * suffix_bytes)
            pl->fuse_cascade = 0;
    }
    int64_t target = tu.target_workgroups;
    if (pl->fuse_cascade) target -= prefix_wgs;
    const int64_t per_item = ceil_div(total * pl->head_blocks, target);
    int64_t chunk = std::max<int64_t>(tu.min_split_tokens, per_item);
    chunk = align_up(chunk, pkv::kSplitQuantum);
    chunk = std::min<int64_t>(chunk, pkv::max_chunk_tokens(geo.rs, geo.nhl, geo.tpi, G, D));
    pl->split_tokens = (int32_t)chunk;
    pl->num_chunks = ceil_div(total, chunk);
    pl->num_work_items = pl->num_chunks * pl->head_blocks;
    // Partial states per request: the chunks its range touches.
    int64_t pos = 0, max_parts = 1;
    bool spans = false;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t n = (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b] - prefix_tokens;
        if (n > 0) {
            const int64_t parts = (pos + n - 1) / chunk - pos / chunk + 1;
            max_parts = std::max(max_parts, parts);
            spans |= parts > 1;
        }
        pos += n;
    }
    pl->num_splits = (int32_t)max_parts;
    // A combine kernel follows the paged pass for a cascade step, when a
    // request spans chunks, or to write the output of empty requests.
    pl->needs_reduce = path != PKV_PATH_PAGED || spans || any_empty;

    // Workspace layout.
    int64_t off = 0;
    const int64_t rows = (int64_t)B * H_q;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = align_up(off + bytes, kAlign);
        return at;
    };
    pl->ws_paged_acc = pl->ws_paged_ml = -1;
    pl->ws_prefix_acc = pl->ws_prefix_ml = -1;
    // A cascade step keeps both passes as partial states (prefix ranges, then
    // suffix chunks) that one kernel combines; a request inside one chunk of
    // a paged pass has its output written directly.
    if (spans || path != PKV_PATH_PAGED) {
        pl->ws_paged_acc = take(rows * pl->num_splits * D * 4);
        pl->ws_paged_ml = take(rows * pl->num_splits * 2 * 4);
    }
    if (path != PKV_PATH_PAGED) {
        pl->ws_prefix_acc = take(rows * pl->prefix_splits * D * 4);
        pl->ws_prefix_ml = take(rows * pl->prefix_splits * 2 * 4);
    }
    pl->workspace_bytes = off;
    *out = pl;
    return PKV_OK;
}

pkv_status pkv_plan_get_info(const pkv_plan* pl, pkv_plan_info* info) {
    if (!pl || !info) return PKV_EINVAL;
    info->path = pl->path;
    info->m_eff = pl->m_eff;
    info->shared_pages = pl->shared_pages;
    info->prefix_tokens = pl->prefix_tokens;
    info->split_tokens = pl->split_tokens;
    info->num_splits = pl->num_splits;
    info->heads_per_item = pl->geo.hb;
    info->prefix_splits = pl->prefix_splits;
    info->num_work_items = pl->num_work_items;
    info->workspace_bytes = pl->workspace_bytes;
    return PKV_OK;
}

void pkv_plan_destroy(pkv_plan* pl) { delete pl; }

}  // extern "C"
