// Host half of the library: status strings, page-table lowering, index
// validation and the per-step planner.  Plain C++17, no device code, so it
// also builds and runs without a GPU.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

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

// The prefix kernels run bf16 MFMA: bf16 queries over bf16 K/V, or over fp8
// e4m3 K/V widened in LDS (head_dim 128).
bool prefix_pair_supported(int32_t q, int32_t kv, int32_t d) {
    return q == PKV_BF16 && (kv == PKV_BF16 || (kv == PKV_FP8_E4M3 && d == 128));
}

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

namespace {

// Checks shared by both planners: tuning ranges, sizes, head counts.
pkv_status check_problem(const pkv_problem* pr, const pkv_tuning* tuning, pkv_tuning* tu) {
    if (tuning) {
        *tu = *tuning;
    } else {
        pkv_tuning_defaults(tu);
    }
    if (tu->t_dense < 1 || tu->gate_ratio < 0 || tu->launch_bytes < 0 || tu->target_workgroups < 1 ||
        tu->min_split_tokens < 1 || tu->concurrent_prefix < 0 || tu->concurrent_prefix > 1 ||
        tu->fuse_cascade < 0 || tu->prefix_target_workgroups < 1 || tu->min_prefix_split_tokens < 1 ||
        tu->max_heads_per_item < 0 || tu->prefix_placement < 0 || tu->prefix_placement > 1 ||
        tu->segment_tokens < 0 || tu->cached_prefix_bytes < 0 || tu->cached_reread_bytes < 0)
        return PKV_EINVAL;
    const int32_t B = pr->batch, H_q = pr->num_q_heads, H_kv = pr->num_kv_heads;
    if (B < 0 || H_kv < 1 || H_q < 1 || pr->page_size < 1 || pr->head_dim < 1) return PKV_EINVAL;
    if (H_q % H_kv) return PKV_EINVAL;
    return PKV_OK;
}

// Shapes and dtypes the kernels are built for.
pkv_status check_support(const pkv_problem* pr, const pkv_tuning& tu, pkv::PagedGeometry* geo) {
    const int32_t G = pr->num_q_heads / pr->num_kv_heads;
    const int32_t D = pr->head_dim;
    if ((D != 64 && D != 128) || !dtype_pair_supported(pr->q_dtype, pr->kv_dtype) || !group_supported(G))
        return PKV_EUNSUPPORTED;
    if (!pkv::paged_geometry(pr->kv_dtype, D, G, pr->num_kv_heads, tu.max_heads_per_item, geo))
        return PKV_EUNSUPPORTED;
    return PKV_OK;
}

// Bytes per stored value as the planner's rules count them: an fp8 value
// counts as 2 (bf16's width), because the fp8 paged pass is bound by the
// vector ALU and a token of it takes about as long as a bf16 token.
int64_t rule_bytes(int32_t kv_dtype) { return kv_dtype == PKV_FP8_E4M3 ? 2 : dtype_bytes(kv_dtype); }

// The dispatcher for n_shared requests on prefix_tokens shared tokens
// (whole pages), rows query rows and M_eff = m_eff, in order: a forced path;
// PAGED without two sharers, a shared page or a prefix kernel for the dtype
// pair; PAGED when the bytes saved are under gate_ratio x the combine's
// state traffic plus the launch term, or, for a prefix whose stored K/V fit
// cached_prefix_bytes, under cached_reread_bytes if that is more (gate_ratio
// 0 turns the whole gate off); DENSE at M_eff >= t_dense; CASCADE.
pkv_status choose_path(const pkv_problem* pr, const pkv_tuning& tu, int64_t n_shared, int64_t prefix_tokens,
                       int64_t rows, int64_t m_eff, int32_t* path) {
    const bool capable = prefix_pair_supported(pr->q_dtype, pr->kv_dtype, pr->head_dim);
    if (pr->force_path >= 0) {
        *path = pr->force_path;
        if (*path != PKV_PATH_PAGED) {
            if (!capable) return PKV_EUNSUPPORTED;
            if (prefix_tokens == 0) return PKV_EINVAL;
        }
        return PKV_OK;
    }
    if (!capable || n_shared < 2 || prefix_tokens == 0) {
        *path = PKV_PATH_PAGED;
        return PKV_OK;
    }
    const int64_t D = pr->head_dim;
    const int64_t kv_bytes = 2LL * rule_bytes(pr->kv_dtype);
    const int64_t saved = (n_shared - 1) * prefix_tokens * pr->num_kv_heads * D * kv_bytes;
    const int64_t overhead = 4 * rows * (D + 1) * 4 + tu.launch_bytes;
    // a prefix small enough to stay in L2 costs its re-readers little
    const int64_t stored = prefix_tokens * pr->num_kv_heads * D * 2 * dtype_bytes(pr->kv_dtype);
    int64_t allowed = (int64_t)tu.gate_ratio * overhead;
    if (tu.gate_ratio > 0 && tu.cached_prefix_bytes > 0 && stored <= tu.cached_prefix_bytes)
        allowed = std::max<int64_t>(allowed, tu.cached_reread_bytes);
    if (saved < allowed)
        *path = PKV_PATH_PAGED;
    else if (m_eff >= tu.t_dense)
        *path = PKV_PATH_DENSE;
    else
        *path = PKV_PATH_CASCADE;
    return PKV_OK;
}

void fill_problem(pkv_plan* pl, const pkv_problem* pr, const pkv_tuning& tu, const pkv::PagedGeometry& geo) {
    pl->B = pr->batch;
    pl->H_q = pr->num_q_heads;
    pl->H_kv = pr->num_kv_heads;
    pl->D = pr->head_dim;
    pl->G = pr->num_q_heads / pr->num_kv_heads;
    pl->q_dtype = pr->q_dtype;
    pl->kv_dtype = pr->kv_dtype;
    pl->page_size = pr->page_size;
    pl->geo = geo;
    pl->head_blocks = pr->num_kv_heads / geo.hb;
    pl->concurrent_prefix = tu.concurrent_prefix;
}

// Prefix ranges for prefix_tokens shared tokens read by `tiles` (query tile,
// KV head) pairs, aiming at `target` workgroups: multiples of the token
// quantum, at least the tuning's minimum, at most what the kernel stages.
void prefix_ranges(const pkv_tuning& tu, int64_t prefix_tokens, int64_t tiles, int64_t target, int32_t* split_tokens,
                   int32_t* splits) {
    const int64_t want = std::max<int64_t>(1, ceil_div(target, tiles));
    int64_t ps = align_up(ceil_div(prefix_tokens, want), pkv::kPrefixTokenQuantum);
    ps = std::max<int64_t>(ps, align_up(tu.min_prefix_split_tokens, pkv::kPrefixTokenQuantum));
    ps = std::min<int64_t>(ps, pkv::kMaxPrefixSplitTokens);
    *split_tokens = (int32_t)ps;
    *splits = (int32_t)ceil_div(prefix_tokens, ps);
}

// Prefix workgroups to aim for when the prefix pass shares one launch with
// the suffix pass: a quarter of the workgroup target (measured: long prefix
// items beside many suffix chunks beat more, shorter items), at most the
// unfused target.
int64_t fused_prefix_target(const pkv_tuning& tu) {
    return std::max<int64_t>(1, std::min<int64_t>(tu.prefix_target_workgroups, tu.target_workgroups / 4));
}

// Workgroups the paged pass over `total` positions aims at: a bf16 or fp32
// pass on its own is bound by HBM and runs best with one workgroup per CU
// (half the tuning's target: measured 2.1 % faster on the Llama layer, 1.4 %
// on the short-prefix step's suffix, neutral on short requests), as long as
// its chunks stay within what one workgroup stages (else the chunk cap would
// leave a few workgroups over one per CU: 27 % slower on long requests); an
// fp8 pass (bound by the vector ALU) keeps two per CU to hide its loads; a
// pass that shares its launch with the prefix items takes what they leave.
// A pass whose positions are mostly re-reads of declared shared pages
// (`reread` of `total`: a shared prefix the gate left on PAGED) is served
// from L2 and keeps two workgroups per CU (one per CU measured 26-34 %
// slower on 8-64 requests over a shared prefix).
int64_t paged_target(const pkv_plan* pl, const pkv_tuning& tu, int64_t total, bool fused, int64_t fused_target,
                     int64_t reread) {
    if (fused) return fused_target;
    if (pl->kv_dtype == PKV_FP8_E4M3 || 2 * reread >= total) return tu.target_workgroups;
    const int64_t half = std::max<int64_t>(1, tu.target_workgroups / 2);
    const int64_t chunk = align_up(std::max<int64_t>(tu.min_split_tokens, ceil_div(total * pl->head_blocks, half)),
                                   pkv::kSplitQuantum);
    const int64_t cap = pkv::max_chunk_tokens(pl->geo.rs, pl->geo.nhl, pl->geo.tpi, pl->G, pl->D);
    return chunk <= cap ? half : tu.target_workgroups;
}

// Lane geometry of the fp8 paged pass when the tuning leaves it open: with
// long requests (at least 1,024 attended positions per non-empty request on
// average) a work item takes half the KV heads a wave-wide load covers,
// two tokens per load, which measured 4.2 % faster on the long-context step
// (G = 8) and 2.7 % at 2,048 tokens (G = 4), and 2.6 % slower on
// short requests.
void fp8_long_geometry(pkv_plan* pl, const pkv_tuning& tu, int64_t tokens, int64_t nonempty) {
    if (pl->kv_dtype != PKV_FP8_E4M3 || tu.max_heads_per_item != 0 || nonempty == 0) return;
    if (tokens < 1024 * nonempty) return;
    pkv::PagedGeometry geo;
    if (pkv::paged_geometry(pl->kv_dtype, pl->D, pl->G, pl->H_kv, pl->geo.rs / 2, &geo)) {
        pl->geo = geo;
        pl->head_blocks = pl->H_kv / geo.hb;
    }
}

// Bins of whole requests for the paged pass: when every request of the pass
// is non-empty and fits a workgroup's index stage, requests are packed, largest
// first (ties by index), each into the least loaded of num_chunks bins (ties
// by bin), with a request's load its positions plus tu.segment_tokens.  The
// bins replace the chunks when their most loaded bin is below the most
// loaded chunk under the same cost (a chunk counts one segment per request
// it touches).  The bin's requests are listed in index order.
template <class LenFn>
bool bin_requests(pkv_plan* pl, const pkv_tuning& tu, LenFn n_of, int64_t chunk) {
    const int64_t W = pl->num_chunks, B = pl->B, seg = tu.segment_tokens;
    if (seg == 0 || W < 2 || W > pkv::kMaxRequestBins || B > pkv::kMaxBinnedRequests) return false;
    const int64_t stage = pkv::max_chunk_tokens(pl->geo.rs, pl->geo.nhl, pl->geo.tpi, pl->G, pl->D);
    std::vector<int64_t> n(B);
    int64_t total = 0, longest = 0;
    for (int64_t b = 0; b < B; ++b) {
        n[b] = n_of((int32_t)b);
        if (n[b] == 0 || n[b] > stage) return false;
        total += n[b];
        longest = std::max(longest, n[b]);
    }
    // most loaded chunk of the flat partition
    std::vector<int64_t> chunk_cost(W, 0);
    int64_t pos = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t c0 = pos / chunk, c1 = (pos + n[b] - 1) / chunk;
        for (int64_t c = c0; c <= c1; ++c) chunk_cost[c] += seg;
        pos += n[b];
    }
    int64_t chunk_max = 0;
    for (int64_t c = 0; c < W; ++c) {
        const int64_t toks = std::min<int64_t>((c + 1) * chunk, total) - c * chunk;
        chunk_max = std::max(chunk_max, chunk_cost[c] + toks);
    }
    // largest first into the least loaded bin
    std::vector<int32_t> order(B);
    for (int64_t b = 0; b < B; ++b) order[b] = (int32_t)b;
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return n[x] > n[y]; });
    using Bin = std::pair<int64_t, int32_t>;  // (load, bin)
    std::priority_queue<Bin, std::vector<Bin>, std::greater<Bin>> heap;
    for (int32_t w = 0; w < (int32_t)W; ++w) heap.push({0, w});
    std::vector<int32_t> bin_of(B);
    int64_t bin_max = 0;
    for (int32_t b : order) {
        Bin top = heap.top();
        heap.pop();
        top.first += n[b] + seg;
        bin_max = std::max(bin_max, top.first);
        bin_of[b] = top.second;
        heap.push(top);
    }
    if (bin_max >= chunk_max) return false;
    pl->bin_start.assign(W + 1, 0);
    for (int64_t b = 0; b < B; ++b) ++pl->bin_start[bin_of[b] + 1];
    for (int64_t w = 0; w < W; ++w) pl->bin_start[w + 1] = (uint16_t)(pl->bin_start[w + 1] + pl->bin_start[w]);
    pl->bin_req.assign(B, 0);
    std::vector<int32_t> fill(pl->bin_start.begin(), pl->bin_start.end() - 1);
    for (int64_t b = 0; b < B; ++b) pl->bin_req[fill[bin_of[b]]++] = (uint16_t)b;
    pl->request_bins = (int32_t)W;
    pl->bin_max_tokens = (int32_t)longest;
    return true;
}

// Paged-pass chunking over `total` positions, n_of(b) of them request b's:
// chunk size from the workgroup target, partial states per request.
template <class LenFn>
void plan_chunks(pkv_plan* pl, const pkv_tuning& tu, int64_t total, int64_t target, LenFn n_of, bool* spans,
                 bool* any_empty) {
    pl->paged_tokens = total;
    const int64_t per_item = ceil_div(total * pl->head_blocks, target);
    int64_t chunk = std::max<int64_t>(tu.min_split_tokens, per_item);
    chunk = align_up(chunk, pkv::kSplitQuantum);
    const int64_t cap = pkv::max_chunk_tokens(pl->geo.rs, pl->geo.nhl, pl->geo.tpi, pl->G, pl->D);
    if (chunk > cap) {
        // Capped chunks give more work items than the target: take whole
        // multiples of the target instead, so that no wave runs a remnant
        // (the PAGED leg of a 256 x 4,382-position step: 548 items 777 us,
        // 1,024 items 544 us)
        const int64_t items = ceil_div(total, cap) * pl->head_blocks;
        const int64_t waves = ceil_div(items, target);
        chunk = align_up(ceil_div(total * pl->head_blocks, waves * target), pkv::kSplitQuantum);
        chunk = std::min(std::max<int64_t>(chunk, tu.min_split_tokens), cap);
    }
    pl->split_tokens = (int32_t)chunk;
    pl->num_chunks = ceil_div(total, chunk);
    pl->num_work_items = pl->num_chunks * pl->head_blocks;
    // Partial states per request: the chunks its range touches.
    int64_t pos = 0, max_parts = 1;
    *spans = *any_empty = false;
    for (int32_t b = 0; b < pl->B; ++b) {
        const int64_t n = n_of(b);
        if (n > 0) {
            const int64_t parts = (pos + n - 1) / chunk - pos / chunk + 1;
            max_parts = std::max(max_parts, parts);
            *spans |= parts > 1;
        }
        *any_empty |= n == 0;
        pos += n;
    }
    pl->num_splits = (int32_t)max_parts;
    pl->request_bins = 0;
    pl->bin_start.clear();
    pl->bin_req.clear();
    if (bin_requests(pl, tu, n_of, chunk)) {
        pl->num_splits = 1;
        *spans = false;
    }
}

// Workspace: chunk partials of the paged pass (if kept) and prefix_splits
// prefix partials per row, 256-byte aligned.
void layout_workspace(pkv_plan* pl, bool paged_partials, int32_t prefix_splits) {
    int64_t off = 0;
    const int64_t rows = (int64_t)pl->B * pl->H_q;
    auto take = [&](int64_t bytes) {
        const int64_t at = off;
        off = align_up(off + bytes, kAlign);
        return at;
    };
    pl->ws_paged_acc = pl->ws_paged_ml = -1;
    pl->ws_prefix_acc = pl->ws_prefix_ml = -1;
    if (paged_partials) {
        pl->ws_paged_acc = take(rows * pl->num_splits * pl->D * 4);
        pl->ws_paged_ml = take(rows * pl->num_splits * 2 * 4);
    }
    if (prefix_splits > 0) {
        pl->ws_prefix_acc = take(rows * prefix_splits * pl->D * 4);
        pl->ws_prefix_ml = take(rows * prefix_splits * 2 * 4);
    }
    pl->workspace_bytes = off;
}

}  // namespace

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
    // Dispatcher constants refitted on MI355X from a forced-path sweep (B in
    // {1, 2, 4, 16, 64, 256, 512} x G in {1, 4, 8} x P in {256, 1024, 4096},
    // bf16 and fp8, suffixes U{64..512}, every path timed) and a replay of
    // this planner over candidate constants against the measured times:
    // DENSE (with its fused launch) is never slower than the tiled path by
    // more than noise at any M_eff, so every cascade step goes DENSE; the
    // PAGED gate with R = 3 and a 5 MB launch term picks a path within 19 %
    // of the fastest in every cell, 0.9 % on average (a 10 MB term kept two
    // requests on a 4,096-token prefix PAGED, 1.45x slower than DENSE).
    out->t_dense = 1;
    out->gate_ratio = 3;
    out->launch_bytes = 5LL * 1000 * 1000;
    out->target_workgroups = 512;   // two workgroups per CU
    out->min_split_tokens = 64;
    // measured: the prefix pass on a side stream shortens the short-prefix step by 1-2 % and
    // lengthens others by 2-12 % (a small long-context step most)
    out->concurrent_prefix = 0;
    out->fuse_cascade = 12;  // MFMA flops per suffix byte: fused on c3 (57), separate on c4 (3)
    out->prefix_target_workgroups = 256;
    out->min_prefix_split_tokens = 64;
    out->max_heads_per_item = 0;
    out->prefix_placement = 1;
    // a request segment costs about 2.5 us on the workgroup that sets the end of a
    // 2,560-position chunk, 30 positions' worth; as many segments per workgroup
    // measured the same whatever their lengths
    out->segment_tokens = 32;
    // forced-path sweep (B x G x P, bf16 and fp8): PAGED over shared pages beat
    // the prefix paths with 64 requests over a 256-token prefix (1 MB bf16,
    // 0.84-0.92 of the best prefix path) and with 16 requests over a 1,024-token
    // fp8 prefix (2 MB, 0.77-1.01), and lost at four times those re-reads
    // (1.05-1.59): re-reads of a prefix within half of one XCD's 4 MB L2 come
    // from L2; the re-read allowance sits between the two (66 MB and 264 MB)
    out->cached_prefix_bytes = 2 << 20;
    out->cached_reread_bytes = 128 << 20;
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

namespace {
pkv_status plan_single(const pkv_problem* pr, const pkv_tuning* tuning, pkv_plan** out);
}  // namespace

pkv_status pkv_plan_create(const pkv_problem* pr, const pkv_tuning* tuning, pkv_plan** out) {
    // host containers may throw; nothing may cross the C boundary
    try {
        return plan_single(pr, tuning, out);
    } catch (const std::bad_alloc&) {
        return PKV_ENOMEM;
    }
}

namespace {
pkv_status plan_single(const pkv_problem* pr, const pkv_tuning* tuning, pkv_plan** out) {
    if (!pr || !out) return PKV_EINVAL;
    pkv_tuning tu;
    pkv::PagedGeometry geo;
    pkv_status st = check_problem(pr, tuning, &tu);
    if (st != PKV_OK) return st;
    const int32_t B = pr->batch, H_q = pr->num_q_heads, H_kv = pr->num_kv_heads;
    const int32_t D = pr->head_dim, p = pr->page_size;
    if (B > 0 && !pr->kv_indptr) return PKV_EINVAL;
    int64_t min_len = INT64_MAX;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t L = (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b];
        if (L < 0) return PKV_EINVAL;
        min_len = std::min(min_len, L);
    }
    if (B > 0 && pr->kv_indptr[0] < 0) return PKV_EINVAL;
    const int32_t P = pr->shared_prefix_len;
    if (P < 0 || (B > 0 && P > min_len)) return PKV_EINVAL;
    if (pr->force_path < -1 || pr->force_path > 2) return PKV_EINVAL;
    st = check_support(pr, tu, &geo);
    if (st != PKV_OK) return st;
    const int32_t G = H_q / H_kv;

    // Path choice.
    const int64_t n_shared = P > 0 ? B : 0;
    const int64_t shared_pages = n_shared ? P / p : 0;
    int64_t prefix_tokens = shared_pages * p;
    const int64_t m_eff = (int64_t)B * G;
    // The cached-prefix allowance applies where the DENSE step would not
    // fuse (the fuse rule's flops-per-byte test below): a fused launch hides
    // the prefix pass under the suffix streaming, which PAGED re-reads would
    // lengthen instead.
    pkv_tuning path_tu = tu;
    if (tu.fuse_cascade > 0 && prefix_tokens > 0) {
        int64_t suffix = 0;
        for (int32_t b = 0; b < B; ++b) suffix += (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b] - prefix_tokens;
        const int64_t prefix_flops = 4 * m_eff * prefix_tokens * D * H_kv;
        const int64_t suffix_bytes = suffix * H_kv * D * 2 * rule_bytes(pr->kv_dtype);
        if (prefix_flops >= (int64_t)tu.fuse_cascade * suffix_bytes) path_tu.cached_prefix_bytes = 0;
    }
    int32_t path;
    st = choose_path(pr, path_tu, n_shared, prefix_tokens, (int64_t)B * H_q, m_eff, &path);
    if (st != PKV_OK) return st;
    if (path == PKV_PATH_PAGED) prefix_tokens = 0;
    if (m_eff > INT32_MAX) return PKV_EUNSUPPORTED;

    pkv_plan* pl = new (std::nothrow) pkv_plan();
    if (!pl) return PKV_ENOMEM;
    std::unique_ptr<pkv_plan> owner(pl);
    fill_problem(pl, pr, tu, geo);
    pl->indptr0 = B > 0 ? pr->kv_indptr[0] : 0;
    pl->indptr.assign(pr->kv_indptr, pr->kv_indptr + (B > 0 ? B + 1 : 0));
    pl->prefix_len = P;
    pl->path = path;
    // Prefix placement ("GraniKV", s.1): a prefix stored as one run of
    // consecutive slots is read by the prefix pass as base + offset.
    pl->prefix_base = -1;
    if (path != PKV_PATH_PAGED && tu.prefix_placement && pr->kv_indices) {
        const int32_t* pre = pr->kv_indices + pl->indptr0;
        bool run = true;
        for (int64_t t = 1; t < prefix_tokens && run; ++t) run = (int64_t)pre[t] == (int64_t)pre[0] + t;
        if (run && pre[0] >= 0) pl->prefix_base = pre[0];
    }
    pl->contiguous_prefixes = pl->prefix_base >= 0 ? 1 : 0;
    pl->m_eff = (int32_t)m_eff;
    pl->shared_pages = (int32_t)shared_pages;
    pl->prefix_tokens = (int32_t)prefix_tokens;
    // (the fused launch is built for the DENSE prefix kernels: bf16 K/V, or
    // fp8 K/V at head_dim 128)
    pl->fuse_cascade = tu.fuse_cascade && path == PKV_PATH_DENSE;

    // Paged pass: the attended positions [prefix_tokens, L_b) of all
    // requests, request after request, form one flat sequence that is cut
    // into equal chunks, one workgroup per (chunk, head block).
    const auto n_of = [&](int32_t b) {
        return (int64_t)pr->kv_indptr[b + 1] - pr->kv_indptr[b] - prefix_tokens;
    };
    int64_t total = 0;
    for (int32_t b = 0; b < B; ++b) total += n_of(b);

    // Prefix pass: M_eff query rows per KV head in tiles, the prefix cut into
    // ranges so that the grid fills the GPU.  One launch runs both passes of
    // a DENSE step when the prefix pass is heavy enough to hide suffix
    // streaming under it (fuse_cascade MFMA flops per suffix byte); its
    // prefix ranges then aim at a quarter of the workgroup target (long
    // items, most slots left to the suffix chunks), and it fuses only if the
    // prefix items take at most half of the slots.
    pl->prefix_rows_per_wg = path == PKV_PATH_DENSE ? pkv::kDenseRowsPerWg : pkv::kTiledRowsPerWg;
    pl->prefix_split_tokens = 0;
    pl->prefix_splits = 0;
    int64_t prefix_wgs = 0;
    if (path != PKV_PATH_PAGED) {
        const int64_t tiles = (int64_t)H_kv * ceil_div(m_eff, pl->prefix_rows_per_wg);
        if (pl->fuse_cascade) {
            const int64_t prefix_flops = 4 * m_eff * prefix_tokens * D * H_kv;
            const int64_t suffix_bytes = total * H_kv * D * 2 * rule_bytes(pr->kv_dtype);
            pl->fuse_cascade = prefix_flops >= (int64_t)tu.fuse_cascade * suffix_bytes;
        }
        if (pl->fuse_cascade) {
            prefix_ranges(tu, prefix_tokens, tiles, fused_prefix_target(tu), &pl->prefix_split_tokens,
                          &pl->prefix_splits);
            prefix_wgs = align_up(tiles * pl->prefix_splits, 8);  // a multiple of 8 for the XCD placement
            pl->fuse_cascade = 2 * prefix_wgs <= tu.target_workgroups;
        }
        if (!pl->fuse_cascade)
            prefix_ranges(tu, prefix_tokens, tiles, tu.prefix_target_workgroups, &pl->prefix_split_tokens,
                          &pl->prefix_splits);
    }
    int64_t nonempty = 0;
    for (int32_t b = 0; b < B; ++b) nonempty += n_of(b) > 0;
    if (!pl->fuse_cascade) fp8_long_geometry(pl, tu, total, nonempty);
    // positions a PAGED pass re-reads from a declared shared prefix
    const int64_t reread = path == PKV_PATH_PAGED && n_shared >= 2 ? (n_shared - 1) * shared_pages * p : 0;
    const int64_t target = paged_target(pl, tu, total, pl->fuse_cascade, tu.target_workgroups - prefix_wgs, reread);
    bool spans = false, any_empty = false;
    plan_chunks(pl, tu, total, target, n_of, &spans, &any_empty);
    // A combine kernel follows the paged pass for a cascade step, when a
    // request spans chunks, or to write the output of empty requests.
    pl->needs_reduce = path != PKV_PATH_PAGED || spans || any_empty;

    // Workspace layout.  A cascade step keeps both passes as partial states
    // (prefix ranges, then suffix chunks) that one kernel combines; a request
    // inside one chunk of a paged pass has its output written directly.
    layout_workspace(pl, spans || path != PKV_PATH_PAGED, path != PKV_PATH_PAGED ? pl->prefix_splits : 0);
    *out = owner.release();
    return PKV_OK;
}
}  // namespace

namespace {
pkv_status plan_grouped(const pkv_problem* pr, const pkv_tuning* tuning, const int32_t* page_indptr,
                        const int32_t* page_indices, const int32_t* seq_lens, pkv_plan** out);
}  // namespace

pkv_status pkv_plan_create_grouped(const pkv_problem* pr, const pkv_tuning* tuning, const int32_t* page_indptr,
                                   const int32_t* page_indices, const int32_t* seq_lens, pkv_plan** out) {
    // host containers may throw; nothing may cross the C boundary
    try {
        return plan_grouped(pr, tuning, page_indptr, page_indices, seq_lens, out);
    } catch (const std::bad_alloc&) {
        return PKV_ENOMEM;
    }
}

namespace {
pkv_status plan_grouped(const pkv_problem* pr, const pkv_tuning* tuning, const int32_t* page_indptr,
                        const int32_t* page_indices, const int32_t* seq_lens, pkv_plan** out) {
    if (!pr || !out) return PKV_EINVAL;
    pkv_tuning tu;
    pkv::PagedGeometry geo;
    pkv_status st = check_problem(pr, tuning, &tu);
    if (st != PKV_OK) return st;
    const int32_t B = pr->batch, H_q = pr->num_q_heads, H_kv = pr->num_kv_heads;
    const int32_t D = pr->head_dim, p = pr->page_size;
    if (pr->shared_prefix_len != 0 || pr->force_path < -1 || pr->force_path > 2) return PKV_EINVAL;
    if (B > 0 && (!page_indptr || !seq_lens)) return PKV_EINVAL;
    st = check_support(pr, tu, &geo);
    if (st != PKV_OK) return st;
    const int32_t G = H_q / H_kv;
    // The page table, checked as pkv_lower_page_table checks it.
    int64_t total_tokens = 0;
    if (B > 0 && page_indptr[0] != 0) return PKV_EINVAL;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t n = (int64_t)page_indptr[b + 1] - page_indptr[b];
        const int64_t L = seq_lens[b];
        if (n < 0 || L < 0) return PKV_EINVAL;
        if (n != ceil_div(L, p)) return PKV_ERANGE;
        if (n > 0 && !page_indices) return PKV_EINVAL;
        for (int64_t j = 0; j < n; ++j) {
            const int32_t pg = page_indices[page_indptr[b] + j];
            if (pg < 0 || (int64_t)pg * p + (p - 1) > INT32_MAX) return PKV_ERANGE;
        }
        total_tokens += L;
    }
    if (total_tokens > INT32_MAX || (int64_t)B * G > INT32_MAX) return PKV_ERANGE;

    // Groups: the nodes of the radix tree of the requests' page lists that
    // two or more requests share.  Requests whose first whole page is the
    // same physical page form a root; a group's run is the longest stretch
    // of pages from its parent's end that every member holds in full and
    // all agree on; members that hold the page after the run and agree on it
    // form a child (two or more of them).  Depth-first order, parents before
    // children, siblings by first member.
    struct Node {
        std::vector<int32_t> members;
        int32_t start, end, parent;
    };
    std::vector<Node> nodes;
    // members of `mem` holding page `at` in full, grouped by that page, in
    // order of first member; groups of two or more only
    const auto split = [&](const std::vector<int32_t>& mem, int32_t at) {
        std::unordered_map<int32_t, int32_t> slot;
        std::vector<std::vector<int32_t>> parts;
        for (int32_t b : mem) {
            if (seq_lens[b] / p <= at) continue;
            const int32_t pg = page_indices[page_indptr[b] + at];
            auto it = slot.find(pg);
            if (it == slot.end()) {
                slot.emplace(pg, (int32_t)parts.size());
                parts.push_back({b});
            } else {
                parts[it->second].push_back(b);
            }
        }
        std::vector<std::vector<int32_t>> out;
        for (auto& x : parts)
            if (x.size() >= 2) out.push_back(std::move(x));
        return out;
    };
    {
        struct Todo {
            std::vector<int32_t> members;
            int32_t start, parent;
        };
        std::vector<Todo> stack;
        std::vector<int32_t> all(B);
        for (int32_t b = 0; b < B; ++b) all[b] = b;
        auto roots = split(all, 0);
        for (auto it = roots.rbegin(); it != roots.rend(); ++it) stack.push_back({std::move(*it), 0, -1});
        while (!stack.empty()) {
            Todo t = std::move(stack.back());
            stack.pop_back();
            int32_t end = INT32_MAX;
            for (int32_t b : t.members) end = std::min(end, seq_lens[b] / p);
            const int32_t* first = page_indices + page_indptr[t.members[0]];
            for (size_t i = 1; i < t.members.size(); ++i) {
                const int32_t* mine = page_indices + page_indptr[t.members[i]];
                int32_t j = t.start;
                while (j < end && mine[j] == first[j]) ++j;
                end = j;
            }
            const int32_t me = (int32_t)nodes.size();
            auto kids = split(t.members, end);
            nodes.push_back({std::move(t.members), t.start, end, t.parent});
            for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back({std::move(*it), end, me});
        }
    }
    // Each group is planned as the step it would be on its own over its own
    // run; a group planned PAGED is dissolved (its children still planned).
    // The cached-prefix allowance is left out: a dissolved group's re-reads
    // join the suffix pass that every kept group's prefix items overlap
    // (four prompts of 48 requests: the 512-token prompt dissolved by the
    // allowance took the step from 72.8 to 96.3 us).
    pkv_tuning group_tu = tu;
    group_tu.cached_prefix_bytes = 0;
    struct Group {
        std::vector<int32_t> members;
        int32_t start_tokens, prefix_tokens, parent, path, m_eff, rows_per_wg, row_tiles, split_tokens, splits;
        int32_t slot_base;
        int32_t prefix_base;  // first slot when the run's pages are consecutive, else -1
        int64_t items;
    };
    std::vector<Group> groups;
    std::vector<int32_t> kept_at(nodes.size(), -1);
    std::vector<std::vector<int32_t>> path_of(B);  // kept groups of each request, outermost first
    for (size_t i = 0; i < nodes.size(); ++i) {
        const Node& nd = nodes[i];
        const int64_t n = (int64_t)nd.members.size();
        int32_t path;
        st = choose_path(pr, group_tu, n, (int64_t)(nd.end - nd.start) * p, n * H_q, n * G, &path);
        if (st != PKV_OK) return st;
        if (path == PKV_PATH_PAGED) continue;
        int32_t a = nd.parent;  // nearest kept ancestor
        while (a >= 0 && kept_at[a] < 0) a = nodes[a].parent;
        Group g{};
        g.members = nd.members;
        g.start_tokens = nd.start * p;
        g.prefix_tokens = (nd.end - nd.start) * p;
        g.parent = a >= 0 ? kept_at[a] : -1;
        g.path = path;
        g.m_eff = (int32_t)(n * G);
        g.rows_per_wg = path == PKV_PATH_DENSE ? pkv::kDenseRowsPerWg : pkv::kTiledRowsPerWg;
        g.row_tiles = (int32_t)ceil_div(g.m_eff, g.rows_per_wg);
        // Prefix placement ("GraniKV", s.1): a run stored in consecutive
        // physical pages is one run of consecutive slots, read as base +
        // offset.
        g.prefix_base = -1;
        if (tu.prefix_placement) {
            const int32_t* pages = page_indices + page_indptr[nd.members[0]];
            bool run = true;
            for (int32_t j = nd.start + 1; j < nd.end && run; ++j) run = (int64_t)pages[j] == (int64_t)pages[j - 1] + 1;
            if (run) g.prefix_base = pages[nd.start] * p;
        }
        kept_at[i] = (int32_t)groups.size();
        for (int32_t b : nd.members) path_of[b].push_back(kept_at[i]);
        groups.push_back(std::move(g));
    }
    const int32_t NG = (int32_t)groups.size();

    // Own tokens of every request: all of its tokens outside the runs of
    // its kept groups.
    int64_t suffix_total = 0;
    for (int32_t b = 0; b < B; ++b) {
        suffix_total += seq_lens[b];
        for (int32_t gi : path_of[b]) suffix_total -= groups[gi].prefix_tokens;
    }

    // Prefix ranges: each group gets the share of the prefix pass's target
    // workgroups that its flops (M_eff x P) are of the step's, and is cut
    // as a single-prefix step with that target would be.  When every group
    // runs DENSE the two passes may share one launch under the single-prefix
    // step's rule (flops per suffix byte; ranges against the fused target;
    // prefix items at most half the slots).
    unsigned __int128 work = 0;
    int64_t prefix_flops = 0;
    bool all_dense = NG > 0;
    for (auto& g : groups) {
        work += (unsigned __int128)g.m_eff * g.prefix_tokens;
        prefix_flops += 4LL * g.m_eff * g.prefix_tokens * D * H_kv;
        all_dense &= g.path == PKV_PATH_DENSE;
    }
    int64_t dense_items = 0, tiled_items = 0;
    int32_t max_splits = 0;
    const auto plan_ranges = [&](int64_t target) {
        dense_items = tiled_items = 0;
        max_splits = 0;
        for (auto& g : groups) {
            const int64_t share = (int64_t)((unsigned __int128)target * g.m_eff * g.prefix_tokens / work);
            prefix_ranges(tu, g.prefix_tokens, (int64_t)H_kv * g.row_tiles, std::max<int64_t>(1, share),
                          &g.split_tokens, &g.splits);
            g.items = (int64_t)g.row_tiles * H_kv * g.splits;
            (g.path == PKV_PATH_DENSE ? dense_items : tiled_items) += g.items;
            max_splits = std::max(max_splits, g.splits);
        }
    };
    const int64_t suffix_bytes = suffix_total * H_kv * D * 2 * rule_bytes(pr->kv_dtype);
    bool fuse = tu.fuse_cascade && all_dense && prefix_flops >= (int64_t)tu.fuse_cascade * suffix_bytes;
    if (fuse) {
        plan_ranges(fused_prefix_target(tu));
        fuse = 2 * align_up(dense_items, 8) <= tu.target_workgroups;
    }
    if (!fuse) plan_ranges(tu.prefix_target_workgroups);
    // A request's prefix partial states: its groups' ranges, outermost group
    // first (each group's slots start after its kept ancestors').
    int32_t max_slots = 0;
    for (auto& g : groups) {
        g.slot_base = g.parent >= 0 ? groups[g.parent].slot_base + groups[g.parent].splits : 0;
        max_slots = std::max(max_slots, g.slot_base + g.splits);
    }
    if (dense_items > INT32_MAX || tiled_items > INT32_MAX) return PKV_EUNSUPPORTED;

    pkv_plan* pl = new (std::nothrow) pkv_plan();
    if (!pl) return PKV_ENOMEM;
    fill_problem(pl, pr, tu, geo);
    pl->grouped = 1;
    pl->num_groups = NG;
    pl->fuse_cascade = fuse;
    pl->dense_items = (int32_t)dense_items;
    pl->tiled_items = (int32_t)tiled_items;
    pl->prefix_splits = max_slots;
    pl->path = PKV_PATH_PAGED;
    int64_t prefix_sum = 0, pages_sum = 0;
    for (auto& g : groups) {
        if (g.path == PKV_PATH_DENSE) pl->path = PKV_PATH_DENSE;
        else if (pl->path == PKV_PATH_PAGED) pl->path = PKV_PATH_CASCADE;
        pl->m_eff = std::max(pl->m_eff, g.m_eff);
        prefix_sum += g.prefix_tokens;
        pages_sum += g.prefix_tokens / p;
    }
    pl->prefix_tokens = (int32_t)prefix_sum;
    pl->shared_pages = (int32_t)pages_sum;

    // Metadata block (int32): the public arrays, then the kernels' tables.
    int64_t members_total = 0;
    for (auto& g : groups) members_total += (int64_t)g.members.size();
    int64_t off = 0;
    const auto take = [&](int64_t n) {
        const int64_t at = off;
        off += n;
        return at;
    };
    pl->meta_suffix_indptr = take(B + 1);
    pl->meta_suffix_indices = take(suffix_total);
    pl->meta_group_indptr = take(NG + 1);
    pl->meta_members = take(members_total);
    pl->meta_prefix_indptr = take(NG + 1);
    pl->meta_prefix_indices = take(prefix_sum);
    pl->meta_group_parent = take(NG);
    pl->meta_group_base = take(NG);
    pl->meta_pre_count = take(B);
    pl->meta_desc = take((int64_t)NG * pkv::kGroupDescInts);
    std::unique_ptr<pkv_plan> owner(pl);
    pl->meta.assign(off, 0);
    int32_t* m = pl->meta.data();
    const auto lower = [&](int32_t b, int32_t t0, int32_t t1, int32_t* dst) {
        const int32_t* pages = page_indices + page_indptr[b];
        for (int32_t t = t0; t < t1; ++t) *dst++ = pages[t / p] * p + t % p;
    };
    {
        int32_t* ptr = m + pl->meta_suffix_indptr;
        int32_t* idx = m + pl->meta_suffix_indices;
        ptr[0] = 0;
        for (int32_t b = 0; b < B; ++b) {
            // the tokens outside the runs of b's kept groups (outermost
            // first, so the runs come in increasing position)
            int32_t t = 0, n = 0;
            for (int32_t gi : path_of[b]) {
                const Group& g = groups[gi];
                lower(b, t, g.start_tokens, idx + ptr[b] + n);
                n += g.start_tokens - t;
                t = g.start_tokens + g.prefix_tokens;
            }
            lower(b, t, seq_lens[b], idx + ptr[b] + n);
            n += seq_lens[b] - t;
            ptr[b + 1] = ptr[b] + n;
        }
        int32_t* gptr = m + pl->meta_group_indptr;
        int32_t* mem = m + pl->meta_members;
        int32_t* pptr = m + pl->meta_prefix_indptr;
        int32_t* pidx = m + pl->meta_prefix_indices;
        gptr[0] = pptr[0] = 0;
        for (int32_t i = 0; i < NG; ++i) {
            const Group& g = groups[i];
            std::copy(g.members.begin(), g.members.end(), mem + gptr[i]);
            gptr[i + 1] = gptr[i] + (int32_t)g.members.size();
            lower(g.members[0], g.start_tokens, g.start_tokens + g.prefix_tokens, pidx + pptr[i]);
            pptr[i + 1] = pptr[i] + g.prefix_tokens;
        }
        for (int32_t i = 0; i < NG; ++i) m[pl->meta_group_parent + i] = groups[i].parent;
        for (int32_t i = 0; i < NG; ++i) {
            m[pl->meta_group_base + i] = groups[i].prefix_base;
            pl->contiguous_prefixes += groups[i].prefix_base >= 0;
        }
        for (int32_t b = 0; b < B; ++b) {
            const int32_t last = path_of[b].empty() ? -1 : path_of[b].back();
            m[pl->meta_pre_count + b] = last >= 0 ? groups[last].slot_base + groups[last].splits : 0;
        }
        // group table in launch order: DENSE groups' items, then CASCADE's
        int32_t row = 0, end = 0;
        for (int pass = 0; pass < 2; ++pass)
            for (int32_t i = 0; i < NG; ++i) {
                const Group& g = groups[i];
                if ((g.path == PKV_PATH_DENSE) != (pass == 0)) continue;
                int32_t* d = m + pl->meta_desc + (int64_t)row++ * pkv::kGroupDescInts;
                end += (int32_t)g.items;
                d[0] = end;
                d[1] = pptr[i];
                d[2] = g.prefix_tokens;
                d[3] = g.split_tokens;
                d[4] = g.splits;
                d[5] = g.row_tiles;
                d[6] = gptr[i];
                d[7] = (int32_t)g.members.size();
                d[8] = g.slot_base;
                d[9] = g.prefix_base;
            }
    }

    // Paged pass over every request's suffix (all of its tokens if it is in
    // no group); with groups every request leaves partial states for the
    // combine.
    const int32_t* sptr = m + pl->meta_suffix_indptr;
    const auto n_of = [&](int32_t b) { return (int64_t)sptr[b + 1] - sptr[b]; };
    int64_t nonempty = 0;
    for (int32_t b = 0; b < B; ++b) nonempty += n_of(b) > 0;
    if (!fuse) fp8_long_geometry(pl, tu, suffix_total, nonempty);
    const int64_t target = paged_target(pl, tu, suffix_total, fuse, tu.target_workgroups - align_up(dense_items, 8), 0);
    bool spans = false, any_empty = false;
    plan_chunks(pl, tu, suffix_total, target, n_of, &spans, &any_empty);
    pl->needs_reduce = NG > 0 || spans || any_empty;
    layout_workspace(pl, NG > 0 || spans, max_slots);
    *out = owner.release();
    return PKV_OK;
}
}  // namespace

pkv_status pkv_plan_metadata(const pkv_plan* pl, int32_t* out, int64_t capacity) {
    if (!pl || !pl->grouped) return PKV_EINVAL;
    const int64_t n = (int64_t)pl->meta.size();
    if (capacity < n) return PKV_ERANGE;
    if (n > 0 && !out) return PKV_EINVAL;
    std::copy(pl->meta.begin(), pl->meta.end(), out);
    return PKV_OK;
}

pkv_status pkv_plan_request_bins(const pkv_plan* pl, int32_t* out, int64_t capacity) {
    if (!pl || pl->request_bins == 0 || !out) return PKV_EINVAL;
    const int64_t n = (int64_t)pl->bin_start.size() + (int64_t)pl->bin_req.size();
    if (capacity < n) return PKV_ERANGE;
    std::copy(pl->bin_start.begin(), pl->bin_start.end(), out);
    std::copy(pl->bin_req.begin(), pl->bin_req.end(), out + pl->bin_start.size());
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
    info->num_groups = pl->num_groups;
    info->metadata_ints = (int64_t)pl->meta.size();
    info->prefix_base = pl->grouped ? -1 : pl->prefix_base;
    info->contiguous_prefixes = pl->contiguous_prefixes;
    info->request_bins = pl->request_bins;
    return PKV_OK;
}

void pkv_plan_destroy(pkv_plan* pl) { delete pl; }

}  // extern "C"

// Checks of the checked library (libpkv_checked.so), on host copies of the
// arrays a step's kernels read.
namespace pkv {

pkv_status check_step_indptr(const pkv_plan& pl, const int32_t* kv_indptr) {
    if ((int64_t)pl.indptr.size() != (pl.B > 0 ? pl.B + 1 : 0)) return PKV_EINVAL;  // a grouped plan
    for (size_t i = 0; i < pl.indptr.size(); ++i)
        if (kv_indptr[i] != pl.indptr[i]) return PKV_EINVAL;
    return PKV_OK;
}

pkv_status check_slots(const int32_t* slots, int64_t n, int64_t num_slots) {
    for (int64_t i = 0; i < n; ++i)
        if (slots[i] < 0 || slots[i] >= num_slots) return PKV_ERANGE;
    return PKV_OK;
}

pkv_status check_prefix_slots(const pkv_plan& pl, const int32_t* prefix, int64_t num_slots) {
    const int64_t n = pl.prefix_tokens;
    if (pl.prefix_base < 0) return check_slots(prefix, n, num_slots);
    // the prefix pass reads slots prefix_base + t and not the indices
    if ((int64_t)pl.prefix_base + n > num_slots) return PKV_ERANGE;
    for (int64_t t = 0; t < n; ++t)
        if ((int64_t)prefix[t] != pl.prefix_base + t) return PKV_EINVAL;
    return PKV_OK;
}

pkv_status check_page_indptr(const pkv_plan& pl, const int32_t* page_indptr, int64_t* lo, int64_t* hi) {
    *lo = *hi = 0;
    if (pl.B == 0) return PKV_OK;
    if ((int64_t)pl.indptr.size() != pl.B + 1) return PKV_EINVAL;
    if (page_indptr[0] < 0) return PKV_EINVAL;
    int64_t end = page_indptr[0];
    for (int32_t b = 0; b < pl.B; ++b) {
        const int64_t len = (int64_t)pl.indptr[b + 1] - pl.indptr[b];
        const int64_t need = (len + pl.page_size - 1) / pl.page_size;
        // fewer pages than the request's tokens fill (or a decreasing offset)
        if ((int64_t)page_indptr[b + 1] - page_indptr[b] < need) return PKV_ERANGE;
        end = std::max<int64_t>(end, (int64_t)page_indptr[b] + need);
    }
    *lo = page_indptr[0];
    *hi = end;
    return PKV_OK;
}

pkv_status check_group_metadata(const pkv_plan& pl, const int32_t* meta, int64_t num_slots) {
    if (!pl.grouped) return PKV_EINVAL;
    if (!std::equal(pl.meta.begin(), pl.meta.end(), meta)) return PKV_EINVAL;
    const int32_t* m = pl.meta.data();
    pkv_status st = check_slots(m + pl.meta_suffix_indices, pl.meta_group_indptr - pl.meta_suffix_indices, num_slots);
    if (st != PKV_OK) return st;
    // a run read as base + offset holds exactly those slots (the planner
    // found it in these lowered indices)
    return check_slots(m + pl.meta_prefix_indices, pl.meta_group_parent - pl.meta_prefix_indices, num_slots);
}

}  // namespace pkv
