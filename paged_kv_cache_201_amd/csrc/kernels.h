// Launch interfaces of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

// Arguments of the paged kernel.  All pointers are device memory.  The
// attended positions of all requests (tokens [token_offset, L_b) of each)
// form one flat sequence of total_tokens positions cut into chunks of
// chunk_tokens; a request's partial states are numbered by chunk, from the
// chunk holding its first position.
struct PagedArgs {
    const void* q;            // [B][H_q][D], q dtype
    const void* k;            // pool [slots][H_kv][D]
    const void* v;
    const float* k_scale;     // [H_kv] (fp8)
    const float* v_scale;
    const int32_t* kv_indptr; // [B+1]
    const int32_t* kv_indices;   // token-flat slots; null when the page table is read instead
    const int32_t* page_indptr;  // [B+1], with page_indices: pages of request b
    const int32_t* page_indices;
    int32_t page_size;
    int32_t B;
    int32_t H_kv;
    int32_t token_offset;     // tokens skipped at the start of every request
    int32_t chunk_tokens;
    int64_t total_tokens;
    int32_t max_parts;        // partial states per request the workspace holds
    float scale_log2;         // sm_scale * log2(e)
    // outputs of requests that lie inside one chunk (unless force_partial)
    void* o;                  // [B][H_q][D], q dtype, nullable
    float* o_f32;             // nullable
    float* lse;               // [B][H_q], nullable
    // partial outputs
    float* part_acc;          // [B][max_parts][H_q][D]: sum of 2^(s - M) v
    float* part_ml;           // [B][max_parts][H_q][2]: (M, L), M in log2 units
    int32_t out_dtype;        // dtype of o (q dtype)
    int32_t force_partial;    // every segment writes a partial (cascade suffix)
    // > 0: work items are bins of whole requests instead of chunks: item w
    // takes requests bin_req[bin_start[w] .. bin_start[w + 1]), each as one
    // segment (no request is cut; a partial state, if any, is slot 0)
    int32_t request_bins;
    int32_t bin_max_tokens;   // the longest request of the bins (fits the LDS index stage)
    uint16_t bin_start[kMaxRequestBins + 1];
    uint16_t bin_req[kMaxBinnedRequests];
};

// Launch the paged split kernel for the plan's geometry.
hipError_t launch_paged_split(const pkv_plan& plan, const PagedArgs& a, hipStream_t stream);

// Combine partial states row by row, in order: first the pre_splits
// partials of the shared-prefix pass (optional; [B][pre_splits][H_q]), then
// the chunk partials of the paged pass (optional; [B][max_parts][H_q]), whose
// count per request follows from kv_indptr and the chunking.  With pre_count,
// request b has pre_count[b] prefix partials (pre_splits is then the stride
// only).  With
// skip_whole, rows of non-empty requests that lie inside one chunk are left
// alone (the paged kernel wrote them).  A row with nothing to combine gets
// o = 0, lse = -inf.
struct SplitReduceArgs {
    int32_t B, H_q, D;
    const float* pre_acc;     // nullable
    const float* pre_ml;
    int32_t pre_splits;
    const int32_t* pre_count; // [B], nullable
    const float* part_acc;    // nullable
    const float* part_ml;
    int32_t max_parts;
    const int32_t* kv_indptr; // [B+1]; nullable: no chunk partials, skip nothing
    int32_t token_offset;
    int32_t chunk_tokens;
    int32_t whole_requests;   // the paged pass ran on bins of whole requests: one partial each
    int32_t skip_whole;
    void* o;                  // nullable; out_dtype
    int32_t out_dtype;
    float* o_f32;             // nullable
    float* lse;               // nullable
};
hipError_t launch_split_reduce(const SplitReduceArgs& a, hipStream_t stream);

// Shared-prefix pass (bf16 MFMA; fp8 K/V widened to bf16 operands in registers).  Rows
// r = b * G + j of KV head g attend
// over prefix tokens [split * split_tokens, ...) listed by prefix_indices.
struct PrefixArgs {
    const void* q;            // [B][H_q][D] bf16
    const void* k;            // pool, bf16 or fp8 e4m3 (kv_dtype)
    const void* v;
    int32_t kv_dtype;
    const float* k_scale;     // [H_kv], fp8 only
    const float* v_scale;
    const int32_t* prefix_indices;
    int32_t prefix_base;      // >= 0: prefix token t is slot prefix_base + t (prefix_indices unread)
    int32_t B, H_kv, G, D;
    int32_t prefix_len;
    int32_t split_tokens;
    int32_t num_splits;
    int32_t row_tiles;        // ceil(B * G / rows_per_wg)
    float scale_log2;
    float* o;                 // num_splits == 1: [B][H_q][D] fp32, normalised
    float* lse;               // num_splits == 1: [B][H_q]
    float* part_acc;          // num_splits > 1: [B][num_splits][H_q][D]
    float* part_ml;           // num_splits > 1: [B][num_splits][H_q][2]
    int32_t force_partial;    // write partials even with one split (cascade step)
    // Several prefix groups (groups != nullptr): each item's group, prefix
    // range and query rows come from the group table (kGroupDescInts ints
    // per group, in launch order) instead of the fields above; prefix_indices
    // is then the base that the table's offsets index, members lists the
    // requests of each group, num_splits is the partial-state stride and
    // force_partial must be set.  The launch runs items
    // [item_base, item_base + num_items) of the table.
    const int32_t* groups;
    const int32_t* members;
    int32_t num_groups;
    int32_t item_base;
    int32_t num_items;
};
hipError_t launch_prefix_attn(const PrefixArgs& a, int rows_per_wg, hipStream_t stream);

// Both passes of a DENSE cascade step in one launch (bf16): the prefix work
// items of `pa` (DENSE tiles, partial states) and the chunks of the paged
// pass `sa` (partial states), interleaved so that they run side by side.
hipError_t launch_cascade_fused(const pkv_plan& plan, const PrefixArgs& pa, const PagedArgs& sa,
                                hipStream_t stream);

// Row-wise LSE merge of two fp32 states.
hipError_t launch_merge_states(int32_t rows, int32_t D, const float* o_a, const float* lse_a,
                               const float* o_b, const float* lse_b, void* o_out, int32_t out_dtype,
                               float* lse_out, hipStream_t stream);

}  // namespace pkv
