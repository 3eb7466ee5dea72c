// Launch interfaces of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

// Arguments of the paged split kernel.  All pointers are device memory.
struct PagedArgs {
    const void* q;            // [B][H_q][D], q dtype
    const void* k;            // pool [slots][H_kv][D]
    const void* v;
    const float* k_scale;     // [H_kv] (fp8)
    const float* v_scale;
    const int32_t* kv_indptr; // [B+1]
    const int32_t* kv_indices;
    int32_t H_kv;
    int32_t token_offset;     // tokens skipped at the start of every request
    int32_t split_tokens;
    int32_t num_splits;
    float scale_log2;         // sm_scale * log2(e)
    // direct outputs (num_splits == 1)
    void* o;                  // [B][H_q][D], q dtype, nullable
    float* o_f32;             // nullable
    float* lse;               // [B][H_q], nullable
    // partial outputs (num_splits > 1)
    float* part_acc;          // [B][num_splits][H_q][D]: sum of 2^(s - M) v
    float* part_ml;           // [B][num_splits][H_q][2]: (M, L), M in log2 units
    // num_splits > 1 and non-null: [B][head_blocks] arrival counters (zero on
    // entry, left zero on exit); the last item of a (request, head block) to
    // finish combines the partials and writes o / o_f32 / lse itself.
    int32_t* counters;
    int32_t out_dtype;        // dtype of o (q dtype)
    int32_t force_partial;    // write partials even with one split (cascade suffix)
};

// Launch the paged split kernel for the plan's geometry.
hipError_t launch_paged_split(const pkv_plan& plan, const PagedArgs& a, hipStream_t stream);

// Combine partial states row by row: the pre_splits partials at pre_acc
// (the shared-prefix pass of a cascade step; optional) followed by the
// num_splits partials at part_acc, all in the [B][splits][H_q] layout.
struct SplitReduceArgs {
    int32_t num_splits;
    int32_t B, H_q, D;
    const float* part_acc;
    const float* part_ml;
    const float* pre_acc;     // nullable: [B][pre_splits][H_q][D]
    const float* pre_ml;
    int32_t pre_splits;
    void* o;                  // nullable; out_dtype
    int32_t out_dtype;
    float* o_f32;             // nullable
    float* lse;               // nullable
};
hipError_t launch_split_reduce(const SplitReduceArgs& a, hipStream_t stream);

// Shared-prefix pass (bf16 MFMA).  Rows r = b * G + j of KV head g attend
// over prefix tokens [split * split_tokens, ...) listed by prefix_indices.
struct PrefixArgs {
    const void* q;            // [B][H_q][D] bf16
    const void* k;            // pool, bf16
    const void* v;
    const int32_t* prefix_indices;
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
};
hipError_t launch_prefix_attn(const PrefixArgs& a, int rows_per_wg, hipStream_t stream);

// Row-wise LSE merge of two fp32 states.
hipError_t launch_merge_states(int32_t rows, int32_t D, const float* o_a, const float* lse_a,
                               const float* o_b, const float* lse_b, void* o_out, int32_t out_dtype,
                               float* lse_out, hipStream_t stream);

}  // namespace pkv
