// Internal declarations shared by the host planner and the HIP launchers.
// Nothing here is part of the public ABI (include/pkv.h).
#pragma once

#include <cstdint>
#include <vector>

#include "pkv.h"

namespace pkv {

// How one work item of the paged kernel maps its 64 lanes onto K/V rows.
// A "row" is one (token, KV head) vector of head_dim elements.  Each lane
// loads EPL consecutive elements; LPH lanes cover a row; one wave-wide load
// covers RS = 64 / LPH rows.  A work item covers HB KV heads: either NHL
// loads per token (HB = NHL * RS, one token per load) or TPI tokens per load
// (HB = RS / TPI).
struct PagedGeometry {
    int32_t epl;   // elements per lane per row
    int32_t lph;   // lanes per row
    int32_t rs;    // rows per wave-wide load
    int32_t nhl;   // loads per token (head slots per lane)
    int32_t tpi;   // tokens per load
    int32_t hb;    // KV heads per work item
};

// Lane geometry for a (kv dtype, head_dim, G, H_kv) problem.  Returns false
// if no kernel is built for it.
// max_heads > 0 limits the KV heads per work item.
bool paged_geometry(int32_t kv_dtype, int32_t head_dim, int32_t group, int32_t num_kv_heads, int32_t max_heads,
                    PagedGeometry* out);

// Query rows one prefix-kernel workgroup handles, per path.
constexpr int32_t kDenseRowsPerWg = 128;
constexpr int32_t kTiledRowsPerWg = 64;
// Prefix tokens are split in multiples of this many, at most
// kMaxPrefixSplitTokens per range (the kernel stages a range's indices in LDS).
constexpr int32_t kPrefixTokenQuantum = 64;
// Ints per row of the prefix-group table a grouped step hands the prefix
// kernel: running end of the group's items, offset and length of its prefix
// indices, range size, ranges, query-row tiles, offset and count of its
// members, first partial-state slot of its ranges, slot of the run's first
// token when the run is read as base + offset (else -1).
constexpr int32_t kGroupDescInts = 10;
constexpr int32_t kMaxPrefixSplitTokens = 1024;
// Paged-pass chunks hold a multiple of this many tokens, and at most
// max_chunk_tokens(...): the kernel stages a chunk's slot indices in LDS next
// to its merge buffer (two wave states with one token per load, else one per
// wave and token lane group: 4 bytes x slots x heads per item x G x d), and
// the index stage is sized so that two workgroups still fit in a CU's 160 KB.
constexpr int32_t kSplitQuantum = 16;
// Bins of whole requests travel in the paged kernels' arguments (16-bit
// request ids and bin starts): at most this many bins and requests.
constexpr int32_t kMaxRequestBins = 256;
constexpr int32_t kMaxBinnedRequests = 1024;
constexpr int32_t kMaxSplitTokens = 4096;
constexpr int32_t max_chunk_tokens(int32_t rs, int32_t nhl, int32_t tpi, int32_t group, int32_t head_dim) {
    return 4 * (tpi == 1 ? 2 : 4 * tpi) * (rs * nhl / tpi) * group * head_dim > 40 * 1024 ? 2048
                                                                                           : kMaxSplitTokens;
}

}  // namespace pkv

struct pkv_plan;

namespace pkv {

// Checks of a step's index arrays, made by the checked library
// (libpkv_checked.so) on host copies of what its kernels would read, before
// any launch.  Each returns PKV_OK, PKV_EINVAL (an array that does not
// describe the planned batch) or PKV_ERANGE (a slot or page outside the
// pool).
//
// kv_indptr [B + 1] equals the host kv_indptr the plan was made from.
pkv_status check_step_indptr(const pkv_plan& pl, const int32_t* kv_indptr);
// Every slot of slots[0 .. n) lies in [0, num_slots).
pkv_status check_slots(const int32_t* slots, int64_t n, int64_t num_slots);
// The prefix pass's slots: prefix [plan prefix_tokens] in range, and, when
// the plan reads the prefix as one run of slots (prefix_base >= 0), exactly
// that run.
pkv_status check_prefix_slots(const pkv_plan& pl, const int32_t* prefix, int64_t num_slots);
// A page table for the plan's kv_indptr: page_indptr [B + 1] starts at
// offset >= 0 and gives request b at least ceil(L_b / page_size) pages; the
// page list the kernel reads is then page_indices [*lo, *hi).
pkv_status check_page_indptr(const pkv_plan& pl, const int32_t* page_indptr, int64_t* lo, int64_t* hi);
// A grouped step's metadata block equals the plan's, and its lowered
// suffix and prefix slots lie in the pool.
pkv_status check_group_metadata(const pkv_plan& pl, const int32_t* meta, int64_t num_slots);

}  // namespace pkv

struct pkv_plan {
    // problem
    int32_t B, H_q, H_kv, D, G, q_dtype, kv_dtype, page_size;
    int32_t indptr0;          // host kv_indptr[0]
    std::vector<int32_t> indptr;  // the host kv_indptr [B + 1] the plan was made from (single-prefix plans)
    int32_t prefix_len;       // declared shared prefix (tokens)
    int32_t prefix_base;      // prefix read as slots prefix_base + t (-1: by slot index)
    int32_t contiguous_prefixes; // prefix runs read as base + offset
    // decisions
    int32_t path, m_eff, shared_pages, prefix_tokens;
    // paged pass
    pkv::PagedGeometry geo;
    int32_t head_blocks;
    int32_t split_tokens;     // positions per chunk of the flat sequence
    int32_t num_splits;       // partial states per request (chunks one request touches, max)
    int64_t num_chunks;
    int64_t num_work_items;   // num_chunks * head_blocks
    int32_t needs_reduce;     // a combine kernel follows the paged pass
    int32_t concurrent_prefix; // prefix pass on a side stream in decode_step
    int32_t fuse_cascade;     // decode_step runs both passes in one launch (DENSE)
    int64_t paged_tokens;     // positions the paged pass attends (all requests)
    // prefix pass
    int32_t prefix_rows_per_wg;
    int32_t prefix_split_tokens, prefix_splits;
    // bins of whole requests (request_bins > 0): bin w holds requests
    // bin_req[bin_start[w] .. bin_start[w + 1])
    int32_t request_bins = 0;
    int32_t bin_max_tokens = 0;  // the longest request of a binned pass
    std::vector<uint16_t> bin_start, bin_req;
    // workspace layout (byte offsets; -1 = unused)
    int64_t ws_paged_acc, ws_paged_ml;
    int64_t ws_prefix_acc, ws_prefix_ml;
    int64_t workspace_bytes;
    // several prefix groups (pkv_plan_create_grouped)
    int32_t grouped;
    int32_t num_groups;               // groups that run a prefix pass
    int32_t dense_items, tiled_items; // prefix work items per launch
    // offsets (in ints) of the metadata block's arrays
    int64_t meta_suffix_indptr, meta_suffix_indices, meta_group_indptr, meta_members;
    int64_t meta_prefix_indptr, meta_prefix_indices, meta_group_parent, meta_group_base, meta_pre_count, meta_desc;
    std::vector<int32_t> meta;        // the block itself, copied out by pkv_plan_metadata
};
