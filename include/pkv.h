/*
 * pkv.h -- batched decode attention over a paged KV cache, for AMD gfx950.
 *
 * Plain C ABI.  Every pointer is either host memory or device memory, as each
 * declaration states; no C++ or framework types cross this boundary.  All
 * device work is enqueued on the caller's HIP stream (passed as void*; NULL
 * is the default stream) on the caller's current device, and is asynchronous.
 *
 * Sources for the operations (the pages this library implements):
 *   [P1] "The 25% Page-Size Slowdown That Wasn't" -- sections "Four meanings of
 *        page size" (paged KV cache; lowering a page table into per-token
 *        indices of length B x L), "When source beats intuition" (the
 *        host plan() step; contiguous / block / scattered index layouts).
 *   [P2] "GraniKV: asymmetric KV cache paging for shared-prefix agents" --
 *        section 2 "Reuse saves prefill, not decode reads" (a shared prefix
 *        read once per step for all requests instead of once per request) and
 *        section 3 "Per-step dispatcher" (M_eff = realized batch x GQA group;
 *        dense at or above a threshold, tiled cascade below it).
 *   [P3] "Track C · Document 10 · Shrinking the footprint" -- PagedAttention
 *        Q&A (fixed-size blocks anywhere in memory, results identical to
 *        unpaged attention), block-size paragraph (block-aligned prefix
 *        matching), fp8 cache section.
 *
 * Conventions used throughout
 *   - B requests, H_q query heads, H_kv KV heads, G = H_q / H_kv (query head h
 *     reads KV head h / G), head_dim d.
 *   - q, o: row-major [B][H_q][d];  lse: [B][H_q], natural log, softmax scale
 *     included; partial states (o_f32, lse) are fp32.
 *   - K and V pools: row-major [num_slots][H_kv][d] of the KV dtype, separate
 *     tensors; num_slots = num_pages * page_size; physical page n holds slots
 *     n*p .. n*p+p-1.
 *   - kv_indptr[B+1] and kv_indices[kv_indptr[B]] are int32: request b's
 *     logical token t lives in slot kv_indices[kv_indptr[b] + t].
 *   - An empty token set gives o = 0 and lse = -inf.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory; scratch space is the caller's workspace, sized by the plan
 *     (pkv_decode_step_noalloc instead uses one fixed device array of the
 *     library's code object per GPU).  The library owns only plan handles
 *     (host heap).
 *   - Every call returns a pkv_status.  Host-detectable errors return before
 *     anything is enqueued.  Kernels do not bounds-check kv_indices
 *     (pkv_validate_indices does that on the host); a bad index faults on the
 *     device and surfaces at the caller's next synchronisation.
 *
 * Checked library.  libpkv_checked.so exports the same functions with the
 * same kernels; in it every call that takes device index arrays
 * (pkv_paged_decode_attn, pkv_paged_decode_attn_pages,
 * pkv_cascade_prefix_attn, pkv_decode_step, pkv_decode_step_noalloc,
 * pkv_decode_step_grouped) first synchronises the caller's stream, copies
 * to the host what its kernels would read of those arrays, and returns,
 * with nothing enqueued:
 *   - PKV_EINVAL when kv_indptr differs from the host kv_indptr the plan was
 *     made from, when a grouped step's metadata block differs from
 *     pkv_plan_metadata's, when page_indptr[0] < 0, or when a prefix the
 *     plan reads as one run of slots (pkv_plan_info.prefix_base) is not
 *     that run;
 *   - PKV_ERANGE when a slot the kernels would read lies outside
 *     [0, num_slots), a page outside [0, num_slots / page_size), or a
 *     request's page list holds fewer than ceil(L_b / page_size) pages.
 * It is for debugging: the synchronisation and copies cost time, and a call
 * made while the stream is being captured into a graph fails with PKV_EHIP.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

/* Every function below is exported from libpkv.so; the library's internal
 * symbols are not. */
#if defined(PKV_BUILDING_LIBRARY)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_EINVAL = -1,        /* malformed argument: null pointer, bad size, bad indptr */
    PKV_EUNSUPPORTED = -2,  /* shape / dtype combination not built */
    PKV_EWORKSPACE = -3,    /* workspace missing or smaller than the plan needs */
    PKV_ERANGE = -4,        /* an index or length outside what the tables allow */
    PKV_EHIP = -5,          /* HIP launch error */
    PKV_ENOMEM = -6         /* host allocation of a plan failed */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_BF16 = 1,
    PKV_FP8_E4M3 = 2        /* OCP e4m3fn codes; value = code * per-KV-head fp32 scale */
} pkv_dtype;

typedef enum pkv_path {
    PKV_PATH_PAGED = 0,     /* every request reads all of its tokens ([P1]) */
    PKV_PATH_CASCADE = 1,   /* prefix read once with small query tiles, + suffix, + merge ([P2] s.3) */
    PKV_PATH_DENSE = 2      /* prefix read once with large MFMA query tiles, + suffix, + merge ([P2] s.3) */
} pkv_path;

/* A caller-owned K/V pool in device memory ([P1] "Four meanings of page
 * size"; [P3] PagedAttention Q&A).  The library never frees or keeps it. */
typedef struct pkv_pool {
    const void* k;          /* device, [num_slots][num_kv_heads][head_dim] of kv_dtype */
    const void* v;          /* device, same layout as k */
    const float* k_scale;   /* device, [num_kv_heads]; required iff kv_dtype is FP8;
                               finite and > 0 (not checked: device memory) */
    const float* v_scale;   /* device, [num_kv_heads]; required iff kv_dtype is FP8 */
    int64_t num_slots;      /* must be a multiple of page_size */
    int32_t page_size;      /* tokens per page, >= 1 */
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t kv_dtype;       /* pkv_dtype */
} pkv_pool;

/* One decode step, as the planner sees it (host data only). */
typedef struct pkv_problem {
    int32_t batch;              /* B >= 0 */
    int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
    int32_t num_kv_heads;       /* H_kv >= 1 */
    int32_t head_dim;           /* 64 or 128 */
    int32_t q_dtype;            /* pkv_dtype: F32 with F32 K/V, BF16 with BF16 or FP8 K/V */
    int32_t kv_dtype;           /* pkv_dtype */
    int32_t page_size;          /* >= 1 */
    const int32_t* kv_indptr;   /* host, [B+1]: the same values as the device indptr
                                   later passed to the attention calls */
    int32_t shared_prefix_len;  /* P: the first P tokens of every request are the same
                                   tokens, stored in shared pages; 0 = no shared prefix */
    int32_t force_path;         /* -1: let the planner choose; else a pkv_path */
    const int32_t* kv_indices;  /* host, [kv_indptr[B]], optional (NULL: not given): the same
                                   values as the device indices later passed to the attention
                                   calls.  Lets the planner find a shared prefix stored as one
                                   run of consecutive slots ([P2] s.1, asymmetric placement),
                                   which the prefix pass then reads as base + offset */
} pkv_problem;

/* Constants of the planner.  pkv_tuning_defaults() returns the gfx950 values. */
typedef struct pkv_tuning {
    int32_t t_dense;            /* DENSE when M_eff >= t_dense ([P2] s.3 threshold, refitted) */
    int32_t gate_ratio;         /* PAGED when saved_bytes < gate_ratio * overhead_bytes (0: the
                                   gate is off, including the cached-prefix allowance below) */
    int64_t launch_bytes;       /* byte-equivalent of the two extra launches of a cascade */
    int32_t target_workgroups;  /* paged pass: workgroups to aim for across the GPU when it is
                                   an fp8 pass or shares its launch with prefix items; a bf16
                                   or fp32 pass on its own aims at half of it (one per CU)
                                   when its chunks then stay within one workgroup's stage */
    int32_t min_split_tokens;   /* paged pass: smallest chunk of positions per workgroup */
    int32_t concurrent_prefix;  /* 1: pkv_decode_step runs the prefix pass on a library-owned
                                   side stream (same priority) concurrently with the suffix
                                   pass, joined by events before the combine; 0: one stream */
    int32_t fuse_cascade;       /* k > 0: on a DENSE plan, pkv_decode_step runs the prefix
                                   items and the suffix chunks in one launch, interleaved so
                                   that MFMA work and HBM streaming overlap on every CU, when
                                   the prefix pass has at least k MFMA flops per byte of
                                   suffix K/V and its items fill at most half of
                                   target_workgroups; 0: always one launch per pass */
    int32_t prefix_target_workgroups; /* prefix pass: workgroups to aim for (query tiles x
                                         prefix ranges) */
    int32_t min_prefix_split_tokens;  /* prefix pass: smallest prefix range per workgroup
                                         (rounded up to a multiple of 64) */
    int32_t max_heads_per_item; /* paged pass: at most this many KV heads per work item
                                   (0: as many as one wave-wide load covers, or half of that
                                   for an fp8 pass on its own whose non-empty requests
                                   average at least 1,024 attended positions) */
    int32_t prefix_placement;   /* 1: a shared prefix whose slots are one run of consecutive
                                   slots is read by the prefix pass as base + offset, without
                                   per-token slot indices ([P2] s.1); 0: always by slot index */
    int32_t segment_tokens;     /* paged pass: the cost of one request segment in a work item,
                                   in positions.  When every request of the pass is non-empty
                                   and fits a workgroup's index stage (2,048 or 4,096
                                   positions by geometry), the planner also packs whole requests
                                   into as many bins as chunks (largest first, each to the
                                   least loaded bin) and takes the bins when their most costly
                                   one (positions + segment_tokens per request) costs less than
                                   the most costly chunk; 0: always chunks */
    int64_t cached_prefix_bytes; /* a shared prefix whose stored K and V take at most this many
                                    bytes stays in the L2 of each XCD while every request of a
                                    PAGED pass re-reads it: for such a prefix (and gate_ratio
                                    > 0) pkv_plan_create also takes PAGED while saved_bytes <
                                    cached_reread_bytes (the grouped planner does not: a
                                    dissolved group's re-reads would join the suffix pass that
                                    the kept groups' prefix items overlap); 0: off */
    int64_t cached_reread_bytes; /* see cached_prefix_bytes */
} pkv_tuning;

typedef struct pkv_plan pkv_plan;   /* opaque, immutable, host-only */

typedef struct pkv_plan_info {
    int32_t path;               /* pkv_path chosen */
    int32_t m_eff;              /* B * G ([P2] s.3) */
    int32_t shared_pages;       /* floor(P / page_size) when a prefix is declared, else 0 */
    int32_t prefix_tokens;      /* tokens the prefix pass covers (0 on PAGED) */
    int32_t split_tokens;       /* paged pass: positions per chunk.  The positions the pass
                                   attends, request after request, form one flat sequence
                                   cut into equal chunks, one per workgroup and head block */
    int32_t num_splits;         /* paged pass: most chunks one request touches (partial
                                   states per request) */
    int32_t heads_per_item;     /* paged pass: KV heads one work item covers */
    int32_t prefix_splits;      /* prefix pass: ranges the prefix is cut into */
    int64_t num_work_items;     /* paged pass: workgroups launched (chunks x head blocks) */
    int64_t workspace_bytes;    /* device scratch the plan's calls need (0 allowed) */
    int32_t num_groups;         /* grouped plans: prefix groups that run a prefix pass (else 0) */
    int64_t metadata_ints;      /* grouped plans: int32 entries of the metadata block (else 0) */
    int32_t prefix_base;        /* single-prefix plans: slot of the prefix's first token when the
                                   prefix pass reads it as one run of consecutive slots, else -1 */
    int32_t contiguous_prefixes; /* prefix runs the prefix pass reads as base + offset (single
                                    plan: 0 or 1; grouped plan: kept groups) */
    int32_t request_bins;       /* paged pass: 0 when its work items are chunks of the flat
                                   sequence; else the number of bins of whole requests (one
                                   work item per bin and head block; no request is cut, so
                                   num_splits is 1) */
} pkv_plan_info;

/* Human-readable name of a status code (static storage). */
PKV_API const char* pkv_status_string(int32_t status);

/* Library version string (static storage). */
PKV_API const char* pkv_version(void);

/* Fill *out with the gfx950 planner constants. */
PKV_API void pkv_tuning_defaults(pkv_tuning* out);

/*
 * Page table -> token-flat indices (host).  [P1] "Four meanings of page size":
 * per-page metadata expanded into one index per cached token.  Request b owns
 * pages page_indices[page_indptr[b] .. page_indptr[b+1]) in logical order and
 * seq_lens[b] tokens; token t goes to slot page * page_size + t % page_size of
 * its logical page t / page_size.
 *   page_indptr   host, [B+1], page_indptr[0] == 0, non-decreasing
 *   page_indices  host, [page_indptr[B]]
 *   seq_lens      host, [B]
 *   kv_indptr_out host, [B+1] written
 *   kv_indices_out host, [kv_indices_capacity]; sum(seq_lens) entries written
 * Errors: EINVAL (null pointer, B < 0, page_size < 1, bad indptr, negative
 * length), ERANGE (a request's page count is not ceil(seq_len / page_size), a
 * page index is negative or its slots overflow int32, or the output capacity
 * is too small).  Nothing is written on error.
 */
PKV_API pkv_status pkv_lower_page_table(int32_t batch, int32_t page_size,
                                const int32_t* page_indptr, const int32_t* page_indices,
                                const int32_t* seq_lens,
                                int32_t* kv_indptr_out, int32_t* kv_indices_out,
                                int64_t kv_indices_capacity);

/*
 * Check token-flat indices on the host before handing them to a kernel:
 * kv_indptr[0] == 0, non-decreasing, and 0 <= kv_indices[i] < num_slots.
 *   kv_indptr host [B+1]; kv_indices host [kv_indptr[B]].
 * Errors: EINVAL (null pointer, B < 0, bad indptr), ERANGE (an index outside
 * the pool).
 */
PKV_API pkv_status pkv_validate_indices(const int32_t* kv_indptr, const int32_t* kv_indices,
                                int32_t batch, int64_t num_slots);

/*
 * Plan one decode step (host only, no device work).  [P2] s.3: chooses the
 * path from M_eff = B * G and the declared shared prefix; [P1] "When source
 * beats intuition": the host metadata step before the kernels.  Also fixes the
 * paged pass's work items -- the attended positions of all requests, request
 * after request, cut into equal chunks (by logical position, so results do
 * not depend on page size or page placement) -- the prefix pass's ranges and
 * the workspace size.  tuning may be NULL (gfx950 defaults).  The problem's kv_indptr
 * (and kv_indices, if given) are read during the call and not kept.  Prefix
 * placement ([P2] s.1: a shared prefix stored contiguously is read as a plain
 * strided operand): with the problem's kv_indices given, tuning.prefix_placement
 * set and a CASCADE or DENSE path, a prefix whose slots
 * kv_indices[kv_indptr[0] + t], t < prefix_tokens, are first + t is read by the
 * prefix pass as first + t (info.prefix_base = first); otherwise slot by
 * slot.  *out receives a new handle that the caller frees with
 * pkv_plan_destroy; it can be reused on any stream for any step with the same
 * problem.
 * Errors: EINVAL (null pointer, sizes, non-multiple heads, bad indptr, prefix
 * longer than a request, bad force_path, forced prefix path with no whole
 * shared page), EUNSUPPORTED (head_dim, dtype pair, or group size not built;
 * forced prefix path for a dtype pair without a prefix kernel), ENOMEM.
 */
PKV_API pkv_status pkv_plan_create(const pkv_problem* problem, const pkv_tuning* tuning,
                           pkv_plan** out);

/*
 * Plan a decode step whose requests may share several prefixes, found in the
 * page table itself (host only).  [P3] block-size paragraph, table of
 * prompt-layout mistakes and engine comparison: prefix matching is exact and
 * aligned to blocks from the start of a sequence (two system prompts make two
 * separate trees), and a prefix cache keeps its matches as a radix tree keyed
 * on shared beginnings, so requests share a run of pages exactly when their
 * page tables name the same physical pages there; [P2] s.2-3: each shared
 * run is read once for the requests on it, with its own dispatcher decision
 * from its own realized batch.  Rules:
 *   - a request holds floor(L_b / page_size) whole pages; a partly filled
 *     last page is never shared;
 *   - the groups are the nodes of the radix tree of the requests' page lists
 *     that two or more requests share: requests whose first whole page is the
 *     same physical page form a root; a group's run is the longest stretch of
 *     pages, from where its parent's run ends, that every member holds whole
 *     and all agree on; members that hold the page after it and agree on it
 *     form a child group (two or more of them);
 *   - each group is planned as pkv_plan_create plans a step of its members
 *     alone with its run's tokens as the declared prefix (gate, DENSE or
 *     CASCADE, force_path); a group planned PAGED is dissolved (its run is
 *     read in the paged pass; its children are still planned);
 *   - groups are numbered depth first (parents first, siblings by first
 *     member), members in request order.
 * The problem's kv_indptr is ignored (may be NULL) and its shared_prefix_len
 * must be 0.  page_indptr [B+1], page_indices, seq_lens [B] are host arrays
 * as for pkv_lower_page_table, read during the call.  The plan holds the
 * lowered indices of the step in its metadata block (pkv_plan_metadata),
 * which the caller copies to the device once for pkv_decode_step_grouped.
 * Plan info: path is PAGED without groups, DENSE if a group runs DENSE, else
 * CASCADE; m_eff is the largest group's; shared_pages and prefix_tokens are
 * summed over the groups' runs; prefix_splits is the most prefix partial
 * states of any request (the ranges of all of its groups).
 * Errors: as pkv_plan_create and pkv_lower_page_table; EINVAL also for a
 * non-zero shared_prefix_len.
 */
PKV_API pkv_status pkv_plan_create_grouped(const pkv_problem* problem, const pkv_tuning* tuning,
                                   const int32_t* page_indptr, const int32_t* page_indices,
                                   const int32_t* seq_lens, pkv_plan** out);

/*
 * Copy a grouped plan's metadata block (info.metadata_ints int32 entries)
 * to host memory out[capacity].  Layout, each array right after the one
 * before (NG = info.num_groups):
 *   suffix_indptr  [B+1]   token offsets of each request's own tokens
 *   suffix_indices [suffix_indptr[B]]  slots of request b's tokens outside
 *                  the runs of its kept groups, in logical order
 *   group_indptr   [NG+1]  offsets into group_members
 *   group_members  [group_indptr[NG]]  requests of each group
 *   prefix_indptr  [NG+1]  offsets into prefix_indices
 *   prefix_indices [prefix_indptr[NG]]  slots of each group's run of tokens
 *   group_parent   [NG]    nearest enclosing kept group, -1 for none
 *   group_prefix_base [NG] slot of the first token of each group's run when
 *                  the run is one stretch of consecutive physical pages and the
 *                  tuning's prefix_placement is set (read as base + offset),
 *                  else -1
 *   followed by tables only the kernels read.
 * Errors: EINVAL (null plan, plan not from pkv_plan_create_grouped, null out
 * with a non-empty block), ERANGE (capacity too small).
 */
PKV_API pkv_status pkv_plan_metadata(const pkv_plan* plan, int32_t* out, int64_t capacity);

/* Host inspection of a plan whose paged pass runs on bins of whole requests
 * (pkv_plan_info.request_bins = W > 0; see pkv_tuning.segment_tokens): out
 * receives bin_start [W+1] (bin w holds entries bin_start[w] ..
 * bin_start[w+1] - 1 of the list) followed by the list of request indices
 * [B], each bin's in increasing order.  The bins travel to the kernels with
 * the plan itself; nothing needs uploading.  Errors: EINVAL (null plan, a
 * plan without bins, null out), ERANGE (capacity < W + 1 + B). */
PKV_API pkv_status pkv_plan_request_bins(const pkv_plan* plan, int32_t* out, int64_t capacity);

/* Copy a plan's decisions and sizes into *info.  EINVAL on null pointers. */
PKV_API pkv_status pkv_plan_get_info(const pkv_plan* plan, pkv_plan_info* info);

/* Free a plan handle (NULL is allowed). */
PKV_API void pkv_plan_destroy(pkv_plan* plan);

/*
 * Paged decode attention ([P1] "Four meanings of page size"; [P3]
 * PagedAttention Q&A): each request's query attends over the K/V rows that
 * kv_indices lists for it.  On a PAGED plan the call covers every token of
 * each request; on a CASCADE or DENSE plan it covers only tokens
 * [prefix_tokens, L_b), the suffix that follows the shared prefix, and its
 * fp32 state is then merged with the prefix pass by pkv_merge_states.
 *   q           device, [B][H_q][d] of the plan's q dtype
 *   pool        host struct describing device memory; must match the plan
 *   kv_indptr   device, [B+1] int32, same values as the plan's host indptr
 *   kv_indices  device, [kv_indptr[B]] int32 slots
 *   sm_scale    softmax scale (e.g. 1/sqrt(d)), finite and > 0; else PKV_EINVAL
 *               (the kernels scale row maxima of unscaled scores)
 *   o           device, [B][H_q][d] of the q dtype, normalised output; nullable
 *   o_f32       device, [B][H_q][d] fp32, normalised output; nullable
 *   lse         device, [B][H_q] fp32; nullable
 *   workspace   device scratch of >= the plan's workspace_bytes (nullable if 0),
 *               no initial contents needed.  Calls that share a workspace must
 *               not overlap.
 * At least one of o, o_f32 must be given.  Writes no other memory.
 * Errors: EINVAL (null plan/q/indices, no output, pool not matching the plan,
 * missing fp8 scales), EWORKSPACE, EHIP.
 */
PKV_API pkv_status pkv_paged_decode_attn(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                                 const int32_t* kv_indptr, const int32_t* kv_indices,
                                 float sm_scale, void* o, float* o_f32, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same operation reading the page table instead of token-flat indices
 * ([P1] "A backend where pages really do reach the kernel": per-page
 * metadata consumed by the kernel itself; "Four meanings of page size").
 * Logical position t of request b is slot
 * page_indices[page_indptr[b] + t / page_size] * page_size + t % page_size,
 * with page_size from the plan.  Output is bit for bit that of
 * pkv_paged_decode_attn over the lowered indices (same plan, same kernels).
 *   kv_indptr     device, [B+1] int32 token offsets: kv_indptr[b+1] - kv_indptr[b]
 *                 = L_b, the same values as the plan's host indptr
 *   page_indptr   device, [B+1] int32; request b owns ceil(L_b / page_size) pages
 *   page_indices  device, [page_indptr[B]] int32 physical page numbers
 * Other arguments as pkv_paged_decode_attn.  The kernels do not bounds-check
 * the page table (pkv_lower_page_table does on the host).
 * Errors: EINVAL (null plan/q/indptr/page table, no output, pool not matching
 * the plan, missing fp8 scales), EWORKSPACE, EHIP.
 */
PKV_API pkv_status pkv_paged_decode_attn_pages(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                                       const int32_t* kv_indptr, const int32_t* page_indptr,
                                       const int32_t* page_indices, float sm_scale, void* o,
                                       float* o_f32, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Shared-prefix attention, prefix read once for the whole batch ([P2] s.2:
 * every request needs the whole prefix each step, so it is read once instead
 * of once per request; s.3: DENSE or tiled CASCADE by M_eff).  For each KV
 * head, the G query heads of all B requests (M_eff rows) attend over the
 * prefix_tokens rows listed by prefix_indices.
 *   q              device, [B][H_q][d] bf16
 *   prefix_indices device, [prefix_len] int32 slots (typically request 0's
 *                  first prefix_len entries of kv_indices).  When the plan's
 *                  prefix_base is set the pass reads slots prefix_base + t
 *                  instead and does not read this array (it must hold the
 *                  same slots, as the plan saw them)
 *   prefix_len     must equal the plan's prefix_tokens
 *   o_p            device, [B][H_q][d] fp32, normalised prefix output
 *   lse_p          device, [B][H_q] fp32
 * Errors: EINVAL (PAGED plan, null pointers, prefix_len mismatch, pool not
 * matching), EWORKSPACE, EHIP.
 */
PKV_API pkv_status pkv_cascade_prefix_attn(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                                   const int32_t* prefix_indices, int32_t prefix_len,
                                   float sm_scale, float* o_p, float* lse_p,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Log-sum-exp combine of two partial softmax states over disjoint token sets
 * (the step that joins the read-once prefix with each request's suffix, [P2]
 * s.2-3).  Row by row: M = max(lse_a, lse_b); w = exp(lse - M);
 * o = (w_a o_a + w_b o_b) / (w_a + w_b); lse = M + ln(w_a + w_b); two empty
 * states give o = 0, lse = -inf.
 *   o_a, o_b  device, [rows][d] fp32;  lse_a, lse_b  device, [rows] fp32
 *   o_out     device, [rows][d] of out_dtype (F32 or BF16)
 *   lse_out   device, [rows] fp32; nullable
 * Errors: EINVAL (null pointers, rows < 0, d not in {64,128}),
 * EUNSUPPORTED (out_dtype), EHIP.
 */
PKV_API pkv_status pkv_merge_states(int32_t rows, int32_t head_dim,
                            const float* o_a, const float* lse_a,
                            const float* o_b, const float* lse_b,
                            void* o_out, int32_t out_dtype, float* lse_out, void* stream);

/*
 * One whole decode step as the plan chose it: PAGED is one paged call; CASCADE
 * and DENSE run the prefix pass over kv_indices[kv_indptr[0] ..
 * + prefix_tokens) (request 0's shared pages), the paged pass over each
 * request's suffix, and one kernel that combines both passes' partial
 * states (kept in the workspace).  On a DENSE plan that meets the tuning's
 * fuse_cascade rule the two passes are one launch whose workgroups run
 * either a prefix item or a suffix chunk.  Otherwise, with concurrent_prefix set in the plan's
 * tuning, the prefix pass is enqueued on a side stream that the library
 * creates once per device (default priority), forked from and joined back
 * to `stream` with events, so the MFMA-bound prefix pass and the
 * bandwidth-bound suffix pass overlap; the call is still ordered on
 * `stream` as a whole and can be captured into a graph.  Arguments as in
 * pkv_paged_decode_attn; o is required, lse is nullable.
 */
PKV_API pkv_status pkv_decode_step(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           float sm_scale, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Size of the device scratch array behind pkv_decode_step_noalloc (bytes per
 * GPU, held from the first call on that GPU until the process ends). */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pkv_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same step, same kernels and same results as pkv_decode_step, but the
 * partial states live in a library-owned device array of
 * PKV_NOALLOC_SCRATCH_BYTES per GPU instead of a caller's workspace (its
 * address on the current device is looked up once per device, on the first
 * call there; nothing is allocated by any call).  The prefix pass always
 * runs on `stream` (the plan's concurrent_prefix side stream is not used).
 * The scratch keeps the last call's contents; nothing in it needs clearing.
 * Calls that overlap on one GPU (on different streams or host threads)
 * share the array and race: serialise them.
 *   Arguments as pkv_decode_step, without the workspace; o is required, lse
 *   is nullable.
 * Errors: EINVAL (as pkv_decode_step), EWORKSPACE (the plan's workspace_bytes
 * exceeds PKV_NOALLOC_SCRATCH_BYTES; nothing is enqueued), EHIP.
 */
PKV_API pkv_status pkv_decode_step_noalloc(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                                   const int32_t* kv_indptr, const int32_t* kv_indices, float sm_scale,
                                   void* o, float* lse, void* stream);

/*
 * One decode step of a grouped plan: one prefix pass over every group's run
 * (each read once for the group's requests; DENSE groups and CASCADE groups
 * in one launch each, or with the suffix pass in one launch when every group
 * is DENSE), the paged pass over every request's suffix, and one kernel that
 * combines, per row, the prefix ranges of all its groups and its suffix
 * chunks into o (and lse).  The result is that of attention
 * over each request's whole sequence.
 *   metadata  device copy of the plan's metadata block (pkv_plan_metadata)
 * Other arguments as pkv_decode_step; o is required, lse is nullable.
 * Errors: EINVAL (null plan/q/metadata/o, plan not grouped, pool not
 * matching), EWORKSPACE, EHIP.
 */
PKV_API pkv_status pkv_decode_step_grouped(const pkv_plan* plan, const void* q, const pkv_pool* pool,
                                   const int32_t* metadata, float sm_scale, void* o, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement aid: read `bytes` of device memory at `buf` once (each of
 * num_workgroups workgroups of 256 threads streams one contiguous block with
 * 16-byte non-temporal loads) and write one word per workgroup to
 * out[num_workgroups] (device).  Its duration gives the
 * streaming-read bandwidth ceiling of the GPU, against which the attention
 * kernels' achieved bandwidth is compared ([P1] "When source beats
 * intuition" and "A backend where pages really do reach the kernel" measure
 * decode kernels by their fraction of peak DRAM throughput).
 * Errors: EINVAL (null pointers, bytes not a multiple of 16, misaligned buf,
 * num_workgroups < 1), EHIP.
 */
PKV_API pkv_status pkv_stream_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t num_workgroups,
                                 void* stream);

/*
 * Measurement aid: fill `bytes` of device memory at `buf` with the 32-bit
 * `value` (each of num_workgroups workgroups of 256 threads writes one
 * contiguous block with 16-byte stores).  Its bytes are known exactly, so
 * the write-traffic counters of a profiler can be calibrated against it
 * before they are read for the attention kernels.
 * Errors: EINVAL (null buf, bytes not a multiple of 16, misaligned buf,
 * num_workgroups < 1), EHIP.
 */
PKV_API pkv_status pkv_stream_write_probe(void* buf, int64_t bytes, uint32_t value, int32_t num_workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
