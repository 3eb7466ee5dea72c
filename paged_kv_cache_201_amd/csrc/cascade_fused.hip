// One launch for both passes of a DENSE cascade step (bf16 K/V, or fp8 K/V
// at head_dim 128).
//
// The prefix pass is bound by MFMA and LDS work (the prefix is read once for
// all requests: "GraniKV: asymmetric KV cache paging for shared-prefix
// agents", sections 2 and 3); the suffix pass of the same step streams each
// request's own K/V rows from HBM.  Launched one after the other, each kernel
// leaves the other's resource idle.  Here every workgroup runs either one
// prefix work item or one suffix chunk, so that a CU can hold one of each:
// while the prefix item waits on MFMA results and LDS, the suffix chunk keeps
// HBM reads in flight.  Both bodies use 256 threads and at most 256 VGPRs per
// lane, and they share the LDS allocation, which leaves room for two
// workgroups per CU.  Results are the same partial states the two separate
// kernels write.
//
// Wave priority.  A CU's two roles compete for instruction issue; the
// suffix role runs at wave priority 1 (see below).
//
// Role order.  The dispatcher hands workgroups, in launch order, to the CU
// with the most free room, so the first workgroups of a launch land one per
// CU.  All prefix items therefore come first (the planner fuses only when
// they are at most half its target of workgroups: one per CU at the default
// target of two per CU), then the suffix chunks, which fill the
// second place of every CU.  Interleaving the two kinds in groups of eight
// instead put two prefix items on some CUs and two suffix chunks on others:
// each role alone then ran 18-26 % slower than as its own kernel.
#include <type_traits>

#include "paged_dispatch.h"
#include "prefix_kernel.h"

namespace pkv {

// Role of workgroup i among np prefix workgroups (a multiple of 8), then the
// suffix workgroups.  Prefix index p = i keeps p % 8 == i % 8, the XCD the
// workgroup runs on, as prefix_item assumes.
__device__ __forceinline__ void fused_role(const int i, const int np, bool& is_prefix, int& idx) {
    is_prefix = i < np;
    idx = is_prefix ? i : i - np;
}

template <int KV, int D, int G, int NHL, int TPI>
__global__ void __launch_bounds__(kPagedWaves * 64, 2)
    cascade_fused_kernel(const PrefixArgs pa, const PagedArgs sa, const int np, const int hblks) {
    using PS = typename std::conditional<KV == PKV_FP8_E4M3, PrefixSmem8<D, 32>, PrefixSmem<D, 32>>::type;
    using SS = PagedSmem<KV, D, G, NHL, TPI>;
    constexpr size_t kBytes = sizeof(PS) > sizeof(SS) ? sizeof(PS) : sizeof(SS);
    __shared__ __attribute__((aligned(16))) char smem[kBytes];
    bool is_prefix;
    int idx;
    fused_role(blockIdx.x, np, is_prefix, idx);
    if (is_prefix) {
        prefix_item<KV, D, kPagedWaves, 32>(pa, *reinterpret_cast<PS*>(smem), idx);
    } else {
        // The suffix role's waves issue ahead of the co-resident prefix
        // role's (wave priority 1 against 0), so that its loads keep HBM
        // busy while the prefix item's MFMA and softmax work fills the
        // gaps: the shared-prefix step's fused kernel 79.9 -> 72.3 us, the
        // several-prompt step -1 %, the nested tree +1.5 %
        __builtin_amdgcn_s_setprio(1);
        paged_chunk<KV, D, G, NHL, TPI>(sa, *reinterpret_cast<SS*>(smem), idx / hblks, idx % hblks);
    }
}

namespace {
struct FusedLaunch {
    const pkv_plan& p;
    const PrefixArgs& pa;
    const PagedArgs& sa;
    hipStream_t s;
    template <int KV, int D, int G, int NHL, int TPI>
    hipError_t run() const {
        // bf16, or fp8 at head_dim 128 (the fp8 prefix kernel's shape)
        if constexpr (KV == PKV_F32 || (KV == PKV_FP8_E4M3 && D != 128)) {
            return hipErrorInvalidValue;
        } else {
            const int np = prefix_blocks(pa.groups ? pa.num_items : pa.row_tiles * pa.H_kv * pa.num_splits);
            const int64_t ns = p.num_chunks * p.head_blocks;
            if (np + ns > INT32_MAX) return hipErrorInvalidValue;
            if (np + ns == 0) return hipSuccess;
            cascade_fused_kernel<KV, D, G, NHL, TPI>
                <<<(uint32_t)(np + ns), kPagedWaves * 64, 0, s>>>(pa, sa, np, p.head_blocks);
            return hipGetLastError();
        }
    }
};
}  // namespace

hipError_t launch_cascade_fused(const pkv_plan& p, const PrefixArgs& pa, const PagedArgs& sa, hipStream_t s) {
    if (!pa.groups && pa.split_tokens > kMaxPrefixSplitTokens) return hipErrorInvalidValue;
    if (p.kv_dtype == PKV_FP8_E4M3) return dispatch_kv<PKV_FP8_E4M3>(p, FusedLaunch{p, pa, sa, s});
    return dispatch_kv<PKV_BF16>(p, FusedLaunch{p, pa, sa, s});
}

}  // namespace pkv
