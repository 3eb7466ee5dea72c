// Shared-prefix attention kernels (the body is in prefix_kernel.h).
#include "prefix_kernel.h"

namespace pkv {

template <int D, int NW, int KT>
__global__ void __launch_bounds__(NW * 64, (NW >= 4 ? 2 : 1)) prefix_attn_kernel(const PrefixArgs a) {
    __shared__ PrefixSmem<D, KT> sm;
    prefix_item<D, NW, KT>(a, sm, blockIdx.x);
}

hipError_t launch_prefix_attn(const PrefixArgs& a, int rows_per_wg, hipStream_t stream) {
    const int N = a.groups ? a.num_items : a.row_tiles * a.H_kv * a.num_splits;
    if (N == 0) return hipSuccess;
    if (!a.groups && a.split_tokens > kMaxPrefixSplitTokens) return hipErrorInvalidValue;
    const int grid = prefix_blocks(N);
    // DENSE: 4 waves x 32 rows share each tile; CASCADE: 2 waves x 32 rows
    // (small query tiles, more workgroups per CU).  Both stay within 256
    // registers per lane, so a prefix workgroup and a paged workgroup can be
    // resident on one CU together.
    if (rows_per_wg == kDenseRowsPerWg) {
        if (a.D == 128) prefix_attn_kernel<128, 4, 32><<<grid, 256, 0, stream>>>(a);
        else prefix_attn_kernel<64, 4, 32><<<grid, 256, 0, stream>>>(a);
    } else {
        if (a.D == 128) prefix_attn_kernel<128, 2, 32><<<grid, 128, 0, stream>>>(a);
        else prefix_attn_kernel<64, 2, 32><<<grid, 128, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace pkv
