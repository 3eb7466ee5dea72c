// Shared-prefix attention kernels (the body is in prefix_kernel.h).
#include "prefix_kernel.h"

namespace pkv {

template <int D, int NW, int KT>
__global__ void __launch_bounds__(NW * 64, (NW >= 4 ? 2 : 1)) prefix_attn_kernel(const PrefixArgs a) {
    __shared__ PrefixSmem<D, KT> sm;
    prefix_item<PKV_BF16, D, NW, KT>(a, sm, blockIdx.x);
}

// fp8 e4m3 K/V (head_dim 128): the codes stream into LDS and each MFMA
// operand is widened in registers as it is read (see PrefixSmem8).
template <int NW>
__global__ void __launch_bounds__(NW * 64, (NW >= 4 ? 2 : 1)) prefix_attn_fp8_kernel(const PrefixArgs a) {
    __shared__ PrefixSmem8<128, 32> sm;
    prefix_item<PKV_FP8_E4M3, 128, NW, 32>(a, sm, blockIdx.x);
}

hipError_t launch_prefix_attn(const PrefixArgs& a, int rows_per_wg, hipStream_t stream) {
    const int N = a.groups ? a.num_items : a.row_tiles * a.H_kv * a.num_splits;
    if (N == 0) return hipSuccess;
    if (!a.groups && a.split_tokens > kMaxPrefixSplitTokens) return hipErrorInvalidValue;
    const int grid = prefix_blocks(N);
    // DENSE: 4 waves x 32 rows share each tile, within 256 registers per lane
    // so that a prefix workgroup and a paged workgroup fit on one CU together;
    // CASCADE: 2 waves x 32 rows (small query tiles).
    const bool dense = rows_per_wg == kDenseRowsPerWg;
    if (a.kv_dtype == PKV_FP8_E4M3) {
        if (a.D != 128 || !a.k_scale || !a.v_scale) return hipErrorInvalidValue;
        if (dense) prefix_attn_fp8_kernel<4><<<grid, 256, 0, stream>>>(a);
        else prefix_attn_fp8_kernel<2><<<grid, 128, 0, stream>>>(a);
    } else if (a.kv_dtype == PKV_BF16) {
        if (dense) {
            if (a.D == 128) prefix_attn_kernel<128, 4, 32><<<grid, 256, 0, stream>>>(a);
            else prefix_attn_kernel<64, 4, 32><<<grid, 256, 0, stream>>>(a);
        } else {
            if (a.D == 128) prefix_attn_kernel<128, 2, 32><<<grid, 128, 0, stream>>>(a);
            else prefix_attn_kernel<64, 2, 32><<<grid, 128, 0, stream>>>(a);
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pkv
