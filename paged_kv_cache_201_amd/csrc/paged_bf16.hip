// Paged decode kernels with bf16 K/V.
#include "paged_dispatch.h"

namespace pkv {
hipError_t launch_paged_split_bf16(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    return dispatch_kv<PKV_BF16>(p, PagedLaunch{p, a, s});
}
}  // namespace pkv
