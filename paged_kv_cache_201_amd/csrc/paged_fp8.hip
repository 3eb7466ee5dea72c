// Paged decode kernels with fp8 K/V.
#include "paged_dispatch.h"

namespace pkv {
hipError_t launch_paged_split_fp8(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    return dispatch_kv<PKV_FP8_E4M3>(p, PagedLaunch{p, a, s});
}
}  // namespace pkv
