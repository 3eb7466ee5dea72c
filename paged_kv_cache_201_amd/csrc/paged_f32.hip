// Paged decode kernels with f32 K/V.
#include "paged_dispatch.h"

namespace pkv {
hipError_t launch_paged_split_f32(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    return dispatch_kv<PKV_F32>(p, PagedLaunch{p, a, s});
}
}  // namespace pkv
