// Run-time selection of the paged kernel instantiation for one K/V dtype.
#pragma once

#include "paged_kernel.h"

namespace pkv {

template <int KV, int D, int G, int NHL, int TPI>
hipError_t launch_one(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    const dim3 grid(p.num_splits, p.head_blocks, p.B);
    paged_split_kernel<KV, D, G, NHL, TPI><<<grid, kPagedWaves * 64, 0, s>>>(a);
    return hipGetLastError();
}

template <int KV, int D, int G>
hipError_t dispatch_layout(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    using C1 = PagedCfg<KV, D, G, 1, 1>;
    constexpr int RS = C1::RS;
    const int nhl = p.geo.nhl, tpi = p.geo.tpi;
    if (nhl == 2) {
        if constexpr (2 * G * C1::EPL <= 64) return launch_one<KV, D, G, 2, 1>(p, a, s);
        return hipErrorInvalidValue;
    }
    switch (tpi) {
        case 1: return launch_one<KV, D, G, 1, 1>(p, a, s);
        case 2:
            if constexpr (RS >= 2) return launch_one<KV, D, G, 1, 2>(p, a, s);
            break;
        case 4:
            if constexpr (RS >= 4) return launch_one<KV, D, G, 1, 4>(p, a, s);
            break;
        case 8:
            if constexpr (RS >= 8) return launch_one<KV, D, G, 1, 8>(p, a, s);
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

template <int KV, int D>
hipError_t dispatch_group(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    switch (p.G) {
        case 1: return dispatch_layout<KV, D, 1>(p, a, s);
        case 2: return dispatch_layout<KV, D, 2>(p, a, s);
        case 4: return dispatch_layout<KV, D, 4>(p, a, s);
        case 8: return dispatch_layout<KV, D, 8>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int KV>
hipError_t dispatch_kv(const pkv_plan& p, const PagedArgs& a, hipStream_t s) {
    if (p.geo.epl != KvTraits<KV>::EPL) return hipErrorInvalidValue;
    if (p.D == 128) return dispatch_group<KV, 128>(p, a, s);
    if (p.D == 64) return dispatch_group<KV, 64>(p, a, s);
    return hipErrorInvalidValue;
}

}  // namespace pkv
