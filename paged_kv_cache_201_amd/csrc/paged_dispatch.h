// Run-time selection of a kernel instantiation for the plan's K/V dtype,
// head_dim, group size and lane layout.  A launcher L provides
//   template <int KV, int D, int G, int NHL, int TPI> hipError_t run() const;
#pragma once

#include "paged_kernel.h"

namespace pkv {

template <int KV, int D, int G, class L>
hipError_t dispatch_layout(const pkv_plan& p, const L& l) {
    using C1 = PagedCfg<KV, D, G, 1, 1>;
    constexpr int RS = C1::RS;
    if (p.geo.nhl != 1) return hipErrorInvalidValue;
    switch (p.geo.tpi) {
        case 1: return l.template run<KV, D, G, 1, 1>();
        case 2:
            if constexpr (RS >= 2) return l.template run<KV, D, G, 1, 2>();
            break;
        case 4:
            if constexpr (RS >= 4) return l.template run<KV, D, G, 1, 4>();
            break;
        case 8:
            if constexpr (RS >= 8) return l.template run<KV, D, G, 1, 8>();
            break;
        default: break;
    }
    return hipErrorInvalidValue;
}

template <int KV, int D, class L>
hipError_t dispatch_group(const pkv_plan& p, const L& l) {
    switch (p.G) {
        case 1: return dispatch_layout<KV, D, 1>(p, l);
        case 2: return dispatch_layout<KV, D, 2>(p, l);
        case 4: return dispatch_layout<KV, D, 4>(p, l);
        case 8: return dispatch_layout<KV, D, 8>(p, l);
        default: return hipErrorInvalidValue;
    }
}

template <int KV, class L>
hipError_t dispatch_kv(const pkv_plan& p, const L& l) {
    if (p.geo.epl != KvTraits<KV>::EPL) return hipErrorInvalidValue;
    if (p.D == 128) return dispatch_group<KV, 128>(p, l);
    if (p.D == 64) return dispatch_group<KV, 64>(p, l);
    return hipErrorInvalidValue;
}

// The paged kernel: one workgroup per (chunk, head block).
struct PagedLaunch {
    const pkv_plan& p;
    const PagedArgs& a;
    hipStream_t s;
    template <int KV, int D, int G, int NHL, int TPI>
    hipError_t run() const {
        const dim3 grid((uint32_t)p.num_chunks, p.head_blocks, 1);
        paged_split_kernel<KV, D, G, NHL, TPI><<<grid, kPagedWaves * 64, 0, s>>>(a);
        return hipGetLastError();
    }
};

}  // namespace pkv
