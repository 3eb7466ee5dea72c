// Streaming-read ceiling: reads a device buffer once with 16-byte loads from
// a full grid and folds it into one word per workgroup, so that measured
// bandwidth of the attention kernels can be set against what a plain stream
// achieves on the same GPU ("The 25% Page-Size Slowdown That Wasn't",
// sections "When source beats intuition" and "A backend where pages really
// do reach the kernel": decode kernels measured by their fraction of peak DRAM
// throughput).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv.h"

namespace pkv {

// Each workgroup reads one contiguous block of the buffer, eight 16-byte
// non-temporal loads in flight per thread: on gfx950 this pattern streams
// faster than a grid-strided sweep, whose concurrent accesses crowd the same
// memory channels.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
    constexpr int UNROLL = 8;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < n16 ? beg + per : n16;
    uint32_t acc = 0;
    size_t i = beg + threadIdx.x;
    for (; i + (UNROLL - 1) * 256 < end; i += UNROLL * 256) {
        u32x4_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < end; i += 256) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    __shared__ uint32_t s[256];
    s[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int k = 0; k < 256; ++k) r ^= s[k];
        out[blockIdx.x] = r;
    }
}

// The write-side companion: each workgroup fills one contiguous block with
// 16-byte stores of a constant.  Its bytes are known exactly, which is what a
// write-traffic counter is calibrated against.
__global__ void __launch_bounds__(256) stream_write_kernel(u32x4_t* __restrict__ dst, size_t n16, uint32_t value) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < n16 ? beg + per : n16;
    const u32x4_t v = {value, value, value, value};
    for (size_t i = beg + threadIdx.x; i < end; i += 256) dst[i] = v;
}

}  // namespace pkv

extern "C" pkv_status pkv_stream_read_probe(const void* buf, int64_t bytes, uint32_t* out, int32_t num_workgroups,
                                            void* stream) {
    if (!buf || !out || bytes < 0 || num_workgroups < 1 || (bytes % 16) ||
        (reinterpret_cast<uintptr_t>(buf) % 16))
        return PKV_EINVAL;
    pkv::stream_read_kernel<<<num_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const pkv::u32x4_t*>(buf), (size_t)(bytes / 16), out);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

extern "C" pkv_status pkv_stream_write_probe(void* buf, int64_t bytes, uint32_t value, int32_t num_workgroups,
                                             void* stream) {
    if (!buf || bytes < 0 || num_workgroups < 1 || (bytes % 16) || (reinterpret_cast<uintptr_t>(buf) % 16))
        return PKV_EINVAL;
    pkv::stream_write_kernel<<<num_workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<pkv::u32x4_t*>(buf), (size_t)(bytes / 16), value);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
