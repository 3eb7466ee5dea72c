// Streaming-read ceiling: reads a device buffer once with 16-byte loads from
// a full grid and folds it into one word per workgroup, so that measured
// bandwidth of the attention kernels can be set against what a plain stream
// achieves on the same GPU ("The 25% Page-Size Slowdown That Wasn't",
// sections "When source beats intuition" and "A backend where pages really
// do reach the kernel": decode kernels judged by their fraction of peak DRAM
// throughput).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv.h"

namespace pkv {

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ out) {
    const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t acc = 0;
    size_t i = tid;
    // four independent loads in flight per iteration
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4_t a = __builtin_nontemporal_load(src + i);
        const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
        const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
        acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
    }
    for (; i < n16; i += stride) {
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
