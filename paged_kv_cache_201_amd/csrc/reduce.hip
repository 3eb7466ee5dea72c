// Split-K reduction of the paged pass, and the two-state LSE merge.
//
// Both combine partial softmax states over disjoint token sets.  The
// combination follows from the softmax definition: with state (o, lse) for a
// token set, the state of the union of two sets is
//   M = max(lse_a, lse_b),  w = exp(lse - M),
//   o = (w_a o_a + w_b o_b) / (w_a + w_b),  lse = M + ln(w_a + w_b).
// It is the step that joins a prefix read once for the whole batch with each
// request's own suffix ("GraniKV: asymmetric KV cache paging for
// shared-prefix agents", sections 2 and 3).  Splits are combined in index
// order, so results are reproducible bit for bit.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

// Partials whose loads are issued together.  Four keep the kernel at about
// 50 VGPRs, eight waves per SIMD, so that a grid of 2,048 workgroups (16,384
// rows at head_dim 128) is resident in one round; a row with more partials
// takes one more memory round trip per four.  Rows of five to eight
// partials (a four-range prefix and a suffix) take one batch of eight.
constexpr int kReduceBatch = 4;
constexpr int kReduceBatchWide = 8;

// Thread (row, e4) owns four consecutive outputs of one row.  The row's
// partials are the pre_splits prefix partials (if any) followed by the chunk
// partials of its request (if any); each holds a (max, sum) pair, max = -inf
// for an empty state.  They are consumed in batches whose loads are all
// issued before any is used, so a batch costs one memory round trip;
// batches are combined in order with the usual rescaling.
template <int D, int BATCH>
__global__ void __launch_bounds__(256) split_reduce_kernel(const SplitReduceArgs a) {
    constexpr int CH = D / 4;
    constexpr int RPB = 256 / CH;
    const int row = blockIdx.x * RPB + threadIdx.x / CH;
    const int e4 = threadIdx.x % CH;
    if (row >= a.B * a.H_q) return;
    const int b = row / a.H_q;
    const int qh = row % a.H_q;
    const int npre = a.pre_acc ? (a.pre_count ? a.pre_count[b] : a.pre_splits) : 0;
    int nparts = 0;
    if (a.kv_indptr && a.whole_requests) {
        // bins of whole requests: the plan has no empty request, and each
        // request's positions are one segment with one partial state, so
        // the partials are loaded without a round trip to kv_indptr first
        nparts = a.skip_whole ? 0 : (a.part_acc ? min(1, a.max_parts) : 0);
        if (a.skip_whole) return;  // written by the paged kernel
    } else if (a.kv_indptr) {
        // the chunks that request b's positions [ob, on) of the flat sequence touch
        const int64_t base = (int64_t)a.kv_indptr[0];
        const int64_t ob = a.kv_indptr[b] - base - (int64_t)b * a.token_offset;
        const int64_t on = a.kv_indptr[b + 1] - base - (int64_t)(b + 1) * a.token_offset;
        if (on > ob) {
            nparts = (int)((on - 1) / a.chunk_tokens - ob / a.chunk_tokens + 1);
            if (a.skip_whole && nparts == 1) return;  // written by the paged kernel
            nparts = a.part_acc ? min(nparts, a.max_parts) : 0;
        }
    }
    const int total = npre + nparts;
    float L = 0.f, M = -INFINITY;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < total; k0 += BATCH) {
        f32x2_t ml[BATCH];
        f32x4_t x[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int k = k0 + j;
            if (k < total) {
                const bool pre = k < npre;
                const size_t prow = pre ? ((size_t)b * a.pre_splits + k) * a.H_q + qh
                                        : ((size_t)b * a.max_parts + (k - npre)) * a.H_q + qh;
                ml[j] = *reinterpret_cast<const f32x2_t*>((pre ? a.pre_ml : a.part_ml) + prow * 2);
                x[j] = *reinterpret_cast<const f32x4_t*>((pre ? a.pre_acc : a.part_acc) + prow * D + e4 * 4);
            } else {
                ml[j] = f32x2_t{-INFINITY, 0.f};
                x[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) Mc = fmaxf(Mc, ml[j][0]);
        if (Mc == -INFINITY) continue;
        const float c = M == -INFINITY ? 0.f : exp2f(M - Mc);  // rescale what is summed so far
        L *= c;
        o *= c;
        M = Mc;
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const float w = ml[j][0] == -INFINITY ? 0.f : exp2f(ml[j][0] - M);
            L += w * ml[j][1];
            if (w > 0.f) o += w * x[j];  // an empty item's values are never read into the sum
        }
    }
    o *= L > 0.f ? 1.f / L : 0.f;
    const size_t orow = (size_t)row;
    if (a.o_f32) *reinterpret_cast<f32x4_t*>(a.o_f32 + orow * D + e4 * 4) = o;
    if (a.o) {
        if (a.out_dtype == PKV_F32) {
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.o) + orow * D + e4 * 4) = o;
        } else {
            u32x2_t h = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.o) + orow * D + e4 * 4) = h;
        }
    }
    if (a.lse && e4 == 0) a.lse[orow] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

template <int D>
__global__ void __launch_bounds__(256) merge_states_kernel(int rows, const float* __restrict__ o_a,
                                                           const float* __restrict__ lse_a,
                                                           const float* __restrict__ o_b,
                                                           const float* __restrict__ lse_b,
                                                           void* __restrict__ o_out, int out_dtype,
                                                           float* __restrict__ lse_out) {
    constexpr int CH = D / 4;
    constexpr int RPB = 256 / CH;
    const int row = blockIdx.x * RPB + threadIdx.x / CH;
    const int e4 = threadIdx.x % CH;
    if (row >= rows) return;
    const float la = lse_a[row], lb = lse_b[row];
    const float M = fmaxf(la, lb);
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (M != -INFINITY) {
        const float wa = expf(la - M), wb = expf(lb - M);
        const float inv = 1.f / (wa + wb);
        const f32x4_t xa = *reinterpret_cast<const f32x4_t*>(o_a + (size_t)row * D + e4 * 4);
        const f32x4_t xb = *reinterpret_cast<const f32x4_t*>(o_b + (size_t)row * D + e4 * 4);
        // an empty side has weight 0; never multiply its (possibly stale) values
        if (wa > 0.f) o += (wa * inv) * xa;
        if (wb > 0.f) o += (wb * inv) * xb;
        lse = M + logf(wa + wb);
    }
    if (out_dtype == PKV_F32) {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(o_out) + (size_t)row * D + e4 * 4) = o;
    } else {
        u32x2_t h = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(o_out) + (size_t)row * D + e4 * 4) = h;
    }
    if (lse_out && e4 == 0) lse_out[row] = lse;
}

hipError_t launch_split_reduce(const SplitReduceArgs& a, hipStream_t stream) {
    const int rows = a.B * a.H_q;
    if (rows == 0) return hipSuccess;
    // most partials a row can have
    const int most = (a.pre_acc ? a.pre_splits : 0) + (a.part_acc && a.kv_indptr ? a.max_parts : 0);
    const bool wide = most > kReduceBatch && most <= kReduceBatchWide;
    if (a.D == 128) {
        if (wide) split_reduce_kernel<128, kReduceBatchWide><<<(rows + 7) / 8, 256, 0, stream>>>(a);
        else split_reduce_kernel<128, kReduceBatch><<<(rows + 7) / 8, 256, 0, stream>>>(a);
    } else {
        if (wide) split_reduce_kernel<64, kReduceBatchWide><<<(rows + 15) / 16, 256, 0, stream>>>(a);
        else split_reduce_kernel<64, kReduceBatch><<<(rows + 15) / 16, 256, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_merge_states(int32_t rows, int32_t D, const float* o_a, const float* lse_a,
                               const float* o_b, const float* lse_b, void* o_out, int32_t out_dtype,
                               float* lse_out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    if (D == 128) {
        merge_states_kernel<128><<<(rows + 7) / 8, 256, 0, stream>>>(rows, o_a, lse_a, o_b, lse_b,
                                                                      o_out, out_dtype, lse_out);
    } else {
        merge_states_kernel<64><<<(rows + 15) / 16, 256, 0, stream>>>(rows, o_a, lse_a, o_b, lse_b,
                                                                     o_out, out_dtype, lse_out);
    }
    return hipGetLastError();
}

}  // namespace pkv
