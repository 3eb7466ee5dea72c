// Shared-prefix attention, prefix read once for the whole batch, on MFMA.
//
// "GraniKV: asymmetric KV cache paging for shared-prefix agents", section 2:
// every decode step each request needs the whole shared prefix, so reading it
// once for all requests instead of once per request divides the prefix
// traffic by the batch size; section 3: with M_eff = batch x GQA group query
// rows per KV head the prefix attention is a real dense contraction, run as
// large tiles (DENSE) at high M_eff and small tiles (CASCADE) below.
//
// For KV head g, the M_eff rows are r = b * G + j (request b, query head
// g * G + j).  A workgroup owns 32 * NW rows, one KV head and one range of the
// prefix; its NW waves share each 32-token K/V tile through LDS.
//
// Per tile a wave computes S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: with
// K as the A operand and Q^T as B, a lane of the 32x32 result holds 16 of the
// 32 tokens of one query row, so the row max and sum need one exchange with
// the lane 32 apart.  The exponentiated scores, converted to bf16, are
// already in the B-operand layout of the second product O^T += V^T . P^T
// (both operands' k-slots are taken in the same token order), so P never
// leaves registers.  V is written transposed into LDS so that each lane reads
// eight consecutive tokens of one head-dim column.
//
// Softmax state per row is (m, l) in exp2 units with the same lazily raised
// maximum as the paged kernel; the partial or final result is written in the
// same format as the paged pass so the same reduction and merge apply.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefixTile = 32;  // tokens per K/V tile
constexpr float kPrefixLazySlack = 8.0f;

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 1) prefix_attn_kernel(const PrefixArgs a) {
    constexpr int KT = kPrefixTile;
    constexpr int KROW = D + 8;    // bf16 per LDS row of K (16-byte pad)
    constexpr int VROW = KT + 8;   // bf16 per LDS row of V^T
    constexpr int NKS = D / 16;    // k-steps of the first product
    constexpr int NDB = D / 32;    // 32-wide head-dim blocks of the output
    constexpr int NT = NW * 64;
    // K tile: KT * D/8 16-byte chunks; V tile: KT/2 token pairs * D/8 chunks
    constexpr int KITEMS = KT * D / 8;
    constexpr int VITEMS = (KT / 2) * (D / 8);
    constexpr int KCH = (KITEMS + NT - 1) / NT;
    constexpr int VCH = (VITEMS + NT - 1) / NT;

    __shared__ uint16_t s_k[KT * KROW];
    __shared__ uint16_t s_vt[D * VROW];

    // XCD-aware placement: workgroups are handed to the 8 XCDs round robin,
    // so give each XCD a contiguous run of logical items; row tiles that read
    // the same (KV head, prefix range) then share one L2.
    const int N = a.row_tiles * a.H_kv * a.num_splits;
    const int per_xcd = (N + 7) / 8;
    const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= N) return;
    const int tile = item % a.row_tiles;
    const int g = (item / a.row_tiles) % a.H_kv;
    const int split = item / (a.row_tiles * a.H_kv);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int h = lane >> 5;        // which half of the wave
    const int lr = lane & 31;
    const int G = a.G;
    const int H_q = a.H_kv * G;
    const int M = a.B * G;
    const int ts = split * a.split_tokens;
    const int te = min(ts + a.split_tokens, a.prefix_len);
    const int ntiles = (te - ts + KT - 1) / KT;

    // This lane's query row.
    const int r = tile * 32 * NW + wave * 32 + lr;
    const bool row_ok = r < M;
    const int rb = row_ok ? r / G : 0;
    const int rq = row_ok ? g * G + r % G : 0;
    const size_t qrow = (size_t)rb * H_q + rq;
    bf16x8_t qreg[NKS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D + h * 8;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4_t x = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + ks * 16) : u32x4_t{0, 0, 0, 0};
            qreg[ks] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    const uint16_t* kpool = static_cast<const uint16_t*>(a.k);
    const uint16_t* vpool = static_cast<const uint16_t*>(a.v);
    const size_t slot_stride = (size_t)a.H_kv * D;
    const size_t head_off = (size_t)g * D;

    // Register staging of the next tile.
    u32x4_t kst[KCH];
    u32x4_t vst[VCH][2];
    auto load_tile = [&](int n) {
        const int tb = ts + n * KT;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int id = c * NT + threadIdx.x;
            if (KITEMS % NT != 0 && id >= KITEMS) break;
            const int t = id / (D / 8), ch = id % (D / 8);
            const int slot = a.prefix_indices[min(tb + t, te - 1)];
            kst[c] = *reinterpret_cast<const u32x4_t*>(kpool + (size_t)slot * slot_stride + head_off + ch * 8);
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int id = c * NT + threadIdx.x;
            if (VITEMS % NT != 0 && id >= VITEMS) break;
            const int tp = id / (D / 8), ch = id % (D / 8);
            const int s0 = a.prefix_indices[min(tb + 2 * tp, te - 1)];
            const int s1 = a.prefix_indices[min(tb + 2 * tp + 1, te - 1)];
            vst[c][0] = *reinterpret_cast<const u32x4_t*>(vpool + (size_t)s0 * slot_stride + head_off + ch * 8);
            vst[c][1] = *reinterpret_cast<const u32x4_t*>(vpool + (size_t)s1 * slot_stride + head_off + ch * 8);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int id = c * NT + threadIdx.x;
            if (KITEMS % NT != 0 && id >= KITEMS) break;
            const int t = id / (D / 8), ch = id % (D / 8);
            *reinterpret_cast<u32x4_t*>(s_k + t * KROW + ch * 8) = kst[c];
        }
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int id = c * NT + threadIdx.x;
            if (VITEMS % NT != 0 && id >= VITEMS) break;
            const int tp = id / (D / 8), ch = id % (D / 8);
            // (token 2tp, token 2tp+1) pairs for each of the 8 head-dim elements
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = __builtin_amdgcn_perm(vst[c][1][w], vst[c][0][w], 0x05040100u);
                const uint32_t hi = __builtin_amdgcn_perm(vst[c][1][w], vst[c][0][w], 0x07060302u);
                *reinterpret_cast<uint32_t*>(s_vt + (ch * 8 + 2 * w) * VROW + 2 * tp) = lo;
                *reinterpret_cast<uint32_t*>(s_vt + (ch * 8 + 2 * w + 1) * VROW + 2 * tp) = hi;
            }
        }
    };

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    if (ntiles > 0) load_tile(0);
    for (int n = 0; n < ntiles; ++n) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (n + 1 < ntiles) load_tile(n + 1);

        // S^T = K . Q^T for this wave's 32 rows
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8_t ka = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const u32x4_t*>(s_k + lr * KROW + ks * 16 + h * 8));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s, 0, 0, 0);
        }
        // lane holds row lr, tokens (i/4)*8 + h*4 + i%4
        const int tb = ts + n * KT;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = (i / 4) * 8 + h * 4 + (i % 4);
            s[i] = (tb + t < te) ? s[i] * a.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = (mx > m + kPrefixLazySlack) || (m == -INFINITY && mx != -INFINITY);
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mn = fmaxf(m, mx);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        }
        float p[16];
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = (m == -INFINITY) ? 0.f : fast_exp2(s[i] - m);
            ps += p[i];
        }
        l += ps;
        bf16x8_t pb[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4_t x;
#pragma unroll
            for (int w = 0; w < 4; ++w) x[w] = pack_bf16x2(p[c * 8 + 2 * w], p[c * 8 + 2 * w + 1]);
            pb[c] = __builtin_bit_cast(bf16x8_t, x);
        }
        // O^T += V^T . P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const uint16_t* vr = s_vt + (db * 32 + lr) * VROW + c * 16 + h * 4;
                const u32x2_t x0 = *reinterpret_cast<const u32x2_t*>(vr);
                const u32x2_t x1 = *reinterpret_cast<const u32x2_t*>(vr + 8);
                const u32x4_t x = {x0[0], x0[1], x1[0], x1[1]};
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), pb[c],
                                                                  acc[db], 0, 0, 0);
            }
        }
    }

    // Row totals: the two halves of the wave hold disjoint tokens of a row.
    const float L = l + __shfl_xor(l, 32);
    if (!row_ok) return;
    const bool direct = a.num_splits == 1;
    float* out;
    float scale;
    if (direct) {
        out = a.o + qrow * D;
        scale = L > 0.f ? 1.f / L : 0.f;
    } else {
        out = a.part_acc + (((size_t)rb * a.num_splits + split) * H_q + rq) * D;
        scale = 1.f;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4_t x = {acc[db][q4 * 4] * scale, acc[db][q4 * 4 + 1] * scale, acc[db][q4 * 4 + 2] * scale,
                               acc[db][q4 * 4 + 3] * scale};
            *reinterpret_cast<f32x4_t*>(out + db * 32 + q4 * 8 + h * 4) = x;
        }
    if (h == 0) {
        if (direct) {
            a.lse[qrow] = L > 0.f ? (m + log2f(L)) * kLn2 : -INFINITY;
        } else {
            float* ml = a.part_ml + (((size_t)rb * a.num_splits + split) * H_q + rq) * 2;
            ml[0] = m;
            ml[1] = L;
        }
    }
}

hipError_t launch_prefix_attn(const PrefixArgs& a, int rows_per_wg, hipStream_t stream) {
    const int N = a.row_tiles * a.H_kv * a.num_splits;
    if (N == 0) return hipSuccess;
    const int grid = (N + 7) / 8 * 8;
    if (a.D == 128) {
        if (rows_per_wg == 128) {
            prefix_attn_kernel<128, 4><<<grid, 256, 0, stream>>>(a);
        } else {
            prefix_attn_kernel<128, 1><<<grid, 64, 0, stream>>>(a);
        }
    } else {
        if (rows_per_wg == 128) {
            prefix_attn_kernel<64, 4><<<grid, 256, 0, stream>>>(a);
        } else {
            prefix_attn_kernel<64, 1><<<grid, 64, 0, stream>>>(a);
        }
    }
    return hipGetLastError();
}

}  // namespace pkv
