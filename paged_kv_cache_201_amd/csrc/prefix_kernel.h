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
// leaves registers.  K and V are both kept row-major in LDS; the V^T operand
// (eight tokens of one head-dim column per lane) is read with gfx950's
// transposing LDS read, ds_read_b64_tr_b16: within a group of 16 lanes, lane
// 4c+d receives element d of the 64-bit values read by lanes c, c+4, c+8,
// c+12, so lanes reading four tokens x four column chunks hand each lane
// four tokens of one column.  With e4m3 K/V the tiles stay as codes and
// each operand is widened in registers as it is read, V^T with the 8-bit
// form ds_read_b64_tr_b8 (lane 8c+d receives byte d of lanes c, c+2, ..,
// c+14), which hands each lane eight tokens of one column in one read.
//
// Softmax state per row is (m, l) in exp2 units with the same lazily raised
// maximum as the paged kernel; the partial or final result is written in the
// same format as the paged pass so the same reduction and merge apply.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "kernels.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kPrefixLazySlack = 8.0f;

// NW waves of 32 query rows each share KT-token K/V tiles through an LDS
// ring that global memory fills asynchronously, S - 1 tiles ahead of the
// one being computed.  The range's slot indices are staged in LDS once, so
// no tile waits on an index load.
#ifndef PKV_PREFIX_STAGES
#define PKV_PREFIX_STAGES 4
#endif
// LDS of one bf16 prefix workgroup: a ring of STAGES K and V tiles and the
// slot indices of the workgroup's prefix range.  Tile rows are D bf16 with no
// padding; the 16-byte chunks of row t are stored XOR-swizzled, chunk c at
// position c ^ chunk_swizzle(t), so that both operand reads are free of bank
// conflicts (see chunk_swizzle).
// (16-byte aligned: the operand reads are 16-byte LDS loads, which the
// compiler otherwise splits into pairs of 4-byte loads)
template <int D, int KT>
struct alignas(16) PrefixSmem {
    static constexpr int STAGES = PKV_PREFIX_STAGES;
    static constexpr int BUFS = STAGES;   // tiles the products read from
    uint16_t k[STAGES][KT * D];
    uint16_t v[STAGES][KT * D];
    int idx[kMaxPrefixSplitTokens];
};

// LDS of one fp8 (e4m3) prefix workgroup ("Track C · Document 10", fp8
// cache section: the cache stored at one byte per value): the ring holds the
// stored codes, half the bytes of a bf16 tile, with the 16-byte chunks of
// row t swizzled by chunk_swizzle8(t).  The products read the codes straight
// from the ring and widen each operand in registers, exactly.
template <int D, int KT>
struct alignas(16) PrefixSmem8 {
    static constexpr int STAGES = PKV_PREFIX_STAGES;
    static constexpr int BUFS = STAGES;
    uint8_t k8[STAGES][KT * D];
    uint8_t v8[STAGES][KT * D];
    int idx[kMaxPrefixSplitTokens];
};

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `younger` tiles' copies (PER operations each) are in
// flight, younger in 0..K (a run-time count turned into the immediate that
// s_waitcnt needs).
template <int K, int PER>
__device__ __forceinline__ void wait_younger(int younger) {
    if constexpr (K == 0) {
        wait_vmcnt<0>();
    } else {
        if (younger >= K) wait_vmcnt<K * PER>();
        else wait_younger<K - 1, PER>(younger);
    }
}

// Swizzle of tile row t, CPR 16-byte chunks per row.  A 256-byte row (D =
// 128) spans all 64 LDS banks, so rows differ only by this XOR.  The K reads
// take one chunk of eight consecutive rows per cycle group, which needs eight
// distinct values over any eight consecutive rows; the transposed V reads
// take two adjacent chunks (2k, 2k + 1) of four consecutive rows, which needs
// distinct values of swizzle / 2 over any four consecutive rows.  t mod 16
// rotated left by one bit gives both (t mod 16 alone gives the first only:
// rows 2i and 2i + 1 then share the banks of a chunk pair).  A 128-byte row
// (D = 64) fills half the banks, so even and odd rows never collide and
// t mod 8 serves.  Rows 16 apart share a swizzle.
template <int CPR>
__host__ __device__ constexpr int chunk_swizzle(int t) {
    return CPR == 16 ? (((t << 1) | ((t >> 3) & 1)) & 15) : (t & (CPR - 1));
}

// Swizzle of an e4m3 tile row t (128 codes: eight 16-byte chunks; chunk c
// of row t at position c ^ chunk_swizzle8(t)).  With u = (t >> 1) mod 8 the
// swizzle is u's bits reordered (bit 1, bit 0, bit 2 become bits 0, 1, 2).
// K operand reads take one whole chunk of 16 consecutive rows per cycle
// group: two row parities times eight distinct positions, since the swizzle
// is a bijection of u.  The transposed V reads take one 8-byte half of two
// adjacent chunks of rows {0..3, 8..11} (or {4..7, 12..15}) of a 16-row
// block: per row parity those rows' u differ in bits 0 and 2, which the
// swizzle moves to bits 1 and 2, so with the chunk pair's bit 0 and the half
// every lane of a half-wave lands on its own bank pair.
__host__ __device__ constexpr int chunk_swizzle8(int t) {
    const int u = (t >> 1) & 7;
    return ((u >> 1) & 1) | ((u & 1) << 1) | (u & 4);
}

// This lane's value and that of lane l ^ 32, exchanged between the two
// halves of the wave in registers (gfx950 v_permlane32_swap swaps the upper
// half of its first operand with the lower half of its second; with both
// equal to x, lane l ends up holding x[l] and x[l ^ 32] in its two results)
// rather than through an LDS permute, which queues behind the tile traffic.
__device__ __forceinline__ void halves_pair(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

// Number of prefix blocks to launch for N work items (a multiple of 8, see
// prefix_item).
__host__ __device__ inline int prefix_blocks(int n_items) { return (n_items + 7) / 8 * 8; }

// One prefix work item, run by all NW * 64 threads of a workgroup.  p is the
// workgroup's index among the prefix workgroups of the launch.  KV is the
// stored dtype (bf16, or fp8 e4m3 with per-KV-head scales); SM is the
// matching LDS layout.
template <int KV, int D, int NW, int KT, class SM>
__device__ __forceinline__ void prefix_item(const PrefixArgs& a, SM& sm, const int p) {
    constexpr bool F8 = KV == PKV_FP8_E4M3;
    constexpr int CPR = D / 8;                  // 16-byte bf16 chunks per tile row
    constexpr int S = SM::STAGES;
    constexpr int NBUF = SM::BUFS;
    constexpr int NKS = D / 16;    // k-steps of the first product
    constexpr int NDB = D / 32;    // 32-wide head-dim blocks of the output
    constexpr int NTB = KT / 32;   // 32-token blocks per tile
    constexpr int NT = NW * 64;
    constexpr int BLOCKS = KT * D * (F8 ? 1 : 2) / 1024;   // 1 KB wave-wide LDS copies per K (or V) tile
    static_assert(BLOCKS % NW == 0, "each wave copies whole 1 KB blocks of a tile");
    constexpr int PER_WAVE = BLOCKS / NW;
    int* const s_idx = sm.idx;

    // XCD-aware placement: workgroups are handed to the 8 XCDs round robin,
    // so give each XCD a contiguous run of logical items; row tiles that read
    // the same (KV head, prefix range) then share one L2.
    const int N = a.groups ? a.num_items : a.row_tiles * a.H_kv * a.num_splits;
    const int per_xcd = (N + 7) / 8;
    int item = (p % 8) * per_xcd + p / 8;
    if (item >= N) return;
    // This item's prefix group: the whole batch with one shared prefix, or
    // one row of the group table (items of a group are consecutive; the
    // table's first column is the running end of each group's items).
    int row_tiles = a.row_tiles, prefix_len = a.prefix_len, split_tokens = a.split_tokens;
    int M = a.B * a.G;
    const int32_t* prefix = a.prefix_indices;
    int prefix_base = a.prefix_base;  // >= 0: the run is slots prefix_base + t, no index reads
    const int32_t* members = nullptr;
    int slot_base = 0;  // first partial-state slot of this group's ranges
    if (a.groups) {
        item += a.item_base;
        int lo = 0, hi = a.num_groups - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (a.groups[mid * kGroupDescInts] > item) hi = mid;
            else lo = mid + 1;
        }
        const int32_t* gd = a.groups + lo * kGroupDescInts;
        item -= lo ? a.groups[(lo - 1) * kGroupDescInts] : 0;
        prefix += gd[1];
        prefix_len = gd[2];
        split_tokens = gd[3];
        row_tiles = gd[5];
        members = a.members + gd[6];
        M = gd[7] * a.G;
        slot_base = gd[8];
        prefix_base = gd[9];
    }
    prefix_base = __builtin_amdgcn_readfirstlane(prefix_base);
    const int tile = item % row_tiles;
    const int g = (item / row_tiles) % a.H_kv;
    const int split = item / (row_tiles * a.H_kv);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;        // which half of the wave
    const int lr = lane & 31;
    const int G = a.G;
    const int H_q = a.H_kv * G;
    const int ts = split * split_tokens;
    const int te = min(ts + split_tokens, prefix_len);
    const int n_tok = te - ts;
    const int ntiles = (n_tok + KT - 1) / KT;

    // the range's slot indices, padded with the last one to whole tiles (a
    // prefix placed as one run of slots needs none: "GraniKV", s.1)
    if (prefix_base < 0)
        for (int i = threadIdx.x; i < ntiles * KT; i += NT) s_idx[i] = prefix[ts + min(i, n_tok - 1)];

    // This lane's query row: (request, query head) of the item's rows.
    const int r = tile * 32 * NW + wave * 32 + lr;
    const bool row_ok = r < M;
    const int rb = row_ok ? (members ? members[r / G] : r / G) : 0;
    const int rq = row_ok ? g * G + r % G : 0;
    const size_t qrow = (size_t)rb * H_q + rq;
    // k-step ks of the first product covers, for this lane's half h, head-dim
    // columns ks * 16 + h * 8 .. + 8 (bf16 tiles: one 16-byte chunk of a
    // row); with e4m3 tiles, where one 16-byte chunk holds 16 columns, k-steps
    // 2j and 2j + 1 cover the two halves of chunk 2j + h, columns
    // (2j + h) * 16 + (ks % 2) * 8 .. + 8.  K rows and Q^T take the same order.
    bf16x8_t qreg[NKS];
    {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int col = F8 ? (2 * (ks >> 1) + h) * 16 + (ks & 1) * 8 : ks * 16 + h * 8;
            u32x4_t x = row_ok ? *reinterpret_cast<const u32x4_t*>(qp + col) : u32x4_t{0, 0, 0, 0};
            qreg[ks] = __builtin_bit_cast(bf16x8_t, x);
        }
    }

    const size_t slot_stride = (size_t)a.H_kv * D;   // elements
    const size_t head_off = (size_t)g * D;
    // fp8 codes are widened exactly; the per-head scales multiply the scores
    // (folded into the exp2 scale) and the output
    const float sl2 = F8 ? a.scale_log2 * a.k_scale[g] : a.scale_log2;

    // Tile n goes to ring stage n % S straight from global memory with
    // gfx950's global_load_lds_dwordx4: lane l of a wave-wide copy fetches one
    // 16-byte chunk and the hardware stores it at LDS block base + 16 l, so
    // no registers hold tiles in flight and S - 1 tiles can be outstanding.
    // Each lane picks the global chunk that belongs at its LDS position
    // (row t, swizzled chunk q holds chunk q ^ (t mod CPR)).
    // The copies are issued as inline assembly: the waits for them are the
    // explicit vmcnt waits of the tile loop (the compiler, which cannot tell
    // the ring stages apart, would otherwise drain every copy before each LDS
    // read).  Each statement sets M0 itself; nothing else in these kernels
    // uses M0.
    typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
    // LDS byte addresses of the two rings (M0 takes a 32-bit LDS address)
    uint32_t k_lds, v_lds;
    if constexpr (F8) {
        typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
        k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8_t*)&sm.k8[0][0]);
        v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8_t*)&sm.v8[0][0]);
    } else {
        k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u16_t*)&sm.k[0][0]);
        v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u16_t*)&sm.v[0][0]);
    }
    auto lds_copy16 = [](const void* src, uint32_t m0) {
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
    };
    // The slot of the tile row each of this lane's copies reads.  They are
    // read from LDS a tile ahead (read_slots), so that issuing a tile right
    // after the barrier does not wait on an LDS round trip; a run placed
    // contiguously gives them as base + position (padded rows repeat the
    // last token, as the staged indices do).
    int next_slot[PER_WAVE];
    auto read_slots = [&](int n) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int p = (wave * PER_WAVE + j) * 64 + lane;
            const int row = n * KT + (F8 ? p / (D / 16) : p / CPR);
            next_slot[j] = prefix_base >= 0 ? prefix_base + ts + min(row, n_tok - 1) : s_idx[row];
        }
    };
    // Issue the copies of tile n, whose slots read_slots(n) has fetched.
    auto issue_tile = [&](int n) {
        const int stage = n % S;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int blk = wave * PER_WAVE + j;
            const int p = blk * 64 + lane;
            if constexpr (F8) {
                // rows of D codes: position p holds chunk (p mod D/16) ^ swizzle of row p / (D/16)
                const int t = p / (D / 16);
                const int c = (p % (D / 16)) ^ chunk_swizzle8(t);
                const size_t off = (size_t)next_slot[j] * slot_stride + head_off + c * 16;
                const uint32_t dst = (uint32_t)(stage * KT * D + blk * 1024);
                lds_copy16(static_cast<const uint8_t*>(a.k) + off, k_lds + dst);
                lds_copy16(static_cast<const uint8_t*>(a.v) + off, v_lds + dst);
            } else {
                const int t = p / CPR;
                const int c = (p % CPR) ^ chunk_swizzle<CPR>(t);
                const size_t off = (size_t)next_slot[j] * slot_stride + head_off + c * 8;
                const uint32_t dst = (uint32_t)(stage * KT * D + blk * 512) * 2;
                lds_copy16(static_cast<const uint16_t*>(a.k) + off, k_lds + dst);
                lds_copy16(static_cast<const uint16_t*>(a.v) + off, v_lds + dst);
            }
        }
    };
    // Transposed-read addresses of this lane for the V^T operand: lane group
    // (h, dh) of 16 lanes covers columns db*32 + dh*16 .. +15 and tokens
    // c*16 + h*4 (+8 for the second read); lane s of the group reads token
    // s/4 of those four at columns 4*(s%4) .. +3 of the group's sixteen.
    // Rows c*16 + r keep the swizzle of row r.
    const int tr_s = lane & 15;
    const int tr_dh = (lane >> 4) & 1;
    const int tr_row = (tr_s >> 2) + h * 4;
    const int tr_chunk = tr_dh * 2 + ((tr_s & 3) >> 1);  // chunk within a 32-column block
    const int tr_elem = (tr_s & 1) * 4;
    auto tr_off = [&](int row, int db) {
        return row * D + (((db * 4 + tr_chunk) ^ chunk_swizzle<CPR>(row)) << 3) + tr_elem;
    };
    const int kr_swz = chunk_swizzle<CPR>(lr);  // swizzle of the K rows this lane reads (rows tb*32 + lr)
    // e4m3 tiles: transposed 8-bit reads (ds_read_b64_tr_b8: within a group
    // of 16 lanes, lane 8c + d receives byte d of the 8-byte values read by
    // lanes c, c + 2, .., c + 14, in that order).  Lane s of a group reads
    // 8 columns, half s % 2 of the group's 16, of token (i & 3) + 4h +
    // 8 (i >> 2) of the 16-token chunk, i = s / 2: lane 8c + d then holds
    // column 16 (group % 2) + 8c + d = lane mod 32 of the 32-column block, for
    // the 8 tokens of its half in the k-slot order of P^T.
    const int tr8_i = (lane & 15) >> 1;
    const int tr8_row = (tr8_i & 3) + h * 4 + (tr8_i >> 2) * 8;
    const int tr8_g1 = (lane >> 4) & 1;
    const int tr8_base = tr8_row * D + (lane & 1) * 8;
    const int tr8_sw = chunk_swizzle8(tr8_row);  // rows c*16 + r keep the swizzle of row r

    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    // S^T = K . Q^T for tile n (one 32x32 block per 32 tokens; lane holds row
    // lr and tokens tb*32 + (i/4)*8 + h*4 + i%4), in two independent
    // accumulation chains (even and odd k-steps) so that consecutive MFMAs
    // do not wait on each other's results.  The chains are added where the
    // scores are used, a tile later, when the matrix cores are long done.
    auto qk = [&](int buf, f32x16_t (&se)[NTB], f32x16_t (&so)[NTB]) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            se[tb] = f32x16_t{};
            so[tb] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < NKS; ks += 2) {
                if constexpr (F8) {
                    // one 16-byte chunk of codes: the A operands of k-steps ks and ks + 1
                    const int row = tb * 32 + lr;
                    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(
                        &sm.k8[buf][row * D + (((ks + h) ^ chunk_swizzle8(row)) << 4)]);
                    const u32x4_t w0 = {fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
                                        fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
                    const u32x4_t w1 = {fp8x2_to_bf16x2<false>(x[2]), fp8x2_to_bf16x2<true>(x[2]),
                                        fp8x2_to_bf16x2<false>(x[3]), fp8x2_to_bf16x2<true>(x[3])};
                    se[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w0), qreg[ks],
                                                                     se[tb], 0, 0, 0);
                    so[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w1), qreg[ks + 1],
                                                                     so[tb], 0, 0, 0);
                } else {
                const bf16x8_t ka0 = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                  &sm.k[buf][(tb * 32 + lr) * D + (((ks * 2 + h) ^ kr_swz) << 3)]));
                const bf16x8_t ka1 = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                  &sm.k[buf][(tb * 32 + lr) * D + (((ks * 2 + 2 + h) ^ kr_swz) << 3)]));
                se[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qreg[ks], se[tb], 0, 0, 0);
                so[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qreg[ks + 1], so[tb], 0, 0, 0);
                }
            }
        }
    };

    // Probabilities 2^(s*scale - m) of a tile against max m, packed to bf16
    // as the B operand of P.V, and their sum.
    auto probs = [&](const f32x16_t (&s)[NTB], float mneg, bf16x8_t (&pb)[2 * NTB]) {
        float ps = 0.f;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                u32x4_t x;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float p0 = fast_exp2(fmaf(s[tb][c * 8 + 2 * w], sl2, mneg));
                    const float p1 = fast_exp2(fmaf(s[tb][c * 8 + 2 * w + 1], sl2, mneg));
                    ps += p0 + p1;
                    x[w] = pack_bf16x2(p0, p1);
                }
                pb[tb * 2 + c] = __builtin_bit_cast(bf16x8_t, x);
            }
        return ps;
    };

    // Online softmax of tile n's scores and O^T += V^T . P^T.  The
    // probabilities are first taken against the running max; only when the
    // tile raises the max by more than the lazy slack (a uniform, rare
    // branch) are the accumulators rescaled and the probabilities taken
    // again.  The common path has no branch, so the scores of the next tile
    // (already issued to the matrix cores) overlap this arithmetic.
    auto softmax_pv = [&](const f32x16_t (&se)[NTB], const f32x16_t (&so)[NTB], int n, int buf) {
        f32x16_t s[NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) s[tb] = se[tb] + so[tb];
        const int valid = n_tok - n * KT;
        if (valid < KT) {  // padded tail tokens get -inf
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (tb * 32 + (i / 4) * 8 + h * 4 + (i % 4) >= valid) s[tb][i] = -INFINITY;
        }
        // running max over raw scores (the scale is positive)
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[tb][i]);
        {
            float x0, x1;
            halves_pair(mx, x0, x1);
            mx = fmaxf(x0, x1) * sl2;
        }
        bf16x8_t pb[2 * NTB];
        float ps = probs(s, (m == -INFINITY) ? 0.f : -m, pb);
        const bool need = (mx > m + kPrefixLazySlack) || (m == -INFINITY && mx != -INFINITY);
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mn = fmaxf(m, mx);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            ps = probs(s, (m == -INFINITY) ? 0.f : -m, pb);
        }
        l += ps;
        // O^T += V^T . P^T over 16-token chunks; the head-dim blocks are the
        // inner loop, so that consecutive MFMAs update different accumulators
#pragma unroll
        for (int c = 0; c < 2 * NTB; ++c) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (F8) {
                    typedef int v2i_t __attribute__((ext_vector_type(2)));
                    typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
                    const uint8_t* vb = &sm.v8[buf][c * 16 * D];
                    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_v2i_t*)(vb + tr8_base + (((db * 2 + tr8_g1) ^ tr8_sw) << 4)));
                    const u32x4_t x = {fp8x2_to_bf16x2<false>((uint32_t)r[0]), fp8x2_to_bf16x2<true>((uint32_t)r[0]),
                                       fp8x2_to_bf16x2<false>((uint32_t)r[1]), fp8x2_to_bf16x2<true>((uint32_t)r[1])};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), pb[c], acc[db],
                                                                      0, 0, 0);
                } else {
                typedef short v4s_t __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
                const uint16_t* vb = &sm.v[buf][c * 16 * D];
                const v4s_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(vb + tr_off(tr_row, db)));
                const v4s_t x1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(vb + tr_off(tr_row + 8, db)));
                const u32x2_t y0 = __builtin_bit_cast(u32x2_t, x0);
                const u32x2_t y1 = __builtin_bit_cast(u32x2_t, x1);
                const u32x4_t x = {y0[0], y0[1], y1[0], y1[1]};
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), pb[c],
                                                                  acc[db], 0, 0, 0);
                }
            }
        }
    };

    // The query loads above must not be left in flight: the tile loop's
    // vmcnt waits count only the copies.
    wait_vmcnt<0>();
    __syncthreads();  // s_idx ready
    for (int n = 0; n < S - 1 && n < ntiles; ++n) {
        read_slots(n);
        issue_tile(n);
    }
    if (S - 1 < ntiles) read_slots(S - 1);
    static_assert(S >= 3 && 2 * PER_WAVE * (S - 2) < 64, "ring depth within the vmcnt range");
    // Wait until this wave's copies of tile n have landed: at most the copies
    // of the tiles issued after it (up to tile `last`) may still be in flight
    // (two per block: K and V).
    auto wait_tile = [&](int n, int last) { wait_younger<S - 2, 2 * PER_WAVE>(min(ntiles - 1, last) - n); };
    // Software pipeline: while the softmax and P.V of tile n run, the scores
    // of tile n + 1 are already on the matrix cores and tiles n + 2, n + 3
    // are on their way into the ring.  Two score buffers alternate (the loop
    // takes two tiles per trip), so no scores are copied between them.
    f32x16_t sa_e[NTB], sa_o[NTB], sb_e[NTB], sb_o[NTB];
    auto step = [&](int n, const f32x16_t (&ce)[NTB], const f32x16_t (&co)[NTB], f32x16_t (&ne)[NTB],
                    f32x16_t (&no)[NTB]) {
        if (n + 1 < ntiles) {
            // tiles 0 .. n + S - 2 have been issued
            wait_tile(n + 1, n + S - 2);
            __syncthreads();  // tile n + 1 landed; every wave is done with tile n - 1
            if (n + S - 1 < ntiles) {
                issue_tile(n + S - 1);  // into the stage of tile n - 1
                if (n + S < ntiles) read_slots(n + S);
            }
            qk((n + 1) % NBUF, ne, no);
        }
        softmax_pv(ce, co, n, n % NBUF);
    };
    if (ntiles > 0) {
        wait_tile(0, S - 2);
        __syncthreads();
        qk(0, sa_e, sa_o);
    }
    for (int n = 0; n < ntiles; n += 2) {
        step(n, sa_e, sa_o, sb_e, sb_o);
        if (n + 1 < ntiles) step(n + 1, sb_e, sb_o, sa_e, sa_o);
    }

    // Row totals: the two halves of the wave hold disjoint tokens of a row.
    float L;
    {
        float l0, l1;
        halves_pair(l, l0, l1);
        L = l0 + l1;
    }
    if (!row_ok) return;
    const bool direct = a.num_splits == 1 && !a.force_partial;
    float* out;
    float scale;
    if (direct) {
        out = a.o + qrow * D;
        scale = L > 0.f ? 1.f / L : 0.f;
        if constexpr (F8) scale *= a.v_scale[g];
    } else {
        out = a.part_acc + (((size_t)rb * a.num_splits + slot_base + split) * H_q + rq) * D;
        scale = F8 ? a.v_scale[g] : 1.f;
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
            float* ml = a.part_ml + (((size_t)rb * a.num_splits + slot_base + split) * H_q + rq) * 2;
            ml[0] = m;
            ml[1] = L;
        }
    }
}

}  // namespace pkv
