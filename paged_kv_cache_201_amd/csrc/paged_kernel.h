// Paged decode attention for gfx950: gather K/V rows through token-flat
// indices, split-K online softmax, LDS merge across waves.
//
// The operation ("The 25% Page-Size Slowdown That Wasn't", section "Four
// meanings of page size"; "Track C · Document 10", PagedAttention Q&A): each
// request's single query token, with G query heads per KV head, attends over
// the cached K/V rows that kv_indices lists for it, in logical order.
//
// Work decomposition.  The tokens the pass attends, request after request,
// form one flat sequence that is cut into equal chunks of chunk_tokens
// positions; a workgroup (4 waves) owns one (chunk, head block) pair and
// walks the requests its chunk touches, one segment per request.  Every
// workgroup therefore streams the same number of K/V rows whatever the mix of
// request lengths.  A request that lies inside one chunk gets its output
// written directly; a request cut by chunk boundaries leaves one partial
// softmax state per chunk, combined afterwards in chunk order.  Inside a
// segment each wave takes a contiguous quarter of the positions.  The 64
// lanes of a wave span (KV head, head-dim chunk): LPH lanes read one row, so
// a wave-wide load reads RS rows -- one token's HB heads when TPI == 1 (the
// slot is then wave-uniform and the address is scalar), or TPI tokens when
// the block has fewer heads than a load has rows.
//
// Per token a lane forms G partial dot products (one per query head of its
// KV head), and the row's LPH lanes reduce-scatter them with DPP moves so
// that each lane ends up owning one query head's score.  The softmax state
// (running max m, sum l) is then lane-local.  Probabilities are shuffled back
// along the same DPP pattern for the P.V update; for bf16 and fp8 K/V two
// consecutive tokens are paired so that P.V runs on v_dot2_f32_bf16.
//
// The running max is raised lazily: the accumulator is rescaled only when a
// score exceeds the current max by more than 2^8 (in the exp2 domain), so
// probabilities stay <= 256 and the rescale is rare.  The result is the same
// softmax up to rounding.
//
// Everything is ordered by logical token position, so the output does not
// depend on page size, page placement or timing: runs are bitwise
// reproducible and page-size invariant.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pkv {

template <int KV>
struct KvTraits;
template <>
struct KvTraits<PKV_F32> {
    static constexpr int BK = 4, EPL = 4, LW = 4;  // bytes/elem, elems/lane, dwords/lane
};
template <>
struct KvTraits<PKV_BF16> {
    static constexpr int BK = 2, EPL = 8, LW = 4;
};
template <>
struct KvTraits<PKV_FP8_E4M3> {
    static constexpr int BK = 1, EPL = 8, LW = 2;
};

template <int LW>
struct LoadVec;
template <>
struct LoadVec<4> {
    using T = u32x4_t;
};
template <>
struct LoadVec<2> {
    using T = u32x2_t;
};

#ifndef PKV_PAGED_WAVES
#define PKV_PAGED_WAVES 4
#endif
#ifndef PKV_STREAM_LOADS
#define PKV_STREAM_LOADS 1  // K/V rows are read once per step: non-temporal loads
#endif
constexpr int kPagedWaves = PKV_PAGED_WAVES;
#ifndef PKV_PAGED_PIPE
#define PKV_PAGED_PIPE 2
#endif
constexpr int kPagedPipe = PKV_PAGED_PIPE;  // register buffers of K/V loads (2 or 3)
// fp8 K/V: tokens per iteration and pipeline depth (the fp8 kernel is bound
// by vector ALU work, so its loads need to run further ahead)
#ifndef PKV_FP8_PIPE
#define PKV_FP8_PIPE 2
#endif
#ifndef PKV_FP8_U
#define PKV_FP8_U 0
#endif
#ifndef PKV_BF16_U
#define PKV_BF16_U 0
#endif
constexpr float kLazyMaxSlack = 8.0f;  // log2 units

template <int KV, int D, int G, int NHL, int TPI>
struct PagedCfg {
    using Tr = KvTraits<KV>;
    static constexpr int BK = Tr::BK, EPL = Tr::EPL, LW = Tr::LW;
    static constexpr int LPH = D / EPL;
    static constexpr int RS = 64 / LPH;
    static constexpr int HB = RS * NHL / TPI;
    static constexpr int NW = kPagedWaves;
    static constexpr bool QF32 = (KV == PKV_F32);
    static constexpr int QW = QF32 ? EPL : EPL / 2;  // q registers per (slot, head)
    // steps per iteration: 8 KB of K+V in flight per wave per buffer
    static constexpr int U0 = (KV == PKV_FP8_E4M3 && PKV_FP8_U > 0)  ? PKV_FP8_U
                              : (KV == PKV_BF16 && PKV_BF16_U > 0)    ? PKV_BF16_U
                                                                      : 32 / (NHL * 2 * LW);
    static constexpr int U = U0 < 2 ? 2 : U0;
    static constexpr int PIPE = KV == PKV_FP8_E4M3 ? PKV_FP8_PIPE : kPagedPipe;
    static constexpr int TU = U * TPI;  // tokens per wave iteration
    static constexpr int PARTIALS = NW * TPI;
    // With one token per load the four waves merge pairwise (waves 2, 3 into
    // 0, 1, then 1 into 0) through two LDS slots; otherwise every partial
    // gets a slot and the output loop combines them all.
    static constexpr bool TREE = TPI == 1 && NW == 4;
    static constexpr int MERGE_SLOTS = TREE ? 2 : PARTIALS;
    static constexpr int OUT_PARTIALS = TREE ? 1 : PARTIALS;
    static constexpr int MERGE_FLOATS = MERGE_SLOTS * HB * G * D;
    // slot indices of a chunk, padded by whole wave iterations
    static constexpr int IDX_INTS = max_chunk_tokens(RS, NHL, TPI, G, D) + NW * TU;
    static_assert(G <= LPH, "one query head per lane after the row reduction");
    static_assert(TPI == 1 || NHL == 1, "several tokens per load only with one head slot");
    static_assert(U % 2 == 0, "tokens are paired for the P.V dot products");
};

// LDS of one paged workgroup: the per-wave partial accumulators and (max,
// sum) pairs of a segment, and the slot indices of the current segment.
template <int KV, int D, int G, int NHL, int TPI>
struct PagedSmem {
    using C = PagedCfg<KV, D, G, NHL, TPI>;
    float buf[C::MERGE_FLOATS];
    int idx[C::IDX_INTS];
    float ml[C::MERGE_SLOTS * C::HB * G * 2];
    int first_request;
};

// One segment: n_tok > 0 consecutive positions of request b, whose slot
// indices start at kv_indices[idx_beg] (with a page table instead: logical
// positions from idx_beg - kv_indptr[b] on), for the HB KV heads of head block
// hblk.  slot < 0: the segment is the whole request and its normalised output
// goes to o / o_f32 / lse; slot >= 0: its partial state goes to partial
// index `slot` of request b.  staged: sm.idx already holds the segment's slot
// indices (and at least a whole iteration past its end).  Called by every
// thread of the workgroup.
template <int KV, int D, int G, int NHL, int TPI>
__device__ __forceinline__ void paged_segment(const PagedArgs& a, PagedSmem<KV, D, G, NHL, TPI>& sm, const int b,
                                              const int hblk, const int idx_beg, const int n_tok,
                                              const int slot, const bool staged) {
    using C = PagedCfg<KV, D, G, NHL, TPI>;
    constexpr int BK = C::BK, EPL = C::EPL, LW = C::LW, LPH = C::LPH, RS = C::RS, HB = C::HB;
    constexpr int NW = C::NW, QW = C::QW, U = C::U, TU = C::TU;
    using LV = typename LoadVec<LW>::T;
    float* const s_buf = sm.buf;
    float* const s_ml = sm.ml;

    const int lane = threadIdx.x & 63;
    // wave-uniform, so everything derived from it lives in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H_kv = a.H_kv;
    const int H_q = H_kv * G;

    // This wave's contiguous token range [w0, w1) within the item; every
    // wave range starts on a whole iteration.
    const int per_wave = ((n_tok + NW - 1) / NW + TU - 1) / TU * TU;
    const int w0 = min(wave * per_wave, n_tok);
    const int w1 = min(w0 + per_wave, n_tok);
    const int niter = (w1 - w0 + TU - 1) / TU;

    // Stage this segment's slot indices in LDS, padded with the last slot up
    // to a whole iteration so that the tail needs no clamping (padded tokens
    // are masked out of the softmax).
    int* const s_idx = sm.idx;
    if (!staged) {
        const int n_pad = (n_tok + TU - 1) / TU * TU;
        if (a.page_indices) {
            // from the page table: logical position t of request b lives in
            // slot page_indices[page_indptr[b] + t / p] * p + t % p
            const int t0 = idx_beg - a.kv_indptr[b];
            const int32_t* pages = a.page_indices + a.page_indptr[b];
            const int p = a.page_size;
            for (int i = threadIdx.x; i < n_pad; i += NW * 64) {
                const int t = t0 + min(i, n_tok - 1);
                s_idx[i] = pages[t / p] * p + t % p;
            }
        } else {
            for (int i = threadIdx.x; i < n_pad; i += NW * 64) s_idx[i] = a.kv_indices[idx_beg + min(i, n_tok - 1)];
        }
        __syncthreads();
    }

    const int lrow = lane / LPH;
    const int lch = lane % LPH;
    const int tau = TPI > 1 ? lrow / HB : 0;
    const int fl = head_of_lane<LPH, G>(lch);
    auto head_local = [&](int i) { return TPI > 1 ? lrow % HB : i * RS + lrow; };

    // Queries, in the lane's XOR-permuted head order: slot u holds head u ^ fl.
    uint32_t qv[NHL][G][QW];
    float sc[NHL];
#pragma unroll
    for (int i = 0; i < NHL; ++i) {
        const int kvh = hblk * HB + head_local(i);
        float s = a.scale_log2;
        if constexpr (KV == PKV_FP8_E4M3) s *= a.k_scale[kvh];
        sc[i] = s;
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int qh = kvh * G + (u ^ fl);
            const char* qp = static_cast<const char*>(a.q) +
                             ((size_t)b * H_q + qh) * D * (C::QF32 ? 4 : 2) +
                             (size_t)lch * EPL * (C::QF32 ? 4 : 2);
            if constexpr (QW == 4) {
                const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qp);
#pragma unroll
                for (int w = 0; w < 4; ++w) qv[i][u][w] = x[w];
            } else {
#pragma unroll
                for (int w = 0; w < QW; ++w) qv[i][u][w] = reinterpret_cast<const uint32_t*>(qp)[w];
            }
        }
    }

    float m[NHL], l[NHL];
    float acc[NHL][G][EPL];
#pragma unroll
    for (int i = 0; i < NHL; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.f;
#pragma unroll
        for (int u = 0; u < G; ++u)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[i][u][e] = 0.f;
    }

    // bytes per slot (H_kv * D * BK, far below 4 GB): a 32-bit factor, so each
    // row address is one 32 x 32 -> 64-bit multiply-add
    const uint32_t slot_stride = (uint32_t)H_kv * D * BK;
    const char* kbase = static_cast<const char*>(a.k) + (size_t)hblk * HB * D * BK;
    const char* vbase = static_cast<const char*>(a.v) + (size_t)hblk * HB * D * BK;
    uint32_t loff[NHL];
#pragma unroll
    for (int i = 0; i < NHL; ++i) loff[i] = head_local(i) * D * BK + lch * EPL * BK;

    LV kb[C::PIPE][U][NHL], vb[C::PIPE][U][NHL];

    auto issue = [&](int it, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const int tk0 = w0 + it * TU;
        int slots[U];
        if constexpr (TPI == 1) {
            // one slot per step, the same for the whole wave: vector LDS
            // reads of consecutive entries, then into scalar registers
            if constexpr (U % 4 == 0) {
#pragma unroll
                for (int j = 0; j < U; j += 4) {
                    const int4 v = *reinterpret_cast<const int4*>(s_idx + tk0 + j);
                    slots[j] = __builtin_amdgcn_readfirstlane(v.x);
                    slots[j + 1] = __builtin_amdgcn_readfirstlane(v.y);
                    slots[j + 2] = __builtin_amdgcn_readfirstlane(v.z);
                    slots[j + 3] = __builtin_amdgcn_readfirstlane(v.w);
                }
            } else {
#pragma unroll
                for (int j = 0; j < U; j += 2) {
                    const int2 v = *reinterpret_cast<const int2*>(s_idx + tk0 + j);
                    slots[j] = __builtin_amdgcn_readfirstlane(v.x);
                    slots[j + 1] = __builtin_amdgcn_readfirstlane(v.y);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < U; ++j) slots[j] = s_idx[tk0 + j * TPI + tau];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint64_t off = (uint64_t)(uint32_t)slots[j] * slot_stride;
            gbytes_t kr = as_global(kbase) + off;
            gbytes_t vr = as_global(vbase) + off;
            if constexpr (TPI == 1) {
                // The row base is wave-uniform: keep it in scalar registers
                // and opaque, so that each load is (scalar base + 32-bit lane
                // offset) rather than 64-bit per-lane address arithmetic.
                asm("" : "+s"(kr));
                asm("" : "+s"(vr));
            }
#pragma unroll
            for (int i = 0; i < NHL; ++i) {
                if constexpr (PKV_STREAM_LOADS) {
                    kb[buf][j][i] = load_global_stream<LV>(kr + loff[i]);
                    vb[buf][j][i] = load_global_stream<LV>(vr + loff[i]);
                } else {
                    kb[buf][j][i] = load_global<LV>(kr + loff[i]);
                    vb[buf][j][i] = load_global<LV>(vr + loff[i]);
                }
            }
        }
    };

    auto compute = [&](int it, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        float s[U][NHL];
#pragma unroll
        for (int j = 0; j < U; ++j) {
#pragma unroll
            for (int i = 0; i < NHL; ++i) {
                float part[G];
                if constexpr (KV == PKV_F32) {
#pragma unroll
                    for (int u = 0; u < G; ++u) {
                        float t = 0.f;
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            t = fmaf(__uint_as_float(qv[i][u][e]), __uint_as_float(kb[buf][j][i][e]), t);
                        part[u] = t;
                    }
                } else if constexpr (KV == PKV_BF16) {
#pragma unroll
                    for (int u = 0; u < G; ++u) {
                        float t = dot2_bf16_first(qv[i][u][0], kb[buf][j][i][0]);
#pragma unroll
                        for (int w = 1; w < 4; ++w) t = dot2_bf16(qv[i][u][w], kb[buf][j][i][w], t);
                        part[u] = t;
                    }
                } else {
                    uint32_t kc[4];
                    kc[0] = fp8x2_to_bf16x2<false>(kb[buf][j][i][0]);
                    kc[1] = fp8x2_to_bf16x2<true>(kb[buf][j][i][0]);
                    kc[2] = fp8x2_to_bf16x2<false>(kb[buf][j][i][1]);
                    kc[3] = fp8x2_to_bf16x2<true>(kb[buf][j][i][1]);
#pragma unroll
                    for (int u = 0; u < G; ++u) {
                        float t = dot2_bf16_first(qv[i][u][0], kc[0]);
#pragma unroll
                        for (int w = 1; w < 4; ++w) t = dot2_bf16(qv[i][u][w], kc[w], t);
                        part[u] = t;
                    }
                }
                s[j][i] = row_reduce_scatter<LPH, G>(part);  // unscaled: sc[i] > 0 joins in the exponent
            }
        }
        // Padded tail tokens get -inf; only the last iteration of a wave's
        // range holds any, so the other iterations skip the compares.
        if (w0 + (it + 1) * TU > w1) {
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const bool valid = (w0 + it * TU + j * TPI + tau) < w1;
#pragma unroll
                for (int i = 0; i < NHL; ++i) s[j][i] = valid ? s[j][i] : -INFINITY;
            }
        }

        // Online softmax with a lazily raised maximum (in scaled units: the
        // scale is positive, so the scaled maximum is the maximum's scaling).
        bool need = false;
        float tmax[NHL];
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            float t = s[0][i];
#pragma unroll
            for (int j = 1; j < U; ++j) t = fmaxf(t, s[j][i]);
            t *= sc[i];
            tmax[i] = t;
            need |= (t > m[i] + kLazyMaxSlack) || (m[i] == -INFINITY && t != -INFINITY);
        }
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int i = 0; i < NHL; ++i) {
                const float mn = fmaxf(m[i], tmax[i]);
                const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m[i] - mn);
                m[i] = mn;
                l[i] *= alpha;
                static_for<G>([&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    const float au = xor_shfl<lane_mask_for_head_xor<LPH, G>(u)>(alpha);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[i][u][e] *= au;
                });
            }
        }

        float p[U][NHL];
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            // 2^(s * sc - m) as one fma; with no finite score yet (m = -inf)
            // every probability is 2^-inf = 0
            const float mneg = m[i] == -INFINITY ? -INFINITY : -m[i];
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < U; ++j) {
                p[j][i] = fast_exp2(fmaf(s[j][i], sc[i], mneg));
                sum += p[j][i];
            }
            l[i] += sum;
        }

        // P.V
        if constexpr (KV == PKV_F32) {
#pragma unroll
            for (int j = 0; j < U; ++j)
#pragma unroll
                for (int i = 0; i < NHL; ++i)
                    static_for<G>([&](auto uc) {
                        constexpr int u = decltype(uc)::value;
                        const float pu = xor_shfl<lane_mask_for_head_xor<LPH, G>(u)>(p[j][i]);
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            acc[i][u][e] = fmaf(pu, __uint_as_float(vb[buf][j][i][e]), acc[i][u][e]);
                    });
        } else {
#pragma unroll
            for (int j = 0; j < U; j += 2)
#pragma unroll
                for (int i = 0; i < NHL; ++i) {
                    // value pairs (token j, token j+1) per head-dim element
                    uint32_t vp[EPL];
                    if constexpr (KV == PKV_BF16) {
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            vp[2 * w] = __builtin_amdgcn_perm(vb[buf][j + 1][i][w], vb[buf][j][i][w], 0x05040100u);
                            vp[2 * w + 1] = __builtin_amdgcn_perm(vb[buf][j + 1][i][w], vb[buf][j][i][w], 0x07060302u);
                        }
                    } else {
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const uint32_t x0 = __builtin_amdgcn_perm(vb[buf][j + 1][i][w], vb[buf][j][i][w], 0x05010400u);
                            const uint32_t x1 = __builtin_amdgcn_perm(vb[buf][j + 1][i][w], vb[buf][j][i][w], 0x07030602u);
                            vp[4 * w + 0] = fp8x2_to_bf16x2<false>(x0);
                            vp[4 * w + 1] = fp8x2_to_bf16x2<true>(x0);
                            vp[4 * w + 2] = fp8x2_to_bf16x2<false>(x1);
                            vp[4 * w + 3] = fp8x2_to_bf16x2<true>(x1);
                        }
                    }
                    const uint32_t pp = pack_bf16x2(p[j][i], p[j + 1][i]);
                    static_for<G>([&](auto uc) {
                        constexpr int u = decltype(uc)::value;
                        const uint32_t pu = xor_shfl_u32<lane_mask_for_head_xor<LPH, G>(u)>(pp);
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[i][u][e] = dot2_bf16(vp[e], pu, acc[i][u][e]);
                    });
                }
        }
    };

    // Register pipeline C::PIPE deep: the loads of the next C::PIPE - 1
    // iterations are in flight while one iteration is computed.
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if constexpr (C::PIPE == 2) {
        if (niter > 0) issue(0, B0{});
        for (int it = 0; it < niter; it += 2) {
            if (it + 1 < niter) issue(it + 1, B1{});
            compute(it, B0{});
            if (it + 1 < niter) {
                if (it + 2 < niter) issue(it + 2, B0{});
                compute(it + 1, B1{});
            }
        }
    } else {
        using B2 = std::integral_constant<int, 2>;
        if (niter > 0) issue(0, B0{});
        if (niter > 1) issue(1, B1{});
        for (int it = 0; it < niter; it += 3) {
            if (it + 2 < niter) issue(it + 2, B2{});
            compute(it, B0{});
            if (it + 1 < niter) {
                if (it + 3 < niter) issue(it + 3, B0{});
                compute(it + 1, B1{});
            }
            if (it + 2 < niter) {
                if (it + 4 < niter) issue(it + 4, B1{});
                compute(it + 2, B2{});
            }
        }
    }

    // Merge the NW * TPI partial states of this segment in a fixed order.
    __syncthreads();  // every wave is done with s_idx
    // A partial state in LDS slot `sl`: acc rows of G query heads and the
    // (max, sum) pair of this lane's head, at the positions this lane owns.
    auto publish = [&](int sl) {
#pragma unroll
        for (int i = 0; i < NHL; ++i) {
            const int hl = head_local(i);
#pragma unroll
            for (int u = 0; u < G; ++u) {
                float* dst = s_buf + ((size_t)(sl * HB + hl) * G + (u ^ fl)) * D + lch * EPL;
#pragma unroll
                for (int e = 0; e < EPL; e += 4) {
                    f32x4_t x = {acc[i][u][e], acc[i][u][e + 1], acc[i][u][e + 2], acc[i][u][e + 3]};
                    *reinterpret_cast<f32x4_t*>(dst + e) = x;
                }
            }
            float* mlp = s_ml + ((sl * HB + hl) * G + fl) * 2;
            mlp[0] = m[i];
            mlp[1] = l[i];
        }
    };
    if constexpr (C::TREE) {
        // Combine the state in slot `sl` into this wave's registers.
        auto absorb = [&](int sl) {
#pragma unroll
            for (int i = 0; i < NHL; ++i) {
                const int hl = head_local(i);
                const float* mlp = s_ml + ((sl * HB + hl) * G + fl) * 2;
                const float m2 = mlp[0], l2 = mlp[1];
                const float mn = fmaxf(m[i], m2);
                const float wa = (m[i] == -INFINITY) ? 0.f : fast_exp2(m[i] - mn);
                const float wb = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
                m[i] = mn;
                l[i] = l[i] * wa + l2 * wb;
                static_for<G>([&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    const float au = xor_shfl<lane_mask_for_head_xor<LPH, G>(u)>(wa);
                    const float bu = xor_shfl<lane_mask_for_head_xor<LPH, G>(u)>(wb);
                    const float* src = s_buf + ((size_t)(sl * HB + hl) * G + (u ^ fl)) * D + lch * EPL;
#pragma unroll
                    for (int e = 0; e < EPL; e += 4) {
                        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(src + e);
#pragma unroll
                        for (int k = 0; k < 4; ++k) acc[i][u][e + k] = acc[i][u][e + k] * au + x[k] * bu;
                    }
                });
            }
        };
        if (wave >= 2) publish(wave - 2);
        __syncthreads();
        if (wave < 2) absorb(wave);
        __syncthreads();
        if (wave == 1) publish(0);
        __syncthreads();
        if (wave == 0) {
            absorb(0);
            publish(0);
        }
    } else {
        publish(wave * TPI + tau);
    }
    __syncthreads();

    constexpr int CH = D / 4;  // float4 chunks per head
    const bool direct = slot < 0;
    for (int c = threadIdx.x; c < HB * G * CH; c += NW * 64) {
        const int qhl = c / CH;
        const int e4 = c % CH;
        float M = -INFINITY;
#pragma unroll
        for (int pp = 0; pp < C::OUT_PARTIALS; ++pp) M = fmaxf(M, s_ml[(pp * HB * G + qhl) * 2]);
        float L = 0.f;
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
        if (M != -INFINITY) {
#pragma unroll
            for (int pp = 0; pp < C::OUT_PARTIALS; ++pp) {
                const float mp = s_ml[(pp * HB * G + qhl) * 2];
                if (mp == -INFINITY) continue;
                const float w = fast_exp2(mp - M);
                L += w * s_ml[(pp * HB * G + qhl) * 2 + 1];
                const f32x4_t x = *reinterpret_cast<const f32x4_t*>(s_buf + ((size_t)pp * HB * G + qhl) * D + e4 * 4);
                o += w * x;
            }
        }
        const int kvh = hblk * HB + qhl / G;
        const int qh = kvh * G + qhl % G;
        if constexpr (KV == PKV_FP8_E4M3) o *= a.v_scale[kvh];
        const size_t row = (size_t)b * H_q + qh;
        if (direct) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            o *= inv;
            if (a.o_f32) *reinterpret_cast<f32x4_t*>(a.o_f32 + row * D + e4 * 4) = o;
            if (a.o) {
                if constexpr (C::QF32) {
                    *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.o) + row * D + e4 * 4) = o;
                } else {
                    u32x2_t h = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                    *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(a.o) + row * D + e4 * 4) = h;
                }
            }
            if (a.lse && e4 == 0) a.lse[row] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
        } else {
            const size_t prow = ((size_t)b * a.max_parts + slot) * H_q + qh;
            *reinterpret_cast<f32x4_t*>(a.part_acc + prow * D + e4 * 4) = o;
            if (e4 == 0) {
                a.part_ml[prow * 2] = M;
                a.part_ml[prow * 2 + 1] = L;
            }
        }
    }
}

// Offset of request i's first attended position in the flat sequence.
__device__ __forceinline__ int64_t flat_offset(const PagedArgs& a, int i) {
    return (int64_t)a.kv_indptr[i] - a.kv_indptr[0] - (int64_t)i * a.token_offset;
}

// One (chunk, head block) work item: positions [w * chunk, (w + 1) * chunk)
// of the flat sequence, segment by segment; or, when the plan packed whole
// requests into bins, bin w's requests.
template <int KV, int D, int G, int NHL, int TPI>
__device__ __forceinline__ void paged_chunk(const PagedArgs& a, PagedSmem<KV, D, G, NHL, TPI>& sm, const int w,
                                            const int hblk) {
    constexpr int NT = kPagedWaves * 64;
    const int64_t C = a.chunk_tokens;
    if (a.request_bins > 0) {
        // a bin of whole requests, one segment each (direct output, or the
        // request's one partial state)
        const int r0 = a.bin_start[w], r1 = a.bin_start[w + 1];
        for (int k = r0; k < r1; ++k) {
            const int b = a.bin_req[k];
            const int64_t ob = flat_offset(a, b), on = flat_offset(a, b + 1);
            // kv_indptr does not describe the planned batch: no request of
            // the plan is empty or longer than its longest (which fits the
            // LDS index stage)
            if (on <= ob || on - ob > a.bin_max_tokens) return;
            if (k > r0) __syncthreads();  // the previous segment is done with LDS
            paged_segment<KV, D, G, NHL, TPI>(a, sm, b, hblk, a.kv_indptr[b] + a.token_offset, (int)(on - ob),
                                              a.force_partial ? 0 : -1, false);
        }
        return;
    }
    const int64_t c0 = (int64_t)w * C;
    const int64_t c1 = c0 + C < a.total_tokens ? c0 + C : a.total_tokens;
    // Without a skipped prefix the flat sequence is kv_indices itself, so
    // the chunk's slot indices are staged at once, while the request holding
    // position c0 (the one non-empty request whose flat range contains it)
    // is looked up.
    const bool flat = a.token_offset == 0 && a.page_indices == nullptr;
    if (flat) {
        constexpr int TU = PagedCfg<KV, D, G, NHL, TPI>::TU;
        const int n = (int)(c1 - c0);
        const int64_t beg = (int64_t)a.kv_indptr[0] + c0;
        for (int i = threadIdx.x; i < n + TU; i += NT) sm.idx[i] = a.kv_indices[beg + min(i, n - 1)];
    }
    if (threadIdx.x == 0) sm.first_request = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < a.B; i += NT)
        if (flat_offset(a, i) <= c0 && c0 < flat_offset(a, i + 1)) sm.first_request = i;
    __syncthreads();
    int b = __builtin_amdgcn_readfirstlane(sm.first_request);
    if (b < 0) return;  // kv_indptr does not describe the planned batch
    bool first = true;
    for (; b < a.B; ++b) {
        const int64_t ob = flat_offset(a, b);
        if (ob >= c1) break;
        const int64_t on = flat_offset(a, b + 1);
        const int64_t lo = c0 > ob ? c0 : ob;
        const int64_t hi = c1 < on ? c1 : on;
        if (hi <= lo) continue;  // empty request
        const bool whole = lo == ob && hi == on;
        const int slot = (whole && !a.force_partial) ? -1 : (int)(w - ob / C);
        // kv_indptr does not describe the planned batch: a partial state the
        // workspace has no room for (or no partial buffer at all)
        if (slot >= a.max_parts || (slot >= 0 && a.part_acc == nullptr)) return;
        if (!first) __syncthreads();  // the previous segment is done with LDS
        first = false;
        // the first segment starts at c0: its indices are staged already
        paged_segment<KV, D, G, NHL, TPI>(a, sm, b, hblk, a.kv_indptr[b] + a.token_offset + (int)(lo - ob),
                                          (int)(hi - lo), slot, flat && lo == c0);
    }
}

#ifndef PKV_PAGED_OCC
#define PKV_PAGED_OCC 2
#endif
template <int KV, int D, int G, int NHL, int TPI>
__global__ void __launch_bounds__(kPagedWaves * 64) __attribute__((amdgpu_waves_per_eu(PKV_PAGED_OCC)))
paged_split_kernel(const PagedArgs a) {
    __shared__ PagedSmem<KV, D, G, NHL, TPI> sm;
    paged_chunk<KV, D, G, NHL, TPI>(a, sm, blockIdx.x, blockIdx.y);
}

}  // namespace pkv
