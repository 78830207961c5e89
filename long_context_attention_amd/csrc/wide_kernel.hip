// wide_kernel.hip -- the kernel for calls with more than 96 rows per KV head
// (prefill chunks, wide verify).
#include <type_traits>

#include "kernels_common.h"

namespace kvattn_dev {

// ---------------------------------------------------------------------------
// Wide kernel (prefill chunks, and any call with more than 96 rows per KV
// head).  A workgroup of 8 or 12 waves handles one split of one KV head for a
// block of 256 or 384 rows; wave w owns rows 32w .. 32w + 31 (two 16-row
// tiles) over every chunk of the split, so no combine across waves is needed.
// Per 32-key chunk the workgroup first turns the staged codes into binary16
// K' = c * d_K and V' = (n - 8) * d_V once (the f16 working view of the
// pages' wide-prefill path), shared through LDS by all 256 rows; the matrix
// cores then run on K' and V' with no per-block scale work in the row loop.
// Each of K', V' is one rounding from the exact product (relative 2^-11).
// Pipeline per step of two chunks (one barrier): wait for the raw chunks of
// the next step, barrier, issue the raw chunks of the step after, dequantise
// the next step's chunks into their views, compute this step's chunks.  Raw
// chunks land in a ring of four buffers by direct-to-LDS loads, a chunk's load
// instructions spread over the waves.
// ---------------------------------------------------------------------------
// Workgroup shapes: 8 waves (256-row blocks) or 12 waves (384-row blocks;
// three waves per SIMD overlap matrix-core and vector work better, measured
// +14 % on the 1,280-row prefill chunk despite its partly empty last block).
constexpr int kWideRowsPerWave = 32;
// Two chunks per barrier halve the barriers and let a wave's matrix-core work
// on one chunk overlap its vector work on the other (measured +7 % on the
// prefill chunk against one; three per barrier, with rings of six, ran 4 %
// slower for Q8_0/Q4_0 and 1-2 % slower for Q4_0/Q4_0 and do not fit the LDS
// for F16).
constexpr int kViewBytes = 16384;  // K' [tt][b][lane] x 16 B, then V' [n][lane] x 16 B

// Scores for NT row tiles from the f16 view, relative to each tile's
// reference (the MFMA accumulator starts at -reference): S^T = K' Q^T, four
// blocks accumulated in the MFMA.
template <int NT>
__device__ __forceinline__ void view_scores(const RowState (&st)[NT], const uint8_t *view, int lane,
                                            float (&s)[NT][8]) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        floatx4 d[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float ref = score_ref(st[t]);
            d[t] = floatx4{-ref, -ref, -ref, -ref};
        }
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const half8 kf = *reinterpret_cast<const half8 *>(view + ((tt * 4 + b) * 64 + lane) * 16);
#pragma unroll
            for (int t = 0; t < NT; t++) d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, st[t].qf[b], d[t], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int v = 0; v < 4; v++) s[t][4 * tt + v] = d[t][v];
    }
}

// Softmax step of one chunk for one row tile from its relative scores (lazy
// reference as in chunk_probs); P rounded to binary16 once.
__device__ __forceinline__ void view_probs(RowState &st, float (&s)[8], half8 &pf, uint32_t *counter) {
    update_reference(st, s, counter);
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        p[i] = fast_exp2(s[i]);
        lsum += p[i];
    }
    st.l_run += lsum;
    pf = half8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
               (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
}

template <int NT>
__device__ __forceinline__ void view_pv(RowState (&st)[NT], const uint8_t *view, int lane, const half8 (&pf)[NT]) {
#pragma unroll
    for (int n = 0; n < 8; n++) {
        const half8 vf = *reinterpret_cast<const half8 *>(view + 8192 + (n * 64 + lane) * 16);
#pragma unroll
        for (int t = 0; t < NT; t++) st[t].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[t], st[t].acc[n], 0, 0, 0);
    }
}

__device__ __forceinline__ half8 h8_mul(half8 x, uint4 sc) {
    const half2v a = bits_h2(sc.x), b = bits_h2(sc.y), c = bits_h2(sc.z), d = bits_h2(sc.w);
    return half8{x[0] * a.x, x[1] * a.y, x[2] * b.x, x[3] * b.y, x[4] * c.x, x[5] * c.y, x[6] * d.x, x[7] * d.y};
}

// Dequantise one staged raw chunk into the f16 view.  Threads 0..255: key
// tile tt = q / 2 and blocks b0 = 2 (q mod 2), b0 + 1 of lane l (q = t / 64,
// l = t mod 64); threads 256..511: value block h = (t - 256) / 64, dim tiles
// 2h and 2h + 1 of lane l.  n_valid < 32 marks the chunk holding the end of
// the history: V' of keys at or past it is zeroed (their codes and scales
// are page padding).  F16 data are copied as they are.
template <int KT, int VT>
__device__ __forceinline__ void dequant_view(const uint8_t *raw, uint8_t *view, uint32_t n_valid) {
    using C = Chunk<KT, VT>;
    const int t = threadIdx.x, l = t & 63;
    if (t < 256) {
        const int q = t >> 6, tt = q >> 1, b0 = 2 * (q & 1);
        half8 o0, o1;
        if constexpr (KT == kTypeF16) {
            o0 = *reinterpret_cast<const half8 *>(raw + tt * 4096 + b0 * 1024 + l * 16);
            o1 = *reinterpret_cast<const half8 *>(raw + tt * 4096 + (b0 + 1) * 1024 + l * 16);
        } else {
            half8 k0, k1;
            if constexpr (KT == kTypeQ8_0) {
                const uint4 w = *reinterpret_cast<const uint4 *>(raw + q * 1024 + l * 16);
                k0 = q8_to_half8(w.x, w.y);
                k1 = q8_to_half8(w.z, w.w);
            } else {
                const uint2 w = *reinterpret_cast<const uint2 *>(raw + tt * 1024 + l * 16 + b0 * 4);
                k0 = q4_to_half8(w.x);
                k1 = q4_to_half8(w.y);
            }
            const uint32_t key = 16 * tt + (l & 15);
            const uint32_t sc = *reinterpret_cast<const uint32_t *>(raw + C::off_ks + key * 8 + b0 * 2);
            const _Float16 d0 = bits_h2(sc).x, d1 = bits_h2(sc).y;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                o0[i] = k0[i] * d0;
                o1[i] = k1[i] * d1;
            }
        }
        *reinterpret_cast<half8 *>(view + ((tt * 4 + b0) * 64 + l) * 16) = o0;
        *reinterpret_cast<half8 *>(view + ((tt * 4 + b0 + 1) * 64 + l) * 16) = o1;
    } else if (t < 512) {
        const int h = (t - 256) >> 6, g = l >> 4;
        half8 v0, v1;
        if constexpr (VT == kTypeF16) {
            v0 = *reinterpret_cast<const half8 *>(raw + C::off_v + (2 * h) * 1024 + l * 16);
            v1 = *reinterpret_cast<const half8 *>(raw + C::off_v + (2 * h + 1) * 1024 + l * 16);
        } else {
            const uint4 sc = *reinterpret_cast<const uint4 *>(raw + C::off_vs + (h * 4 + g) * 16);
            if constexpr (VT == kTypeQ4_0) {
                const uint2 w = *reinterpret_cast<const uint2 *>(raw + C::off_v + (h >> 1) * 1024 + l * 16 + (h & 1) * 8);
                v0 = h8_mul(q4_to_half8(w.x), sc);
                v1 = h8_mul(q4_to_half8(w.y), sc);
            } else {
                const uint4 w = *reinterpret_cast<const uint4 *>(raw + C::off_v + h * 1024 + l * 16);
                v0 = h8_mul(q8_to_half8(w.x, w.y), sc);
                v1 = h8_mul(q8_to_half8(w.z, w.w), sc);
            }
        }
        if (n_valid < 32) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t key = 16 * (j >> 2) + 4 * g + (j & 3);  // key of operand slot j
                if (key >= n_valid) {
                    v0[j] = (_Float16)0.f;
                    v1[j] = (_Float16)0.f;
                }
            }
        }
        *reinterpret_cast<half8 *>(view + 8192 + ((2 * h) * 64 + l) * 16) = v0;
        *reinterpret_cast<half8 *>(view + 8192 + ((2 * h + 1) * 64 + l) * 16) = v1;
    }
}

// COUNT: the test instantiation that counts softmax re-reference events.
template <int KT, int VT, int WAVES, bool COUNT>
__global__ __launch_bounds__((64 * WAVES), 1) void wide_kernel(const SplitArgs a) {
    using C = Chunk<KT, VT>;
    constexpr int NT = 2;
    constexpr int kRows = kWideRowsPerWave * WAVES;
    // a chunk's loads, spread over the waves: wave w issues loads w, w + WAVES, ...
    constexpr int kLoadsMax = (C::dma + WAVES - 1) / WAVES;
    // two chunks per barrier: raw chunks and f16 views in rings of four
    __shared__ __attribute__((aligned(16))) uint8_t raw_ring[4][C::bytes];
    __shared__ __attribute__((aligned(16))) uint8_t views[4][kViewBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4;
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.y;
    const uint32_t block_row0 = blockIdx.z * kRows;
    const uint32_t wave_row0 = block_row0 + kWideRowsPerWave * wave;
    const uint32_t rows_kv = a.W * a.G;
    const uint32_t n_chunks_all = (a.n_tokens + 31) >> 5;
    const uint32_t cpp = a.T >> 5;
    // a split is a range of split_chunks chunks, or (page list) one page
    const uint32_t split = blockIdx.x;
    uint32_t c_begin, c_end;
    if (a.page_list) {
        c_begin = table_at(a.page_list, a.list_offset + split) * cpp;
        c_end = min(c_begin + cpp, n_chunks_all);
    } else {
        c_begin = split * a.split_chunks;
        c_end = min(c_begin + a.split_chunks, n_chunks_all);
    }
    const uint32_t n = c_end - c_begin;  // chunks of this split (>= 1)
    const uint32_t clean_end = (a.n_tokens - a.W + 1) >> 5;
    const bool active = wave_row0 < rows_kv;  // wave has rows to compute

    // this wave's share of a chunk's direct-to-LDS loads
    uint32_t my_loads = 0;
#pragma unroll
    for (int i = 0; i < kLoadsMax; i++) my_loads += (uint32_t)(wave + WAVES * i < C::dma);
    auto issue = [&](uint32_t p) {
        if (my_loads == 0) return;
        const uint32_t chunk = c_begin + p;
        const uint32_t page = chunk / cpp;
        const uint32_t jj0 = (chunk - page * cpp) << 5;
        const uint8_t *base = resolve_page(a, page);
        const uint32_t dst = lds_addr(raw_ring[p & 3]);
#pragma unroll
        for (int i = 0; i < kLoadsMax; i++)
            if (wave + WAVES * i < C::dma) issue_chunk_part<KT, VT, false>(a, base, kvh, jj0, lane, dst, wave + WAVES * i);
    };
    static_assert(2 * kLoadsMax <= 8, "wait_vmcnt_upto range");
    auto n_valid_of = [&](uint32_t p) {
        const uint32_t c = c_begin + p;
        return 32 * c + 32 > a.n_tokens ? a.n_tokens - 32 * c : 32u;
    };

    // ---- queries (two 16-row tiles per wave), converted before any ring load
    RowState st[NT];
    float4 qraw[NT][8];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        st[t].row_pos = -1;
        st[t].m_ref = kNegInf;
        st[t].l_run = 0.f;
#pragma unroll
        for (int k = 0; k < 8; k++) st[t].acc[k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; i++) qraw[t][i] = float4{0.f, 0.f, 0.f, 0.f};
        const uint32_t r = wave_row0 + 16 * t + c16;
        if (r < rows_kv) {
            const uint32_t w = r / a.G, hh = r - w * a.G;
            const uint32_t h = kvh * a.G + hh;
            st[t].row_pos = (int)(a.n_tokens - a.W + w);
            const float4 *qp = reinterpret_cast<const float4 *>(a.q + ((size_t)w * a.Hq + h) * 128 + 8 * grp);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                qraw[t][2 * b] = qp[8 * b];
                qraw[t][2 * b + 1] = qp[8 * b + 1];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float4 x = qraw[t][2 * b], y = qraw[t][2 * b + 1];
            st[t].qf[b] = half8{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale), (_Float16)(x.z * a.qscale),
                                (_Float16)(x.w * a.qscale), (_Float16)(y.x * a.qscale), (_Float16)(y.y * a.qscale),
                                (_Float16)(y.z * a.qscale), (_Float16)(y.w * a.qscale)};
            asm volatile("" ::"v"(st[t].qf[b]) : "memory");
        }

    // ---- prologue: raw chunks 0..3 in flight, chunks 0 and 1 into views 0, 1
#pragma unroll
    for (uint32_t p = 0; p < 4; p++)
        if (p < n) issue(p);
    wait_vmcnt_upto((min(n, 4u) - min(n, 2u)) * my_loads);
    __syncthreads();
    dequant_view<KT, VT>(raw_ring[0], views[0], n_valid_of(0));
    if (1 < n) dequant_view<KT, VT>(raw_ring[1], views[1], n_valid_of(1));

    auto compute_chunk = [&](uint32_t p) {
        const uint8_t *view = views[p & 3];
        const uint32_t c = c_begin + p;
        float s[NT][8];
        half8 pf[NT];
        view_scores<NT>(st, view, lane, s);
        if (c >= clean_end) mask_scores<NT>(st, 32 * c, grp, s);
#pragma unroll
        for (int t = 0; t < NT; t++) view_probs(st[t], s[t], pf[t], COUNT ? a.rescale_count : nullptr);
        view_pv<NT>(st, view, lane, pf);
    };
    // step of two chunks: p and p + 1 are computed from their views while
    // p + 2, p + 3 are dequantised and p + 4, p + 5 are loaded (chunk q's raw
    // buffer and view: q mod 4)
    for (uint32_t p = 0; p < n; p += 2) {
        // raw chunks p + 2, p + 3 landed (nothing was issued after them)
        if (p + 2 < n) wait_vmcnt_upto(0);
        __syncthreads();
        if (p + 4 < n) issue(p + 4);
        if (p + 5 < n) issue(p + 5);
        if (p + 2 < n) dequant_view<KT, VT>(raw_ring[(p + 2) & 3], views[(p + 2) & 3], n_valid_of(p + 2));
        if (p + 3 < n) dequant_view<KT, VT>(raw_ring[(p + 3) & 3], views[(p + 3) & 3], n_valid_of(p + 3));
        if (active) {
            compute_chunk(p);
            if (p + 1 < n) compute_chunk(p + 1);
        }
    }

    // ---- partials of this wave's rows (slot `split`; an accumulating slot
    // combines with what it holds: the wave owns the row, so its reads of
    // the stored values precede its writes)
    const uint32_t units = a.W * a.Hq;
    const bool accum = split < a.accum_slots;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        float l = st[t].l_run;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const uint32_t r = wave_row0 + 16 * t + c16;
        if (r < rows_kv) {
            const uint32_t w = r / a.G, hh = r - w * a.G;
            const uint32_t unit = w * a.Hq + kvh * a.G + hh;
            const size_t pu = (size_t)split * units + unit;
            float m = st[t].m_ref;
            if (accum) {
                const PartCombine c = part_combine(a.part_ml[pu * 2], a.part_ml[pu * 2 + 1], m, l);
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const floatx4 old = *reinterpret_cast<const floatx4 *>(a.part_o + pu * 128 + 16 * k + 4 * grp);
                    st[t].acc[k] = (c.w0 > 0.f ? c.w0 * old : floatx4{0.f, 0.f, 0.f, 0.f}) + c.w1 * st[t].acc[k];
                }
                m = c.m;
                l = c.l;
            }
#pragma unroll
            for (int k = 0; k < 8; k++)
                *reinterpret_cast<floatx4 *>(a.part_o + pu * 128 + 16 * k + 4 * grp) = st[t].acc[k];
            if (grp == 0) {
                a.part_ml[pu * 2] = m;
                a.part_ml[pu * 2 + 1] = l;
            }
        }
    }
}

}  // namespace kvattn_dev

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t kvattn_launch_wide(const SplitArgs &a, uint32_t n_splits, uint32_t n_row_blocks, int waves, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
    using namespace kvattn_dev;
    (void)hipGetLastError();
    if (waves != 8 && waves != 12) return hipErrorInvalidValue;
    const dim3 grid(n_splits, a.Hkv, n_row_blocks), block(64 * waves);
    auto go = [&](auto kern) {
        if (ev_start)
            hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev_start, ev_stop, 0, a);
        else
            hipLaunchKernelGGL(kern, grid, block, 0, s, a);
    };
    const bool count = a.rescale_count != nullptr;
    auto pick = [&](auto ktc, auto vtc) {
        constexpr int KT = decltype(ktc)::value, VT = decltype(vtc)::value;
        if (waves == 8)
            count ? go(wide_kernel<KT, VT, 8, true>) : go(wide_kernel<KT, VT, 8, false>);
        else
            count ? go(wide_kernel<KT, VT, 12, true>) : go(wide_kernel<KT, VT, 12, false>);
    };
    using F16 = std::integral_constant<int, kTypeF16>;
    using Q4 = std::integral_constant<int, kTypeQ4_0>;
    using Q8 = std::integral_constant<int, kTypeQ8_0>;
    if (a.k_type == kTypeQ8_0 && a.v_type == kTypeQ4_0)
        pick(Q8{}, Q4{});
    else if (a.k_type == kTypeQ8_0 && a.v_type == kTypeQ8_0)
        pick(Q8{}, Q8{});
    else if (a.k_type == kTypeQ4_0 && a.v_type == kTypeQ4_0)
        pick(Q4{}, Q4{});
    else if (a.k_type == kTypeF16 && a.v_type == kTypeF16)
        pick(F16{}, F16{});
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

uint32_t kvattn_wide_rows_per_wave() { return kvattn_dev::kWideRowsPerWave; }
