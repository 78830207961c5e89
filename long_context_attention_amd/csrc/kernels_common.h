// kernels_common.h -- device helpers shared by the gfx950 kernels for paged
// Q8_0-K / Q4_0-V attention (split_kernel.hip, wide_kernel.hip,
// writer_kernel.hip, copy_kernels.hip).
//
//   split_kernel  calls with up to 32 rows per KV head (decode, verify): one
//                 workgroup per (split of 32-key chunks, KV head); every wave
//                 streams its own chunks into an LDS ring with direct-to-LDS
//                 loads and computes all rows of the block.
//   wide_kernel   calls with more rows (prefill chunks): one workgroup per
//                 (split, KV head, 256-row block); each chunk is turned into
//                 an f16 view of K and V once and shared by all 256 rows.
//   merge_kernel  log-sum-exp merge of the split partials in split order;
//                 splits with l = 0 are skipped (the zero guard the review
//                 finds missing in the chunk normaliser).
// Both attention kernels write one un-normalised partial (m, l, acc[128]) per
// split and row ("troed's fork of Raymond's adaptive KV streaming", section
// "Keep the stock attention order": per-span partials, then one final
// reduction; "Block KV cache streaming ...", maintainer review: kernels with a
// partial-output mode followed by a combine).
//
// Arithmetic (per KV head, 16 keys x 16 query rows per matrix-core tile,
// v_mfma_f32_16x16x32_f16, fp32 accumulation).  Split kernel:
//   S^T = K . Q^T     A = K codes (int8 -> exact f16 by a byte permute), one
//                     MFMA per 32-dim block, each block's fp32 dot scaled by
//                     its own binary16 d_K before the blocks are summed;
//                     B = Q * softmax_scale * log2(e), rounded to f16.
//   O^T += V^T . P'^T A = V codes (n - 8, exact f16), B = P * d_V per (row,
//                     key, 32-dim block), rounded to f16 once.
// Wide kernel: K' = c * d_K and V' = (n - 8) * d_V rounded to binary16 once
// each (the f16 working view), P rounded to f16.
// Softmax in fp32 with exp2 and a lazily moved per-row reference; row max and
// sum reduced across the four 16-lane groups of a wavefront.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace kvattn_dev {

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Code conversion.  Byte b | 0x6400 as binary16 is 1024 + b exactly (ulp 1 in
// [1024, 2048)), so one v_perm places two codes into an f16 pair and one
// packed subtract removes the bias.
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v bits_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// 8 int8 codes (two dwords) -> 8 exact f16, byte i -> element i.
__device__ __forceinline__ half8 q8_to_half8(uint32_t w0, uint32_t w1) {
    const uint32_t k64 = 0x64646464u;
    const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;  // c + 128 in [0, 255]
    half2v a = bits_h2(__builtin_amdgcn_perm(k64, u0, 0x04010400u)) - bias;
    half2v b = bits_h2(__builtin_amdgcn_perm(k64, u0, 0x04030402u)) - bias;
    half2v c = bits_h2(__builtin_amdgcn_perm(k64, u1, 0x04010400u)) - bias;
    half2v d = bits_h2(__builtin_amdgcn_perm(k64, u1, 0x04030402u)) - bias;
    return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// 8 Q4_0 codes in one dword -> 8 exact f16 (n - 8): element m (0..3) is the
// low nibble of byte m, element 4 + m the high nibble of byte m.
__device__ __forceinline__ half8 q4_to_half8(uint32_t w) {
    const uint32_t k64 = 0x64646464u;
    const half2v bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    half2v a = bits_h2(__builtin_amdgcn_perm(k64, lo, 0x04010400u)) - bias;
    half2v b = bits_h2(__builtin_amdgcn_perm(k64, lo, 0x04030402u)) - bias;
    half2v c = bits_h2(__builtin_amdgcn_perm(k64, hi, 0x04010400u)) - bias;
    half2v d = bits_h2(__builtin_amdgcn_perm(k64, hi, 0x04030402u)) - bias;
    return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ float h2f_lo(uint32_t u) { return (float)bits_h2(u).x; }
__device__ __forceinline__ float h2f_hi(uint32_t u) { return (float)bits_h2(u).y; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Page resolution: device page-table entry -> page base address.
//   e < 0x80000000            pool page e
//   0x80000000 | s (bit 30 0) ring slot s placed by the caller
//   0xC0000000 | o            streamed page with per-layer ordinal o: ring
//                             slot (ring_base + o) mod n_ring_slots
// The entry index is wave-uniform, so the entry comes through a scalar load.
// ---------------------------------------------------------------------------
__device__ __forceinline__ const uint8_t *page_base(const SplitArgs &a, uint32_t e) {
    if (e < 0x80000000u) return a.pool + (size_t)e * a.page_bytes;
    uint32_t v = e & 0x3FFFFFFFu;
    if (e & 0x40000000u) v = (a.ring_base + v) % a.n_ring_slots;  // both < 2^30: no overflow
    return a.ring + (size_t)v * a.page_bytes;
}

// Page-table and page-list reads through the constant address space: the
// tables do not change during a launch, so wave-uniform reads become scalar
// loads even after the loads the compiler cannot see (direct-to-LDS asm).
typedef __attribute__((address_space(4))) const uint32_t const_u32;
__device__ __forceinline__ uint32_t table_at(const uint32_t *t, uint32_t i) {
    return reinterpret_cast<const_u32 *>(reinterpret_cast<uintptr_t>(t))[i];
}

__device__ __forceinline__ const uint8_t *resolve_page(const SplitArgs &a, uint32_t logical_page) {
    return page_base(a, table_at(a.page_table, logical_page));
}

// ---------------------------------------------------------------------------
// One 32-key chunk of one KV head as staged in LDS (6656 bytes; each section
// keeps the page's byte order):
//   [0, 4096)     K codes, two 16-key tiles of 2048 bytes; a 64-lane read of
//                 16 bytes per lane covers one 1024-byte quarter
//   [4096, 6144)  V codes, two quarters
//   [6144, 6400)  K scales, [key][block] binary16
//   [6400, 6656)  the chunk's V-scale tile
// Every wave owns a ring of kStages such buffers, filled by direct-to-LDS
// loads (global_load_lds_dwordx4: 16 bytes per lane, no registers), so
// kStages - 1 chunks stay in flight while the wave computes on another.
// ---------------------------------------------------------------------------
constexpr int kChunkBytes = 6656;
constexpr int kOffV = 4096, kOffKS = 6144, kOffVS = 6400;
constexpr int kStages = 3;  // raw-chunk ring of the wide kernel
constexpr int kDmaPerChunk = 7;  // 4 K, 2 V, 1 scales

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from g to LDS bytes [lds + 16 lane, +16).  m0 holds the
// wave's LDS destination; one wait state separates its write from the load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// The compiler does not track the loads above, so the waits are explicit
// (and are compiler barriers for memory accesses).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until at most `newer` (< S) chunks issued after the one needed are in
// flight, for a ring of S stages.
template <int S>
__device__ __forceinline__ void wait_chunk(uint32_t newer) {
    static_assert(S == 2 || S == 3, "rings of two or three stages");
    if (S == 3 && newer >= 2)
        wait_vmcnt<2 * kDmaPerChunk>();
    else if (newer >= 1)
        wait_vmcnt<kDmaPerChunk>();
    else
        wait_vmcnt<0>();
}

// Wide kernel: a wave issues at most one load per chunk.
__device__ __forceinline__ void wait_chunk_wide(uint32_t newer) {
    if (newer >= 2)
        wait_vmcnt<2>();
    else if (newer == 1)
        wait_vmcnt<1>();
    else
        wait_vmcnt<0>();
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Issue the direct-to-LDS loads of chunk `chunk` of KV head kvh (page base
// `base`) into the buffer at LDS address dst.
__device__ __forceinline__ void issue_chunk(const SplitArgs &a, const uint8_t *base, uint32_t kvh, uint32_t jj0,
                                            int lane, uint32_t dst) {
    const size_t kv = (size_t)kvh * a.T + jj0;  // first key of the chunk in the head's section
    const uint8_t *kc = base + kv * 128 + lane * 16;
    const uint8_t *vc = base + a.sec_vc + kv * 64 + lane * 16;
#pragma unroll
    for (int q = 0; q < 4; q++) dma16(kc + 1024 * q, dst + 1024 * q);
#pragma unroll
    for (int q = 0; q < 2; q++) dma16(vc + 1024 * q, dst + kOffV + 1024 * q);
    if (lane < 32) {
        const uint8_t *sp = lane < 16 ? base + a.sec_kd + kv * 8 + lane * 16
                                      : base + a.sec_vd + (size_t)kvh * a.T * 8 + (size_t)(jj0 >> 5) * 256 + (lane - 16) * 16;
        dma16(sp, dst + kOffKS);
    }
}

__device__ __forceinline__ void put4(uint32_t *d, const uint4 &x) {
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
}

// K codes of the lane: kq[8tt + ...] = dwords of 16-key tile tt (blocks 2k,
// 2k + 1 of quarter k, 8 codes each).
__device__ __forceinline__ void read_kcodes(const uint8_t *stg, int lane, uint32_t kq[16]) {
#pragma unroll
    for (int q = 0; q < 4; q++) put4(kq + 4 * q, *reinterpret_cast<const uint4 *>(stg + 1024 * q + 16 * lane));
}

// K scales as the lane uses them: kd[8tt + ...] binary16 pairs, key 4g + v
// of tile tt, block b at half 4v + b.
__device__ __forceinline__ void read_kscales(const uint8_t *stg, int grp, uint32_t kd[16]) {
    const uint4 *k4 = reinterpret_cast<const uint4 *>(stg + kOffKS);  // key j at bytes 8j
    put4(kd + 0, k4[2 * grp]);
    put4(kd + 4, k4[2 * grp + 1]);
    put4(kd + 8, k4[8 + 2 * grp]);
    put4(kd + 12, k4[8 + 2 * grp + 1]);
}

// V scales: vd[4b + ...] binary16 pairs of block b, operand slots 2i, 2i + 1.
__device__ __forceinline__ void read_vscales(const uint8_t *stg, int grp, uint32_t vd[16]) {
    const uint4 *v4 = reinterpret_cast<const uint4 *>(stg + kOffVS);
#pragma unroll
    for (int b = 0; b < 4; b++) put4(vd + 4 * b, v4[b * 4 + grp]);
}

// V codes of the lane: one dword per 16-dim tile.
__device__ __forceinline__ void read_vcodes(const uint8_t *stg, int lane, uint32_t vq[8]) {
#pragma unroll
    for (int q = 0; q < 2; q++) put4(vq + 4 * q, *reinterpret_cast<const uint4 *>(stg + kOffV + 1024 * q + 16 * lane));
}

// binary16 half `i` of a packed array (lo half = even index)
__device__ __forceinline__ float half_of(const uint32_t *w, int i) { return (i & 1) ? h2f_hi(w[i >> 1]) : h2f_lo(w[i >> 1]); }

// Softmax reference of a row moves only when a score exceeds it by more than
// kRescale (log2 units), so P = exp2(s - ref) <= 2^kRescale stays exact
// enough in binary16 and the accumulators are rarely rescaled.  Any
// reference gives the same result in exact arithmetic; the partial carries
// the reference it used.
constexpr float kRescale = 8.0f;

// Per-wave state of one tile of 16 query rows (the lane's row is c16).
struct RowState {
    half8 qf[4];     // B operand of S^T = K Q^T, block b
    int row_pos;     // position of the lane's row; -1 = padding row
    float m_ref;     // softmax reference (log2 units), uniform per row
    float l_run;     // lane's share of the softmax denominator
    floatx4 acc[8];  // O^T tile n: dims 16n + 4g + v of the lane's row
};

// Scores of one chunk for NT row tiles: s[t][4tt + v] is key 16tt + 4g + v
// of the chunk for tile t, log2-scaled.  Each K fragment is dequantised once
// and feeds one MFMA per tile and 32-dim block, scaled by that block's d_K.
template <int NT>
__device__ __forceinline__ void chunk_scores(const RowState (&st)[NT], const uint32_t kq[16], const uint32_t kd[16],
                                             float (&s)[NT][8]) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        // all MFMAs of the key tile first, so none waits on the one before
        floatx4 d[4][NT];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const uint32_t *w = kq + 8 * tt + 4 * (b >> 1) + 2 * (b & 1);
            const half8 kf = q8_to_half8(w[0], w[1]);
#pragma unroll
            for (int t = 0; t < NT; t++)
                d[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, st[t].qf[b], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; t++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                // fma with the binary16 operand read in place (v_fma_mix_f32)
                float acc = half_of(kd + 8 * tt, 4 * v) * d[0][t][v];
#pragma unroll
                for (int b = 1; b < 4; b++) acc = __builtin_fmaf(half_of(kd + 8 * tt, 4 * v + b), d[b][t][v], acc);
                s[t][4 * tt + v] = acc;
            }
    }
}

// Causal mask of a chunk holding keys past some row's position.
template <int NT>
__device__ __forceinline__ void mask_scores(const RowState (&st)[NT], uint32_t kpos0, int grp, float (&s)[NT][8]) {
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int key = (int)(kpos0 + 16 * (i >> 2) + 4 * grp + (i & 3));
            if (key > st[t].row_pos) s[t][i] = kNegInf;
        }
}

// Keys at or past the history length sit on page padding whose V scales may
// be anything (NaN included); zero them in the staged tile so P * d_V is 0
// for those keys (their P is 0).  Lane l owns tile bytes 4l .. 4l + 3:
// block l / 16, keys 16 hi + 4 q + r with q = (l / 4) mod 4, hi = (l mod 4) / 2,
// r = 2 (l mod 2) + i for the dword's half i.
__device__ __forceinline__ void sanitize_vscales(uint8_t *stg, int lane, uint32_t n_valid) {
    uint32_t *w = reinterpret_cast<uint32_t *>(stg + kOffVS) + lane;
    const uint32_t key0 = 16 * ((lane & 3) >> 1) + 4 * ((lane >> 2) & 3) + 2 * (lane & 1);
    uint32_t v = *w;
    if (key0 >= n_valid) v &= 0xFFFF0000u;
    if (key0 + 1 >= n_valid) v &= 0x0000FFFFu;
    *w = v;
}

// Softmax step of one chunk for one row tile: lazy reference update
// (rescaling the accumulators, which already hold every earlier chunk),
// probabilities, the denominator, and the P' operands P * d_V of the four
// value blocks.
__device__ __forceinline__ void chunk_probs(RowState &st, const float s[8], const uint32_t vd[16], half8 pf[4]) {
    float m = s[0];
#pragma unroll
    for (int i = 1; i < 8; i++) m = fmaxf(m, s[i]);
    if (__any(m > st.m_ref + kRescale)) {
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float m_new = fmaxf(st.m_ref, m);
        const float alpha = (st.m_ref == kNegInf) ? 0.f : fast_exp2(st.m_ref - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int n = 0; n < 8; n++) st.acc[n] *= alpha;
        st.m_ref = m_new;
    }
    const float mu = (st.m_ref == kNegInf) ? 0.f : st.m_ref;
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        p[i] = fast_exp2(s[i] - mu);
        lsum += p[i];
    }
    st.l_run += lsum;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; i++) e[i] = __builtin_fmaf(p[i], half_of(vd + 4 * b, i), 0.0f);
        pf[b] = half8{(_Float16)e[0], (_Float16)e[1], (_Float16)e[2], (_Float16)e[3],
                      (_Float16)e[4], (_Float16)e[5], (_Float16)e[6], (_Float16)e[7]};
    }
}

// O^T += V^T P'^T for one chunk and NT row tiles: dim tile n = 2b + nn of
// value block b; each V fragment is dequantised once.
template <int NT>
__device__ __forceinline__ void chunk_pv(RowState (&st)[NT], const uint32_t vq[8], const half8 (&pf)[NT][4]) {
#pragma unroll
    for (int n = 0; n < 8; n++) {
        const half8 vf = q4_to_half8(vq[n]);
#pragma unroll
        for (int t = 0; t < NT; t++)
            st[t].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[t][n >> 1], st[t].acc[n], 0, 0, 0);
    }
}

}  // namespace kvattn_dev
