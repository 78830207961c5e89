// attn_kernels.hip -- gfx950 kernels for paged Q8_0-K / Q4_0-V attention.
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

// ---------------------------------------------------------------------------
// Split kernel.  A workgroup of 8 waves handles one split (a range of 32-key
// chunks) of one KV head for a block of 16 * NT query rows; the waves take
// the split's chunks round robin and each computes every row of the block,
// so a chunk is loaded and dequantised once per block.  Rows of a KV head
// are ordered (w, hh): r = w * G + hh, hh < G.
// Each wave streams its chunks through its own LDS ring and overlaps chunk
// i's Q.K^T with chunk i-1's P.V, whose operands it carries over.
// ---------------------------------------------------------------------------
// Shape per row-tile count: one tile (<= 16 rows per KV head) needs few
// registers, so 12 waves (three per SIMD) with two-stage rings; two tiles
// need about 250 registers, so 8 waves with three-stage rings.  Both fill
// 159,744 bytes of LDS.
template <int NT>
struct SplitCfg {
    static constexpr int waves = NT == 1 ? 12 : 8;
    static constexpr int stages = NT == 1 ? 2 : 3;
    static constexpr int ring_bytes = stages * kChunkBytes;
    static constexpr int lds_bytes = waves * ring_bytes;
};

template <int NT>
__global__ __launch_bounds__(64 * SplitCfg<NT>::waves, 1) void split_kernel(const SplitArgs a) {
    constexpr int kSplitWaves = SplitCfg<NT>::waves;
    constexpr int kStages = SplitCfg<NT>::stages;
    constexpr int kWaveRingBytes = SplitCfg<NT>::ring_bytes;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // rings; reused by the combine and merge

    const int lane = threadIdx.x & 63;
    // wave index, made visibly uniform so chunk bookkeeping stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4;  // 16-lane group
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.y;
    const uint32_t block_row0 = blockIdx.z * (16 * NT);
    const uint32_t rows_kv = a.W * a.G;
    const uint32_t n_chunks_all = (a.n_tokens + 31) >> 5;
    const uint32_t cpp = a.T >> 5;  // chunks per page

    // ---- split -> chunk range
    uint32_t split, c_begin, c_end;
    if (a.page_list) {
        split = table_at(a.page_list, a.list_offset + blockIdx.x);
        c_begin = split * cpp;
        c_end = min(c_begin + cpp, n_chunks_all);
    } else {
        split = blockIdx.x;
        c_begin = blockIdx.x * a.split_chunks;
        c_end = min(c_begin + a.split_chunks, n_chunks_all);
    }
    // chunks whose keys every row sees (keys <= n_tokens - W) need no mask
    const uint32_t clean_end = (a.n_tokens - a.W + 1) >> 5;
    // this wave's chunks: first + kSplitWaves * k, k < n_local
    const uint32_t first = c_begin + wave;
    const uint32_t n_local = first < c_end ? (c_end - 1 - first) / kSplitWaves + 1 : 0;

    uint8_t *ring = smem + wave * kWaveRingBytes;
    const uint32_t ring_lds = lds_addr(ring);
    auto chunk_page = [&](uint32_t k) { return (first + kSplitWaves * k) / cpp; };
    auto issue = [&](uint32_t k, uint32_t entry, uint32_t stage) {
        const uint32_t chunk = first + kSplitWaves * k;
        const uint32_t jj0 = (chunk - (chunk / cpp) * cpp) << 5;
        issue_chunk(a, page_base(a, entry), kvh, jj0, lane, ring_lds + stage * kChunkBytes);
    };

    // ---- query loads and the first page entries, one round trip together;
    // the queries are converted before the ring prologue, so no wait on them
    // (the compiler's vmcnt counts only its own loads) covers the ring loads
    RowState st[NT];
    float4 qraw[NT][8];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        st[t].row_pos = -1;
        st[t].m_ref = kNegInf;
        st[t].l_run = 0.f;
#pragma unroll
        for (int n = 0; n < 8; n++) st[t].acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 8; i++) qraw[t][i] = float4{0.f, 0.f, 0.f, 0.f};
        const uint32_t r = block_row0 + 16 * t + c16;
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
    uint32_t entry0[kStages];
#pragma unroll
    for (uint32_t k = 0; k < kStages; k++) entry0[k] = k < n_local ? table_at(a.page_table, chunk_page(k)) : 0u;

    // ---- query fragments: lane (row c16, group g) holds dims 32b + 8g .. +8
    // of block b, pre-scaled by softmax_scale * log2(e)
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float4 x = qraw[t][2 * b], y = qraw[t][2 * b + 1];
            st[t].qf[b] = half8{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale), (_Float16)(x.z * a.qscale),
                                (_Float16)(x.w * a.qscale), (_Float16)(y.x * a.qscale), (_Float16)(y.y * a.qscale),
                                (_Float16)(y.z * a.qscale), (_Float16)(y.w * a.qscale)};
        }

    // the fragments exist before the first ring load is issued
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int b = 0; b < 4; b++) asm volatile("" ::"v"(st[t].qf[b]) : "memory");

    // ---- ring prologue: chunks 0 .. kStages - 2 in flight; page entries
    // (scalar loads) run one chunk ahead of their use
#pragma unroll
    for (uint32_t k = 0; k < kStages - 1; k++)
        if (k < n_local) issue(k, entry0[k], k);
    uint32_t entry_next = entry0[kStages - 1];

    if (n_local > 0) {
        uint32_t pv_vq[8];
        half8 pv_pf[NT][4];
        uint32_t stage = 0;
        for (uint32_t k = 0; k < n_local; k++) {
            // refill the buffer chunk k - 1 used (its reads are complete)
            if (k + kStages - 1 < n_local) {
                wait_lgkmcnt0();
                issue(k + kStages - 1, entry_next, stage == 0 ? kStages - 1 : stage - 1);
                if (k + kStages < n_local) entry_next = table_at(a.page_table, chunk_page(k + kStages));
            }
            wait_chunk<kStages>(min((uint32_t)(kStages - 1), n_local - 1 - k));
            const uint8_t *stg = ring + stage * kChunkBytes;
            const uint32_t c = first + kSplitWaves * k;
            uint32_t kq[16], kd[16], vd[16];
            float s[NT][8];
            read_kcodes(stg, lane, kq);
            read_kscales(stg, grp, kd);
            chunk_scores<NT>(st, kq, kd, s);
            if (c >= clean_end) mask_scores<NT>(st, 32 * c, grp, s);
            if (k > 0) chunk_pv<NT>(st, pv_vq, pv_pf);
            if (32 * c + 32 > a.n_tokens) sanitize_vscales(ring + stage * kChunkBytes, lane, a.n_tokens - 32 * c);
            read_vscales(stg, grp, vd);
#pragma unroll
            for (int t = 0; t < NT; t++) chunk_probs(st[t], s[t], vd, pv_pf[t]);
            read_vcodes(stg, lane, pv_vq);
            stage = stage == kStages - 1 ? 0 : stage + 1;
        }
        chunk_pv<NT>(st, pv_vq, pv_pf);
    }

    // ---- combine the waves (fixed wave order) and write the partials; the
    // rings are reused once every wave is done with its own
    wait_vmcnt<0>();
    __syncthreads();
    constexpr int R = 16 * NT;  // rows per block
    constexpr int OS = 132;     // padded row stride
    float *sm_m = reinterpret_cast<float *>(smem);
    float *sm_l = sm_m + kSplitWaves * R;
    float *sm_o = sm_l + kSplitWaves * R;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        float l = st[t].l_run;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int row = 16 * t + c16;
        if (grp == 0) {
            sm_m[wave * R + row] = st[t].m_ref;
            sm_l[wave * R + row] = l;
        }
#pragma unroll
        for (int n = 0; n < 8; n++)
            *reinterpret_cast<floatx4 *>(&sm_o[(wave * R + row) * OS + 16 * n + 4 * grp]) = st[t].acc[n];
    }
    __syncthreads();

    const uint32_t units = a.W * a.Hq;
    const uint32_t rows_here = min((uint32_t)R, rows_kv - block_row0);
    for (uint32_t idx = threadIdx.x; idx < rows_here * 128; idx += blockDim.x) {
        const uint32_t r = idx >> 7, t = idx & 127;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kSplitWaves; w++) M = fmaxf(M, sm_m[w * R + r]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kSplitWaves; w++) {
                const float mw = sm_m[w * R + r];
                if (mw == kNegInf) continue;
                const float f = fast_exp2(mw - M);
                L += f * sm_l[w * R + r];
                A += f * sm_o[(w * R + r) * OS + t];
            }
        }
        const uint32_t rk = block_row0 + r;
        const uint32_t wq = rk / a.G, hh = rk - wq * a.G;
        const uint32_t unit = wq * a.Hq + kvh * a.G + hh;
        const size_t pu = (size_t)split * units + unit;
        a.part_o[pu * 128 + t] = A;
        if (t == 0) {
            a.part_ml[pu * 2] = M;
            a.part_ml[pu * 2 + 1] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// Wide kernel (prefill chunks, and any call with more than 32 rows per KV
// head).  A workgroup of 8 waves handles one split of one KV head for a block
// of 256 rows; wave w owns rows 32w .. 32w + 31 (two 16-row tiles) over every
// chunk of the split, so no combine across waves is needed.
// Per 32-key chunk the workgroup first turns the staged codes into binary16
// K' = c * d_K and V' = (n - 8) * d_V once (the f16 working view of the
// pages' wide-prefill path), shared through LDS by all 256 rows; the matrix
// cores then run on K' and V' with no per-block scale work in the row loop.
// Each of K', V' is one rounding from the exact product (relative 2^-11).
// Pipeline per chunk p (one barrier): wait for raw chunk p + 1, barrier,
// issue raw chunk p + 3, dequantise p + 1 into the other view buffer,
// compute p.  Raw chunks land in a 3-stage ring by direct-to-LDS loads, the
// seven load instructions of a chunk spread over waves 0..6.
// ---------------------------------------------------------------------------
constexpr int kWideRows = 256;
constexpr int kViewBytes = 16384;  // K' [tt][b][lane] x 16 B, then V' [n][lane] x 16 B

// Scores for NT row tiles from the f16 view: S^T = K' Q^T, four blocks
// accumulated in the MFMA.
template <int NT>
__device__ __forceinline__ void view_scores(const RowState (&st)[NT], const uint8_t *view, int lane,
                                            float (&s)[NT][8]) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        floatx4 d[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) d[t] = floatx4{0.f, 0.f, 0.f, 0.f};
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

// Softmax step of one chunk for one row tile (lazy reference as in
// chunk_probs); P rounded to binary16 once.
__device__ __forceinline__ void view_probs(RowState &st, const float s[8], half8 &pf) {
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

// Dequantise one staged raw chunk into the f16 view.  Threads 0..255: K
// quarter q = t / 64 of lane l = t mod 64 (key tile q / 2, blocks 2 (q mod 2)
// and +1); threads 256..511: V dwords 2h, 2h + 1 of lane l (value block h).
// n_valid < 32 marks the chunk holding the end of the history: V' of keys at
// or past it is zeroed (their scales are page padding).
__device__ __forceinline__ void dequant_view(const uint8_t *raw, uint8_t *view, uint32_t n_valid) {
    const int t = threadIdx.x, l = t & 63;
    if (t < 256) {
        const int q = t >> 6, tt = q >> 1, b0 = 2 * (q & 1);
        const uint4 w = *reinterpret_cast<const uint4 *>(raw + q * 1024 + l * 16);
        const uint32_t key = 16 * tt + (l & 15);
        const uint32_t sc = *reinterpret_cast<const uint32_t *>(raw + kOffKS + key * 8 + b0 * 2);
        const half8 k0 = q8_to_half8(w.x, w.y), k1 = q8_to_half8(w.z, w.w);
        const _Float16 d0 = bits_h2(sc).x, d1 = bits_h2(sc).y;
        half8 o0, o1;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            o0[i] = k0[i] * d0;
            o1[i] = k1[i] * d1;
        }
        *reinterpret_cast<half8 *>(view + ((tt * 4 + b0) * 64 + l) * 16) = o0;
        *reinterpret_cast<half8 *>(view + ((tt * 4 + b0 + 1) * 64 + l) * 16) = o1;
    } else {
        const int h = (t - 256) >> 6, g = l >> 4;
        const uint2 w = *reinterpret_cast<const uint2 *>(raw + kOffV + (h >> 1) * 1024 + l * 16 + (h & 1) * 8);
        const uint4 sc = *reinterpret_cast<const uint4 *>(raw + kOffVS + (h * 4 + g) * 16);
        half8 v0 = h8_mul(q4_to_half8(w.x), sc), v1 = h8_mul(q4_to_half8(w.y), sc);
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

__global__ __launch_bounds__(512, 1) void wide_kernel(const SplitArgs a) {
    constexpr int NT = 2;
    __shared__ __attribute__((aligned(16))) uint8_t raw_ring[kStages][kChunkBytes];
    __shared__ __attribute__((aligned(16))) uint8_t views[2][kViewBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4;
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.y;
    const uint32_t block_row0 = blockIdx.z * kWideRows;
    const uint32_t wave_row0 = block_row0 + 32 * wave;
    const uint32_t rows_kv = a.W * a.G;
    const uint32_t n_chunks_all = (a.n_tokens + 31) >> 5;
    const uint32_t cpp = a.T >> 5;
    const uint32_t split = blockIdx.x;
    const uint32_t c_begin = split * a.split_chunks;
    const uint32_t c_end = min(c_begin + a.split_chunks, n_chunks_all);
    const uint32_t n = c_end - c_begin;  // chunks of this split (>= 1)
    const uint32_t clean_end = (a.n_tokens - a.W + 1) >> 5;
    const bool active = wave_row0 < rows_kv;  // wave has rows to compute

    // this wave's share of a chunk's seven direct-to-LDS loads
    auto issue = [&](uint32_t p) {
        if (wave >= kDmaPerChunk) return;
        const uint32_t chunk = c_begin + p;
        const uint32_t page = chunk / cpp;
        const uint32_t jj0 = (chunk - page * cpp) << 5;
        const uint8_t *base = resolve_page(a, page);
        const size_t kv = (size_t)kvh * a.T + jj0;
        const uint32_t dst = lds_addr(raw_ring[p % kStages]);
        if (wave < 4) {
            dma16(base + kv * 128 + lane * 16 + 1024 * wave, dst + 1024 * wave);
        } else if (wave < 6) {
            dma16(base + a.sec_vc + kv * 64 + lane * 16 + 1024 * (wave - 4), dst + kOffV + 1024 * (wave - 4));
        } else if (lane < 32) {
            const uint8_t *sp = lane < 16 ? base + a.sec_kd + kv * 8 + lane * 16
                                          : base + a.sec_vd + (size_t)kvh * a.T * 8 + (size_t)(jj0 >> 5) * 256 + (lane - 16) * 16;
            dma16(sp, dst + kOffKS);
        }
    };
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

    // ---- prologue: raw chunks 0..2 in flight, chunk 0 into view 0
#pragma unroll
    for (uint32_t p = 0; p < kStages; p++)
        if (p < n) issue(p);
    wait_chunk_wide(min(n - 1, 2u));
    __syncthreads();
    dequant_view(raw_ring[0], views[0], n_valid_of(0));

    for (uint32_t p = 0; p < n; p++) {
        // raw chunk p + 1 landed (every wave waited for its own share)
        if (p + 1 < n) wait_chunk_wide(min(n - 2 - p, 1u));
        __syncthreads();
        if (p + kStages < n) issue(p + kStages);
        if (p + 1 < n) dequant_view(raw_ring[(p + 1) % kStages], views[(p + 1) & 1], n_valid_of(p + 1));
        if (active) {
            const uint8_t *view = views[p & 1];
            const uint32_t c = c_begin + p;
            float s[NT][8];
            half8 pf[NT];
            view_scores<NT>(st, view, lane, s);
            if (c >= clean_end) mask_scores<NT>(st, 32 * c, grp, s);
#pragma unroll
            for (int t = 0; t < NT; t++) view_probs(st[t], s[t], pf[t]);
            view_pv<NT>(st, view, lane, pf);
        }
    }

    // ---- partials of this wave's rows
    const uint32_t units = a.W * a.Hq;
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
#pragma unroll
            for (int k = 0; k < 8; k++)
                *reinterpret_cast<floatx4 *>(a.part_o + pu * 128 + 16 * k + 4 * grp) = st[t].acc[k];
            if (grp == 0) {
                a.part_ml[pu * 2] = st[t].m_ref;
                a.part_ml[pu * 2 + 1] = l;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Merge
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) x = fmaxf(x, __shfl_xor(x, k));
    return x;
}

// Butterfly sum: a + b == b + a, so every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) x += __shfl_xor(x, k);
    return x;
}

// Block-wide log-sum-exp merge (Flash-Decoding's reduction step) of nrows
// (row, query head) units over n_splits >= 1 split partials (m, l, acc[128]).
// For row r (unit unit_of(r)): M = max m_s over splits with l_s > 0,
// w_s = 2^(m_s - M) (0 for empty splits), L = sum w_s l_s, out[t] =
// (sum_s w_s acc_s[t]) / L.  One wave per row computes M, w and L (lane j
// sums splits j, j + 64, ... then a butterfly); dimension t sums splits in
// order.
// Latency: each thread issues its first (m, l) and the first 32 splits of
// its first two dimensions before anything waits, so up to 32 splits and
// 2 x blockDim dimensions take one memory round trip.
// wl: LDS for nrows * n_splits float2; row_ml: LDS for nrows float2.
constexpr int kMergeBatch = 32;

template <class UnitOf>
__device__ __forceinline__ void merge_rows(const float *part_ml, const float *part_o, float *out, uint32_t n_splits,
                                           uint32_t units, uint32_t nrows, UnitOf unit_of, float2 *wl,
                                           float2 *row_ml) {
    const uint32_t nt = blockDim.x, tid = threadIdx.x;
    const size_t mls = (size_t)units * 2, pos = (size_t)units * 128;
    const uint32_t n_ml = nrows * n_splits, n_items = nrows * 128;
    auto ml_at = [&](uint32_t i) {
        const uint32_t r = i / n_splits, s = i - r * n_splits;
        return *reinterpret_cast<const float2 *>(part_ml + s * mls + (size_t)unit_of(r) * 2);
    };
    auto po_of = [&](uint32_t i) { return part_o + (size_t)unit_of(i >> 7) * 128 + (i & 127); };
    // clamped addresses keep every early load unconditional
    const float2 ml0 = ml_at(min(tid, n_ml - 1));
    const float *po0 = po_of(min(tid, n_items - 1)), *po1 = po_of(min(tid + nt, n_items - 1));
    float o0[kMergeBatch], o1[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; k++) {
        const size_t off = (size_t)min((uint32_t)k, n_splits - 1) * pos;
        o0[k] = po0[off];
        o1[k] = po1[off];
    }
    if (tid < n_ml) wl[tid] = ml0;
    for (uint32_t i = tid + nt; i < n_ml; i += nt) wl[i] = ml_at(i);
    __syncthreads();
    const uint32_t lane = tid & 63, nw = nt >> 6;
    for (uint32_t r = __builtin_amdgcn_readfirstlane(tid >> 6); r < nrows; r += nw) {
        float2 *row = wl + r * n_splits;
        float M = kNegInf;
        for (uint32_t s = lane; s < n_splits; s += 64) {
            const float2 v = row[s];
            if (v.y > 0.f) M = fmaxf(M, v.x);
        }
        M = wave_max(M);
        float L = 0.f;
        for (uint32_t s = lane; s < n_splits; s += 64) {
            const float2 v = row[s];
            const float w = v.y > 0.f ? fast_exp2(v.x - M) : 0.f;
            row[s].x = w;
            L += w * v.y;
        }
        L = wave_sum(L);
        if (lane == 0) row_ml[r] = make_float2(M, L);
    }
    __syncthreads();
    const uint32_t nb0 = min(n_splits, (uint32_t)kMergeBatch);
    // dimension i: splits [0, 32) from `first`, the rest loaded here
    auto finish = [&](uint32_t i, const float(&first)[kMergeBatch]) {
        const uint32_t r = i >> 7;
        const float2 *row = wl + r * n_splits;
        const float *po = po_of(i);
        float A = 0.f;
#pragma unroll
        for (int k = 0; k < kMergeBatch; k++)
            if ((uint32_t)k < nb0) A += row[k].x * first[k];
        for (uint32_t s0 = kMergeBatch; s0 < n_splits; s0 += kMergeBatch) {
            float ob[kMergeBatch];
#pragma unroll
            for (int k = 0; k < kMergeBatch; k++) ob[k] = po[(size_t)min(s0 + k, n_splits - 1) * pos];
#pragma unroll
            for (int k = 0; k < kMergeBatch; k++)
                if (s0 + k < n_splits) A += row[s0 + k].x * ob[k];
        }
        out[(size_t)unit_of(r) * 128 + (i & 127)] = A / row_ml[r].y;
    };
    if (tid < n_items) finish(tid, o0);
    if (tid + nt < n_items) finish(tid + nt, o1);
    for (uint32_t i = tid + 2 * nt; i < n_items; i += nt) {
        const float *po = po_of(i);
        float ob[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; k++) ob[k] = po[(size_t)min((uint32_t)k, n_splits - 1) * pos];
        finish(i, ob);
    }
}

// U (row, query head) units per workgroup of 128 U threads: U = 4 for calls
// with thousands of units (prefill chunks) while the splits fit 512 per unit
// in LDS, else one unit per workgroup for up to 4096 splits.
constexpr int kMergeMaxSplits = 4096;
constexpr int kMergeWideUnits = 4, kMergeWideSplits = 512;

template <int U>
__global__ __launch_bounds__(128 * U) void merge_kernel(const MergeArgs a) {
    constexpr int kSplits = U == 1 ? kMergeMaxSplits : kMergeWideSplits;
    __shared__ float2 wl[U * kSplits];
    __shared__ float2 row_ml[U];
    const uint32_t unit0 = blockIdx.x * U;
    const uint32_t nrows = min((uint32_t)U, a.units - unit0);
    merge_rows(a.part_ml, a.part_o, a.out, a.n_splits, a.units, nrows, [=](uint32_t r) { return unit0 + r; }, wl,
               row_ml);
}

// ---------------------------------------------------------------------------
// KV writer ("troed's fork ...", section "KV data movement and attention":
// the new rows are quantised into the tail page before attention reads
// them).  Q8_0 for K: d = amax / 127 rounded to binary16, code =
// round-half-even(x / d) clamped to +-127 (zero scale: codes 0).  Q4_0 for
// V: m = the element of largest magnitude (first on ties), d = m / -8
// rounded to binary16, code = round-half-even(x / d) + 8 clamped to [0, 15]
// (zero scale: codes 8).  Every decision is taken in binary32 (correctly
// rounded division, round-to-nearest-even conversions).
// One workgroup per (32-token tile, KV head): a V byte holds the nibbles of
// tokens j and j + 16 of one tile, so the tile's owner merges new nibbles
// with the ones already there and no two workgroups touch one byte.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint8_t *writer_page(const WriterArgs &a, uint32_t logical_page) {
    const uint32_t e = a.page_table[logical_page];
    if (e < 0x80000000u) return a.pool + (size_t)e * a.page_bytes;
    uint32_t v = e & 0x3FFFFFFFu;
    if (e & 0x40000000u) v = (a.ring_base + v) % a.n_ring_slots;
    return a.ring + (size_t)v * a.page_bytes;
}

__global__ __launch_bounds__(256) void writer_kernel(const WriterArgs a) {
    __shared__ uint8_t nib[32][128];  // V codes of the tile's new tokens
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t h = blockIdx.y;
    const uint32_t tile = a.n_old / 32 + blockIdx.x;
    const uint32_t tb = tile * 32;                       // first position of the tile
    const uint32_t lo = max(a.n_old, tb), hi = min(a.n_old + a.R, tb + 32);
    const uint32_t P = tb / a.T;
    const uint32_t j0 = tb - P * a.T;                    // tile start inside the page
    uint8_t *page = writer_page(a, P);
    const size_t T = a.T;

    const uint32_t e0 = 2 * lane;                        // elements e0, e0 + 1 of block b
    const uint32_t b = lane >> 4, i0 = e0 & 31;
    for (uint32_t jt = wave; jt < 32; jt += 4) {
        const uint32_t pos = tb + jt;
        if (pos < lo || pos >= hi) continue;            // wave-uniform
        const uint32_t r = pos - a.n_old, j = j0 + jt;  // new row, token in the page
        const float2 xk = *reinterpret_cast<const float2 *>(a.k + ((size_t)r * a.Hkv + h) * 128 + e0);
        const float2 xv = *reinterpret_cast<const float2 *>(a.v + ((size_t)r * a.Hkv + h) * 128 + e0);

        // K: Q8_0
        float amax = fmaxf(fabsf(xk.x), fabsf(xk.y));
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) amax = fmaxf(amax, __shfl_xor(amax, k));
        const _Float16 dk16 = (_Float16)(amax / 127.0f);
        const float dk = (float)dk16;
        int c0 = 0, c1 = 0;
        if (dk != 0.0f) {
            c0 = (int)fminf(fmaxf(rintf(xk.x / dk), -127.0f), 127.0f);
            c1 = (int)fminf(fmaxf(rintf(xk.y / dk), -127.0f), 127.0f);
        }
        // byte of (token j, dim t): tile j/16, then (t/64)*1024 +
        // (((t%32)/8)*16 + j%16)*16 + ((t/32)%2)*8 + t%8; e0 is even so the
        // pair is two adjacent bytes
        const uint32_t t = e0;
        const size_t kb = (size_t)h * T * 128 + (size_t)(j / 16) * 2048 + (t / 64) * 1024 +
                          (((t % 32) / 8) * 16 + j % 16) * 16 + ((t / 32) % 2) * 8 + t % 8;
        *reinterpret_cast<uint16_t *>(page + kb) = (uint16_t)((uint8_t)c0 | ((uint16_t)(uint8_t)c1 << 8));
        if ((lane & 15) == 0)
            *reinterpret_cast<_Float16 *>(page + a.sec_kd + ((size_t)h * T + j) * 8 + b * 2) = dk16;

        // V: Q4_0, first element of largest magnitude
        float best = fabsf(xv.x), val = xv.x;
        uint32_t idx = i0;
        if (fabsf(xv.y) > best) {
            best = fabsf(xv.y);
            val = xv.y;
            idx = i0 + 1;
        }
#pragma unroll
        for (int k = 1; k < 16; k <<= 1) {
            const float ob = __shfl_xor(best, k), ov = __shfl_xor(val, k);
            const uint32_t oi = __shfl_xor(idx, k);
            if (ob > best || (ob == best && oi < idx)) {
                best = ob;
                val = ov;
                idx = oi;
            }
        }
        const _Float16 dv16 = (_Float16)(val / -8.0f);
        const float dv = (float)dv16;
        uint32_t n0 = 8, n1 = 8;
        if (dv != 0.0f) {
            n0 = (uint32_t)fminf(fmaxf(rintf(xv.x / dv) + 8.0f, 0.0f), 15.0f);
            n1 = (uint32_t)fminf(fmaxf(rintf(xv.y / dv) + 8.0f, 0.0f), 15.0f);
        }
        nib[jt][e0] = (uint8_t)n0;
        nib[jt][e0 + 1] = (uint8_t)n1;
        if ((lane & 15) == 0) {
            const uint32_t jj = jt;  // token inside the 32-token tile
            *reinterpret_cast<_Float16 *>(page + a.sec_vd + (size_t)h * T * 8 + (size_t)(j / 32) * 256 +
                                          (b * 4 + (jj % 16) / 4) * 16 + ((jj / 16) * 4 + jj % 4) * 2) = dv16;
        }
    }
    __syncthreads();

    // V bytes of the tile: byte of (token jl < 16, dim t) at (t/64)*1024 +
    // ((jl/4)*16 + t%16)*16 + ((t/16)%4)*4 + jl%4, low nibble token jl, high
    // nibble token jl + 16; keep the nibble of a token not written now
    uint8_t *vt = page + a.sec_vc + (size_t)h * T * 64 + (size_t)(j0 / 32) * 2048;
    for (uint32_t i = threadIdx.x; i < 16 * 128; i += blockDim.x) {
        const uint32_t jl = i >> 7, t = i & 127;
        const bool new_lo = tb + jl >= lo && tb + jl < hi;
        const bool new_hi = tb + jl + 16 >= lo && tb + jl + 16 < hi;
        if (!new_lo && !new_hi) continue;
        uint8_t *byte = vt + (t / 64) * 1024 + ((jl / 4) * 16 + t % 16) * 16 + ((t / 16) % 4) * 4 + jl % 4;
        uint8_t v = (new_lo && new_hi) ? 0 : *byte;
        if (new_lo) v = (uint8_t)((v & 0xF0) | nib[jl][t]);
        if (new_hi) v = (uint8_t)((v & 0x0F) | (nib[jl + 16][t] << 4));
        *byte = v;
    }
}

// ---------------------------------------------------------------------------
// Ring copy: the GPU reads the pinned host pages over the host link itself
// (one launch gathers a whole chunk of scattered pages, which a DMA copy per
// run of consecutive pages cannot keep busy).  A workgroup copies one slice
// of one page with four 16-byte loads in flight per thread.
// ---------------------------------------------------------------------------
constexpr int kCopySlices = 8;

__global__ __launch_bounds__(256) void ring_copy_kernel(const RingCopyArgs a) {
    const uint32_t o = a.first + blockIdx.x / kCopySlices;
    const uint32_t sl = blockIdx.x % kCopySlices;
    const size_t n16 = a.page_bytes / 16;
    const size_t per = (n16 + kCopySlices - 1) / kCopySlices;
    const size_t b = sl * per, e = min(n16, b + per);
    const uint4 *src = reinterpret_cast<const uint4 *>(a.history + (size_t)a.list[o] * a.page_bytes);
    uint4 *dst = reinterpret_cast<uint4 *>(a.ring + (size_t)((a.ring_base + o) % a.n_slots) * a.page_bytes);
    const size_t step = blockDim.x;
    for (size_t i = b + threadIdx.x; i < e; i += 4 * step) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (i + u * step < e) v[u] = src[i + u * step];
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (i + u * step < e) dst[i + u * step] = v[u];
    }
}

// ---------------------------------------------------------------------------
// Debug page read: copy a logical page's bytes via the kernels' resolver.
// ---------------------------------------------------------------------------
__global__ void read_page_kernel(const SplitArgs a, uint32_t logical_page, uint8_t *dst) {
    const uint8_t *src = resolve_page(a, logical_page);
    const size_t n16 = a.page_bytes / 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        reinterpret_cast<uint4 *>(dst)[i] = reinterpret_cast<const uint4 *>(src)[i];
}

}  // namespace kvattn_dev

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
size_t kvattn_split_smem_bytes(int rt) {
    return rt == 1 ? (size_t)kvattn_dev::SplitCfg<1>::lds_bytes : (size_t)kvattn_dev::SplitCfg<2>::lds_bytes;
}

uint32_t kvattn_merge_max_splits() { return kvattn_dev::kMergeMaxSplits; }

hipError_t kvattn_split_setup() {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kvattn_dev::split_kernel<1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kvattn_split_smem_bytes(1));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kvattn_dev::split_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kvattn_split_smem_bytes(2));
    return e;
}

// rt: row tiles of 16 per workgroup (1 or 2); n_row_blocks blocks of 16 * rt rows.
// With events, the launch records them at the dispatch's own start and end
// (timing without extra stream packets).
hipError_t kvattn_launch_split(const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int rt, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();  // clear a stale error so the check below reports this launch
    dim3 grid(n_items, a.Hkv, n_row_blocks);
    dim3 block(64 * (rt == 1 ? kvattn_dev::SplitCfg<1>::waves : kvattn_dev::SplitCfg<2>::waves));
    const uint32_t smem = (uint32_t)kvattn_split_smem_bytes(rt);
    if (ev_start) {
        if (rt == 1)
            hipExtLaunchKernelGGL(kvattn_dev::split_kernel<1>, grid, block, smem, s, ev_start, ev_stop, 0, a);
        else
            hipExtLaunchKernelGGL(kvattn_dev::split_kernel<2>, grid, block, smem, s, ev_start, ev_stop, 0, a);
    } else if (rt == 1) {
        hipLaunchKernelGGL(kvattn_dev::split_kernel<1>, grid, block, smem, s, a);
    } else {
        hipLaunchKernelGGL(kvattn_dev::split_kernel<2>, grid, block, smem, s, a);
    }
    return hipGetLastError();
}

hipError_t kvattn_launch_wide(const SplitArgs &a, uint32_t n_splits, uint32_t n_row_blocks, hipStream_t s,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();
    dim3 grid(n_splits, a.Hkv, n_row_blocks), block(512);
    if (ev_start)
        hipExtLaunchKernelGGL(kvattn_dev::wide_kernel, grid, block, 0, s, ev_start, ev_stop, 0, a);
    else
        hipLaunchKernelGGL(kvattn_dev::wide_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

uint32_t kvattn_wide_rows() { return kvattn_dev::kWideRows; }

hipError_t kvattn_launch_writer(const WriterArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    const uint32_t tiles = (a.n_old + a.R - 1) / 32 - a.n_old / 32 + 1;
    hipLaunchKernelGGL(kvattn_dev::writer_kernel, dim3(tiles, a.Hkv), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_ring_copy(const RingCopyArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::ring_copy_kernel, dim3(a.count * kvattn_dev::kCopySlices), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_merge(const MergeArgs &a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();
    // few units (decode, verify): one per workgroup, the most parallel
    // latency; thousands (prefill chunks): four per workgroup
    if (a.units >= 1024 && a.n_splits <= kvattn_dev::kMergeWideSplits) {
        constexpr int U = kvattn_dev::kMergeWideUnits;
        dim3 grid((a.units + U - 1) / U), block(128 * U);
        if (ev_start)
            hipExtLaunchKernelGGL(kvattn_dev::merge_kernel<U>, grid, block, 0, s, ev_start, ev_stop, 0, a);
        else
            hipLaunchKernelGGL(kvattn_dev::merge_kernel<U>, grid, block, 0, s, a);
    } else {
        dim3 grid(a.units), block(128);
        if (ev_start)
            hipExtLaunchKernelGGL(kvattn_dev::merge_kernel<1>, grid, block, 0, s, ev_start, ev_stop, 0, a);
        else
            hipLaunchKernelGGL(kvattn_dev::merge_kernel<1>, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t kvattn_launch_read_page(const SplitArgs &a, uint32_t logical_page, uint8_t *dst, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::read_page_kernel, dim3(64), dim3(256), 0, s, a, logical_page, dst);
    return hipGetLastError();
}
