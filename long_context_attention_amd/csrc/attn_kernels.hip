// attn_kernels.hip -- gfx950 kernels for paged Q8_0-K / Q4_0-V attention.
//
// Two kernels:
//   kvattn_split_kernel   one workgroup per (split of logical pages, KV head,
//                         32-row block).  Dequantises Q8_0 / Q4_0 codes in
//                         registers from 16-byte loads, runs Q.K^T and P.V on
//                         the matrix cores (v_mfma_f32_16x16x32_f16), keeps an
//                         online softmax per query row, and writes one
//                         un-normalised partial (m, l, acc[128]) per split and
//                         row ("troed's fork of Raymond's adaptive KV
//                         streaming", section "Keep the stock attention
//                         order": per-span partials, then one final reduction;
//                         "Block KV cache streaming ...", maintainer review:
//                         kernels with a partial-output mode followed by a
//                         combine).
//   kvattn_merge_kernel   log-sum-exp merge of the split partials in logical
//                         split order; splits with l = 0 are skipped (the zero
//                         guard the review finds missing in the chunk
//                         normaliser).
//
// Arithmetic (per KV head, 16 keys x 16 query rows per matrix-core tile):
//   S^T = K . Q^T    A = K codes (int8 -> f16, exact), one MFMA per 32-dim
//                    block, so each block's fp32 dot is scaled by its own
//                    binary16 d_K before the blocks are summed.
//                    B = Q * softmax_scale * log2(e), rounded to f16.
//   O^T += V^T . P'^T  A = V codes (n - 8 -> f16, exact), B = P * d_V per
//                    (row, key, 32-dim block), rounded to f16 once.
//   Softmax in fp32 with exp2; row max / sum reduced across the four
//   16-lane groups of a wavefront.
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
// ---------------------------------------------------------------------------
__device__ __forceinline__ const uint8_t *resolve_page(const SplitArgs &a, uint32_t logical_page) {
    uint32_t e = a.page_table[logical_page];
    if (e < 0x80000000u) return a.pool + (size_t)e * a.page_bytes;
    uint32_t v = e & 0x3FFFFFFFu;
    if (e & 0x40000000u) v = (a.ring_base + v) % a.n_ring_slots;  // both < 2^30: no overflow
    return a.ring + (size_t)v * a.page_bytes;
}

// ---------------------------------------------------------------------------
// One 32-key chunk of one KV head.
// In flight (registers): the lane's code bytes and 8 bytes of scales.
//   kq[16]  K codes of 16-key tile tt (dwords 8tt .. 8tt+7): blocks 2k, 2k+1
//           of load k, 8 codes each
//   vq[8]   V codes, one dword per 16-dim tile
//   sc      lanes 0-31: K scales of the chunk's 32 keys ([key][block], 256
//           bytes); lanes 32-63: the chunk's V-scale tile (256 bytes)
// The scales are shared by the 16 lanes of a group, so they go through a
// 512-byte LDS slot per wave instead of being loaded 16 times.
// ---------------------------------------------------------------------------
struct ChunkG {
    uint32_t kq[16];
    uint32_t vq[8];
    uint2 sc;
};

// Scales of one chunk as the lane uses them.
//   kd[16]  [tt][8]: binary16 pairs, key 4g + v of tile tt, block b at half 4v + b
//   vd[16]  [b][4]: binary16 pairs of block b, operand slots 2i, 2i + 1
struct ChunkS {
    uint32_t kd[16];
    uint32_t vd[16];
};

__device__ __forceinline__ void put4(uint32_t *d, const uint4 &x) {
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
}

__device__ __forceinline__ void load_chunk(const SplitArgs &a, uint32_t kvh, uint32_t chunk, int lane, ChunkG &r) {
    const uint32_t cpp = a.T >> 5;  // chunks per page
    const uint32_t page = chunk / cpp;
    const uint32_t jj0 = (chunk - page * cpp) << 5;
    const uint8_t *base = resolve_page(a, page);
    const size_t T = a.T;
    const uint4 *kcp = reinterpret_cast<const uint4 *>(base + (size_t)kvh * T * 128 + (size_t)(jj0 >> 4) * 2048) + lane;
    const uint4 *vcp = reinterpret_cast<const uint4 *>(base + a.sec_vc + (size_t)kvh * T * 64 + (size_t)(jj0 >> 5) * 2048) + lane;
    const uint8_t *scp = lane < 32 ? base + a.sec_kd + ((size_t)kvh * T + jj0) * 8 + lane * 8
                                   : base + a.sec_vd + (size_t)kvh * T * 8 + (size_t)(jj0 >> 5) * 256 + (lane - 32) * 8;
    put4(r.kq + 0, kcp[0]);
    put4(r.kq + 4, kcp[64]);
    put4(r.kq + 8, kcp[128]);
    put4(r.kq + 12, kcp[192]);
    put4(r.vq + 0, vcp[0]);
    put4(r.vq + 4, vcp[64]);
    r.sc = *reinterpret_cast<const uint2 *>(scp);
}

// Stage the chunk's scales through the wave's LDS slot (64 x uint2) and read
// back the lane's K scales; the V scales are read when the P' operands are
// formed (read_vscales), so they do not occupy registers during Q.K^T.
__device__ __forceinline__ void stage_scales(uint2 *slot, const ChunkG &g, int lane, int grp, ChunkS &s) {
    slot[lane] = g.sc;
    const uint4 *k4 = reinterpret_cast<const uint4 *>(slot);  // K scales: key j at bytes 8j
    put4(s.kd + 0, k4[2 * grp]);                              // keys 4g .. 4g+3
    put4(s.kd + 4, k4[2 * grp + 1]);
    put4(s.kd + 8, k4[8 + 2 * grp]);                          // keys 16 + 4g ..
    put4(s.kd + 12, k4[8 + 2 * grp + 1]);
}

__device__ __forceinline__ void read_vscales(const uint2 *slot, int grp, ChunkS &s) {
    const uint4 *v4 = reinterpret_cast<const uint4 *>(slot + 32);  // V tile
#pragma unroll
    for (int b = 0; b < 4; b++) put4(s.vd + 4 * b, v4[b * 4 + grp]);
}

// binary16 half `i` of a packed array (lo half = even index)
__device__ __forceinline__ float half_of(const uint32_t *w, int i) { return (i & 1) ? h2f_hi(w[i >> 1]) : h2f_lo(w[i >> 1]); }

// Softmax reference of a row moves only when a score exceeds it by more than
// kRescale (log2 units), so P = exp2(s - ref) <= 2^kRescale stays exact
// enough in binary16 and the accumulators are rarely rescaled.  Any
// reference gives the same result in exact arithmetic; the partial carries
// the reference it used.
constexpr float kRescale = 8.0f;

// Per-wave state: one tile of 16 query rows (the lane's row is c16).
struct RowState {
    half8 qf[4];     // B operand of S^T = K Q^T, block b
    int row_pos;     // position of the lane's row; -1 = padding row
    float m_ref;     // softmax reference (log2 units), uniform per row
    float l_run;     // lane's share of the softmax denominator
    floatx4 acc[8];  // O^T tile n: dims 16n + 4g + v of the lane's row
};

// Scores of one chunk: s[4tt + v] is key 16tt + 4g + v of the chunk,
// log2-scaled.  One MFMA per 32-dim block, scaled by that block's d_K.
template <bool MASK>
__device__ __forceinline__ void chunk_scores(const RowState &st, const ChunkG &r, const ChunkS &sc, uint32_t kpos0,
                                             int grp, float s[8]) {
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const uint32_t *w = r.kq + 8 * tt + 4 * (b >> 1) + 2 * (b & 1);
            const half8 kf = q8_to_half8(w[0], w[1]);
            const floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, st.qf[b], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                // fma with the binary16 operand read in place (v_fma_mix_f32)
                const float dk = half_of(sc.kd + 8 * tt, 4 * v + b);
                s[4 * tt + v] = __builtin_fmaf(dk, d[v], b == 0 ? 0.0f : s[4 * tt + v]);
            }
        }
    }
    if (MASK) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int key = (int)(kpos0 + 16 * (i >> 2) + 4 * grp + (i & 3));
            if (key > st.row_pos) s[i] = kNegInf;
        }
    }
}

// Softmax step of one chunk: lazy reference update (rescaling the
// accumulators, which already hold every earlier chunk), probabilities, the
// denominator, and the P' operands P * d_V of the four value blocks.
template <bool MASK>
__device__ __forceinline__ void chunk_probs(RowState &st, const float s[8], const uint2 *slot, int grp, half8 pf[4]) {
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
    ChunkS sc;
    read_vscales(slot, grp, sc);
#pragma unroll
    for (int b = 0; b < 4; b++) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float pd = __builtin_fmaf(p[i], half_of(sc.vd + 4 * b, i), 0.0f);
            // masked keys have p = 0 but may sit on garbage (NaN) scales
            e[i] = MASK ? ((p[i] == 0.f) ? 0.f : pd) : pd;
        }
        pf[b] = half8{(_Float16)e[0], (_Float16)e[1], (_Float16)e[2], (_Float16)e[3],
                      (_Float16)e[4], (_Float16)e[5], (_Float16)e[6], (_Float16)e[7]};
    }
}

// O^T += V^T P'^T for one chunk: dim tile n = 2b + nn of value block b.
__device__ __forceinline__ void chunk_pv(RowState &st, const uint32_t vq[8], const half8 pf[4]) {
#pragma unroll
    for (int n = 0; n < 8; n++) {
        const half8 vf = q4_to_half8(vq[n]);
        st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[n >> 1], st.acc[n], 0, 0, 0);
    }
}

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
// order.  The bits depend only on the partials, never on the block size, so
// the fused merge and the merge kernel agree exactly.
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

// ---------------------------------------------------------------------------
// Split kernel.  A workgroup of 8 waves handles one split (a range of 32-key
// chunks) of one KV head for RT tiles of 16 query rows; 8 / RT waves share a
// row tile and take its chunks round robin.  Rows of a KV head are ordered
// (w, hh): r = w * G + hh, hh < G.
// Each wave keeps the next chunk's loads in flight and overlaps chunk i's
// Q.K^T with chunk i-1's P.V, whose operands it carries over.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;
// dynamic LDS of the split kernel: per wave 16 m, 16 l and 16 x 132 acc
constexpr int kSplitLdsFloats = kSplitWaves * 16 * (2 + 132);

template <int RT>
__global__ __launch_bounds__(64 * kSplitWaves, 1) void split_kernel(const SplitArgs a) {
    constexpr int RTW = kSplitWaves / RT;  // waves per row tile
    extern __shared__ float smem[];        // [waves][16] m, [waves][16] l, [waves][16][132] acc
    __shared__ uint2 sc_slot[kSplitWaves][64];

    const int lane = threadIdx.x & 63;
    // wave index, made visibly uniform so chunk bookkeeping stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rt = wave / RTW, cw = wave - rt * RTW;
    const int grp = lane >> 4;  // 16-lane group
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.y;
    const uint32_t row0 = blockIdx.z * (16 * RT) + 16 * rt;  // first row of this wave's tile
    const uint32_t rows_kv = a.W * a.G;
    const uint32_t n_chunks_all = (a.n_tokens + 31) >> 5;

    // ---- split -> chunk range
    uint32_t split, c_begin, c_end;
    if (a.page_list) {
        split = a.page_list[a.list_offset + blockIdx.x];
        c_begin = split * (a.T >> 5);
        c_end = min(c_begin + (a.T >> 5), n_chunks_all);
    } else {
        split = blockIdx.x;
        c_begin = blockIdx.x * a.split_chunks;
        c_end = min(c_begin + a.split_chunks, n_chunks_all);
    }
    // chunks whose keys every row sees (keys <= n_tokens - W) need no mask
    const uint32_t clean_end = (a.n_tokens - a.W + 1) >> 5;

    // ---- row state and raw query loads (issued first: their latency then
    // overlaps the chunk loads issued next)
    RowState st;
    float4 qraw[8];
    st.row_pos = -1;
    st.m_ref = kNegInf;
    st.l_run = 0.f;
#pragma unroll
    for (int n = 0; n < 8; n++) st.acc[n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; i++) qraw[i] = float4{0.f, 0.f, 0.f, 0.f};
    {
        const uint32_t r = row0 + c16;
        if (r < rows_kv) {
            const uint32_t w = r / a.G, hh = r - w * a.G;
            const uint32_t h = kvh * a.G + hh;
            st.row_pos = (int)(a.n_tokens - a.W + w);
            const float4 *qp = reinterpret_cast<const float4 *>(a.q + ((size_t)w * a.Hq + h) * 128 + 8 * grp);
#pragma unroll
            for (int b = 0; b < 4; b++) {
                qraw[2 * b] = qp[8 * b];
                qraw[2 * b + 1] = qp[8 * b + 1];
            }
        }
    }

    uint2 *slot = sc_slot[wave];
    uint32_t c = c_begin + cw;
    // this wave's last chunk; the prefetch past it reloads that chunk (an L2
    // hit) so every iteration issues the same loads and the wait for the
    // current chunk never covers the next one
    const uint32_t c_last = c < c_end ? c + ((c_end - 1 - c) / RTW) * RTW : c;
    ChunkG ga, gb;
    if (c < c_end) load_chunk(a, kvh, c, lane, ga);

    // ---- query fragments: lane (row c16, group g) holds dims 32b + 8g .. +8
    // of block b, pre-scaled by softmax_scale * log2(e)
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const float4 x = qraw[2 * b], y = qraw[2 * b + 1];
        st.qf[b] = half8{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale), (_Float16)(x.z * a.qscale),
                         (_Float16)(x.w * a.qscale), (_Float16)(y.x * a.qscale), (_Float16)(y.y * a.qscale),
                         (_Float16)(y.z * a.qscale), (_Float16)(y.w * a.qscale)};
    }

    if (c < c_end) {
        ChunkS cs;
        float s[8];
        uint32_t pv_vq[8];
        half8 pv_pf[4];
        // first chunk: scores and probabilities only
        load_chunk(a, kvh, min(c + RTW, c_last), lane, gb);
        stage_scales(slot, ga, lane, grp, cs);
        if (c < clean_end) {
            chunk_scores<false>(st, ga, cs, 32 * c, grp, s);
            chunk_probs<false>(st, s, slot, grp, pv_pf);
        } else {
            chunk_scores<true>(st, ga, cs, 32 * c, grp, s);
            chunk_probs<true>(st, s, slot, grp, pv_pf);
        }
#pragma unroll
        for (int i = 0; i < 8; i++) pv_vq[i] = ga.vq[i];
        c += RTW;
        // steady state: scores of chunk c, values of the chunk before it
#define KVATTN_STEP(CUR, NXT)                                                   \
    if (c >= c_end) break;                                                      \
    load_chunk(a, kvh, min(c + RTW, c_last), lane, NXT);                        \
    stage_scales(slot, CUR, lane, grp, cs);                                     \
    if (c < clean_end) {                                                        \
        chunk_scores<false>(st, CUR, cs, 32 * c, grp, s);                       \
        chunk_pv(st, pv_vq, pv_pf);                                             \
        chunk_probs<false>(st, s, slot, grp, pv_pf);                                   \
    } else {                                                                    \
        chunk_scores<true>(st, CUR, cs, 32 * c, grp, s);                        \
        chunk_pv(st, pv_vq, pv_pf);                                             \
        chunk_probs<true>(st, s, slot, grp, pv_pf);                                    \
    }                                                                           \
    for (int i = 0; i < 8; i++) pv_vq[i] = CUR.vq[i];                           \
    c += RTW;
        while (true) {
            KVATTN_STEP(gb, ga)
            KVATTN_STEP(ga, gb)
        }
#undef KVATTN_STEP
        chunk_pv(st, pv_vq, pv_pf);
    }

    // ---- combine the waves of each row tile (fixed wave order), write partials
    constexpr int OS = 132;  // padded row stride
    float *sm_m = smem;
    float *sm_l = smem + kSplitWaves * 16;
    float *sm_o = smem + 2 * kSplitWaves * 16;
    {
        float l = st.l_run;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (grp == 0) {
            sm_m[wave * 16 + c16] = st.m_ref;
            sm_l[wave * 16 + c16] = l;
        }
#pragma unroll
        for (int n = 0; n < 8; n++)
            *reinterpret_cast<floatx4 *>(&sm_o[(wave * 16 + c16) * OS + 16 * n + 4 * grp]) = st.acc[n];
    }
    __syncthreads();

    const uint32_t units = a.W * a.Hq;
    const uint32_t block_row0 = blockIdx.z * (16 * RT);
    const uint32_t rows_here = min((uint32_t)(16 * RT), rows_kv - block_row0);
    for (uint32_t idx = threadIdx.x; idx < rows_here * 128; idx += blockDim.x) {
        const uint32_t r = idx >> 7, t = idx & 127;
        const uint32_t w0 = (r >> 4) * RTW, rr = r & 15;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < RTW; w++) M = fmaxf(M, sm_m[(w0 + w) * 16 + rr]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < RTW; w++) {
                const float mw = sm_m[(w0 + w) * 16 + rr];
                if (mw == kNegInf) continue;
                const float f = fast_exp2(mw - M);
                L += f * sm_l[(w0 + w) * 16 + rr];
                A += f * sm_o[((w0 + w) * 16 + rr) * OS + t];
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

    // ---- fused merge: the last workgroup of this (KV head, row block) folds
    // every split of its rows, in split order, into the output
    if (a.counters) {
        // One thread fences for the whole workgroup: every wave waits for its
        // partial stores to complete, the barrier orders them before that
        // thread's device-scope release (an L2 write-back on this chip), and
        // its acquire (an L2 invalidate) before the merge's loads.  Eight waves each fencing would flush and
        // invalidate the XCD's L2 eight times per workgroup.
        __shared__ uint32_t sm_last;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have reached L2
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t *cnt = a.counters + (size_t)kvh * gridDim.z + blockIdx.z;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = (old == a.n_splits - 1);
            if (last) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                *cnt = 0;  // ready for the next call on the stream
            }
            sm_last = last;
        }
        __syncthreads();
        if (!sm_last) return;
        __shared__ float2 sm_row_ml[16 * RT];
        const uint32_t G = a.G, Hq = a.Hq;
        merge_rows(
            a.part_ml, a.part_o, a.out, a.n_splits, units, rows_here,
            [=](uint32_t r) {
                const uint32_t rk = block_row0 + r;
                const uint32_t wq = rk / G, hh = rk - wq * G;
                return wq * Hq + kvh * G + hh;
            },
            reinterpret_cast<float2 *>(smem), sm_row_ml);
    }
}

// ---------------------------------------------------------------------------
// Merge kernel (layers with streamed pages, whose splits come from several
// launches): one 128-thread workgroup per (row, query head) unit, thread t
// folds dimension t with the same arithmetic as the fused merge.
// ---------------------------------------------------------------------------
constexpr int kMergeMaxSplits = 4096;

__global__ __launch_bounds__(128) void merge_kernel(const MergeArgs a) {
    __shared__ float2 wl[kMergeMaxSplits];
    __shared__ float2 row_ml[1];
    const uint32_t unit = blockIdx.x;
    merge_rows(a.part_ml, a.part_o, a.out, a.n_splits, a.units, 1, [=](uint32_t) { return unit; }, wl, row_ml);
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
    (void)rt;
    return (size_t)kvattn_dev::kSplitLdsFloats * sizeof(float);
}

uint32_t kvattn_merge_max_splits() { return kvattn_dev::kMergeMaxSplits; }
uint32_t kvattn_fused_merge_max_entries() { return kvattn_dev::kSplitLdsFloats / 2; }

hipError_t kvattn_split_setup() {
    const int bytes = (int)kvattn_split_smem_bytes(1);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kvattn_dev::split_kernel<1>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(&kvattn_dev::split_kernel<2>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// rt: row tiles of 16 per workgroup (1 or 2); n_row_blocks blocks of 16 * rt rows.
// With events, the launch records them at the dispatch's own start and end
// (timing without extra stream packets).
hipError_t kvattn_launch_split(const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int rt, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();  // clear a stale error so the check below reports this launch
    dim3 grid(n_items, a.Hkv, n_row_blocks), block(64 * kvattn_dev::kSplitWaves);
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

hipError_t kvattn_launch_ring_copy(const RingCopyArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::ring_copy_kernel, dim3(a.count * kvattn_dev::kCopySlices), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_merge(const MergeArgs &a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();
    dim3 grid(a.units), block(128);
    if (ev_start)
        hipExtLaunchKernelGGL(kvattn_dev::merge_kernel, grid, block, 0, s, ev_start, ev_stop, 0, a);
    else
        hipLaunchKernelGGL(kvattn_dev::merge_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_read_page(const SplitArgs &a, uint32_t logical_page, uint8_t *dst, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::read_page_kernel, dim3(64), dim3(256), 0, s, a, logical_page, dst);
    return hipGetLastError();
}
