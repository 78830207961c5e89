// kernels_common.h -- device helpers shared by the gfx950 kernels for paged
// Q8_0-K / Q4_0-V attention (split_kernel.hip, wide_kernel.hip,
// writer_kernel.hip, copy_kernels.hip).
//
//   split_kernel  calls with up to 96 rows per KV head (decode, verify): one
//                 workgroup per (split of 32-key chunks, KV head, block of up
//                 to 32 rows); every wave streams its own chunks into an LDS
//                 ring with direct-to-LDS loads and computes all rows of the
//                 block.
//   wide_kernel   calls with more rows (prefill chunks, wide verify): one
//                 workgroup per (split, KV head, 256- or 384-row block); each
//                 chunk is turned into an f16 view of K and V once and shared
//                 by all rows of the block.
//   merge_small_kernel, merge_many_kernel
//                 log-sum-exp merge of the split partials in split order;
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
//   S^T = K . Q^T     A = K codes (int8 -> exact f16 by a byte permute, left
//                     biased by +1152, the bias removed by the
//                     accumulator's start value), one MFMA per 32-dim
//                     block, each block's fp32 dot scaled by its own binary16
//                     d_K before the blocks are summed;
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

// 8 int8 codes -> 8 f16 of c + 1152 (exact, byte i -> element i), without
// the bias subtraction: the split kernel starts each block's Q . K^T sum at
// -1152 * sum(q) instead, which removes it exactly up to fp32 rounding of
// that one term.
__device__ __forceinline__ half8 q8_biased_half8(uint32_t w0, uint32_t w1) {
    const uint32_t k64 = 0x64646464u;
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const uint4 r{__builtin_amdgcn_perm(k64, u0, 0x04010400u), __builtin_amdgcn_perm(k64, u0, 0x04030402u),
                  __builtin_amdgcn_perm(k64, u1, 0x04010400u), __builtin_amdgcn_perm(k64, u1, 0x04030402u)};
    return __builtin_bit_cast(half8, r);
}

// 8 Q4_0 codes in one dword -> 8 exact f16 (n - 8) in the order of
// q4_swizzle: (w & 0x000F000F) | 0x64006400 is the f16 pair 1024 + n of the
// low nibbles of bytes 0 and 2, the mask 0x00F000F0 gives 1024 + 16 n for
// their high nibbles (scaled back by a packed fma), and the same on w >> 8
// covers bytes 1 and 3: nine instructions where the byte-permute form takes
// eleven.
// (w & mask) | bits in one v_and_or_b32 (the compiler splits it in two when
// both constants are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(bits));
    return r;
}

__device__ __forceinline__ half8 q4_swz_half8(uint32_t w) {
    const uint32_t k64 = 0x64006400u, w8 = w >> 8;
    const half2v bias_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f}, bias_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const half2v a = bits_h2(and_or(w, 0x000F000Fu, k64)) - bias_lo;   // elements 0, 2
    const half2v b = bits_h2(and_or(w8, 0x000F000Fu, k64)) - bias_lo;  // 1, 3
    const half2v c = __builtin_elementwise_fma(bits_h2(and_or(w, 0x00F000F0u, k64)), sixteenth, bias_hi);   // 4, 6
    const half2v d = __builtin_elementwise_fma(bits_h2(and_or(w8, 0x00F000F0u, k64)), sixteenth, bias_hi);  // 5, 7
    return half8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}
// element e of q4_swz_half8 holds code q4_swizzle(e) of the dword (an
// involution: 0 2 1 3 4 6 5 7)
__host__ __device__ constexpr int q4_swizzle(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); }

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
__device__ __forceinline__ const uint8_t *page_base(const SplitArgs &a, const uint8_t *pool, const uint8_t *ring,
                                                   uint32_t e) {
    if (e < 0x80000000u) return pool + (size_t)e * a.page_bytes;
    uint32_t v = e & 0x3FFFFFFFu;
    if (e & 0x40000000u) v = (a.ring_base + v) % a.n_ring_slots;  // both < 2^30: no overflow
    return ring + (size_t)v * a.page_bytes;
}
__device__ __forceinline__ const uint8_t *page_base(const SplitArgs &a, uint32_t e) {
    return page_base(a, a.pool, a.ring, e);
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
// Entry of logical page `page` for range split whose first page is p0: one
// of the split's launch-carried entries (pre, already in registers; pre_ok:
// this workgroup's split has them) when it is one of its first kPrePages
// pages, else from the table.
static_assert(kPrePages == 4, "split_entry selects among four entries");
__device__ __forceinline__ uint32_t split_entry(const SplitArgs &a, bool pre_ok, uint4 pre, uint32_t p0, uint32_t page) {
    const uint32_t k = page - p0;
    if (pre_ok && k < kPrePages) return k == 0 ? pre.x : (k == 1 ? pre.y : (k == 2 ? pre.z : pre.w));
    return table_at(a.page_table, page);
}

// ---------------------------------------------------------------------------
// Element types (the header's KVATTN_TYPE_* values) and the staged chunk.
// One 32-key chunk of one KV head as staged in LDS keeps the page's byte
// order, section by section:
//   [0, kbytes)            K codes, two 16-key tiles; a 64-lane read of 16
//                          bytes per lane covers one 1024-byte quarter
//   [off_v, +vbytes)       V codes (one 32-key tile), in quarters
//   [off_ks, +256)         K scales, [key][block] binary16 (block K types)
//   [off_vs, +256)         the chunk's V-scale tile (block V types)
// Sizes: Q8_0 K / Q4_0 V 6656 bytes, Q8_0 / Q8_0 8704, Q4_0 / Q4_0 4608,
// F16 / F16 16384.  The chunk arrives by direct-to-LDS loads
// (global_load_lds_dwordx4: 16 bytes per lane, no registers), `dma` load
// instructions per chunk: one per code quarter plus one for both scale
// tiles (lanes 0..15 K, 16..31 V).
// ---------------------------------------------------------------------------
constexpr int kTypeF16 = 1, kTypeQ4_0 = 2, kTypeQ8_0 = 8;

template <int KT, int VT>
struct Chunk {
    static_assert((KT == kTypeQ8_0 && VT == kTypeQ4_0) || (KT == kTypeQ8_0 && VT == kTypeQ8_0) ||
                      (KT == kTypeQ4_0 && VT == kTypeQ4_0) || (KT == kTypeF16 && VT == kTypeF16),
                  "supported K/V element-type pairs");
    static constexpr int code_bytes(int t) { return t == kTypeQ8_0 ? 128 : t == kTypeQ4_0 ? 64 : 256; }
    static constexpr bool kblk = KT != kTypeF16, vblk = VT != kTypeF16;
    static constexpr int kc = code_bytes(KT), vc = code_bytes(VT);  // code bytes per key
    static constexpr int k_quarters = 32 * kc / 1024, v_quarters = 32 * vc / 1024;
    static constexpr int off_v = 32 * kc;
    static constexpr int off_ks = off_v + 32 * vc;
    static constexpr int off_vs = off_ks + (kblk ? 256 : 0);
    static constexpr int bytes = off_vs + (vblk ? 256 : 0);
    static constexpr int dma = k_quarters + v_quarters + (kblk ? 1 : 0);
    static constexpr int kw = kc / 8, vw = vc / 8;  // code dwords per lane and chunk
    static constexpr int pf_blocks = vblk ? 4 : 1;  // distinct P' operands per row tile
};


#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from g to LDS bytes [lds + 16 lane, +16).  m0 holds the
// wave's LDS destination; one wait state separates its write from the load.
// STREAM: non-temporal hint (nt) for data read once, which the split kernel
// streams (measured +6 % on the 40,960-key decode and +10 % on the
// 163,840-key single-row verify against the default policy); the wide kernel
// keeps the default, as its row blocks re-read each chunk through the caches.
template <bool STREAM>
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    // the destination is wave-uniform; readfirstlane keeps it in an SGPR even
    // where the compiler cannot prove that
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                     "s"(__builtin_amdgcn_readfirstlane(lds))
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// The compiler does not track the loads above, so the waits are explicit
// (and are compiler barriers for memory accesses).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait until at most `newer` (< S) chunks of D loads each, issued after the
// one needed, are in flight, for a ring of S stages.
template <int S, int D>
__device__ __forceinline__ void wait_chunk(uint32_t newer) {
    static_assert(S == 2 || S == 3, "rings of two or three stages");
    static_assert(2 * D <= 63, "vmcnt range");
    if (S == 3 && newer >= 2)
        wait_vmcnt<2 * D>();
    else if (newer >= 1)
        wait_vmcnt<D>();
    else
        wait_vmcnt<0>();
}

// Wide kernel: wait until at most n of the wave's loads are in flight (n is
// wave-uniform and small).
__device__ __forceinline__ void wait_vmcnt_upto(uint32_t n) {
    switch (n) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        default: wait_vmcnt<8>(); break;
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Direct-to-LDS load number d (0 <= d < Chunk::dma) of the chunk whose first
// key is jj0 in KV head kvh of the page at `base`, into the chunk buffer at
// LDS address dst.
template <int KT, int VT, bool STREAM>
__device__ __forceinline__ void issue_chunk_part(const SplitArgs &a, const uint8_t *base, uint32_t kvh, uint32_t jj0,
                                                 int lane, uint32_t dst, int d) {
    using C = Chunk<KT, VT>;
    const size_t kv = (size_t)kvh * a.T + jj0;  // first key of the chunk in the head's section
    if (d < C::k_quarters) {
        dma16<STREAM>(base + kv * C::kc + lane * 16 + 1024 * d, dst + 1024 * d);
    } else if (d < C::k_quarters + C::v_quarters) {
        const int q = d - C::k_quarters;
        dma16<STREAM>(base + a.sec_vc + kv * C::vc + lane * 16 + 1024 * q, dst + C::off_v + 1024 * q);
    } else if (lane < 32) {
        const uint8_t *sp = lane < 16 ? base + a.sec_kd + kv * 8 + lane * 16
                                      : base + a.sec_vd + (size_t)kvh * a.T * 8 + (size_t)(jj0 >> 5) * 256 + (lane - 16) * 16;
        dma16<STREAM>(sp, dst + C::off_ks);
    }
}

template <int KT, int VT, bool STREAM>
__device__ __forceinline__ void issue_chunk(const SplitArgs &a, const uint8_t *base, uint32_t kvh, uint32_t jj0,
                                            int lane, uint32_t dst) {
#pragma unroll
    for (int d = 0; d < Chunk<KT, VT>::dma; d++) issue_chunk_part<KT, VT, STREAM>(a, base, kvh, jj0, lane, dst, d);
}

__device__ __forceinline__ void put4(uint32_t *d, const uint4 &x) {
    d[0] = x.x;
    d[1] = x.y;
    d[2] = x.z;
    d[3] = x.w;
}

// K codes of the lane, quarter by quarter: kq[4q .. 4q + 3] = its 16 bytes of
// quarter q.  Q8_0: quarter q = key tile q / 2, blocks 2 (q mod 2) and +1
// (8 codes each); Q4_0: quarter = key tile, one dword per block; F16:
// quarter q = key tile q / 4, block q mod 4, eight binary16.
template <int KT, int VT>
__device__ __forceinline__ void read_kcodes(const uint8_t *stg, int lane, uint32_t (&kq)[Chunk<KT, VT>::kw]) {
#pragma unroll
    for (int q = 0; q < Chunk<KT, VT>::k_quarters; q++)
        put4(kq + 4 * q, *reinterpret_cast<const uint4 *>(stg + 1024 * q + 16 * lane));
}

// The lane's K operand (8 f16: key 16 tt + c16, dims 32 b + 8 g .. +8) of
// key tile tt and block b: Q8_0 c + 1152 (the bias leaves through the
// accumulator start, RowState::kcorr), Q4_0 n - 8 in q4_swizzle order of the
// dims (the query fragment follows it), F16 the value.
template <int KT>
__device__ __forceinline__ half8 k_frag(const uint32_t *kq, int tt, int b) {
    if constexpr (KT == kTypeQ8_0) {
        const uint32_t *w = kq + 8 * tt + 4 * (b >> 1) + 2 * (b & 1);
        return q8_biased_half8(w[0], w[1]);
    } else if constexpr (KT == kTypeQ4_0) {
        return q4_swz_half8(kq[4 * tt + b]);
    } else {
        const uint32_t *w = kq + 16 * tt + 4 * b;
        return __builtin_bit_cast(half8, uint4{w[0], w[1], w[2], w[3]});
    }
}

// K scales as the lane uses them: kd[8tt + ...] binary16 pairs, key 4g + v
// of tile tt, block b at half 4v + b.
template <int KT, int VT>
__device__ __forceinline__ void read_kscales(const uint8_t *stg, int grp, uint32_t kd[16]) {
    const uint4 *k4 = reinterpret_cast<const uint4 *>(stg + Chunk<KT, VT>::off_ks);  // key j at bytes 8j
    put4(kd + 0, k4[2 * grp]);
    put4(kd + 4, k4[2 * grp + 1]);
    put4(kd + 8, k4[8 + 2 * grp]);
    put4(kd + 12, k4[8 + 2 * grp + 1]);
}

// V scales: vd[4b + ...] binary16 pairs of block b, operand slots 2i, 2i + 1.
template <int KT, int VT>
__device__ __forceinline__ void read_vscales(const uint8_t *stg, int grp, uint32_t vd[16]) {
    const uint4 *v4 = reinterpret_cast<const uint4 *>(stg + Chunk<KT, VT>::off_vs);
#pragma unroll
    for (int b = 0; b < 4; b++) put4(vd + 4 * b, v4[b * 4 + grp]);
}

// V codes of the lane, quarter by quarter.  Q4_0: one dword per 16-dim tile;
// Q8_0: two dwords per tile; F16: four (eight binary16).
template <int KT, int VT>
__device__ __forceinline__ void read_vcodes(const uint8_t *stg, int lane, uint32_t (&vq)[Chunk<KT, VT>::vw]) {
#pragma unroll
    for (int q = 0; q < Chunk<KT, VT>::v_quarters; q++)
        put4(vq + 4 * q, *reinterpret_cast<const uint4 *>(stg + Chunk<KT, VT>::off_v + 1024 * q + 16 * lane));
}

// The lane's V^T operand of 16-dim tile n (8 f16 over the lane's key slots),
// exact: Q4_0 n - 8 (slots in q4_swizzle order; the P' operand follows it),
// Q8_0 c, F16 the value.
template <int VT>
__device__ __forceinline__ half8 v_frag(const uint32_t *vq, int n) {
    if constexpr (VT == kTypeQ4_0) {
        return q4_swz_half8(vq[n]);
    } else if constexpr (VT == kTypeQ8_0) {
        return q8_to_half8(vq[2 * n], vq[2 * n + 1]);
    } else {
        return __builtin_bit_cast(half8, uint4{vq[4 * n], vq[4 * n + 1], vq[4 * n + 2], vq[4 * n + 3]});
    }
}

// F16 values carry no scale to clear: keys at or past the history length
// (page padding, possibly NaN) get value 0 in the lane's operands instead.
// Operand slot i of group g is key 16 (i / 4) + 4 g + i mod 4; a dword holds
// slots 2i, 2i + 1.
template <int KT, int VT>
__device__ __forceinline__ void clear_padding_vcodes(uint32_t *vq, int grp, uint32_t n_valid) {
#pragma unroll
    for (int w = 0; w < 4; w++) {
        const uint32_t key0 = 16 * (w >> 1) + 4 * grp + 2 * (w & 1);
        const uint32_t keep = (key0 < n_valid ? 0x0000FFFFu : 0u) | (key0 + 1 < n_valid ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int n = 0; n < 8; n++) vq[4 * n + w] &= keep;
    }
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
    floatx4 kcorr[4];  // Q8_0 keys: start of block b's sum, -1152 * (sum of the row's qf over it)
    int row_pos;     // position of the lane's row; -1 = padding row
    float m_ref;     // softmax reference (log2 units), uniform per row
    float l_run;     // lane's share of the softmax denominator
    floatx4 acc[8];  // O^T tile n: dims 16n + 4g + v of the lane's row
};

// The softmax reference a tile's scores are taken relative to: the row's
// lazy reference, or 0 before the first key.
__device__ __forceinline__ float score_ref(const RowState &st) { return st.m_ref == kNegInf ? 0.f : st.m_ref; }

// Q8_0 keys enter the matrix cores biased (c + 1152, no subtraction); the
// start values cost 16 registers per row tile (measured +1 to +4 % on the
// two-tile verify widths, +1.3 % with one tile, against the subtraction).

// Scores of one chunk for NT row tiles, relative to the tile's reference:
// s[t][4tt + v] = score(key 16tt + 4g + v of the chunk) - score_ref(tile t),
// log2-scaled.  Each K fragment is converted once and feeds one MFMA per tile
// and 32-dim block; block types scale each block's fp32 dot by its own
// binary16 d_K, F16 keys accumulate the four blocks in the MFMA.  The
// reference enters as the start of the sum, so the softmax needs no
// subtraction.
template <int NT, int KT>
__device__ __forceinline__ void chunk_scores(const RowState (&st)[NT], const uint32_t *kq, const uint32_t kd[16],
                                             float (&s)[NT][8]) {
    float ref[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) ref[t] = score_ref(st[t]);
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        if constexpr (KT == kTypeF16) {
            floatx4 d[NT];
#pragma unroll
            for (int t = 0; t < NT; t++) d[t] = floatx4{-ref[t], -ref[t], -ref[t], -ref[t]};
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const half8 kf = k_frag<KT>(kq, tt, b);
#pragma unroll
                for (int t = 0; t < NT; t++) d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, st[t].qf[b], d[t], 0, 0, 0);
            }
#pragma unroll
            for (int t = 0; t < NT; t++)
#pragma unroll
                for (int v = 0; v < 4; v++) s[t][4 * tt + v] = d[t][v];
        } else {
            // all MFMAs of the key tile first, so none waits on the one before
            floatx4 d[4][NT];
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const half8 kf = k_frag<KT>(kq, tt, b);
#pragma unroll
                for (int t = 0; t < NT; t++) {
                    const floatx4 c0 = KT == kTypeQ8_0 ? st[t].kcorr[b] : floatx4{0.f, 0.f, 0.f, 0.f};
                    d[b][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, st[t].qf[b], c0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++)
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    // fma with the binary16 operand read in place (v_fma_mix_f32)
                    float acc = __builtin_fmaf(half_of(kd + 8 * tt, 4 * v), d[0][t][v], -ref[t]);
#pragma unroll
                    for (int b = 1; b < 4; b++) acc = __builtin_fmaf(half_of(kd + 8 * tt, 4 * v + b), d[b][t][v], acc);
                    s[t][4 * tt + v] = acc;
                }
        }
    }
}

// Lazy reference update of one row tile from its relative scores s (mask:
// -inf): when some score exceeds the reference by more than kRescale (or
// before the first key) the reference moves to the row maximum, the
// accumulators and the denominator are rescaled, and s is shifted to the new
// reference.
// counter (test aid, normally null): one is added per event in which a row
// tile that already had a reference moves it, so a test can show that its
// inputs reach this branch.
__device__ __forceinline__ void update_reference(RowState &st, float (&s)[8], uint32_t *counter) {
    float m = s[0];
#pragma unroll
    for (int i = 1; i < 8; i++) m = fmaxf(m, s[i]);
    const float thr = st.m_ref == kNegInf ? kNegInf : kRescale;
    if (__any(m > thr)) {
        if (counter && __any(st.m_ref != kNegInf) && (threadIdx.x & 63) == 0) atomicAdd(counter, 1u);
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float ref = score_ref(st);
        const float m_new = fmaxf(st.m_ref, ref + m);
        const float alpha = (st.m_ref == kNegInf) ? 0.f : fast_exp2(st.m_ref - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int n = 0; n < 8; n++) st.acc[n] *= alpha;
        st.m_ref = m_new;
        // a row with no visible key yet keeps -inf scores (no shift by inf)
        const float shift = m_new == kNegInf ? 0.f : ref - m_new;
#pragma unroll
        for (int i = 0; i < 8; i++) s[i] += shift;
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
template <int KT, int VT>
__device__ __forceinline__ void sanitize_vscales(uint8_t *stg, int lane, uint32_t n_valid) {
    uint32_t *w = reinterpret_cast<uint32_t *>(stg + Chunk<KT, VT>::off_vs) + lane;
    const uint32_t key0 = 16 * ((lane & 3) >> 1) + 4 * ((lane >> 2) & 3) + 2 * (lane & 1);
    uint32_t v = *w;
    if (key0 >= n_valid) v &= 0xFFFF0000u;
    if (key0 + 1 >= n_valid) v &= 0x0000FFFFu;
    *w = v;
}

// binary16 of p * (half H of the binary16 pair s), written into the low
// (mix_lo) or high (mix_hi) half of a dword: one v_fma_mix per element.
template <int H>
__device__ __forceinline__ uint32_t mix_lo(float p, uint32_t s) {
    uint32_t r;
    if constexpr (H)
        asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(s));
    else
        asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(s));
    return r;
}
template <int H>
__device__ __forceinline__ uint32_t mix_hi(uint32_t r, float p, uint32_t s) {
    if constexpr (H)
        asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p), "v"(s));
    else
        asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "+v"(r) : "v"(p), "v"(s));
    return r;
}

// Dword k of the P' operand of one value block: slots 2k, 2k + 1 of the
// operand (key slots in q4_swizzle order for Q4_0 values), P * d_V each.
template <int VT, int K>
__device__ __forceinline__ uint32_t pv_pair(const float (&p)[8], const uint32_t *vdb) {
    constexpr int i0 = VT == kTypeQ4_0 ? q4_swizzle(2 * K) : 2 * K;
    constexpr int i1 = VT == kTypeQ4_0 ? q4_swizzle(2 * K + 1) : 2 * K + 1;
    return mix_hi<i1 & 1>(mix_lo<i0 & 1>(p[i0], vdb[i0 >> 1]), p[i1], vdb[i1 >> 1]);
}

// Softmax step of one chunk for one row tile from its relative scores: lazy
// reference update, probabilities P = 2^s, the denominator, and the P'
// operands: P * d_V per value block for block V types, P itself for F16
// values.
template <int VT>
__device__ __forceinline__ void chunk_probs(RowState &st, float (&s)[8], const uint32_t vd[16],
                                            half8 (&pf)[VT == kTypeF16 ? 1 : 4], uint32_t *counter) {
    update_reference(st, s, counter);
    float p[8];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        p[i] = fast_exp2(s[i]);
        lsum += p[i];
    }
    st.l_run += lsum;
    if constexpr (VT == kTypeF16) {
        pf[0] = half8{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                      (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
    } else {
#pragma unroll
        for (int b = 0; b < 4; b++) {
            uint4 w;
            w.x = pv_pair<VT, 0>(p, vd + 4 * b);
            w.y = pv_pair<VT, 1>(p, vd + 4 * b);
            w.z = pv_pair<VT, 2>(p, vd + 4 * b);
            w.w = pv_pair<VT, 3>(p, vd + 4 * b);
            pf[b] = __builtin_bit_cast(half8, w);
        }
    }
}

// O^T += V^T P'^T for one chunk and NT row tiles: dim tile n = 2b + nn of
// value block b; each V fragment is converted once.
template <int NT, int VT>
__device__ __forceinline__ void chunk_pv(RowState (&st)[NT], const uint32_t *vq,
                                         const half8 (&pf)[NT][VT == kTypeF16 ? 1 : 4]) {
#pragma unroll
    for (int n = 0; n < 8; n++) {
        const half8 vf = v_frag<VT>(vq, n);
#pragma unroll
        for (int t = 0; t < NT; t++)
            st[t].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[t][VT == kTypeF16 ? 0 : (n >> 1)], st[t].acc[n],
                                                                  0, 0, 0);
    }
}

// Log-sum-exp combination of a stored partial (m0, l0, a0) with a new one
// (m1, l1, a1), in log2 units; a side with l = 0 (no visible key) drops out.
struct PartCombine {
    float w0, w1, m, l;
};
__device__ __forceinline__ PartCombine part_combine(float m0, float l0, float m1, float l1) {
    PartCombine c;
    const bool e0 = !(l0 > 0.f), e1 = !(l1 > 0.f);
    c.m = e0 ? m1 : (e1 ? m0 : fmaxf(m0, m1));
    c.w0 = e0 ? 0.f : fast_exp2(m0 - c.m);
    c.w1 = e1 ? 0.f : fast_exp2(m1 - c.m);
    c.l = c.w0 * l0 + c.w1 * l1;
    return c;
}

}  // namespace kvattn_dev
