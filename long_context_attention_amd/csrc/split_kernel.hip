// split_kernel.hip -- the split-KV kernel (decode, verify: up to 32 rows per
// KV head in a workgroup, calls of up to 96 rows as two or three row blocks)
// and the log-sum-exp merge of the split partials.
#include <type_traits>

#include "kernels_common.h"

namespace kvattn_dev {

// ---------------------------------------------------------------------------
// Split kernel.  A workgroup (12, 8 or 4 waves, SplitCfg) handles one split
// (a range of 32-key chunks) of one KV head for a block of 16 * NT query
// rows; the waves take the split's chunks round robin and each computes every
// row of the block, so a chunk is loaded and dequantised once per block.  Rows of a KV head
// are ordered (w, hh): r = w * G + hh, hh < G.
// Each wave streams its chunks through its own LDS ring; chunk i-1's P.V,
// whose operands the wave carries over in registers, runs at the start of
// chunk i, just before chunk i's Q.K^T.
// ---------------------------------------------------------------------------
// Shape per row-tile count and element-type pair, each filling most of the
// 160 KiB of LDS with chunk rings: Q8_0 K / Q4_0 V and Q4_0 / Q4_0 with one
// tile (<= 16 rows per KV head) need few registers, so 12 waves (three per
// SIMD) with two-stage rings; two tiles need about 220 registers, so 8 waves
// with three-stage rings.  The larger Q8_0 / Q8_0 chunks take 8 waves with
// two stages, F16 / F16 chunks (16 KiB) 4 waves with two stages.
template <int NT, int KT, int VT>
struct SplitCfg {
    using C = Chunk<KT, VT>;
    static constexpr bool big = C::bytes > 8192;
    static constexpr int waves = C::bytes > 12288 ? 4 : (NT == 1 && !big) ? 12 : 8;
    static constexpr int stages = (NT == 1 || big) ? 2 : 3;
    static constexpr int ring_bytes = stages * C::bytes;
    // the combine after the loop reuses the rings: per wave and row of one
    // 16-row tile, m, l and a padded 132-float accumulator row
    static constexpr int combine_bytes = waves * 16 * (2 + 132) * 4 + 32 * 4;
    static constexpr int lds_bytes = waves * ring_bytes > combine_bytes ? waves * ring_bytes : combine_bytes;
    static_assert(lds_bytes <= 163840, "LDS budget");
};

// STREAM: chunk loads carry the non-temporal hint (each chunk is read by one
// workgroup); calls of several row blocks, whose blocks read the same chunks,
// load without it.  COUNT: the test instantiation that counts softmax
// re-reference events (SplitArgs::rescale_count); the others carry no trace
// of the counter.
template <int NT, int KT, int VT, bool STREAM, bool COUNT>
__global__ __launch_bounds__((64 * SplitCfg<NT, KT, VT>::waves), 1) void split_kernel(const SplitArgs a) {
    using C = Chunk<KT, VT>;
    constexpr int kSplitWaves = SplitCfg<NT, KT, VT>::waves;
    constexpr int kStages = SplitCfg<NT, KT, VT>::stages;
    constexpr int kWaveRingBytes = SplitCfg<NT, KT, VT>::ring_bytes;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // rings; reused by the combine

    // ---- every argument the prologue reads, in one round trip: the split's
    // launch-carried page entries (index clamped into the array) and the
    // scalar fields, all loaded before the first wait (left to itself the
    // compiler loads them in dependent batches, one round trip each)
    // workgroup (KV head, item, row block): consecutive workgroups take
    // different KV heads, so with the round-robin placement of workgroups on
    // the 8 XCDs all splits of a KV head (8 heads) share one XCD's L2 with the
    // merge workgroups of its query heads (merge_unit)
    const uint32_t item = blockIdx.y;
    const uint32_t pre_base = min(item, kPreSplits - 1) * kPrePages;
    const uint4 pre{a.pre_entries[pre_base], a.pre_entries[pre_base + 1], a.pre_entries[pre_base + 2],
                    a.pre_entries[pre_base + 3]};
    asm volatile("" ::"s"(a.page_list), "s"(a.list_offset), "s"(a.n_tokens), "s"(a.T), "s"(a.W), "s"(a.G), "s"(a.Hq),
                 "s"(a.split_chunks), "s"(a.dynamic_order), "s"(a.q), "s"(a.qscale), "s"(a.n_pre_splits),
                 "s"(a.page_table), "s"(a.pool), "s"(a.ring), "s"(a.page_bytes), "s"(a.sec_kd), "s"(a.sec_vc),
                 "s"(a.sec_vd), "s"(a.ring_base), "s"(a.n_ring_slots), "s"(pre.x), "s"(pre.y), "s"(pre.z),
                 "s"(pre.w));

    const int lane = threadIdx.x & 63;
    // wave index, made visibly uniform so chunk bookkeeping stays scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = lane >> 4;  // 16-lane group
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.x;
    const uint32_t block_row0 = blockIdx.z * (16 * NT);
    const uint32_t rows_kv = a.W * a.G;
    const uint32_t n_chunks_all = (a.n_tokens + 31) >> 5;
    const uint32_t cpp = a.T >> 5;  // chunks per page

    // ---- split -> chunk range
    uint32_t split, c_begin, c_end;
    if (a.page_list) {
        split = table_at(a.page_list, a.list_offset + item);
        c_begin = split * cpp;
        c_end = min(c_begin + cpp, n_chunks_all);
    } else {
        split = item;
        c_begin = item * a.split_chunks;
        c_end = min(c_begin + a.split_chunks, n_chunks_all);
    }
    const uint32_t p0 = c_begin / cpp;  // first page of the split
    const bool pre_ok = !a.page_list && item < a.n_pre_splits;
    // chunks whose keys every row sees (keys <= n_tokens - W) need no mask
    const uint32_t clean_end = (a.n_tokens - a.W + 1) >> 5;
    // Chunk order.  A wave's first kStages - 1 chunks are first + kSplitWaves
    // * k; later ones continue that sequence (static order: the chunk-to-wave
    // map and so the bits are fixed) or are claimed from the workgroup's
    // counter as ring buffers free up (dynamic order: waves whose data arrive
    // early take more chunks, so the waves finish together).
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    const uint32_t first = c_begin + wave;
    __shared__ uint32_t next_claim;
    const bool dynamic = a.dynamic_order != 0;
    uint32_t static_k = 0;  // the wave's next index in the static sequence
    auto next_chunk = [&]() -> uint32_t {
        uint32_t c;
        if (!dynamic || static_k < kStages - 1) {
            c = first + kSplitWaves * static_k;
            static_k++;
        } else {
            uint32_t claimed = 0;
            if (lane == 0) claimed = atomicAdd(&next_claim, 1u);
            c = __builtin_amdgcn_readfirstlane(claimed);
        }
        return c < c_end ? c : kNone;
    };

    uint8_t *ring = smem + wave * kWaveRingBytes;
    const uint32_t ring_lds = lds_addr(ring);
    // the pool and ring bases as loaded above (opaque, so the choice between
    // them is not turned back into a load of one of the two arguments)
    const uint8_t *pool_base = a.pool, *ring_base = a.ring;
    asm volatile("" : "+s"(pool_base), "+s"(ring_base));
    auto issue = [&](uint32_t chunk, uint32_t entry, uint32_t stage) {
        const uint32_t jj0 = (chunk - (chunk / cpp) * cpp) << 5;
        issue_chunk<KT, VT, STREAM>(a, page_base(a, pool_base, ring_base, entry), kvh, jj0, lane, ring_lds + stage * C::bytes);
    };

    // ---- query loads, then the ring prologue: the first kStages - 1 chunks
    // of every wave go out without waiting for the queries.  Loads return in
    // issue order, so the compiler's wait before the query conversion (it
    // counts only its own loads) also waits for those chunks, which the first
    // compute needs anyway.
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
    // the ring's chunks in stage order from the one computed next (q[0]);
    // `pend` is issued at the next refill, its page entry already loaded
    uint32_t q[kStages], pend, pend_entry = 0;
    uint32_t entry0[kStages - 1];
#pragma unroll
    for (int i = 0; i < kStages - 1; i++) {
        q[i] = next_chunk();
        entry0[i] = q[i] != kNone ? split_entry(a, pre_ok, pre, p0, q[i] / cpp) : 0u;
    }
    q[kStages - 1] = kNone;
#pragma unroll
    for (int i = 0; i < kStages - 1; i++)
        if (q[i] != kNone) issue(q[i], entry0[i], i);
    // dynamic order: the counter is set before the first claim
    if (dynamic) {
        if (threadIdx.x == 0) next_claim = c_begin + kSplitWaves * (kStages - 1);
        __syncthreads();
    }
    pend = next_chunk();
    if (pend != kNone) pend_entry = split_entry(a, pre_ok, pre, p0, pend / cpp);

    // ---- query fragments: lane (row c16, group g) holds dims 32b + 8g .. +8
    // of block b (in q4_swizzle order for Q4_0 keys, matching their operand),
    // pre-scaled by softmax_scale * log2(e).  Q8_0 keys enter the matrix
    // cores as c + 1152, so each block's sum starts at -1152 times the sum of
    // the row's rounded query over the block (the four groups' shares added
    // across lanes in a fixed order).
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const float4 x = qraw[t][2 * b], y = qraw[t][2 * b + 1];
            const float v[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            half8 h;
#pragma unroll
            for (int e = 0; e < 8; e++) h[e] = (_Float16)(v[KT == kTypeQ4_0 ? q4_swizzle(e) : e] * a.qscale);
            st[t].qf[b] = h;
            if constexpr (KT == kTypeQ8_0) {
                float sum = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++) sum += (float)h[e];
                sum += __shfl_xor(sum, 16);
                sum += __shfl_xor(sum, 32);
                const float c0 = -1152.0f * sum;
                st[t].kcorr[b] = floatx4{c0, c0, c0, c0};
            }
        }


    if (q[0] != kNone) {
        uint32_t pv_vq[C::vw];
        half8 pv_pf[NT][C::pf_blocks];
        uint32_t stage = 0;
        bool have_pv = false;
        while (q[0] != kNone) {
            // refill the buffer the previous chunk used (its reads are complete)
            if (pend != kNone) {
                wait_lgkmcnt0();
                issue(pend, pend_entry, stage == 0 ? kStages - 1 : stage - 1);
                q[kStages - 1] = pend;
                pend = next_chunk();
                if (pend != kNone) pend_entry = split_entry(a, pre_ok, pre, p0, pend / cpp);
            }
            uint32_t newer = 0;  // chunks issued after this one
#pragma unroll
            for (int i = 1; i < kStages; i++) newer += q[i] != kNone ? 1u : 0u;
            wait_chunk<kStages, C::dma>(newer);
            uint8_t *stg = ring + stage * C::bytes;
            const uint32_t c = q[0];
            const bool tail = 32 * c + 32 > a.n_tokens;  // chunk reaches into page padding
            uint32_t kq[C::kw], kd[16], vd[16];
            float s[NT][8];
            read_kcodes<KT, VT>(stg, lane, kq);
            if constexpr (C::kblk) read_kscales<KT, VT>(stg, grp, kd);
            // the previous chunk's P.V first: its operands die before this
            // chunk's scores need registers (measured 0.5 % faster than after
            // the scores, and about 25 fewer registers)
            if (have_pv) chunk_pv<NT, VT>(st, pv_vq, pv_pf);
            chunk_scores<NT, KT>(st, kq, kd, s);
            if (c >= clean_end) mask_scores<NT>(st, 32 * c, grp, s);
            if constexpr (C::vblk) {
                if (tail) sanitize_vscales<KT, VT>(stg, lane, a.n_tokens - 32 * c);
                read_vscales<KT, VT>(stg, grp, vd);
            }
#pragma unroll
            for (int t = 0; t < NT; t++) chunk_probs<VT>(st[t], s[t], vd, pv_pf[t], COUNT ? a.rescale_count : nullptr);
            read_vcodes<KT, VT>(stg, lane, pv_vq);
            if constexpr (!C::vblk)
                if (tail) clear_padding_vcodes<KT, VT>(pv_vq, grp, a.n_tokens - 32 * c);
            have_pv = true;
#pragma unroll
            for (int i = 0; i < kStages - 1; i++) q[i] = q[i + 1];
            q[kStages - 1] = kNone;
            stage = stage == kStages - 1 ? 0 : stage + 1;
        }
        chunk_pv<NT, VT>(st, pv_vq, pv_pf);
    }

    // ---- combine the waves (fixed wave order) and write the partials, one
    // 16-row tile at a time; the rings are reused once every wave is done
    // with its own
    wait_vmcnt<0>();
    constexpr int OS = 132;  // padded row stride
    float *sm_m = reinterpret_cast<float *>(smem);
    float *sm_l = sm_m + kSplitWaves * 16;
    float *sm_o = sm_l + kSplitWaves * 16;
    float *sm_old = sm_o + kSplitWaves * 16 * OS;  // stored (m, l) of the tile's rows (accumulating slots)
    const uint32_t units = a.W * a.Hq;
    // partial written by this workgroup: its slot, or its page / range split
    const uint32_t pidx = a.slot_partials ? item : split;
    const bool accum = item < a.accum_slots;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        __syncthreads();  // rings (first tile) or the previous tile's reads are done
        float l = st[t].l_run;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        // only rows that exist are combined, so only they are staged
        if (block_row0 + 16 * t + c16 < rows_kv) {
            if (grp == 0) {
                sm_m[wave * 16 + c16] = st[t].m_ref;
                sm_l[wave * 16 + c16] = l;
            }
#pragma unroll
            for (int n = 0; n < 8; n++)
                *reinterpret_cast<floatx4 *>(&sm_o[(wave * 16 + c16) * OS + 16 * n + 4 * grp]) = st[t].acc[n];
        }
        const uint32_t row0 = block_row0 + 16 * t;
        const uint32_t rows_here = row0 < rows_kv ? min(16u, rows_kv - row0) : 0u;
        // an accumulating slot's stored (m, l) are read before any thread
        // overwrites them
        if (accum && threadIdx.x < rows_here) {
            const uint32_t rk = row0 + threadIdx.x;
            const uint32_t wq = rk / a.G, hh = rk - wq * a.G;
            const size_t pu = (size_t)pidx * units + wq * a.Hq + kvh * a.G + hh;
            sm_old[2 * threadIdx.x] = a.part_ml[pu * 2];
            sm_old[2 * threadIdx.x + 1] = a.part_ml[pu * 2 + 1];
        }
        __syncthreads();
        for (uint32_t idx = threadIdx.x; idx < rows_here * 128; idx += blockDim.x) {
            const uint32_t r = idx >> 7, d = idx & 127;  // a wave's 64 threads share row r
            // all reads first, no branch between them: a wave with no visible
            // key has m = -inf, l = 0 and a zero accumulator, and
            // 2^(-inf - M) = 0 adds nothing
            float mv[kSplitWaves], lv[kSplitWaves], ov[kSplitWaves];
#pragma unroll
            for (int w = 0; w < kSplitWaves; w++) {
                mv[w] = sm_m[w * 16 + r];
                lv[w] = sm_l[w * 16 + r];
                ov[w] = sm_o[(w * 16 + r) * OS + d];
            }
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < kSplitWaves; w++) M = fmaxf(M, mv[w]);
            float L = 0.f, A = 0.f;
            if (M != kNegInf) {
#pragma unroll
                for (int w = 0; w < kSplitWaves; w++) {
                    const float f = fast_exp2(mv[w] - M);
                    L += f * lv[w];
                    A += f * ov[w];
                }
            }
            const uint32_t rk = row0 + r;
            const uint32_t wq = rk / a.G, hh = rk - wq * a.G;
            const uint32_t unit = wq * a.Hq + kvh * a.G + hh;
            const size_t pu = (size_t)pidx * units + unit;
            if (accum) {
                const PartCombine c = part_combine(sm_old[2 * r], sm_old[2 * r + 1], M, L);
                A = (c.w0 > 0.f ? c.w0 * a.part_o[pu * 128 + d] : 0.f) + c.w1 * A;
                M = c.m;
                L = c.l;
            }
            a.part_o[pu * 128 + d] = A;
            if (d == 0) {
                a.part_ml[pu * 2] = M;
                a.part_ml[pu * 2 + 1] = L;
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

// Log-sum-exp merge (Flash-Decoding's reduction step) of the split partials
// (m, l, acc[128]) of each (row, query head) unit: M = max m_s over splits
// with l_s > 0, w_s = 2^(m_s - M) (0 for empty splits), L = sum w_s l_s,
// out[t] = (sum_s w_s acc_s[t]) / L, dimension t summed in split order.
constexpr int kMergeMaxSplits = 4096;  // splits per unit (one per page at most)
constexpr uint32_t kMergeSmallMax = 64;  // up to this many splits take merge_small_kernel

// Unit merged by workgroup b: KV head b mod Hkv first, so that workgroup b
// runs on the XCD that held the split workgroups of that KV head (the split
// kernel's grid puts the KV head innermost).  A bijection of [0, units):
// b = (w * G + hh) * Hkv + kvh.
__device__ __forceinline__ uint32_t merge_unit(const MergeArgs &a, uint32_t b) {
    const uint32_t r = b / a.Hkv, kvh = b - r * a.Hkv;
    const uint32_t w = r / a.G, hh = r - w * a.G;
    return (w * a.Hkv + kvh) * a.G + hh;
}

// Merge of calls with few splits (decode, verify, prefill chunks: n_splits
// <= KMAX <= 64): one unit per 128-thread workgroup, thread d owns dimension
// d.  No LDS and no barrier: lane s of each wave loads split s's (m, l); M,
// the weights w_s and L come from wave reductions, and w_s reaches every lane
// by v_readlane, so the only wait is the one memory round trip of the loads,
// all issued first.
template <int KMAX>
__global__ __launch_bounds__(128) void merge_small_kernel(const MergeArgs a) {
    const uint32_t unit = merge_unit(a, blockIdx.x);
    const uint32_t d = threadIdx.x, lane = threadIdx.x & 63, ns = a.n_splits;
    const size_t mls = (size_t)a.units * 2, pos = (size_t)a.units * 128;
    const float *po = a.part_o + (size_t)unit * 128 + d;
    float o[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; k++) o[k] = po[(size_t)min((uint32_t)k, ns - 1) * pos];
    const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + (size_t)min(lane, ns - 1) * mls + (size_t)unit * 2);
    asm volatile("" ::: "memory");  // every load above is issued before any result is used
    const bool live = lane < ns && ml.y > 0.f;  // splits with l = 0 (no visible key) are skipped
    const float M = wave_max(live ? ml.x : kNegInf);
    const float w = live ? fast_exp2(ml.x - M) : 0.f;
    const float L = wave_sum(w * ml.y);
    float A = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; k++)
        if ((uint32_t)k < ns) A += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), k)) * o[k];
    a.out[(size_t)unit * 128 + d] = A / L;
}

// Merge of calls with more than 64 splits (streamed layers and resident
// layers split one page per split: one split per page): one unit per
// workgroup of 512 threads.  M, the weights w_s and L reduced over the
// threads in a fixed order; dimension d is summed in four parts (splits
// congruent to q mod 4, in split order), which then add in part order, so
// each thread waits for a quarter of the batches of 32 loads.
constexpr int kManyParts = 4;
constexpr int kMergeBatch = 32;

__global__ __launch_bounds__(128 * kManyParts) void merge_many_kernel(const MergeArgs a) {
    __shared__ float2 wl[kMergeMaxSplits];
    __shared__ float part_sum[kManyParts][128];
    __shared__ float wave_red[2 * kManyParts];
    const uint32_t unit = merge_unit(a, blockIdx.x), tid = threadIdx.x, nt = blockDim.x, ns = a.n_splits;
    const uint32_t lane = tid & 63, wave = tid >> 6;
    const size_t mls = (size_t)a.units * 2, pos = (size_t)a.units * 128;
    const uint32_t d = tid & 127, q = tid >> 7;
    const float *po = a.part_o + (size_t)unit * 128 + d;
    // first batch of this thread's values, issued before anything waits
    float first[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; k++) first[k] = po[(size_t)min(q + kManyParts * k, ns - 1) * pos];
    for (uint32_t s = tid; s < ns; s += nt) wl[s] = *reinterpret_cast<const float2 *>(a.part_ml + s * mls + (size_t)unit * 2);
    __syncthreads();
    float M = kNegInf;
    for (uint32_t s = tid; s < ns; s += nt)
        if (wl[s].y > 0.f) M = fmaxf(M, wl[s].x);
    M = wave_max(M);
    if (lane == 0) wave_red[wave] = M;
    __syncthreads();
    M = wave_red[0];
    for (uint32_t w = 1; w < nt / 64; w++) M = fmaxf(M, wave_red[w]);
    __syncthreads();  // wave_red is reused below
    float L = 0.f;
    for (uint32_t s = tid; s < ns; s += nt) {
        const float2 v = wl[s];
        const float w = v.y > 0.f ? fast_exp2(v.x - M) : 0.f;
        wl[s].x = w;
        L += w * v.y;
    }
    L = wave_sum(L);
    if (lane == 0) wave_red[wave] = L;
    __syncthreads();
    L = 0.f;
    for (uint32_t w = 0; w < nt / 64; w++) L += wave_red[w];
    // dimension d, part q: splits q, q + 4, ... in order
    float A = 0.f;
    const uint32_t nq = ns > q ? (ns - q + kManyParts - 1) / kManyParts : 0;  // splits in this part
#pragma unroll
    for (int k = 0; k < kMergeBatch; k++)
        if ((uint32_t)k < nq) A += wl[q + kManyParts * k].x * first[k];
    for (uint32_t k0 = kMergeBatch; k0 < nq; k0 += kMergeBatch) {
        float ob[kMergeBatch];
#pragma unroll
        for (int k = 0; k < kMergeBatch; k++) ob[k] = po[(size_t)min(q + kManyParts * (k0 + k), ns - 1) * pos];
#pragma unroll
        for (int k = 0; k < kMergeBatch; k++)
            if (k0 + k < nq) A += wl[q + kManyParts * (k0 + k)].x * ob[k];
    }
    part_sum[q][d] = A;
    __syncthreads();
    if (q == 0) {
        float t = part_sum[0][d];
#pragma unroll
        for (int p = 1; p < kManyParts; p++) t += part_sum[p][d];
        a.out[(size_t)unit * 128 + d] = t / L;
    }
}

}  // namespace kvattn_dev

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
namespace {

// Calls f(kernel, waves, lds bytes) with the split kernel of row tiles rt and
// the element-type pair (without the non-temporal hint when `blocks`: several
// row blocks, which have two row tiles; the counting instantiation when
// `count`); false for an unsupported pair.
template <class F>
bool with_split_kernel(int rt, uint32_t kt, uint32_t vt, bool blocks, bool count, F f) {
    using namespace kvattn_dev;
    auto pick = [&](auto nt, auto ktc, auto vtc) {
        constexpr int NT = decltype(nt)::value, KT = decltype(ktc)::value, VT = decltype(vtc)::value;
        using Cfg = SplitCfg<NT, KT, VT>;
        const uint32_t lds = (uint32_t)Cfg::lds_bytes;
        if constexpr (NT == 2) {
            if (blocks) {
                if (count)
                    f(&split_kernel<NT, KT, VT, false, true>, Cfg::waves, lds);
                else
                    f(&split_kernel<NT, KT, VT, false, false>, Cfg::waves, lds);
                return true;
            }
        }
        if (count)
            f(&split_kernel<NT, KT, VT, true, true>, Cfg::waves, lds);
        else
            f(&split_kernel<NT, KT, VT, true, false>, Cfg::waves, lds);
        return true;
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using F16 = std::integral_constant<int, kTypeF16>;
    using Q4 = std::integral_constant<int, kTypeQ4_0>;
    using Q8 = std::integral_constant<int, kTypeQ8_0>;
    if (kt == kTypeQ8_0 && vt == kTypeQ4_0) return rt == 1 ? pick(I1{}, Q8{}, Q4{}) : pick(I2{}, Q8{}, Q4{});
    if (kt == kTypeQ8_0 && vt == kTypeQ8_0) return rt == 1 ? pick(I1{}, Q8{}, Q8{}) : pick(I2{}, Q8{}, Q8{});
    if (kt == kTypeQ4_0 && vt == kTypeQ4_0) return rt == 1 ? pick(I1{}, Q4{}, Q4{}) : pick(I2{}, Q4{}, Q4{});
    if (kt == kTypeF16 && vt == kTypeF16) return rt == 1 ? pick(I1{}, F16{}, F16{}) : pick(I2{}, F16{}, F16{});
    return false;
}

}  // namespace

size_t kvattn_split_smem_bytes(int rt, uint32_t k_type, uint32_t v_type) {
    size_t bytes = 0;
    with_split_kernel(rt, k_type, v_type, false, false, [&](auto, int, uint32_t lds) { bytes = lds; });
    return bytes;
}

uint32_t kvattn_merge_max_splits() { return kvattn_dev::kMergeMaxSplits; }

hipError_t kvattn_split_setup() {
    const uint32_t pairs[4][2] = {{kvattn_dev::kTypeQ8_0, kvattn_dev::kTypeQ4_0},
                                  {kvattn_dev::kTypeQ8_0, kvattn_dev::kTypeQ8_0},
                                  {kvattn_dev::kTypeQ4_0, kvattn_dev::kTypeQ4_0},
                                  {kvattn_dev::kTypeF16, kvattn_dev::kTypeF16}};
    hipError_t err = hipSuccess;
    for (const auto &pr : pairs)
        for (int rt = 1; rt <= 2; rt++)
            for (int blocks = 0; blocks <= 1; blocks++)
                for (int count = 0; count <= 1; count++)
                    with_split_kernel(rt, pr[0], pr[1], blocks != 0, count != 0, [&](auto kern, int, uint32_t lds) {
                        if (err == hipSuccess)
                            err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                    });
    return err;
}

// rt: row tiles of 16 per workgroup (1 or 2); n_row_blocks blocks of 16 * rt rows.
// With events, the launch records them at the dispatch's own start and end
// (timing without extra stream packets).
hipError_t kvattn_launch_split(const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int rt, hipStream_t s,
                               hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();  // clear a stale error so the check below reports this launch
    const dim3 grid(a.Hkv, n_items, n_row_blocks);  // n_items <= 4096 pages
    const bool ok = with_split_kernel(rt, a.k_type, a.v_type, n_row_blocks > 1, a.rescale_count != nullptr,
                                      [&](auto kern, int waves, uint32_t lds) {
        if (ev_start)
            hipExtLaunchKernelGGL(kern, grid, dim3(64 * waves), lds, s, ev_start, ev_stop, 0, a);
        else
            hipLaunchKernelGGL(kern, grid, dim3(64 * waves), lds, s, a);
    });
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t kvattn_launch_merge(const MergeArgs &a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
    (void)hipGetLastError();
    auto go = [&](auto kern, dim3 grid, dim3 block) {
        if (ev_start)
            hipExtLaunchKernelGGL(kern, grid, block, 0, s, ev_start, ev_stop, 0, a);
        else
            hipLaunchKernelGGL(kern, grid, block, 0, s, a);
    };
    // up to 64 splits (decode, verify, prefill chunks): one unit per
    // 128-thread workgroup without LDS or barriers; more (streamed layers and
    // resident layers split one page per split): one unit per 512-thread
    // workgroup
    const dim3 grid(a.units);
    if (a.n_splits > kvattn_dev::kMergeSmallMax)
        go(kvattn_dev::merge_many_kernel, grid, dim3(128 * kvattn_dev::kManyParts));
    else if (a.n_splits <= 8)
        go(kvattn_dev::merge_small_kernel<8>, grid, dim3(128));
    else if (a.n_splits <= 16)
        go(kvattn_dev::merge_small_kernel<16>, grid, dim3(128));
    else if (a.n_splits <= 32)
        go(kvattn_dev::merge_small_kernel<32>, grid, dim3(128));
    else
        go(kvattn_dev::merge_small_kernel<64>, grid, dim3(128));
    return hipGetLastError();
}
