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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernels.h"

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

namespace kvattn_dev {

constexpr int kWaves = 4;
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
    if (e & 0x40000000u) v = (uint32_t)(((uint64_t)a.ring_base + v) % a.n_ring_slots);
    return a.ring + (size_t)v * a.page_bytes;
}

// ---------------------------------------------------------------------------
// Split kernel.  NRT = row tiles of 16 query rows per wave (1 or 2).
// Rows of a KV head are ordered (w, hh): r = w * G + hh, hh < G.
// ---------------------------------------------------------------------------
template <int NRT>
__global__ __launch_bounds__(256) void split_kernel(const SplitArgs a) {
    constexpr int ROWS = NRT * 16;
    extern __shared__ float smem[];  // [waves][ROWS] m, [waves][ROWS] l, [waves][ROWS][132] acc

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int grp = lane >> 4;  // 16-lane group
    const int c16 = lane & 15;
    const uint32_t kvh = blockIdx.y;
    const uint32_t row0 = blockIdx.z * ROWS;  // first row of this block within the KV head
    const uint32_t rows_kv = a.W * a.G;

    // ---- split -> logical page range
    uint32_t split, first_page, n_pg;
    if (a.page_list) {
        split = a.page_list[a.list_offset + blockIdx.x];
        first_page = split;
        n_pg = 1;
    } else {
        split = blockIdx.x;
        first_page = blockIdx.x * a.split_pages;
        n_pg = min(a.split_pages, a.n_pages - first_page);
    }
    const uint32_t k_begin = first_page * a.T;
    const uint32_t k_end = min(k_begin + n_pg * a.T, a.n_tokens);
    const uint32_t n_chunks = (k_end - k_begin + 31) >> 5;

    // ---- query fragments (B operand of S^T = K Q^T): lane (row c16, group g)
    // holds dims 32b + 8g .. +8 of block b, pre-scaled by softmax_scale*log2(e).
    half8 qf[NRT][4];
    int row_pos[NRT];  // position of the lane's row (as a column of S^T); -1 = padding
#pragma unroll
    for (int rt = 0; rt < NRT; rt++) {
        uint32_t r = row0 + rt * 16 + c16;
        row_pos[rt] = -1;
        if (r < rows_kv) {
            uint32_t w = r / a.G, hh = r - w * a.G;
            uint32_t h = kvh * a.G + hh;
            row_pos[rt] = (int)(a.n_tokens - a.W + w);
            const float *qp = a.q + ((size_t)w * a.Hq + h) * 128;
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const float4 *p4 = reinterpret_cast<const float4 *>(qp + 32 * b + 8 * grp);
                float4 x = p4[0], y = p4[1];
                qf[rt][b] = half8{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale),
                                  (_Float16)(x.z * a.qscale), (_Float16)(x.w * a.qscale),
                                  (_Float16)(y.x * a.qscale), (_Float16)(y.y * a.qscale),
                                  (_Float16)(y.z * a.qscale), (_Float16)(y.w * a.qscale)};
            }
        } else {
#pragma unroll
            for (int b = 0; b < 4; b++) qf[rt][b] = half8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    float m_run[NRT], l_run[NRT];
    floatx4 acc[NRT][8];
#pragma unroll
    for (int rt = 0; rt < NRT; rt++) {
        m_run[rt] = kNegInf;
        l_run[rt] = 0.f;
#pragma unroll
        for (int n = 0; n < 8; n++) acc[rt][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t T = a.T;
    for (uint32_t c = wave; c < n_chunks; c += kWaves) {
        const uint32_t kpos0 = k_begin + 32 * c;
        const uint32_t page = kpos0 / a.T;
        const uint32_t jj0 = kpos0 - page * a.T;
        const uint8_t *base = resolve_page(a, page);

        // ---- loads: K codes (2 tiles x 2), K scales (2 x 32 B), V codes (2), V scales (2 x 32 B)
        const uint4 *kcp = reinterpret_cast<const uint4 *>(base + (size_t)kvh * T * 128 + (size_t)(jj0 >> 4) * 2048) + lane;
        uint4 kq[2][2];
        kq[0][0] = kcp[0];
        kq[0][1] = kcp[64];
        kq[1][0] = kcp[128];
        kq[1][1] = kcp[192];
        const uint4 *kdp = reinterpret_cast<const uint4 *>(base + a.sec_kd + (((size_t)kvh * T + jj0 + 4 * grp) * 4) * 2);
        uint4 kd[2][2];
        kd[0][0] = kdp[0];
        kd[0][1] = kdp[1];
        kd[1][0] = kdp[8];  // +16 keys = 128 bytes
        kd[1][1] = kdp[9];
        const uint4 *vcp = reinterpret_cast<const uint4 *>(base + a.sec_vc + (size_t)kvh * T * 64 + (size_t)(jj0 >> 5) * 2048) + lane;
        uint4 vq[2];
        vq[0] = vcp[0];
        vq[1] = vcp[64];
        const uint4 *vdp = reinterpret_cast<const uint4 *>(base + a.sec_vd + (((size_t)kvh * T + jj0 + 4 * grp) * 4) * 2);
        uint4 vd[2][2];
        vd[0][0] = vdp[0];
        vd[0][1] = vdp[1];
        vd[1][0] = vdp[8];
        vd[1][1] = vdp[9];

        // ---- scores S^T: lane holds keys 16tt + 4g + v (v = 0..3) of its row c16
        float s[NRT][2][4];
#pragma unroll
        for (int tt = 0; tt < 2; tt++) {
            // d_K for the lane's 4 keys: key v, block b at half (4v + b)
            const uint32_t dk[8] = {kd[tt][0].x, kd[tt][0].y, kd[tt][0].z, kd[tt][0].w,
                                    kd[tt][1].x, kd[tt][1].y, kd[tt][1].z, kd[tt][1].w};
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const uint4 &w = kq[tt][b >> 1];
                half8 kf = (b & 1) ? q8_to_half8(w.z, w.w) : q8_to_half8(w.x, w.y);
#pragma unroll
                for (int rt = 0; rt < NRT; rt++) {
                    floatx4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[rt][b], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        // half index 4v + b -> dword (4v + b) / 2, lo if even
                        const int hi = 4 * v + b;
                        float scale = (hi & 1) ? h2f_hi(dk[hi >> 1]) : h2f_lo(dk[hi >> 1]);
                        s[rt][tt][v] = (b == 0) ? scale * d[v] : __builtin_fmaf(scale, d[v], s[rt][tt][v]);
                    }
                }
            }
        }

        // ---- mask, online softmax
        float p[NRT][2][4];
#pragma unroll
        for (int rt = 0; rt < NRT; rt++) {
            float mloc = kNegInf;
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    int key = (int)(kpos0 + 16 * tt + 4 * grp + v);
                    if (key > row_pos[rt]) s[rt][tt][v] = kNegInf;
                    mloc = fmaxf(mloc, s[rt][tt][v]);
                }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float m_new = fmaxf(m_run[rt], mloc);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[rt] - m_use);
            float lsum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    p[rt][tt][v] = fast_exp2(s[rt][tt][v] - m_use);
                    lsum += p[rt][tt][v];
                }
            l_run[rt] = l_run[rt] * alpha + lsum;
            m_run[rt] = m_new;
#pragma unroll
            for (int n = 0; n < 8; n++) acc[rt][n] *= alpha;
        }

        // ---- O^T += V^T P'^T, one 16-dim tile n at a time; block b = n / 2
        const uint32_t vw[8] = {vq[0].x, vq[0].y, vq[0].z, vq[0].w, vq[1].x, vq[1].y, vq[1].z, vq[1].w};
        const uint32_t dv[2][8] = {{vd[0][0].x, vd[0][0].y, vd[0][0].z, vd[0][0].w, vd[0][1].x, vd[0][1].y, vd[0][1].z, vd[0][1].w},
                                   {vd[1][0].x, vd[1][0].y, vd[1][0].z, vd[1][0].w, vd[1][1].x, vd[1][1].y, vd[1][1].z, vd[1][1].w}};
#pragma unroll
        for (int b = 0; b < 4; b++) {
            half8 pf[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; rt++) {
                float e[8];
#pragma unroll
                for (int tt = 0; tt < 2; tt++)
#pragma unroll
                    for (int v = 0; v < 4; v++) {
                        const int hi = 4 * v + b;
                        float scale = (hi & 1) ? h2f_hi(dv[tt][hi >> 1]) : h2f_lo(dv[tt][hi >> 1]);
                        // masked keys have p = 0 but may sit on garbage scales
                        e[4 * tt + v] = (p[rt][tt][v] == 0.f) ? 0.f : p[rt][tt][v] * scale;
                    }
                pf[rt] = half8{(_Float16)e[0], (_Float16)e[1], (_Float16)e[2], (_Float16)e[3],
                               (_Float16)e[4], (_Float16)e[5], (_Float16)e[6], (_Float16)e[7]};
            }
#pragma unroll
            for (int nn = 0; nn < 2; nn++) {
                const int n = 2 * b + nn;
                half8 vf = q4_to_half8(vw[n]);
#pragma unroll
                for (int rt = 0; rt < NRT; rt++) acc[rt][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rt], acc[rt][n], 0, 0, 0);
            }
        }
    }

    // ---- combine the waves of the workgroup (fixed wave order), write partials
    float *sm_m = smem;
    float *sm_l = smem + kWaves * ROWS;
    float *sm_o = smem + 2 * kWaves * ROWS;
    constexpr int OS = 132;  // padded row stride
#pragma unroll
    for (int rt = 0; rt < NRT; rt++) {
        float l = l_run[rt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int r = rt * 16 + c16;
        if (grp == 0) {
            sm_m[wave * ROWS + r] = m_run[rt];
            sm_l[wave * ROWS + r] = l;
        }
#pragma unroll
        for (int n = 0; n < 8; n++)
            *reinterpret_cast<floatx4 *>(&sm_o[(wave * ROWS + r) * OS + 16 * n + 4 * grp]) = acc[rt][n];
    }
    __syncthreads();

    const uint32_t units = a.W * a.Hq;
    const uint32_t rows_here = min((uint32_t)ROWS, rows_kv - row0);
    for (uint32_t idx = threadIdx.x; idx < rows_here * 128; idx += blockDim.x) {
        const uint32_t r = idx >> 7, t = idx & 127;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, sm_m[w * ROWS + r]);
        float L = 0.f, A = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                float f = fast_exp2(sm_m[w * ROWS + r] - M);
                L += f * sm_l[w * ROWS + r];
                A += f * sm_o[(w * ROWS + r) * OS + t];
            }
        }
        const uint32_t rk = row0 + r;
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
// Merge kernel: one wavefront per (row, query head) unit; lane owns dims
// 2*lane, 2*lane + 1.  Splits are folded in index order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
    const int lane = threadIdx.x & 63;
    const uint32_t unit = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= a.units) return;
    float M = kNegInf, L = 0.f, o0 = 0.f, o1 = 0.f;
    for (uint32_t s = 0; s < a.n_splits; s++) {
        const size_t pu = (size_t)s * a.units + unit;
        const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + pu * 2);
        if (!(ml.y > 0.f)) continue;  // empty split
        const float2 v = *reinterpret_cast<const float2 *>(a.part_o + pu * 128 + 2 * lane);
        const float Mn = fmaxf(M, ml.x);
        const float fa = fast_exp2(M - Mn), fb = fast_exp2(ml.x - Mn);
        L = L * fa + ml.y * fb;
        o0 = o0 * fa + v.x * fb;
        o1 = o1 * fa + v.y * fb;
        M = Mn;
    }
    const float inv = 1.f / L;
    *reinterpret_cast<float2 *>(a.out + (size_t)unit * 128 + 2 * lane) = float2{o0 * inv, o1 * inv};
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
size_t kvattn_split_smem_bytes(int nrt) { return (size_t)kvattn_dev::kWaves * nrt * 16 * (2 + 132) * sizeof(float); }

hipError_t kvattn_launch_split(const SplitArgs &a, uint32_t n_items, uint32_t n_row_blocks, int nrt, hipStream_t s) {
    dim3 grid(n_items, a.Hkv, n_row_blocks), block(256);
    size_t smem = kvattn_split_smem_bytes(nrt);
    if (nrt == 1)
        hipLaunchKernelGGL(kvattn_dev::split_kernel<1>, grid, block, smem, s, a);
    else
        hipLaunchKernelGGL(kvattn_dev::split_kernel<2>, grid, block, smem, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_merge(const MergeArgs &a, hipStream_t s) {
    dim3 grid((a.units + 3) / 4), block(256);
    hipLaunchKernelGGL(kvattn_dev::merge_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_read_page(const SplitArgs &a, uint32_t logical_page, uint8_t *dst, hipStream_t s) {
    hipLaunchKernelGGL(kvattn_dev::read_page_kernel, dim3(64), dim3(256), 0, s, a, logical_page, dst);
    return hipGetLastError();
}
