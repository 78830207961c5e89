// writer_kernel.hip -- the KV writer: quantise new K/V rows into their pages.
#include "kernels_common.h"

namespace kvattn_dev {

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

}  // namespace kvattn_dev

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t kvattn_launch_writer(const WriterArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    const uint32_t tiles = (a.n_old + a.R - 1) / 32 - a.n_old / 32 + 1;
    hipLaunchKernelGGL(kvattn_dev::writer_kernel, dim3(tiles, a.Hkv), dim3(256), 0, s, a);
    return hipGetLastError();
}
