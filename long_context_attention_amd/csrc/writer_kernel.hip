// writer_kernel.hip -- the KV writer: quantise new K/V rows into their pages.
#include "kernels_common.h"

namespace kvattn_dev {

// ---------------------------------------------------------------------------
// KV writer ("troed's fork ...", section "KV data movement and attention":
// the new rows are quantised into the tail page before attention reads
// them).  Q8_0: d = amax / 127 rounded to binary16, code =
// round-half-even(x / d) clamped to +-127 (zero scale: codes 0).  Q4_0: m =
// the element of largest magnitude (first on ties), d = m / -8 rounded to
// binary16, code = round-half-even(x / d) + 8 clamped to [0, 15] (zero
// scale: codes 8).  F16: x rounded to binary16 (nearest even).  Every
// decision is taken in binary32 (correctly rounded division,
// round-to-nearest-even conversions).
// One workgroup per (32-token tile, KV head): a Q4_0 V byte holds the
// nibbles of tokens j and j + 16 of one tile, so the tile's owner merges new
// nibbles with the ones already there and no two workgroups touch one byte.
// Lane l of a wave handles elements 2l and 2l + 1 of a head row (block
// l / 16, so a block's 32 elements sit in 16 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint8_t *writer_page(const WriterArgs &a, uint32_t logical_page) {
    const uint32_t e = a.page_table[logical_page];
    if (e < 0x80000000u) return a.pool + (size_t)e * a.page_bytes;
    uint32_t v = e & 0x3FFFFFFFu;
    if (e & 0x40000000u) v = (a.ring_base + v) % a.n_ring_slots;
    return a.ring + (size_t)v * a.page_bytes;
}

struct Coded {
    _Float16 d;    // block scale
    uint32_t c0, c1;  // codes of the lane's two elements (Q8_0: the int8 as a byte)
};

// Q8_0 of the lane's pair within its 16-lane block.
__device__ __forceinline__ Coded encode_q8_0(float2 x) {
    float amax = fmaxf(fabsf(x.x), fabsf(x.y));
#pragma unroll
    for (int k = 1; k < 16; k <<= 1) amax = fmaxf(amax, __shfl_xor(amax, k));
    Coded o;
    o.d = (_Float16)(amax / 127.0f);
    const float d = (float)o.d;
    int c0 = 0, c1 = 0;
    if (d != 0.0f) {
        c0 = (int)fminf(fmaxf(rintf(x.x / d), -127.0f), 127.0f);
        c1 = (int)fminf(fmaxf(rintf(x.y / d), -127.0f), 127.0f);
    }
    o.c0 = (uint8_t)c0;
    o.c1 = (uint8_t)c1;
    return o;
}

// Q4_0 of the lane's pair (elements i0, i0 + 1 of the block).
__device__ __forceinline__ Coded encode_q4_0(float2 x, uint32_t i0) {
    float best = fabsf(x.x), val = x.x;
    uint32_t idx = i0;
    if (fabsf(x.y) > best) {
        best = fabsf(x.y);
        val = x.y;
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
    Coded o;
    o.d = (_Float16)(val / -8.0f);
    const float d = (float)o.d;
    o.c0 = o.c1 = 8;
    if (d != 0.0f) {
        o.c0 = (uint32_t)fminf(fmaxf(rintf(x.x / d) + 8.0f, 0.0f), 15.0f);
        o.c1 = (uint32_t)fminf(fmaxf(rintf(x.y / d) + 8.0f, 0.0f), 15.0f);
    }
    return o;
}

__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

__global__ __launch_bounds__(256) void writer_kernel(const WriterArgs a) {
    __shared__ uint8_t nib[32][128];  // Q4_0 V codes of the tile's new tokens
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
    const uint32_t t = e0;
    for (uint32_t jt = wave; jt < 32; jt += 4) {
        const uint32_t pos = tb + jt;
        if (pos < lo || pos >= hi) continue;            // wave-uniform
        const uint32_t r = pos - a.n_old, j = j0 + jt;  // new row, token in the page
        const float2 xk = *reinterpret_cast<const float2 *>(a.k + ((size_t)r * a.Hkv + h) * 128 + e0);
        const float2 xv = *reinterpret_cast<const float2 *>(a.v + ((size_t)r * a.Hkv + h) * 128 + e0);
        // K-tile lane of (token j, dim t): the 16-byte row a reader lane loads
        const uint32_t klane = ((t % 32) / 8) * 16 + j % 16;

        // ---- K
        if (a.k_type == kTypeF16) {
            // (j/16)*4096 + (t/32)*1024 + klane*16 + (t%8)*2: the pair is one dword
            const size_t kb = (size_t)h * T * 256 + (size_t)(j / 16) * 4096 + (t / 32) * 1024 + klane * 16 + (t % 8) * 2;
            *reinterpret_cast<uint32_t *>(page + kb) = f16_bits(xk.x) | ((uint32_t)f16_bits(xk.y) << 16);
        } else {
            Coded ck;
            if (a.k_type == kTypeQ8_0) {
                ck = encode_q8_0(xk);
                // (j/16)*2048 + (t/64)*1024 + klane*16 + ((t/32)%2)*8 + t%8: two adjacent bytes
                const size_t kb = (size_t)h * T * 128 + (size_t)(j / 16) * 2048 + (t / 64) * 1024 + klane * 16 +
                                  ((t / 32) % 2) * 8 + t % 8;
                *reinterpret_cast<uint16_t *>(page + kb) = (uint16_t)(ck.c0 | (ck.c1 << 8));
            } else {
                ck = encode_q4_0(xk, i0);
                // (j/16)*1024 + klane*16 + (t/32)*4 + (t%8)%4: dims t and t + 4
                // share a byte (low, high nibble); the lane of dims t, t + 1
                // with t % 8 < 4 takes the high nibbles from the lane 2 above
                const uint32_t h0 = __shfl(ck.c0, (int)lane + 2), h1 = __shfl(ck.c1, (int)lane + 2);
                if (t % 8 < 4) {
                    const size_t kb = (size_t)h * T * 64 + (size_t)(j / 16) * 1024 + klane * 16 + (t / 32) * 4 + t % 8;
                    *reinterpret_cast<uint16_t *>(page + kb) = (uint16_t)((ck.c0 | (h0 << 4)) | ((ck.c1 | (h1 << 4)) << 8));
                }
            }
            if ((lane & 15) == 0) *reinterpret_cast<_Float16 *>(page + a.sec_kd + ((size_t)h * T + j) * 8 + b * 2) = ck.d;
        }

        // ---- V (token jj of the 32-token tile: operand group g, slot s)
        const uint32_t jj = jt, g = (jj % 16) / 4, slot = (jj / 16) * 4 + jj % 4;
        if (a.v_type == kTypeF16) {
            // (j/32)*8192 + (t/16)*1024 + (g*16 + t%16)*16 + slot*2, per element
            uint8_t *vt = page + a.sec_vc + (size_t)h * T * 256 + (size_t)(j / 32) * 8192;
            *reinterpret_cast<uint16_t *>(vt + (t / 16) * 1024 + (g * 16 + t % 16) * 16 + slot * 2) = f16_bits(xv.x);
            *reinterpret_cast<uint16_t *>(vt + ((t + 1) / 16) * 1024 + (g * 16 + (t + 1) % 16) * 16 + slot * 2) =
                f16_bits(xv.y);
        } else {
            Coded cv;
            if (a.v_type == kTypeQ8_0) {
                cv = encode_q8_0(xv);
                // (j/32)*4096 + (t/32)*1024 + (g*16 + t%16)*16 + ((t/16)%2)*8 + slot
                uint8_t *vt = page + a.sec_vc + (size_t)h * T * 128 + (size_t)(j / 32) * 4096;
                vt[(t / 32) * 1024 + (g * 16 + t % 16) * 16 + ((t / 16) % 2) * 8 + slot] = (uint8_t)cv.c0;
                vt[((t + 1) / 32) * 1024 + (g * 16 + (t + 1) % 16) * 16 + (((t + 1) / 16) % 2) * 8 + slot] =
                    (uint8_t)cv.c1;
            } else {
                cv = encode_q4_0(xv, i0);
                nib[jt][e0] = (uint8_t)cv.c0;
                nib[jt][e0 + 1] = (uint8_t)cv.c1;
            }
            if ((lane & 15) == 0)
                *reinterpret_cast<_Float16 *>(page + a.sec_vd + (size_t)h * T * 8 + (size_t)(j / 32) * 256 +
                                              (b * 4 + g) * 16 + slot * 2) = cv.d;
        }
    }
    if (a.v_type != kTypeQ4_0) return;  // uniform over the workgroup
    __syncthreads();

    // Q4_0 V bytes of the tile: byte of (token jl < 16, dim t) at (t/64)*1024
    // + ((jl/4)*16 + t%16)*16 + ((t/16)%4)*4 + jl%4, low nibble token jl,
    // high nibble token jl + 16; keep the nibble of a token not written now
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
