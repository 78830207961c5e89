// debug_kernels.hip -- test aids that run beside the hot path: the ring-slot
// generation tags and slot poisoning that check the streaming schedule on
// the device.
#include "kernels_common.h"

namespace kvattn_dev {

// ---------------------------------------------------------------------------
// Ring-slot tags: the generation of each slot of a streamed chunk (the
// page's global ordinal), written on the copy stream after the chunk's copy
// and checked on the compute stream just before and just after the compute
// that reads it.  A slot refilled before its reader finished, or read before
// its copy finished, holds another generation.
// ---------------------------------------------------------------------------
template <bool CHECK>
__global__ __launch_bounds__(256) void ring_tag_kernel(const RingTagArgs a) {
    uint32_t bad = 0, seen = 0;
    for (uint32_t i = threadIdx.x; i < a.count; i += blockDim.x) {
        const uint32_t o = a.first + i;
        const uint32_t slot = (uint32_t)(((uint64_t)a.ring_base + o) % a.n_slots);
        if (CHECK) {
            bad += a.tags[slot] != a.ord_lo + o ? 1u : 0u;
            seen++;
        } else {
            a.tags[slot] = a.ord_lo + o + a.skew;
        }
    }
    if (CHECK && seen) {
        atomicAdd(&a.counter[0], bad);
        atomicAdd(&a.counter[1], seen);
    }
}

// Poisoning: once a chunk's readers are done, its slots are filled with
// 0xFF bytes (NaN binary16 scales and values) before the consumed fence, so
// a read of a recycled slot before its refill turns the output into NaN.
constexpr int kPoisonSlices = 8;

__global__ __launch_bounds__(256) void ring_poison_kernel(const RingTagArgs a) {
    const uint32_t o = a.first + blockIdx.x / kPoisonSlices;
    const uint32_t sl = blockIdx.x % kPoisonSlices;
    const uint32_t slot = (uint32_t)(((uint64_t)a.ring_base + o) % a.n_slots);
    const size_t n16 = a.page_bytes / 16;
    const size_t per = (n16 + kPoisonSlices - 1) / kPoisonSlices;
    const size_t b = sl * per, e = min(n16, b + per);
    uint4 *dst = reinterpret_cast<uint4 *>(a.ring + (size_t)slot * a.page_bytes);
    const uint4 nan4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    for (size_t i = b + threadIdx.x; i < e; i += blockDim.x) dst[i] = nan4;
}

}  // namespace kvattn_dev

hipError_t kvattn_launch_ring_tag(const RingTagArgs &a, bool check, hipStream_t s) {
    (void)hipGetLastError();
    if (!a.tags || a.n_slots == 0 || (check && !a.counter)) return hipErrorInvalidValue;
    if (check)
        hipLaunchKernelGGL(kvattn_dev::ring_tag_kernel<true>, dim3(1), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(kvattn_dev::ring_tag_kernel<false>, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_ring_poison(const RingTagArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    if (!a.ring || a.n_slots == 0 || a.count == 0 || a.page_bytes % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kvattn_dev::ring_poison_kernel, dim3(a.count * kvattn_dev::kPoisonSlices), dim3(256), 0, s, a);
    return hipGetLastError();
}
