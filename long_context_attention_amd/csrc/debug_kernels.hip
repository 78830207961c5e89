// debug_kernels.hip -- test aids that run beside the hot path: the ring-slot
// generation tags that check the streaming schedule on the device.
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
