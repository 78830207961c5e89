// copy_kernels.hip -- the host-to-ring gather copy and the debug page read.
#include "kernels_common.h"

namespace kvattn_dev {

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

// ---------------------------------------------------------------------------
// Table write: entries carried by the launch arguments (one wave).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void table_write_kernel(const TableWriteArgs a) {
    const uint32_t i = threadIdx.x;
    if (i < a.n) {
        a.dst_a[i] = a.a[i];
        if (a.dst_b) a.dst_b[i] = a.b[i];
    }
}

}  // namespace kvattn_dev

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t kvattn_launch_ring_copy(const RingCopyArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::ring_copy_kernel, dim3(a.count * kvattn_dev::kCopySlices), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t kvattn_launch_read_page(const SplitArgs &a, uint32_t logical_page, uint8_t *dst, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL(kvattn_dev::read_page_kernel, dim3(64), dim3(256), 0, s, a, logical_page, dst);
    return hipGetLastError();
}

hipError_t kvattn_launch_table_write(const TableWriteArgs &a, hipStream_t s) {
    (void)hipGetLastError();
    if (a.n > kTableWriteMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kvattn_dev::table_write_kernel, dim3(1), dim3(64), 0, s, a);
    return hipGetLastError();
}
