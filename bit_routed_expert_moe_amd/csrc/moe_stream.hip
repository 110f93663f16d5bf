// moe_stream.hip -- a plain streaming read of device memory, the measured
// reference for the expert kernels' HBM rates: the same 16-byte nontemporal
// loads the weight streams use, with no dequantisation, no dependence on
// routing and no hand-off, so its rate is what this chip's HBM delivers to a
// read-only stream of the same size.
//
// Workgroup b of n reads the b-th of n nearly equal contiguous slices (whole
// 16-byte vectors); each thread keeps U loads in flight, lane-consecutive 16-byte
// vectors so that one wave instruction reads 1 KB of contiguous bytes.  The
// loaded words are folded into one XOR per thread, and a thread stores it only
// if it equals a value the data practically never produce, so the loads stay
// and nothing is written.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kStreamUnroll = 8;
constexpr uint32_t kStreamNever = 0x5EED1E55u;

__global__ __launch_bounds__(kBlock) void k_stream_read(const u32x4* src, size_t n16, uint32_t* sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t lo = b0 < n16 ? b0 : n16;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0u;
    size_t i = lo + threadIdx.x;
    // full rounds: every one of the U vectors of the round lies below hi
    for (; i + (size_t)kBlock * (kStreamUnroll - 1) < hi; i += (size_t)kBlock * kStreamUnroll) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = ldg_nt(src + i + (size_t)kBlock * u);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const uint32_t a = v[u][0], b = v[u][1], c = v[u][2], d = v[u][3];
            acc ^= (a ^ b) ^ (c ^ d);
        }
    }
    for (; i < hi; i += kBlock) {  // the slice's tail, one vector at a time
        const u32x4 v = ldg_nt(src + i);
        const uint32_t a = v[0], b = v[1], c = v[2], d = v[3];
        acc ^= (a ^ b) ^ (c ^ d);
    }
    if (acc == kStreamNever) sink[0] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, int n_blocks, uint32_t* sink, hipStream_t s) {
    launch_kernel(k_stream_read, dim3(n_blocks), dim3(kBlock), 0, s, (const u32x4*)src, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
