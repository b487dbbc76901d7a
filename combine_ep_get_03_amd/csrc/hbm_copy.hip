// hbm_copy.hip -- plain 128-bit device copy: the HBM copy-bandwidth yardstick and the
// known-size reference for hardware byte counters. Not a step of the dispatch path.
#include "ep_internal.hpp"

namespace ep {
namespace {

#ifndef EP_FAN_U
#define EP_FAN_U 1
#endif

constexpr int kCopyThreads = 256;
constexpr int kCopyU = 4;

__global__ __launch_bounds__(kCopyThreads) void hbm_copy_kernel(const u32x4* __restrict__ in,
                                                                u32x4* __restrict__ out,
                                                                int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads * kCopyU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyU + threadIdx.x;
         base < n; base += stride) {
        u32x4 v[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
            if (i < n) v[u] = load_stream(in + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyU; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
            if (i < n) store_stream(out + i, v[u]);
        }
    }
}

// Mixed-direction yardstick: word i of each of the fan_out output slabs is the XOR of
// word i of the fan_in input slabs (slab = n words, contiguous). fan_in F, fan_out 1
// moves F reads per write, the direction mix of the combine; fan_in 1, fan_out F one
// read per F writes, the mix of the dispatch. Every access is a sequential stream, so
// the time is what HBM sustains for that mix. One-shot threads of U words each.
template <int U>
__global__ __launch_bounds__(kCopyThreads) void hbm_fan_kernel(const u32x4* __restrict__ in,
                                                               u32x4* __restrict__ out,
                                                               int64_t n, int fan_in,
                                                               int fan_out) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * U + threadIdx.x;
    u32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
    for (int s = 0; s < fan_in; s += 8) {
        u32x4 v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (i < n && s + q < fan_in) v[u][q] = load_stream(in + (s + q) * n + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (s + q < fan_in) acc[u] ^= v[u][q];
    }
    for (int j = 0; j < fan_out; ++j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
            if (i < n) store_stream(out + j * n + i, acc[u]);
        }
    }
}

}  // namespace

hipError_t launch_hbm_fan(const void* src, void* dst, size_t slab_bytes, int fan_in,
                          int fan_out, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(slab_bytes / 16);
    if (n == 0) return hipSuccess;
    // a lane keeps about eight loads in flight: U words of fan_in slabs each
    if (fan_in >= 4) {
        constexpr int U = EP_FAN_U;
        const int64_t grid = (n + kCopyThreads * U - 1) / (kCopyThreads * U);
        if (!grid_fits(grid, kCopyThreads)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(hbm_fan_kernel<U>, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads),
                           0, stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n,
                           fan_in, fan_out);
    } else {
        const int64_t grid = (n + kCopyThreads * kCopyU - 1) / (kCopyThreads * kCopyU);
        if (!grid_fits(grid, kCopyThreads)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(hbm_fan_kernel<kCopyU>, dim3(static_cast<unsigned>(grid)),
                           dim3(kCopyThreads), 0, stream, static_cast<const u32x4*>(src),
                           static_cast<u32x4*>(dst), n, fan_in, fan_out);
    }
    return hipGetLastError();
}

hipError_t launch_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t per_block = kCopyThreads * kCopyU;
    // One block per 16 KiB: each thread moves one batch of kCopyU words and exits. On
    // MI355X this one-shot grid measured up to 10% faster than a grid-stride loop over
    // 4096 blocks (2 GiB: 6.16 against 5.52 TB/s); the cap only keeps the work-item
    // count in 32 bits.
    const int64_t grid = std::min<int64_t>((n + per_block - 1) / per_block, int64_t(1) << 22);
    hipLaunchKernelGGL(hbm_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), 0,
                       stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace ep
