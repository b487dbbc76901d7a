// hbm_copy.hip -- 128-bit streams of a fixed read/write mix: the HBM copy-bandwidth
// yardstick, the yardstick for the direction mixes of dispatch and combine, and the
// known-size reference for hardware byte counters, and the combine's fan-in spread over
// one sequential stream per rank. Not a step of the dispatch path.
//
// Each stream takes the cache policy that measured fastest for its mix on MI355X, in
// sequential streams of 512 MiB slabs (beyond the 256 MB Infinity Cache), best of three:
// - one read per write (the copy): non-temporal loads, and stores at device scope (sc1),
//   which write through the L2: 6.45 against 5.44 TB/s with non-temporal stores;
// - reads that outnumber writes (the combine's mix): non-temporal loads and stores;
//   device-scope stores were 1-5% slower from two reads per write up;
// - one read per several writes (the dispatch's mix): cached loads, and stores that are
//   non-temporal and at device scope (nt sc1); at the dispatch's own slab (58.7 MB, 1 to
//   7) cached loads took 74.8 against 87.6 us with non-temporal ones, and nt sc1 stores
//   74.9 against 75.5-76.3 us with nt stores (device-scope stores without nt: 84-85 us).
// Byte counters read the same with either store form (FETCH_SIZE 0.501 and WRITE_SIZE
// 1.000 of the bytes moved, on the copy and on both mixes).
#include "ep.h"
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
    constexpr int64_t per_block = kCopyThreads * kCopyU;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * per_block;
    for (int64_t b0 = static_cast<int64_t>(blockIdx.x) * per_block; b0 < n; b0 += stride) {
        const int64_t left = n - b0;
        const int bytes = static_cast<int>(left < per_block ? left : per_block) * 16;
        // The block's words as two buffers of `bytes` bytes. Their bounds checks stand in
        // for per-word guards: guarded stores each sit in a branch of their own, and the
        // compiler then waits for all memory operations before every store, so the stores
        // of a lane go out one at a time (measured 5.9 TB/s against 6.3 without the waits).
        const __amdgpu_buffer_rsrc_t src = raw_buffer(in + b0, bytes);
        const __amdgpu_buffer_rsrc_t dst = raw_buffer(out + b0, bytes);
        u32x4 v[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; ++u)
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(
                src, (u * kCopyThreads + static_cast<int>(threadIdx.x)) * 16, 0, kPolicyNt);
#pragma unroll
        for (int u = 0; u < kCopyU; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(
                v[u], dst, (u * kCopyThreads + static_cast<int>(threadIdx.x)) * 16, 0,
                kPolicySc1);
    }
}

// Mixed-direction yardstick: word i of each of the fan_out output slabs is the XOR of
// word i of the fan_in input slabs (slab = n words, contiguous). fan_in F, fan_out 1
// moves F reads per write, the direction mix of the combine; fan_in 1, fan_out F one
// read per F writes, the mix of the dispatch. Every access is a sequential stream, so
// the time is what HBM sustains for that mix. One-shot threads of U words each; loads
// are cached with kCached, else non-temporal; with kAll8 every lane issues eight loads
// per batch of slabs (for fan_in >= 4), else only those of existing slabs and words.
template <int U, bool kCached, bool kAll8>
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
        if constexpr (kAll8) {
            // Eight loads per lane, unconditionally: a slab index past fan_in loads the last
            // slab again (the same address; the counters show no extra traffic) and a word
            // past n the last word. With guarded loads, seven input slabs to one output took
            // 77.5 against 73.3 us at 56 MiB slabs on MI355X (8 to 1: 82.7 against 81.4).
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = min(base + static_cast<int64_t>(u) * kCopyThreads, n - 1);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int64_t f = min(s + q, fan_in - 1);
                    v[u][q] = kCached ? in[f * n + i] : load_stream(in + f * n + i);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (i < n && s + q < fan_in)
                        v[u][q] = kCached ? in[(s + q) * n + i] : load_stream(in + (s + q) * n + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (s + q < fan_in) acc[u] ^= v[u][q];
    }
    if constexpr (kCached) {
        // reads fewer than writes: unguarded stores, non-temporal at device scope, through
        // a buffer of the block's words of each output slab (its bounds check drops the
        // words past n), as the dispatch stores its rows
        const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kCopyThreads * U;
        const uint32_t bytes = static_cast<uint32_t>(min<int64_t>(n - b0, kCopyThreads * U)) * 16u;
        for (int j = 0; j < fan_out; ++j) {
            const __amdgpu_buffer_rsrc_t dst = raw_buffer(out + j * n + b0, bytes);
#pragma unroll
            for (int u = 0; u < U; ++u)
                __builtin_amdgcn_raw_buffer_store_b128(
                    acc[u], dst, (u * kCopyThreads + static_cast<int>(threadIdx.x)) * 16, 0,
                    kPolicyNt | kPolicySc1);
        }
    } else {
        for (int j = 0; j < fan_out; ++j) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
                if (i < n) store_stream(out + j * n + i, acc[u]);
            }
        }
    }
}

// Fan-in yardstick with the reads spread over S sequential streams, the way the combine's
// source rows lie in one block of the receive buffer per rank. Block b XORs the input
// chunks j = F b + q (q < F) of kSpreadWords words into output chunk b; chunk j is chunk
// j / S of region j % S (regions of region_words words, back to back), so every region
// is read from its start in order while the grid walks the output. Eight loads per lane,
// unconditionally, as in the fan's form for seven or more slabs: q past F loads chunk
// F b + F - 1 again.
constexpr int kSpreadWords = EP_HBM_SPREAD_CHUNK_BYTES / 16;  // one word per lane
static_assert(kSpreadWords == kCopyThreads, "a spread block is one chunk");

__global__ __launch_bounds__(kCopyThreads) void hbm_spread_kernel(const u32x4* __restrict__ in,
                                                                  u32x4* __restrict__ out,
                                                                  int fan_in, int regions,
                                                                  int64_t region_words) {
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    // chunk j0 = fan_in * b < 2^27 (fan_in <= 8, at most 2^24 blocks); one 32-bit division
    // per wave, then each next chunk is one region further on
    const uint32_t j0 = static_cast<uint32_t>(fan_in) * static_cast<uint32_t>(blockIdx.x);
    uint32_t r = j0 % static_cast<uint32_t>(regions);
    uint32_t c = j0 / static_cast<uint32_t>(regions);
    u32x4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (q > 0 && q < fan_in && ++r == static_cast<uint32_t>(regions)) {
            r = 0;
            ++c;
        }
        v[q] = load_stream(in + r * region_words + static_cast<int64_t>(c) * kSpreadWords + tid);
    }
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (q < fan_in) acc ^= v[q];
    store_stream(out + b * kSpreadWords + tid, acc);
}

}  // namespace

hipError_t launch_hbm_fan(const void* src, void* dst, size_t slab_bytes, int fan_in,
                          int fan_out, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(slab_bytes / 16);
    if (n == 0) return hipSuccess;
    // a lane keeps about eight loads in flight: U words of fan_in slabs each; reads fewer
    // than writes take cached loads (the dispatch's own row loads are cached)
    const auto in = static_cast<const u32x4*>(src);
    const auto out = static_cast<u32x4*>(dst);
    const bool cached = fan_in < fan_out;
    if (fan_in >= 4) {
        constexpr int U = EP_FAN_U;
        const int64_t grid = (n + kCopyThreads * U - 1) / (kCopyThreads * U);
        if (!grid_fits(grid, kCopyThreads)) return hipErrorInvalidConfiguration;
        const dim3 g(static_cast<unsigned>(grid));
        if (cached)
            hipLaunchKernelGGL((hbm_fan_kernel<U, true, true>), g, dim3(kCopyThreads), 0, stream,
                               in, out, n, fan_in, fan_out);
        else
            hipLaunchKernelGGL((hbm_fan_kernel<U, false, true>), g, dim3(kCopyThreads), 0, stream,
                               in, out, n, fan_in, fan_out);
    } else {
        const int64_t grid = (n + kCopyThreads * kCopyU - 1) / (kCopyThreads * kCopyU);
        if (!grid_fits(grid, kCopyThreads)) return hipErrorInvalidConfiguration;
        const dim3 g(static_cast<unsigned>(grid));
        if (cached)
            hipLaunchKernelGGL((hbm_fan_kernel<kCopyU, true, false>), g, dim3(kCopyThreads), 0,
                               stream, in, out, n, fan_in, fan_out);
        else
            hipLaunchKernelGGL((hbm_fan_kernel<kCopyU, false, false>), g, dim3(kCopyThreads), 0,
                               stream, in, out, n, fan_in, fan_out);
    }
    return hipGetLastError();
}

hipError_t launch_hbm_spread(const void* src, void* dst, size_t out_bytes, int fan_in,
                             int regions, hipStream_t stream) {
    const int64_t nb = static_cast<int64_t>(out_bytes / (16 * kSpreadWords));
    if (nb == 0) return hipSuccess;
    // the caller guarantees (fan_in * nb) % regions == 0: src is exactly fan_in * nb chunks
    const int64_t region_words = fan_in * nb / regions * kSpreadWords;
    if (!grid_fits(nb, kCopyThreads)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(hbm_spread_kernel, dim3(static_cast<unsigned>(nb)), dim3(kCopyThreads), 0,
                       stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), fan_in,
                       regions, region_words);
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
