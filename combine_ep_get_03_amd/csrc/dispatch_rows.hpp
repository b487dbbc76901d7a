// dispatch_rows.hpp -- the row copy of the (token, destination) dispatch waves: a token's
// row loaded into registers and stored to a receive row with the destination rank's view
// of the routing. Shared by dispatch.hip and by the one-launch layout + dispatch of a
// single 256-token group in layout.hip.
#pragma once

#include <type_traits>

#include "ep_internal.hpp"

namespace ep {
namespace {

#ifndef EP_ROW_STORE_POLICY
#define EP_ROW_STORE_POLICY (kPolicyNt | kPolicySc1)
#endif

// One pass of a destination row: words v0 + 64 i + lane (i < WPL) of a row of V words
// (the same row for every lane of the wave). The row is addressed through a buffer
// resource of V words, whose bounds check drops the words at V and beyond, so no store
// waits behind a per-word guard. The stores are non-temporal at device scope (nt sc1).
// Measured on MI355X against guarded non-temporal stores, same box, identical outputs:
// the dispatch 81.3 against 82.6 us at 4096 tokens (top-8 over 32 ranks, 7168 channels)
// and 333.8 against 341.4 us at 16384 tokens over 64 ranks, the dispatch with its slots
// 82.0 against 83.6 and 334.7 against 340.4 us. Unguarded stores that were non-temporal
// only ran as the guarded ones, and device-scope stores that were not non-temporal ran
// 12-15% slower. The same policy on the combine's output rows was slower at 4096 tokens.
template <int WPL>
__device__ __forceinline__ void store_row_pass(u32x4* row, int V, int v0,
                                               const u32x4 (&v)[WPL]) {
    // readfirstlane returns a signed int: each half goes through uint32_t, so the low half
    // is not sign-extended into the high one
    const uint64_t a = reinterpret_cast<uint64_t>(row);
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32))));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))));
    const uint64_t ua = (static_cast<uint64_t>(hi) << 32) | lo;
    const __amdgpu_buffer_rsrc_t rr =
        raw_buffer(reinterpret_cast<const void*>(ua), static_cast<uint32_t>(V) * 16u);
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < WPL; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(v[i], rr, (v0 + i * kWave + lane) * 16, 0,
                                               EP_ROW_STORE_POLICY);
}

// A token's k-slot routing as it travels with its row. Lane j < 64 holds slot j (loaded
// once); larger k reloads per destination. With kRankView the routing written to row sd
// is rank `rank`'s view: the local expert id and the weight where the expert is on that
// rank, else -1 and +0.0f; without it the ids and weights are copied unchanged.
struct Routing {
    const int64_t* idx_row;  // [k]; non-null whenever dst_idx or dst_w is
    const float* w_row;      // [k] or null (weights read as 0)
    int k;
    int64_t e0;
    float w0;

    __device__ __forceinline__ Routing(const int64_t* idx, const float* w, int k_, bool meta)
        : idx_row(idx), w_row(w), k(k_), e0(-1), w0(0.0f) {
        const int lane = lane_id();
        if (meta && lane < k) {
            e0 = idx_row[lane];
            if (w_row) w0 = w_row[lane];
        }
    }

    template <bool kRankView>
    __device__ __forceinline__ void write(int64_t sd, int rank, int er, int64_t* dst_idx,
                                          float* dst_w) const {
        const int lane = lane_id();
        for (int j0 = 0; j0 < k; j0 += kWave) {
            const int j = j0 + lane;
            if (j >= k) continue;
            const int64_t e = j0 == 0 ? e0 : idx_row[j];
            const float wv = j0 == 0 ? w0 : (w_row ? w_row[j] : 0.0f);
            if (kRankView) {
                const int64_t lo = static_cast<int64_t>(rank) * er;
                const bool local = e >= lo && e < lo + er;
                if (dst_idx) dst_idx[sd * k + j] = local ? e - lo : -1;
                if (dst_w) dst_w[sd * k + j] = local ? wv : 0.0f;
            } else {
                if (dst_idx) dst_idx[sd * k + j] = e;
                if (dst_w) dst_w[sd * k + j] = wv;
            }
        }
    }
};

// One pass of a row (words v0 .. v0 + 64 WPL, WPL words per lane in registers) into
// destination row sd; the first pass also writes the routing (rank `rank`'s view with
// kRankView) and the source id. Rows wider than one pass (V > 64 WPL) take the kernels'
// kMulti pass loop; without it the loop is known to run once, which keeps the register
// count down.
template <int WPL, bool kRankView>
__device__ __forceinline__ void put_row(const u32x4 (&v)[WPL], int v0, int V, int64_t sd,
                                        int rank, const Routing& rt, int er, int32_t src,
                                        u32x4* __restrict__ dst_x, int64_t* __restrict__ dst_idx,
                                        float* __restrict__ dst_w, int32_t* __restrict__ dst_src) {
    const int lane = lane_id();
    store_row_pass(dst_x + sd * V, V, v0, v);
    if (v0 != 0) return;
    if (dst_idx || dst_w) rt.write<kRankView>(sd, rank, er, dst_idx, dst_w);
    if (dst_src && lane == 0) dst_src[sd] = src;
}

// A pass inside the row (the whole row at 7168 channels) loads at fixed offsets; in a pass
// that runs past the row's end, a lane past it loads the row's last word again instead of
// skipping the load (its stores are skipped). Either way every load is unconditional, so
// the compiler keeps them all in flight at once: with guarded loads it waited for each
// before issuing the next at 7 words per lane.
template <int WPL>
__device__ __forceinline__ void load_row_cached(u32x4 (&v)[WPL], const u32x4* __restrict__ xr,
                                                int v0, int V) {
    const int lane = lane_id();
    if (v0 + WPL * kWave <= V) {
#pragma unroll
        for (int i = 0; i < WPL; ++i) v[i] = xr[v0 + i * kWave + lane];
    } else {
#pragma unroll
        for (int i = 0; i < WPL; ++i) v[i] = xr[min(v0 + i * kWave + lane, V - 1)];
    }
}

// Index of the calling wave in the grid (wave-uniform).
template <int kThreads>
__device__ __forceinline__ int grid_wave() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kThreads / kWave) +
                                          static_cast<int>(threadIdx.x) / kWave);
}

// The (token, destination index) of wave p in a launch over tokens [t0, t_end): wave p
// is (t0 + p / D, p % D).
__device__ __forceinline__ bool dest_wave_at(int p, int64_t t0, int64_t t_end, FastDiv D,
                                             int64_t& t, int& d) {
    const int q = D.div(p);
    t = t0 + q;
    d = p - q * D.d;
    return t < t_end;
}

template <int kThreads>
__device__ __forceinline__ bool dest_wave(int64_t t0, int64_t t_end, FastDiv D, int64_t& t, int& d) {
    return dest_wave_at(grid_wave<kThreads>(), t0, t_end, D, t, d);
}

// Calls f(WPL, kMulti) with the smallest words-per-lane count (1, 2, 4, 7, ..., kMax)
// whose single pass holds a row of `words`, or with kMax and several passes beyond that.
// kLoop asks for the pass-loop form at every width.
template <int kMax, bool kLoop, typename F>
hipError_t with_row_width(int words, F&& f) {
    using One = std::integral_constant<bool, kLoop>;
    if (words <= kWave) f(std::integral_constant<int, 1>{}, One{});
    else if (words <= 2 * kWave) f(std::integral_constant<int, 2>{}, One{});
    else if (words <= 4 * kWave) f(std::integral_constant<int, 4>{}, One{});
    else if (words <= 7 * kWave) f(std::integral_constant<int, 7>{}, One{});
    else if (kMax > 7 && words <= kMax * kWave) f(std::integral_constant<int, kMax>{}, One{});
    else f(std::integral_constant<int, kMax>{}, std::true_type{});
    return hipGetLastError();
}

}  // namespace
}  // namespace ep
