// dispatch.hip -- token-major dispatch permute on gfx950.
//
// Every (token, rank) pair with a receive slot s gets row s of recv_x = the token's bf16
// row, plus the rank's view of the token's top-k routing and the token id. On one GPU
// the intra-node hop of the pages ("[PR #347] Feature/sm free normal kernel", section
// 3.3.2) is an HBM-to-HBM copy, and rows are written straight to their final place with
// no staging buffer (the zero-copy idea of "[PR #453] ... Zero-Copy and TMA Offloading").
//
// Design: one wave64 owns one token. Each lane loads its share of the row (up to 14
// 128-bit words, so a 7168-wide bf16 row is fully in registers) with all loads in flight
// at once. The destinations are found with a ballot over the token_slot row and walked
// in ascending rank with readlane, so the destination row address is wave-uniform and
// each destination row is written as one sequential burst of non-temporal 128-bit
// stores. No LDS and no block barrier. The work per token is bounded by min(k, R)
// destinations whatever the skew of the per-rank counts. HBM-write bound.
// Batches small enough that the one-token grid would be resident at once take a form
// with two tokens per wave (dispatch_pair_kernel, and dispatch_send_pair_kernel for the
// send phase), which overlaps the second token's loads with the first token's stores.
// Block sizes and the pass-loop form are chosen per kernel by measurement (below).
#include <atomic>
#include <type_traits>

#include "ep_internal.hpp"

namespace ep {
namespace {

#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 1
#endif

// Launch shapes, one token (or staged row) per wave, chosen by same-box A/B timing on
// MI355X at the 4096 x 7168 and 16384 x 7168 top-8 shapes: the one-call dispatch, the
// permute and the send phase run the pass-loop form in 512-thread blocks (the one-pass
// form ran 4-5% slower for them), the receive phase and the FP8 dispatch the one-pass
// form in 256-thread blocks (5% faster for the receive phase).
constexpr int kRowThreads = 512;
constexpr int kRecvThreads = 256;
constexpr int kFp8Threads = 256;
constexpr int kPairThreads = 256;  // two tokens per wave (small batches): 256 beat 512

// Token waves the one-token dispatch grid keeps resident at once: 16 per compute unit
// (two 512-thread blocks at its register use). Below this the grid does not fill the
// chip, and the two-tokens-per-wave form is faster. Queried per device and cached.
int resident_token_waves() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];  // zero until first queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int waves = cache[dev].load(std::memory_order_relaxed);
    if (waves == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        waves = 16 * cus;
        cache[dev].store(waves, std::memory_order_relaxed);
    }
    return waves;
}

__device__ __forceinline__ void store_row_word(u32x4* p, u32x4 v) {
#if EP_DISPATCH_NT_STORE
    store_stream(p, v);
#else
    *p = v;
#endif
}

// The destination walk of every dispatch kernel. Slot c of the calling wave's row of C
// slots, when >= 0, names destination row slot + c * cbase (a slot >= cap is an overflow:
// skipped, and the error bit set). Destinations are found with one ballot per 64 slots
// and visited in ascending c through readlane, so the row index handed to visit(row, c)
// is wave-uniform.
// One chunk of the walk: lane l holds slot c0 + l (-1 where there is none).
template <typename Visit>
__device__ __forceinline__ void visit_chunk(int32_t s, int c0, int64_t cbase, int64_t cap,
                                            int32_t& errbits, Visit&& visit) {
    if (s >= cap) {
        errbits |= kErrRecvOverflow;
        s = -1;
    }
    uint64_t m = wave_ballot(s >= 0);
    while (m) {
        const int src_lane = __builtin_ctzll(m);
        m &= m - 1;
        const int cd = c0 + src_lane;
        visit(static_cast<int64_t>(__builtin_amdgcn_readlane(s, src_lane)) + cd * cbase, cd);
    }
}

template <typename Visit>
__device__ __forceinline__ void for_each_destination(const int32_t* __restrict__ srow, int C,
                                                     int64_t cbase, int64_t cap,
                                                     int32_t& errbits, Visit&& visit) {
    const int lane = lane_id();
    for (int c0 = 0; c0 < C; c0 += kWave)
        visit_chunk(c0 + lane < C ? srow[c0 + lane] : -1, c0, cbase, cap, errbits, visit);
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

// One source row of V 128-bit words, WPL words per lane in registers per pass, to every
// destination of the walk, with the routing (rank rank0 + c's view with kRankView) and
// the source id written once per destination. Rows wider than one pass (V > 64 WPL) need
// kMulti; without it the pass loop is known to run once, which keeps the register count
// down (96 against 116 VGPRs at WPL = 14).
// One pass of a row (words v0 .. v0 + 64 WPL) into destination row sd; the first pass
// also writes the rank's view of the routing and the source id.
template <int WPL, bool kRankView>
__device__ __forceinline__ void put_row(const u32x4 (&v)[WPL], int v0, int V, int64_t sd,
                                        int rank, const Routing& rt, int er, int32_t src,
                                        u32x4* __restrict__ dst_x, int64_t* __restrict__ dst_idx,
                                        float* __restrict__ dst_w, int32_t* __restrict__ dst_src) {
    const int lane = lane_id();
    u32x4* row = dst_x + sd * V;
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
        const int vi = v0 + i * kWave + lane;
        if (vi < V) store_row_word(row + vi, v[i]);
    }
    if (v0 != 0) return;
    if (dst_idx || dst_w) rt.write<kRankView>(sd, rank, er, dst_idx, dst_w);
    if (dst_src && lane == 0) dst_src[sd] = src;
}

template <int WPL>
__device__ __forceinline__ void load_row(u32x4 (&v)[WPL], const u32x4* __restrict__ xr, int v0,
                                         int V) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
        const int vi = v0 + i * kWave + lane;
        if (vi < V) v[i] = load_stream(xr + vi);
    }
}

template <int WPL, bool kMulti, bool kRankView>
__device__ __forceinline__ void scatter_row(
    const u32x4* __restrict__ xr, int V, const Routing& rt, int er, int32_t src,
    const int32_t* __restrict__ srow, int C, int64_t cbase, int rank0, int64_t cap,
    u32x4* __restrict__ dst_x, int64_t* __restrict__ dst_idx, float* __restrict__ dst_w,
    int32_t* __restrict__ dst_src, int32_t& errbits) {
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        u32x4 v[WPL];
        load_row(v, xr, v0, V);
        for_each_destination(srow, C, cbase, cap, errbits, [&](int64_t sd, int cd) {
            put_row<WPL, kRankView>(v, v0, V, sd, rank0 + cd, rt, er, src, dst_x, dst_idx, dst_w,
                                    dst_src);
        });
        if constexpr (!kMulti) break;
    }
}

template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int R, int er,
    const int32_t* __restrict__ token_slot, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    int32_t errbits = 0;
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     recv_idx || recv_w);
    scatter_row<WPL, kMulti, true>(x + t * V, V, rt, er, static_cast<int32_t>(t), token_slot + t * R, R,
                           0, 0, cap, recv_x, recv_idx, recv_w, recv_src, errbits);
    if (errbits) raise_error(error_flag, errbits);
}

// Small batches (C <= 64 slots, k <= 64, one pass per row): each wave owns two tokens,
// t and t + W (W waves in the grid). Token t's row, slot row and routing are loaded
// first and token t + W's right after, so token t's writes wait only for its own loads
// and token t + W's loads arrive meanwhile. Token t's row goes to destination row
// slot + c * cbase for every slot c >= 0 of its row, with the routing (rank c's view with
// kRankView, else unchanged) and the source id. Used while the one-token grid would be
// resident at once. On MI355X at 1024, 2048 and 4096 tokens of 7168 channels the
// dispatch ran 16%, 9% and 2% faster than one token per wave (2-3% slower at 8192 and
// 16384), and the send phase 26%, 19% and 5.5% faster.
template <int WPL, bool kRankView, int kThreads>
__device__ __forceinline__ void pair_scatter(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int er,
    const int32_t* __restrict__ slot_tab, int C, int64_t cbase, int64_t cap,
    u32x4* __restrict__ dst_x, int64_t* __restrict__ dst_idx, float* __restrict__ dst_w,
    int32_t* __restrict__ dst_src, int32_t* __restrict__ error_flag) {
    const int lane = lane_id();
    constexpr int kWpb = kThreads / kWave;
    const int64_t W = static_cast<int64_t>(gridDim.x) * kWpb;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWpb + threadIdx.x / kWave;
    if (t0 >= T) return;
    const int64_t t1 = t0 + W;
    const bool has1 = t1 < T;
    const bool meta = dst_idx || dst_w;
    u32x4 a[WPL], b[WPL];
    load_row(a, x + t0 * V, 0, V);
    const int32_t s0 = lane < C ? slot_tab[t0 * C + lane] : -1;
    const Routing r0(topk_idx ? topk_idx + t0 * k : nullptr, topk_w ? topk_w + t0 * k : nullptr,
                     k, meta);
    int32_t s1 = -1;
    if (has1) {
        load_row(b, x + t1 * V, 0, V);
        s1 = lane < C ? slot_tab[t1 * C + lane] : -1;
    }
    int32_t errbits = 0;
    visit_chunk(s0, 0, cbase, cap, errbits, [&](int64_t sd, int cd) {
        put_row<WPL, kRankView>(a, 0, V, sd, cd, r0, er, static_cast<int32_t>(t0), dst_x, dst_idx,
                                dst_w, dst_src);
    });
    if (has1) {
        const Routing r1(topk_idx ? topk_idx + t1 * k : nullptr,
                         topk_w ? topk_w + t1 * k : nullptr, k, meta);
        visit_chunk(s1, 0, cbase, cap, errbits, [&](int64_t sd, int cd) {
            put_row<WPL, kRankView>(b, 0, V, sd, cd, r1, er, static_cast<int32_t>(t1), dst_x,
                                    dst_idx, dst_w, dst_src);
        });
    }
    if (errbits) raise_error(error_flag, errbits);
}

template <int WPL, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_pair_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int R, int er,
    const int32_t* __restrict__ token_slot, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag) {
    pair_scatter<WPL, true, kThreads>(x, topk_idx, topk_w, T, V, k, er, token_slot, R, 0, cap, recv_x,
                            recv_idx, recv_w, recv_src, error_flag);
}

// The send phase's small-batch form: node slots, rows n * Tmax + slot, routing unchanged.
template <int WPL, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_send_pair_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int N,
    const int32_t* __restrict__ node_slot, int64_t Tmax, u32x4* __restrict__ stage_x,
    int64_t* __restrict__ stage_idx, float* __restrict__ stage_w, int32_t* __restrict__ stage_src,
    int32_t* __restrict__ error_flag) {
    pair_scatter<WPL, false, kThreads>(x, topk_idx, topk_w, T, V, k, 0, node_slot, N, Tmax, Tmax, stage_x,
                             stage_idx, stage_w, stage_src, error_flag);
}

// The permute's small-batch form (k <= 64 slots, one pass per row): two tokens per wave as
// above. Slot j's weight is loaded by lane j with the slot row and read back with
// readlane, since the walk hands over a wave-uniform j.
template <int WPL, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_permute_pair_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ topk_w, int64_t T, int V, int k,
    const int32_t* __restrict__ expert_slot, u32x4* __restrict__ perm_x,
    float* __restrict__ perm_w, int32_t* __restrict__ perm_src, int64_t cap,
    int32_t* __restrict__ error_flag) {
    const int lane = lane_id();
    constexpr int kWpb = kThreads / kWave;
    const int64_t W = static_cast<int64_t>(gridDim.x) * kWpb;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWpb + threadIdx.x / kWave;
    if (t0 >= T) return;
    const int64_t t1 = t0 + W;
    const bool has1 = t1 < T;
    u32x4 a[WPL], b[WPL];
    load_row(a, x + t0 * V, 0, V);
    const int32_t s0 = lane < k ? expert_slot[t0 * k + lane] : -1;
    const float w0 = perm_w && lane < k ? topk_w[t0 * k + lane] : 0.0f;
    int32_t s1 = -1;
    float w1 = 0.0f;
    if (has1) {
        load_row(b, x + t1 * V, 0, V);
        s1 = lane < k ? expert_slot[t1 * k + lane] : -1;
        w1 = perm_w && lane < k ? topk_w[t1 * k + lane] : 0.0f;
    }
    int32_t errbits = 0;
    auto put = [&](const u32x4 (&v)[WPL], int64_t t, float w, int64_t qd, int j) {
        u32x4* row = perm_x + qd * V;
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int vi = i * kWave + lane;
            if (vi < V) store_row_word(row + vi, v[i]);
        }
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        if (lane == 0) {
            if (perm_w) perm_w[qd] = wj;
            if (perm_src) perm_src[qd] = static_cast<int32_t>(t);
        }
    };
    visit_chunk(s0, 0, 0, cap, errbits, [&](int64_t qd, int j) { put(a, t0, w0, qd, j); });
    if (has1) visit_chunk(s1, 0, 0, cap, errbits, [&](int64_t qd, int j) { put(b, t1, w1, qd, j); });
    if (errbits) raise_error(error_flag, errbits);
}

// Two-phase dispatch ("[PR #347] Feature/sm free normal kernel", section 2.1), send
// phase: each token's row, its k expert ids and weights and its id go once to every
// node holding one of its experts, at row node_slot[t][n] of node n's block of Tmax rows
// (the large per-node buffer that holds a whole batch, section 2.2.2).
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_send_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int N,
    const int32_t* __restrict__ node_slot, int64_t Tmax, u32x4* __restrict__ stage_x,
    int64_t* __restrict__ stage_idx, float* __restrict__ stage_w, int32_t* __restrict__ stage_src,
    int32_t* __restrict__ error_flag) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    int32_t errbits = 0;
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     stage_idx || stage_w);
    scatter_row<WPL, kMulti, false>(x + t * V, V, rt, 0, static_cast<int32_t>(t), node_slot + t * N, N,
                            Tmax, 0, Tmax, stage_x, stage_idx, stage_w, stage_src, errbits);
    if (errbits) raise_error(error_flag, errbits);
}

// Receive phase (the intra-node hop, same page, section 3.3.2): block (b, n) owns staged
// rows [W b, W b + W) of node n (W waves per block), one wave each; rows at or past count_n[n] are idle. A
// staged row goes to every rank of node n with a receive slot for its token, with that
// rank's view of the staged routing, exactly as the one-call dispatch writes it.
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_recv_kernel(
    const u32x4* __restrict__ stage_x, const int64_t* __restrict__ stage_idx,
    const float* __restrict__ stage_w, const int32_t* __restrict__ stage_src,
    const int32_t* __restrict__ count_n, int64_t Tmax, int64_t T, int V, int k, int R, int rpn,
    int er, const int32_t* __restrict__ token_slot, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag) {
    const int n = blockIdx.y;
    const int64_t s = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    int64_t cnt = count_n[n];
    int32_t errbits = 0;
    if (cnt < 0 || cnt > Tmax || cnt > T) {
        errbits |= kErrRecvOverflow;
        cnt = cnt < 0 ? 0 : (Tmax < T ? Tmax : T);
    }
    if (s < cnt) {
        const int64_t q = static_cast<int64_t>(n) * Tmax + s;
        const int64_t t = stage_src[q];
        if (t < 0 || t >= T) {
            errbits |= kErrSlotRange;
        } else {
            const Routing rt(stage_idx ? stage_idx + q * k : nullptr,
                             stage_w ? stage_w + q * k : nullptr, k, recv_idx || recv_w);
            scatter_row<WPL, kMulti, true>(stage_x + q * V, V, rt, er, static_cast<int32_t>(t),
                                   token_slot + t * R + n * rpn, rpn, 0, n * rpn, cap, recv_x,
                                   recv_idx, recv_w, recv_src, errbits);
        }
    }
    if (errbits && (s < cnt || s == 0)) raise_error(error_flag, errbits);
}

// FP8 dispatch: the same walk, but each token is first quantised once, in registers.
// Lane l of a pass owns the word pair (2 pi, 2 pi + 1), pi = 64 * pass + l: 16 channels,
// whose 16 codes leave as one 128-bit store. A group of 128 channels is 8 pairs, i.e. 8
// aligned lanes, so its largest |x| is reduced with three xor shuffles; scale = amax /
// 448, codes = e4m3(x * (448 / amax)) through the gfx950 packed fp8 convert (round to
// nearest even; the product is clamped to +-448, which only ever removes rounding
// excess above 448). Each destination row gets the codes as one burst of 128-bit
// stores and its H/128 scales (one lane per group). Against one word per lane (64-bit
// code stores, a 16-lane reduction) this measured 5% faster on MI355X at 4096 x 7168.
template <int WPP, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int R, int er,
    const int32_t* __restrict__ token_slot, u32x4* __restrict__ recv_codes,
    float* __restrict__ recv_scales, int64_t* __restrict__ recv_idx, float* __restrict__ recv_w,
    int32_t* __restrict__ recv_src, int64_t cap, int32_t* __restrict__ error_flag) {
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const int P2 = V / 2;  // word pairs per row (V % 16 == 0)
    const int G = V / 16;  // scale groups per row
    const bool meta = recv_idx || recv_w;
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     meta);
    const u32x4* xr = x + t * V;
    int32_t errbits = 0;

    for (int p0 = 0; p0 < P2; p0 += kWave * WPP) {
        u32x4 code[WPP];
        float scale[WPP];
        {
            u32x4 v[2 * WPP];
#pragma unroll
            for (int i = 0; i < WPP; ++i) {
                const int pi = p0 + i * kWave + lane;
                if (pi < P2) {
                    v[2 * i] = load_stream(xr + 2 * pi);
                    v[2 * i + 1] = load_stream(xr + 2 * pi + 1);
                }
            }
#pragma unroll
            for (int i = 0; i < WPP; ++i) {
                const int pi = p0 + i * kWave + lane;
                float f[16];
                float amax = 0.0f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t wq = pi < P2 ? v[2 * i + h][q] : 0u;
                        f[8 * h + 2 * q] = __uint_as_float(wq << 16);
                        f[8 * h + 2 * q + 1] = __uint_as_float(wq & 0xffff0000u);
                        amax = fmaxf(amax, fmaxf(fabsf(f[8 * h + 2 * q]), fabsf(f[8 * h + 2 * q + 1])));
                    }
                }
#pragma unroll
                for (int m = 4; m >= 1; m >>= 1)
                    amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
                const float inv = amax > 0.0f ? 448.0f / amax : 1.0f;
                scale[i] = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float c[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        c[u] = fminf(fmaxf(f[4 * q + u] * inv, -448.0f), 448.0f);
                    const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
                    code[i][q] = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], wd, true));
                }
            }
        }
        for_each_destination(token_slot + t * R, R, 0, cap, errbits, [&](int64_t sd, int rd) {
            u32x4* row = recv_codes + sd * P2;
            float* srow_out = recv_scales + sd * G;
#pragma unroll
            for (int i = 0; i < WPP; ++i) {
                const int pi = p0 + i * kWave + lane;
                if (pi < P2) {
                    store_stream(row + pi, code[i]);
                    if ((lane & 7) == 0) srow_out[pi / 8] = scale[i];
                }
            }
            if (p0 != 0) return;
            if (meta) rt.write<true>(sd, rd, er, recv_idx, recv_w);
            if (recv_src && lane == 0) recv_src[sd] = static_cast<int32_t>(t);
        });
        if constexpr (!kMulti) break;
    }
    if (errbits) raise_error(error_flag, errbits);
}

// Dispatch + permute: the token row goes once to each of its (token, slot) rows in the
// expert-major order (expert_slot from the layout), with the slot's weight and the
// source token. Same wave-per-token walk, over the k expert_slot entries.
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_permute_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ topk_w, int64_t T, int V, int k,
    const int32_t* __restrict__ expert_slot, u32x4* __restrict__ perm_x,
    float* __restrict__ perm_w, int32_t* __restrict__ perm_src, int64_t cap,
    int32_t* __restrict__ error_flag) {
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const u32x4* xr = x + t * V;
    int32_t errbits = 0;
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        u32x4 v[WPL];
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int vi = v0 + i * kWave + lane;
            if (vi < V) v[i] = load_stream(xr + vi);
        }
        for_each_destination(expert_slot + t * k, k, 0, cap, errbits, [&](int64_t qd, int j) {
            u32x4* row = perm_x + qd * V;
#pragma unroll
            for (int i = 0; i < WPL; ++i) {
                const int vi = v0 + i * kWave + lane;
                if (vi < V) store_row_word(row + vi, v[i]);
            }
            if (v0 == 0 && lane == 0) {
                if (perm_w) perm_w[qd] = topk_w[t * k + j];
                if (perm_src) perm_src[qd] = static_cast<int32_t>(t);
            }
        });
        if constexpr (!kMulti) break;
    }
    if (errbits) raise_error(error_flag, errbits);
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

hipError_t launch_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                           int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                           void* recv_x, int64_t* recv_idx, float* recv_w, int32_t* recv_src,
                           int64_t cap, int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    if (V <= 14 * kWave && R <= kWave && k <= kWave && T <= resident_token_waves()) {
        constexpr int kPT = kPairThreads;
        const int64_t waves = (T + 1) / 2;
        const int64_t pgrid = (waves + kPT / kWave - 1) / (kPT / kWave);
        return with_row_width<14, false>(V, [&](auto wpl, auto) {
            hipLaunchKernelGGL((dispatch_pair_kernel<decltype(wpl)::value, kPT>),
                               dim3(static_cast<unsigned>(pgrid)), dim3(kPT), 0, stream,
                               static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, R, E / R,
                               token_slot, static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src,
                               cap, error_flag);
        });
    }
    constexpr int kThreads = kRowThreads;
    const int64_t grid = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (!grid_fits(grid, kThreads)) return hipErrorInvalidConfiguration;
    return with_row_width<14, true>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((dispatch_kernel<decltype(wpl)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, R, E / R,
                           token_slot, static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src,
                           cap, error_flag);
    });
}

hipError_t launch_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_w,
                               int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                               void* recv_codes, float* recv_scales, int64_t* recv_idx,
                               float* recv_w, int32_t* recv_src, int64_t cap, int32_t* error_flag,
                               hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    constexpr int kThreads = kFp8Threads;
    const int64_t grid = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (!grid_fits(grid, kThreads)) return hipErrorInvalidConfiguration;
    // word pairs per lane: 7 covers a 7168-wide row in one pass
    return with_row_width<7, false>(V / 2, [&](auto wpp, auto multi) {
        hipLaunchKernelGGL((dispatch_fp8_kernel<decltype(wpp)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, R, E / R,
                           token_slot, static_cast<u32x4*>(recv_codes), recv_scales, recv_idx,
                           recv_w, recv_src, cap, error_flag);
    });
}

hipError_t launch_dispatch_permute(const void* x, const float* topk_w, int64_t T, int H, int k,
                                   const int32_t* expert_slot, void* perm_x, float* perm_w,
                                   int32_t* perm_src, int64_t cap, int32_t* error_flag,
                                   hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    if (V <= 14 * kWave && k <= kWave && T <= resident_token_waves()) {
        constexpr int kPT = kPairThreads;
        const int64_t waves = (T + 1) / 2;
        const int64_t pgrid = (waves + kPT / kWave - 1) / (kPT / kWave);
        return with_row_width<14, false>(V, [&](auto wpl, auto) {
            hipLaunchKernelGGL((dispatch_permute_pair_kernel<decltype(wpl)::value, kPT>),
                               dim3(static_cast<unsigned>(pgrid)), dim3(kPT), 0, stream,
                               static_cast<const u32x4*>(x), topk_w, T, V, k, expert_slot,
                               static_cast<u32x4*>(perm_x), perm_w, perm_src, cap, error_flag);
        });
    }
    constexpr int kThreads = kRowThreads;
    const int64_t grid = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (!grid_fits(grid, kThreads)) return hipErrorInvalidConfiguration;
    return with_row_width<14, true>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((dispatch_permute_kernel<decltype(wpl)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_w, T, V, k, expert_slot,
                           static_cast<u32x4*>(perm_x), perm_w, perm_src, cap, error_flag);
    });
}

hipError_t launch_dispatch_send(const void* x, const int64_t* topk_idx, const float* topk_w,
                                int64_t T, int H, int k, int N, const int32_t* node_slot,
                                int64_t Tmax, void* stage_x, int64_t* stage_idx, float* stage_w,
                                int32_t* stage_src, int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    if (V <= 14 * kWave && N <= kWave && k <= kWave && T <= resident_token_waves()) {
        constexpr int kPT = kPairThreads;
        const int64_t waves = (T + 1) / 2;
        const int64_t pgrid = (waves + kPT / kWave - 1) / (kPT / kWave);
        return with_row_width<14, false>(V, [&](auto wpl, auto) {
            hipLaunchKernelGGL((dispatch_send_pair_kernel<decltype(wpl)::value, kPT>),
                               dim3(static_cast<unsigned>(pgrid)), dim3(kPT), 0, stream,
                               static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, N,
                               node_slot, Tmax, static_cast<u32x4*>(stage_x), stage_idx, stage_w,
                               stage_src, error_flag);
        });
    }
    constexpr int kThreads = kRowThreads;
    const int64_t grid = (T + kThreads / kWave - 1) / (kThreads / kWave);
    if (!grid_fits(grid, kThreads)) return hipErrorInvalidConfiguration;
    return with_row_width<14, true>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((dispatch_send_kernel<decltype(wpl)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, N, node_slot,
                           Tmax, static_cast<u32x4*>(stage_x), stage_idx, stage_w, stage_src,
                           error_flag);
    });
}

hipError_t launch_dispatch_recv(const void* stage_x, const int64_t* stage_idx,
                                const float* stage_w, const int32_t* stage_src,
                                const int32_t* count_n, int N, int64_t Tmax, int H, int k, int E,
                                int R, const int32_t* token_slot, int64_t T, void* recv_x,
                                int64_t* recv_idx, float* recv_w, int32_t* recv_src, int64_t cap,
                                int32_t* error_flag, hipStream_t stream) {
    const int64_t rows = std::min(T, Tmax);  // a node holds at most min(T, Tmax) rows
    if (rows == 0) return hipSuccess;
    const int V = H / 8;
    constexpr int kThreads = kRecvThreads;
    const int64_t bx = (rows + kThreads / kWave - 1) / (kThreads / kWave);
    if (!grid_fits(bx * N, kThreads) || N > 65535) return hipErrorInvalidConfiguration;
    return with_row_width<14, false>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((dispatch_recv_kernel<decltype(wpl)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(bx), N), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(stage_x), stage_idx, stage_w, stage_src,
                           count_n, Tmax, T, V, k, R, R / N, E / R, token_slot,
                           static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src, cap,
                           error_flag);
    });
}

}  // namespace ep
