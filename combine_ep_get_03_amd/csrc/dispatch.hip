// dispatch.hip -- dispatch permute on gfx950.
//
// Every (token, rank) pair with a receive slot s gets row s of recv_x = the token's bf16
// row, plus the rank's view of the token's top-k routing and the token id. On one GPU
// the intra-node hop of the pages ("[PR #347] Feature/sm free normal kernel", section
// 3.3.2) is an HBM-to-HBM copy, and rows are written straight to their final place with
// no staging buffer (the zero-copy idea of "[PR #453] ... Zero-Copy and TMA Offloading").
//
// Design: one wave64 per (token, destination). Wave (t, d) finds token t's d-th
// destination (a ballot over its token_slot row, ascending column), loads the row into
// registers (up to 14 128-bit words per lane, so a 7168-wide bf16 row is one pass, all
// loads in flight at once), writes it to that destination as one sequential burst of
// non-temporal 128-bit stores with the destination's view of the routing, and exits.
// No LDS and no block barrier. A launch holds about one short-lived wave per receive
// row, so the hardware dispatches waves over a sliding range of tokens and the rows
// being written at any moment stay close together in the receive buffer. A token's
// waves are dispatched next to each other and read its row with plain (cached) loads:
// with 4 waves per block, a top-8 token's waves fill two neighbouring blocks, which the
// hardware deals to two XCDs, so each of those L2s fetches the row once (counters: twice
// the row bytes are read) and the token's other waves hit. Remapping block indices so
// both blocks share an XCD, to save the second fetch, ran 3-6% slower, and 512-thread
// blocks (one block per token) ran 4-6% slower; non-temporal row loads, which miss for
// every wave, ran 30% slower in a probe of the same form. One wave per token (all its
// destinations in turn) ran 13-19% slower on MI355X from 4096 to 16384 tokens of 7168
// channels, top-8, because the whole resident grid then writes across the whole buffer
// at once. HBM-write bound. The expert-major permute uses the same form; the FP8
// dispatch and the two-phase send phase give each wave a range of a token's destinations
// (at most one block of waves per token), and the receive phase two waves per staged row
// (each measured faster that way, see their kernels).
#include <type_traits>

#include "dispatch_rows.hpp"

namespace ep {
namespace {

// Launch shapes, chosen by same-box A/B timing on MI355X at 1024 to 16384 tokens of 7168
// channels, top-8: 256-thread blocks for every dispatch kernel (4-6% faster than 512 at
// every size but the smallest, 20-35% faster than 128).
constexpr int kDestThreads = 256;
constexpr int kRecvThreads = 256;
constexpr int kRecvWavesPerRow = 2;  // waves per staged row in the receive phase
// Waves per launch of a (token, destination) kernel; larger batches are split over token
// ranges, so a wave's index stays a 32-bit value and one launch stays far below the
// dispatch packet's 2^32 work-item limit.
constexpr int64_t kDestMaxWaves = int64_t{1} << 22;
// The FP8 dispatch and the send phase give a token at most one block of waves (several
// destinations per wave when it has more): same-box A/B on MI355X at 7168 channels, top-8,
// FP8 over 32 ranks 45 against 68 us with one wave per destination, send over 8 nodes
// 232 against 258 us at 16384 tokens. The one-call dispatch and the permute keep one
// destination per wave, which measured faster for them (78.7 against 82.8 us at 4096).
constexpr int kMaxWavesPerToken = kDestThreads / kWave;

// A wave's share of a token's destinations: the destinations with index in [lo, hi),
// in ascending column order (hi = INT32_MAX for the token's last wave, which so also takes
// every destination past the expected count: a caller-built slot table may have more
// valid entries in a row). s_first is the calling lane's entry of the slot row's first 64
// columns, loaded before the routing and the row so the ballot waits only for it.
template <typename Visit>
__device__ __forceinline__ void visit_destinations(int32_t s_first, const int32_t* __restrict__ srow,
                                                   int C, int64_t cbase, int64_t cap, int lo, int hi,
                                                   int32_t& errbits, Visit&& visit) {
    const int lane = lane_id();
    int seen = 0;
    for (int c0 = 0; c0 < C; c0 += kWave) {
        int32_t s = c0 == 0 ? s_first : (c0 + lane < C ? srow[c0 + lane] : -1);
        if (s >= cap) {
            errbits |= kErrRecvOverflow;
            s = -1;
        }
        uint64_t m = wave_ballot(s >= 0);
        while (m && seen < lo) {  // destinations before lo belong to other waves
            m &= m - 1;
            ++seen;
        }
        while (m) {
            if (seen >= hi) return;
            const int src_lane = __builtin_ctzll(m);
            m &= m - 1;
            ++seen;
            const int cd = c0 + src_lane;
            visit(static_cast<int64_t>(__builtin_amdgcn_readlane(s, src_lane)) + cd * cbase, cd);
        }
    }
}

// The destination range of wave d of D, P destinations each; the last wave's is open.
__device__ __forceinline__ void dest_range(int d, int D, int P, int& lo, int& hi) {
    lo = d * P;
    hi = d == D - 1 ? INT32_MAX : lo + P;
}

// Token t's row to destination d of its slot row: rank c's view of the routing with
// kRankView (c = the destination's column), else the routing unchanged.
template <int WPL, bool kMulti, bool kRankView>
__device__ __forceinline__ void dest_scatter(
    int p, const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int er,
    const int32_t* __restrict__ slot_tab, int C, int64_t cbase, int64_t cap, FastDiv D, int P,
    u32x4* __restrict__ dst_x, int64_t* __restrict__ dst_idx, float* __restrict__ dst_w,
    int32_t* __restrict__ dst_src, int32_t* __restrict__ error_flag) {
    int64_t t;
    int d;
    if (!dest_wave_at(p, t0, t_end, D, t, d)) return;
    const int lane = lane_id();
    const int32_t* srow = slot_tab + t * C;
    const int32_t s_first = lane < C ? srow[lane] : -1;
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     dst_idx || dst_w);
    const u32x4* xr = x + t * V;
    int lo, hi;
    dest_range(d, D.d, P, lo, hi);
    int32_t errbits = 0;
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        u32x4 v[WPL];
        load_row_cached(v, xr, v0, V);
        visit_destinations(s_first, srow, C, cbase, cap, lo, hi, errbits, [&](int64_t sd, int cd) {
            put_row<WPL, kRankView>(v, v0, V, sd, cd, rt, er, static_cast<int32_t>(t), dst_x,
                                    dst_idx, dst_w, dst_src);
        });
        if constexpr (!kMulti) break;
    }
    if (errbits) raise_error(error_flag, errbits);
}

template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int R, int er,
    const int32_t* __restrict__ token_slot, FastDiv D, int P, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag) {
    dest_scatter<WPL, kMulti, true>(grid_wave<kThreads>(), x, topk_idx, topk_w, t0, t_end, V, k,
                                    er, token_slot, R, 0, cap, D, P, recv_x, recv_idx, recv_w,
                                    recv_src, error_flag);
}

// The rank, node and expert counts and offsets of the counts path, from the count
// launch's per-block tables: head block h of ep_dispatch_layout's first launch takes expert
// columns [256 h, 256 h + 256). A column sum of the blocks' inclusive expert prefixes is
// expert_offset[e + 1]; the count is its difference with the column before, which each
// thread sums as well (no LDS, no barrier: the dispatch kernel stays free of both). Head
// block 0 also sums the node columns, and its first wave the rank columns (lane r), whose
// scan across the wave gives the rank offsets.
__device__ __forceinline__ void counts_head_block(const CountsWorkspace& cw, int h, int nb,
                                                  int E, int R, int N,
                                                  int32_t* __restrict__ count_r,
                                                  int32_t* __restrict__ rank_offset,
                                                  int32_t* __restrict__ count_n,
                                                  int32_t* __restrict__ count_e,
                                                  int32_t* __restrict__ expert_offset) {
    constexpr int kB = 8;  // loads in flight per lane
    const int tid = threadIdx.x;
    if (h == 0 && tid < kWave && (count_r || rank_offset)) {
        int tot = 0;
        for (int b0 = 0; b0 < nb; b0 += kB) {
            int v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u)
                v[u] = (b0 + u < nb && tid < R) ? cw.blk_rank[static_cast<int64_t>(b0 + u) * R + tid] : 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) tot += v[u];
        }
        int x = tot;  // inclusive scan over the wave
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(x, d, kWave);
            if (tid >= d) x += y;
        }
        if (tid < R) {
            if (count_r) count_r[tid] = tot;
            if (rank_offset) rank_offset[tid] = x - tot;
        }
        if (tid == kWave - 1 && rank_offset) rank_offset[R] = x;
    }
    const int e = h * kDestThreads + tid;
    if ((count_e || expert_offset) && e < E) {
        int sum = 0, before = 0;  // column e, and column e - 1 (0 for e = 0)
        for (int b0 = 0; b0 < nb; b0 += kB) {
            int v[kB], u0[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const int64_t row = static_cast<int64_t>(b0 + u) * E;
                v[u] = b0 + u < nb ? cw.blk_exp[row + e] : 0;
                u0[u] = (b0 + u < nb && e > 0) ? cw.blk_exp[row + e - 1] : 0;
            }
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                sum += v[u];
                before += u0[u];
            }
        }
        if (expert_offset) {
            expert_offset[e + 1] = sum;
            if (e == 0) expert_offset[0] = 0;
        }
        if (count_e) count_e[e] = sum - before;
    }
    if (h == 0 && count_n && tid < N) {
        int sum = 0;
        for (int bb = 0; bb < nb; ++bb) sum += cw.blk_node[static_cast<int64_t>(bb) * N + tid];
        count_n[tid] = sum;
    }
}

// glob[b][lane] for a batch of at most kCountsLocalBlocks blocks: the receive row of
// block b's first token on rank `lane`, from that rank's count in every block (cnt[u],
// loaded by the caller): the rank's offset (a scan of the rank totals across the wave)
// plus its counts in the blocks before b.
__device__ __forceinline__ int32_t local_glob(const int (&cnt)[kCountsLocalBlocks], int64_t b) {
    int tot = 0, g = 0;
#pragma unroll
    for (int u = 0; u < kCountsLocalBlocks; ++u) {
        tot += cnt[u];
        if (u < b) g += cnt[u];
    }
    int x = tot;  // inclusive scan of the rank totals across the wave
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane_id() >= d) x += y;
    }
    return g + x - tot;
}

// Dispatch of the counts path (R <= 64): the same (token, destination) waves as
// dispatch_kernel, but the receive rows come from the count launch's tables instead of a
// token_slot row. Lane r < R holds, for rank r: the receive row of the token's block's
// first token on r, the count of the block's earlier waves' tokens on r, and the ballot
// of the token's wave for r; these loads, the token's rank mask (one word) and the row's
// loads are all issued together. The token's row on rank r is then
//     glob[b][r] + pfx[b][w][r] + popcount(ball[b][w][r] & (bits below the token)),
// so a wave waits on one memory round trip before its stores, as dispatch_kernel does.
// With kLocal (batches of at most kCountsLocalBlocks blocks, whose count launch has no
// cross-block phase), lane r instead loads rank r's count in every block (at most 16
// loads, issued with the rest) and forms glob[b][r] itself: the rank offset (a scan of the
// totals across the wave) plus the counts of the blocks before b.
// The token's first wave also writes the token's token_slot row and bitmap row. The first
// `nhead` blocks are head blocks (counts_head_block) instead.
template <int WPL, bool kMulti, bool kLocal, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_layout_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int R, int er,
    CountsWorkspace cw, FastDiv D, int32_t* __restrict__ token_slot,
    uint8_t* __restrict__ in_rank, u32x4* __restrict__ recv_x, int64_t* __restrict__ recv_idx,
    float* __restrict__ recv_w, int32_t* __restrict__ recv_src, int64_t cap, int nhead, int nb,
    int E, int N, int32_t* __restrict__ count_r, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ count_n, int32_t* __restrict__ count_e,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ error_flag) {
    if (static_cast<int>(blockIdx.x) < nhead) {
        counts_head_block(cw, blockIdx.x, nb, E, R, N, count_r, rank_offset, count_n, count_e,
                          expert_offset);
        return;
    }
    int64_t t;
    int d;
    if (!dest_wave_at(grid_wave<kThreads>() - nhead * (kThreads / kWave), t0, t_end, D, t, d))
        return;
    const int lane = lane_id();
    constexpr int kBlk = kLayoutBlockTokens;
    const int64_t b = t / kBlk;
    const int w = static_cast<int>(t % kBlk) / kWave;
    const int l = static_cast<int>(t % kWave);
    const uint64_t m = cw.mask[t];
    int32_t g = 0, pf = 0;
    uint64_t bl = 0;
    int cnt[kLocal ? kCountsLocalBlocks : 1];  // rank `lane`'s count in each block
    if constexpr (kLocal) {
#pragma unroll
        for (int u = 0; u < kCountsLocalBlocks; ++u)
            cnt[u] = (u < nb && lane < R) ? cw.blk_rank[u * R + lane] : 0;
    } else if (lane < R) {
        g = cw.glob[b * R + lane];
    }
    if (lane < R) {
        const int64_t cell = (b * (kBlk / kWave) + w) * R + lane;
        pf = cw.pfx[cell];
        bl = cw.ball[cell];
    }
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     recv_idx || recv_w);
    const u32x4* xr = x + t * V;
    u32x4 v[WPL];
    load_row_cached(v, xr, 0, V);  // first pass, issued with the tables' loads
    if constexpr (kLocal) g = local_glob(cnt, b);  // the counts arrive with the tables
    const bool on = lane < R && ((m >> lane) & 1ull);
    const int32_t slot = on ? g + pf + __popcll(bl & ((1ull << l) - 1ull)) : -1;
    if (d == 0 && lane < R) {
        token_slot[t * R + lane] = slot;
        if (in_rank) in_rank[t * R + lane] = on ? 1 : 0;
    }
    uint64_t rest = m;  // the token's d-th destination rank, ascending
    for (int i = 0; i < d && rest; ++i) rest &= rest - 1;
    if (!rest) return;
    const int rd = __builtin_ctzll(rest);
    const int64_t sd = __builtin_amdgcn_readlane(slot, rd);
    if (sd < 0 || sd >= cap) {  // (a negative row only comes from tables of a misused workspace)
        if (lane == 0) raise_error(error_flag, kErrRecvOverflow);
        return;
    }
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        if (v0 != 0) load_row_cached(v, xr, v0, V);
        put_row<WPL, true>(v, v0, V, sd, rd, rt, er, static_cast<int32_t>(t), recv_x, recv_idx,
                           recv_w, recv_src);
        if constexpr (!kMulti) break;
    }
}

// ep_get_layout's second launch for a batch of 2 to kCountsLocalBlocks blocks (R <= 64, no
// node or expert slots), after the counts path's count launch: one wave per token writes
// its token_slot and bitmap rows from the count launch's tables, each row formed as the
// counts path's dispatch forms it; the first `nhead` blocks are head blocks
// (counts_head_block: the counts and offsets).
template <int kThreads>
__global__ __launch_bounds__(kThreads) void counts_slots_kernel(
    int64_t T, int R, CountsWorkspace cw, int32_t* __restrict__ token_slot,
    uint8_t* __restrict__ in_rank, int nhead, int nb, int E, int N,
    int32_t* __restrict__ count_r, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ count_n, int32_t* __restrict__ count_e,
    int32_t* __restrict__ expert_offset) {
    if (static_cast<int>(blockIdx.x) < nhead) {
        counts_head_block(cw, blockIdx.x, nb, E, R, N, count_r, rank_offset, count_n, count_e,
                          expert_offset);
        return;
    }
    const int64_t t = grid_wave<kThreads>() - nhead * (kThreads / kWave);
    if (t >= T) return;
    const int lane = lane_id();
    constexpr int kBlk = kLayoutBlockTokens;
    const int64_t b = t / kBlk;
    const int w = static_cast<int>(t % kBlk) / kWave;
    const int l = static_cast<int>(t % kWave);
    const uint64_t m = cw.mask[t];
    int cnt[kCountsLocalBlocks];  // rank `lane`'s count in each block
#pragma unroll
    for (int u = 0; u < kCountsLocalBlocks; ++u)
        cnt[u] = (u < nb && lane < R) ? cw.blk_rank[u * R + lane] : 0;
    int32_t pf = 0;
    uint64_t bl = 0;
    if (lane < R) {
        const int64_t cell = (b * (kBlk / kWave) + w) * R + lane;
        pf = cw.pfx[cell];
        bl = cw.ball[cell];
    }
    const int32_t g = local_glob(cnt, b);
    const bool on = lane < R && ((m >> lane) & 1ull);
    if (lane < R) {
        token_slot[t * R + lane] = on ? g + pf + __popcll(bl & ((1ull << l) - 1ull)) : -1;
        if (in_rank) in_rank[t * R + lane] = on ? 1 : 0;
    }
}

// Dispatch + permute of the counts path (at most kCountsPermuteBlocks 256-token blocks):
// wave (t, j) forms pair (t, j)'s expert-major row itself, as expert_offset[e] + the pairs
// naming e in the blocks before t's block + the pair's rank in its own block (the count
// launch's expert_rank). Lane u < nb loads block u's inclusive expert prefix at e and at
// e - 1: summed over every block, the prefix at e - 1 is expert_offset[e]; summed over the
// blocks before t's, the difference is the second term. The pair's id and rank are loaded
// with the row's first pass, the prefixes once the id has arrived. The first `nhead`
// blocks are head blocks (the expert counts and offsets).
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_permute_layout_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int E, int N,
    const int32_t* __restrict__ expert_rank, CountsWorkspace cw, int nb, FastDiv D,
    u32x4* __restrict__ perm_x, float* __restrict__ perm_w, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ expert_slot, int64_t cap, int nhead, int32_t* __restrict__ count_e,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ error_flag) {
    if (static_cast<int>(blockIdx.x) < nhead) {
        counts_head_block(cw, blockIdx.x, nb, E, 0, N, nullptr, nullptr, nullptr, count_e,
                          expert_offset);
        return;
    }
    int64_t t;
    int j;
    if (!dest_wave_at(grid_wave<kThreads>() - nhead * (kThreads / kWave), t0, t_end, D, t, j))
        return;
    const int lane = lane_id();
    const int64_t pair = t * k + j;
    const int64_t e = topk_idx[pair];
    const int rk = expert_rank[pair];
    const float w = perm_w ? topk_w[pair] : 0.0f;
    const u32x4* xr = x + t * V;
    u32x4 v[WPL];
    load_row_cached(v, xr, 0, V);  // first pass, issued with the pair's loads
    if (e < 0 || e >= E) {         // masked (or bad: the count launch flagged it)
        if (expert_slot && lane == 0) expert_slot[pair] = -1;
        return;
    }
    const int ei = static_cast<int>(e);
    const int64_t b = t / kLayoutBlockTokens;
    int cur = 0, prev = 0;
    if (lane < nb) {
        cur = cw.blk_exp[static_cast<int64_t>(lane) * E + ei];
        prev = ei > 0 ? cw.blk_exp[static_cast<int64_t>(lane) * E + ei - 1] : 0;
    }
    int before = lane < b ? cur - prev : 0;
    int off = prev;
#pragma unroll
    for (int s = kWave / 2; s > 0; s >>= 1) {
        before += __shfl_xor(before, s, kWave);
        off += __shfl_xor(off, s, kWave);
    }
    const int64_t q = static_cast<int64_t>(off) + before + rk;
    if (expert_slot && lane == 0) expert_slot[pair] = static_cast<int32_t>(q);
    if (q >= cap) {
        if (lane == 0) raise_error(error_flag, kErrRecvOverflow);
        return;
    }
    u32x4* row = perm_x + q * V;
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        if (v0 != 0) load_row_cached(v, xr, v0, V);
        store_row_pass(row, V, v0, v);
        if constexpr (!kMulti) break;
    }
    if (lane == 0) {
        if (perm_w) perm_w[q] = w;
        if (perm_src) perm_src[q] = static_cast<int32_t>(t);
    }
}

// Two-phase dispatch ("[PR #347] Feature/sm free normal kernel", section 2.1), send
// phase: each token's row, its k expert ids and weights and its id go once to every
// node holding one of its experts, at row node_slot[t][n] of node n's block of Tmax rows
// (the large per-node buffer that holds a whole batch, section 2.2.2). Wave (t, d) takes
// the token's nodes [d P, d P + P), with P chosen so a token has at most one block of waves.
// The grid may be smaller than one wave per (t, d): each wave then takes (t, d) pairs
// p, p + W, p + 2W, ... (W = the grid's waves), so the send occupies a bounded part of
// the GPU and leaves the rest to work on other queues (the page's hook mode frees SMs for
// compute while the data moves, section 2.2.2).
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_send_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int N,
    const int32_t* __restrict__ node_slot, int64_t Tmax, FastDiv D, int P, u32x4* __restrict__ stage_x,
    int64_t* __restrict__ stage_idx, float* __restrict__ stage_w, int32_t* __restrict__ stage_src,
    int32_t* __restrict__ error_flag) {
    const int nw = static_cast<int>((t_end - t0) * D.d);
    const int stride = static_cast<int>(gridDim.x) * (kThreads / kWave);
    for (int p = grid_wave<kThreads>(); p < nw; p += stride)
        dest_scatter<WPL, kMulti, false>(p, x, topk_idx, topk_w, t0, t_end, V, k, 0, node_slot, N,
                                         Tmax, Tmax, D, P, stage_x, stage_idx, stage_w, stage_src,
                                         error_flag);
}

// Dispatch + permute: token t's row goes to each of its (token, slot) rows in the
// expert-major order (expert_slot from the layout), with the slot's weight and the source
// token. Wave (t, j) takes slot j (D = k), if it is routed. The row's loads are issued
// before the slot arrives: 4% faster at 4096 x 7168 on MI355X, unchanged at 16384.
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_permute_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ topk_w, int64_t t0, int64_t t_end,
    int V, int k, const int32_t* __restrict__ expert_slot, FastDiv D, u32x4* __restrict__ perm_x,
    float* __restrict__ perm_w, int32_t* __restrict__ perm_src, int64_t cap,
    int32_t* __restrict__ error_flag) {
    int64_t t;
    int j;
    if (!dest_wave<kThreads>(t0, t_end, D, t, j)) return;
    const int lane = lane_id();
    const int64_t q = expert_slot[t * k + j];
    const float w = perm_w ? topk_w[t * k + j] : 0.0f;
    const u32x4* xr = x + t * V;
    u32x4 v[WPL];
    load_row_cached(v, xr, 0, V);  // first pass, issued before the slot is known
    if (q < 0) return;
    if (q >= cap) {
        if (lane == 0) raise_error(error_flag, kErrRecvOverflow);
        return;
    }
    u32x4* row = perm_x + q * V;
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        if (v0 != 0) load_row_cached(v, xr, v0, V);
        store_row_pass(row, V, v0, v);
        if constexpr (!kMulti) break;
    }
    if (lane == 0) {
        if (perm_w) perm_w[q] = w;
        if (perm_src) perm_src[q] = static_cast<int32_t>(t);
    }
}

// Receive phase (the intra-node hop, same page, section 3.3.2): a staged row goes to every
// rank of node n with a receive slot for its token, with that rank's view of the staged
// routing, exactly as the one-call dispatch writes it. Block (b, n) holds waves p of node
// n; wave p takes staged row s = p / D of node n and its destinations [d P, d P + P),
// d = p % D, with D = 2 waves per staged row (the second wave reads the row from L2).
// The wave issues the staged row's loads before the chain that the destinations need
// (staged token id, then its slot row), so the two overlap. Measured on MI355X at 7168
// channels, top-8 over 32 ranks on 4 nodes (about two destinations per staged row): 94.8
// against 119.6 us for one wave per staged row that loaded the row after the chain; with
// the new load order, one wave per staged row ran 95.0 at 4096 tokens but 582.6 against
// 544.9 at 16384 over 64 ranks on 8 nodes, and one wave per destination (8 per staged
// row, most idle) 131.6.
template <int WPL, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_recv_kernel(
    const u32x4* __restrict__ stage_x, const int64_t* __restrict__ stage_idx,
    const float* __restrict__ stage_w, const int32_t* __restrict__ stage_src,
    const int32_t* __restrict__ count_n, int64_t Tmax, int64_t T, int V, int k, int R, int rpn,
    int er, const int32_t* __restrict__ token_slot, FastDiv D, int P, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag) {
    const int n = blockIdx.y;
    const int lane = lane_id();
    const int p = static_cast<int>(blockIdx.x) * (kThreads / kWave) + static_cast<int>(threadIdx.x) / kWave;
    const int q0 = D.div(p);
    const int64_t s = q0;
    const int d = p - q0 * D.d;
    int64_t cnt = count_n[n];
    int32_t errbits = 0;
    if (cnt < 0 || cnt > Tmax || cnt > T) {
        errbits |= kErrRecvOverflow;
        cnt = cnt < 0 ? 0 : (Tmax < T ? Tmax : T);
    }
    if (s < cnt) {
        const int64_t q = static_cast<int64_t>(n) * Tmax + s;
        const u32x4* xr = stage_x + q * V;
        u32x4 v[WPL];
        load_row_cached(v, xr, 0, V);  // first pass, issued before the token-id chain
        const int64_t t = stage_src[q];
        if (t < 0 || t >= T) {
            errbits |= kErrSlotRange;
        } else {
            const int32_t* srow = token_slot + t * R + static_cast<int64_t>(n) * rpn;
            const int32_t s_first = lane < rpn ? srow[lane] : -1;
            const Routing rt(stage_idx ? stage_idx + q * k : nullptr,
                             stage_w ? stage_w + q * k : nullptr, k, recv_idx || recv_w);
            int lo, hi;
            dest_range(d, D.d, P, lo, hi);
            for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
                if (v0 != 0) load_row_cached(v, xr, v0, V);
                visit_destinations(s_first, srow, rpn, 0, cap, lo, hi, errbits,
                                   [&](int64_t sd, int cd) {
                    put_row<WPL, true>(v, v0, V, sd, n * rpn + cd, rt, er,
                                       static_cast<int32_t>(t), recv_x, recv_idx, recv_w,
                                       recv_src);
                });
                if constexpr (!kMulti) break;
            }
        }
    }
    if (errbits && (s < cnt || (s == 0 && d == 0))) raise_error(error_flag, errbits);
}

// One pass of a row's FP8 quantisation: lane l owns the word pair pi = p0 + 64 i + l
// (16 channels) of every i < WPP; code[i] gets its 16 e4m3 codes and scale[i] its group's
// scale (one group of 128 channels = 8 aligned lanes).
template <int WPP>
__device__ __forceinline__ void quantize_fp8_pass(const u32x4* __restrict__ xr, int p0, int P2,
                                                  u32x4 (&code)[WPP], float (&scale)[WPP]) {
    const int lane = lane_id();
    u32x4 v[2 * WPP];
#pragma unroll
    for (int i = 0; i < WPP; ++i) {
        const int pi = p0 + i * kWave + lane;
        if (pi < P2) {
            v[2 * i] = xr[2 * pi];  // cached: the token's other waves hit in L2
            v[2 * i + 1] = xr[2 * pi + 1];
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

// One pass of FP8 codes and scales into destination row sd; the first pass also writes
// rank rd's view of the routing and the source id.
template <int WPP>
__device__ __forceinline__ void put_fp8_row(const u32x4 (&code)[WPP], const float (&scale)[WPP],
                                            int p0, int P2, int G, int64_t sd, int rd,
                                            const Routing& rt, int er, int32_t src,
                                            u32x4* __restrict__ recv_codes,
                                            float* __restrict__ recv_scales,
                                            int64_t* __restrict__ recv_idx,
                                            float* __restrict__ recv_w,
                                            int32_t* __restrict__ recv_src) {
    const int lane = lane_id();
    // Guarded non-temporal stores: the bf16 rows' unguarded device-scope stores, tried for
    // the codes, made this dispatch slower (48.6 against 45.5-46.6 us at 4096 tokens,
    // top-8 over 32 ranks, 7168 channels).
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
    if (recv_idx || recv_w) rt.write<true>(sd, rd, er, recv_idx, recv_w);
    if (recv_src && lane == 0) recv_src[sd] = src;
}

// FP8 dispatch: wave (t, d) quantises token t's row in registers and writes it to the
// token's destinations [d P, d P + P), at most kMaxWavesPerToken waves per token (P = 2 at
// top-8). Lane l of a pass owns the word pair (2 pi, 2 pi + 1), pi = 64 * pass + l: 16
// channels, whose 16 codes leave as one 128-bit store. A group of 128 channels is 8 pairs,
// i.e. 8 aligned lanes, so its largest |x| is reduced with three xor shuffles; scale =
// amax / 448, codes = e4m3(x * (448 / amax)) through the gfx950 packed fp8 convert (round
// to nearest even; the product is clamped to +-448, which only ever removes rounding
// excess above 448). Each destination row gets the codes as one burst of 128-bit stores
// and its H/128 scales (one lane per group). Row loads are cached, so a token's other
// waves read the row from L2. Measured on MI355X at 7168 channels, top-8 over 32 ranks,
// against one wave per token (non-temporal loads): 45.3 against 52.6 us at 4096 tokens,
// 83.7 against 109 at 8192; one wave per destination (8 quantisations per token) ran
// 67.6. The word-pair mapping measured 5% faster than one word per lane (64-bit code
// stores, a 16-lane reduction).
template <int WPP, bool kMulti, int kThreads>
__global__ __launch_bounds__(kThreads) void dispatch_fp8_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t t0, int64_t t_end, int V, int k, int R, int er,
    const int32_t* __restrict__ token_slot, FastDiv D, int P, u32x4* __restrict__ recv_codes,
    float* __restrict__ recv_scales, int64_t* __restrict__ recv_idx, float* __restrict__ recv_w,
    int32_t* __restrict__ recv_src, int64_t cap, int32_t* __restrict__ error_flag) {
    int64_t t;
    int d;
    if (!dest_wave<kThreads>(t0, t_end, D, t, d)) return;
    const int lane = lane_id();
    const int P2 = V / 2;
    const int G = V / 16;
    const int32_t* srow = token_slot + t * R;
    const int32_t s_first = lane < R ? srow[lane] : -1;
    const Routing rt(topk_idx ? topk_idx + t * k : nullptr, topk_w ? topk_w + t * k : nullptr, k,
                     recv_idx || recv_w);
    const u32x4* xr = x + t * V;
    int lo, hi;
    dest_range(d, D.d, P, lo, hi);
    int32_t errbits = 0;
    for (int p0 = 0; p0 < P2; p0 += kWave * WPP) {
        u32x4 code[WPP];
        float scale[WPP];
        quantize_fp8_pass<WPP>(xr, p0, P2, code, scale);
        visit_destinations(s_first, srow, R, 0, cap, lo, hi, errbits, [&](int64_t sd, int rd) {
            put_fp8_row<WPP>(code, scale, p0, P2, G, sd, rd, rt, er, static_cast<int32_t>(t),
                             recv_codes, recv_scales, recv_idx, recv_w, recv_src);
        });
        if constexpr (!kMulti) break;
    }
    if (errbits) raise_error(error_flag, errbits);
}

// Launches f(t0, t_end, grid) over consecutive token ranges of at most kDestMaxWaves / D
// tokens (D waves per token). Each launch's error is checked before the next; the first
// one is returned.
template <typename F>
hipError_t for_each_token_range(int64_t T, int D, F&& f) {
    constexpr int kWpb = kDestThreads / kWave;
    const int64_t per = std::max<int64_t>(1, kDestMaxWaves / D);
    for (int64_t t0 = 0; t0 < T; t0 += per) {
        const int64_t t_end = std::min(T, t0 + per);
        f(t0, t_end, static_cast<unsigned>(((t_end - t0) * D + kWpb - 1) / kWpb));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// with_row_width over a launch split into token ranges: the first launch error, if any.
template <int kMax, typename F>
hipError_t launch_by_token_range(int V, int64_t T, int D, F&& f) {
    hipError_t err = hipSuccess;
    const hipError_t last = with_row_width<kMax, false>(V, [&](auto wpl, auto multi) {
        err = for_each_token_range(T, D, [&](int64_t t0, int64_t t_end, unsigned grid) {
            f(wpl, multi, t0, t_end, grid);
        });
    });
    return err != hipSuccess ? err : last;
}

}  // namespace

hipError_t launch_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                           int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                           void* recv_x, int64_t* recv_idx, float* recv_w, int32_t* recv_src,
                           int64_t cap, int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int P = 1;                // destinations per wave
    const int D = std::min(k, R);   // waves per token: ranks a token can reach
    const FastDiv fd = FastDiv::make(D);
    return launch_by_token_range<14>(V, T, D, [&](auto wpl, auto multi, int64_t t0, int64_t t_end,
                                                  unsigned grid) {
        hipLaunchKernelGGL((dispatch_kernel<decltype(wpl)::value, decltype(multi)::value, kDestThreads>),
                           dim3(grid), dim3(kDestThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, t0, t_end, V, k, R,
                           E / R, token_slot, fd, P, static_cast<u32x4*>(recv_x), recv_idx, recv_w,
                           recv_src, cap, error_flag);
    });
}

hipError_t launch_dispatch_layout(const void* x, const int64_t* topk_idx, const float* topk_w,
                                  int64_t T, int H, int k, int E, int R, int N,
                                  const CountsWorkspace& cw, int32_t* token_slot, uint8_t* in_rank,
                                  void* recv_x, int64_t* recv_idx, float* recv_w,
                                  int32_t* recv_src, int64_t cap, int32_t* count_r,
                                  int32_t* rank_offset, int32_t* count_n, int32_t* count_e,
                                  int32_t* expert_offset, int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int D = std::min(k, R);  // waves per token: ranks a token can reach
    const FastDiv fd = FastDiv::make(D);
    const int nb = static_cast<int>((T + kLayoutBlockTokens - 1) / kLayoutBlockTokens);
    // head blocks of the first launch, a multiple of the 8 XCDs so that the dispatch's
    // blocks keep the placement they have without them (a top-8 token's two blocks on
    // neighbouring XCDs)
    int head = 0;
    if (count_e || expert_offset) head = (E + kDestThreads - 1) / kDestThreads;
    else if (count_n || count_r || rank_offset) head = 1;
    head = (head + 7) / 8 * 8;
    const bool local = nb <= kCountsLocalBlocks;
    return launch_by_token_range<14>(V, T, D, [&](auto wpl, auto multi, int64_t t0, int64_t t_end,
                                                  unsigned grid) {
        const int nhead = t0 == 0 ? head : 0;
        auto go = [&](auto loc) {
            hipLaunchKernelGGL((dispatch_layout_kernel<decltype(wpl)::value, decltype(multi)::value,
                                                       decltype(loc)::value, kDestThreads>),
                               dim3(grid + nhead), dim3(kDestThreads), 0, stream,
                               static_cast<const u32x4*>(x), topk_idx, topk_w, t0, t_end, V, k, R,
                               E / R, cw, fd, token_slot, in_rank, static_cast<u32x4*>(recv_x),
                               recv_idx, recv_w, recv_src, cap, nhead, nb, E, N, count_r,
                               rank_offset, count_n, count_e, expert_offset, error_flag);
        };
        if (local)
            go(std::true_type{});
        else
            go(std::false_type{});
    });
}

hipError_t launch_counts_slots(int64_t T, int E, int R, int N, const CountsWorkspace& cw,
                               int32_t* token_slot, uint8_t* in_rank, int32_t* count_r,
                               int32_t* rank_offset, int32_t* count_n, int32_t* count_e,
                               int32_t* expert_offset, hipStream_t stream) {
    const int nb = static_cast<int>((T + kLayoutBlockTokens - 1) / kLayoutBlockTokens);
    if (T == 0 || nb > kCountsLocalBlocks || R > kCountsMaxRanks) return hipErrorInvalidValue;
    constexpr int kWpb = kDestThreads / kWave;
    const int nhead = (count_e || expert_offset) ? (E + kDestThreads - 1) / kDestThreads : 1;
    const unsigned grid = static_cast<unsigned>(nhead + (T + kWpb - 1) / kWpb);
    hipLaunchKernelGGL(counts_slots_kernel<kDestThreads>, dim3(grid), dim3(kDestThreads), 0,
                       stream, T, R, cw, token_slot, in_rank, nhead, nb, E, N, count_r,
                       rank_offset, count_n, count_e, expert_offset);
    return hipGetLastError();
}

hipError_t launch_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_w,
                               int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                               void* recv_codes, float* recv_scales, int64_t* recv_idx,
                               float* recv_w, int32_t* recv_src, int64_t cap, int32_t* error_flag,
                               hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int P = (std::min(k, R) + kMaxWavesPerToken - 1) / kMaxWavesPerToken;
    const int D = (std::min(k, R) + P - 1) / P;  // waves per token, at most one block
    const FastDiv fd = FastDiv::make(D);
    // word pairs per lane: 7 covers a 7168-wide row in one pass
    return launch_by_token_range<7>(V / 2, T, D, [&](auto wpp, auto multi, int64_t t0, int64_t t_end,
                                                    unsigned grid) {
        hipLaunchKernelGGL((dispatch_fp8_kernel<decltype(wpp)::value, decltype(multi)::value, kDestThreads>),
                           dim3(grid), dim3(kDestThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, t0, t_end, V, k, R,
                           E / R, token_slot, fd, P, static_cast<u32x4*>(recv_codes),
                           recv_scales, recv_idx, recv_w, recv_src, cap, error_flag);
    });
}

hipError_t launch_dispatch_permute(const void* x, const float* topk_w, int64_t T, int H, int k,
                                   const int32_t* expert_slot, void* perm_x, float* perm_w,
                                   int32_t* perm_src, int64_t cap, int32_t* error_flag,
                                   hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const FastDiv fd = FastDiv::make(k);
    return launch_by_token_range<14>(V, T, k, [&](auto wpl, auto multi, int64_t t0, int64_t t_end,
                                                  unsigned grid) {
        hipLaunchKernelGGL((dispatch_permute_kernel<decltype(wpl)::value, decltype(multi)::value, kDestThreads>),
                           dim3(grid), dim3(kDestThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_w, t0, t_end, V, k, expert_slot,
                           fd, static_cast<u32x4*>(perm_x), perm_w, perm_src, cap, error_flag);
    });
}

hipError_t launch_dispatch_permute_layout(const void* x, const int64_t* topk_idx,
                                          const float* topk_w, int64_t T, int H, int k, int E,
                                          int N, const int32_t* expert_rank,
                                          const CountsWorkspace& cw, void* perm_x, float* perm_w,
                                          int32_t* perm_src, int32_t* expert_slot, int64_t cap,
                                          int32_t* count_e, int32_t* expert_offset,
                                          int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const FastDiv fd = FastDiv::make(k);  // one wave per (token, slot)
    const int nb = static_cast<int>((T + kLayoutBlockTokens - 1) / kLayoutBlockTokens);
    int head = (count_e || expert_offset) ? (E + kDestThreads - 1) / kDestThreads : 0;
    head = (head + 7) / 8 * 8;  // keeps the permute's blocks on their XCDs, as in the dispatch
    return launch_by_token_range<14>(V, T, k, [&](auto wpl, auto multi, int64_t t0, int64_t t_end,
                                                  unsigned grid) {
        const int nhead = t0 == 0 ? head : 0;
        hipLaunchKernelGGL((dispatch_permute_layout_kernel<decltype(wpl)::value,
                                                           decltype(multi)::value, kDestThreads>),
                           dim3(grid + nhead), dim3(kDestThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, t0, t_end, V, k, E, N,
                           expert_rank, cw, nb, fd, static_cast<u32x4*>(perm_x), perm_w, perm_src,
                           expert_slot, cap, nhead, count_e, expert_offset, error_flag);
    });
}

hipError_t launch_dispatch_send(const void* x, const int64_t* topk_idx, const float* topk_w,
                                int64_t T, int H, int k, int N, const int32_t* node_slot,
                                int64_t Tmax, void* stage_x, int64_t* stage_idx, float* stage_w,
                                int32_t* stage_src, int32_t* error_flag, int max_blocks,
                                hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int P = (std::min(k, N) + kMaxWavesPerToken - 1) / kMaxWavesPerToken;
    const int D = (std::min(k, N) + P - 1) / P;  // waves per token, at most one block
    const FastDiv fd = FastDiv::make(D);
    return launch_by_token_range<14>(V, T, D, [&](auto wpl, auto multi, int64_t t0, int64_t t_end,
                                                  unsigned grid) {
        if (max_blocks > 0) grid = std::min(grid, static_cast<unsigned>(max_blocks));
        hipLaunchKernelGGL((dispatch_send_kernel<decltype(wpl)::value, decltype(multi)::value, kDestThreads>),
                           dim3(grid), dim3(kDestThreads), 0, stream,
                           static_cast<const u32x4*>(x), topk_idx, topk_w, t0, t_end, V, k, N,
                           node_slot, Tmax, fd, P, static_cast<u32x4*>(stage_x), stage_idx, stage_w,
                           stage_src, error_flag);
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
    const int reach = std::min(k, R / N);  // ranks of a node a staged row can reach
    const int D = std::min(kRecvWavesPerRow, reach);
    const int P = (reach + D - 1) / D;
    const int64_t bx = (rows * D + kThreads / kWave - 1) / (kThreads / kWave);
    if (rows * D > INT32_MAX || !grid_fits(bx * N, kThreads) || N > 65535)
        return hipErrorInvalidConfiguration;
    return with_row_width<14, false>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((dispatch_recv_kernel<decltype(wpl)::value, decltype(multi)::value, kThreads>),
                           dim3(static_cast<unsigned>(bx), N), dim3(kThreads), 0, stream,
                           static_cast<const u32x4*>(stage_x), stage_idx, stage_w, stage_src,
                           count_n, Tmax, T, V, k, R, R / N, E / R, token_slot, FastDiv::make(D), P,
                           static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src, cap,
                           error_flag);
    });
}

}  // namespace ep
