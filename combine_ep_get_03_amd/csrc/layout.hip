// layout.hip -- the dispatch layout of one batch of top-k routing on gfx950.
//
// What it computes ("[PR #347] Feature/sm free normal kernel" names get_dispatch_layout
// in its commit list; "[PR #634] Hybrid ep nixl restripe" names the scan over tokens
// per local expert): per-rank, per-node and per-expert token counts, the token-in-rank
// bitmap, exclusive prefix offsets, and for every (token, rank) pair its receive row
// = rank_offset[r] + (tokens before it on rank r).
//
// Three launches, no inter-block communication inside a launch, integer only, so the
// result is the same on every run:
//   1. count: one token per lane, 256 tokens per block. Rank and node sets of a token
//      are bit masks; a wave64 ballot per rank gives the wave's count; per-expert
//      counts go through an LDS histogram. Per-block counts go to the workspace.
//   2. scan: one block walks the per-block counts column by column through an LDS tile
//      (an exclusive prefix per rank over blocks), reduces nodes and experts, and scans
//      the per-rank and per-expert totals into offsets.
//   3. slot: each block rebuilds its ballots and writes token_slot and the bitmap
//      row-major with consecutive lanes on consecutive words; a slot is the block's
//      base for the rank plus the popcount of the ballot bits below the token.
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kBT = kLayoutBlockTokens;      // tokens (= threads) per block
constexpr int kWavesBT = kBT / kWave;        // 4
constexpr int kScanThreads = 1024;
constexpr int kTileInts = 8192;              // 32 KiB LDS tile for the column walks

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Rank mask (and optionally node mask) of one token; expert -1 and out-of-range ids
// are skipped, the latter reported through `bad`.
template <int NW, bool kCount>
__device__ __forceinline__ void token_masks(const int64_t* __restrict__ row, int k, int E, int er,
                                            int rpn, uint64_t (&rm)[NW], uint64_t (&nm)[NW],
                                            int32_t* s_hist, int& bad) {
    for (int j = 0; j < k; ++j) {
        const int64_t e = row[j];
        if (e < 0 || e >= E) {
            if (e != -1) bad = 1;
            continue;
        }
        const int r = static_cast<int>(e) / er;
        if (kCount) atomicAdd(&s_hist[e], 1);
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if ((r >> 6) == w) rm[w] |= 1ull << (r & 63);
        if (kCount) {
            const int n = r / rpn;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if ((n >> 6) == w) nm[w] |= 1ull << (n & 63);
        }
    }
}

// Per wave: for each of `count` bit positions, ballot the bit across the wave and leave
// popcount(ballot) (kPop) or the ballot itself in lane b of word w. Result stored to
// dst[64*w + lane] for the lanes that own a position.
template <int NW, bool kPop, typename Out>
__device__ __forceinline__ void wave_ballots(const uint64_t (&mask)[NW], int count, Out* dst) {
    const int lane = lane_id();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int base = w * kWave;
        if (base < count) {
            const int lim = min(kWave, count - base);
            Out mine = 0;
            for (int b = 0; b < lim; ++b) {
                const uint64_t m = wave_ballot((mask[w] >> b) & 1ull);
                if (lane == b) mine = kPop ? static_cast<Out>(__popcll(m)) : static_cast<Out>(m);
            }
            if (lane < lim) dst[base + lane] = mine;
        }
    }
}

template <int NW>
__global__ __launch_bounds__(kBT) void layout_count_kernel(const int64_t* __restrict__ topk_idx,
                                                            int64_t T, int k, int E, int R, int N,
                                                            int er, int rpn, LayoutWorkspace ws) {
    extern __shared__ int32_t smem[];
    int32_t* s_hist = smem;               // [E]
    int32_t* s_wr = s_hist + E;           // [4][R]
    int32_t* s_wn = s_wr + kWavesBT * R;  // [4][N]
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * kBT + tid;

    for (int e = tid; e < E; e += kBT) s_hist[e] = 0;
    __syncthreads();

    uint64_t rm[NW], nm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) rm[w] = nm[w] = 0;
    int bad = 0;
    if (t < T) token_masks<NW, true>(topk_idx + t * k, k, E, er, rpn, rm, nm, s_hist, bad);

    wave_ballots<NW, true>(rm, R, s_wr + wave * R);
    wave_ballots<NW, true>(nm, N, s_wn + wave * N);
    __syncthreads();

    const int64_t b = blockIdx.x;
    for (int r = tid; r < R; r += kBT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) c += s_wr[w * R + r];
        ws.blk_rank[b * R + r] = c;
    }
    for (int n = tid; n < N; n += kBT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) c += s_wn[w * N + n];
        ws.blk_node[b * N + n] = c;
    }
    for (int e = tid; e < E; e += kBT) ws.blk_exp[b * E + e] = s_hist[e];
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) ws.blk_err[b] = any_bad;
}

// Exclusive prefix of one value per thread over the block; `total` gets the sum.
__device__ int block_exclusive_scan(int v, int32_t* s_tmp /*[17]*/, int& total) {
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    int x = v;
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s_tmp[wave] = x;
    __syncthreads();
    if (wave == 0) {
        const int ws = lane < nwaves ? s_tmp[lane] : 0;
        int xs = ws;
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(xs, d, kWave);
            if (lane >= d) xs += y;
        }
        if (lane < nwaves) s_tmp[lane] = xs - ws;
        if (lane == nwaves - 1) s_tmp[16] = xs;
    }
    __syncthreads();
    const int res = x - v + s_tmp[wave];
    total = s_tmp[16];
    __syncthreads();
    return res;
}

// Columns [c0, c0+width) of a [rows][cols] int32 matrix, one column per thread
// (width <= blockDim), rows walked in order through an LDS tile. With kPrefix every
// entry becomes the sum of the entries above it in its column. Returns the column
// total in threads tid < width.
template <bool kPrefix>
__device__ int column_walk(int32_t* __restrict__ m, int rows, int cols, int c0, int width,
                           int32_t* s_tile) {
    const int tid = threadIdx.x;
    const int ch = max(1, kTileInts / width);
    int carry = 0;
    for (int r0 = 0; r0 < rows; r0 += ch) {
        const int nr = min(ch, rows - r0);
        for (int i = tid; i < nr * width; i += blockDim.x) {
            const int rr = i / width;
            s_tile[i] = m[static_cast<int64_t>(r0 + rr) * cols + c0 + (i - rr * width)];
        }
        __syncthreads();
        if (tid < width) {
            for (int rr = 0; rr < nr; ++rr) {
                const int v = s_tile[rr * width + tid];
                if (kPrefix) s_tile[rr * width + tid] = carry;
                carry += v;
            }
        }
        __syncthreads();
        if (kPrefix) {
            for (int i = tid; i < nr * width; i += blockDim.x) {
                const int rr = i / width;
                m[static_cast<int64_t>(r0 + rr) * cols + c0 + (i - rr * width)] = s_tile[i];
            }
            __syncthreads();
        }
    }
    return carry;
}

__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int nb, int E, int R, int N, LayoutWorkspace ws, int32_t* __restrict__ count_r,
    int32_t* __restrict__ count_n, int32_t* __restrict__ count_e,
    int32_t* __restrict__ rank_offset, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ error_flag) {
    __shared__ int32_t s_tile[kTileInts];
    __shared__ int32_t s_scan[17];
    const int tid = threadIdx.x;

    // ranks: per-block exclusive prefix in place, totals, offsets (R <= blockDim)
    const int tot = column_walk<true>(ws.blk_rank, nb, R, 0, R, s_tile);
    int M = 0;
    const int ex = block_exclusive_scan(tid < R ? tot : 0, s_scan, M);
    if (tid < R) {
        count_r[tid] = tot;
        rank_offset[tid] = ex;
    }
    if (tid == 0) rank_offset[R] = M;

    if (count_n) {
        const int tn = column_walk<false>(ws.blk_node, nb, N, 0, N, s_tile);
        if (tid < N) count_n[tid] = tn;
    }

    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kScanThreads) {
        const int width = min(kScanThreads, E - c0);
        const int te = column_walk<false>(ws.blk_exp, nb, E, c0, width, s_tile);
        int chunk = 0;
        const int exe = block_exclusive_scan(tid < width ? te : 0, s_scan, chunk);
        if (tid < width) {
            if (count_e) count_e[c0 + tid] = te;
            if (expert_offset) expert_offset[c0 + tid] = carry + exe;
        }
        carry += chunk;
    }
    if (expert_offset && tid == 0) expert_offset[E] = carry;

    int bad = 0;
    for (int i = tid; i < nb; i += blockDim.x) bad |= ws.blk_err[i];
    bad = __syncthreads_or(bad);
    if (tid == 0) *error_flag = bad ? kErrTopkRange : 0;
}

template <int NW>
__global__ __launch_bounds__(kBT) void layout_slot_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int er,
    const int32_t* __restrict__ blk_prefix, const int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank) {
    extern __shared__ uint64_t smem64[];
    uint64_t* s_ball = smem64;                                         // [4][R]
    int32_t* s_base = reinterpret_cast<int32_t*>(s_ball + kWavesBT * R);  // [4][R]
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBT;
    const int64_t t = t0 + tid;

    uint64_t rm[NW], nm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) rm[w] = nm[w] = 0;
    int bad = 0;
    if (t < T) token_masks<NW, false>(topk_idx + t * k, k, E, er, 1, rm, nm, nullptr, bad);
    wave_ballots<NW, false>(rm, R, s_ball + wave * R);
    __syncthreads();

    const int64_t b = blockIdx.x;
    for (int r = tid; r < R; r += kBT) {
        int base = rank_offset[r] + blk_prefix[b * R + r];
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) {
            s_base[w * R + r] = base;
            base += __popcll(s_ball[w * R + r]);
        }
    }
    __syncthreads();

    const int nt = static_cast<int>(min<int64_t>(kBT, T - t0));
    const int total = nt * R;
    int32_t* slot_out = token_slot + t0 * R;
    uint8_t* bit_out = in_rank ? in_rank + t0 * R : nullptr;
    for (int f = tid; f < total; f += kBT) {
        const int tt = f / R;
        const int r = f - tt * R;
        const int w = tt / kWave;
        const int l = tt % kWave;
        const uint64_t m = s_ball[w * R + r];
        const bool on = (m >> l) & 1ull;
        const int below = __popcll(m & ((1ull << l) - 1ull));
        slot_out[f] = on ? s_base[w * R + r] + below : -1;
        if (bit_out) bit_out[f] = on ? 1 : 0;
    }
}

template <int NW>
hipError_t layout_impl(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                       int32_t* count_r, int32_t* count_n, int32_t* count_e, uint8_t* in_rank,
                       int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                       int32_t* error_flag, const LayoutWorkspace& ws, hipStream_t stream) {
    const int64_t nb = (T + kBT - 1) / kBT;
    const int er = E / R;
    const int rpn = R / N;
    if (!grid_fits(nb, kBT)) return hipErrorInvalidConfiguration;
    if (nb > 0) {
        const size_t shm = sizeof(int32_t) * (static_cast<size_t>(E) + kWavesBT * (R + N));
        hipLaunchKernelGGL(layout_count_kernel<NW>, dim3(static_cast<unsigned>(nb)), dim3(kBT),
                           shm, stream, topk_idx, T, k, E, R, N, er, rpn, ws);
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                       static_cast<int>(nb), E, R, N, ws, count_r, count_n, count_e, rank_offset,
                       expert_offset, error_flag);
    if (nb > 0) {
        const size_t shm = static_cast<size_t>(kWavesBT) * R * (sizeof(uint64_t) + sizeof(int32_t));
        hipLaunchKernelGGL(layout_slot_kernel<NW>, dim3(static_cast<unsigned>(nb)), dim3(kBT), shm,
                           stream, topk_idx, T, k, E, R, er, ws.blk_rank, rank_offset, token_slot,
                           in_rank);
    }
    return hipGetLastError();
}

}  // namespace

size_t layout_workspace_bytes(int64_t T, int E, int R, int N) {
    const size_t nb = static_cast<size_t>((T + kBT - 1) / kBT);
    return align_up(nb * R * 4, 256) + align_up(nb * N * 4, 256) + align_up(nb * E * 4, 256) +
           align_up(nb * 4, 256);
}

LayoutWorkspace carve_layout_workspace(void* base, int64_t T, int E, int R, int N) {
    const size_t nb = static_cast<size_t>((T + kBT - 1) / kBT);
    char* p = static_cast<char*>(base);
    LayoutWorkspace ws;
    ws.blk_rank = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * R * 4, 256);
    ws.blk_node = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * N * 4, 256);
    ws.blk_exp = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * E * 4, 256);
    ws.blk_err = reinterpret_cast<int32_t*>(p);
    return ws;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                         int32_t* count_r, int32_t* count_n, int32_t* count_e, uint8_t* in_rank,
                         int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                         int32_t* error_flag, const LayoutWorkspace& ws, hipStream_t stream) {
#define EP_LAYOUT_CASE(NW)                                                                     \
    return layout_impl<NW>(topk_idx, T, k, E, R, N, count_r, count_n, count_e, in_rank,        \
                           rank_offset, expert_offset, token_slot, error_flag, ws, stream)
    if (R <= 64) EP_LAYOUT_CASE(1);
    if (R <= 128) EP_LAYOUT_CASE(2);
    if (R <= 256) EP_LAYOUT_CASE(4);
    if (R <= 512) EP_LAYOUT_CASE(8);
    EP_LAYOUT_CASE(16);
#undef EP_LAYOUT_CASE
}

}  // namespace ep
