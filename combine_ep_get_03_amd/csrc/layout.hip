// layout.hip -- the dispatch layout of one batch of top-k routing on gfx950.
//
// What it computes ("[PR #347] Feature/sm free normal kernel" names get_dispatch_layout
// in its commit list; "[PR #634] Hybrid ep nixl restripe" names the scan over tokens
// per local expert): per-rank, per-node and per-expert token counts, the token-in-rank
// bitmap, exclusive prefix offsets, and for every (token, rank) pair its receive row
// = rank_offset[r] + (tokens before it on rank r).
//
// Integer only and no inter-block communication inside a launch, so every run gives
// the same result. Blocks own 256 consecutive tokens, one per lane.
//   1. count: the rank and node sets of a token are bit masks; a 64x64 bit transpose
//      across the wave turns the lanes' masks into one ballot per rank (node), whose
//      popcount is the wave's count; per-expert counts go through an LDS
//      histogram, stored as the block's inclusive prefix over experts. Per-block
//      counts go to the workspace.
//   2. slot: each block rebuilds its ballots; a slot is rank_offset[r] + the block's
//      prefix for r + the popcount of the ballot bits below the token. token_slot and
//      the bitmap are written row-major, consecutive threads on consecutive words.
//      Expert offsets are column sums of the per-block inclusive prefixes, so they need
//      no scan: the slot blocks split the expert columns between them.
// When the per-block rank table is small (up to 64 blocks and 4096 cells, R <= 256)
// every slot block reduces that table itself (two launches in all); otherwise a
// one-block scan launch between the two computes the per-block rank prefixes.
// Small tables are read with several loads in flight per lane: the path is latency
// bound, so each block waits on as few memory round trips as possible.
#include <atomic>
#include <mutex>

#include "dispatch_rows.hpp"
#include "ep_internal.hpp"

namespace ep {

// Device scratch for ep_get_layout_no_alloc, the entry point for callers that cannot
// allocate: the per-block count tables go here instead of a caller workspace. Each GPU
// holds its own copy at its own address until the process ends. In host code the name
// is only a host-side stand-in: kernels get the address layout_scratch_address returns.
static __device__ __align__(256) unsigned char scratch[kLayoutScratchBytes];

namespace {

constexpr int kBT = kLayoutBlockTokens;  // tokens (= threads) per block
static_assert(kRestripeThreads == kBT, "restripe blocks ride along in layout launches");
constexpr int kWavesBT = kBT / kWave;    // 4
constexpr int kScanThreads = 1024;
constexpr int kTileInts = 8192;          // 32 KiB LDS tile for the one-block column walks
constexpr int kFusedMaxBlocks = 64;
constexpr int kFusedMaxCells = 4096;
constexpr int kFusedMaxRanks = kBT;
constexpr int kBatch = 8;                // loads in flight per lane for table reads
// Largest [nb][ncol] expert slice of one fused slot block: ncol <= E / (4 nb) + 2.
constexpr int kFusedMaxSlice = kMaxExperts / 4 + 2 * 64;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Rank mask (and optionally node mask) of one token; expert -1 and out-of-range ids
// are skipped, the latter reported through `bad`. The k ids are loaded 8 at a time so
// their latencies overlap.
template <int NW, bool kCount, bool kNodes = kCount>
__device__ __forceinline__ void token_masks(const int64_t* __restrict__ row, int k, int E,
                                            FastDiv er, FastDiv rpn, uint64_t (&rm)[NW],
                                            uint64_t (&nm)[NW], int32_t* s_hist, int& bad) {
    for (int j0 = 0; j0 < k; j0 += kBatch) {
        int64_t ev[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) ev[u] = (j0 + u < k) ? row[j0 + u] : -1;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t e = ev[u];
            if (e < 0 || e >= E) {
                if (e != -1) bad = 1;
                continue;
            }
            const int r = er.div(static_cast<int>(e));
            if (kCount) atomicAdd(&s_hist[e], 1);
#pragma unroll
            for (int w = 0; w < NW; ++w)
                if ((r >> 6) == w) rm[w] |= 1ull << (r & 63);
            if (kNodes) {
                const int n = rpn.div(r);
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    if ((n >> 6) == w) nm[w] |= 1ull << (n & 63);
            }
        }
    }
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int lane_mask) {
    const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), lane_mask, kWave));
    const uint32_t hi =
        static_cast<uint32_t>(__shfl_xor(static_cast<int>(v >> 32), lane_mask, kWave));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Transpose of a 64x64 bit matrix held one row per lane: afterwards bit i of lane j is
// bit j of lane i's input. Six rounds; round s swaps the off-diagonal s x s sub-blocks
// between lanes i and i ^ s.
__device__ __forceinline__ uint64_t wave_transpose64(uint64_t row) {
    const int lane = lane_id();
    constexpr uint64_t kKeep[6] = {0x00000000FFFFFFFFull, 0x0000FFFF0000FFFFull,
                                   0x00FF00FF00FF00FFull, 0x0F0F0F0F0F0F0F0Full,
                                   0x3333333333333333ull, 0x5555555555555555ull};
#pragma unroll
    for (int i = 0; i < 6; ++i) {
        const int s = 32 >> i;
        const uint64_t other = shfl_xor64(row, s);
        row = (lane & s) ? ((row & ~kKeep[i]) | ((other & ~kKeep[i]) >> s))
                         : ((row & kKeep[i]) | ((other & kKeep[i]) << s));
    }
    return row;
}

// Per wave: the ballot of each of `count` bit positions of the lanes' masks, i.e. the
// columns of the wave's (lanes x positions) bit matrix, taken 64 positions at a time
// by a transpose. dst[p] gets the ballot of position p (or its popcount with kPop).
template <int NW, bool kPop, typename Out>
__device__ __forceinline__ void wave_ballots(const uint64_t (&mask)[NW], int count, Out* dst) {
    const int lane = lane_id();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int base = w * kWave;
        if (base < count) {
            const uint64_t col = wave_transpose64(mask[w]);
            if (base + lane < count)
                dst[base + lane] = kPop ? static_cast<Out>(__popcll(col)) : static_cast<Out>(col);
        }
    }
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

// For i in [0, n), strided over the block: acc[col(i)] += src(i) (LDS atomics), with
// kBatch loads in flight per lane. Used for small [rows][cols] tables.
template <typename Src, typename Col>
__device__ __forceinline__ void accumulate_columns(int n, Src src, Col col, int32_t* acc) {
    for (int i0 = threadIdx.x; i0 < n; i0 += blockDim.x * kBatch) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * blockDim.x;
            v[u] = i < n ? src(i) : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < n && v[u] != 0) atomicAdd(&acc[col(i)], v[u]);
        }
    }
}

// token_slot and the bitmap of one block's tokens, row-major, from the block's ballots
// (s_ball[w][r]: which of wave w's tokens are on rank r) and slot bases (s_base[w][r]).
// With R <= 256 each thread keeps one rank column and its four ballots in registers,
// so consecutive threads write consecutive words of a row and the loop needs no
// division or LDS access.
__device__ __forceinline__ void write_block_slots(const uint64_t* s_ball, const int32_t* s_base,
                                                  int64_t T, int64_t t0, int R,
                                                  int32_t* __restrict__ token_slot,
                                                  uint8_t* __restrict__ in_rank) {
    const int tid = threadIdx.x;
    const int nt = static_cast<int>(min<int64_t>(kBT, T - t0));
    int32_t* slot_out = token_slot + t0 * R;
    uint8_t* bit_out = in_rank ? in_rank + t0 * R : nullptr;
    if (R <= kBT) {
        const int rows_per_pass = kBT / R;
        const int r = tid % R;
        const int q0 = tid / R;
        if (q0 >= rows_per_pass) return;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) {
            const uint64_t m = s_ball[w * R + r];
            const int base = s_base[w * R + r];
            for (int l = q0; l < kWave; l += rows_per_pass) {
                const int tt = w * kWave + l;
                if (tt >= nt) break;
                const bool on = (m >> l) & 1ull;
                const int below = __popcll(m & ((1ull << l) - 1ull));
                slot_out[tt * R + r] = on ? base + below : -1;
                if (bit_out) bit_out[tt * R + r] = on ? 1 : 0;
            }
        }
        return;
    }
    const int total = nt * R;
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

// token_slot and the bitmap of one wave's 64 tokens starting at tq0, from that wave's
// ballots (ball[r]) and slot bases (base[r]). With `vec` (R % 4 == 0 and aligned
// outputs) a thread writes four ranks of a token: one 128-bit and one 32-bit store.
__device__ __forceinline__ void write_wave_slots(const uint64_t* ball, const int32_t* base,
                                                 int64_t T, int64_t tq0, int R, bool vec,
                                                 int32_t* __restrict__ token_slot,
                                                 uint8_t* __restrict__ in_rank) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int nt = static_cast<int>(min<int64_t>(kWave, T - tq0));
    if (nt <= 0) return;
    int32_t* slot_out = token_slot + tq0 * R;
    uint8_t* bit_out = in_rank ? in_rank + tq0 * R : nullptr;
    if (vec) {
        const int cols = R / 4;
        const int rows_per_pass = kBT / cols;
        const int c = tid % cols;
        const int l0 = tid / cols;
        if (l0 >= rows_per_pass) return;
        uint64_t m[4];
        int bs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            m[u] = ball[4 * c + u];
            bs[u] = base[4 * c + u];
        }
        for (int l = l0; l < nt; l += rows_per_pass) {
            const uint64_t below = (1ull << l) - 1ull;
            i32x4 o;
            uint32_t bits = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t on = static_cast<uint32_t>((m[u] >> l) & 1ull);
                o[u] = on ? bs[u] + __popcll(m[u] & below) : -1;
                bits |= on << (8 * u);
            }
            *reinterpret_cast<i32x4*>(slot_out + l * R + 4 * c) = o;
            if (bit_out) *reinterpret_cast<uint32_t*>(bit_out + l * R + 4 * c) = bits;
        }
        return;
    }
    const int total = nt * R;
    for (int f = tid; f < total; f += kBT) {
        const int l = f / R;
        const int r = f - l * R;
        const uint64_t m = ball[r];
        const bool on = (m >> l) & 1ull;
        slot_out[f] = on ? base[r] + __popcll(m & ((1ull << l) - 1ull)) : -1;
        if (bit_out) bit_out[f] = on ? 1 : 0;
    }
}

// Blocks past the layout's own `nlb` blocks run the dense restripe that may ride along in
// the layout's first launch (they return before any block barrier).
template <int NW>
__global__ __launch_bounds__(kBT) void layout_count_kernel(const int64_t* __restrict__ topk_idx,
                                                            int64_t T, int k, int E, int R, int N,
                                                            FastDiv er, FastDiv rpn,
                                                            LayoutWorkspace ws, int64_t nlb,
                                                            RestripeTask rs) {
    if (static_cast<int64_t>(blockIdx.x) >= nlb) {
        restripe_task_block(rs, static_cast<int64_t>(blockIdx.x) - nlb);
        return;
    }
    extern __shared__ int32_t smem[];
    int32_t* s_hist = smem;                                      // [E]
    uint16_t* s_wr = reinterpret_cast<uint16_t*>(s_hist + E);    // [4][R] per-wave counts
    uint16_t* s_wn = s_wr + kWavesBT * R;                        // [4][N]
    __shared__ int32_t s_scan[17];
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
    // inclusive prefix of this block's expert histogram
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kBT) {
        const int e = c0 + tid;
        const int h = e < E ? s_hist[e] : 0;
        int chunk = 0;
        const int ex = block_exclusive_scan(h, s_scan, chunk);
        if (e < E) ws.blk_exp[b * E + e] = carry + ex + h;
        carry += chunk;
    }
    const int any_bad = __syncthreads_or(bad);
    if (tid == 0) ws.blk_err[b] = any_bad;
}

// Slot kernel with the rank scan folded in (small per-block rank tables only). Four
// launch blocks share each 256-token group: each rebuilds the group's ballots (one wave
// per 64 tokens) and reduces the per-block rank table, and each writes the rows of its
// own 64 tokens, so the writes are spread over four times as many CUs.
constexpr int kQuarters = kWavesBT;

template <int NW>
__global__ __launch_bounds__(kBT) void layout_slot_fused_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int N, FastDiv er, int nb,
    LayoutWorkspace ws, int32_t* __restrict__ count_r, int32_t* __restrict__ count_n,
    int32_t* __restrict__ count_e, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ error_flag,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank, int vec_out,
    int want_expert_base, FastDiv rpn, int32_t* __restrict__ node_slot, int vec_node) {
    __shared__ int32_t s_cnt[kFusedMaxCells];               // [nb][R] per-group rank counts
    __shared__ uint64_t s_ball[kWavesBT * kFusedMaxRanks];  // [4][R] the group's ballots
    __shared__ int32_t s_base[kFusedMaxRanks];              // slot base of this quarter, per rank
    __shared__ int32_t s_tab[kFusedMaxSlice];               // [nb][ncol] expert slice
    __shared__ int32_t s_col[kMaxExperts / kQuarters + 2];  // column sums of the slice
    __shared__ int32_t s_node[kFusedMaxRanks];              // N <= R
    __shared__ uint64_t s_nball[kWavesBT * kFusedMaxRanks];  // [4][N] node ballots
    __shared__ int32_t s_npre[kFusedMaxRanks];               // node counts of earlier groups
    __shared__ int32_t s_nbase[kFusedMaxRanks];              // packed node row base, per node
    __shared__ int32_t s_scan[17];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int g = blockIdx.x;
    const int grp = g / kQuarters;
    const int q = g % kQuarters;
    const int nblk = gridDim.x;
    const int64_t t0 = static_cast<int64_t>(grp) * kBT;
    const int64_t t = t0 + tid;
    // expert columns [c0, c1) belong to this block; slice column c is expert c0 - 1 + c
    const int cw = (E + nblk - 1) / nblk;
    const int c0 = min(E, g * cw);
    const int c1 = min(E, c0 + cw);
    const int ncol = c1 - c0 + 1;

    for (int i = tid; i < N; i += kBT) {
        s_node[i] = 0;
        s_npre[i] = 0;
    }
    __syncthreads();

    // Issue the rank-table loads, then the token's ids, then park the table in LDS.
    const int ncell = nb * R;
    constexpr int kCellsPerLane = kFusedMaxCells / kBT;
    int cell[kCellsPerLane];
#pragma unroll
    for (int u = 0; u < kCellsPerLane; ++u) {
        const int i = tid + u * kBT;
        cell[u] = i < ncell ? ws.blk_rank[i] : 0;
    }
    uint64_t rm[NW], nm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) rm[w] = nm[w] = 0;
    int bad = 0;
    if (t < T) {
        if (node_slot)
            token_masks<NW, false, true>(topk_idx + t * k, k, E, er, rpn, rm, nm, nullptr, bad);
        else
            token_masks<NW, false>(topk_idx + t * k, k, E, er, FastDiv{1, 0}, rm, nm, nullptr, bad);
    }
#pragma unroll
    for (int u = 0; u < kCellsPerLane; ++u) {
        const int i = tid + u * kBT;
        if (i < ncell) s_cnt[i] = cell[u];
    }
    // the expert slice [nb][ncol] of the per-block inclusive prefixes, kBatch loads in flight
    const int nslice = nb * ncol;
    for (int i0 = tid; i0 < nslice; i0 += kBT * kBatch) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kBT;
            const int e = c0 - 1 + i % ncol;
            v[u] = (i < nslice && e >= 0) ? ws.blk_exp[static_cast<int64_t>(i / ncol) * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * kBT;
            if (i < nslice) s_tab[i] = v[u];
        }
    }
    int any_bad = 0;
    if (g == 0) {
        accumulate_columns(
            nb * N, [&](int i) { return ws.blk_node[i]; }, [&](int i) { return i % N; }, s_node);
        for (int i = tid; i < nb; i += kBT) any_bad |= ws.blk_err[i];
    }
    if (node_slot) {
        accumulate_columns(
            grp * N, [&](int i) { return ws.blk_node[i]; }, [&](int i) { return i % N; }, s_npre);
        wave_ballots<NW, false>(nm, N, s_nball + wave * N);
    }
    wave_ballots<NW, false>(rm, R, s_ball + wave * R);
    __syncthreads();

    // rank totals, this group's prefix, exclusive rank offsets (R <= blockDim)
    int tot = 0, pre = 0;
    if (tid < R) {
        for (int bb = 0; bb < nb; ++bb) {
            const int v = s_cnt[bb * R + tid];
            pre += bb < grp ? v : 0;
            tot += v;
        }
    }
    int M = 0;
    const int ro = block_exclusive_scan(tid < R ? tot : 0, s_scan, M);
    if (tid < R) {
        int base = ro + pre;
        for (int w = 0; w < q; ++w) base += __popcll(s_ball[w * R + tid]);
        s_base[tid] = base;
        if (g == 0) {
            count_r[tid] = tot;
            rank_offset[tid] = ro;
        }
    }
    if (g == 0 && tid == 0) rank_offset[R] = M;
    if (node_slot && tid < N) {
        int base = s_npre[tid];
        for (int w = 0; w < q; ++w) base += __popcll(s_nball[w * N + tid]);
        s_nbase[tid] = base;
    }
    // column sums of the inclusive prefixes: expert_offset[e + 1] for e = c0 - 1 + c
    for (int c = tid; c < ncol; c += kBT) {
        int sum = 0;
        for (int bb = 0; bb < nb; ++bb) sum += s_tab[bb * ncol + c];
        s_col[c] = sum;
    }
    __syncthreads();
    for (int c = tid + 1; c < ncol; c += kBT) {
        const int e = c0 - 1 + c;
        if (count_e) count_e[e] = s_col[c] - s_col[c - 1];
        if (expert_offset) expert_offset[e + 1] = s_col[c];
        if (want_expert_base) {
            // first expert-major row of expert e in each block: offset[e] plus the
            // pairs naming e in earlier blocks (histogram = difference of prefixes)
            int run = s_col[c - 1];
            for (int bb = 0; bb < nb; ++bb) {
                ws.blk_exp_base[static_cast<int64_t>(bb) * E + e] = run;
                run += s_tab[bb * ncol + c] - s_tab[bb * ncol + c - 1];
            }
        }
    }
    if (g == 0) {
        if (expert_offset && tid == 0) expert_offset[0] = 0;
        if (count_n)
            for (int n = tid; n < N; n += kBT) count_n[n] = s_node[n];
    }
    __syncthreads();

    write_wave_slots(s_ball + q * R, s_base, T, t0 + q * kWave, R, vec_out != 0, token_slot,
                     in_rank);
    if (node_slot)
        write_wave_slots(s_nball + q * N, s_nbase, T, t0 + q * kWave, N, vec_node != 0, node_slot,
                         nullptr);
    if (g == 0) {
        any_bad = __syncthreads_or(any_bad);
        if (tid == 0) *error_flag = any_bad ? kErrTopkRange : 0;
    }
}

// The whole layout of a batch of at most one 256-token group (up to 256 tokens, R <= 256)
// in one block: the counts, offsets and slots need no cross-block exchange, so the count
// and slot kernels collapse into one, with block barriers only. Same outputs as the
// two-launch path; the expert-major slots (when asked for) still take the expert-slot
// launch, whose per-block base is then the expert offset itself. With flag_first the
// block clears the error flag as it starts and ORs its bit in at the end (other blocks of
// the launch may raise bits meanwhile); else it stores the flag once at the end. With
// token_slot NULL it writes no slots (nor the bitmap).
template <int NW>
__device__ __forceinline__ void layout_single_block(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int N, FastDiv er,
    FastDiv rpn, int32_t* __restrict__ count_r, int32_t* __restrict__ count_n,
    int32_t* __restrict__ count_e, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ error_flag,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank, int vec_out,
    int32_t* __restrict__ exp_base, int32_t* __restrict__ node_slot, int vec_node,
    bool flag_first) {
    if (flag_first && threadIdx.x == 0)
        __hip_atomic_store(error_flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    extern __shared__ int32_t s_hist[];                        // [E]
    __shared__ uint64_t s_ball[kWavesBT * kFusedMaxRanks];     // [4][R]
    __shared__ uint64_t s_nball[kWavesBT * kFusedMaxRanks];    // [4][N]
    __shared__ int32_t s_base[kWavesBT * kFusedMaxRanks];      // [4][R] slot base per wave
    __shared__ int32_t s_nbase[kWavesBT * kFusedMaxRanks];     // [4][N]
    __shared__ int32_t s_scan[17];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    for (int e = tid; e < E; e += kBT) s_hist[e] = 0;
    __syncthreads();

    uint64_t rm[NW], nm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) rm[w] = nm[w] = 0;
    int bad = 0;
    if (tid < T) token_masks<NW, true, true>(topk_idx + tid * k, k, E, er, rpn, rm, nm, s_hist, bad);
    wave_ballots<NW, false>(rm, R, s_ball + wave * R);
    wave_ballots<NW, false>(nm, N, s_nball + wave * N);
    __syncthreads();

    // ranks: totals, exclusive offsets and each wave's slot base (R <= blockDim)
    int tot = 0;
    if (tid < R) {
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) tot += __popcll(s_ball[w * R + tid]);
    }
    int M = 0;
    const int ro = block_exclusive_scan(tid < R ? tot : 0, s_scan, M);
    if (tid < R) {
        count_r[tid] = tot;
        rank_offset[tid] = ro;
        int base = ro;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) {
            s_base[w * R + tid] = base;
            base += __popcll(s_ball[w * R + tid]);
        }
    }
    if (tid == 0) rank_offset[R] = M;
    if (tid < N) {
        int base = 0;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) {
            s_nbase[w * N + tid] = base;
            base += __popcll(s_nball[w * N + tid]);
        }
        if (count_n) count_n[tid] = base;
    }
    // experts: counts and exclusive offsets
    int carry = 0;
    for (int c0 = 0; c0 < E; c0 += kBT) {
        const int e = c0 + tid;
        const int h = e < E ? s_hist[e] : 0;
        int chunk = 0;
        const int ex = block_exclusive_scan(h, s_scan, chunk);
        if (e < E) {
            if (count_e) count_e[e] = h;
            if (expert_offset) expert_offset[e] = carry + ex;
            if (exp_base) exp_base[e] = carry + ex;
        }
        carry += chunk;
    }
    if (tid == 0 && expert_offset) expert_offset[E] = carry;
    const int any_bad = __syncthreads_or(bad);  // also orders the slot bases before the reads
    if (tid == 0) {
        if (!flag_first)
            *error_flag = any_bad ? kErrTopkRange : 0;
        else if (any_bad)
            raise_error(error_flag, kErrTopkRange);
    }

#pragma unroll
    for (int q = 0; q < kWavesBT; ++q) {
        if (token_slot)
            write_wave_slots(s_ball + q * R, s_base + q * R, T, q * kWave, R, vec_out != 0,
                             token_slot, in_rank);
        if (node_slot)
            write_wave_slots(s_nball + q * N, s_nbase + q * N, T, q * kWave, N, vec_node != 0,
                             node_slot, nullptr);
    }
}

template <int NW>
__global__ __launch_bounds__(kBT) void layout_single_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int N, FastDiv er,
    FastDiv rpn, int32_t* __restrict__ count_r, int32_t* __restrict__ count_n,
    int32_t* __restrict__ count_e, int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ expert_offset, int32_t* __restrict__ error_flag,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank, int vec_out,
    int32_t* __restrict__ exp_base, int32_t* __restrict__ node_slot, int vec_node,
    RestripeTask rs) {
    if (blockIdx.x >= 1) {  // a dense restripe riding along (see layout_count_kernel)
        restripe_task_block(rs, static_cast<int64_t>(blockIdx.x) - 1);
        return;
    }
    layout_single_block<NW>(topk_idx, T, k, E, R, N, er, rpn, count_r, count_n, count_e,
                            rank_offset, expert_offset, error_flag, token_slot, in_rank, vec_out,
                            exp_base, node_slot, vec_node, false);
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

// One block: per-block exclusive rank prefixes (in place), totals, offsets, node and
// expert counts, error flag. Used when the per-block rank table is too large to be
// reduced by every slot block.
__global__ __launch_bounds__(kScanThreads) void layout_scan_kernel(
    int nb, int E, int R, int N, LayoutWorkspace ws, int32_t* __restrict__ count_r,
    int32_t* __restrict__ count_n, int32_t* __restrict__ count_e,
    int32_t* __restrict__ rank_offset, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ error_flag, int want_expert_base, int want_node_prefix) {
    __shared__ int32_t s_tile[kTileInts];
    __shared__ int32_t s_last[kScanThreads];
    __shared__ int32_t s_scan[17];
    const int tid = threadIdx.x;

    const int tot = column_walk<true>(ws.blk_rank, nb, R, 0, R, s_tile);
    int M = 0;
    const int ex = block_exclusive_scan(tid < R ? tot : 0, s_scan, M);
    if (tid < R) {
        count_r[tid] = tot;
        rank_offset[tid] = ex;
    }
    if (tid == 0) rank_offset[R] = M;

    if (want_node_prefix) {
        // per-block exclusive node prefixes in place (for node_slot), totals as counts
        const int tn = column_walk<true>(ws.blk_node, nb, N, 0, N, s_tile);
        if (count_n && tid < N) count_n[tid] = tn;
    } else if (count_n) {
        const int tn = column_walk<false>(ws.blk_node, nb, N, 0, N, s_tile);
        if (tid < N) count_n[tid] = tn;
    }

    // the column sums of the per-block inclusive expert prefixes are expert_offset[e+1]
    int before = 0;
    for (int c0 = 0; c0 < E; c0 += kScanThreads) {
        const int width = min(kScanThreads, E - c0);
        const int te = column_walk<false>(ws.blk_exp, nb, E, c0, width, s_tile);
        if (tid < width) s_last[tid] = te;
        __syncthreads();
        if (tid < width) {
            const int prev = tid == 0 ? before : s_last[tid - 1];
            if (count_e) count_e[c0 + tid] = te - prev;
            if (expert_offset) expert_offset[c0 + tid + 1] = te;
        }
        before = s_last[width - 1];
        __syncthreads();
    }
    if (expert_offset && tid == 0) expert_offset[0] = 0;

    if (want_expert_base) {
        // first expert-major row of expert e in each block: offset[e] plus the pairs
        // naming e in earlier blocks; one column per thread, rows in order
        for (int e = tid; e < E; e += blockDim.x) {
            int off = 0;
            for (int bb = 0; bb < nb; ++bb)
                off += e > 0 ? ws.blk_exp[static_cast<int64_t>(bb) * E + e - 1] : 0;
            int run = off;
            for (int bb = 0; bb < nb; ++bb) {
                ws.blk_exp_base[static_cast<int64_t>(bb) * E + e] = run;
                const int64_t row = static_cast<int64_t>(bb) * E;
                run += ws.blk_exp[row + e] - (e > 0 ? ws.blk_exp[row + e - 1] : 0);
            }
        }
    }

    int bad = 0;
    for (int i = tid; i < nb; i += blockDim.x) bad |= ws.blk_err[i];
    bad = __syncthreads_or(bad);
    if (tid == 0) *error_flag = bad ? kErrTopkRange : 0;
}

template <int NW>
__global__ __launch_bounds__(kBT) void layout_slot_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, FastDiv er,
    const int32_t* __restrict__ blk_prefix, const int32_t* __restrict__ rank_offset,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank, int N, FastDiv rpn,
    const int32_t* __restrict__ blk_node_prefix, int32_t* __restrict__ node_slot) {
    extern __shared__ uint64_t smem64[];
    uint64_t* s_ball = smem64;                                            // [4][R]
    int32_t* s_base = reinterpret_cast<int32_t*>(s_ball + kWavesBT * R);  // [4][R]
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kBT;
    const int64_t t = t0 + tid;

    uint64_t rm[NW], nm[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) rm[w] = nm[w] = 0;
    int bad = 0;
    if (t < T) token_masks<NW, false, true>(topk_idx + t * k, k, E, er, rpn, rm, nm, nullptr, bad);
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
    write_block_slots(s_ball, s_base, T, t0, R, token_slot, in_rank);

    if (node_slot) {
        // second pass over the same LDS, N <= R: node ballots and packed-row bases
        __syncthreads();
        wave_ballots<NW, false>(nm, N, s_ball + wave * N);
        __syncthreads();
        for (int n = tid; n < N; n += kBT) {
            int base = blk_node_prefix[b * N + n];
#pragma unroll
            for (int w = 0; w < kWavesBT; ++w) {
                s_base[w * N + n] = base;
                base += __popcll(s_ball[w * N + n]);
            }
        }
        __syncthreads();
        write_block_slots(s_ball, s_base, T, t0, N, node_slot, nullptr);
    }
}

// Length of a wave's row of 16-bit expert counts in LDS: E rounded up to even, so that
// every row starts 4-byte aligned.
__host__ __device__ inline int run_row(int E) { return (E + 1) & ~1; }
constexpr int kIdBits = 13;  // bits of an expert id below kMaxExperts
static_assert((1 << kIdBits) == kMaxExperts, "the expert-rank ballots cover every id bit");

// In-block ranks of one wave's (token, slot) pairs among the pairs of its 256-token block
// that name the same expert, in (token, slot) order. A stable ranking without a sort: wave
// w owns the block's tokens [64w, 64w + 64), i.e. its 64k pairs in (token, slot) order, and
// walks them in k rounds of 64 consecutive pairs, lane l holding pair 64r + l, so rounds in
// order are the sort order. In a round, lanes naming the same expert are matched with one
// ballot per id bit; a lane's rank is the count of its matching lanes below it plus the
// wave's running count for the expert (`run`, this wave's row of an LDS table
// [4][run_row(E)] of 16-bit counts; a wave counts at most 64 k <= 1024 pairs per expert),
// which the highest matching lane then advances. key[r] is the expert of round r's pair
// (-1 for a masked or bad id) and loc[r] its rank within the wave; after a barrier the
// caller adds the earlier waves' totals for the expert (the rows above). Issuing the
// rounds' LDS updates as atomics, all before any result is used, measured no faster.
template <int kK>
__device__ __forceinline__ void wave_expert_ranks(const int64_t* __restrict__ ids, int64_t npairs,
                                                  int k, int E, uint16_t* run,
                                                  int (&key)[kK], int (&loc)[kK]) {
    const int lane = lane_id();
    int64_t e_in[kK];
#pragma unroll
    for (int r = 0; r < kK; ++r) {  // all loads first, in flight together
        const int p = r * kWave + lane;
        e_in[r] = (r < k && p < npairs) ? ids[p] : -1;
    }
#pragma unroll
    for (int r = 0; r < kK; ++r) {
        key[r] = -1;
        loc[r] = 0;
        if (r < k) {
            const int64_t e = e_in[r];
            const int kr = (e >= 0 && e < E) ? static_cast<int>(e) : -1;
            uint64_t peers = wave_ballot(kr >= 0);
            // every id bit an expert can have (ids < EP_MAX_EXPERTS = 2^13): a bit above
            // the highest id's is zero in every lane and leaves `peers` as it is, and the
            // fixed trip count lets the rounds' ballots interleave
#pragma unroll
            for (int bit = 0; bit < kIdBits; ++bit) {
                const bool on = kr >= 0 && ((kr >> bit) & 1);
                const uint64_t m = wave_ballot(on);
                peers &= on ? m : ~m;
            }
            if (kr >= 0) {
                const int before = __popcll(peers & ((1ull << lane) - 1ull));
                const int cur = run[kr];
                loc[r] = cur + before;
                if ((peers >> lane) == 1ull) run[kr] = static_cast<uint16_t>(cur + __popcll(peers));
            }
            key[r] = kr;
        }
    }
}

// Expert-major row of every (token, slot) of one 256-token block: the block's base for
// the expert (left in the workspace by the slot launch) plus the pair's in-block rank
// (wave_expert_ranks).
template <int kK>  // rounds: k <= kK
__global__ __launch_bounds__(kBT) void layout_expert_slot_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E,
    const int32_t* __restrict__ blk_exp_base, int32_t* __restrict__ expert_slot) {
    extern __shared__ uint16_t s_run[];  // [kWavesBT][Ep], running count per wave and expert
    const int Ep = run_row(E);
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int64_t b = blockIdx.x;
    for (int i = tid; i < kWavesBT * Ep; i += kBT) s_run[i] = 0;
    __syncthreads();

    const int64_t t0 = b * kBT + static_cast<int64_t>(wave) * kWave;  // the wave's first token
    const int64_t npairs = max<int64_t>(0, min<int64_t>(kWave, T - t0)) * k;
    int key[kK];
    int loc[kK];
    wave_expert_ranks<kK>(topk_idx + t0 * k, npairs, k, E, s_run + wave * Ep, key, loc);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kK; ++r) {
        const int p = r * kWave + lane;
        if (r < k && p < npairs) {
            int slot = -1;
            if (key[r] >= 0) {
                slot = blk_exp_base[b * E + key[r]] + loc[r];
                for (int w = 0; w < wave; ++w) slot += s_run[w * Ep + key[r]];
            }
            expert_slot[t0 * k + p] = slot;
        }
    }
}

// The expert-slot launch over `blocks` blocks, with as many ranking rounds as k needs.
void launch_expert_slots(const int64_t* topk_idx, int64_t T, int k, int E,
                         const int32_t* blk_exp_base, int32_t* expert_slot, int64_t blocks,
                         hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(blocks));
    const size_t lds = sizeof(uint16_t) * kWavesBT * run_row(E);
    if (k <= 8)
        hipLaunchKernelGGL(layout_expert_slot_kernel<8>, grid, dim3(kBT), lds, stream, topk_idx, T,
                           k, E, blk_exp_base, expert_slot);
    else
        hipLaunchKernelGGL(layout_expert_slot_kernel<kExpertSlotMaxK>, grid, dim3(kBT), lds,
                           stream, topk_idx, T, k, E, blk_exp_base, expert_slot);
}

template <int NW>
hipError_t layout_impl(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                       int32_t* count_r, int32_t* count_n, int32_t* count_e, uint8_t* in_rank,
                       int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                       int32_t* expert_slot, int32_t* node_slot, int32_t* error_flag,
                       const LayoutWorkspace& ws, const RestripeTask* rs_in,
                       hipStream_t stream) {
    const int want_base = expert_slot != nullptr ? 1 : 0;
    const int64_t nb = (T + kBT - 1) / kBT;
    const FastDiv er = FastDiv::make(E / R);
    const FastDiv rpn = FastDiv::make(R / N);
    RestripeTask rs{};  // no restripe blocks unless one rides along
    if (rs_in != nullptr) rs = *rs_in;
    if (!grid_fits(nb + rs.blocks, kBT)) return hipErrorInvalidConfiguration;
    if constexpr (NW * kWave <= kFusedMaxRanks) {
        if (nb == 1) {
            const bool vec = R % 4 == 0 && reinterpret_cast<uintptr_t>(token_slot) % 16 == 0 &&
                             reinterpret_cast<uintptr_t>(in_rank) % 4 == 0;
            const bool vec_node = N % 4 == 0 && reinterpret_cast<uintptr_t>(node_slot) % 16 == 0;
            hipLaunchKernelGGL(layout_single_kernel<NW>, dim3(static_cast<unsigned>(1 + rs.blocks)),
                               dim3(kBT), sizeof(int32_t) * static_cast<size_t>(E), stream, topk_idx,
                               T, k, E, R, N, er, rpn, count_r, count_n, count_e, rank_offset,
                               expert_offset, error_flag, token_slot, in_rank, vec ? 1 : 0,
                               want_base ? ws.blk_exp_base : nullptr, node_slot, vec_node ? 1 : 0,
                               rs);
            EP_RETURN_IF_LAUNCH_FAILED();
            if (want_base) {
                launch_expert_slots(topk_idx, T, k, E, ws.blk_exp_base, expert_slot, 1,
                                    stream);
                EP_RETURN_IF_LAUNCH_FAILED();
            }
            return hipSuccess;
        }
    }
    if (nb > 0) {
        const size_t shm = sizeof(int32_t) * static_cast<size_t>(E) +
                           sizeof(uint16_t) * kWavesBT * (R + N);
        hipLaunchKernelGGL(layout_count_kernel<NW>, dim3(static_cast<unsigned>(nb + rs.blocks)),
                           dim3(kBT), shm, stream, topk_idx, T, k, E, R, N, er, rpn, ws, nb, rs);
        EP_RETURN_IF_LAUNCH_FAILED();
    }
    bool fused = false;
    if constexpr (NW * kWave <= kFusedMaxRanks)  // the fused kernel needs R <= 256
        fused = nb > 0 && nb <= kFusedMaxBlocks && nb * R <= kFusedMaxCells;
    if (fused) {
        if constexpr (NW * kWave <= kFusedMaxRanks) {
        const bool vec = R % 4 == 0 && reinterpret_cast<uintptr_t>(token_slot) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(in_rank) % 4 == 0;
        const bool vec_node = N % 4 == 0 && reinterpret_cast<uintptr_t>(node_slot) % 16 == 0;
        hipLaunchKernelGGL(layout_slot_fused_kernel<NW>,
                           dim3(static_cast<unsigned>(nb * kQuarters)), dim3(kBT), 0, stream,
                           topk_idx, T, k, E, R, N, er, static_cast<int>(nb), ws, count_r,
                           count_n, count_e, rank_offset, expert_offset, error_flag, token_slot,
                           in_rank, vec ? 1 : 0, want_base, rpn, node_slot, vec_node ? 1 : 0);
        EP_RETURN_IF_LAUNCH_FAILED();
        }
    } else {
        hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                           static_cast<int>(nb), E, R, N, ws, count_r, count_n, count_e,
                           rank_offset, expert_offset, error_flag, want_base,
                           node_slot != nullptr ? 1 : 0);
        EP_RETURN_IF_LAUNCH_FAILED();
        if (nb > 0) {
            const size_t shm =
                static_cast<size_t>(kWavesBT) * R * (sizeof(uint64_t) + sizeof(int32_t));
            hipLaunchKernelGGL(layout_slot_kernel<NW>, dim3(static_cast<unsigned>(nb)), dim3(kBT),
                               shm, stream, topk_idx, T, k, E, R, er, ws.blk_rank, rank_offset,
                               token_slot, in_rank, N, rpn, ws.blk_node, node_slot);
            EP_RETURN_IF_LAUNCH_FAILED();
        }
    }
    if (want_base && nb > 0) {
        launch_expert_slots(topk_idx, T, k, E, ws.blk_exp_base, expert_slot, nb, stream);
        EP_RETURN_IF_LAUNCH_FAILED();
    }
    return hipSuccess;
}

// ------------------------------------------------------------------- the counts path
// Count launch of ep_layout_counts (R <= 64, one mask word per token). Each block counts
// its 256 tokens as layout_count_kernel does and publishes, for ep_dispatch_layout: each
// token's rank mask, each wave's rank ballots and the tokens of its earlier waves per
// rank, the block's rank and node counts and the inclusive prefix of its expert
// histogram. A batch of at most kCountsLocalBlocks blocks stops there: the dispatch's
// waves sum the per-block rank counts themselves. In a larger batch every block then takes
// a ticket; the block that draws the last one (no block waits for another) turns the
// blocks' rank counts into the receive row of each block's first token on each rank and
// zeroes the ticket for the next call. Blocks past `nlb` run the dense restripe riding
// along in this launch.
template <int kK>  // 0: no expert ranks; else their rounds, k <= kK
__global__ __launch_bounds__(kBT) void layout_counts_kernel(
    const int64_t* __restrict__ topk_idx, int64_t T, int k, int E, int R, int N, FastDiv er,
    FastDiv rpn, CountsWorkspace cw, int nlb, RestripeTask rs, int32_t* __restrict__ error_flag,
    int32_t* __restrict__ expert_rank) {
    if (static_cast<int>(blockIdx.x) >= nlb) {
        restripe_task_block(rs, static_cast<int64_t>(blockIdx.x) - nlb);
        return;
    }
    extern __shared__ int32_t s_hist[];                      // [E], then (expert_rank) [4][E] u16
    __shared__ uint64_t s_ball[kWavesBT * kCountsMaxRanks];  // [4][R] rank ballots per wave
    __shared__ uint16_t s_wn[kWavesBT * kCountsMaxRanks];    // [4][N] node counts per wave
    __shared__ int32_t s_part[kBT];                          // last block: partial column sums
    __shared__ int32_t s_ro[kCountsMaxRanks];                // last block: rank offsets
    __shared__ int32_t s_scan[17];
    __shared__ int32_t s_last;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int b = blockIdx.x;
    const int64_t t = static_cast<int64_t>(b) * kBT + tid;

    // The flag is cleared by block 0 as it starts (the hardware starts blocks in index
    // order, and a block raises a bit only after its counting pass, microseconds later) and
    // is only ORed into afterwards, so the last block cannot erase a bit another block
    // raised.
    if (b == 0 && tid == 0) __hip_atomic_store(error_flag, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint16_t* s_run = reinterpret_cast<uint16_t*>(s_hist + E);
    const int Ep = run_row(E);
    for (int e = tid; e < E; e += kBT) s_hist[e] = 0;
    if constexpr (kK > 0)
        for (int i = tid; i < kWavesBT * Ep; i += kBT) s_run[i] = 0;
    __syncthreads();
    uint64_t rm[1] = {0}, nm[1] = {0};
    int bad = 0;
    if (t < T) {
        token_masks<1, true, true>(topk_idx + t * k, k, E, er, rpn, rm, nm, s_hist, bad);
        cw.mask[t] = rm[0];
    }
    wave_ballots<1, false>(rm, R, s_ball + wave * R);
    wave_ballots<1, true>(nm, N, s_wn + wave * N);
    __syncthreads();

    for (int i = tid; i < kWavesBT * R; i += kBT) {
        const int w = i / R, r = i - w * R;
        int before = 0;
        for (int v = 0; v < w; ++v) before += __popcll(s_ball[v * R + r]);
        cw.ball[static_cast<int64_t>(b) * kWavesBT * R + i] = s_ball[i];
        cw.pfx[static_cast<int64_t>(b) * kWavesBT * R + i] = before;
        if (w == kWavesBT - 1) cw.blk_rank[static_cast<int64_t>(b) * R + r] = before + __popcll(s_ball[i]);
    }
    for (int n = tid; n < N; n += kBT) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) c += s_wn[w * N + n];
        cw.blk_node[static_cast<int64_t>(b) * N + n] = c;
    }
    int carry = 0;  // inclusive prefix of the block's expert histogram
    for (int c0 = 0; c0 < E; c0 += kBT) {
        const int e = c0 + tid;
        const int h = e < E ? s_hist[e] : 0;
        int chunk = 0;
        const int ex = block_exclusive_scan(h, s_scan, chunk);
        if (e < E) cw.blk_exp[static_cast<int64_t>(b) * E + e] = carry + ex + h;
        carry += chunk;
    }
    const int any_bad = __syncthreads_or(bad);
    if constexpr (kK > 0) {  // each pair's rank among the block's pairs naming its expert
        const int lane = lane_id();
        const int64_t t0 = static_cast<int64_t>(b) * kBT + static_cast<int64_t>(wave) * kWave;
        const int64_t npairs = max<int64_t>(0, min<int64_t>(kWave, T - t0)) * k;
        int key[kK];
        int loc[kK];
        wave_expert_ranks<kK>(topk_idx + t0 * k, npairs, k, E, s_run + wave * Ep, key, loc);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kK; ++r) {
            const int p = r * kWave + lane;
            if (r < k && p < npairs) {
                int rank = -1;
                if (key[r] >= 0) {
                    rank = loc[r];
                    for (int w = 0; w < wave; ++w) rank += s_run[w * Ep + key[r]];
                }
                expert_rank[t0 * k + p] = rank;
            }
        }
    }
    if (nlb <= kCountsLocalBlocks) {  // no cross-block phase: the dispatch sums the counts
        if (tid == 0 && any_bad) raise_error(error_flag, kErrTopkRange);
        return;
    }
    if (tid == 0) cw.blk_err[b] = any_bad;

    // Publish, then draw a ticket. Each wave waits until its table stores have reached
    // the L2; after the barrier, thread 0's device-scope release fence writes the XCD's
    // L2 back once for the whole block (a fence per wave writes it back four times over,
    // 3 us more at 64 blocks on MI355X).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int drawn = atomicAdd(cw.ticket, 1);
        s_last = drawn == nlb - 1;
        // a ticket outside [0, nlb): the ticket was not zero on entry
        if (drawn < 0 || drawn >= nlb) raise_error(error_flag, kErrWorkspace);
    }
    __syncthreads();
    if (!s_last) return;
    // acquire: the other blocks' tables (one fence, ordered before the block's loads by
    // the barrier, as on the release side)
    if (tid == 0) __threadfence();
    __syncthreads();

    // rank columns of blk_rank [nb][R]: thread (c, r) sums rows [c q, c q + q) of column r
    const int C = kBT / R;
    const int q = (nlb + C - 1) / C;
    const int r = tid % R, c = tid / R;
    const bool col = c < C;
    const int b0 = col ? min(nlb, c * q) : 0, b1 = col ? min(nlb, b0 + q) : 0;
    const int32_t* __restrict__ blk_rank = cw.blk_rank;
    int32_t* __restrict__ glob = cw.glob;
    int part = 0;
    int keep[kBatch];  // the first batch's rows, reused below when they are all of them
    for (int bb = b0; bb < b1; bb += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = bb + u < b1 ? blk_rank[static_cast<int64_t>(bb + u) * R + r] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            part += v[u];
            if (bb == b0) keep[u] = v[u];
        }
    }
    int any = 0;
    for (int bb = tid; bb < nlb; bb += kBT) any |= cw.blk_err[bb];
    if (col) s_part[c * R + r] = part;
    __syncthreads();
    int tot = 0;
    if (tid < R) {  // exclusive prefix of the parts over c, per rank
        for (int cc = 0; cc < C; ++cc) {
            const int p = s_part[cc * R + tid];
            s_part[cc * R + tid] = tot;
            tot += p;
        }
    }
    int M = 0;
    const int ro = block_exclusive_scan(tid < R ? tot : 0, s_scan, M);
    if (tid < R) s_ro[tid] = ro;
    __syncthreads();
    if (col) {  // receive row of each block's first token on rank r
        int run = s_ro[r] + s_part[c * R + r];
        for (int bb = b0; bb < b1; bb += kBatch) {
            int v[kBatch];  // a batch of rows in flight at once (L2 hits after the sums)
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                v[u] = b1 - b0 <= kBatch ? keep[u]
                       : bb + u < b1     ? blk_rank[static_cast<int64_t>(bb + u) * R + r]
                                         : 0;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (bb + u < b1) glob[static_cast<int64_t>(bb + u) * R + r] = run;
                run += v[u];
            }
        }
    }
    any = __syncthreads_or(any);
    if (tid == 0) {
        if (any) raise_error(error_flag, kErrTopkRange);
        __hip_atomic_store(cw.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------- layout + dispatch in one launch
// ep_layout_dispatch: the layout, the dispatch and the restripe of a batch of at most one
// 256-token group in one launch, no block waiting for another.
// - Block 0 is the single-group layout (layout_single_block) without the slots: counts and
//   offsets. It clears the error flag as it starts and ORs its bit in at its end. Another
//   block raises a bit (a receive row past the capacity) only after its ids' round trip
//   and a block barrier, microseconds after block 0, which the hardware starts first.
// - Blocks 1 .. ndisp each hold four (token, destination) waves of the dispatch, as
//   dispatch_layout_kernel's. A block recomputes the group's rank masks and each wave's
//   rank ballots in LDS while its rows' loads are in flight (the ids are 16 KiB at top-8
//   and are L2 hits after the first blocks), and forms its receive rows from them: rank r's offset is
//   the scan of the group's rank totals across the wave, and a token's row on r adds the
//   group's tokens before it on r. A token's first wave also writes its token_slot and
//   bitmap rows, which keeps those writes off the layout block, the longest one.
// - The blocks after those run the dense restripe.
// This replaces the counts path's count launch for such a batch: its fixed cost is the
// largest part of a decode-sized step.
template <int WPL, bool kMulti>
__global__ __launch_bounds__(kBT) void layout_dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int E, int R, int N, FastDiv er,
    FastDiv rpn, FastDiv D, int ndisp, RestripeTask rs, int32_t* __restrict__ count_r,
    int32_t* __restrict__ count_n, int32_t* __restrict__ count_e,
    int32_t* __restrict__ rank_offset, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ token_slot, uint8_t* __restrict__ in_rank,
    u32x4* __restrict__ recv_x, int64_t* __restrict__ recv_idx, float* __restrict__ recv_w,
    int32_t* __restrict__ recv_src, int64_t cap, int32_t* __restrict__ error_flag) {
    const int b = blockIdx.x;
    if (b == 0) {  // counts and offsets; the dispatch waves write the slots
        layout_single_block<1>(topk_idx, T, k, E, R, N, er, rpn, count_r, count_n, count_e,
                               rank_offset, expert_offset, error_flag, nullptr, nullptr, 0,
                               nullptr, nullptr, 0, true);
        return;
    }
    if (b > ndisp) {
        restripe_task_block(rs, static_cast<int64_t>(b - 1 - ndisp));
        return;
    }
    __shared__ uint64_t s_mask[kBT];                          // each token's rank mask
    __shared__ uint64_t s_wball[kWavesBT * kCountsMaxRanks];  // [4][R] rank ballots per wave
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = lane_id();
    int64_t t;
    int d;
    // a wave past the batch still computes its share of the masks and meets the barrier
    const bool live = dest_wave_at((b - 1) * kWavesBT + wave, 0, T, D, t, d);
    if (!live) t = 0;
    // Thread i forms token i's rank mask. Its first kBatch ids are loaded before the row's
    // first pass, unconditionally at clamped indices (out-of-range ones are ignored below),
    // so the mask is formed while the row is still in flight.
    const int ti = min(tid, static_cast<int>(T) - 1);
    const int64_t* ids = topk_idx + static_cast<int64_t>(ti) * k;
    int64_t ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) ev[u] = ids[min(u, k - 1)];
    const Routing rt(topk_idx + t * k, topk_w ? topk_w + t * k : nullptr, k, recv_idx || recv_w);
    const u32x4* xr = x + t * V;
    u32x4 v[WPL];
    load_row_cached(v, xr, 0, V);  // first pass
    uint64_t rm[1] = {0};
    const bool own = tid < T;
    auto add_id = [&](int64_t e, bool use) {
        if (use && e >= 0 && e < E) rm[0] |= 1ull << er.div(static_cast<int>(e));
    };
#pragma unroll
    for (int u = 0; u < kBatch; ++u) add_id(ev[u], own && u < k);
    for (int j0 = kBatch; j0 < k; j0 += kBatch) {  // top-k beyond kBatch: the rest in turn
#pragma unroll
        for (int u = 0; u < kBatch; ++u) ev[u] = ids[min(j0 + u, k - 1)];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) add_id(ev[u], own && j0 + u < k);
    }
    s_mask[tid] = rm[0];
    wave_ballots<1, false>(rm, R, s_wball + wave * R);
    __syncthreads();
    if (!live) return;
    const int wt = static_cast<int>(t) / kWave, lt = static_cast<int>(t) % kWave;
    int tot = 0, before = 0;  // lane r: the group's tokens on r, and those before t
    if (lane < R) {
#pragma unroll
        for (int w = 0; w < kWavesBT; ++w) {
            const uint64_t bl = s_wball[w * R + lane];
            const int c = __popcll(bl);
            tot += c;
            if (w < wt) before += c;
            else if (w == wt) before += __popcll(bl & ((1ull << lt) - 1ull));
        }
    }
    int xs = tot;  // inclusive scan of the totals across the wave
    for (int s = 1; s < kWave; s <<= 1) {
        const int y = __shfl_up(xs, s, kWave);
        if (lane >= s) xs += y;
    }
    const uint64_t m = s_mask[t];
    const bool on = lane < R && ((m >> lane) & 1ull);
    const int32_t slot = on ? xs - tot + before : -1;
    if (d == 0 && lane < R) {  // the token's first wave writes its slot row and bitmap row
        token_slot[t * R + lane] = slot;
        if (in_rank) in_rank[t * R + lane] = on ? 1 : 0;
    }
    uint64_t rest = m;  // the token's d-th destination rank, ascending
    for (int i = 0; i < d && rest; ++i) rest &= rest - 1;
    if (!rest) return;
    const int rd = __builtin_ctzll(rest);
    const int64_t sd = __builtin_amdgcn_readlane(slot, rd);
    if (sd >= cap) {
        if (lane == 0) raise_error(error_flag, kErrRecvOverflow);
        return;
    }
    for (int v0 = 0; v0 < V; v0 += kWave * WPL) {
        if (v0 != 0) load_row_cached(v, xr, v0, V);
        put_row<WPL, true>(v, v0, V, sd, rd, rt, er.d, static_cast<int32_t>(t), recv_x, recv_idx,
                           recv_w, recv_src);
        if constexpr (!kMulti) break;
    }
}

__global__ __launch_bounds__(kBT) void zero_ints_kernel(ZeroInts z) {
#pragma unroll
    for (int a = 0; a < kZeroArrays; ++a)
        for (int i = threadIdx.x; i < z.n[a]; i += kBT) z.p[a][i] = 0;
}

}  // namespace

hipError_t launch_zero_ints(const ZeroInts& z_in, hipStream_t stream) {
    ZeroInts z = z_in;
    int total = 0;
    for (int a = 0; a < kZeroArrays; ++a) {
        if (!z.p[a]) z.n[a] = 0;
        total += z.n[a];
    }
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(kBT), 0, stream, z);
    return hipGetLastError();
}

namespace {
// Batches that ep_get_layout counts with the counts path's count launch and turns into
// slots from its tables (counts_slots_kernel), when no node or expert slots are asked for:
// more than one 256-token block (one block takes the one-block kernel) and at most
// kCountsLocalBlocks, whose rows need no cross-block phase; one rank-mask word per token.
bool counts_layout_shape(int64_t T, int R) {
    const int64_t nb = (T + kBT - 1) / kBT;
    return R <= kCountsMaxRanks && nb > 1 && nb <= kCountsLocalBlocks;
}
}  // namespace

size_t layout_workspace_bytes(int64_t T, int E, int R, int N) {
    const size_t nb = static_cast<size_t>((T + kBT - 1) / kBT);
    const size_t own = align_up(nb * R * 4, 256) + align_up(nb * N * 4, 256) +
                       2 * align_up(nb * E * 4, 256) + align_up(nb * 4, 256);
    // batches that take the counts path's tables need room for those instead
    return counts_layout_shape(T, R) ? std::max(own, counts_workspace_bytes(T, E, R, N)) : own;
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
    ws.blk_exp_base = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * E * 4, 256);
    ws.blk_err = reinterpret_cast<int32_t*>(p);
    return ws;
}

namespace {
constexpr int kScratchMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// Looked up with the device current, once per device; later calls read the kept address.
hipError_t layout_scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                         int32_t* count_r, int32_t* count_n, int32_t* count_e, uint8_t* in_rank,
                         int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                         int32_t* expert_slot, int32_t* node_slot, int32_t* error_flag,
                         void* ws_base, const RestripeTask* rs, hipStream_t stream) {
    if (counts_layout_shape(T, R) && !expert_slot && !node_slot) {
        const CountsWorkspace cw = carve_counts_workspace(ws_base, T, E, R, N);
        const hipError_t e =
            launch_layout_counts(topk_idx, T, k, E, R, N, error_flag, nullptr, cw, rs, stream);
        if (e != hipSuccess) return e;
        return launch_counts_slots(T, E, R, N, cw, token_slot, in_rank, count_r, rank_offset,
                                   count_n, count_e, expert_offset, stream);
    }
    const LayoutWorkspace ws = carve_layout_workspace(ws_base, T, E, R, N);
#define EP_LAYOUT_CASE(NW)                                                                     \
    return layout_impl<NW>(topk_idx, T, k, E, R, N, count_r, count_n, count_e, in_rank,        \
                           rank_offset, expert_offset, token_slot, expert_slot, node_slot,      \
                           error_flag, ws, rs, stream)
    if (R <= 64) EP_LAYOUT_CASE(1);
    if (R <= 128) EP_LAYOUT_CASE(2);
    if (R <= 256) EP_LAYOUT_CASE(4);
    if (R <= 512) EP_LAYOUT_CASE(8);
    EP_LAYOUT_CASE(16);
#undef EP_LAYOUT_CASE
}

size_t counts_workspace_bytes(int64_t T, int E, int R, int N) {
    const size_t nb = static_cast<size_t>((T + kBT - 1) / kBT);
    return align_up(4, 256) + 2 * align_up(nb * R * 4, 256) +
           align_up(nb * kWavesBT * R * 4, 256) + align_up(nb * kWavesBT * R * 8, 256) +
           align_up(static_cast<size_t>(T) * 8, 256) + align_up(nb * 4, 256) +
           align_up(nb * N * 4, 256) + align_up(nb * E * 4, 256);
}

CountsWorkspace carve_counts_workspace(void* base, int64_t T, int E, int R, int N) {
    const size_t nb = static_cast<size_t>((T + kBT - 1) / kBT);
    char* p = static_cast<char*>(base);
    CountsWorkspace cw;
    cw.ticket = reinterpret_cast<int32_t*>(p);
    p += align_up(4, 256);
    cw.blk_rank = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * R * 4, 256);
    cw.glob = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * R * 4, 256);
    cw.pfx = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * kWavesBT * R * 4, 256);
    cw.ball = reinterpret_cast<uint64_t*>(p);
    p += align_up(nb * kWavesBT * R * 8, 256);
    cw.mask = reinterpret_cast<uint64_t*>(p);
    p += align_up(static_cast<size_t>(T) * 8, 256);
    cw.blk_err = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * 4, 256);
    cw.blk_node = reinterpret_cast<int32_t*>(p);
    p += align_up(nb * N * 4, 256);
    cw.blk_exp = reinterpret_cast<int32_t*>(p);
    return cw;
}

hipError_t launch_layout_counts(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                                int32_t* error_flag, int32_t* expert_rank,
                                const CountsWorkspace& cw, const RestripeTask* rs_in,
                                hipStream_t stream) {
    RestripeTask rs{};
    if (rs_in != nullptr) rs = *rs_in;
    const int64_t nb = (T + kBT - 1) / kBT;
    if (nb == 0) {  // an empty batch: no error, nothing to count or restripe
        ZeroInts z{};
        z.p[0] = error_flag;
        z.n[0] = 1;
        return launch_zero_ints(z, stream);
    }
    if (nb > INT32_MAX || !grid_fits(nb + rs.blocks, kBT)) return hipErrorInvalidConfiguration;
    const FastDiv er = FastDiv::make(E / R);
    const FastDiv rpn = FastDiv::make(R / N);
    const size_t run_bytes = sizeof(uint16_t) * kWavesBT * static_cast<size_t>(run_row(E));
    const size_t lds = sizeof(int32_t) * static_cast<size_t>(E) + (expert_rank ? run_bytes : 0);
    const dim3 grid(static_cast<unsigned>(nb + rs.blocks));
    if (!expert_rank)
        hipLaunchKernelGGL(layout_counts_kernel<0>, grid, dim3(kBT), lds, stream, topk_idx, T, k,
                           E, R, N, er, rpn, cw, static_cast<int>(nb), rs, error_flag, expert_rank);
    else if (k <= 8)
        hipLaunchKernelGGL(layout_counts_kernel<8>, grid, dim3(kBT), lds, stream, topk_idx, T, k,
                           E, R, N, er, rpn, cw, static_cast<int>(nb), rs, error_flag, expert_rank);
    else
        hipLaunchKernelGGL(layout_counts_kernel<kExpertSlotMaxK>, grid, dim3(kBT), lds, stream,
                           topk_idx, T, k, E, R, N, er, rpn, cw, static_cast<int>(nb), rs,
                           error_flag, expert_rank);
    return hipGetLastError();
}


hipError_t launch_layout_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                                  int64_t T, int H, int k, int E, int R, int N,
                                  const RestripeTask* rs_in, int32_t* count_r,
                                  int32_t* rank_offset, int32_t* count_n, int32_t* count_e,
                                  int32_t* expert_offset, int32_t* token_slot, uint8_t* in_rank,
                                  void* recv_x, int64_t* recv_idx, float* recv_w,
                                  int32_t* recv_src, int64_t cap, int32_t* error_flag,
                                  hipStream_t stream) {
    if (T == 0) {  // an empty batch: no error, zero counts and offsets, nothing to move
        const ZeroInts z{{error_flag, count_r, rank_offset, count_n, count_e, expert_offset},
                         {1, R, R + 1, N, E, E + 1}};
        return launch_zero_ints(z, stream);
    }
    if (T > kBT || R > kCountsMaxRanks) return hipErrorInvalidValue;
    RestripeTask rs{};
    if (rs_in != nullptr) rs = *rs_in;
    const int V = H / 8;
    const int D = std::min(k, R);  // waves per token
    const int ndisp = static_cast<int>((T * D + kWavesBT - 1) / kWavesBT);
    if (!grid_fits(1 + ndisp + rs.blocks, kBT)) return hipErrorInvalidConfiguration;
    const FastDiv er = FastDiv::make(E / R), rpn = FastDiv::make(R / N), fd = FastDiv::make(D);
    const dim3 grid(static_cast<unsigned>(1 + ndisp + rs.blocks));
    const size_t shm = sizeof(int32_t) * static_cast<size_t>(E);
    return with_row_width<14, false>(V, [&](auto wpl, auto multi) {
        hipLaunchKernelGGL((layout_dispatch_kernel<decltype(wpl)::value, decltype(multi)::value>),
                           grid, dim3(kBT), shm, stream, static_cast<const u32x4*>(x), topk_idx,
                           topk_w, T, V, k, E, R, N, er, rpn, fd, ndisp, rs, count_r, count_n,
                           count_e, rank_offset, expert_offset, token_slot, in_rank,
                           static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src, cap,
                           error_flag);
    });
}

}  // namespace ep
