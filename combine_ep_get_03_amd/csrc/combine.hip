// combine.hip -- gather-reduce of per-rank partial rows on gfx950.
//
// out[t][h] = bf16( sum over ranks r in ascending order with s = token_slot[t][r] >= 0 of
// partial[s][h] ), summed in fp32 from +0.0f and rounded once to nearest-even. Combine
// moves the same payload as dispatch in the other direction ("[PR #347] Feature/sm free
// normal kernel", section 3.2.1 tables give combine the same bytes as dispatch).
//
// Design: a block owns a few consecutive tokens; wave ballots over the token_slot row
// compact each token's source slots (ascending rank) into LDS. Each lane then owns one
// 128-bit word (8 bf16) of a token's output: it issues the loads of up to 8 source rows
// at once, widens bf16 to fp32 by shifting, adds in rank order and rounds with the
// gfx950 packed bf16 convert. HBM-read bound (about 7 reads per write at top-8).
// A 1024-thread block per 7168-wide token puts the loads of every source row of the
// token in flight together; on MI355X that measured about 8% faster than 256 threads
// looping over the row.
//
// The same kernel serves the two-phase combine ("[PR #347] Feature/sm free normal
// kernel", sections 2.1 and 3.3.2): its send phase sums, per token and node, the rows of
// the node's ranks into the node's staged row (grouped mode); its receive phase sums each
// token's staged node rows, addressed by node-local slots, into the output.
#include "ep_internal.hpp"

namespace ep {
namespace {

#ifndef EP_COMBINE_BLOCK_WORDS
#define EP_COMBINE_BLOCK_WORDS 1024
#endif
#ifndef EP_COMBINE_THREADS
#define EP_COMBINE_THREADS 1024
#endif

constexpr int kCT = EP_COMBINE_THREADS;               // threads per block
constexpr int kCLoads = 8;                            // source rows loaded together
constexpr int kCBlockWords = EP_COMBINE_BLOCK_WORDS;  // output words a block aims to own

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const uint16_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
    const uint16_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

// Sum of the c source rows listed at sl (ascending), word vv, fp32 from +0.0f, rounded
// once to bf16. Up to kCLoads rows are loaded together.
__device__ __forceinline__ u32x4 sum_rows(const u32x4* __restrict__ partial,
                                          const int32_t* sl, int c, int V, int vv) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int d0 = 0; d0 < c; d0 += kCLoads) {
        u32x4 p[kCLoads];
#pragma unroll
        for (int i = 0; i < kCLoads; ++i)
            if (d0 + i < c) p[i] = load_stream(partial + static_cast<int64_t>(sl[d0 + i]) * V + vv);
#pragma unroll
        for (int i = 0; i < kCLoads; ++i) {
            if (d0 + i < c) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = acc[2 * q] + lo_bf16(p[i][q]);
                    acc[2 * q + 1] = acc[2 * q + 1] + hi_bf16(p[i][q]);
                }
            }
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16(acc[2 * q], acc[2 * q + 1]);
    return o;
}

// Grouped sums of word vv: the c = gs[G] source rows listed at sl (ascending) form G
// consecutive groups, group g being sl[gs[g] .. gs[g+1]); group g's fp32 sum (from +0.0f,
// in list order) is rounded once to bf16 and stored at row g * obase + os[g] of out when
// os[g] >= 0 (os[g] >= obase is an overflow: skipped, error bit set). Up to kCLoads rows
// of the whole list are loaded together, so a lane has the loads of every group in
// flight at once rather than one group's at a time. Against one (group, word) per lane
// (about two loads in flight at top-8 over 4 nodes), measured on MI355X at 7168 channels:
// 111.2 against 114.4 us at 4096 tokens, 531.8 against 571.4 at 16384 over 8 nodes.
__device__ __forceinline__ void sum_groups(const u32x4* __restrict__ partial, const int32_t* sl,
                                           const int32_t* gs, const int32_t* os, int G, int V,
                                           int vv, int64_t obase, u32x4* __restrict__ out,
                                           int32_t& errbits) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    int g = 0;
    auto close_group = [&]() {
        const int32_t o = os[g];
        if (o >= 0) {
            if (o >= obase) {
                errbits |= kErrRecvOverflow;
            } else {
                u32x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = pack_bf16(acc[2 * q], acc[2 * q + 1]);
                store_stream(out + (g * obase + o) * V + vv, w);
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        ++g;
    };
    const int c = gs[G];
    for (int d0 = 0; d0 < c; d0 += kCLoads) {
        u32x4 p[kCLoads];
#pragma unroll
        for (int i = 0; i < kCLoads; ++i)
            if (d0 + i < c) p[i] = load_stream(partial + static_cast<int64_t>(sl[d0 + i]) * V + vv);
#pragma unroll
        for (int i = 0; i < kCLoads; ++i) {
            if (d0 + i < c) {
                while (d0 + i >= gs[g + 1]) close_group();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = acc[2 * q] + lo_bf16(p[i][q]);
                    acc[2 * q + 1] = acc[2 * q + 1] + hi_bf16(p[i][q]);
                }
            }
        }
    }
    while (g < G) close_group();
}

// Source slots: row t of slot_tab holds C columns; column c with slot s >= 0 names source
// row s + c * cbase (with cbase > 0 a slot must also be below cbase). Without kGrouped
// every token's sources are summed into out[t]. With kGrouped the C columns form G
// consecutive groups of C / G; group g of token t is summed into row
// g * obase + out_slot[t][g] of out when out_slot[t][g] >= 0 (the two-phase combine's
// send phase: one sum per node of the token).
template <bool kGrouped>
__device__ __forceinline__ void combine_body(
    const u32x4* __restrict__ partial, int64_t rows, const int32_t* __restrict__ slot_tab,
    int C, int64_t cbase, int64_t T, int V, u32x4* __restrict__ out,
    const int32_t* __restrict__ out_slot, int G, int64_t obase,
    int32_t* __restrict__ error_flag, int tpb) {
    extern __shared__ int32_t smem[];
    // flat: s_cnt [tpb]; grouped: group starts [tpb][G + 1] and output rows [tpb][G]
    const int head = kGrouped ? tpb * (2 * G + 1) : tpb;
    int32_t* s_cnt = smem;
    int32_t* s_gs = smem;
    int32_t* s_os = smem + tpb * (G + 1);
    int32_t* s_slot = smem + head;  // [tpb][C]
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int gsize = C / G;
    const int64_t ngroups = (T + tpb - 1) / tpb;
    int32_t errbits = 0;

    for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        const int64_t t0 = grp * tpb;
        const int nt = static_cast<int>(min<int64_t>(tpb, T - t0));

        // source slots of each token, ascending column, compacted by wave ballots
        for (int tt = wave; tt < nt; tt += kCT / kWave) {
            const int32_t* srow = slot_tab + (t0 + tt) * C;
            int found = 0;
            for (int c0 = 0; c0 < C; c0 += kWave) {
                const int c = c0 + lane;
                int32_t s = c < C ? srow[c] : -1;
                int64_t a = static_cast<int64_t>(s) + c * cbase;
                if (s >= 0 && (a >= rows || (cbase > 0 && s >= cbase))) {
                    errbits |= kErrSlotRange;
                    s = -1;
                }
                const uint64_t m = wave_ballot(s >= 0);
                const int pos = found + lanes_below(m);
                if (s >= 0) s_slot[tt * C + pos] = static_cast<int32_t>(a);
                if (kGrouped && c < C && c % gsize == 0) s_gs[tt * (G + 1) + c / gsize] = pos;
                found += __popcll(m);
            }
            if (lane == 0) {
                if (kGrouped) s_gs[tt * (G + 1) + G] = found;
                else s_cnt[tt] = found;
            }
            if (kGrouped) {
                for (int g = lane; g < G; g += kWave) s_os[tt * G + g] = out_slot[(t0 + tt) * G + g];
            }
        }
        __syncthreads();

        if (!kGrouped) {
            const int total = nt * V;
            for (int f = tid; f < total; f += kCT) {
                const int tt = f / V;
                const int vv = f - tt * V;
                store_stream(out + (t0 + tt) * V + vv,
                             sum_rows(partial, s_slot + tt * C, s_cnt[tt], V, vv));
            }
        } else {
            const int total = nt * V;
            for (int f = tid; f < total; f += kCT) {
                const int tt = f / V;
                const int vv = f - tt * V;
                sum_groups(partial, s_slot + tt * C, s_gs + tt * (G + 1), s_os + tt * G, G, V, vv,
                           obase, out, errbits);
            }
        }
        if (gridDim.x < ngroups) __syncthreads();  // the next group reuses the LDS lists
    }
    if (errbits) raise_error(error_flag, errbits);
}

// One kernel name per call, so traces and counters tell them apart.
#define EP_COMBINE_KERNEL(NAME, GROUPED)                                                       \
    __global__ __launch_bounds__(kCT) void NAME(                                             \
        const u32x4* __restrict__ partial, int64_t rows, const int32_t* __restrict__ slot_tab, \
        int C, int64_t cbase, int64_t T, int V, u32x4* __restrict__ out,                     \
        const int32_t* __restrict__ out_slot, int G, int64_t obase,                          \
        int32_t* __restrict__ error_flag, int tpb) {                                          \
        combine_body<GROUPED>(partial, rows, slot_tab, C, cbase, T, V, out, out_slot, G, obase, \
                              error_flag, tpb);                                               \
    }
EP_COMBINE_KERNEL(combine_kernel, false)       // ep_combine
EP_COMBINE_KERNEL(combine_send_kernel, true)   // ep_combine_send
EP_COMBINE_KERNEL(combine_recv_kernel, false)  // ep_combine_recv
#undef EP_COMBINE_KERNEL

}  // namespace

// Tokens per block: enough words for about kCBlockWords outputs, and LDS lists within
// 32 KB.
static int combine_tokens_per_block(int V, int lds_ints_per_token) {
    int tpb = std::max(1, std::min(64, kCBlockWords / V));
    return std::max(1, std::min(tpb, 8192 / lds_ints_per_token));
}

// max_blocks > 0 caps the grid: each block then takes token groups b, b + grid, ...
template <bool kGrouped, typename Kernel>
static hipError_t launch_combine_impl(Kernel kernel, const void* partial, int64_t rows,
                                      const int32_t* slot_tab, int C, int64_t cbase, int64_t T,
                                      int H, void* out, const int32_t* out_slot, int G,
                                      int64_t obase, int32_t* error_flag, int max_blocks,
                                      hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int per_token = C + (kGrouped ? 2 * G + 1 : 1);
    const int tpb = combine_tokens_per_block(V, per_token);
    const int64_t groups = (T + tpb - 1) / tpb;
    const int64_t grid = max_blocks > 0 ? std::min<int64_t>(groups, max_blocks) : groups;
    if (!grid_fits(grid, kCT)) return hipErrorInvalidConfiguration;
    const size_t shm = sizeof(int32_t) * static_cast<size_t>(tpb) * per_token;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kCT),
                       shm, stream, static_cast<const u32x4*>(partial), rows, slot_tab, C, cbase,
                       T, V, static_cast<u32x4*>(out), out_slot, G, obase, error_flag, tpb);
    return hipGetLastError();
}

hipError_t launch_combine(const void* partial, int64_t rows, const int32_t* token_slot,
                          int64_t T, int H, int R, void* out, int32_t* error_flag,
                          hipStream_t stream) {
    return launch_combine_impl<false>(combine_kernel, partial, rows, token_slot, R, 0, T, H, out,
                                      nullptr, 1, 0, error_flag, 0, stream);
}

hipError_t launch_combine_send(const void* partial, int64_t rows, const int32_t* token_slot,
                               int64_t T, int H, int R, int N, const int32_t* node_slot,
                               int64_t Tmax, void* stage, int32_t* error_flag, int max_blocks,
                               hipStream_t stream) {
    return launch_combine_impl<true>(combine_send_kernel, partial, rows, token_slot, R, 0, T, H,
                                     stage, node_slot, N, Tmax, error_flag, max_blocks, stream);
}

hipError_t launch_combine_recv(const void* stage, int N, int64_t Tmax, const int32_t* node_slot,
                               int64_t T, int H, void* out, int32_t* error_flag,
                               hipStream_t stream) {
    return launch_combine_impl<false>(combine_recv_kernel, stage, static_cast<int64_t>(N) * Tmax,
                                      node_slot, N, Tmax, T, H, out, nullptr, 1, 0, error_flag,
                                      0, stream);
}

}  // namespace ep
