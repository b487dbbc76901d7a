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
#include "ep_internal.hpp"

namespace ep {
namespace {

#ifndef EP_COMBINE_BLOCK_WORDS
#define EP_COMBINE_BLOCK_WORDS 1024
#endif
#ifndef EP_COMBINE_THREADS
#define EP_COMBINE_THREADS 1024
#endif
#ifndef EP_COMBINE_GRID_CAP
#define EP_COMBINE_GRID_CAP 0
#endif

constexpr int kCT = EP_COMBINE_THREADS;               // threads per block
constexpr int kCLoads = 8;                            // source rows loaded together
constexpr int kCBlockWords = EP_COMBINE_BLOCK_WORDS;  // output words a block aims to own
constexpr int kCGridCap = EP_COMBINE_GRID_CAP;        // 0: one block per token group

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const uint16_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
    const uint16_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

__global__ __launch_bounds__(kCT) void combine_kernel(const u32x4* __restrict__ partial,
                                                      int64_t rows,
                                                      const int32_t* __restrict__ token_slot,
                                                      int64_t T, int V, int R,
                                                      u32x4* __restrict__ out,
                                                      int32_t* __restrict__ error_flag, int tpb) {
    extern __shared__ int32_t smem[];
    int32_t* s_cnt = smem;          // [tpb]
    int32_t* s_slot = s_cnt + tpb;  // [tpb][R]
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int64_t ngroups = (T + tpb - 1) / tpb;
    int32_t errbits = 0;

    for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
        const int64_t t0 = grp * tpb;
        const int nt = static_cast<int>(min<int64_t>(tpb, T - t0));

        // source slots of each token, ascending rank, compacted by wave ballots
        for (int tt = wave; tt < nt; tt += kCT / kWave) {
            const int32_t* srow = token_slot + (t0 + tt) * R;
            int found = 0;
            for (int r0 = 0; r0 < R; r0 += kWave) {
                const int r = r0 + lane;
                int32_t s = r < R ? srow[r] : -1;
                if (s >= rows) {
                    errbits |= kErrSlotRange;
                    s = -1;
                }
                const uint64_t m = wave_ballot(s >= 0);
                const int pos = found + lanes_below(m);
                if (s >= 0) s_slot[tt * R + pos] = s;
                found += __popcll(m);
            }
            if (lane == 0) s_cnt[tt] = found;
        }
        __syncthreads();

        const int total = nt * V;
        for (int f = tid; f < total; f += kCT) {
            const int tt = f / V;
            const int vv = f - tt * V;
            const int c = s_cnt[tt];
            const int32_t* sl = s_slot + tt * R;
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
            store_stream(out + (t0 + tt) * V + vv, o);
        }
        if (kCGridCap > 0) __syncthreads();  // the next group reuses the LDS lists
    }
    if (errbits) raise_error(error_flag, errbits);
}

}  // namespace

hipError_t launch_combine(const void* partial, int64_t rows, const int32_t* token_slot,
                          int64_t T, int H, int R, void* out, int32_t* error_flag,
                          hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    int tpb = std::max(1, std::min(64, kCBlockWords / V));
    tpb = std::max(1, std::min(tpb, 8192 / R));
    const int64_t groups = (T + tpb - 1) / tpb;
    const int64_t grid = kCGridCap > 0 ? std::min<int64_t>(groups, kCGridCap) : groups;
    if (!grid_fits(grid, kCT)) return hipErrorInvalidConfiguration;
    const size_t shm = sizeof(int32_t) * (static_cast<size_t>(tpb) + static_cast<size_t>(tpb) * R);
    hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCT), shm, stream,
                       static_cast<const u32x4*>(partial), rows, token_slot, T, V, R,
                       static_cast<u32x4*>(out), error_flag, tpb);
    return hipGetLastError();
}

}  // namespace ep
