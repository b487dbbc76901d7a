// dispatch.hip -- token-major dispatch permute on gfx950.
//
// Every (token, rank) pair with a receive slot s gets row s of recv_x = the token's bf16
// row, plus the rank's view of the token's top-k routing and the token id. On one GPU
// the intra-node hop of the pages ("[PR #347] Feature/sm free normal kernel", section
// 3.3.2) is an HBM-to-HBM copy, and rows are written straight to their final place with
// no staging buffer (the zero-copy idea of "[PR #453] ... Zero-Copy and TMA Offloading").
//
// Design: a block owns a few consecutive tokens. Wave-level ballots over the token_slot
// row compact each token's destination slots (ascending rank) into an LDS list. Then
// every lane reads each 128-bit word of the x rows once (several words in flight per
// lane) and stores it to every destination row with non-temporal stores: each wave
// store covers 1 KiB of one destination row. The work per token is bounded by
// min(k, R) destinations, whatever the skew of the per-rank counts. HBM-write bound.
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kDT = 256;  // threads per block
constexpr int kDU = 4;    // 128-bit words in flight per lane

__global__ __launch_bounds__(kDT) void dispatch_kernel(
    const u32x4* __restrict__ x, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t T, int V, int k, int E, int R, int er,
    const int32_t* __restrict__ token_slot, u32x4* __restrict__ recv_x,
    int64_t* __restrict__ recv_idx, float* __restrict__ recv_w, int32_t* __restrict__ recv_src,
    int64_t cap, int32_t* __restrict__ error_flag, int tpb, int maxd) {
    extern __shared__ int32_t smem[];
    int32_t* s_cnt = smem;                  // [tpb]
    int32_t* s_slot = s_cnt + tpb;          // [tpb][maxd]
    int32_t* s_rank = s_slot + tpb * maxd;  // [tpb][maxd]
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
    const int nt = static_cast<int>(min<int64_t>(tpb, T - t0));
    int32_t errbits = 0;

    // 1. destination lists, ascending rank
    for (int tt = wave; tt < nt; tt += kDT / kWave) {
        const int32_t* srow = token_slot + (t0 + tt) * R;
        int found = 0;
        for (int r0 = 0; r0 < R; r0 += kWave) {
            const int r = r0 + lane;
            int32_t s = r < R ? srow[r] : -1;
            if (s >= cap) {
                errbits |= kErrRecvOverflow;
                s = -1;
            }
            const uint64_t m = wave_ballot(s >= 0);
            const int pos = found + lanes_below(m);
            if (s >= 0) {
                if (pos < maxd) {
                    s_slot[tt * maxd + pos] = s;
                    s_rank[tt * maxd + pos] = r;
                } else {
                    errbits |= kErrSlotRange;
                }
            }
            found += __popcll(m);
        }
        if (lane == 0) s_cnt[tt] = min(found, maxd);
    }
    __syncthreads();

    // 2. rows: each 128-bit word of x read once, stored to every destination
    const int total = nt * V;
    const u32x4* xb = x + t0 * V;
    for (int f0 = 0; f0 < total; f0 += kDT * kDU) {
        u32x4 v[kDU];
        int tt[kDU], vv[kDU];
#pragma unroll
        for (int u = 0; u < kDU; ++u) {
            const int f = f0 + u * kDT + tid;
            tt[u] = f / V;
            vv[u] = f - tt[u] * V;
            if (f < total) v[u] = load_stream(xb + f);
        }
#pragma unroll
        for (int u = 0; u < kDU; ++u) {
            const int f = f0 + u * kDT + tid;
            if (f < total) {
                const int c = s_cnt[tt[u]];
                const int32_t* sl = s_slot + tt[u] * maxd;
                for (int d = 0; d < c; ++d)
                    store_stream(recv_x + static_cast<int64_t>(sl[d]) * V + vv[u], v[u]);
            }
        }
    }

    // 3. per-row routing view and source token
    if (recv_idx || recv_w || recv_src) {
        const int per_tok = maxd * k;
        const int total3 = nt * per_tok;
        for (int f = tid; f < total3; f += kDT) {
            const int tt = f / per_tok;
            const int rem = f - tt * per_tok;
            const int d = rem / k;
            const int j = rem - d * k;
            if (d < s_cnt[tt]) {
                const int64_t s = s_slot[tt * maxd + d];
                const int r = s_rank[tt * maxd + d];
                const int64_t t = t0 + tt;
                const int64_t e = topk_idx ? topk_idx[t * k + j] : -1;
                const bool local = e >= 0 && e < E && static_cast<int>(e) / er == r;
                if (recv_idx) recv_idx[s * k + j] = local ? e - static_cast<int64_t>(r) * er : -1;
                if (recv_w) recv_w[s * k + j] = local ? topk_w[t * k + j] : 0.0f;
                if (recv_src && j == 0) recv_src[s] = static_cast<int32_t>(t);
            }
        }
    }
    if (errbits) raise_error(error_flag, errbits);
}

}  // namespace

hipError_t launch_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                           int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                           void* recv_x, int64_t* recv_idx, float* recv_w, int32_t* recv_src,
                           int64_t cap, int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const int V = H / 8;
    const int maxd = std::min(k, R);
    int tpb = std::max(1, std::min(64, (kDT * kDU * 2) / V));
    tpb = std::max(1, std::min(tpb, 4096 / maxd));
    const int64_t grid = (T + tpb - 1) / tpb;
    if (!grid_fits(grid, kDT)) return hipErrorInvalidConfiguration;
    const size_t shm = sizeof(int32_t) * (static_cast<size_t>(tpb) + 2ull * tpb * maxd);
    hipLaunchKernelGGL(dispatch_kernel, dim3(static_cast<unsigned>(grid)), dim3(kDT), shm, stream,
                       static_cast<const u32x4*>(x), topk_idx, topk_w, T, V, k, E, R, E / R,
                       token_slot, static_cast<u32x4*>(recv_x), recv_idx, recv_w, recv_src, cap,
                       error_flag, tpb, maxd);
    return hipGetLastError();
}

}  // namespace ep
