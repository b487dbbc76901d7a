// restripe.hip -- prob from [T][N][P] (token-major) to [N][Tmax][P] (destination-major)
// on gfx950 ("[PR #634] Hybrid ep nixl restripe", section "Fix": after the restripe the
// slices one destination needs for a run of consecutive tokens are contiguous, so one
// put per (chunk, destination) replaces one put per token).
//
// Design: the pages launch one block per (token, destination) copying P floats. Here a
// block owns a run of consecutive tokens and walks their N*P words in source order, so
// the loads are one contiguous stream and each P-word slice lands as one contiguous run
// in its node block (512 B at P = 128). Several 128-bit words are in flight per lane.
// Pure copy: HBM bound at 2*T*N*P*4 bytes.
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kRT = kRestripeThreads;
constexpr int kRU = kRestripeU;

template <typename W>
__global__ __launch_bounds__(kRT) void restripe_kernel(const W* __restrict__ in, int64_t T,
                                                       int NV, int VP, int64_t Tmax,
                                                       W* __restrict__ out, int tpb) {
    restripe_run<W, kRU>(in, T, NV, VP, Tmax, out, tpb, blockIdx.x);
}

// Sparse path: only routed (token, node) slices move, to row node_slot[t][n] of the node's
// block (packed in token order). Same source-order walk as the dense restripe; the
// destination row comes from node_slot (one int32 per slice, cached across its words).
// The slice words are loaded together with the slots rather than after them: a read of
// the few unrouted slices (a tenth at top-8 over four nodes) is cheaper than a second
// dependent memory round trip in a kernel this short.
template <typename W>
__global__ __launch_bounds__(kRT) void restripe_sparse_kernel(
    const W* __restrict__ in, int64_t T, int N, int NV, int VP, const int32_t* __restrict__ node_slot,
    int64_t Tmax, W* __restrict__ out, int32_t* __restrict__ error_flag, int tpb) {
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
    const int nt = static_cast<int>(min<int64_t>(tpb, T - t0));
    const int total = nt * NV;
    const W* src = in + t0 * NV;
    int32_t errbits = 0;
    for (int f0 = 0; f0 < total; f0 += kRT * kRU) {
        // A lane past the end takes the last word, as in the dense walk: its loads need no
        // guard, and its store, if any, repeats that word's.
        W v[kRU];
        int32_t s[kRU];
        int f[kRU];
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            f[u] = min(f0 + u * kRT + tid, total - 1);
            const int tt = f[u] / NV;
            const int n = (f[u] - tt * NV) / VP;
            s[u] = node_slot[(t0 + tt) * N + n];
            v[u] = __builtin_nontemporal_load(src + f[u]);
        }
#pragma unroll
        for (int u = 0; u < kRU; ++u) {
            if (s[u] >= 0) {
                if (s[u] >= Tmax) {
                    errbits |= kErrRecvOverflow;
                    continue;
                }
                const int tt = f[u] / NV;
                const int rem = f[u] - tt * NV;
                const int n = rem / VP;
                const int vv = rem - n * VP;
                __builtin_nontemporal_store(v[u], out + (static_cast<int64_t>(n) * Tmax + s[u]) * VP + vv);
            }
        }
    }
    if (errbits) raise_error(error_flag, errbits);
}

}  // namespace

RestripeTask plan_restripe(const float* prob, int64_t T, int N, int P, int64_t Tmax, float* out) {
    RestripeTask rs{};
    rs.in = prob;
    rs.out = out;
    rs.T = T;
    rs.Tmax = Tmax;
    rs.vec = (P % 4 == 0) && (reinterpret_cast<uintptr_t>(prob) % 16 == 0) &&
             (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    rs.VP = rs.vec ? P / 4 : P;
    rs.NV = N * rs.VP;
    rs.tpb = std::max(1, (kRT * kRU) / rs.NV);
    rs.blocks = T > 0 ? (T + rs.tpb - 1) / rs.tpb : 0;
    return rs;
}

hipError_t launch_restripe(const float* prob, int64_t T, int N, int P, int64_t Tmax, float* out,
                           hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const RestripeTask rs = plan_restripe(prob, T, N, P, Tmax, out);
    if (!grid_fits(rs.blocks, kRT)) return hipErrorInvalidConfiguration;
    if (rs.vec) {
        hipLaunchKernelGGL(restripe_kernel<u32x4>, dim3(static_cast<unsigned>(rs.blocks)), dim3(kRT),
                           0, stream, reinterpret_cast<const u32x4*>(prob), T, rs.NV, rs.VP, Tmax,
                           reinterpret_cast<u32x4*>(out), rs.tpb);
    } else {
        hipLaunchKernelGGL(restripe_kernel<uint32_t>, dim3(static_cast<unsigned>(rs.blocks)),
                           dim3(kRT), 0, stream, reinterpret_cast<const uint32_t*>(prob), T, rs.NV,
                           rs.VP, Tmax, reinterpret_cast<uint32_t*>(out), rs.tpb);
    }
    return hipGetLastError();
}

}  // namespace ep

namespace ep {

hipError_t launch_restripe_sparse(const float* prob, int64_t T, int N, int P,
                                  const int32_t* node_slot, int64_t Tmax, float* out,
                                  int32_t* error_flag, hipStream_t stream) {
    if (T == 0) return hipSuccess;
    const bool vec = (P % 4 == 0) && (reinterpret_cast<uintptr_t>(prob) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    const int VP = vec ? P / 4 : P;
    const int NV = N * VP;
    const int tpb = std::max(1, (kRT * kRU) / NV);
    const int64_t grid = (T + tpb - 1) / tpb;
    if (!grid_fits(grid, kRT)) return hipErrorInvalidConfiguration;
    if (vec) {
        hipLaunchKernelGGL(restripe_sparse_kernel<u32x4>, dim3(static_cast<unsigned>(grid)),
                           dim3(kRT), 0, stream, reinterpret_cast<const u32x4*>(prob), T, N, NV, VP,
                           node_slot, Tmax, reinterpret_cast<u32x4*>(out), error_flag, tpb);
    } else {
        hipLaunchKernelGGL(restripe_sparse_kernel<uint32_t>, dim3(static_cast<unsigned>(grid)),
                           dim3(kRT), 0, stream, reinterpret_cast<const uint32_t*>(prob), T, N, NV,
                           VP, node_slot, Tmax, reinterpret_cast<uint32_t*>(out), error_flag, tpb);
    }
    return hipGetLastError();
}

}  // namespace ep
