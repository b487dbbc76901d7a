// ep_internal.hpp -- device helpers and kernel launchers shared by the HIP sources of
// the EP dispatch/combine library (gfx950, wave64). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;
constexpr int kMaxRanks = 1024;    // = EP_MAX_RANKS of the public header
constexpr int kMaxExperts = 8192;  // = EP_MAX_EXPERTS of the public header

// Lane id (0..63) and the number of set bits of `mask` on lanes below this one
// (v_mbcnt_lo / v_mbcnt_hi).
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// Division by a launch-constant divisor: a shift when it is a power of two (the usual
// experts-per-rank and ranks-per-node counts), else the integer division.
struct FastDiv {
    int d;
    int shift;  // log2(d) when d is a power of two, else -1
    static FastDiv make(int d) {
        int s = -1;
        if (d > 0 && (d & (d - 1)) == 0) {
            s = 0;
            while ((1 << s) != d) ++s;
        }
        return FastDiv{d, s};
    }
    __device__ __forceinline__ int div(int n) const { return shift >= 0 ? n >> shift : n / d; }
};

// 128-bit word used for every row move.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// Raw buffer resources (untyped, stride 0): word 3 of such a resource on gfx9-family
// targets, and the cache-policy bits of a buffer access's aux operand. Buffer ops through
// the resource are bounds-checked against its byte count: a load past it returns zero
// and a store past it is dropped.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kPolicySc0 = 1;
constexpr int kPolicyNt = 2;
constexpr int kPolicySc1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRawBufferWord3);
}

// Sticky device error word: bits are only ever added.
__device__ __forceinline__ void raise_error(int32_t* flag, int32_t bits) {
    if (flag) atomicOr(flag, bits);
}

// An HSA dispatch packet counts work-items in 32 bits.
inline bool grid_fits(int64_t blocks, int threads) {
    return blocks >= 0 && blocks * static_cast<int64_t>(threads) <= static_cast<int64_t>(UINT32_MAX);
}

constexpr int32_t kErrTopkRange = 1;
constexpr int32_t kErrRecvOverflow = 2;
constexpr int32_t kErrSlotRange = 4;
constexpr int32_t kErrWorkspace = 8;

// ---------------------------------------------------------------- dense restripe
// prob [T][N][P] -> [N][Tmax][P] in words W (128-bit when P % 4 == 0 and both pointers are
// 16-byte aligned, else 32-bit): NV = N * VP words per token, VP per (token, node) slice.
// A block of kRestripeThreads owns tokens [b tpb, b tpb + tpb) (about kRestripeU words per
// lane) and walks their words in source order; each slice lands as one contiguous run of
// its node's block. The restripe's own kernel runs one block per run with kRestripeU
// words in flight per lane. A layout launch can carry the same blocks after its own
// (ep_layout_counts, ep_dispatch_preprocess); there they keep one word in flight per
// lane, so that their stream does not delay the count blocks' loads, whose end is the
// launch's. Measured on MI355X, one word against four: at 4096 tokens (top-8 over 32
// ranks, 4 x 64 floats per token) the count launch took 6.07 against 6.46 us and the
// whole step 172.8 against 173.7 us; at 16384 tokens (64 ranks, 8 x 64 floats) the step
// took 702.5 against 700.7 us.
constexpr int kRestripeThreads = 256;
constexpr int kRestripeU = 4;

struct RestripeTask {
    const void* in;
    void* out;
    int64_t T;
    int64_t Tmax;
    int NV, VP, tpb;
    int vec;         // 128-bit words
    int64_t blocks;  // blocks of kRestripeThreads covering the T tokens
};

// Device-scope stores (one buffer resource over a block's output span, sc1) made the
// restripe faster alone (4.3 against 4.8 us at [4096][8][128], 4.4 against 5.4 us at
// [16384][8][32], 2.4 against 2.6 us at [4096][4][64] on MI355X) but the kernels after
// it slower: at 16384 tokens (top-8 over 64 ranks) the counts-path step took 698.3
// against 688.0 us with them inside the count launch, and one call per step 714.8
// against 700.2 us with them in the restripe's own launch. Both keep non-temporal stores.
template <typename W, int kU>
__device__ __forceinline__ void restripe_run(const W* __restrict__ in, int64_t T, int NV, int VP,
                                             int64_t Tmax, W* __restrict__ out, int tpb,
                                             int64_t block) {
    const int tid = threadIdx.x;
    const int64_t t0 = block * tpb;
    const int nt = static_cast<int>(min<int64_t>(tpb, T - t0));
    const int total = nt * NV;
    const W* src = in + t0 * NV;
    for (int f0 = 0; f0 < total; f0 += kRestripeThreads * kU) {
        // A lane past the end takes the last word: it loads it and stores it again, the
        // same value to the same place, so no access needs a guard. A guarded access sits
        // in a branch of its own, and before each one the compiler then waits for every
        // memory operation in flight, which leaves one word in flight per lane (the
        // restripe's own launch at 4096 x 4 x 64 floats: 4.3 against 2.6 us).
        W v[kU];
        int f[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            f[u] = min(f0 + u * kRestripeThreads + tid, total - 1);
            v[u] = __builtin_nontemporal_load(src + f[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int tt = f[u] / NV;
            const int rem = f[u] - tt * NV;
            const int n = rem / VP;
            const int vv = rem - n * VP;
            __builtin_nontemporal_store(v[u],
                                        out + (static_cast<int64_t>(n) * Tmax + t0 + tt) * VP + vv);
        }
    }
}

// One restripe block inside a layout launch: one word in flight per lane.
__device__ __forceinline__ void restripe_task_block(const RestripeTask& rs, int64_t block) {
    if (rs.vec)
        restripe_run<u32x4, 1>(static_cast<const u32x4*>(rs.in), rs.T, rs.NV, rs.VP, rs.Tmax,
                               static_cast<u32x4*>(rs.out), rs.tpb, block);
    else
        restripe_run<uint32_t, 1>(static_cast<const uint32_t*>(rs.in), rs.T, rs.NV, rs.VP,
                                  rs.Tmax, static_cast<uint32_t*>(rs.out), rs.tpb, block);
}

// The blocks of a dense restripe (blocks == 0 when T == 0 or there is nothing to do).
RestripeTask plan_restripe(const float* prob, int64_t T, int N, int P, int64_t Tmax, float* out);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the error reported at launch. Arguments have been
// validated by the C ABI layer.

// HIP records the status of every runtime call as the thread's last error, so a later
// successful launch would hide an earlier failed one: a launcher that enqueues several
// kernels checks after each launch and returns the first failure.
#define EP_RETURN_IF_LAUNCH_FAILED()                             \
    do {                                                         \
        const hipError_t ep_launch_err_ = hipGetLastError();     \
        if (ep_launch_err_ != hipSuccess) return ep_launch_err_; \
    } while (0)

struct LayoutWorkspace {
    int32_t* blk_rank;   // [nb][R]  per-block rank counts, then per-block exclusive prefix
    int32_t* blk_node;   // [nb][N]
    int32_t* blk_exp;    // [nb][E]  per-block inclusive prefix of the expert histogram
    int32_t* blk_exp_base;  // [nb][E]  first expert-major row of each block, per expert
    int32_t* blk_err;    // [nb]
};

constexpr int kLayoutBlockTokens = 256;  // one token per thread

size_t layout_workspace_bytes(int64_t T, int E, int R, int N);
LayoutWorkspace carve_layout_workspace(void* base, int64_t T, int E, int R, int N);

// Size of the static device scratch that stands in for the workspace in the entry point
// that allocates nothing (= EP_LAYOUT_SCRATCH_BYTES of the public header).
constexpr size_t kLayoutScratchBytes = size_t{4} << 20;
// The current device's address of that scratch array (looked up once per device).
hipError_t layout_scratch_address(void** out);

// `rs` (may be null): a dense restripe whose blocks ride along in the layout's first
// launch, after the layout's own blocks.
// ws_base: a workspace of layout_workspace_bytes(T, E, R, N) bytes, 16-byte aligned.
hipError_t launch_layout(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                         int32_t* count_r, int32_t* count_n, int32_t* count_e, uint8_t* in_rank,
                         int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                         int32_t* expert_slot, int32_t* node_slot, int32_t* error_flag,
                         void* ws_base, const RestripeTask* rs, hipStream_t stream);

constexpr int kExpertSlotMaxK = 16;  // top-k limit of the expert-major slot output

// Workspace of the counts path (ep_layout_counts, then ep_dispatch_layout; R <= 64). The
// ticket counter comes first: it must be zero before the first call, and every call leaves
// it zero again. The rest is rewritten by each call: per-256-token-block tables and one rank
// mask per token.
constexpr int kCountsMaxRanks = 64;
struct CountsWorkspace {
    int32_t* ticket;    // [1]     blocks of the count launch that have published
    int32_t* blk_rank;  // [nb][R] tokens per rank in each block
    int32_t* glob;      // [nb][R] receive row of each block's first token on each rank
                        //         (written only for batches past kCountsLocalBlocks blocks)
    int32_t* pfx;       // [nb][4][R] tokens on each rank in the block's earlier waves
    uint64_t* ball;     // [nb][4][R] which of each wave's 64 tokens are on each rank
    uint64_t* mask;     // [T] the ranks of each token
    int32_t* blk_err;   // [nb] a bad expert id in the block
    int32_t* blk_node;  // [nb][N] tokens per node in each block
    int32_t* blk_exp;   // [nb][E] inclusive prefix over experts of each block's histogram
};
size_t counts_workspace_bytes(int64_t T, int E, int R, int N);
CountsWorkspace carve_counts_workspace(void* base, int64_t T, int E, int R, int N);

// Zero fill of up to six int32 arrays (NULL ones skipped) with a kernel, so that the
// fill can be captured into a graph.
constexpr int kZeroArrays = 6;
struct ZeroInts {
    int32_t* p[kZeroArrays];
    int n[kZeroArrays];
};
hipError_t launch_zero_ints(const ZeroInts& z, hipStream_t stream);

// dispatch.hip: ep_get_layout's slot launch from the counts path's tables (2 to
// kCountsLocalBlocks blocks, R <= kCountsMaxRanks).
hipError_t launch_counts_slots(int64_t T, int E, int R, int N, const CountsWorkspace& cw,
                               int32_t* token_slot, uint8_t* in_rank, int32_t* count_r,
                               int32_t* rank_offset, int32_t* count_n, int32_t* count_e,
                               int32_t* expert_offset, hipStream_t stream);

// layout.hip: the layout, the dispatch and (with rs) the restripe of a batch of at most
// one 256-token group (R <= kCountsMaxRanks) in one launch.
hipError_t launch_layout_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                                  int64_t T, int H, int k, int E, int R, int N,
                                  const RestripeTask* rs, int32_t* count_r, int32_t* rank_offset,
                                  int32_t* count_n, int32_t* count_e, int32_t* expert_offset,
                                  int32_t* token_slot, uint8_t* in_rank, void* recv_x,
                                  int64_t* recv_idx, float* recv_w, int32_t* recv_src,
                                  int64_t cap, int32_t* error_flag, hipStream_t stream);

// Batches of at most this many 256-token blocks take the counts path without a ticket:
// each dispatch wave sums the per-block rank counts it needs itself (one load per block
// per lane), so the count launch has no cross-block phase. Larger batches keep the
// ticket, whose last block writes each block's first receive row per rank.
constexpr int kCountsLocalBlocks = 16;
// The counts path's permute forms each pair's expert-major row from every block's expert
// prefix, one block per lane: at most this many 256-token blocks.
constexpr int kCountsPermuteBlocks = 64;

// The count launch of the counts path (the restripe's blocks may ride along): the error
// flag and the tables ep_dispatch_layout reads; with expert_rank ([T][k], k <=
// kExpertSlotMaxK), also each pair's rank among its 256-token block's pairs naming the same
// expert, which ep_dispatch_permute_layout turns into expert-major rows.
hipError_t launch_layout_counts(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                                int32_t* error_flag, int32_t* expert_rank,
                                const CountsWorkspace& cw, const RestripeTask* rs,
                                hipStream_t stream);

// dispatch.hip: one-call dispatch, FP8 dispatch, expert-major permute, and the two
// phases of the two-phase dispatch
hipError_t launch_dispatch(const void* x, const int64_t* topk_idx, const float* topk_w,
                           int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                           void* recv_x, int64_t* recv_idx, float* recv_w, int32_t* recv_src,
                           int64_t cap, int32_t* error_flag, hipStream_t stream);
hipError_t launch_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_w,
                               int64_t T, int H, int k, int E, int R, const int32_t* token_slot,
                               void* recv_codes, float* recv_scales, int64_t* recv_idx,
                               float* recv_w, int32_t* recv_src, int64_t cap, int32_t* error_flag,
                               hipStream_t stream);
hipError_t launch_dispatch_permute(const void* x, const float* topk_w, int64_t T, int H, int k,
                                   const int32_t* expert_slot, void* perm_x, float* perm_w,
                                   int32_t* perm_src, int64_t cap, int32_t* error_flag,
                                   hipStream_t stream);
hipError_t launch_dispatch_send(const void* x, const int64_t* topk_idx, const float* topk_w,
                                int64_t T, int H, int k, int N, const int32_t* node_slot,
                                int64_t Tmax, void* stage_x, int64_t* stage_idx, float* stage_w,
                                int32_t* stage_src, int32_t* error_flag, int max_blocks,
                                hipStream_t stream);
// The dispatch of the counts path: each wave computes its token's receive rows from the
// count launch's tables; the token's first wave also writes its token_slot and bitmap rows.
// A few leading blocks of the first launch write the node and expert counts and offsets.
hipError_t launch_dispatch_layout(const void* x, const int64_t* topk_idx, const float* topk_w,
                                  int64_t T, int H, int k, int E, int R, int N,
                                  const CountsWorkspace& cw, int32_t* token_slot, uint8_t* in_rank,
                                  void* recv_x, int64_t* recv_idx, float* recv_w,
                                  int32_t* recv_src, int64_t cap, int32_t* count_r,
                                  int32_t* rank_offset, int32_t* count_n, int32_t* count_e,
                                  int32_t* expert_offset, int32_t* error_flag, hipStream_t stream);
hipError_t launch_dispatch_permute_layout(const void* x, const int64_t* topk_idx,
                                          const float* topk_w, int64_t T, int H, int k, int E,
                                          int N, const int32_t* expert_rank,
                                          const CountsWorkspace& cw, void* perm_x, float* perm_w,
                                          int32_t* perm_src, int32_t* expert_slot, int64_t cap,
                                          int32_t* count_e, int32_t* expert_offset,
                                          int32_t* error_flag, hipStream_t stream);
hipError_t launch_dispatch_recv(const void* stage_x, const int64_t* stage_idx,
                                const float* stage_w, const int32_t* stage_src,
                                const int32_t* count_n, int N, int64_t Tmax, int H, int k, int E,
                                int R, const int32_t* token_slot, int64_t T, void* recv_x,
                                int64_t* recv_idx, float* recv_w, int32_t* recv_src, int64_t cap,
                                int32_t* error_flag, hipStream_t stream);

// restripe.hip: dense and sparse-path restripe of prob
hipError_t launch_restripe(const float* prob, int64_t T, int N, int P, int64_t Tmax, float* out,
                           hipStream_t stream);
hipError_t launch_restripe_sparse(const float* prob, int64_t T, int N, int P,
                                  const int32_t* node_slot, int64_t Tmax, float* out,
                                  int32_t* error_flag, hipStream_t stream);

// combine.hip: one-call combine and the two phases of the two-phase combine
hipError_t launch_combine(const void* partial, int64_t rows, const int32_t* token_slot,
                          int64_t T, int H, int R, void* out, int32_t* error_flag,
                          hipStream_t stream);
hipError_t launch_combine_send(const void* partial, int64_t rows, const int32_t* token_slot,
                               int64_t T, int H, int R, int N, const int32_t* node_slot,
                               int64_t Tmax, void* stage, int32_t* error_flag, int max_blocks,
                               hipStream_t stream);
hipError_t launch_combine_recv(const void* stage, int N, int64_t Tmax, const int32_t* node_slot,
                               int64_t T, int H, void* out, int32_t* error_flag,
                               hipStream_t stream);

// hbm_copy.hip: the copy-bandwidth yardstick
hipError_t launch_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_hbm_fan(const void* src, void* dst, size_t slab_bytes, int fan_in,
                          int fan_out, hipStream_t stream);
hipError_t launch_hbm_spread(const void* src, void* dst, size_t out_bytes, int fan_in,
                             int regions, hipStream_t stream);

}  // namespace ep
