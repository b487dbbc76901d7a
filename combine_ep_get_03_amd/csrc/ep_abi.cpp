// ep_abi.cpp -- the extern "C" boundary declared in include/ep.h: host-side argument
// checks, then the kernel launches on the caller's stream. Nothing is enqueued when a
// check fails, and no C++ exception leaves this file.
#include "ep.h"

#include <limits.h>

#include "ep_internal.hpp"

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Topology sizes shared by layout and dispatch.
static_assert(EP_LAYOUT_DISPATCH_MAX_TOKENS == ep::kLayoutBlockTokens,
              "ep_layout_dispatch covers one block of the layout");
static_assert(EP_COUNTS_MAX_RANKS == ep::kCountsMaxRanks, "one rank mask word per token");

bool topology_ok(int k, int E, int R, int N) {
    if (E < 1 || E > EP_MAX_EXPERTS || R < 1 || R > EP_MAX_RANKS || N < 1) return false;
    if (E % R != 0 || R % N != 0) return false;
    if (k < 1 || k > E) return false;
    return true;
}

bool slots_fit_int32(int64_t T, int k, int R) {
    const int64_t per = k < R ? k : R;
    return T >= 0 && (T == 0 || T <= static_cast<int64_t>(INT32_MAX) / per);
}

// Every check of ep_get_layout except those of the workspace.
int check_layout_args(const int64_t* topk_idx, int64_t T, int k, int E, int R, int N,
                      const int32_t* count_r, const int32_t* count_n, const int32_t* count_e,
                      const int32_t* rank_offset, const int32_t* expert_offset,
                      const int32_t* token_slot, const int32_t* expert_slot,
                      const int32_t* node_slot, const int32_t* error_flag) {
    if (!topology_ok(k, E, R, N) || !slots_fit_int32(T, k, R)) return EP_ERR_ARG;
    if (!count_r || !rank_offset || !error_flag) return EP_ERR_ARG;
    if (T > 0 && (!topk_idx || !token_slot)) return EP_ERR_ARG;
    if (expert_slot && k > EP_EXPERT_SLOT_MAX_K) return EP_ERR_ARG;
    // per-expert counts, expert offsets and expert-major rows count (token, slot) pairs
    // in int32: up to T * k of them
    if ((count_e || expert_offset || expert_slot) && T > static_cast<int64_t>(INT32_MAX) / k)
        return EP_ERR_ARG;
    if (!aligned(topk_idx, 8) || !aligned(count_r, 4) || !aligned(expert_slot, 4) ||
        !aligned(node_slot, 4) || !aligned(count_n, 4) || !aligned(count_e, 4) ||
        !aligned(rank_offset, 4) || !aligned(expert_offset, 4) || !aligned(token_slot, 4) ||
        !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return EP_OK;
}

}  // namespace

extern "C" {

const char* ep_status_string(int status) {
    switch (status) {
        case EP_OK: return "EP_OK";
        case EP_ERR_ARG: return "EP_ERR_ARG: a count or size is out of range or a required pointer is NULL";
        case EP_ERR_ALIGN: return "EP_ERR_ALIGN: a pointer or row length breaks the alignment rule";
        case EP_ERR_CAPACITY: return "EP_ERR_CAPACITY: a destination or the workspace is too small";
        case EP_ERR_HIP: return "EP_ERR_HIP: the HIP runtime reported an error at launch";
        default: return "unknown ep status";
    }
}

size_t ep_layout_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                 int num_nodes) {
    if (num_tokens < 0 || num_experts < 1 || num_experts > EP_MAX_EXPERTS || num_ranks < 1 ||
        num_ranks > EP_MAX_RANKS || num_nodes < 1 || num_experts % num_ranks != 0 ||
        num_ranks % num_nodes != 0)
        return 0;
    return ep::layout_workspace_bytes(num_tokens, num_experts, num_ranks, num_nodes);
}

int ep_get_layout(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                  int num_ranks, int num_nodes, int32_t* num_tokens_per_rank,
                  int32_t* num_tokens_per_node, int32_t* num_tokens_per_expert,
                  uint8_t* is_token_in_rank, int32_t* rank_offset, int32_t* expert_offset,
                  int32_t* token_slot, int32_t* expert_slot, int32_t* node_slot,
                  int32_t* error_flag, void* workspace, size_t workspace_bytes, void* stream) {
    const int64_t T = num_tokens;
    const int k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    const int st = check_layout_args(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                     num_tokens_per_node, num_tokens_per_expert, rank_offset,
                                     expert_offset, token_slot, expert_slot, node_slot,
                                     error_flag);
    if (st != EP_OK) return st;
    if (!aligned(workspace, 16)) return EP_ERR_ALIGN;
    const size_t need = ep::layout_workspace_bytes(T, E, R, N);
    if (workspace_bytes < need || (need > 0 && !workspace)) return EP_ERR_CAPACITY;
    return hip_status(ep::launch_layout(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                        num_tokens_per_node, num_tokens_per_expert,
                                        is_token_in_rank, rank_offset, expert_offset, token_slot,
                                        expert_slot, node_slot, error_flag, workspace, nullptr,
                                        static_cast<hipStream_t>(stream)));
}

int ep_get_layout_no_alloc(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int num_nodes,
                           int32_t* num_tokens_per_rank, int32_t* num_tokens_per_node,
                           int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                           int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                           int32_t* expert_slot, int32_t* node_slot, int32_t* error_flag,
                           void* stream) {
    const int64_t T = num_tokens;
    const int k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    const int st = check_layout_args(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                     num_tokens_per_node, num_tokens_per_expert, rank_offset,
                                     expert_offset, token_slot, expert_slot, node_slot,
                                     error_flag);
    if (st != EP_OK) return st;
    if (ep::layout_workspace_bytes(T, E, R, N) > EP_LAYOUT_SCRATCH_BYTES) return EP_ERR_CAPACITY;
    // The kernels run on the stream's device and use that device's copy of the scratch
    // array, whose address is looked up with that device current.
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
    if (stream != nullptr) {
        int sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return EP_ERR_HIP;
        if (sdev != dev) return EP_ERR_ARG;
    }
    void* scratch = nullptr;
    if (ep::layout_scratch_address(&scratch) != hipSuccess) return EP_ERR_HIP;
    return hip_status(ep::launch_layout(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                        num_tokens_per_node, num_tokens_per_expert,
                                        is_token_in_rank, rank_offset, expert_offset, token_slot,
                                        expert_slot, node_slot, error_flag, scratch, nullptr,
                                        static_cast<hipStream_t>(stream)));
}

int ep_dispatch_preprocess(const int64_t* topk_idx, int64_t num_tokens, int num_topk,
                           int num_experts, int num_ranks, int num_nodes,
                           int32_t* num_tokens_per_rank, int32_t* num_tokens_per_node,
                           int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                           int32_t* rank_offset, int32_t* expert_offset, int32_t* token_slot,
                           int32_t* expert_slot, int32_t* node_slot, int32_t* error_flag,
                           const float* prob, int prob_per_token, int64_t max_tokens_per_rank,
                           float* prob_dest_major, void* workspace, size_t workspace_bytes,
                           void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int k = num_topk, E = num_experts, R = num_ranks, N = num_nodes, P = prob_per_token;
    const int st = check_layout_args(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                     num_tokens_per_node, num_tokens_per_expert, rank_offset,
                                     expert_offset, token_slot, expert_slot, node_slot,
                                     error_flag);
    if (st != EP_OK) return st;
    if (P < 1 || static_cast<int64_t>(N) * P > (1 << 26)) return EP_ERR_ARG;
    if (T > 0 && (!prob || !prob_dest_major)) return EP_ERR_ARG;
    if (!aligned(prob, 4) || !aligned(prob_dest_major, 4) || !aligned(workspace, 16))
        return EP_ERR_ALIGN;
    if (Tmax < T) return EP_ERR_CAPACITY;
    const size_t need = ep::layout_workspace_bytes(T, E, R, N);
    if (workspace_bytes < need || (need > 0 && !workspace)) return EP_ERR_CAPACITY;
    const ep::RestripeTask rs = ep::plan_restripe(prob, T, N, P, Tmax, prob_dest_major);
    return hip_status(ep::launch_layout(topk_idx, T, k, E, R, N, num_tokens_per_rank,
                                        num_tokens_per_node, num_tokens_per_expert,
                                        is_token_in_rank, rank_offset, expert_offset, token_slot,
                                        expert_slot, node_slot, error_flag, workspace, &rs,
                                        static_cast<hipStream_t>(stream)));
}

size_t ep_layout_counts_workspace_bytes(int64_t num_tokens, int num_experts, int num_ranks,
                                        int num_nodes) {
    if (num_tokens < 0 || num_experts < 1 || num_experts > EP_MAX_EXPERTS || num_ranks < 1 ||
        num_ranks > EP_COUNTS_MAX_RANKS || num_nodes < 1 || num_experts % num_ranks != 0 ||
        num_ranks % num_nodes != 0)
        return 0;
    return ep::counts_workspace_bytes(num_tokens, num_experts, num_ranks, num_nodes);
}

int ep_layout_counts(const int64_t* topk_idx, int64_t num_tokens, int num_topk, int num_experts,
                     int num_ranks, int num_nodes, int32_t* error_flag, int32_t* expert_rank,
                     const float* prob, int prob_per_token, int64_t max_tokens_per_rank,
                     float* prob_dest_major, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int k = num_topk, E = num_experts, R = num_ranks, N = num_nodes, P = prob_per_token;
    if (!topology_ok(k, E, R, N) || R > EP_COUNTS_MAX_RANKS || !slots_fit_int32(T, k, R) ||
        T > static_cast<int64_t>(INT32_MAX) / k)
        return EP_ERR_ARG;
    if (!error_flag) return EP_ERR_ARG;
    if (T > 0 && !topk_idx) return EP_ERR_ARG;
    if (expert_rank && k > EP_EXPERT_SLOT_MAX_K) return EP_ERR_ARG;
    if (prob) {
        if (P < 1 || static_cast<int64_t>(N) * P > (1 << 26)) return EP_ERR_ARG;
        if (T > 0 && !prob_dest_major) return EP_ERR_ARG;
    }
    if (!aligned(topk_idx, 8) || !aligned(error_flag, 4) || !aligned(expert_rank, 4) ||
        !aligned(prob, 4) || !aligned(prob_dest_major, 4) || !aligned(workspace, 16))
        return EP_ERR_ALIGN;
    if (prob && Tmax < T) return EP_ERR_CAPACITY;
    const size_t need = ep::counts_workspace_bytes(T, E, R, N);
    if (workspace_bytes < need || !workspace) return EP_ERR_CAPACITY;
    const ep::CountsWorkspace cw = ep::carve_counts_workspace(workspace, T, E, R, N);
    ep::RestripeTask rs{};
    if (prob) rs = ep::plan_restripe(prob, T, N, P, Tmax, prob_dest_major);
    return hip_status(ep::launch_layout_counts(topk_idx, T, k, E, R, N, error_flag, expert_rank,
                                               cw, &rs, static_cast<hipStream_t>(stream)));
}

int ep_dispatch_layout(const void* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int num_ranks, int num_nodes, int32_t* num_tokens_per_rank,
                       int32_t* rank_offset, int32_t* num_tokens_per_node,
                       int32_t* num_tokens_per_expert, int32_t* expert_offset,
                       int32_t* token_slot, uint8_t* is_token_in_rank, void* recv_x,
                       int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* recv_src_idx,
                       int64_t recv_capacity, int32_t* error_flag, const void* workspace,
                       size_t workspace_bytes, void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    if (!topology_ok(k, E, R, N) || R > EP_COUNTS_MAX_RANKS || !slots_fit_int32(T, k, R) ||
        T > static_cast<int64_t>(INT32_MAX) / k || H < 1 || recv_capacity < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0) {
        if (!x || !token_slot || !recv_x || !topk_idx) return EP_ERR_ARG;
        if (recv_topk_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(token_slot, 4) || !aligned(recv_topk_idx, 8) ||
        !aligned(recv_topk_weights, 4) || !aligned(recv_src_idx, 4) || !aligned(error_flag, 4) ||
        !aligned(num_tokens_per_node, 4) || !aligned(num_tokens_per_expert, 4) ||
        !aligned(expert_offset, 4) || !aligned(num_tokens_per_rank, 4) ||
        !aligned(rank_offset, 4) || !aligned(workspace, 16))
        return EP_ERR_ALIGN;
    const size_t need = ep::counts_workspace_bytes(T, E, R, N);
    if (workspace_bytes < need || !workspace) return EP_ERR_CAPACITY;
    if (T == 0) {  // an empty batch: zero counts and offsets, nothing to dispatch
        const ep::ZeroInts z{{num_tokens_per_rank, rank_offset, num_tokens_per_node,
                              num_tokens_per_expert, expert_offset},
                             {R, R + 1, N, E, E + 1}};
        return hip_status(ep::launch_zero_ints(z, static_cast<hipStream_t>(stream)));
    }
    const ep::CountsWorkspace cw =
        ep::carve_counts_workspace(const_cast<void*>(workspace), T, E, R, N);
    return hip_status(ep::launch_dispatch_layout(
        x, topk_idx, topk_weights, T, H, k, E, R, N, cw, token_slot, is_token_in_rank, recv_x,
        recv_topk_idx, recv_topk_weights, recv_src_idx, recv_capacity, num_tokens_per_rank,
        rank_offset, num_tokens_per_node, num_tokens_per_expert, expert_offset, error_flag,
        static_cast<hipStream_t>(stream)));
}

int ep_layout_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                       int64_t num_tokens, int hidden, int num_topk, int num_experts,
                       int num_ranks, int num_nodes, int32_t* num_tokens_per_rank,
                       int32_t* rank_offset, int32_t* num_tokens_per_node,
                       int32_t* num_tokens_per_expert, int32_t* expert_offset,
                       int32_t* token_slot, uint8_t* is_token_in_rank, void* recv_x,
                       int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* recv_src_idx,
                       int64_t recv_capacity, const float* prob, int prob_per_token,
                       int64_t max_tokens_per_rank, float* prob_dest_major, int32_t* error_flag,
                       void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    const int P = prob_per_token;
    if (!topology_ok(k, E, R, N) || R > EP_COUNTS_MAX_RANKS || T < 0 ||
        T > EP_LAYOUT_DISPATCH_MAX_TOKENS || H < 1 || recv_capacity < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (!error_flag) return EP_ERR_ARG;
    if (T > 0) {
        if (!x || !topk_idx || !token_slot || !recv_x || !num_tokens_per_rank || !rank_offset)
            return EP_ERR_ARG;
        if (recv_topk_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (prob) {
        if (P < 1 || static_cast<int64_t>(N) * P > (1 << 26)) return EP_ERR_ARG;
        if (T > 0 && !prob_dest_major) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(token_slot, 4) || !aligned(recv_topk_idx, 8) ||
        !aligned(recv_topk_weights, 4) || !aligned(recv_src_idx, 4) || !aligned(error_flag, 4) ||
        !aligned(num_tokens_per_node, 4) || !aligned(num_tokens_per_expert, 4) ||
        !aligned(expert_offset, 4) || !aligned(num_tokens_per_rank, 4) ||
        !aligned(rank_offset, 4) || !aligned(prob, 4) || !aligned(prob_dest_major, 4))
        return EP_ERR_ALIGN;
    if (prob && Tmax < T) return EP_ERR_CAPACITY;
    ep::RestripeTask rs{};
    if (prob && T > 0) rs = ep::plan_restripe(prob, T, N, P, Tmax, prob_dest_major);
    return hip_status(ep::launch_layout_dispatch(
        x, topk_idx, topk_weights, T, H, k, E, R, N, &rs, num_tokens_per_rank, rank_offset,
        num_tokens_per_node, num_tokens_per_expert, expert_offset, token_slot, is_token_in_rank,
        recv_x, recv_topk_idx, recv_topk_weights, recv_src_idx, recv_capacity, error_flag,
        static_cast<hipStream_t>(stream)));
}

int ep_dispatch_permute_layout(const void* x, const int64_t* topk_idx,
                               const float* topk_weights, int64_t num_tokens, int hidden,
                               int num_topk, int num_experts, int num_ranks, int num_nodes,
                               const int32_t* expert_rank, int32_t* num_tokens_per_expert,
                               int32_t* expert_offset, int32_t* expert_slot, void* perm_x,
                               float* perm_weights, int32_t* perm_src_idx, int64_t perm_capacity,
                               int32_t* error_flag, const void* workspace, size_t workspace_bytes,
                               void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    if (!topology_ok(k, E, R, N) || R > EP_COUNTS_MAX_RANKS || k > EP_EXPERT_SLOT_MAX_K ||
        T > static_cast<int64_t>(ep::kCountsPermuteBlocks) * ep::kLayoutBlockTokens || H < 1 ||
        perm_capacity < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (T > 0) {
        if (!x || !topk_idx || !expert_rank || !perm_x) return EP_ERR_ARG;
        if (perm_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(perm_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(expert_rank, 4) || !aligned(expert_slot, 4) ||
        !aligned(perm_weights, 4) || !aligned(perm_src_idx, 4) || !aligned(error_flag, 4) ||
        !aligned(num_tokens_per_expert, 4) || !aligned(expert_offset, 4) ||
        !aligned(workspace, 16))
        return EP_ERR_ALIGN;
    const size_t need = ep::counts_workspace_bytes(T, E, R, N);
    if (workspace_bytes < need || !workspace) return EP_ERR_CAPACITY;
    if (T == 0) {  // an empty batch: zero counts and offsets, nothing to move
        const ep::ZeroInts z{{num_tokens_per_expert, expert_offset, nullptr, nullptr, nullptr},
                             {E, E + 1, 0, 0, 0}};
        return hip_status(ep::launch_zero_ints(z, static_cast<hipStream_t>(stream)));
    }
    const ep::CountsWorkspace cw =
        ep::carve_counts_workspace(const_cast<void*>(workspace), T, E, R, N);
    return hip_status(ep::launch_dispatch_permute_layout(
        x, topk_idx, topk_weights, T, H, k, E, N, expert_rank, cw, perm_x, perm_weights,
        perm_src_idx, expert_slot, perm_capacity, num_tokens_per_expert, expert_offset, error_flag,
        static_cast<hipStream_t>(stream)));
}

int ep_dispatch(const void* x, const int64_t* topk_idx, const float* topk_weights,
                int64_t num_tokens, int hidden, int num_topk, int num_experts, int num_ranks,
                const int32_t* token_slot, void* recv_x, int64_t* recv_topk_idx,
                float* recv_topk_weights, int32_t* recv_src_idx, int64_t recv_capacity,
                int32_t* error_flag, void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks;
    if (!topology_ok(k, E, R, 1) || !slots_fit_int32(T, k, R) || H < 1 || recv_capacity < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0) {
        if (!x || !token_slot || !recv_x) return EP_ERR_ARG;
        if ((recv_topk_idx || recv_topk_weights) && !topk_idx) return EP_ERR_ARG;
        if (recv_topk_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(token_slot, 4) || !aligned(recv_topk_idx, 8) ||
        !aligned(recv_topk_weights, 4) || !aligned(recv_src_idx, 4) || !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_dispatch(x, topk_idx, topk_weights, T, H, k, E, R, token_slot,
                                          recv_x, recv_topk_idx, recv_topk_weights, recv_src_idx,
                                          recv_capacity, error_flag,
                                          static_cast<hipStream_t>(stream)));
}

int ep_dispatch_fp8(const void* x, const int64_t* topk_idx, const float* topk_weights,
                    int64_t num_tokens, int hidden, int num_topk, int num_experts,
                    int num_ranks, const int32_t* token_slot, uint8_t* recv_x_fp8,
                    float* recv_scales, int64_t* recv_topk_idx, float* recv_topk_weights,
                    int32_t* recv_src_idx, int64_t recv_capacity, int32_t* error_flag,
                    void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks;
    if (!topology_ok(k, E, R, 1) || !slots_fit_int32(T, k, R) || H < 1 || recv_capacity < 0)
        return EP_ERR_ARG;
    if (H % 128 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0) {
        if (!x || !token_slot || !recv_x_fp8 || !recv_scales) return EP_ERR_ARG;
        if ((recv_topk_idx || recv_topk_weights) && !topk_idx) return EP_ERR_ARG;
        if (recv_topk_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(recv_x_fp8, 16) || !aligned(recv_scales, 4) ||
        !aligned(topk_idx, 8) || !aligned(topk_weights, 4) || !aligned(token_slot, 4) ||
        !aligned(recv_topk_idx, 8) || !aligned(recv_topk_weights, 4) ||
        !aligned(recv_src_idx, 4) || !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_dispatch_fp8(x, topk_idx, topk_weights, T, H, k, E, R,
                                              token_slot, recv_x_fp8, recv_scales, recv_topk_idx,
                                              recv_topk_weights, recv_src_idx, recv_capacity,
                                              error_flag, static_cast<hipStream_t>(stream)));
}

int ep_dispatch_permute(const void* x, const float* topk_weights, int64_t num_tokens, int hidden,
                        int num_topk, const int32_t* expert_slot, void* perm_x,
                        float* perm_weights, int32_t* perm_src_idx, int64_t capacity,
                        int32_t* error_flag, void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, k = num_topk;
    if (T < 0 || H < 1 || k < 1 || capacity < 0) return EP_ERR_ARG;
    if (T > 0 && T > static_cast<int64_t>(INT32_MAX) / k) return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0 && (!x || !expert_slot || !perm_x)) return EP_ERR_ARG;
    if (T > 0 && perm_weights && !topk_weights) return EP_ERR_ARG;
    if (!aligned(x, 16) || !aligned(perm_x, 16) || !aligned(topk_weights, 4) ||
        !aligned(expert_slot, 4) || !aligned(perm_weights, 4) || !aligned(perm_src_idx, 4) ||
        !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_dispatch_permute(x, topk_weights, T, H, k, expert_slot, perm_x,
                                                  perm_weights, perm_src_idx, capacity,
                                                  error_flag, static_cast<hipStream_t>(stream)));
}

int ep_restripe_prob(const float* prob, int64_t num_tokens, int num_nodes, int prob_per_token,
                     int64_t max_tokens_per_rank, float* prob_dest_major, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int N = num_nodes, P = prob_per_token;
    if (T < 0 || N < 1 || P < 1 || static_cast<int64_t>(N) * P > (1 << 26)) return EP_ERR_ARG;
    if (Tmax < T) return EP_ERR_CAPACITY;
    if (T > 0 && (!prob || !prob_dest_major)) return EP_ERR_ARG;
    if (!aligned(prob, 4) || !aligned(prob_dest_major, 4)) return EP_ERR_ALIGN;
    return hip_status(ep::launch_restripe(prob, T, N, P, Tmax, prob_dest_major,
                                          static_cast<hipStream_t>(stream)));
}

int ep_restripe_prob_sparse(const float* prob, int64_t num_tokens, int num_nodes,
                            int prob_per_token, const int32_t* node_slot,
                            int64_t max_tokens_per_rank, float* prob_dest_major,
                            int32_t* error_flag, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int N = num_nodes, P = prob_per_token;
    if (T < 0 || N < 1 || P < 1 || static_cast<int64_t>(N) * P > (1 << 26)) return EP_ERR_ARG;
    if (Tmax < T) return EP_ERR_CAPACITY;
    if (T > 0 && (!prob || !prob_dest_major || !node_slot)) return EP_ERR_ARG;
    if (!aligned(prob, 4) || !aligned(prob_dest_major, 4) || !aligned(node_slot, 4) ||
        !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_restripe_sparse(prob, T, N, P, node_slot, Tmax, prob_dest_major,
                                                 error_flag, static_cast<hipStream_t>(stream)));
}

int ep_combine(const void* partial, int64_t num_partial_rows, const int32_t* token_slot,
               int64_t num_tokens, int hidden, int num_ranks, void* out, int32_t* error_flag,
               void* stream) {
    const int64_t T = num_tokens;
    const int H = hidden, R = num_ranks;
    if (T < 0 || H < 1 || R < 1 || R > EP_MAX_RANKS || num_partial_rows < 0) return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0 && (!token_slot || !out)) return EP_ERR_ARG;
    if (T > 0 && num_partial_rows > 0 && !partial) return EP_ERR_ARG;
    if (!aligned(partial, 16) || !aligned(out, 16) || !aligned(token_slot, 4) ||
        !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_combine(partial, num_partial_rows, token_slot, T, H, R, out,
                                         error_flag, static_cast<hipStream_t>(stream)));
}

int ep_dispatch_send(const void* x, const int64_t* topk_idx, const float* topk_weights,
                     int64_t num_tokens, int hidden, int num_topk, int num_nodes,
                     const int32_t* node_slot, int64_t max_tokens_per_rank, void* stage_x,
                     int64_t* stage_topk_idx, float* stage_topk_weights, int32_t* stage_src,
                     int32_t* error_flag, int num_workgroups, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int H = hidden, k = num_topk, N = num_nodes;
    if (T < 0 || H < 1 || k < 1 || N < 1 || N > EP_MAX_RANKS || Tmax < 0 || Tmax > INT32_MAX ||
        num_workgroups < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > INT32_MAX) return EP_ERR_ARG;
    if (T > 0) {
        if (!x || !node_slot || !stage_x || !stage_src) return EP_ERR_ARG;
        if ((stage_topk_idx || stage_topk_weights) && !topk_idx) return EP_ERR_ARG;
        if (stage_topk_weights && !topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(x, 16) || !aligned(stage_x, 16) || !aligned(topk_idx, 8) ||
        !aligned(topk_weights, 4) || !aligned(node_slot, 4) || !aligned(stage_topk_idx, 8) ||
        !aligned(stage_topk_weights, 4) || !aligned(stage_src, 4) || !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_dispatch_send(x, topk_idx, topk_weights, T, H, k, N, node_slot,
                                               Tmax, stage_x, stage_topk_idx, stage_topk_weights,
                                               stage_src, error_flag, num_workgroups,
                                               static_cast<hipStream_t>(stream)));
}

int ep_dispatch_recv(const void* stage_x, const int64_t* stage_topk_idx,
                     const float* stage_topk_weights, const int32_t* stage_src,
                     const int32_t* count_n, int num_nodes, int64_t max_tokens_per_rank,
                     int hidden, int num_topk, int num_experts, int num_ranks,
                     const int32_t* token_slot, int64_t num_tokens, void* recv_x,
                     int64_t* recv_topk_idx, float* recv_topk_weights, int32_t* recv_src_idx,
                     int64_t recv_capacity, int32_t* error_flag, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int H = hidden, k = num_topk, E = num_experts, R = num_ranks, N = num_nodes;
    if (!topology_ok(k, E, R, N) || !slots_fit_int32(T, k, R) || H < 1 || recv_capacity < 0 ||
        Tmax < 0 || Tmax > INT32_MAX)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0 && Tmax > 0) {
        if (!stage_x || !stage_src || !count_n || !token_slot || !recv_x) return EP_ERR_ARG;
        if ((recv_topk_idx || recv_topk_weights) && !stage_topk_idx) return EP_ERR_ARG;
        if (recv_topk_weights && !stage_topk_weights) return EP_ERR_ARG;
    }
    if (!aligned(stage_x, 16) || !aligned(recv_x, 16) || !aligned(stage_topk_idx, 8) ||
        !aligned(stage_topk_weights, 4) || !aligned(stage_src, 4) || !aligned(count_n, 4) ||
        !aligned(token_slot, 4) || !aligned(recv_topk_idx, 8) || !aligned(recv_topk_weights, 4) ||
        !aligned(recv_src_idx, 4) || !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_dispatch_recv(stage_x, stage_topk_idx, stage_topk_weights,
                                               stage_src, count_n, N, Tmax, H, k, E, R,
                                               token_slot, T, recv_x, recv_topk_idx,
                                               recv_topk_weights, recv_src_idx, recv_capacity,
                                               error_flag, static_cast<hipStream_t>(stream)));
}

int ep_combine_send(const void* partial, int64_t num_partial_rows, const int32_t* token_slot,
                    int64_t num_tokens, int hidden, int num_ranks, int num_nodes,
                    const int32_t* node_slot, int64_t max_tokens_per_rank, void* stage,
                    int32_t* error_flag, int num_workgroups, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int H = hidden, R = num_ranks, N = num_nodes;
    if (T < 0 || H < 1 || R < 1 || R > EP_MAX_RANKS || N < 1 || R % N != 0 ||
        num_partial_rows < 0 || num_partial_rows > INT32_MAX || Tmax < 0 || Tmax > INT32_MAX ||
        num_workgroups < 0)
        return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 * N > INT32_MAX) return EP_ERR_ARG;
    if (T > 0 && (!token_slot || !node_slot || !stage)) return EP_ERR_ARG;
    if (T > 0 && num_partial_rows > 0 && !partial) return EP_ERR_ARG;
    if (!aligned(partial, 16) || !aligned(stage, 16) || !aligned(token_slot, 4) ||
        !aligned(node_slot, 4) || !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_combine_send(partial, num_partial_rows, token_slot, T, H, R, N,
                                              node_slot, Tmax, stage, error_flag, num_workgroups,
                                              static_cast<hipStream_t>(stream)));
}

int ep_combine_recv(const void* stage, int num_nodes, int64_t max_tokens_per_rank,
                    const int32_t* node_slot, int64_t num_tokens, int hidden, void* out,
                    int32_t* error_flag, void* stream) {
    const int64_t T = num_tokens, Tmax = max_tokens_per_rank;
    const int H = hidden, N = num_nodes;
    if (T < 0 || H < 1 || N < 1 || N > EP_MAX_RANKS || Tmax < 0) return EP_ERR_ARG;
    if (static_cast<int64_t>(N) * Tmax > INT32_MAX) return EP_ERR_ARG;
    if (H % 8 != 0) return EP_ERR_ALIGN;
    if (static_cast<int64_t>(H) / 8 * 64 > INT32_MAX) return EP_ERR_ARG;
    if (T > 0 && (!node_slot || !out)) return EP_ERR_ARG;
    if (T > 0 && Tmax > 0 && !stage) return EP_ERR_ARG;
    if (!aligned(stage, 16) || !aligned(out, 16) || !aligned(node_slot, 4) ||
        !aligned(error_flag, 4))
        return EP_ERR_ALIGN;
    return hip_status(ep::launch_combine_recv(stage, N, Tmax, node_slot, T, H, out, error_flag,
                                              static_cast<hipStream_t>(stream)));
}

int ep_hbm_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes > 0 && (!src || !dst)) return EP_ERR_ARG;
    if (bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16)) return EP_ERR_ALIGN;
    return hip_status(ep::launch_hbm_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

int ep_hbm_fan(const void* src, void* dst, size_t slab_bytes, int fan_in, int fan_out,
               void* stream) {
    if (fan_in < 1 || fan_out < 1 || fan_in > 64 || fan_out > 64) return EP_ERR_ARG;
    if (slab_bytes > 0 && (!src || !dst)) return EP_ERR_ARG;
    if (slab_bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16)) return EP_ERR_ALIGN;
    return hip_status(ep::launch_hbm_fan(src, dst, slab_bytes, fan_in, fan_out,
                                         static_cast<hipStream_t>(stream)));
}

int ep_hbm_spread(const void* src, void* dst, size_t out_bytes, int fan_in, int regions,
                  void* stream) {
    if (fan_in < 1 || fan_in > 8 || regions < 1 || regions > EP_MAX_RANKS) return EP_ERR_ARG;
    if (out_bytes % EP_HBM_SPREAD_CHUNK_BYTES != 0) return EP_ERR_ARG;
    const uint64_t chunks = static_cast<uint64_t>(fan_in) * (out_bytes / EP_HBM_SPREAD_CHUNK_BYTES);
    if (chunks % static_cast<uint64_t>(regions) != 0) return EP_ERR_ARG;
    if (out_bytes > 0 && (!src || !dst)) return EP_ERR_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16)) return EP_ERR_ALIGN;
    return hip_status(ep::launch_hbm_spread(src, dst, out_bytes, fan_in, regions,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
