"""ctypes binding over libep.so: one Python function per C entry point of include/ep.h,
with the same names. Argument marshalling only: shapes, dtypes and devices of the torch
tensors are checked, their device pointers and the current HIP stream are passed on,
and a non-zero status becomes an ``EPError``. Every step of the path runs in the HIP
kernels behind the C ABI; there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep.so")

EP_OK, EP_ERR_ARG, EP_ERR_ALIGN, EP_ERR_CAPACITY, EP_ERR_HIP = 0, -1, -2, -3, -4
EP_DEVERR_TOPK_RANGE, EP_DEVERR_RECV_OVERFLOW, EP_DEVERR_SLOT_RANGE = 1, 2, 4
EP_DEVERR_WORKSPACE = 8
EP_MAX_RANKS, EP_MAX_EXPERTS, EP_EXPERT_SLOT_MAX_K = 1024, 8192, 16
EP_LAYOUT_SCRATCH_BYTES = 4 << 20
EP_COUNTS_MAX_RANKS = 64
EP_LAYOUT_DISPATCH_MAX_TOKENS = 256
EP_HBM_SPREAD_CHUNK_BYTES = 4096

_lib = None


class EPError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {ep_status_string(status)}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libep.so (built in-tree by __graft_entry__.build()); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.ep_status_string.argtypes = [i32]
    L.ep_status_string.restype = ctypes.c_char_p
    L.ep_layout_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.ep_layout_workspace_bytes.restype = sz
    L.ep_get_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, sz,
                                P]
    L.ep_get_layout_no_alloc.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                         P, P]
    L.ep_layout_counts_workspace_bytes.argtypes = [i64, i32, i32, i32]
    L.ep_layout_counts_workspace_bytes.restype = sz
    L.ep_layout_counts.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, i32, i64, P, P, sz, P]
    L.ep_dispatch_permute_layout.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P, P,
                                             P, P, i64, P, P, sz, P]
    L.ep_layout_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                     P, P, P, P, i64, P, i32, i64, P, P, P]
    L.ep_dispatch_layout.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                     P, P, P, P, i64, P, P, sz, P]
    L.ep_dispatch_preprocess.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P,
                                         P, P, i32, i64, P, P, sz, P]
    L.ep_restripe_prob_sparse.argtypes = [P, i64, i32, i32, P, i64, P, P, P]
    L.ep_dispatch_permute.argtypes = [P, P, i64, i32, i32, P, P, P, P, i64, P, P]
    L.ep_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, i64, P, P]
    L.ep_dispatch_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, i64, P,
                                  P]
    L.ep_restripe_prob.argtypes = [P, i64, i32, i32, i64, P, P]
    L.ep_combine.argtypes = [P, i64, P, i64, i32, i32, P, P, P]
    L.ep_dispatch_send.argtypes = [P, P, P, i64, i32, i32, i32, P, i64, P, P, P, P, P, i32, P]
    L.ep_dispatch_recv.argtypes = [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, i64, P, P, P,
                                   P, i64, P, P]
    L.ep_combine_send.argtypes = [P, i64, P, i64, i32, i32, i32, P, i64, P, P, i32, P]
    L.ep_combine_recv.argtypes = [P, i32, i64, P, i64, i32, P, P, P]
    L.ep_hbm_copy.argtypes = [P, P, sz, P]
    L.ep_hbm_fan.argtypes = [P, P, sz, i32, i32, P]
    L.ep_hbm_spread.argtypes = [P, P, sz, i32, i32, P]
    for f in ("ep_get_layout", "ep_get_layout_no_alloc", "ep_dispatch_preprocess",
              "ep_layout_counts", "ep_dispatch_layout", "ep_dispatch_permute_layout", "ep_dispatch", "ep_dispatch_fp8", "ep_dispatch_permute",
              "ep_restripe_prob", "ep_restripe_prob_sparse", "ep_combine", "ep_dispatch_send",
              "ep_dispatch_recv", "ep_combine_send", "ep_combine_recv", "ep_hbm_copy",
              "ep_hbm_fan", "ep_hbm_spread"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def ep_status_string(status: int) -> str:
    return load().ep_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor], dtype, name: str, nullable: bool = False):
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    _on_current_device(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _on_current_device(t: torch.Tensor, name: str) -> None:
    """Kernels run on the current device's stream, so every buffer must live there."""
    cur = torch.cuda.current_device()
    if t.device.index != cur:
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{cur}")


def _shape(t: Optional[torch.Tensor], shape, name: str) -> None:
    """Exact shape check; a leading entry of None in `shape` is not compared."""
    if t is None:
        return
    if t.dim() != len(shape) or any(w is not None and int(g) != int(w)
                                    for g, w in zip(t.shape, shape)):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _at_least(t: Optional[torch.Tensor], n: int, name: str) -> None:
    if t is not None and t.numel() < n:
        raise ValueError(f"{name}: needs at least {n} elements, has {t.numel()}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        cur = torch.cuda.current_device()
        if stream.device.index != cur:
            raise ValueError(f"stream is on {stream.device}, but the current device is cuda:{cur}")
        stream = stream.cuda_stream
    return ctypes.c_void_p(int(stream))


def _check(status: int, where: str) -> None:
    if status != EP_OK:
        raise EPError(status, where)


def ep_layout_workspace_bytes(num_tokens: int, num_experts: int, num_ranks: int,
                              num_nodes: int) -> int:
    return int(load().ep_layout_workspace_bytes(num_tokens, num_experts, num_ranks, num_nodes))


def _layout_outputs(topk_idx, E: int, R: int, N: int, num_tokens_per_rank, num_tokens_per_node,
                    num_tokens_per_expert, is_token_in_rank, rank_offset, expert_offset,
                    token_slot, expert_slot, node_slot, error_flag):
    """Shape checks and pointers of ep_get_layout's outputs, in the C argument order."""
    T, k = topk_idx.shape
    _at_least(num_tokens_per_rank, R, "num_tokens_per_rank")
    _at_least(num_tokens_per_node, N, "num_tokens_per_node")
    _at_least(num_tokens_per_expert, E, "num_tokens_per_expert")
    _shape(is_token_in_rank, (T, R), "is_token_in_rank")
    _at_least(rank_offset, R + 1, "rank_offset")
    _at_least(expert_offset, E + 1, "expert_offset")
    _shape(token_slot, (T, R), "token_slot")
    _shape(expert_slot, (T, k), "expert_slot")
    _shape(node_slot, (T, N), "node_slot")
    _at_least(error_flag, 1, "error_flag")
    return (_ptr(topk_idx, torch.int64, "topk_idx"), T, k, E, R, N,
            _ptr(num_tokens_per_rank, torch.int32, "num_tokens_per_rank"),
            _ptr(num_tokens_per_node, torch.int32, "num_tokens_per_node", True),
            _ptr(num_tokens_per_expert, torch.int32, "num_tokens_per_expert", True),
            _ptr(is_token_in_rank, torch.uint8, "is_token_in_rank", True),
            _ptr(rank_offset, torch.int32, "rank_offset"),
            _ptr(expert_offset, torch.int32, "expert_offset", True),
            _ptr(token_slot, torch.int32, "token_slot"),
            _ptr(expert_slot, torch.int32, "expert_slot", True),
            _ptr(node_slot, torch.int32, "node_slot", True),
            _ptr(error_flag, torch.int32, "error_flag"))


def ep_get_layout(topk_idx, num_experts: int, num_ranks: int, num_nodes: int, *,
                  num_tokens_per_rank, num_tokens_per_node, num_tokens_per_expert,
                  is_token_in_rank, rank_offset, expert_offset, token_slot, error_flag,
                  workspace, expert_slot=None, node_slot=None, stream=None) -> None:
    args = _layout_outputs(topk_idx, num_experts, num_ranks, num_nodes, num_tokens_per_rank,
                           num_tokens_per_node, num_tokens_per_expert, is_token_in_rank,
                           rank_offset, expert_offset, token_slot, expert_slot, node_slot,
                           error_flag)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().ep_get_layout(*args, _ptr(workspace, torch.uint8, "workspace", True),
                                ws_bytes, _stream(stream)), "ep_get_layout")


def ep_get_layout_no_alloc(topk_idx, num_experts: int, num_ranks: int, num_nodes: int, *,
                           num_tokens_per_rank, num_tokens_per_node, num_tokens_per_expert,
                           is_token_in_rank, rank_offset, expert_offset, token_slot,
                           error_flag, expert_slot=None, node_slot=None, stream=None) -> None:
    """ep_get_layout without a workspace: the library's static device scratch holds the
    per-block tables (sizes up to EP_LAYOUT_SCRATCH_BYTES of tables; calls overlapping in
    time on one GPU race on it)."""
    args = _layout_outputs(topk_idx, num_experts, num_ranks, num_nodes, num_tokens_per_rank,
                           num_tokens_per_node, num_tokens_per_expert, is_token_in_rank,
                           rank_offset, expert_offset, token_slot, expert_slot, node_slot,
                           error_flag)
    _check(load().ep_get_layout_no_alloc(*args, _stream(stream)), "ep_get_layout_no_alloc")


def ep_dispatch_preprocess(topk_idx, num_experts: int, num_ranks: int, num_nodes: int, prob,
                           prob_dest_major, *, num_tokens_per_rank, num_tokens_per_node,
                           num_tokens_per_expert, is_token_in_rank, rank_offset, expert_offset,
                           token_slot, error_flag, workspace, expert_slot=None, node_slot=None,
                           stream=None) -> None:
    """ep_get_layout and ep_restripe_prob in one call (the restripe rides along in the
    layout's first launch): prob fp32 [T][N][P] -> prob_dest_major fp32 [N][Tmax][P]."""
    T = topk_idx.shape[0]
    if prob.dim() != 3 or prob_dest_major.dim() != 3:
        raise ValueError("prob must be [T][N][P] and prob_dest_major [N][Tmax][P]")
    Tp, N, P = prob.shape
    Nd, Tmax, Pd = prob_dest_major.shape
    if Tp != T or N != num_nodes or Nd != N or Pd != P:
        raise ValueError(f"prob {tuple(prob.shape)} / prob_dest_major "
                         f"{tuple(prob_dest_major.shape)} do not match T={T}, N={num_nodes}")
    args = _layout_outputs(topk_idx, num_experts, num_ranks, num_nodes, num_tokens_per_rank,
                           num_tokens_per_node, num_tokens_per_expert, is_token_in_rank,
                           rank_offset, expert_offset, token_slot, expert_slot, node_slot,
                           error_flag)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().ep_dispatch_preprocess(
        *args, _ptr(prob, torch.float32, "prob"), P, Tmax,
        _ptr(prob_dest_major, torch.float32, "prob_dest_major"),
        _ptr(workspace, torch.uint8, "workspace", True), ws_bytes, _stream(stream)),
        "ep_dispatch_preprocess")


def ep_layout_counts_workspace_bytes(num_tokens: int, num_experts: int, num_ranks: int,
                                     num_nodes: int) -> int:
    return int(load().ep_layout_counts_workspace_bytes(num_tokens, num_experts, num_ranks,
                                                       num_nodes))


def ep_layout_counts(topk_idx, num_experts: int, num_ranks: int, num_nodes: int, *,
                     error_flag, workspace, prob=None, prob_dest_major=None, expert_rank=None,
                     stream=None) -> None:
    """The count launch of the counts path (num_ranks <= EP_COUNTS_MAX_RANKS): the
    per-block tables in `workspace` and the error flag; with expert_rank (int32 [T][k]) each
    pair's rank in its block among the pairs naming its expert; with prob the restripe of
    prob. The first 4 bytes of `workspace` (uint8, ep_layout_counts_workspace_bytes) must
    be zero before its first use; every call leaves them zero."""
    T, k = topk_idx.shape
    E, R, N = num_experts, num_ranks, num_nodes
    _at_least(error_flag, 1, "error_flag")
    _shape(expert_rank, (T, k), "expert_rank")
    P, Tmax = 0, 0
    if prob is not None:
        if prob.dim() != 3 or prob_dest_major is None or prob_dest_major.dim() != 3:
            raise ValueError("prob must be [T][N][P] and prob_dest_major [N][Tmax][P]")
        Tp, Np, P = prob.shape
        Nd, Tmax, Pd = prob_dest_major.shape
        if Tp != T or Np != N or Nd != N or Pd != P:
            raise ValueError("prob / prob_dest_major do not match the batch")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().ep_layout_counts(
        _ptr(topk_idx, torch.int64, "topk_idx"), T, k, E, R, N,
        _ptr(error_flag, torch.int32, "error_flag"),
        _ptr(expert_rank, torch.int32, "expert_rank", True),
        _ptr(prob, torch.float32, "prob", True), P, Tmax,
        _ptr(prob_dest_major, torch.float32, "prob_dest_major", True),
        _ptr(workspace, torch.uint8, "workspace"), ws_bytes, _stream(stream)), "ep_layout_counts")


def ep_dispatch_layout(x, topk_idx, topk_weights, num_experts: int, num_ranks: int,
                       num_nodes: int, *, token_slot, recv_x, workspace, is_token_in_rank=None,
                       num_tokens_per_rank=None, rank_offset=None, num_tokens_per_node=None,
                       num_tokens_per_expert=None, expert_offset=None, recv_topk_idx=None,
                       recv_topk_weights=None, recv_src_idx=None, error_flag=None,
                       stream=None) -> None:
    """The dispatch of the counts path, after ep_layout_counts on the same batch and
    workspace: ep_dispatch's outputs plus token_slot [T][R], is_token_in_rank [T][R] and the
    rank, node and expert counts and offsets."""
    T, H = x.shape
    k = topk_idx.shape[1]
    E, R, N = num_experts, num_ranks, num_nodes
    cap = recv_x.shape[0]
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(token_slot, (T, R), "token_slot")
    _shape(is_token_in_rank, (T, R), "is_token_in_rank")
    _at_least(num_tokens_per_rank, R, "num_tokens_per_rank")
    _at_least(rank_offset, R + 1, "rank_offset")
    _at_least(num_tokens_per_node, N, "num_tokens_per_node")
    _at_least(num_tokens_per_expert, E, "num_tokens_per_expert")
    _at_least(expert_offset, E + 1, "expert_offset")
    _shape(recv_x, (cap, H), "recv_x")
    _shape(recv_topk_idx, (cap, k), "recv_topk_idx")
    _shape(recv_topk_weights, (cap, k), "recv_topk_weights")
    _shape(recv_src_idx, (cap,), "recv_src_idx")
    _at_least(error_flag, 1, "error_flag")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().ep_dispatch_layout(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx"),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, E, R, N,
        _ptr(num_tokens_per_rank, torch.int32, "num_tokens_per_rank", True),
        _ptr(rank_offset, torch.int32, "rank_offset", True),
        _ptr(num_tokens_per_node, torch.int32, "num_tokens_per_node", True),
        _ptr(num_tokens_per_expert, torch.int32, "num_tokens_per_expert", True),
        _ptr(expert_offset, torch.int32, "expert_offset", True),
        _ptr(token_slot, torch.int32, "token_slot"),
        _ptr(is_token_in_rank, torch.uint8, "is_token_in_rank", True),
        _ptr(recv_x, torch.bfloat16, "recv_x"),
        _ptr(recv_topk_idx, torch.int64, "recv_topk_idx", True),
        _ptr(recv_topk_weights, torch.float32, "recv_topk_weights", True),
        _ptr(recv_src_idx, torch.int32, "recv_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True),
        _ptr(workspace, torch.uint8, "workspace"), ws_bytes, _stream(stream)),
        "ep_dispatch_layout")


def ep_layout_dispatch(x, topk_idx, topk_weights, num_experts: int, num_ranks: int,
                       num_nodes: int, *, token_slot, recv_x, num_tokens_per_rank, rank_offset,
                       error_flag, is_token_in_rank=None, num_tokens_per_node=None,
                       num_tokens_per_expert=None, expert_offset=None, recv_topk_idx=None,
                       recv_topk_weights=None, recv_src_idx=None, prob=None,
                       prob_dest_major=None, stream=None) -> None:
    """The layout, the dispatch and (with prob) the restripe of a batch of at most
    EP_LAYOUT_DISPATCH_MAX_TOKENS tokens in one launch: ep_get_layout's counts, offsets,
    token_slot and bitmap, ep_dispatch's outputs and prob_dest_major, and the error flag."""
    T, H = x.shape
    k = topk_idx.shape[1]
    E, R, N = num_experts, num_ranks, num_nodes
    cap = recv_x.shape[0]
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(token_slot, (T, R), "token_slot")
    _shape(is_token_in_rank, (T, R), "is_token_in_rank")
    _at_least(num_tokens_per_rank, R, "num_tokens_per_rank")
    _at_least(rank_offset, R + 1, "rank_offset")
    _at_least(num_tokens_per_node, N, "num_tokens_per_node")
    _at_least(num_tokens_per_expert, E, "num_tokens_per_expert")
    _at_least(expert_offset, E + 1, "expert_offset")
    _shape(recv_x, (cap, H), "recv_x")
    _shape(recv_topk_idx, (cap, k), "recv_topk_idx")
    _shape(recv_topk_weights, (cap, k), "recv_topk_weights")
    _shape(recv_src_idx, (cap,), "recv_src_idx")
    _at_least(error_flag, 1, "error_flag")
    P, Tmax = 0, 0
    if prob is not None:
        if prob.dim() != 3 or prob_dest_major is None or prob_dest_major.dim() != 3:
            raise ValueError("prob must be [T][N][P] and prob_dest_major [N][Tmax][P]")
        Tp, Np, P = prob.shape
        Nd, Tmax, Pd = prob_dest_major.shape
        if Tp != T or Np != N or Nd != N or Pd != P:
            raise ValueError("prob / prob_dest_major do not match the batch")
    _check(load().ep_layout_dispatch(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx"),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, E, R, N,
        _ptr(num_tokens_per_rank, torch.int32, "num_tokens_per_rank"),
        _ptr(rank_offset, torch.int32, "rank_offset"),
        _ptr(num_tokens_per_node, torch.int32, "num_tokens_per_node", True),
        _ptr(num_tokens_per_expert, torch.int32, "num_tokens_per_expert", True),
        _ptr(expert_offset, torch.int32, "expert_offset", True),
        _ptr(token_slot, torch.int32, "token_slot"),
        _ptr(is_token_in_rank, torch.uint8, "is_token_in_rank", True),
        _ptr(recv_x, torch.bfloat16, "recv_x"),
        _ptr(recv_topk_idx, torch.int64, "recv_topk_idx", True),
        _ptr(recv_topk_weights, torch.float32, "recv_topk_weights", True),
        _ptr(recv_src_idx, torch.int32, "recv_src_idx", True), cap,
        _ptr(prob, torch.float32, "prob", True), P, Tmax,
        _ptr(prob_dest_major, torch.float32, "prob_dest_major", True),
        _ptr(error_flag, torch.int32, "error_flag"), _stream(stream)), "ep_layout_dispatch")


def ep_dispatch_permute_layout(x, topk_idx, topk_weights, num_experts: int, num_ranks: int,
                               num_nodes: int, *, expert_rank, perm_x, workspace,
                               perm_weights=None, perm_src_idx=None, expert_slot=None,
                               num_tokens_per_expert=None, expert_offset=None, error_flag=None,
                               stream=None) -> None:
    """The counts path's dispatch + permute, after ep_layout_counts on the same batch and
    workspace with expert_rank: ep_dispatch_permute's outputs, the rows formed in the
    permute's waves; optionally expert_slot [T][k] and the expert counts and offsets.
    T <= 16384."""
    T, H = x.shape
    k = topk_idx.shape[1]
    E, R, N = num_experts, num_ranks, num_nodes
    cap = perm_x.shape[0]
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(expert_rank, (T, k), "expert_rank")
    _shape(expert_slot, (T, k), "expert_slot")
    _at_least(num_tokens_per_expert, E, "num_tokens_per_expert")
    _at_least(expert_offset, E + 1, "expert_offset")
    _shape(perm_x, (cap, H), "perm_x")
    _shape(perm_weights, (cap,), "perm_weights")
    _shape(perm_src_idx, (cap,), "perm_src_idx")
    _at_least(error_flag, 1, "error_flag")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().ep_dispatch_permute_layout(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx"),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, E, R, N,
        _ptr(expert_rank, torch.int32, "expert_rank"),
        _ptr(num_tokens_per_expert, torch.int32, "num_tokens_per_expert", True),
        _ptr(expert_offset, torch.int32, "expert_offset", True),
        _ptr(expert_slot, torch.int32, "expert_slot", True),
        _ptr(perm_x, torch.bfloat16, "perm_x"),
        _ptr(perm_weights, torch.float32, "perm_weights", True),
        _ptr(perm_src_idx, torch.int32, "perm_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True),
        _ptr(workspace, torch.uint8, "workspace"), ws_bytes, _stream(stream)),
        "ep_dispatch_permute_layout")


def ep_dispatch(x, topk_idx, topk_weights, num_experts: int, num_ranks: int, token_slot, *,
                recv_x, recv_topk_idx=None, recv_topk_weights=None, recv_src_idx=None,
                error_flag=None, stream=None) -> None:
    T, H = x.shape
    k = topk_idx.shape[1]
    cap = recv_x.shape[0]
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(token_slot, (T, num_ranks), "token_slot")
    _shape(recv_x, (cap, H), "recv_x")
    _shape(recv_topk_idx, (cap, k), "recv_topk_idx")
    _shape(recv_topk_weights, (cap, k), "recv_topk_weights")
    _shape(recv_src_idx, (cap,), "recv_src_idx")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_dispatch(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx"),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, num_experts,
        num_ranks, _ptr(token_slot, torch.int32, "token_slot"),
        _ptr(recv_x, torch.bfloat16, "recv_x"),
        _ptr(recv_topk_idx, torch.int64, "recv_topk_idx", True),
        _ptr(recv_topk_weights, torch.float32, "recv_topk_weights", True),
        _ptr(recv_src_idx, torch.int32, "recv_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)), "ep_dispatch")


def ep_dispatch_fp8(x, topk_idx, topk_weights, num_experts: int, num_ranks: int, token_slot, *,
                    recv_x_fp8, recv_scales, recv_topk_idx=None, recv_topk_weights=None,
                    recv_src_idx=None, error_flag=None, stream=None) -> None:
    """recv_x_fp8: uint8 or float8_e4m3fn [cap][H]; recv_scales: fp32 [cap][H/128]."""
    T, H = x.shape
    k = topk_idx.shape[1]
    cap = recv_x_fp8.shape[0]
    if recv_x_fp8.dtype == torch.float8_e4m3fn:
        recv_x_fp8 = recv_x_fp8.view(torch.uint8)
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(token_slot, (T, num_ranks), "token_slot")
    _shape(recv_x_fp8, (cap, H), "recv_x_fp8")
    _shape(recv_scales, (cap, H // 128), "recv_scales")
    _shape(recv_topk_idx, (cap, k), "recv_topk_idx")
    _shape(recv_topk_weights, (cap, k), "recv_topk_weights")
    _shape(recv_src_idx, (cap,), "recv_src_idx")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_dispatch_fp8(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx"),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, num_experts,
        num_ranks, _ptr(token_slot, torch.int32, "token_slot"),
        _ptr(recv_x_fp8, torch.uint8, "recv_x_fp8"),
        _ptr(recv_scales, torch.float32, "recv_scales"),
        _ptr(recv_topk_idx, torch.int64, "recv_topk_idx", True),
        _ptr(recv_topk_weights, torch.float32, "recv_topk_weights", True),
        _ptr(recv_src_idx, torch.int32, "recv_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)), "ep_dispatch_fp8")


def ep_dispatch_permute(x, topk_weights, expert_slot, *, perm_x, perm_weights=None,
                        perm_src_idx=None, error_flag=None, stream=None) -> None:
    """x: bf16 [T][H]; expert_slot: int32 [T][k]; perm_x: bf16 [cap][H]."""
    T, H = x.shape
    k = expert_slot.shape[1]
    cap = perm_x.shape[0]
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(expert_slot, (T, k), "expert_slot")
    _shape(perm_x, (cap, H), "perm_x")
    _shape(perm_weights, (cap,), "perm_weights")
    _shape(perm_src_idx, (cap,), "perm_src_idx")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_dispatch_permute(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_weights, torch.float32, "topk_weights", True),
        T, H, k, _ptr(expert_slot, torch.int32, "expert_slot"),
        _ptr(perm_x, torch.bfloat16, "perm_x"),
        _ptr(perm_weights, torch.float32, "perm_weights", True),
        _ptr(perm_src_idx, torch.int32, "perm_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)), "ep_dispatch_permute")


def ep_restripe_prob(prob, prob_dest_major, stream=None) -> None:
    """prob: fp32 [T][N][P]; prob_dest_major: fp32 [N][Tmax][P]."""
    T, N, P = prob.shape
    if prob_dest_major.dim() != 3 or prob_dest_major.shape[0] != N or \
            prob_dest_major.shape[2] != P:
        raise ValueError("prob_dest_major must be [N][Tmax][P]")
    _check(load().ep_restripe_prob(
        _ptr(prob, torch.float32, "prob"), T, N, P, prob_dest_major.shape[1],
        _ptr(prob_dest_major, torch.float32, "prob_dest_major"), _stream(stream)),
        "ep_restripe_prob")


def ep_restripe_prob_sparse(prob, node_slot, prob_dest_major, error_flag=None,
                            stream=None) -> None:
    """prob: fp32 [T][N][P]; node_slot: int32 [T][N]; prob_dest_major: fp32 [N][Tmax][P]."""
    T, N, P = prob.shape
    if prob_dest_major.dim() != 3 or prob_dest_major.shape[0] != N or \
            prob_dest_major.shape[2] != P:
        raise ValueError("prob_dest_major must be [N][Tmax][P]")
    _shape(node_slot, (T, N), "node_slot")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_restripe_prob_sparse(
        _ptr(prob, torch.float32, "prob"), T, N, P, _ptr(node_slot, torch.int32, "node_slot"),
        prob_dest_major.shape[1], _ptr(prob_dest_major, torch.float32, "prob_dest_major"),
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)),
        "ep_restripe_prob_sparse")


def ep_combine(partial, token_slot, *, out, error_flag=None, stream=None) -> None:
    """partial: bf16 [rows][H]; token_slot: int32 [T][R]; out: bf16 [T][H]."""
    rows, H = partial.shape
    T, R = token_slot.shape
    _shape(out, (T, H), "out")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_combine(
        _ptr(partial, torch.bfloat16, "partial"), rows, _ptr(token_slot, torch.int32, "token_slot"),
        T, H, R, _ptr(out, torch.bfloat16, "out"),
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)), "ep_combine")


def _stage_dims(stage_x, name="stage_x"):
    if stage_x.dim() != 3:
        raise ValueError(f"{name} must be [N][Tmax][H]")
    return tuple(int(d) for d in stage_x.shape)


def ep_dispatch_send(x, topk_idx, topk_weights, node_slot, *, stage_x, stage_topk_idx=None,
                     stage_topk_weights=None, stage_src, error_flag=None, num_workgroups: int = 0,
                     stream=None) -> None:
    """Send phase of the two-phase dispatch. x: bf16 [T][H]; node_slot: int32 [T][N];
    stage_x: bf16 [N][Tmax][H]; stage_topk_idx / weights: [N][Tmax][k]; stage_src: [N][Tmax].
    num_workgroups: 0 = full grid, else the most workgroups the send occupies."""
    T, H = x.shape
    N, Tmax, Hs = _stage_dims(stage_x)
    k = topk_idx.shape[1] if topk_idx is not None else 1
    if Hs != H:
        raise ValueError("stage_x: hidden size differs from x")
    _shape(topk_idx, (T, k), "topk_idx")
    _shape(topk_weights, (T, k), "topk_weights")
    _shape(node_slot, (T, N), "node_slot")
    _shape(stage_topk_idx, (N, Tmax, k), "stage_topk_idx")
    _shape(stage_topk_weights, (N, Tmax, k), "stage_topk_weights")
    _shape(stage_src, (N, Tmax), "stage_src")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_dispatch_send(
        _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int64, "topk_idx", True),
        _ptr(topk_weights, torch.float32, "topk_weights", True), T, H, k, N,
        _ptr(node_slot, torch.int32, "node_slot"), Tmax, _ptr(stage_x, torch.bfloat16, "stage_x"),
        _ptr(stage_topk_idx, torch.int64, "stage_topk_idx", True),
        _ptr(stage_topk_weights, torch.float32, "stage_topk_weights", True),
        _ptr(stage_src, torch.int32, "stage_src"),
        _ptr(error_flag, torch.int32, "error_flag", True), int(num_workgroups), _stream(stream)),
        "ep_dispatch_send")


def ep_dispatch_recv(stage_x, stage_topk_idx, stage_topk_weights, stage_src, count_n,
                     num_experts: int, num_ranks: int, token_slot, *, recv_x, recv_topk_idx=None,
                     recv_topk_weights=None, recv_src_idx=None, num_topk: Optional[int] = None,
                     error_flag=None, stream=None) -> None:
    """Receive phase: forwards the staged rows to the ranks of each node, writing exactly
    what ep_dispatch writes. count_n: int32 [N] (num_tokens_per_node)."""
    N, Tmax, H = _stage_dims(stage_x)
    T, R = token_slot.shape
    if num_topk is None:
        if stage_topk_idx is None:
            raise ValueError("num_topk is needed when stage_topk_idx is None")
        num_topk = stage_topk_idx.shape[2]
    k = num_topk
    cap = recv_x.shape[0]
    _shape(stage_topk_idx, (N, Tmax, k), "stage_topk_idx")
    _shape(stage_topk_weights, (N, Tmax, k), "stage_topk_weights")
    _shape(stage_src, (N, Tmax), "stage_src")
    _at_least(count_n, N, "count_n")
    _shape(recv_x, (cap, H), "recv_x")
    _shape(recv_topk_idx, (cap, k), "recv_topk_idx")
    _shape(recv_topk_weights, (cap, k), "recv_topk_weights")
    _shape(recv_src_idx, (cap,), "recv_src_idx")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_dispatch_recv(
        _ptr(stage_x, torch.bfloat16, "stage_x"),
        _ptr(stage_topk_idx, torch.int64, "stage_topk_idx", True),
        _ptr(stage_topk_weights, torch.float32, "stage_topk_weights", True),
        _ptr(stage_src, torch.int32, "stage_src"), _ptr(count_n, torch.int32, "count_n"), N, Tmax,
        H, k, num_experts, num_ranks, _ptr(token_slot, torch.int32, "token_slot"), T,
        _ptr(recv_x, torch.bfloat16, "recv_x"),
        _ptr(recv_topk_idx, torch.int64, "recv_topk_idx", True),
        _ptr(recv_topk_weights, torch.float32, "recv_topk_weights", True),
        _ptr(recv_src_idx, torch.int32, "recv_src_idx", True), cap,
        _ptr(error_flag, torch.int32, "error_flag", True), _stream(stream)), "ep_dispatch_recv")


def ep_combine_send(partial, token_slot, node_slot, *, stage, error_flag=None,
                    num_workgroups: int = 0, stream=None) -> None:
    """Send phase of the two-phase combine: per (token, node) bf16 sums of the node's
    partial rows. partial: bf16 [rows][H]; stage: bf16 [N][Tmax][H].
    num_workgroups: 0 = full grid, else the most workgroups the send occupies."""
    rows, H = partial.shape
    T, R = token_slot.shape
    N, Tmax, Hs = _stage_dims(stage, "stage")
    if Hs != H:
        raise ValueError("stage: hidden size differs from partial")
    _shape(node_slot, (T, N), "node_slot")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_combine_send(
        _ptr(partial, torch.bfloat16, "partial"), rows, _ptr(token_slot, torch.int32, "token_slot"),
        T, H, R, N, _ptr(node_slot, torch.int32, "node_slot"), Tmax,
        _ptr(stage, torch.bfloat16, "stage"), _ptr(error_flag, torch.int32, "error_flag", True),
        int(num_workgroups), _stream(stream)), "ep_combine_send")


def ep_combine_recv(stage, node_slot, *, out, error_flag=None, stream=None) -> None:
    """Receive phase: out[t] = bf16 of the fp32 sum of t's staged node rows."""
    N, Tmax, H = _stage_dims(stage, "stage")
    T = node_slot.shape[0]
    _shape(node_slot, (T, N), "node_slot")
    _shape(out, (T, H), "out")
    _at_least(error_flag, 1, "error_flag")
    _check(load().ep_combine_recv(
        _ptr(stage, torch.bfloat16, "stage"), N, Tmax, _ptr(node_slot, torch.int32, "node_slot"),
        T, H, _ptr(out, torch.bfloat16, "out"), _ptr(error_flag, torch.int32, "error_flag", True),
        _stream(stream)), "ep_combine_recv")


def ep_hbm_copy(src, dst, nbytes: Optional[int] = None, stream=None) -> None:
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be device tensors")
    _on_current_device(src, "src")
    _on_current_device(dst, "dst")
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    if nbytes > src.numel() * src.element_size() or nbytes > dst.numel() * dst.element_size():
        raise ValueError("nbytes exceeds a buffer")
    _check(load().ep_hbm_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                              nbytes, _stream(stream)), "ep_hbm_copy")


def ep_hbm_fan(src, dst, slab_bytes: int, fan_in: int, fan_out: int, stream=None) -> None:
    """Measurement helper: each of the fan_out slabs of dst becomes the XOR of the fan_in
    slabs of src (slabs of slab_bytes, contiguous)."""
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be device tensors")
    _on_current_device(src, "src")
    _on_current_device(dst, "dst")
    if (fan_in * slab_bytes > src.numel() * src.element_size() or
            fan_out * slab_bytes > dst.numel() * dst.element_size()):
        raise ValueError("fan_in / fan_out slabs exceed a buffer")
    _check(load().ep_hbm_fan(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                             slab_bytes, fan_in, fan_out, _stream(stream)), "ep_hbm_fan")



def ep_hbm_spread(src, dst, out_bytes: int, fan_in: int, regions: int, stream=None) -> None:
    """Measurement helper: output chunk b of dst (chunks of EP_HBM_SPREAD_CHUNK_BYTES)
    becomes the XOR of the input chunks fan_in*b .. fan_in*b + fan_in - 1 of src, input
    chunk j being chunk j // regions of region j % regions (src = fan_in * out_bytes bytes
    in `regions` equal regions)."""
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be device tensors")
    _on_current_device(src, "src")
    _on_current_device(dst, "dst")
    if (fan_in * out_bytes > src.numel() * src.element_size() or
            out_bytes > dst.numel() * dst.element_size()):
        raise ValueError("fan_in * out_bytes or out_bytes exceeds a buffer")
    _check(load().ep_hbm_spread(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                out_bytes, fan_in, regions, _stream(stream)), "ep_hbm_spread")
