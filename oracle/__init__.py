"""CPU oracle -- TEST INFRASTRUCTURE.

numpy front end over ``liboracle.so`` (plain single-threaded C, see oracle.c).
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """The oracle library; EP_ORACLE_LIB names another build of oracle.c (the mutation
    tests load deliberately broken builds this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("EP_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.oracle_dispatch.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i64, P, P, P, P]
        L.oracle_restripe_prob.argtypes = [P, i64, i32, i32, i64, P]
        L.oracle_combine.argtypes = [P, i64, P, i64, i32, i32, P]
        L.oracle_f32_to_bf16_array.argtypes = [P, i64, P]
        L.oracle_f32_to_bf16_array.restype = None
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_quantize_fp8.argtypes = [P, i64, i32, P, P]
        L.oracle_dispatch_fp8.argtypes = [P, P, P, i64, i32, i32, i32, i32, P, i64, P, P, P, P,
                                          P]
        L.oracle_expert_slots.argtypes = [P, i64, i32, i32, P]
        L.oracle_node_slots.argtypes = [P, i64, i32, i32, i32, i32, P]
        L.oracle_restripe_prob_sparse.argtypes = [P, i64, i32, i32, P, i64, P]
        L.oracle_dispatch_permute.argtypes = [P, P, P, i64, i32, i32, P, i64, P, P, P]
        L.oracle_hook_dispatch_send.argtypes = [P, P, P, i64, i32, i32, i32, P, i64, P, P, P, P]
        L.oracle_hook_dispatch_recv.argtypes = [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P,
                                                i64, i64, P, P, P, P]
        L.oracle_hook_combine_send.argtypes = [P, i64, P, i64, i32, i32, i32, P, i64, P]
        L.oracle_hook_combine_recv.argtypes = [P, i32, i64, P, i64, i32, P]
        L.oracle_f32_to_e4m3_array.argtypes = [P, i64, P]
        L.oracle_f32_to_e4m3_array.restype = None
        L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f32.restype = ctypes.c_float
        for f in ("oracle_layout", "oracle_dispatch", "oracle_restripe_prob", "oracle_combine",
                  "oracle_quantize_fp8", "oracle_dispatch_fp8", "oracle_expert_slots",
                  "oracle_dispatch_permute", "oracle_node_slots",
                  "oracle_restripe_prob_sparse", "oracle_hook_dispatch_send",
                  "oracle_hook_dispatch_recv", "oracle_hook_combine_send",
                  "oracle_hook_combine_recv"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def layout(topk_idx, E: int, R: int, N: int) -> dict:
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    out = dict(
        count_r=np.zeros(R, np.int32), count_n=np.zeros(N, np.int32),
        count_e=np.zeros(E, np.int32), in_rank=np.zeros((T, R), np.uint8),
        rank_offset=np.zeros(R + 1, np.int32), expert_offset=np.zeros(E + 1, np.int32),
        token_slot=np.zeros((T, R), np.int32), error_flag=np.zeros(1, np.int32))
    rc = lib().oracle_layout(_p(idx), T, k, E, R, N, _p(out["count_r"]), _p(out["count_n"]),
                             _p(out["count_e"]), _p(out["in_rank"]), _p(out["rank_offset"]),
                             _p(out["expert_offset"]), _p(out["token_slot"]),
                             _p(out["error_flag"]))
    if rc != 0:
        raise ValueError("oracle_layout: bad arguments")
    return out


def dispatch(x, topk_idx, topk_w, E: int, R: int, token_slot, cap: int) -> dict:
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    slot = _c(token_slot, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    out = dict(recv_x=np.zeros((cap, H), np.uint16), recv_idx=np.zeros((cap, k), np.int64),
               recv_w=np.zeros((cap, k), np.float32), recv_src=np.zeros(cap, np.int32))
    rc = lib().oracle_dispatch(_p(x), _p(idx), _p(w), T, H, k, E, R, _p(slot), cap,
                               _p(out["recv_x"]), _p(out["recv_idx"]), _p(out["recv_w"]),
                               _p(out["recv_src"]))
    if rc != 0:
        raise ValueError("oracle_dispatch: bad arguments or slot beyond capacity")
    return out


def restripe_prob(prob, Tmax: int, out=None) -> np.ndarray:
    """prob: float32 [T][N][P] (copied as 32-bit words). Returns [N][Tmax][P]."""
    pw = np.ascontiguousarray(prob).view(np.uint32)
    T, N, P = pw.shape
    if out is None:
        out = np.zeros((N, Tmax, P), np.float32)
    ow = out.view(np.uint32)
    rc = lib().oracle_restripe_prob(_p(pw), T, N, P, Tmax, _p(ow))
    if rc != 0:
        raise ValueError("oracle_restripe_prob: bad arguments")
    return out


def combine(partial, token_slot, R: int) -> np.ndarray:
    partial = _c(partial, np.uint16)
    slot = _c(token_slot, np.int32)
    rows, H = partial.shape
    T = slot.shape[0]
    out = np.zeros((T, H), np.uint16)
    rc = lib().oracle_combine(_p(partial), rows, _p(slot), T, H, R, _p(out))
    if rc != 0:
        raise ValueError("oracle_combine: bad arguments or slot beyond the partial rows")
    return out


def f32_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(_p(a), a.size, _p(out))
    return out


def bf16_to_f32(b) -> np.ndarray:
    """bf16 bit patterns widened to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_e4m3(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().oracle_f32_to_e4m3_array(_p(a), a.size, _p(out))
    return out


def e4m3_to_f32(codes) -> np.ndarray:
    L = lib()
    table = np.array([L.oracle_e4m3_to_f32(c) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def quantize_fp8(x) -> tuple:
    """bf16 bits [T][H] -> (e4m3 codes uint8 [T][H], fp32 scales [T][H/128])."""
    x = _c(x, np.uint16)
    T, H = x.shape
    codes = np.zeros((T, H), np.uint8)
    scales = np.zeros((T, max(H // 128, 1)), np.float32)
    if lib().oracle_quantize_fp8(_p(x), T, H, _p(codes), _p(scales)) != 0:
        raise ValueError("oracle_quantize_fp8: H must be a multiple of 128")
    return codes, scales


def dispatch_fp8(x, topk_idx, topk_w, E: int, R: int, token_slot, cap: int) -> dict:
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    slot = _c(token_slot, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    G = max(H // 128, 1)
    out = dict(recv_codes=np.zeros((cap, H), np.uint8), recv_scales=np.zeros((cap, G), np.float32),
               recv_idx=np.zeros((cap, k), np.int64), recv_w=np.zeros((cap, k), np.float32),
               recv_src=np.zeros(cap, np.int32))
    rc = lib().oracle_dispatch_fp8(_p(x), _p(idx), _p(w), T, H, k, E, R, _p(slot), cap,
                                   _p(out["recv_codes"]), _p(out["recv_scales"]),
                                   _p(out["recv_idx"]), _p(out["recv_w"]), _p(out["recv_src"]))
    if rc != 0:
        raise ValueError("oracle_dispatch_fp8: bad arguments or slot beyond capacity")
    return out


def expert_slots(topk_idx, E: int) -> np.ndarray:
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    out = np.zeros((T, k), np.int32)
    if lib().oracle_expert_slots(_p(idx), T, k, E, _p(out)) != 0:
        raise ValueError("oracle_expert_slots: bad arguments")
    return out


def dispatch_permute(x, topk_idx, topk_w, expert_slot, cap: int) -> dict:
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    es = _c(expert_slot, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    out = dict(perm_x=np.zeros((cap, H), np.uint16), perm_w=np.zeros(cap, np.float32),
               perm_src=np.zeros(cap, np.int32))
    rc = lib().oracle_dispatch_permute(_p(x), _p(idx), _p(w), T, H, k, _p(es), cap,
                                       _p(out["perm_x"]), _p(out["perm_w"]), _p(out["perm_src"]))
    if rc != 0:
        raise ValueError("oracle_dispatch_permute: bad arguments or row beyond capacity")
    return out


def node_slots(topk_idx, E: int, R: int, N: int) -> np.ndarray:
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    out = np.zeros((T, N), np.int32)
    if lib().oracle_node_slots(_p(idx), T, k, E, R, N, _p(out)) != 0:
        raise ValueError("oracle_node_slots: bad arguments")
    return out


def restripe_prob_sparse(prob, node_slot, Tmax: int, out=None) -> np.ndarray:
    pw = np.ascontiguousarray(prob).view(np.uint32)
    T, N, P = pw.shape
    ns = _c(node_slot, np.int32)
    if out is None:
        out = np.zeros((N, Tmax, P), np.float32)
    rc = lib().oracle_restripe_prob_sparse(_p(pw), T, N, P, _p(ns), Tmax, _p(out.view(np.uint32)))
    if rc != 0:
        raise ValueError("oracle_restripe_prob_sparse: bad arguments")
    return out


def hook_dispatch_send(x, topk_idx, topk_w, node_slot, Tmax: int, out=None) -> dict:
    """Send phase of the two-phase dispatch. Returns (or fills) the staging buffers
    stage_x [N][Tmax][H] (bf16 bits), stage_idx [N][Tmax][k], stage_w, stage_src [N][Tmax]."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    ns = _c(node_slot, np.int32)
    T, H = x.shape
    k = idx.shape[1]
    N = ns.shape[1]
    if out is None:
        out = dict(stage_x=np.zeros((N, Tmax, H), np.uint16),
                   stage_idx=np.zeros((N, Tmax, k), np.int64),
                   stage_w=np.zeros((N, Tmax, k), np.float32),
                   stage_src=np.zeros((N, Tmax), np.int32))
    rc = lib().oracle_hook_dispatch_send(_p(x), _p(idx), _p(w), T, H, k, N, _p(ns), Tmax,
                                         _p(out["stage_x"]), _p(out["stage_idx"]),
                                         _p(out["stage_w"]), _p(out["stage_src"]))
    if rc != 0:
        raise ValueError("oracle_hook_dispatch_send: bad arguments or node slot beyond Tmax")
    return out


def hook_dispatch_recv(stage: dict, count_n, E: int, R: int, token_slot, cap: int,
                       out=None) -> dict:
    """Receive phase: forwards the staged rows to the ranks of each node."""
    sx = stage["stage_x"]
    N, Tmax, H = sx.shape
    k = stage["stage_idx"].shape[2]
    slot = _c(token_slot, np.int32)
    cn = _c(count_n, np.int32)
    T = slot.shape[0]
    if out is None:
        out = dict(recv_x=np.zeros((cap, H), np.uint16), recv_idx=np.zeros((cap, k), np.int64),
                   recv_w=np.zeros((cap, k), np.float32), recv_src=np.zeros(cap, np.int32))
    rc = lib().oracle_hook_dispatch_recv(
        _p(sx), _p(stage["stage_idx"]), _p(stage["stage_w"]), _p(stage["stage_src"]), _p(cn),
        N, Tmax, H, k, E, R, _p(slot), T, cap, _p(out["recv_x"]), _p(out["recv_idx"]),
        _p(out["recv_w"]), _p(out["recv_src"]))
    if rc != 0:
        raise ValueError("oracle_hook_dispatch_recv: bad arguments, staged token or slot "
                         "out of range")
    return out


def hook_combine_send(partial, token_slot, R: int, node_slot, Tmax: int, out=None) -> np.ndarray:
    """Send phase of the two-phase combine: per (token, node) bf16 sums, [N][Tmax][H]."""
    partial = _c(partial, np.uint16)
    slot = _c(token_slot, np.int32)
    ns = _c(node_slot, np.int32)
    rows, H = partial.shape
    T, N = ns.shape
    if out is None:
        out = np.zeros((N, Tmax, H), np.uint16)
    rc = lib().oracle_hook_combine_send(_p(partial), rows, _p(slot), T, H, R, N, _p(ns), Tmax,
                                        _p(out))
    if rc != 0:
        raise ValueError("oracle_hook_combine_send: bad arguments or slot out of range")
    return out


def hook_combine_recv(stage, node_slot) -> np.ndarray:
    """Receive phase: out[t] = bf16 of the fp32 sum of t's staged node rows."""
    stage = _c(stage, np.uint16)
    ns = _c(node_slot, np.int32)
    N, Tmax, H = stage.shape
    T = ns.shape[0]
    out = np.zeros((T, H), np.uint16)
    if lib().oracle_hook_combine_recv(_p(stage), N, Tmax, _p(ns), T, H, _p(out)) != 0:
        raise ValueError("oracle_hook_combine_recv: bad arguments or node slot beyond Tmax")
    return out
