"""Single-GPU core of MoE expert-parallel dispatch/combine for AMD Instinct MI355X.

The four steps (layout, dispatch permute, restripe_prob, combine) run in hand-written
gfx950 HIP kernels behind the C ABI of include/ep.h; this package binds that ABI with
the same function names and uses torch only for device memory and streams.
"""
from ._binding import (EP_DEVERR_RECV_OVERFLOW, EP_DEVERR_SLOT_RANGE, EP_DEVERR_TOPK_RANGE,
                       EP_DEVERR_WORKSPACE,
                       EP_ERR_ALIGN, EP_ERR_ARG, EP_ERR_CAPACITY, EP_ERR_HIP,
                       EP_COUNTS_MAX_RANKS, EP_EXPERT_SLOT_MAX_K, EP_HBM_SPREAD_CHUNK_BYTES,
                       EP_LAYOUT_DISPATCH_MAX_TOKENS,
                       EP_LAYOUT_SCRATCH_BYTES,
                       EP_MAX_EXPERTS,
                       EP_MAX_RANKS, EP_OK, LIB_PATH, EPError, ep_combine, ep_combine_recv,
                       ep_combine_send, ep_dispatch, ep_dispatch_fp8, ep_dispatch_permute,
                       ep_dispatch_layout, ep_dispatch_permute_layout, ep_dispatch_preprocess, ep_dispatch_recv,
                       ep_layout_dispatch,
                       ep_dispatch_send, ep_layout_counts, ep_layout_counts_workspace_bytes,
                       ep_get_layout, ep_get_layout_no_alloc, ep_hbm_copy, ep_hbm_fan,
                       ep_hbm_spread,
                       ep_layout_workspace_bytes, ep_restripe_prob, ep_restripe_prob_sparse,
                       ep_status_string, load)
from .buffers import DispatchBuffers, LayoutBuffers, StageBuffers

__all__ = [
    "ep_get_layout", "ep_get_layout_no_alloc", "ep_dispatch_preprocess", "ep_layout_counts",
    "ep_layout_counts_workspace_bytes", "ep_dispatch_layout", "ep_dispatch_permute_layout",
    "ep_layout_dispatch",
    "ep_dispatch",
    "ep_dispatch_fp8", "ep_dispatch_permute", "ep_restripe_prob", "ep_restripe_prob_sparse",
    "ep_combine", "ep_dispatch_send", "ep_dispatch_recv", "ep_combine_send", "ep_combine_recv",
    "ep_hbm_copy", "ep_hbm_fan", "ep_hbm_spread", "ep_layout_workspace_bytes", "ep_status_string", "load",
    "EPError", "LIB_PATH", "LayoutBuffers", "DispatchBuffers", "StageBuffers",
    "EP_OK", "EP_ERR_ARG", "EP_ERR_ALIGN", "EP_ERR_CAPACITY", "EP_ERR_HIP",
    "EP_DEVERR_TOPK_RANGE", "EP_DEVERR_RECV_OVERFLOW", "EP_DEVERR_SLOT_RANGE",
    "EP_DEVERR_WORKSPACE",
    "EP_MAX_RANKS", "EP_MAX_EXPERTS", "EP_EXPERT_SLOT_MAX_K", "EP_LAYOUT_SCRATCH_BYTES",
    "EP_COUNTS_MAX_RANKS", "EP_LAYOUT_DISPATCH_MAX_TOKENS", "EP_HBM_SPREAD_CHUNK_BYTES",
]
