"""One batch through the whole path on the GPU, on one stream, in three forms with the same
outputs:
- the counts path (R <= EP_COUNTS_MAX_RANKS): ep_layout_counts (counts, offsets and the
  restripe in one launch), ep_dispatch_layout (the dispatch computing the receive rows and
  writing the slot table), ep_combine; for a batch of at most
  EP_LAYOUT_DISPATCH_MAX_TOKENS tokens the first two are one call, ep_layout_dispatch;
- the preprocess path: ep_dispatch_preprocess (layout and restripe in one call),
  ep_dispatch, ep_combine;
- one call per step: ep_get_layout, ep_dispatch, ep_restripe_prob, ep_combine.
`step()` takes the one-call layout + dispatch or the counts path where they apply. Also the two-phase ("hook") form of
dispatch and combine, whose send phase returns a callable that enqueues the receive phase
later.

Device buffers are allocated once per shape (torch, memory plumbing only); the step
functions enqueue their calls and return without synchronising.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _binding as B
from .buffers import DispatchBuffers, LayoutBuffers, StageBuffers


@dataclasses.dataclass
class DeviceBatch:
    topk_idx: torch.Tensor                 # int64 [T][k]
    topk_weights: torch.Tensor             # fp32 [T][k]
    x: torch.Tensor                        # bf16 [T][H]
    prob: torch.Tensor                     # fp32 [T][N][P]
    partials: Optional[torch.Tensor]       # bf16 [rows][H]; None = combine the dispatched rows

    @classmethod
    def from_host(cls, topk_idx, topk_weights, x_bits, prob, partial_bits=None,
                  device="cuda") -> "DeviceBatch":
        """numpy inputs (bf16 as uint16 bit patterns) copied to the device."""
        import numpy as np

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)

        return cls(torch.from_numpy(np.ascontiguousarray(topk_idx)).to(device),
                   torch.from_numpy(np.ascontiguousarray(topk_weights)).to(device),
                   bf16(x_bits), torch.from_numpy(np.ascontiguousarray(prob)).to(device),
                   None if partial_bits is None else bf16(partial_bits))


class Path:
    """Buffers and calls for one shape: T tokens, hidden H, E experts, top-k, R ranks,
    N nodes, P prob floats per (token, node), Tmax rows per node block."""

    def __init__(self, T: int, H: int, E: int, k: int, R: int, N: int, P: int, Tmax: int,
                 device="cuda", recv_capacity: Optional[int] = None, node_slots: bool = False):
        self.T, self.H, self.E, self.k, self.R, self.N, self.P, self.Tmax = T, H, E, k, R, N, P, Tmax
        self.cap = T * min(k, R) if recv_capacity is None else recv_capacity
        self.layout_buf = LayoutBuffers.alloc(T, E, R, N, device, node_slots=node_slots)
        self.recv = DispatchBuffers.alloc(self.cap, H, k, device)
        self.prob_dest_major = torch.empty((N, Tmax, P), dtype=torch.float32, device=device)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
        self.stage: Optional[StageBuffers] = None
        self._dispatch_pending = False  # a dispatch send whose receive hook has not run
        # The counts path writes no node slots, so a Path that keeps them for the two-phase
        # calls steps on the preprocess path.
        self.counts_path = R <= B.EP_COUNTS_MAX_RANKS and not node_slots
        self.counts_ws: Optional[torch.Tensor] = None  # workspace of the counts path
        if self.counts_path:
            self._counts_workspace()

    @property
    def error_flag(self) -> torch.Tensor:
        return self.layout_buf.error_flag

    def layout(self, b: DeviceBatch, stream=None) -> None:
        self.layout_buf.compute(b.topk_idx, self.E, self.R, self.N, stream=stream)

    def dispatch(self, b: DeviceBatch, stream=None) -> None:
        r = self.recv
        B.ep_dispatch(b.x, b.topk_idx, b.topk_weights, self.E, self.R,
                      self.layout_buf.token_slot, recv_x=r.recv_x, recv_topk_idx=r.recv_topk_idx,
                      recv_topk_weights=r.recv_topk_weights, recv_src_idx=r.recv_src_idx,
                      error_flag=self.error_flag, stream=stream)

    def restripe(self, b: DeviceBatch, stream=None) -> None:
        B.ep_restripe_prob(b.prob, self.prob_dest_major, stream=stream)

    def combine(self, b: DeviceBatch, stream=None) -> None:
        partial = self.recv.recv_x if b.partials is None else b.partials
        B.ep_combine(partial, self.layout_buf.token_slot, out=self.out,
                     error_flag=self.error_flag, stream=stream)

    def preprocess(self, b: DeviceBatch, stream=None) -> None:
        """layout() and restripe() in one call: the restripe's blocks run in the layout's
        first launch (ep_dispatch_preprocess)."""
        self.layout_buf.compute_with_restripe(b.topk_idx, self.E, self.R, self.N, b.prob,
                                              self.prob_dest_major, stream=stream)

    def step(self, b: DeviceBatch, stream=None) -> None:
        """The whole path on one batch: where R allows it and the Path keeps no node slots,
        step_small() for a batch of at most EP_LAYOUT_DISPATCH_MAX_TOKENS tokens and
        step_counts() for a larger one; else step_preprocess()."""
        if self.counts_path and 0 < self.T <= B.EP_LAYOUT_DISPATCH_MAX_TOKENS:
            self.step_small(b, stream)
        elif self.counts_path:
            self.step_counts(b, stream)
        else:
            self.step_preprocess(b, stream)

    def step_small(self, b: DeviceBatch, stream=None) -> None:
        """The same outputs as step_counts() in two launches: ep_layout_dispatch (layout,
        dispatch and restripe), ep_combine. Needs T <= EP_LAYOUT_DISPATCH_MAX_TOKENS and
        R <= EP_COUNTS_MAX_RANKS."""
        self.layout_dispatch(b, stream)
        self.combine(b, stream)

    def layout_dispatch(self, b: DeviceBatch, stream=None) -> None:
        """Layout, dispatch and restripe of a batch of at most EP_LAYOUT_DISPATCH_MAX_TOKENS
        tokens in one launch."""
        lb, r = self.layout_buf, self.recv
        B.ep_layout_dispatch(b.x, b.topk_idx, b.topk_weights, self.E, self.R, self.N,
                             token_slot=lb.token_slot, recv_x=r.recv_x,
                             num_tokens_per_rank=lb.num_tokens_per_rank,
                             rank_offset=lb.rank_offset, error_flag=self.error_flag,
                             is_token_in_rank=lb.is_token_in_rank,
                             num_tokens_per_node=lb.num_tokens_per_node,
                             num_tokens_per_expert=lb.num_tokens_per_expert,
                             expert_offset=lb.expert_offset, recv_topk_idx=r.recv_topk_idx,
                             recv_topk_weights=r.recv_topk_weights,
                             recv_src_idx=r.recv_src_idx, prob=b.prob,
                             prob_dest_major=self.prob_dest_major, stream=stream)

    def step_preprocess(self, b: DeviceBatch, stream=None) -> None:
        """Layout and restripe (one call), dispatch, combine."""
        self.preprocess(b, stream)
        self.dispatch(b, stream)
        self.combine(b, stream)

    def _counts_workspace(self) -> torch.Tensor:
        if self.counts_ws is None:
            if self.R > B.EP_COUNTS_MAX_RANKS:
                raise ValueError(f"the counts path needs num_ranks <= {B.EP_COUNTS_MAX_RANKS}")
            n = B.ep_layout_counts_workspace_bytes(self.T, self.E, self.R, self.N)
            # zero-filled once: every call leaves the ticket at the start zero again
            self.counts_ws = torch.zeros(max(16, n), dtype=torch.uint8, device=self.out.device)
        return self.counts_ws

    def step_counts(self, b: DeviceBatch, stream=None) -> None:
        """The same outputs as step_preprocess() in one launch less: ep_layout_counts
        (counts, and the restripe in the same launch), ep_dispatch_layout (the dispatch
        computing every receive row itself, writing token_slot and the bitmap),
        ep_combine. Needs R <= EP_COUNTS_MAX_RANKS."""
        self.layout_counts(b, stream)
        self.dispatch_layout(b, stream)
        self.combine(b, stream)

    def layout_counts(self, b: DeviceBatch, stream=None) -> None:
        """The counts path's first call: the per-block tables in the workspace, and the
        restripe in the same launch."""
        B.ep_layout_counts(b.topk_idx, self.E, self.R, self.N, error_flag=self.error_flag,
                           workspace=self._counts_workspace(), prob=b.prob,
                           prob_dest_major=self.prob_dest_major, stream=stream)

    def dispatch_layout(self, b: DeviceBatch, stream=None) -> None:
        """The counts path's dispatch, after layout_counts() on the same batch."""
        ws, lb, r = self._counts_workspace(), self.layout_buf, self.recv
        B.ep_dispatch_layout(b.x, b.topk_idx, b.topk_weights, self.E, self.R, self.N,
                             token_slot=lb.token_slot, is_token_in_rank=lb.is_token_in_rank,
                             num_tokens_per_rank=lb.num_tokens_per_rank,
                             rank_offset=lb.rank_offset,
                             num_tokens_per_node=lb.num_tokens_per_node,
                             num_tokens_per_expert=lb.num_tokens_per_expert,
                             expert_offset=lb.expert_offset,
                             recv_x=r.recv_x, recv_topk_idx=r.recv_topk_idx,
                             recv_topk_weights=r.recv_topk_weights, recv_src_idx=r.recv_src_idx,
                             error_flag=self.error_flag, workspace=ws, stream=stream)

    def step_separate(self, b: DeviceBatch, stream=None) -> None:
        """The same outputs as step_preprocess(), one call per step of the path."""
        self.layout(b, stream)
        self.dispatch(b, stream)
        self.restripe(b, stream)
        self.combine(b, stream)

    # --- two-phase ("hook") dispatch and combine -----------------------------------------

    def _hook_buffers(self) -> StageBuffers:
        if self.stage is None:
            self.stage = StageBuffers.alloc(self.N, self.Tmax, self.H, self.k,
                                            self.out.device)
        if self.layout_buf.node_slot is None:
            raise ValueError("the two-phase calls need node slots: build the Path with "
                             "node_slots=True and run layout() first")
        return self.stage

    def dispatch_send(self, b: DeviceBatch, stream=None, num_workgroups: int = 0):
        """Enqueue the send phase; returns the receive hook, a callable(stream=None) that
        enqueues the receive phase (on a stream ordered after this one). num_workgroups > 0
        bounds the workgroups the send occupies (room for compute on another queue)."""
        st, lb = self._hook_buffers(), self.layout_buf
        B.ep_dispatch_send(b.x, b.topk_idx, b.topk_weights, lb.node_slot, stage_x=st.stage_x,
                           stage_topk_idx=st.stage_topk_idx,
                           stage_topk_weights=st.stage_topk_weights, stage_src=st.stage_src,
                           error_flag=self.error_flag, num_workgroups=num_workgroups,
                           stream=stream)

        self._dispatch_pending = True

        def recv_hook(stream=None) -> None:
            self._dispatch_pending = False
            r = self.recv
            B.ep_dispatch_recv(st.stage_x, st.stage_topk_idx, st.stage_topk_weights,
                               st.stage_src, lb.num_tokens_per_node, self.E, self.R,
                               lb.token_slot, recv_x=r.recv_x, recv_topk_idx=r.recv_topk_idx,
                               recv_topk_weights=r.recv_topk_weights,
                               recv_src_idx=r.recv_src_idx, error_flag=self.error_flag,
                               stream=stream)
        return recv_hook

    def combine_send(self, b: DeviceBatch, stream=None, num_workgroups: int = 0):
        """Enqueue the combine's send phase (per-node sums); returns its receive hook.
        The sums reuse the dispatch's staging rows, so a pending dispatch receive hook
        must have been enqueued first."""
        if self._dispatch_pending:
            raise RuntimeError("combine_send would overwrite the staged dispatch rows: run the "
                               "dispatch receive hook first")
        st, lb = self._hook_buffers(), self.layout_buf
        partial = self.recv.recv_x if b.partials is None else b.partials
        B.ep_combine_send(partial, lb.token_slot, lb.node_slot, stage=st.stage_x,
                          error_flag=self.error_flag, num_workgroups=num_workgroups,
                          stream=stream)

        def recv_hook(stream=None) -> None:
            B.ep_combine_recv(st.stage_x, lb.node_slot, out=self.out, error_flag=self.error_flag,
                              stream=stream)
        return recv_hook
