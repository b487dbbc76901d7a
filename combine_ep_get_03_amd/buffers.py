"""Device buffers for one batch, allocated with torch (memory plumbing only).

Receive buffers are sized by the bound M <= T * min(k, R), so no count has to be read
back to the host before dispatch.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _binding as B


@dataclasses.dataclass
class LayoutBuffers:
    num_tokens_per_rank: torch.Tensor    # int32 [R]
    num_tokens_per_node: torch.Tensor    # int32 [N]
    num_tokens_per_expert: torch.Tensor  # int32 [E]
    is_token_in_rank: torch.Tensor       # uint8 [T][R]
    rank_offset: torch.Tensor            # int32 [R+1]
    expert_offset: torch.Tensor          # int32 [E+1]
    token_slot: torch.Tensor             # int32 [T][R]
    error_flag: torch.Tensor             # int32 [1]
    workspace: torch.Tensor              # uint8 [ep_layout_workspace_bytes]
    expert_slot: Optional[torch.Tensor] = None  # int32 [T][k], when expert-major rows are wanted
    node_slot: Optional[torch.Tensor] = None    # int32 [T][N], for the sparse restripe

    @classmethod
    def alloc(cls, T: int, E: int, R: int, N: int, device="cuda",
              k_expert_slots: int = 0, node_slots: bool = False) -> "LayoutBuffers":
        """k_expert_slots > 0 also allocates expert_slot [T][k] (expert-major rows);
        node_slots also allocates node_slot [T][N] (sparse restripe)."""
        i32 = dict(dtype=torch.int32, device=device)
        ws = max(16, B.ep_layout_workspace_bytes(T, E, R, N))
        return cls(torch.empty(R, **i32), torch.empty(N, **i32), torch.empty(E, **i32),
                   torch.empty((T, R), dtype=torch.uint8, device=device),
                   torch.empty(R + 1, **i32), torch.empty(E + 1, **i32),
                   torch.empty((T, R), **i32), torch.zeros(1, **i32),
                   torch.empty(ws, dtype=torch.uint8, device=device),
                   torch.empty((T, k_expert_slots), **i32) if k_expert_slots else None,
                   torch.empty((T, N), **i32) if node_slots else None)

    def _outputs(self) -> dict:
        return dict(num_tokens_per_rank=self.num_tokens_per_rank,
                    num_tokens_per_node=self.num_tokens_per_node,
                    num_tokens_per_expert=self.num_tokens_per_expert,
                    is_token_in_rank=self.is_token_in_rank, rank_offset=self.rank_offset,
                    expert_offset=self.expert_offset, token_slot=self.token_slot,
                    error_flag=self.error_flag, workspace=self.workspace,
                    expert_slot=self.expert_slot, node_slot=self.node_slot)

    def compute_with_restripe(self, topk_idx: torch.Tensor, E: int, R: int, N: int,
                              prob: torch.Tensor, prob_dest_major: torch.Tensor,
                              stream=None) -> None:
        """The layout and the dense restripe of prob in one call (ep_dispatch_preprocess)."""
        B.ep_dispatch_preprocess(topk_idx, E, R, N, prob, prob_dest_major, stream=stream,
                                 **self._outputs())

    def compute(self, topk_idx: torch.Tensor, E: int, R: int, N: int, stream=None) -> None:
        B.ep_get_layout(topk_idx, E, R, N, num_tokens_per_rank=self.num_tokens_per_rank,
                        num_tokens_per_node=self.num_tokens_per_node,
                        num_tokens_per_expert=self.num_tokens_per_expert,
                        is_token_in_rank=self.is_token_in_rank, rank_offset=self.rank_offset,
                        expert_offset=self.expert_offset, token_slot=self.token_slot,
                        error_flag=self.error_flag, workspace=self.workspace,
                        expert_slot=self.expert_slot, node_slot=self.node_slot, stream=stream)


@dataclasses.dataclass
class DispatchBuffers:
    recv_x: torch.Tensor              # bf16 [cap][H]
    recv_topk_idx: torch.Tensor       # int64 [cap][k]
    recv_topk_weights: torch.Tensor   # fp32 [cap][k]
    recv_src_idx: torch.Tensor        # int32 [cap]

    @classmethod
    def alloc(cls, cap: int, H: int, k: int, device="cuda") -> "DispatchBuffers":
        return cls(torch.empty((cap, H), dtype=torch.bfloat16, device=device),
                   torch.empty((cap, k), dtype=torch.int64, device=device),
                   torch.empty((cap, k), dtype=torch.float32, device=device),
                   torch.empty(cap, dtype=torch.int32, device=device))


@dataclasses.dataclass
class StageBuffers:
    """Per-node staging of the two-phase dispatch/combine: Tmax rows per node, the whole
    batch (staged row (n, s) is row n * Tmax + s). The combine's send phase writes its
    per-node sums into stage_x, so the dispatch's receive phase must run before it."""
    stage_x: torch.Tensor             # bf16 [N][Tmax][H]: dispatch rows, then combine sums
    stage_topk_idx: torch.Tensor      # int64 [N][Tmax][k]
    stage_topk_weights: torch.Tensor  # fp32 [N][Tmax][k]
    stage_src: torch.Tensor           # int32 [N][Tmax]

    @classmethod
    def alloc(cls, N: int, Tmax: int, H: int, k: int, device="cuda") -> "StageBuffers":
        return cls(torch.empty((N, Tmax, H), dtype=torch.bfloat16, device=device),
                   torch.empty((N, Tmax, k), dtype=torch.int64, device=device),
                   torch.empty((N, Tmax, k), dtype=torch.float32, device=device),
                   torch.empty((N, Tmax), dtype=torch.int32, device=device))
