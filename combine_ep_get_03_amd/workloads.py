"""Seeded synthetic workloads for the MoE expert-parallel dispatch/combine path.

This module draws inputs only: routing, gate weights, hidden rows, per-rank
partial outputs and the prob tensor. It holds none of the arithmetic of the
path itself (no counts, offsets, slots, copies or sums), so the HIP path and
the CPU oracle can both be fed from it without sharing any of the method.

The shapes follow the pages' own benchmark workload: 4096 tokens per rank,
hidden 7168, top-8 experts ("[PR #347] Feature/sm free normal kernel",
section 3.1 "Experiment Setup"), a 256-expert DeepSeek-V3-style router, and a
prob tensor of [tokens][nodes][prob_per_token] fp32 with prob_per_token equal
to the experts held by one node ("[PR #634] Hybrid ep nixl restripe", section
"Baseline problem": 16 experts x 8 ranks gives 128 floats).

Every config draws from one ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed order: routing, gate logits, hidden rows, partials, prob.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    T tokens, hidden H (bf16), E experts, top-k, R simulated ranks (expert e
    lives on rank e // (E // R)), N nodes (rank r lives on node r // (R // N)),
    P prob floats per (token, node), Tmax rows per node in the restriped prob.
    ``routing`` is "uniform" (k distinct experts uniformly) or "zipf" (k
    distinct experts drawn without replacement with weight i**-zipf_s over a
    seeded expert permutation). ``partials`` is "random" (bf16 N(0,1) rows,
    one per receive slot) or "roundtrip" (the dispatched rows themselves are
    the expert outputs).
    """

    name: str
    T: int
    H: int
    E: int
    k: int
    R: int
    N: int
    P: int
    Tmax: int
    chunk: int = 256
    routing: str = "uniform"
    zipf_s: float = 1.2
    partials: str = "random"
    seed: int = 0

    @property
    def cap(self) -> int:
        """Receive rows that can never overflow: every token on min(k, R) ranks."""
        return self.T * min(self.k, self.R)

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads. P defaults to the experts held by one node (E // N).
CONFIGS = {
    "tiny": Config("tiny", T=256, H=1024, E=16, k=4, R=4, N=2, P=8, Tmax=256),
    # Restripe/prob workload: [4096][8][128] fp32 -> [8][4096][128]; the
    # dispatch side of it is run with R = N = 8 ranks of 16 experts.
    "restripe": Config("restripe", T=4096, H=4096, E=128, k=8, R=8, N=8, P=128,
                       Tmax=4096, chunk=256),
    "dsv3": Config("dsv3", T=4096, H=7168, E=256, k=8, R=32, N=4, P=64, Tmax=4096),
    "skewed": Config("skewed", T=4096, H=7168, E=256, k=8, R=32, N=4, P=64, Tmax=4096,
                     routing="zipf"),
    "large": Config("large", T=16384, H=7168, E=256, k=8, R=64, N=8, P=32, Tmax=16384,
                    partials="roundtrip"),
}


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns through torch's own conversion (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def routing_uniform(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """k distinct experts per token, uniformly: the first k of a random permutation."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int64)


def routing_zipf(rng: np.random.Generator, T: int, E: int, k: int, s: float) -> np.ndarray:
    """k distinct experts drawn in turn without replacement, P(expert) ~ rank**-s.

    Zipf rank i = 1..E is mapped to an expert id through a seeded permutation.
    Sequential sampling without replacement with weights w equals taking the k
    largest of log(w) + Gumbel noise, in decreasing key order.
    """
    perm = rng.permutation(E)
    logw = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = rng.gumbel(size=(T, E))
    keys = logw[None, :] + g
    order = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return perm[order].astype(np.int64)


def gate_weights(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    """fp32 softmax of N(0,1) logits over the k chosen experts, in sampling order."""
    logits = rng.standard_normal((T, k)).astype(np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)


def hidden_rows(rng: np.random.Generator, rows: int, H: int, chunk_rows: int = 4096) -> np.ndarray:
    """bf16 N(0,1) rows as uint16 bit patterns, drawn in row chunks to bound memory."""
    out = np.empty((rows, H), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = _bf16_bits(rng.standard_normal((r1 - r0, H), dtype=np.float32))
    return out


def hidden_rows_indexed(rows: int, H: int, chunk_rows: int = 4096) -> np.ndarray:
    """bf16 rows that name themselves, cheap enough for batches of hundreds of thousands
    of tokens: channels 0, 1, 2 of row t hold bits 0-9, 10-19 and 20-29 of t in the low
    mantissa/exponent bits over the pattern 0x3C00, the other channels
    0x3C00 | ((t * 40503 + c * 9973) & 0x3FF). Every value is finite, in [2^-7, 2)."""
    if H < 3:
        raise ValueError("hidden_rows_indexed needs H >= 3")
    out = np.empty((rows, H), dtype=np.uint16)
    c = np.arange(H, dtype=np.uint32)[None, :]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        t = np.arange(r0, r1, dtype=np.uint32)[:, None]
        blk = ((t * np.uint32(40503) + c * np.uint32(9973)) & np.uint32(0x3FF)) | np.uint32(0x3C00)
        for j in range(3):
            blk[:, j] = ((t[:, 0] >> np.uint32(10 * j)) & np.uint32(0x3FF)) | np.uint32(0x3C00)
        out[r0:r1] = blk.astype(np.uint16)
    return out


@dataclasses.dataclass
class Inputs:
    cfg: Config
    topk_idx: np.ndarray        # int64 [T][k]
    topk_weights: np.ndarray    # float32 [T][k]
    x: np.ndarray               # uint16 (bf16 bits) [T][H]
    partials: Optional[np.ndarray]  # uint16 [cap][H], or None for the round trip
    prob: np.ndarray            # float32 [T][N][P]


def make_inputs(cfg: Config, with_x: bool = True, with_partials: bool = True,
                with_prob: bool = True) -> Inputs:
    """Draw one config's inputs. Skipped parts still consume nothing from the stream
    only when they come last, so callers that skip parts must skip a suffix."""
    rng = np.random.default_rng(cfg.seed)
    if cfg.routing == "uniform":
        idx = routing_uniform(rng, cfg.T, cfg.E, cfg.k)
    elif cfg.routing == "zipf":
        idx = routing_zipf(rng, cfg.T, cfg.E, cfg.k, cfg.zipf_s)
    else:
        raise ValueError(cfg.routing)
    w = gate_weights(rng, cfg.T, cfg.k)
    x = hidden_rows(rng, cfg.T, cfg.H) if with_x else None
    partials = None
    if with_x and with_partials and cfg.partials == "random":
        partials = hidden_rows(rng, cfg.cap, cfg.H)
    prob = None
    if with_prob:
        prob = rng.random((cfg.T, cfg.N, cfg.P), dtype=np.float32)
    return Inputs(cfg, idx, w, x, partials, prob)


def prob_bit_pattern(T: int, N: int, P: int) -> np.ndarray:
    """prob whose 32-bit words are the distinct integers 0..T*N*P-1 (copied as bits)."""
    return np.arange(T * N * P, dtype=np.uint32).reshape(T, N, P).view(np.float32)
