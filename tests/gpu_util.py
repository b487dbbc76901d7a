"""Helpers for the GPU parity tests: run the HIP path through the C ABI on seeded inputs
and compare every output with the CPU oracle on the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

SENT_U16 = 0x7FC3      # a NaN pattern no bf16 row of the inputs holds
SENT_U32 = 0xDEADBEEF
SENT_I64 = -0x123456789


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return host_u16(t)
    return t.detach().cpu().numpy()


def fill_sentinels(path: Path) -> None:
    path.recv.recv_x.view(torch.int16).fill_(np.int16(np.uint16(SENT_U16).view(np.int16)))
    path.recv.recv_topk_idx.fill_(SENT_I64)
    path.recv.recv_topk_weights.view(torch.int32).fill_(int(np.uint32(SENT_U32).view(np.int32)))
    path.recv.recv_src_idx.fill_(-7)
    path.prob_dest_major.view(torch.int32).fill_(int(np.uint32(SENT_U32).view(np.int32)))
    path.out.view(torch.int16).fill_(np.int16(np.uint16(SENT_U16).view(np.int16)))
    path.layout_buf.token_slot.fill_(-99)
    path.layout_buf.is_token_in_rank.fill_(0xCD)
    for t in (path.layout_buf.num_tokens_per_rank, path.layout_buf.num_tokens_per_node,
              path.layout_buf.num_tokens_per_expert, path.layout_buf.rank_offset,
              path.layout_buf.expert_offset):
        t.fill_(-55)
    path.layout_buf.error_flag.fill_(-1)


def oracle_all(cfg: W.Config, inp: W.Inputs, partial_rows=None) -> dict:
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"],
                        cfg.cap)
    rs_out = np.full((cfg.N, cfg.Tmax, cfg.P), SENT_U32, np.uint32).view(np.float32)
    rs = oracle.restripe_prob(inp.prob, cfg.Tmax, out=rs_out)
    partial = d["recv_x"] if inp.partials is None else inp.partials
    cb = oracle.combine(partial, lay["token_slot"], cfg.R)
    return dict(lay=lay, d=d, rs=rs, cb=cb, M=int(lay["rank_offset"][-1]))


STEP_FORMS = {"separate": "one call per step", "preprocess": "layout+restripe in one call",
              "counts": "counts path (two launches for layout and dispatch)",
              "small": "layout, dispatch and restripe in one launch (T <= 256)",
              "step": "Path.step (the counts path where R allows it)"}


def run_gpu(cfg: W.Config, inp: W.Inputs, device="cuda", fused: bool = True,
            form: str = None) -> Path:
    """One step of the path: form "step" (Path.step; the default), "preprocess" (layout and
    restripe in one call, ep_dispatch_preprocess), "separate" (one call per step), "counts"
    (ep_layout_counts + ep_dispatch_layout) or "small" (ep_layout_dispatch)."""
    form = form or ("step" if fused else "separate")
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials,
                              device=device)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax, device=device)
    fill_sentinels(path)
    {"step": path.step, "preprocess": path.step_preprocess, "separate": path.step_separate,
     "counts": path.step_counts, "small": path.step_small}[form](b)
    torch.cuda.synchronize()
    return path


def run_and_compare_both(cfg: W.Config, inp: W.Inputs, ref: dict, expect_flag: int = 0) -> Path:
    """The step in every form (the counts path where R allows it, and the one-launch layout
    and dispatch where T does too): each must match the oracle. Returns the last path."""
    forms = ["separate", "preprocess"] + (["counts"] if cfg.R <= 64 else [])
    forms += ["small"] if cfg.R <= 64 and 0 < cfg.T <= 256 else []
    for form in forms:
        print(f"  {STEP_FORMS[form]}", flush=True)
        path = run_gpu(cfg, inp, form=form)
        compare_all(cfg, path, ref, expect_flag=expect_flag)
    return path


def combine_tolerance_ok(got: np.ndarray, ref: np.ndarray) -> bool:
    """|gpu - oracle| <= 2^-7 * max(1, |oracle|), both widened from bf16 to fp32."""
    g = oracle.bf16_to_f32(got).astype(np.float64)
    r = oracle.bf16_to_f32(ref).astype(np.float64)
    return bool(np.all(np.abs(g - r) <= 2.0**-7 * np.maximum(1.0, np.abs(r))))


def compare_all(cfg: W.Config, path: Path, ref: dict, expect_flag: int = 0) -> None:
    lay, d, M = ref["lay"], ref["d"], ref["M"]
    L = path.layout_buf
    assert int(host(L.error_flag)[0]) == expect_flag
    np.testing.assert_array_equal(host(L.num_tokens_per_rank), lay["count_r"])
    np.testing.assert_array_equal(host(L.num_tokens_per_node), lay["count_n"])
    np.testing.assert_array_equal(host(L.num_tokens_per_expert), lay["count_e"])
    np.testing.assert_array_equal(host(L.is_token_in_rank), lay["in_rank"])
    np.testing.assert_array_equal(host(L.rank_offset), lay["rank_offset"])
    np.testing.assert_array_equal(host(L.expert_offset), lay["expert_offset"])
    np.testing.assert_array_equal(host(L.token_slot), lay["token_slot"])

    rx = host(path.recv.recv_x)
    np.testing.assert_array_equal(rx[:M], d["recv_x"][:M])
    assert np.all(rx[M:] == SENT_U16)
    ri = host(path.recv.recv_topk_idx)
    np.testing.assert_array_equal(ri[:M], d["recv_idx"][:M])
    assert np.all(ri[M:] == SENT_I64)
    rw = host(path.recv.recv_topk_weights).view(np.uint32)
    np.testing.assert_array_equal(rw[:M], d["recv_w"][:M].view(np.uint32))
    assert np.all(rw[M:] == SENT_U32)
    rsrc = host(path.recv.recv_src_idx)
    np.testing.assert_array_equal(rsrc[:M], d["recv_src"][:M])
    assert np.all(rsrc[M:] == -7)

    np.testing.assert_array_equal(host(path.prob_dest_major).view(np.uint32),
                                  ref["rs"].view(np.uint32))

    out = host(path.out)
    assert combine_tolerance_ok(out, ref["cb"])
    np.testing.assert_array_equal(out, ref["cb"])
