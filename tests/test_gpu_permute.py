"""GPU parity of the expert-major path, against the oracle, bit for bit, in two forms:
ep_get_layout's expert_slot output then ep_dispatch_permute; and the counts path,
ep_layout_counts with expert ranks then ep_dispatch_permute_layout (R <= 64, T <= 16384),
whose rows are formed inside the permute's waves."""
import numpy as np
import pytest
import torch

import oracle
import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.buffers import LayoutBuffers

from gpu_util import host

pytestmark = pytest.mark.gpu


def run_permute(x_bits, idx, w, E, R, N):
    T, H = x_bits.shape
    k = idx.shape[1]
    cap = T * k
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    tidx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    tw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    lb = LayoutBuffers.alloc(T, E, R, N, k_expert_slots=k)
    lb.expert_slot.fill_(-77)
    lb.compute(tidx, E, R, N)
    px = torch.full((cap, H), 0x7FC3, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pw = torch.full((cap,), -5.0, dtype=torch.float32, device="cuda")
    ps = torch.full((cap,), -5, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_permute(x, tw, lb.expert_slot, perm_x=px, perm_weights=pw, perm_src_idx=ps,
                           error_flag=lb.error_flag)
    torch.cuda.synchronize()
    return lb, dict(perm_x=host(px), perm_w=host(pw), perm_src=host(ps))


def run_permute_counts(x_bits, idx, w, E, R, N, cap=None):
    """The counts path: ep_layout_counts (with expert ranks), ep_dispatch_permute_layout."""
    T, H = x_bits.shape
    k = idx.shape[1]
    cap = T * k if cap is None else cap
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()
    tidx = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    tw = torch.from_numpy(np.ascontiguousarray(w)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    ws = torch.zeros(max(16, ep.ep_layout_counts_workspace_bytes(T, E, R, N)), dtype=torch.uint8,
                     device="cuda")
    er = torch.full((T, k), -77, **i32)
    es = torch.full((T, k), -77, **i32)
    ce, eo, flag = torch.full((E,), -5, **i32), torch.full((E + 1,), -5, **i32), torch.full((1,), -5, **i32)
    px = torch.full((cap, H), 0x7FC3, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    pw = torch.full((cap,), -5.0, dtype=torch.float32, device="cuda")
    ps = torch.full((cap,), -5, **i32)
    ep.ep_layout_counts(tidx, E, R, N, error_flag=flag, workspace=ws, expert_rank=er)
    ep.ep_dispatch_permute_layout(x, tidx, tw, E, R, N, expert_rank=er, perm_x=px, workspace=ws,
                                  perm_weights=pw, perm_src_idx=ps, expert_slot=es,
                                  num_tokens_per_expert=ce, expert_offset=eo, error_flag=flag)
    torch.cuda.synchronize()
    return (dict(expert_slot=host(es), expert_offset=host(eo), count_e=host(ce), flag=host(flag)),
            dict(perm_x=host(px), perm_w=host(pw), perm_src=host(ps)))


def check(x_bits, idx, w, E, R, N, flag=0, form="layout"):
    lay = oracle.layout(idx, E, R, N)
    es = oracle.expert_slots(idx, E)
    if form == "layout":
        lb, got = run_permute(x_bits, idx, w, E, R, N)
        np.testing.assert_array_equal(host(lb.expert_slot), es)
        np.testing.assert_array_equal(host(lb.token_slot), lay["token_slot"])
        np.testing.assert_array_equal(host(lb.expert_offset), lay["expert_offset"])
        np.testing.assert_array_equal(host(lb.num_tokens_per_expert), lay["count_e"])
        assert int(host(lb.error_flag)[0]) == flag
    else:
        out, got = run_permute_counts(x_bits, idx, w, E, R, N)
        np.testing.assert_array_equal(out["expert_slot"], es)
        np.testing.assert_array_equal(out["expert_offset"], lay["expert_offset"])
        np.testing.assert_array_equal(out["count_e"], lay["count_e"])
        assert int(out["flag"][0]) == flag
    T, k = idx.shape
    ref = oracle.dispatch_permute(x_bits, idx, w, es, T * k)
    n = int((es >= 0).sum())
    np.testing.assert_array_equal(got["perm_x"][:n], ref["perm_x"][:n])
    np.testing.assert_array_equal(got["perm_w"][:n].view(np.uint32), ref["perm_w"][:n].view(np.uint32))
    np.testing.assert_array_equal(got["perm_src"][:n], ref["perm_src"][:n])
    assert np.all(got["perm_src"][n:] == -5)


FORMS = ["layout", "counts"]


def counts_form_applies(T, R):
    return R <= ep.EP_COUNTS_MAX_RANKS and T <= 16384


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("name", ["tiny", "restripe", "dsv3", "skewed", "large"])
def test_permute_configs(name, form):
    cfg = W.CONFIGS[name]
    if form == "counts" and not counts_form_applies(cfg.T, cfg.R):
        pytest.skip("the counts path's permute takes R <= 64 and T <= 16384")
    print(f"\ncase: permute ({form}) {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    check(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, cfg.N, form=form)


@pytest.mark.parametrize("T,H,E,k,R,N", [
    (1, 64, 16, 4, 4, 2),          # one token
    (300, 16, 1, 1, 1, 1),         # a single expert (no id bits)
    (513, 8, 8192, 8, 64, 8),      # 13 id bits
    (20000, 8, 64, 4, 8, 2),       # three-launch layout
    (8192, 8, 512, 8, 256, 8),     # three-launch layout, wide rank table
    (700, 24, 96, 16, 8, 2),       # largest k for expert slots
    (300, 8192, 64, 4, 8, 2),      # a row wider than one pass of 14 words per lane
    (16384, 8, 256, 8, 64, 8),     # 64 blocks: one per lane in the counts path's permute
    (4097, 3584, 256, 8, 32, 4),   # 7 words per lane, a ragged last block
])
@pytest.mark.parametrize("form", FORMS)
def test_permute_shapes(T, H, E, k, R, N, form):
    if form == "counts" and not counts_form_applies(T, R):
        pytest.skip("the counts path's permute takes R <= 64 and T <= 16384")
    print(f"\ncase: permute ({form}) T={T} H={H} E={E} k={k} R={R} N={N}", flush=True)
    cfg = W.Config("p", T=T, H=H, E=E, k=k, R=R, N=N, P=4, Tmax=T)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    check(inp.x, inp.topk_idx, inp.topk_weights, E, R, N, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_permute_duplicates_masked_and_bad_ids(form):
    print(f"\ncase: permute ({form}) duplicates / masked / bad", flush=True)
    rng = np.random.default_rng(3)
    T, H, E, k, R, N = 900, 16, 32, 6, 4, 2
    idx = rng.integers(-1, E, size=(T, k)).astype(np.int64)   # duplicates and masked slots
    idx[rng.random((T, k)) < 0.02] = E + 3                     # out of range
    idx[10] = 5                                                # every slot the same expert
    w = rng.random((T, k)).astype(np.float32)
    x = W.hidden_rows(rng, T, H)
    check(x, idx, w, E, R, N, flag=ep.EP_DEVERR_TOPK_RANGE, form=form)


def test_permute_counts_short_capacity():
    """Rows past perm_capacity are skipped and set EP_DEVERR_RECV_OVERFLOW; expert_slot
    still holds every pair's row."""
    cfg = W.Config("p_short", T=1000, H=16, E=64, k=4, R=8, N=2, P=4, Tmax=1000)
    print(f"\ncase: permute (counts) short capacity {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    es = oracle.expert_slots(inp.topk_idx, cfg.E)
    cap = int((es >= 0).sum()) - 50
    out, got = run_permute_counts(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, cfg.N,
                                  cap=cap)
    assert int(out["flag"][0]) == ep.EP_DEVERR_RECV_OVERFLOW
    np.testing.assert_array_equal(out["expert_slot"], es)
    ref = oracle.dispatch_permute(inp.x, inp.topk_idx, inp.topk_weights, es, int((es >= 0).sum()))
    np.testing.assert_array_equal(got["perm_x"][:cap], ref["perm_x"][:cap])
    np.testing.assert_array_equal(got["perm_src"][:cap], ref["perm_src"][:cap])


def test_permute_rejects_wide_topk():
    idx = torch.zeros((4, 17), dtype=torch.int64, device="cuda")
    lb = LayoutBuffers.alloc(4, 32, 4, 2, k_expert_slots=17)
    with pytest.raises(ep.EPError) as e:
        lb.compute(idx, 32, 4, 2)
    assert e.value.status == ep.EP_ERR_ARG
