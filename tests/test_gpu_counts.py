"""GPU parity of the counts path (ep_layout_counts, then ep_dispatch_layout): the layout and
the dispatch in two launches, every output bit for bit equal to the oracle's layout,
restripe and dispatch. The parity tests of the whole path (test_gpu_parity.py) run it on
every configuration with R <= 64; these cover what is particular to it: the ticket that
each call leaves zero for the next (calls in a row on one workspace whose sizes change),
graph replays, the empty batch, a short receive buffer, and a batch whose dispatch is split
over token ranges."""
import numpy as np
import pytest
import torch

import combine_ep_get_03_amd as ep
import oracle
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

from gpu_util import SENT_U16, compare_all, fill_sentinels, host, oracle_all, run_gpu

pytestmark = pytest.mark.gpu


def _counts_call(cfg, inp, ws, prob_out=None):
    """Both calls of the counts path through the binding, on a given workspace; returns the
    outputs as host arrays."""
    dev = ws.device
    T, k, E, R, N = cfg.T, cfg.k, cfg.E, cfg.R, cfg.N
    i32 = dict(dtype=torch.int32, device=dev)
    o = dict(count_r=torch.full((R,), -5, **i32), count_n=torch.full((N,), -5, **i32),
             count_e=torch.full((E,), -5, **i32), rank_offset=torch.full((R + 1,), -5, **i32),
             expert_offset=torch.full((E + 1,), -5, **i32), flag=torch.full((1,), -5, **i32),
             token_slot=torch.full((T, R), -99, **i32),
             in_rank=torch.full((T, R), 0xCD, dtype=torch.uint8, device=dev))
    cap = T * min(k, R)
    rx = torch.full((cap, cfg.H), 7, dtype=torch.int16, device=dev).view(torch.bfloat16)
    ri = torch.full((cap, k), -77, dtype=torch.int64, device=dev)
    rw = torch.full((cap, k), -7.0, dtype=torch.float32, device=dev)
    rs = torch.full((cap,), -7, **i32)
    idx = torch.from_numpy(inp.topk_idx).to(dev)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, None, device=dev)
    ep.ep_layout_counts(idx, E, R, N, error_flag=o["flag"], workspace=ws,
                        prob=b.prob if prob_out is not None else None, prob_dest_major=prob_out)
    ep.ep_dispatch_layout(b.x, idx, b.topk_weights, E, R, N, token_slot=o["token_slot"],
                          is_token_in_rank=o["in_rank"], num_tokens_per_rank=o["count_r"],
                          rank_offset=o["rank_offset"], num_tokens_per_node=o["count_n"],
                          num_tokens_per_expert=o["count_e"], expert_offset=o["expert_offset"],
                          recv_x=rx, recv_topk_idx=ri,
                          recv_topk_weights=rw, recv_src_idx=rs, error_flag=o["flag"],
                          workspace=ws)
    torch.cuda.synchronize()
    out = {n: host(t) for n, t in o.items()}
    out.update(recv_x=host(rx), recv_idx=host(ri), recv_w=host(rw), recv_src=host(rs))
    return out


def _check(cfg, inp, got, flag=0):
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"],
                        cfg.T * min(cfg.k, cfg.R))
    assert int(got["flag"][0]) == flag
    for name, want in (("count_r", "count_r"), ("count_n", "count_n"), ("count_e", "count_e"),
                       ("rank_offset", "rank_offset"), ("expert_offset", "expert_offset"),
                       ("token_slot", "token_slot"), ("in_rank", "in_rank")):
        np.testing.assert_array_equal(got[name], lay[want], err_msg=f"{cfg.name}: {name}")
    np.testing.assert_array_equal(got["recv_x"][:M], d["recv_x"][:M])
    assert np.all(got["recv_x"][M:] == 7)
    np.testing.assert_array_equal(got["recv_idx"][:M], d["recv_idx"][:M])
    np.testing.assert_array_equal(got["recv_w"][:M].view(np.uint32), d["recv_w"][:M].view(np.uint32))
    np.testing.assert_array_equal(got["recv_src"][:M], d["recv_src"][:M])
    assert np.all(got["recv_src"][M:] == -7)


# calls in a row on one zero-filled workspace: sizes shrink and grow, E and R change, so
# the ticket must be left zero by every call
SEQUENCE = [
    W.Config("c_dsv3", T=4096, H=64, E=256, k=8, R=32, N=4, P=8, Tmax=4096),
    W.Config("c_small", T=300, H=72, E=16, k=4, R=4, N=2, P=8, Tmax=300),
    W.Config("c_one_block", T=256, H=8, E=64, k=6, R=64, N=8, P=8, Tmax=256),
    W.Config("c_many_blocks", T=20000, H=8, E=8192, k=8, R=64, N=8, P=4, Tmax=20000),
    W.Config("c_ragged", T=1001, H=24, E=96, k=5, R=8, N=2, P=5, Tmax=1100),
    W.Config("c_dsv3_again", T=4096, H=64, E=256, k=8, R=32, N=4, P=8, Tmax=4096,
             routing="zipf"),
    # the first size past 16 blocks, where the count launch takes the ticket again
    W.Config("c_17_blocks", T=4097, H=16, E=256, k=8, R=64, N=8, P=4, Tmax=4100),
    W.Config("c_16_blocks", T=4096, H=16, E=256, k=8, R=64, N=8, P=4, Tmax=4096),
]


def test_calls_in_a_row_on_one_workspace():
    need = max(ep.ep_layout_counts_workspace_bytes(c.T, c.E, c.R, c.N) for c in SEQUENCE)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for cfg in SEQUENCE:
        print(f"\ncase: counts path {cfg}", flush=True)
        inp = W.make_inputs(cfg, with_partials=False)
        prob_out = torch.full((cfg.N, cfg.Tmax, cfg.P), -3.0, dtype=torch.float32, device="cuda")
        got = _counts_call(cfg, inp, ws, prob_out)
        _check(cfg, inp, got)
        rs = oracle.restripe_prob(inp.prob, cfg.Tmax,
                                  out=np.full((cfg.N, cfg.Tmax, cfg.P), -3.0, np.float32))
        np.testing.assert_array_equal(host(prob_out).view(np.uint32), rs.view(np.uint32))
    # the ticket is zero again after the calls
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_masked_and_bad_ids():
    cfg = W.Config("c_bad_ids", T=900, H=32, E=64, k=4, R=8, N=2, P=16, Tmax=900)
    print(f"\ncase: counts path {cfg} with masked and out-of-range ids", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    idx = inp.topk_idx.copy()
    rng = np.random.default_rng(11)
    m = rng.random(idx.shape)
    idx[m < 0.1] = -1
    idx[(m > 0.1) & (m < 0.12)] = 64
    idx[(m > 0.12) & (m < 0.13)] = -5
    idx[5] = -1
    inp.topk_idx = idx
    ws = torch.zeros(ep.ep_layout_counts_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N),
                     dtype=torch.uint8, device="cuda")
    for _ in range(2):  # and again on the same workspace
        got = _counts_call(cfg, inp, ws)
        _check(cfg, inp, got, flag=ep.EP_DEVERR_TOPK_RANGE)
        assert np.all(got["token_slot"][5] == -1)


def test_short_receive_buffer_sets_the_overflow_bit():
    cfg = W.CONFIGS["tiny"]
    print(f"\ncase: counts path {cfg}, receive capacity M - 10", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    cap = M - 10
    ws = torch.zeros(ep.ep_layout_counts_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N),
                     dtype=torch.uint8, device="cuda")
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, None)
    i32 = dict(dtype=torch.int32, device="cuda")
    cr, ro, flag = torch.empty(cfg.R, **i32), torch.empty(cfg.R + 1, **i32), torch.empty(1, **i32)
    slot = torch.empty((cfg.T, cfg.R), **i32)
    rx = torch.full((cap, cfg.H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ep.ep_layout_counts(b.topk_idx, cfg.E, cfg.R, cfg.N, error_flag=flag, workspace=ws)
    ep.ep_dispatch_layout(b.x, b.topk_idx, b.topk_weights, cfg.E, cfg.R, cfg.N, token_slot=slot,
                          num_tokens_per_rank=cr, rank_offset=ro, recv_x=rx, error_flag=flag,
                          workspace=ws)
    torch.cuda.synchronize()
    assert int(flag.item()) == ep.EP_DEVERR_RECV_OVERFLOW
    d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], M)
    np.testing.assert_array_equal(host(rx), d["recv_x"][:cap])
    np.testing.assert_array_equal(host(slot), lay["token_slot"])


def test_empty_batch():
    cfg = W.Config("c_empty", T=0, H=64, E=16, k=4, R=4, N=2, P=8, Tmax=4)
    print(f"\ncase: counts path {cfg}", flush=True)
    path = Path(0, 64, 16, 4, 4, 2, 8, 4)
    for t in (path.layout_buf.num_tokens_per_rank, path.layout_buf.rank_offset,
              path.layout_buf.num_tokens_per_expert, path.layout_buf.expert_offset):
        t.fill_(5)
    inp = W.make_inputs(cfg)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path.step_counts(b)
    torch.cuda.synchronize()
    assert host(path.layout_buf.num_tokens_per_rank).tolist() == [0] * 4
    assert host(path.layout_buf.rank_offset).tolist() == [0] * 5
    assert host(path.layout_buf.num_tokens_per_expert).tolist() == [0] * 16
    assert host(path.layout_buf.expert_offset).tolist() == [0] * 17
    assert int(host(path.error_flag)[0]) == 0


@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_graph_replays(name):
    """The counts path captured in a HIP graph: every replay, with eager work and
    synchronisation in between, reproduces the oracle's outputs (the ticket and totals
    are reset inside each replay)."""
    cfg = W.CONFIGS[name]
    print(f"\ncase: counts path in a graph {cfg}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_all(cfg, inp)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    fill_sentinels(path)
    path.step_counts(b)
    torch.cuda.synchronize()
    compare_all(cfg, path, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path.step_counts(b)
    for _ in range(3):
        fill_sentinels(path)
        path.step_preprocess(b)  # eager work of the other form in between
        fill_sentinels(path)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_all(cfg, path, ref)


def test_dispatch_split_over_token_ranges():
    # 600 000 tokens with 8 waves each: the dispatch takes two launches, and the count
    # launch's last block scans 2344 block rows
    cfg = W.Config("c_split_600k", T=600_000, H=8, E=64, k=8, R=8, N=8, P=4, Tmax=600_000,
                   seed=11)
    print(f"\ncase: counts path {cfg}", flush=True)
    inp = W.make_inputs(cfg)
    ref = oracle_all(cfg, inp)
    path = run_gpu(cfg, inp, form="counts")
    compare_all(cfg, path, ref)


def test_workspace_with_a_nonzero_ticket_is_reported():
    """A workspace whose ticket is not zero on entry (never zero-filled, or shared by calls
    that overlap) sets EP_DEVERR_WORKSPACE in a batch large enough to use the ticket (more
    than 16 blocks of 256 tokens); the outputs of that call are unspecified, but every
    kernel ends and stays in bounds. Zeroing the ticket makes the next call exact."""
    cfg = W.Config("c_ticket", T=8192, H=64, E=256, k=8, R=32, N=4, P=8, Tmax=8192)
    print(f"\ncase: counts path {cfg} with the ticket set to 5", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    ws = torch.zeros(ep.ep_layout_counts_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N),
                     dtype=torch.uint8, device="cuda")
    ws[:4].view(torch.int32).fill_(5)
    got = _counts_call(cfg, inp, ws)
    assert int(got["flag"][0]) & ep.EP_DEVERR_WORKSPACE
    ws[:4].view(torch.int32).zero_()
    got = _counts_call(cfg, inp, ws)
    _check(cfg, inp, got)
