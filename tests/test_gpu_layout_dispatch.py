"""GPU parity of ep_layout_dispatch, the layout, the dispatch and the restripe of a batch of
at most 256 tokens in one launch: every output bit for bit equal to the oracle's layout,
dispatch and restripe, on shapes across the limits (one token, a ragged wave, a full
group, R = 1 and 64, k above R, k = E, a top-k past one batch of ids, rows wider than one
pass), with masked and out-of-range ids, a short receive buffer, calls in a row whose
sizes change, graph replays, and the empty batch. Rows past M and the restriped prob's
rows past T keep their sentinels."""
import numpy as np
import pytest
import torch

import combine_ep_get_03_amd as ep
import oracle
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

from gpu_util import host

pytestmark = pytest.mark.gpu

SHAPES = [
    W.Config("ld_dsv3_256", T=256, H=7168, E=256, k=8, R=32, N=4, P=64, Tmax=256),
    W.Config("ld_one_token", T=1, H=64, E=16, k=4, R=4, N=2, P=8, Tmax=1),
    W.Config("ld_ragged_65", T=65, H=72, E=64, k=6, R=64, N=8, P=5, Tmax=70),
    W.Config("ld_single_rank", T=200, H=128, E=8, k=2, R=1, N=1, P=8, Tmax=200),
    W.Config("ld_k_over_r", T=256, H=40, E=16, k=8, R=4, N=2, P=4, Tmax=256),
    W.Config("ld_all_experts", T=100, H=32, E=8, k=8, R=8, N=2, P=4, Tmax=128),
    W.Config("ld_wide_rows", T=130, H=7168 * 2 + 8, E=64, k=4, R=16, N=4, P=16, Tmax=130),
    W.Config("ld_top20", T=64, H=24, E=64, k=20, R=16, N=4, P=4, Tmax=64),
    W.Config("ld_skewed", T=256, H=256, E=256, k=8, R=32, N=4, P=64, Tmax=256, routing="zipf"),
]


def _call(cfg, inp, cap=None, prob_out=None, flag_init=-5, stream=None):
    """ep_layout_dispatch through the binding on fresh sentinel-filled outputs; returns them
    as host arrays."""
    T, k, E, R, N = cfg.T, cfg.k, cfg.E, cfg.R, cfg.N
    i32 = dict(dtype=torch.int32, device="cuda")
    o = dict(count_r=torch.full((R,), -5, **i32), count_n=torch.full((N,), -5, **i32),
             count_e=torch.full((E,), -5, **i32), rank_offset=torch.full((R + 1,), -5, **i32),
             expert_offset=torch.full((E + 1,), -5, **i32),
             flag=torch.full((1,), flag_init, **i32),
             token_slot=torch.full((T, R), -99, **i32),
             in_rank=torch.full((T, R), 0xCD, dtype=torch.uint8, device="cuda"))
    cap = T * min(k, R) if cap is None else cap
    rx = torch.full((cap, cfg.H), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ri = torch.full((cap, k), -77, dtype=torch.int64, device="cuda")
    rw = torch.full((cap, k), -7.0, dtype=torch.float32, device="cuda")
    rs = torch.full((cap,), -7, **i32)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, None)
    ep.ep_layout_dispatch(b.x, b.topk_idx, b.topk_weights, E, R, N, token_slot=o["token_slot"],
                          recv_x=rx, num_tokens_per_rank=o["count_r"],
                          rank_offset=o["rank_offset"], error_flag=o["flag"],
                          is_token_in_rank=o["in_rank"], num_tokens_per_node=o["count_n"],
                          num_tokens_per_expert=o["count_e"], expert_offset=o["expert_offset"],
                          recv_topk_idx=ri, recv_topk_weights=rw, recv_src_idx=rs,
                          prob=b.prob if prob_out is not None else None,
                          prob_dest_major=prob_out, stream=stream)
    torch.cuda.synchronize()
    out = {n: host(t) for n, t in o.items()}
    out.update(recv_x=host(rx), recv_idx=host(ri), recv_w=host(rw), recv_src=host(rs))
    return out


def _check(cfg, inp, got, flag=0, cap=None):
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    full = cfg.T * min(cfg.k, cfg.R)
    cap = full if cap is None else cap
    d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"],
                        full)
    assert int(got["flag"][0]) == flag
    for name in ("count_r", "count_n", "count_e", "rank_offset", "expert_offset", "token_slot",
                 "in_rank"):
        np.testing.assert_array_equal(got[name], lay[name], err_msg=f"{cfg.name}: {name}")
    n = min(M, cap)
    np.testing.assert_array_equal(got["recv_x"][:n], d["recv_x"][:n])
    assert np.all(got["recv_x"][n:] == 7)
    np.testing.assert_array_equal(got["recv_idx"][:n], d["recv_idx"][:n])
    np.testing.assert_array_equal(got["recv_w"][:n].view(np.uint32),
                                  d["recv_w"][:n].view(np.uint32))
    np.testing.assert_array_equal(got["recv_src"][:n], d["recv_src"][:n])
    assert np.all(got["recv_src"][n:] == -7)


def _restripe_ref(cfg, inp):
    return oracle.restripe_prob(inp.prob, cfg.Tmax,
                                out=np.full((cfg.N, cfg.Tmax, cfg.P), -3.0, np.float32))


@pytest.mark.parametrize("cfg", SHAPES, ids=lambda c: c.name)
def test_layout_dispatch_matches_the_oracle(cfg):
    print(f"\ncase: ep_layout_dispatch {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    prob_out = torch.full((cfg.N, cfg.Tmax, cfg.P), -3.0, dtype=torch.float32, device="cuda")
    got = _call(cfg, inp, prob_out=prob_out)
    _check(cfg, inp, got)
    np.testing.assert_array_equal(host(prob_out).view(np.uint32),
                                  _restripe_ref(cfg, inp).view(np.uint32))


def test_layout_dispatch_equals_the_counts_path():
    # the same batch through ep_layout_counts + ep_dispatch_layout and through the one call
    cfg = W.Config("ld_vs_counts", T=256, H=512, E=256, k=8, R=32, N=4, P=16, Tmax=256)
    print(f"\ncase: ep_layout_dispatch against the counts path {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, None)
    a = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    c = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    a.layout_counts(b)
    a.dispatch_layout(b)
    c.layout_dispatch(b)
    torch.cuda.synchronize()
    M = int(a.layout_buf.rank_offset[-1].item())
    for name in ("token_slot", "is_token_in_rank", "num_tokens_per_rank", "rank_offset",
                 "num_tokens_per_node", "num_tokens_per_expert", "expert_offset"):
        assert torch.equal(getattr(a.layout_buf, name), getattr(c.layout_buf, name)), name
    for name in ("recv_x", "recv_topk_idx", "recv_topk_weights", "recv_src_idx"):
        assert torch.equal(getattr(a.recv, name)[:M], getattr(c.recv, name)[:M]), name
    assert torch.equal(a.prob_dest_major[:, :cfg.T], c.prob_dest_major[:, :cfg.T])
    assert int(c.error_flag.item()) == 0


def test_masked_and_bad_ids():
    cfg = W.Config("ld_bad_ids", T=230, H=32, E=64, k=4, R=8, N=2, P=16, Tmax=230)
    print(f"\ncase: ep_layout_dispatch {cfg} with masked and out-of-range ids", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    idx = inp.topk_idx.copy()
    m = np.random.default_rng(11).random(idx.shape)
    idx[m < 0.1] = -1
    idx[(m > 0.1) & (m < 0.12)] = 64
    idx[(m > 0.12) & (m < 0.13)] = -5
    idx[5] = -1
    inp.topk_idx = idx
    for init in (-5, 0):  # the flag is overwritten, whatever it held
        got = _call(cfg, inp, flag_init=init)
        _check(cfg, inp, got, flag=ep.EP_DEVERR_TOPK_RANGE)
        assert np.all(got["token_slot"][5] == -1)
    # a clean batch afterwards clears it
    clean = W.make_inputs(cfg, with_partials=False)
    _check(cfg, clean, _call(cfg, clean, flag_init=ep.EP_DEVERR_TOPK_RANGE))


def test_short_receive_buffer_sets_the_overflow_bit():
    cfg = W.Config("ld_short", T=256, H=64, E=64, k=6, R=16, N=4, P=8, Tmax=256)
    print(f"\ncase: ep_layout_dispatch {cfg}, receive capacity M - 10", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    M = int(oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)["rank_offset"][-1])
    got = _call(cfg, inp, cap=M - 10)
    _check(cfg, inp, got, flag=ep.EP_DEVERR_RECV_OVERFLOW, cap=M - 10)


def test_calls_in_a_row_and_the_empty_batch():
    seq = [SHAPES[0], SHAPES[2], W.Config("ld_empty", T=0, H=64, E=16, k=4, R=4, N=2, P=8,
                                           Tmax=0), SHAPES[4], SHAPES[1]]
    for cfg in seq:
        print(f"\ncase: ep_layout_dispatch in a row {cfg}", flush=True)
        inp = W.make_inputs(cfg, with_partials=False)
        if cfg.T == 0:
            i32 = dict(dtype=torch.int32, device="cuda")
            z = {n: torch.full((m,), -5, **i32) for n, m in
                 (("cr", cfg.R), ("ro", cfg.R + 1), ("cn", cfg.N), ("ce", cfg.E),
                  ("eo", cfg.E + 1), ("flag", 1))}
            x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
            idx = torch.empty((0, cfg.k), dtype=torch.int64, device="cuda")
            w = torch.empty((0, cfg.k), dtype=torch.float32, device="cuda")
            ep.ep_layout_dispatch(x, idx, w, cfg.E, cfg.R, cfg.N,
                                  token_slot=torch.empty((0, cfg.R), **i32),
                                  recv_x=torch.empty((0, cfg.H), dtype=torch.bfloat16,
                                                     device="cuda"),
                                  num_tokens_per_rank=z["cr"], rank_offset=z["ro"],
                                  num_tokens_per_node=z["cn"], num_tokens_per_expert=z["ce"],
                                  expert_offset=z["eo"], error_flag=z["flag"])
            torch.cuda.synchronize()
            for n, t in z.items():
                assert bool((t == 0).all()), n
            continue
        _check(cfg, inp, _call(cfg, inp))


def test_graph_replays_match_the_eager_call():
    cfg = SHAPES[0]
    print(f"\ncase: ep_layout_dispatch captured in a graph {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, None)
    p = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    p.layout_dispatch(b)
    torch.cuda.synchronize()
    M = int(p.layout_buf.rank_offset[-1].item())
    ref = (p.recv.recv_x[:M].clone(), p.layout_buf.token_slot.clone(), p.prob_dest_major.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        p.layout_dispatch(b)
    for _ in range(3):
        p.recv.recv_x.fill_(0)
        p.layout_buf.token_slot.fill_(-3)
        p.prob_dest_major.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.recv.recv_x[:M], ref[0])
        assert torch.equal(p.layout_buf.token_slot, ref[1])
        assert torch.equal(p.prob_dest_major, ref[2])
        assert int(p.error_flag.item()) == 0


def _random_shapes(n=16, seed=4711):
    """Seeded topologies up to 256 tokens and 64 ranks: ranks off powers of two, odd top-k,
    ragged T, hidden sizes of one and several passes, uniform or Zipf routing."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.choice([1, 2, 3, 4, 8]))
        rpn = int(rng.choice([1, 2, 3, 5, 8]))
        R = N * rpn
        er = int(rng.choice([1, 2, 3, 4, 8]))
        E = R * er
        k = int(rng.integers(1, min(E, 12) + 1))
        T = int(rng.integers(1, 257))
        H = int(rng.choice([8, 64, 200, 1024, 7168, 9000]))
        P = int(rng.integers(1, 40))
        routing = "zipf" if rng.random() < 0.3 else "uniform"
        out.append(W.Config(f"ldr{i}_T{T}_H{H}_E{E}_k{k}_R{R}_N{N}", T=T, H=H, E=E, k=k, R=R,
                            N=N, P=P, Tmax=T + int(rng.integers(0, 20)), routing=routing,
                            seed=2000 + i))
    return out


@pytest.mark.parametrize("cfg", _random_shapes(), ids=lambda c: c.name)
def test_random_shapes(cfg):
    print(f"\ncase: ep_layout_dispatch random shape {cfg}", flush=True)
    inp = W.make_inputs(cfg, with_partials=False)
    prob_out = torch.full((cfg.N, cfg.Tmax, cfg.P), -3.0, dtype=torch.float32, device="cuda")
    got = _call(cfg, inp, prob_out=prob_out)
    _check(cfg, inp, got)
    np.testing.assert_array_equal(host(prob_out).view(np.uint32),
                                  _restripe_ref(cfg, inp).view(np.uint32))
