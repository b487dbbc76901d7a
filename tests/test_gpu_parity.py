"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs. Layout, dispatch and restripe must match bit for bit; combine must be within
2^-7 * max(1, |ref|) and, summing in the same order, is expected to match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from combine_ep_get_03_amd import workloads as W
import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

from gpu_util import (SENT_U32, compare_all, fill_sentinels, host, oracle_all,
                      run_and_compare_both, run_gpu)

pytestmark = pytest.mark.gpu


def _case(cfg, **kw):
    print(f"\ncase: {cfg} {kw}", flush=True)
    inp = W.make_inputs(cfg)
    return inp


@pytest.mark.parametrize("name", ["tiny", "restripe", "dsv3", "skewed", "large"])
def test_config_full_path(name):
    cfg = W.CONFIGS[name]
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    run_and_compare_both(cfg, inp, ref)


EDGE = [
    W.Config("one_token", T=1, H=64, E=16, k=4, R=4, N=2, P=8, Tmax=1),
    W.Config("ragged_257", T=257, H=24, E=12, k=3, R=3, N=3, P=5, Tmax=300),
    W.Config("ragged_1000", T=1000, H=8, E=64, k=8, R=16, N=4, P=16, Tmax=1024),
    W.Config("single_rank", T=300, H=128, E=8, k=2, R=1, N=1, P=8, Tmax=300),
    W.Config("rank_per_expert", T=500, H=64, E=32, k=6, R=32, N=8, P=4, Tmax=500),
    W.Config("all_experts", T=70, H=32, E=8, k=8, R=4, N=2, P=4, Tmax=70),
    W.Config("er_ne_r", T=600, H=40, E=96, k=5, R=8, N=2, P=48, Tmax=640),
    W.Config("r65_two_words", T=333, H=16, E=130, k=6, R=65, N=5, P=26, Tmax=333),
    W.Config("r100", T=513, H=16, E=200, k=10, R=100, N=4, P=52, Tmax=600),
    W.Config("r1024_max", T=700, H=8, E=2048, k=16, R=1024, N=8, P=256, Tmax=700),
    W.Config("e8192_max", T=400, H=16, E=8192, k=8, R=64, N=8, P=1024, Tmax=400),
    # per-block count tables too large for the fused slot kernel: three-launch layout
    W.Config("k80_wide_topk", T=300, H=16, E=256, k=80, R=16, N=4, P=64, Tmax=300),
    W.Config("h8192_two_chunks", T=130, H=8192, E=64, k=6, R=8, N=2, P=32, Tmax=130),
    W.Config("many_blocks", T=20000, H=8, E=64, k=4, R=8, N=2, P=4, Tmax=20000),
    W.Config("wide_table", T=8192, H=8, E=512, k=8, R=256, N=8, P=64, Tmax=8192),
    W.Config("zipf_small_tail", T=4099, H=56, E=256, k=8, R=32, N=4, P=64, Tmax=4099,
             routing="zipf"),
    W.Config("roundtrip_small", T=2000, H=7168, E=256, k=8, R=64, N=8, P=32, Tmax=2000,
             partials="roundtrip"),
]


@pytest.mark.parametrize("cfg", EDGE, ids=lambda c: c.name)
def test_edge_shapes(cfg):
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    run_and_compare_both(cfg, inp, ref)


def test_masked_and_out_of_range_ids():
    cfg = W.Config("bad_ids", T=900, H=32, E=64, k=4, R=8, N=2, P=16, Tmax=900)
    inp = _case(cfg)
    idx = inp.topk_idx.copy()
    rng = np.random.default_rng(11)
    m = rng.random(idx.shape)
    idx[m < 0.1] = -1
    idx[(m > 0.1) & (m < 0.12)] = 64
    idx[(m > 0.12) & (m < 0.13)] = -5
    idx[5] = -1  # a token on no rank at all
    inp.topk_idx = idx
    ref = oracle_all(cfg, inp)
    assert ref["lay"]["error_flag"][0] == 1
    path = run_and_compare_both(cfg, inp, ref, expect_flag=ep.EP_DEVERR_TOPK_RANGE)
    assert np.all(host(path.out)[5] == 0)


def test_determinism_three_runs():
    cfg = W.CONFIGS["dsv3"]
    inp = _case(cfg)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    outs = []
    for _ in range(3):
        fill_sentinels(path)
        path.step(b)
        torch.cuda.synchronize()
        outs.append([host(t).copy() for t in (path.layout_buf.token_slot, path.recv.recv_x,
                                               path.recv.recv_topk_idx, path.prob_dest_major,
                                               path.out)])
    for run in outs[1:]:
        for a, b_ in zip(outs[0], run):
            np.testing.assert_array_equal(a, b_)


def test_layout_reuse_with_other_routing():
    """The workspace carries nothing from one call to the next."""
    cfg = W.CONFIGS["dsv3"].with_(H=64)
    inp = _case(cfg)
    other = W.routing_zipf(np.random.default_rng(3), cfg.T, cfg.E, cfg.k, 1.2)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    for idx in (inp.topk_idx, other, inp.topk_idx):
        dev_idx = torch.from_numpy(idx).cuda()
        path.layout_buf.compute(dev_idx, cfg.E, cfg.R, cfg.N)
        torch.cuda.synchronize()
        lay = oracle.layout(idx, cfg.E, cfg.R, cfg.N)
        np.testing.assert_array_equal(host(path.layout_buf.token_slot), lay["token_slot"])
        np.testing.assert_array_equal(host(path.layout_buf.num_tokens_per_expert), lay["count_e"])


def test_empty_batch():
    cfg = W.Config("empty", T=0, H=64, E=16, k=4, R=4, N=2, P=8, Tmax=4)
    inp = _case(cfg)
    path = Path(0, 64, 16, 4, 4, 2, 8, 4)
    path.layout_buf.num_tokens_per_rank.fill_(5)
    path.layout_buf.rank_offset.fill_(5)
    path.layout_buf.num_tokens_per_expert.fill_(5)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path.step(b)
    torch.cuda.synchronize()
    assert host(path.layout_buf.num_tokens_per_rank).tolist() == [0] * 4
    assert host(path.layout_buf.rank_offset).tolist() == [0] * 5
    assert host(path.layout_buf.num_tokens_per_expert).tolist() == [0] * 16
    assert int(host(path.error_flag)[0]) == 0


def test_recv_capacity_exact_and_short():
    cfg = W.CONFIGS["tiny"]
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    M = ref["M"]
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    for cap, flag in ((M, 0), (M - 37, ep.EP_DEVERR_RECV_OVERFLOW)):
        path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax, recv_capacity=cap)
        fill_sentinels(path)
        path.layout(b)
        path.dispatch(b)
        torch.cuda.synchronize()
        assert int(host(path.error_flag)[0]) == flag
        np.testing.assert_array_equal(host(path.recv.recv_x), ref["d"]["recv_x"][:cap])
        np.testing.assert_array_equal(host(path.recv.recv_src_idx), ref["d"]["recv_src"][:cap])


def test_combine_short_partial_buffer():
    cfg = W.CONFIGS["tiny"]
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    rows = ref["M"] - 100
    slot = ref["lay"]["token_slot"].copy()
    slot[slot >= rows] = -1
    want = oracle.combine(inp.partials[:rows], slot, cfg.R)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials[:rows])
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    path.layout(b)
    path.combine(b)
    torch.cuda.synchronize()
    assert int(host(path.error_flag)[0]) == ep.EP_DEVERR_SLOT_RANGE
    np.testing.assert_array_equal(host(path.out), want)


@pytest.mark.parametrize("T,N,P,Tmax,offset", [(4096, 8, 128, 4096, 1), (1000, 3, 7, 1100, 0),
                                              (77, 2, 12, 80, 0)])
def test_restripe_word_paths(T, N, P, Tmax, offset):
    """Misaligned or P % 4 != 0 buffers take the 32-bit path; same bits either way."""
    print(f"\ncase: restripe T={T} N={N} P={P} Tmax={Tmax} offset={offset}", flush=True)
    prob = W.prob_bit_pattern(T, N, P)
    want = np.full((N, Tmax, P), SENT_U32, np.uint32).view(np.float32)
    oracle.restripe_prob(prob, Tmax, out=want)
    flat_in = torch.empty(T * N * P + offset, dtype=torch.float32, device="cuda")
    flat_in[offset:] = torch.from_numpy(prob.reshape(-1)).cuda()
    src = flat_in[offset:].view(T, N, P)
    flat_out = torch.empty(N * Tmax * P + offset, dtype=torch.float32, device="cuda")
    flat_out.view(torch.int32).fill_(int(np.uint32(SENT_U32).view(np.int32)))
    dst = flat_out[offset:].view(N, Tmax, P)
    ep.ep_restripe_prob(src, dst)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dst).view(np.uint32), want.view(np.uint32))


def test_abi_rejects_bad_arguments_on_gpu():
    cfg = W.CONFIGS["tiny"]
    inp = _case(cfg)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    lb = ep.LayoutBuffers.alloc(cfg.T, cfg.E, cfg.R, cfg.N)
    with pytest.raises(ep.EPError) as e:
        lb.compute(b.topk_idx, 15, cfg.R, cfg.N)  # E % R != 0
    assert e.value.status == ep.EP_ERR_ARG
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(ep.EPError) as e:
        ep.ep_get_layout(b.topk_idx, cfg.E, cfg.R, cfg.N,
                         num_tokens_per_rank=lb.num_tokens_per_rank,
                         num_tokens_per_node=None, num_tokens_per_expert=None,
                         is_token_in_rank=None, rank_offset=lb.rank_offset, expert_offset=None,
                         token_slot=lb.token_slot, error_flag=lb.error_flag, workspace=small)
    assert e.value.status == ep.EP_ERR_CAPACITY
    with pytest.raises(ep.EPError) as e:
        ep.ep_restripe_prob(b.prob, torch.empty((cfg.N, cfg.T - 1, cfg.P), device="cuda"))
    assert e.value.status == ep.EP_ERR_CAPACITY
    x_odd = torch.zeros((cfg.T, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ep.EPError) as e:
        ep.ep_dispatch(x_odd, b.topk_idx, b.topk_weights, cfg.E, cfg.R, lb.token_slot,
                       recv_x=torch.empty((10, 12), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == ep.EP_ERR_ALIGN


def test_binding_rejects_buffers_off_the_current_device(monkeypatch):
    # kernels run on the current device's stream; a buffer elsewhere is refused before any
    # launch (a second device is simulated by reporting another current device)
    cfg = W.CONFIGS["tiny"]
    print(f"\ncase: off-device buffers {cfg.name}", flush=True)
    prob = torch.zeros((cfg.T, cfg.N, cfg.P), dtype=torch.float32, device="cuda")
    out = torch.full((cfg.N, cfg.Tmax, cfg.P), 7.0, dtype=torch.float32, device="cuda")
    other = torch.cuda.current_device() + 1
    monkeypatch.setattr(torch.cuda, "current_device", lambda: other)
    with pytest.raises(ValueError, match="current device"):
        ep.ep_restripe_prob(prob, out)
    with pytest.raises(ValueError, match="current device"):
        ep.ep_hbm_copy(prob, out)
    monkeypatch.undo()
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing was launched
    with pytest.raises(ValueError, match="current device"):
        ep.ep_restripe_prob(prob, out, stream=_OtherDeviceStream())


class _OtherDeviceStream(torch.cuda.Stream):
    """A stream object that reports a device other than the current one."""

    @property
    def device(self):
        return torch.device("cuda", torch.cuda.current_device() + 1)


@pytest.mark.parametrize("T", [1, 2, 3, 4095, 4096, 4097, 8193])
def test_dispatch_token_counts(T):
    # one wave per (token, destination): token counts that leave the last block partly
    # empty, with D = min(k, R) = 6 waves per token not dividing the block's 4 waves
    cfg = W.Config(f"thr_T{T}", T=T, H=512, E=64, k=6, R=16, N=4, P=8, Tmax=T, seed=T)
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    path = run_gpu(cfg, inp)
    compare_all(cfg, path, ref)


def _check_permute_and_send(cfg, inp):
    """The expert-major permute and the two-phase send phase against the oracle."""
    from combine_ep_get_03_amd.buffers import LayoutBuffers

    T = cfg.T
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob)
    lbe = LayoutBuffers.alloc(T, cfg.E, cfg.R, cfg.N, k_expert_slots=cfg.k)
    lbe.compute(b.topk_idx, cfg.E, cfg.R, cfg.N)
    px = torch.full((T * cfg.k, cfg.H), 7.0, dtype=torch.bfloat16, device="cuda")
    pw = torch.empty(T * cfg.k, dtype=torch.float32, device="cuda")
    ps = torch.empty(T * cfg.k, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_permute(b.x, b.topk_weights, lbe.expert_slot, perm_x=px, perm_weights=pw,
                           perm_src_idx=ps, error_flag=lbe.error_flag)
    es = oracle.expert_slots(inp.topk_idx, cfg.E)
    want = oracle.dispatch_permute(inp.x, inp.topk_idx, inp.topk_weights, es, T * cfg.k)
    torch.cuda.synchronize()
    assert int(lbe.error_flag.item()) == 0
    np.testing.assert_array_equal(host(px), want["perm_x"])
    np.testing.assert_array_equal(host(pw).view(np.uint32), want["perm_w"].view(np.uint32))
    np.testing.assert_array_equal(host(ps), want["perm_src"])
    del px, pw, ps, lbe, want

    path = Path(T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax, node_slots=True)
    path.layout(b)
    path.dispatch_send(b)
    torch.cuda.synchronize()
    ns = oracle.node_slots(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    st = oracle.hook_dispatch_send(inp.x, inp.topk_idx, inp.topk_weights, ns, cfg.Tmax)
    assert int(path.error_flag.item()) == 0
    for n in range(cfg.N):
        cnt = int((ns[:, n] >= 0).sum())
        np.testing.assert_array_equal(host(path.stage.stage_x[n, :cnt]), st["stage_x"][n, :cnt])
        np.testing.assert_array_equal(host(path.stage.stage_topk_idx[n, :cnt]), st["stage_idx"][n, :cnt])
        np.testing.assert_array_equal(host(path.stage.stage_topk_weights[n, :cnt]).view(np.uint32),
                                      st["stage_w"][n, :cnt].view(np.uint32))
        np.testing.assert_array_equal(host(path.stage.stage_src[n, :cnt]), st["stage_src"][n, :cnt])


@pytest.mark.parametrize("T", [3, 4095, 4097])
def test_permute_and_send_token_counts(T):
    # the same (token, destination) form: k = 6 waves per token for the permute,
    # min(k, N) = 4 for the send phase
    cfg = W.Config(f"thr2_T{T}", T=T, H=512, E=64, k=6, R=16, N=4, P=8, Tmax=T + 5, seed=T + 1)
    _check_permute_and_send(cfg, _case(cfg))


def test_launches_split_over_token_ranges():
    # a (token, destination) launch holds at most 2^22 waves: 600 000 tokens with 8 waves
    # each take two launches of dispatch, permute and send (and the first range's last
    # block must not run into the second range's tokens)
    cfg = W.Config("split_600k", T=600_000, H=8, E=64, k=8, R=8, N=8, P=4, Tmax=600_000,
                   seed=11)
    assert cfg.T * min(cfg.k, cfg.R) > (1 << 22)
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    path = run_gpu(cfg, inp)
    compare_all(cfg, path, ref)
    del path, ref
    torch.cuda.empty_cache()
    _check_permute_and_send(cfg, inp)


@pytest.mark.parametrize("form", ["counts", "preprocess"])
@pytest.mark.parametrize("name", ["tiny", "dsv3"])
def test_graph_replay_matches_eager(name, form):
    """The whole step captured in a HIP graph, in both step forms: every replay, with eager
    work and synchronisation in between, reproduces the eager outputs bit for bit."""
    cfg = W.CONFIGS[name]
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    step = path.step_counts if form == "counts" else path.step_preprocess
    fill_sentinels(path)
    step(b)
    torch.cuda.synchronize()
    compare_all(cfg, path, ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(b)
    for _ in range(3):
        fill_sentinels(path)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_all(cfg, path, ref)


def test_dispatch_rows_only():
    """Metadata outputs are optional: with all three NULL only recv_x is written."""
    cfg = W.CONFIGS["tiny"]
    inp = _case(cfg)
    ref = oracle_all(cfg, inp)
    M = ref["M"]
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)
    fill_sentinels(path)
    path.layout(b)
    ep.ep_dispatch(b.x, b.topk_idx, None, cfg.E, cfg.R, path.layout_buf.token_slot,
                   recv_x=path.recv.recv_x, error_flag=path.error_flag)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(path.recv.recv_x)[:M], ref["d"]["recv_x"][:M])
    assert np.all(host(path.recv.recv_topk_idx) == -0x123456789)
    assert np.all(host(path.recv.recv_src_idx) == -7)
