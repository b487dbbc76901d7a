"""Pins for the oracle's two-phase ("hook") dispatch and combine.

Dispatch: send then receive must give exactly the one-call dispatch (itself pinned
against brute force and numpy gathers), and the staged rows of each node must be the
numpy boolean-mask gather of the tokens routed there. Combine: with small-integer
partials every sum is exact, so the staged node sums and the output equal integer sums
computed with numpy; with one rank per node, or one node, the two-phase combine reduces
to the one-call combine bit for bit; random partials stay within the error bound of two
bf16 roundings around fp64 sums.
"""
import numpy as np
import pytest

from combine_ep_get_03_amd import workloads as W

SENT16 = np.uint16(0xBEEF)


def node_mask(idx, E, N):
    """[T][N]: token t has an expert (valid id) on node n."""
    T, k = idx.shape
    on = np.zeros((T, N), bool)
    valid = (idx >= 0) & (idx < E)
    tt = np.repeat(np.arange(T), k).reshape(T, k)[valid]
    on[tt, idx[valid] // (E // N)] = True
    return on


def sentinel_stage(N, Tmax, H, k):
    return dict(stage_x=np.full((N, Tmax, H), SENT16, np.uint16),
                stage_idx=np.full((N, Tmax, k), -7, np.int64),
                stage_w=np.full((N, Tmax, k), -3.5, np.float32),
                stage_src=np.full((N, Tmax), -9, np.int32))


def sentinel_recv(cap, H, k):
    return dict(recv_x=np.full((cap, H), SENT16, np.uint16),
                recv_idx=np.full((cap, k), -7, np.int64),
                recv_w=np.full((cap, k), -3.5, np.float32),
                recv_src=np.full(cap, -9, np.int32))


CASES = [W.CONFIGS["tiny"], W.CONFIGS["dsv3"].with_(T=700, H=64),
         W.CONFIGS["skewed"].with_(T=513, H=32), W.CONFIGS["restripe"].with_(T=300, H=16),
         W.CONFIGS["large"].with_(T=257, H=8)]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_send_then_recv_is_the_dispatch(orc, cfg):
    inp = W.make_inputs(cfg)
    idx, w = inp.topk_idx, inp.topk_weights
    lay = orc.layout(idx, cfg.E, cfg.R, cfg.N)
    ns = orc.node_slots(idx, cfg.E, cfg.R, cfg.N)
    cap = cfg.T * min(cfg.k, cfg.R)
    st = orc.hook_dispatch_send(inp.x, idx, w, ns, cfg.Tmax,
                                out=sentinel_stage(cfg.N, cfg.Tmax, cfg.H, cfg.k))
    got = orc.hook_dispatch_recv(st, lay["count_n"], cfg.E, cfg.R, lay["token_slot"], cap,
                                 out=sentinel_recv(cap, cfg.H, cfg.k))
    want = orc.dispatch(inp.x, idx, w, cfg.E, cfg.R, lay["token_slot"], cap)
    M = int(lay["rank_offset"][-1])
    for key in ("recv_x", "recv_idx", "recv_w", "recv_src"):
        np.testing.assert_array_equal(got[key][:M].view(np.uint8), want[key][:M].view(np.uint8), key)
    assert np.all(got["recv_x"][M:] == SENT16) and np.all(got["recv_src"][M:] == -9)


@pytest.mark.parametrize("cfg", CASES[:3], ids=lambda c: c.name)
def test_send_stages_the_mask_gather_per_node(orc, cfg):
    inp = W.make_inputs(cfg)
    idx = inp.topk_idx
    ns = orc.node_slots(idx, cfg.E, cfg.R, cfg.N)
    st = orc.hook_dispatch_send(inp.x, idx, inp.topk_weights, ns, cfg.Tmax,
                                out=sentinel_stage(cfg.N, cfg.Tmax, cfg.H, cfg.k))
    on = node_mask(idx, cfg.E, cfg.N)
    lay = orc.layout(idx, cfg.E, cfg.R, cfg.N)
    for n in range(cfg.N):
        c = int(on[:, n].sum())
        assert c == lay["count_n"][n]
        np.testing.assert_array_equal(st["stage_x"][n, :c], inp.x[on[:, n]])
        np.testing.assert_array_equal(st["stage_src"][n, :c], np.nonzero(on[:, n])[0])
        np.testing.assert_array_equal(st["stage_idx"][n, :c], idx[on[:, n]])
        np.testing.assert_array_equal(st["stage_w"][n, :c].view(np.uint32),
                                      inp.topk_weights[on[:, n]].view(np.uint32))
        assert np.all(st["stage_x"][n, c:] == SENT16) and np.all(st["stage_src"][n, c:] == -9)


def test_dispatch_masked_and_bad_ids(orc):
    E, R, N, k, H = 16, 8, 4, 3, 8
    idx = np.array([[0, -1, 15], [-1, -1, -1], [3, 20, 4], [-5, 8, 9], [1, 1, 2]], np.int64)
    T = idx.shape[0]
    x = (np.arange(T * H, dtype=np.uint16).reshape(T, H) * 37) & 0x3FFF
    w = np.linspace(0.1, 1.5, T * k, dtype=np.float32).reshape(T, k)
    lay = orc.layout(idx, E, R, N)
    ns = orc.node_slots(idx, E, R, N)
    st = orc.hook_dispatch_send(x, idx, w, ns, T)
    got = orc.hook_dispatch_recv(st, lay["count_n"], E, R, lay["token_slot"], T * k)
    want = orc.dispatch(x, idx, w, E, R, lay["token_slot"], T * k)
    for key in want:
        np.testing.assert_array_equal(got[key], want[key])
    assert list(ns[1]) == [-1] * N                 # a fully masked token is staged nowhere


def test_recv_rejects_bad_staged_token(orc):
    stage = sentinel_stage(1, 2, 8, 1)
    stage["stage_src"][0, 0] = 5                   # token 5 of a 2-token batch
    with pytest.raises(ValueError):
        orc.hook_dispatch_recv(stage, np.array([1], np.int32), 2, 1, np.zeros((2, 1), np.int32), 4)


def small_int_partials(rng, rows, H):
    v = rng.integers(-4, 5, size=(rows, H)).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16), v


@pytest.mark.parametrize("cfg", [W.CONFIGS["dsv3"].with_(T=500, H=24),
                                 W.CONFIGS["tiny"].with_(H=16),
                                 W.CONFIGS["large"].with_(T=300, H=8)], ids=lambda c: c.name)
def test_combine_small_integers_exact(orc, cfg):
    rng = np.random.default_rng(11)
    idx = W.make_inputs(cfg, with_x=False, with_prob=False).topk_idx
    lay = orc.layout(idx, cfg.E, cfg.R, cfg.N)
    ns = orc.node_slots(idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    bits, vals = small_int_partials(rng, M, cfg.H)
    stage = orc.hook_combine_send(bits, lay["token_slot"], cfg.R, ns, cfg.Tmax)
    slot = lay["token_slot"]
    rpn = cfg.R // cfg.N
    total = np.zeros((cfg.T, cfg.H))
    for n in range(cfg.N):
        node_sum = np.zeros((cfg.T, cfg.H))
        for r in range(n * rpn, (n + 1) * rpn):
            has = slot[:, r] >= 0
            node_sum[has] += vals[slot[has, r]]
        routed = ns[:, n] >= 0
        got = orc.bf16_to_f32(stage[n, ns[routed, n]])
        np.testing.assert_array_equal(got, node_sum[routed])
        total += node_sum
    out = orc.hook_combine_recv(stage, ns)
    np.testing.assert_array_equal(orc.bf16_to_f32(out), total)
    np.testing.assert_array_equal(out, orc.combine(bits, slot, cfg.R))


def test_combine_one_rank_per_node_is_the_flat_combine(orc):
    cfg = W.CONFIGS["restripe"].with_(T=400, H=48)          # R = N = 8
    inp = W.make_inputs(cfg, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    ns = orc.node_slots(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    part = inp.partials[:M]
    stage = orc.hook_combine_send(part, lay["token_slot"], cfg.R, ns, cfg.Tmax)
    np.testing.assert_array_equal(orc.hook_combine_recv(stage, ns),
                                  orc.combine(part, lay["token_slot"], cfg.R))


def test_combine_one_node_is_the_flat_combine(orc):
    cfg = W.CONFIGS["dsv3"].with_(T=300, H=40, N=1)
    inp = W.make_inputs(cfg, with_prob=False)
    inp.topk_idx[7] = -1                                      # a token on no rank gets +0
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    ns = orc.node_slots(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    part = inp.partials[:int(lay["rank_offset"][-1])]
    out = orc.hook_combine_recv(orc.hook_combine_send(part, lay["token_slot"], cfg.R, ns, cfg.Tmax), ns)
    np.testing.assert_array_equal(out, orc.combine(part, lay["token_slot"], cfg.R))
    assert np.all(out[7] == 0)


def test_combine_within_two_roundings_of_fp64(orc):
    cfg = W.CONFIGS["dsv3"].with_(T=400, H=64)
    inp = W.make_inputs(cfg, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    ns = orc.node_slots(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    part = inp.partials[:M]
    pf = orc.bf16_to_f32(part).astype(np.float64)
    stage = orc.hook_combine_send(part, lay["token_slot"], cfg.R, ns, cfg.Tmax)
    out = orc.bf16_to_f32(orc.hook_combine_recv(stage, ns)).astype(np.float64)
    slot = lay["token_slot"]
    rpn = cfg.R // cfg.N
    exact = np.zeros((cfg.T, cfg.H))
    bound = np.zeros((cfg.T, cfg.H))
    for n in range(cfg.N):
        e_n = np.zeros((cfg.T, cfg.H))
        mag = np.zeros((cfg.T, cfg.H))
        for r in range(n * rpn, (n + 1) * rpn):
            has = slot[:, r] >= 0
            e_n[has] += pf[slot[has, r]]
            mag[has] += np.abs(pf[slot[has, r]])
        routed = ns[:, n] >= 0
        st = orc.bf16_to_f32(stage[n, ns[routed, n]]).astype(np.float64)
        # one bf16 rounding (half an ulp, 2^-8 relative) after an fp32 sum of <= rpn terms
        assert np.all(np.abs(st - e_n[routed]) <= 2.0**-8 * np.abs(e_n[routed]) + 2.0**-22 * mag[routed])
        exact += e_n
        bound += 2.0**-8 * np.abs(e_n) + 2.0**-22 * mag
    assert np.all(np.abs(out - exact) <= 2.0**-8 * np.abs(exact) * 1.01 + bound * 1.01)


def test_empty_batch(orc):
    idx = np.zeros((0, 4), np.int64)
    ns = orc.node_slots(idx, 16, 4, 2)
    st = orc.hook_dispatch_send(np.zeros((0, 8), np.uint16), idx, np.zeros((0, 4), np.float32), ns, 0)
    assert st["stage_x"].shape == (2, 0, 8)
    assert orc.hook_combine_recv(np.zeros((2, 0, 8), np.uint16), ns).shape == (0, 8)
