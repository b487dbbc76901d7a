"""Pins for the oracle's sparse restripe: node slots against a sorted (node, token)
enumeration and numpy cumsums, the layout's per-node counts, and the packed layout
against numpy boolean-mask gathers; each chunk's routed slices form one run."""
import itertools

import numpy as np
import pytest

from combine_ep_get_03_amd import workloads as W

SENT = np.uint32(0xDEADBEEF)


def brute_node_slots(idx, E, R, N):
    epn = E // N
    pairs = sorted({(int(e) // epn, t) for t, row in enumerate(idx) for e in row if 0 <= e < E})
    pos = {}
    for n in range(N):
        for q, (nn, t) in enumerate(p for p in pairs if p[0] == n):
            pos[(n, t)] = q
    return np.array([[pos.get((n, t), -1) for n in range(N)] for t in range(len(idx))], np.int32)


def test_exhaustive_tiny(orc):
    for E, R, N in ((4, 2, 2), (4, 4, 2), (6, 3, 3)):
        choices = list(itertools.product(range(-1, E), repeat=2))
        for combo in itertools.product(choices, repeat=2):
            idx = np.array(combo, np.int64).reshape(2, 2)
            np.testing.assert_array_equal(orc.node_slots(idx, E, R, N), brute_node_slots(idx, E, R, N))


@pytest.mark.parametrize("name", ["tiny", "restripe", "dsv3", "skewed", "large"])
def test_node_slots_closed_form(orc, name):
    cfg = W.CONFIGS[name]
    idx = W.make_inputs(cfg, with_x=False, with_prob=False).topk_idx
    ns = orc.node_slots(idx, cfg.E, cfg.R, cfg.N)
    on = np.zeros((cfg.T, cfg.N), bool)
    on[np.repeat(np.arange(cfg.T), cfg.k), (idx // (cfg.E // cfg.N)).ravel()] = True
    np.testing.assert_array_equal(ns, np.where(on, np.cumsum(on, 0) - 1, -1))
    lay = orc.layout(idx, cfg.E, cfg.R, cfg.N)
    np.testing.assert_array_equal((ns >= 0).sum(0), lay["count_n"])


def test_sparse_restripe_packs_routed_slices(orc):
    cfg = W.CONFIGS["dsv3"].with_(T=1000)
    inp = W.make_inputs(cfg, with_x=False)
    ns = orc.node_slots(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    out = np.full((cfg.N, cfg.Tmax, cfg.P), SENT, np.uint32).view(np.float32)
    orc.restripe_prob_sparse(inp.prob, ns, cfg.Tmax, out=out)
    ow = out.view(np.uint32)
    pw = inp.prob.view(np.uint32)
    for n in range(cfg.N):
        routed = ns[:, n] >= 0
        cnt = int(routed.sum())
        np.testing.assert_array_equal(ow[n, :cnt], pw[routed, n, :])
        assert np.all(ow[n, cnt:] == SENT)
        # a chunk of consecutive tokens: its routed slices are one contiguous run
        for c0 in range(0, cfg.T, cfg.chunk):
            s = ns[c0:c0 + cfg.chunk, n]
            s = s[s >= 0]
            if s.size:
                assert np.all(np.diff(s) == 1)


def test_sparse_equals_dense_when_every_token_is_everywhere(orc):
    T, N, P = 50, 2, 8
    idx = np.tile(np.array([0, 3], np.int64), (T, 1))       # E = 4, R = 2, N = 2: both nodes
    ns = orc.node_slots(idx, 4, 2, N)
    prob = np.random.default_rng(0).random((T, N, P), dtype=np.float32)
    sparse = orc.restripe_prob_sparse(prob, ns, T)
    np.testing.assert_array_equal(sparse.view(np.uint32), orc.restripe_prob(prob, T).view(np.uint32))
