"""Pins for the oracle's dispatch permute: numpy boolean-mask gathers per rank,
invariants of the receive layout, and the single-rank special case."""
import numpy as np
import pytest

from combine_ep_get_03_amd import workloads as W


def _small(name, **kw):
    """The config's routing structure at a hidden size the CPU suite can afford."""
    cfg = W.CONFIGS[name]
    return cfg.with_(**kw) if kw else cfg


@pytest.mark.parametrize("cfg", [
    _small("tiny"),
    _small("dsv3", T=512, H=64),
    _small("skewed", T=512, H=64),
    _small("large", T=1024, H=32),
    W.Config("ragged", T=77, H=24, E=12, k=3, R=3, N=1, P=4, Tmax=77),
])
def test_mask_gather_closed_form(orc, cfg):
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    E, R = cfg.E, cfg.R
    er = E // R
    lay = orc.layout(inp.topk_idx, E, R, cfg.N)
    d = orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, E, R, lay["token_slot"], cfg.cap)
    ro = lay["rank_offset"]
    M = int(ro[R])
    bitmap = lay["in_rank"].astype(bool)
    per_token_local = np.zeros(cfg.T, np.int64)
    for r in range(R):
        rows = slice(ro[r], ro[r + 1])
        src = np.nonzero(bitmap[:, r])[0]
        np.testing.assert_array_equal(d["recv_src"][rows], src)
        np.testing.assert_array_equal(d["recv_x"][rows], inp.x[bitmap[:, r]])
        ids = inp.topk_idx[src]
        on_r = (ids // er) == r
        np.testing.assert_array_equal(d["recv_idx"][rows], np.where(on_r, ids - r * er, -1))
        np.testing.assert_array_equal(d["recv_w"][rows].view(np.uint32),
                                      np.where(on_r, inp.topk_weights[src], 0.0)
                                      .astype(np.float32).view(np.uint32))
        np.add.at(per_token_local, src, (d["recv_idx"][rows] >= 0).sum(1))
    # every routed slot lands on exactly one rank
    np.testing.assert_array_equal(per_token_local, np.full(cfg.T, cfg.k))
    # rows past M are never written
    assert not d["recv_x"][M:].any() and not d["recv_src"][M:].any()
    # each (token, rank) pair once: (src, rank-of-row) pairs are all distinct
    rank_of_row = np.searchsorted(ro, np.arange(M), side="right") - 1
    pairs = set(zip(d["recv_src"][:M].tolist(), rank_of_row.tolist()))
    assert len(pairs) == M == int(bitmap.sum())


def test_single_rank_is_memcpy(orc):
    cfg = W.Config("r1", T=100, H=16, E=8, k=2, R=1, N=1, P=4, Tmax=100)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, 1, 1)
    d = orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, 1, lay["token_slot"], cfg.cap)
    np.testing.assert_array_equal(d["recv_x"], inp.x)
    np.testing.assert_array_equal(d["recv_idx"], inp.topk_idx)
    np.testing.assert_array_equal(d["recv_w"], inp.topk_weights)


def test_hand_example(orc):
    """Two tokens, four experts on two ranks; the expected rows written out by hand."""
    x = np.array([[1, 2], [3, 4]], np.uint16)
    idx = np.array([[3, 0], [2, 3]], np.int64)
    w = np.array([[0.25, 0.75], [0.5, 0.5]], np.float32)
    lay = orc.layout(idx, 4, 2, 1)
    assert lay["token_slot"].tolist() == [[0, 1], [-1, 2]]
    d = orc.dispatch(x, idx, w, 4, 2, lay["token_slot"], 4)
    assert d["recv_x"][:3].tolist() == [[1, 2], [1, 2], [3, 4]]
    assert d["recv_src"][:3].tolist() == [0, 0, 1]
    assert d["recv_idx"][:3].tolist() == [[-1, 0], [1, -1], [0, 1]]
    assert d["recv_w"][:3].tolist() == [[0.0, 0.75], [0.25, 0.0], [0.5, 0.5]]


def test_capacity_overflow_rejected(orc):
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], M)
    with pytest.raises(ValueError):
        orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], M - 1)
