"""Pins for the oracle's expert-major permute: a stable sort of (expert, token, slot)
keys written with Python's sorted(), numpy's stable argsort, the layout's expert offsets,
and the rank-range property (each rank's local experts form one contiguous block)."""
import itertools

import numpy as np
import pytest

from combine_ep_get_03_amd import workloads as W


def brute_expert_slots(idx, E):
    items = [(int(e), t, j) for t, row in enumerate(idx) for j, e in enumerate(row) if 0 <= e < E]
    order = {(t, j): q for q, (_, t, j) in enumerate(sorted(items))}
    return np.array([[order.get((t, j), -1) for j in range(idx.shape[1])] for t in range(len(idx))],
                    np.int32)


def test_exhaustive_tiny(orc):
    for E, k, T in ((3, 2, 3), (4, 2, 2)):
        choices = list(itertools.product(range(-1, E + 1), repeat=k))   # masked, bad and duplicates
        for combo in itertools.product(choices, repeat=T):
            idx = np.array(combo, np.int64).reshape(T, k)
            np.testing.assert_array_equal(orc.expert_slots(idx, E), brute_expert_slots(idx, E))


@pytest.mark.parametrize("name", ["tiny", "dsv3", "skewed", "large"])
def test_stable_argsort_and_offsets(orc, name):
    cfg = W.CONFIGS[name]
    idx = W.make_inputs(cfg, with_x=False, with_prob=False).topk_idx
    es = orc.expert_slots(idx, cfg.E)
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")          # (token, slot) order kept within an expert
    want = np.empty(flat.size, np.int32)
    want[order] = np.arange(flat.size, dtype=np.int32)
    np.testing.assert_array_equal(es.ravel(), want)
    lay = orc.layout(idx, cfg.E, cfg.R, cfg.N)
    eo = lay["expert_offset"]
    # expert e's rows are exactly expert_offset[e] .. expert_offset[e+1]-1
    np.testing.assert_array_equal(np.searchsorted(eo, es.ravel(), side="right") - 1, flat)
    # rank r's rows are one contiguous block: its local experts in order
    er = cfg.E // cfg.R
    rank_of_row = np.empty(flat.size, np.int64)
    rank_of_row[es.ravel()] = flat // er
    assert np.all(np.diff(rank_of_row) >= 0)


def test_permute_rows(orc):
    cfg = W.CONFIGS["dsv3"].with_(T=300, H=64)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    es = orc.expert_slots(inp.topk_idx, cfg.E)
    d = orc.dispatch_permute(inp.x, inp.topk_idx, inp.topk_weights, es, cfg.T * cfg.k)
    q = es.ravel()
    t = np.repeat(np.arange(cfg.T), cfg.k)
    np.testing.assert_array_equal(d["perm_x"][q], inp.x[t])
    np.testing.assert_array_equal(d["perm_w"][q], inp.topk_weights.ravel())
    np.testing.assert_array_equal(d["perm_src"][q], t)
    # within each expert the source tokens ascend
    flat = inp.topk_idx.ravel()
    for e in range(cfg.E):
        rows = np.sort(q[flat == e])
        assert np.all(np.diff(d["perm_src"][rows]) > 0)


def test_masked_and_capacity(orc):
    idx = np.array([[2, -1], [0, 2], [5, 2]], np.int64)   # 5 is out of range for E = 4
    es = orc.expert_slots(idx, 4)
    assert es.tolist() == [[1, -1], [0, 2], [-1, 3]]
    x = np.arange(6, dtype=np.uint16).reshape(3, 2)
    w = np.ones((3, 2), np.float32)
    with pytest.raises(ValueError):
        orc.dispatch_permute(x, idx, w, es, 3)
