"""GPU test of ep_get_layout_no_alloc, the layout entry point that takes no workspace and
allocates nothing (its per-block tables live in the library's static device scratch):
through the C ABI, every output must equal ep_get_layout's with a caller workspace, bit
for bit, on calls in a row whose sizes shrink and grow, so stale scratch contents from an
earlier, larger call are exercised."""
import numpy as np
import pytest
import torch

import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd import workloads as W

pytestmark = pytest.mark.gpu

# dsv3-shaped first, then a smaller batch, the one-block path, the path with a separate
# scan launch (79 blocks), and a small batch again after it
SEQUENCE = [
    W.Config("dsv3_shape", T=4096, H=8, E=256, k=8, R=32, N=4, P=8, Tmax=4096),
    W.Config("smaller", T=1000, H=8, E=64, k=6, R=8, N=2, P=8, Tmax=1000),
    W.Config("one_block", T=200, H=8, E=16, k=4, R=4, N=2, P=8, Tmax=200),
    W.Config("many_blocks", T=20000, H=8, E=64, k=4, R=8, N=2, P=4, Tmax=20000),
    W.Config("smaller_again", T=777, H=8, E=128, k=8, R=16, N=4, P=8, Tmax=777),
]


def _outputs(T, k, E, R, N, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    o = dict(num_tokens_per_rank=torch.empty(R, **i32), num_tokens_per_node=torch.empty(N, **i32),
             num_tokens_per_expert=torch.empty(E, **i32),
             is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
             rank_offset=torch.empty(R + 1, **i32), expert_offset=torch.empty(E + 1, **i32),
             token_slot=torch.empty((T, R), **i32), expert_slot=torch.empty((T, k), **i32),
             node_slot=torch.empty((T, N), **i32), error_flag=torch.empty(1, **i32))
    for name, t in o.items():  # sentinels: every element the call defines must be written
        t.fill_(-77 if t.dtype == torch.int32 else 0xCD)
    return o


def _layout_pair(cfg, idx_host, dev):
    idx = torch.from_numpy(idx_host).to(dev)
    ref = _outputs(cfg.T, cfg.k, cfg.E, cfg.R, cfg.N, dev)
    ws = torch.empty(max(16, ep.ep_layout_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N)),
                     dtype=torch.uint8, device=dev)
    ep.ep_get_layout(idx, cfg.E, cfg.R, cfg.N, workspace=ws, **ref)
    got = _outputs(cfg.T, cfg.k, cfg.E, cfg.R, cfg.N, dev)
    ep.ep_get_layout_no_alloc(idx, cfg.E, cfg.R, cfg.N, **got)
    torch.cuda.synchronize()
    return ref, got


def _assert_equal(ref, got, where):
    for name in ref:
        a, b = ref[name].cpu().numpy(), got[name].cpu().numpy()
        assert np.array_equal(a, b), f"{where}: {name} differs"


def test_no_alloc_layout_matches_the_workspace_layout_on_calls_in_a_row():
    dev = torch.device("cuda", torch.cuda.current_device())
    for cfg in SEQUENCE:
        print(f"\ncase: ep_get_layout_no_alloc {cfg}", flush=True)
        need = ep.ep_layout_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N)
        assert 0 < need <= ep.EP_LAYOUT_SCRATCH_BYTES
        inp = W.make_inputs(cfg, with_x=False)
        ref, got = _layout_pair(cfg, inp.topk_idx, dev)
        _assert_equal(ref, got, cfg.name)
        assert int(got["error_flag"][0]) == 0
        M = int(got["rank_offset"][-1])
        assert M == int(got["num_tokens_per_rank"].sum())
        assert sorted(got["token_slot"][got["token_slot"] >= 0].tolist()) == list(range(M))


def test_no_alloc_layout_reports_bad_ids_like_the_workspace_layout():
    dev = torch.device("cuda", torch.cuda.current_device())
    cfg = W.Config("bad_ids", T=900, H=8, E=64, k=4, R=8, N=2, P=8, Tmax=900)
    print(f"\ncase: ep_get_layout_no_alloc {cfg} with masked and out-of-range ids", flush=True)
    idx = W.make_inputs(cfg, with_x=False).topk_idx.copy()
    rng = np.random.default_rng(5)
    idx[rng.integers(0, cfg.T, 40), rng.integers(0, cfg.k, 40)] = -1
    idx[rng.integers(0, cfg.T, 7), rng.integers(0, cfg.k, 7)] = cfg.E + 3
    ref, got = _layout_pair(cfg, idx, dev)
    _assert_equal(ref, got, cfg.name)
    assert int(got["error_flag"][0]) == ep.EP_DEVERR_TOPK_RANGE


def test_no_alloc_layout_rejects_tables_past_the_scratch():
    dev = torch.device("cuda", torch.cuda.current_device())
    T, E, R, N, k = 458753, 256, 64, 8, 1
    assert ep.ep_layout_workspace_bytes(T, E, R, N) > ep.EP_LAYOUT_SCRATCH_BYTES
    idx = torch.zeros((T, k), dtype=torch.int64, device=dev)
    o = _outputs(T, k, E, R, N, dev)
    with pytest.raises(ep.EPError) as err:
        ep.ep_get_layout_no_alloc(idx, E, R, N, **o)
    assert err.value.status == ep.EP_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(o["error_flag"][0]) == -77  # nothing was enqueued
