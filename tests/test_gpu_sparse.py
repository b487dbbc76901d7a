"""GPU parity of the sparse-path restripe: ep_get_layout's node_slot output and
ep_restripe_prob_sparse, against the oracle, bit for bit (padding rows untouched)."""
import numpy as np
import pytest
import torch

import oracle
import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.buffers import LayoutBuffers

from gpu_util import SENT_U32, host

pytestmark = pytest.mark.gpu


def check(cfg, inp):
    T, N, P, Tmax = cfg.T, cfg.N, cfg.P, cfg.Tmax
    tidx = torch.from_numpy(inp.topk_idx).cuda()
    lb = LayoutBuffers.alloc(T, cfg.E, cfg.R, N, node_slots=True)
    lb.node_slot.fill_(-77)
    lb.compute(tidx, cfg.E, cfg.R, N)
    prob = torch.from_numpy(inp.prob).cuda()
    out = torch.empty((N, Tmax, P), dtype=torch.float32, device="cuda")
    out.view(torch.int32).fill_(int(np.uint32(SENT_U32).view(np.int32)))
    ep.ep_restripe_prob_sparse(prob, lb.node_slot, out, error_flag=lb.error_flag)
    torch.cuda.synchronize()
    ns = oracle.node_slots(inp.topk_idx, cfg.E, cfg.R, N)
    np.testing.assert_array_equal(host(lb.node_slot), ns)
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, N)
    np.testing.assert_array_equal(host(lb.token_slot), lay["token_slot"])
    np.testing.assert_array_equal(host(lb.num_tokens_per_node), lay["count_n"])
    assert int(host(lb.error_flag)[0]) == 0
    want = np.full((N, Tmax, P), SENT_U32, np.uint32).view(np.float32)
    oracle.restripe_prob_sparse(inp.prob, ns, Tmax, out=want)
    np.testing.assert_array_equal(host(out).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "restripe", "dsv3", "skewed", "large"])
def test_sparse_configs(name):
    cfg = W.CONFIGS[name]
    print(f"\ncase: sparse restripe {cfg}", flush=True)
    check(cfg, W.make_inputs(cfg, with_x=False))


@pytest.mark.parametrize("cfg", [
    W.Config("s_one", T=1, H=8, E=16, k=4, R=4, N=2, P=8, Tmax=3),
    W.Config("s_ragged", T=257, H=8, E=12, k=3, R=3, N=3, P=5, Tmax=300),
    W.Config("s_many_blocks", T=20000, H=8, E=64, k=4, R=8, N=2, P=4, Tmax=20000),
    W.Config("s_wide_table", T=8192, H=8, E=512, k=8, R=256, N=8, P=64, Tmax=8192),
    W.Config("s_r1024", T=700, H=8, E=2048, k=16, R=1024, N=8, P=256, Tmax=700),
    W.Config("s_n1", T=333, H=8, E=32, k=4, R=8, N=1, P=12, Tmax=400),
    W.Config("s_n_eq_r", T=600, H=8, E=64, k=6, R=16, N=16, P=4, Tmax=600),
], ids=lambda c: c.name)
def test_sparse_shapes(cfg):
    print(f"\ncase: sparse restripe {cfg}", flush=True)
    check(cfg, W.make_inputs(cfg, with_x=False))
