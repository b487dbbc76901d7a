"""Independent calls on two streams at once: two batches with their own buffers, their
steps enqueued alternately on two streams so their kernels overlap on the GPU. Each must
match the oracle bit for bit; the library keeps no state between calls, so nothing is
shared between the two paths."""
import pytest
import torch

from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

from gpu_util import compare_all, fill_sentinels, oracle_all

pytestmark = pytest.mark.gpu


def test_two_paths_on_two_streams():
    cfgs = [W.CONFIGS["tiny"].with_(name="tiny_s0"),
            W.Config("mid_s1", T=1500, H=2048, E=64, k=6, R=16, N=4, P=16, Tmax=1600, seed=11)]
    print(f"\ncase: concurrent streams {[c.name for c in cfgs]}", flush=True)
    inps = [W.make_inputs(c) for c in cfgs]
    refs = [oracle_all(c, i) for c, i in zip(cfgs, inps)]
    batches = [DeviceBatch.from_host(i.topk_idx, i.topk_weights, i.x, i.prob, i.partials)
               for i in inps]
    paths = [Path(c.T, c.H, c.E, c.k, c.R, c.N, c.P, c.Tmax) for c in cfgs]
    for p in paths:
        fill_sentinels(p)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.layout(b, stream=s)
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.dispatch(b, stream=s)
                p.restripe(b, stream=s)
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.combine(b, stream=s)
    torch.cuda.synchronize()
    for c, p, r in zip(cfgs, paths, refs):
        compare_all(c, p, r)
    # the counts path, interleaved the same way: each Path has its own workspace
    for p in paths:
        fill_sentinels(p)
    torch.cuda.synchronize()
    for _ in range(3):
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.layout_counts(b, stream=s)
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.dispatch_layout(b, stream=s)
        for p, b, s in zip(paths, batches, streams):
            with torch.cuda.stream(s):
                p.combine(b, stream=s)
    torch.cuda.synchronize()
    for c, p, r in zip(cfgs, paths, refs):
        compare_all(c, p, r)
