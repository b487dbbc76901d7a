"""Caller-built slot tables with more valid entries per row than the token's experts can
reach. The (token, destination) kernels launch min(k, C) destinations' worth of waves
per token; the token's last wave must take every destination past that, so each valid
entry still gets its row, exactly as the oracle (which writes every entry >= 0) does.
Covers the one-call dispatch, the FP8 dispatch (one and two destinations per wave) and
the two-phase send phase, with slot rows of one and two 64-column chunks."""
import numpy as np
import pytest
import torch

import oracle
import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd import workloads as W

from gpu_util import host

pytestmark = pytest.mark.gpu


def _column_slots(rng, T, C, p, per_column_base):
    """A random [T][C] table: entry (t, c) set with probability p; set entries are numbered
    in token order within a column, columns one after another (per_column_base=False), or
    from 0 in every column (True, the per-node staging rows)."""
    bm = rng.random((T, C)) < p
    slot = np.full((T, C), -1, np.int32)
    base = 0
    counts = bm.sum(axis=0)
    for c in range(C):
        rows = np.nonzero(bm[:, c])[0]
        slot[rows, c] = (0 if per_column_base else base) + np.arange(len(rows), dtype=np.int32)
        base += len(rows)
    return slot, int(base), counts


def _inputs(rng, T, H, E, k):
    cfg_rng = np.random.default_rng(int(rng.integers(1 << 30)))
    idx = W.routing_uniform(cfg_rng, T, E, k)
    w = cfg_rng.random((T, k), dtype=np.float32)
    x = W.hidden_rows(cfg_rng, T, H)
    return idx, w, x


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda")


CASES = [  # T, H, E, k, R
    (300, 128, 16, 2, 16),   # 2 waves per token, rows with up to 16 destinations
    (257, 256, 64, 8, 16),   # FP8: 4 waves of 2 destinations, the last open
    (130, 128, 96, 3, 96),   # slot rows of two 64-column chunks
]


@pytest.mark.parametrize("T,H,E,k,R", CASES)
def test_dispatch_and_fp8_take_every_valid_slot(T, H, E, k, R):
    print(f"\ncase: caller-built token_slot T={T} H={H} E={E} k={k} R={R}", flush=True)
    rng = np.random.default_rng(T * 1000 + R)
    idx, w, x = _inputs(rng, T, H, E, k)
    slot, M, _ = _column_slots(rng, T, R, 0.5, False)
    assert (slot >= 0).sum(axis=1).max() > min(k, R)
    ref = oracle.dispatch(x, idx, w, E, R, slot, M)
    fref = oracle.dispatch_fp8(x, idx, w, E, R, slot, M)
    xd = _dev(x.view(np.int16), torch.bfloat16)
    idd, wd, sd = _dev(idx), _dev(w), _dev(slot)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    rx = torch.full((M, H), 3.0, dtype=torch.bfloat16, device="cuda")
    ri = torch.full((M, k), -9, dtype=torch.int64, device="cuda")
    rw = torch.full((M, k), -9.0, dtype=torch.float32, device="cuda")
    rs = torch.full((M,), -9, dtype=torch.int32, device="cuda")
    ep.ep_dispatch(xd, idd, wd, E, R, sd, recv_x=rx, recv_topk_idx=ri, recv_topk_weights=rw,
                   recv_src_idx=rs, error_flag=flag)
    codes = torch.full((M, H), 0xA7, dtype=torch.uint8, device="cuda")
    scales = torch.full((M, H // 128), -1.0, dtype=torch.float32, device="cuda")
    fi = torch.full((M, k), -9, dtype=torch.int64, device="cuda")
    fw = torch.full((M, k), -9.0, dtype=torch.float32, device="cuda")
    fs = torch.full((M,), -9, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_fp8(xd, idd, wd, E, R, sd, recv_x_fp8=codes, recv_scales=scales,
                       recv_topk_idx=fi, recv_topk_weights=fw, recv_src_idx=fs, error_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    np.testing.assert_array_equal(host(rx), ref["recv_x"][:M])
    np.testing.assert_array_equal(host(ri), ref["recv_idx"][:M])
    np.testing.assert_array_equal(host(rw).view(np.uint32), ref["recv_w"][:M].view(np.uint32))
    np.testing.assert_array_equal(host(rs), ref["recv_src"][:M])
    np.testing.assert_array_equal(host(codes), fref["recv_codes"][:M])
    np.testing.assert_array_equal(host(scales).view(np.uint32), fref["recv_scales"][:M].view(np.uint32))
    np.testing.assert_array_equal(host(fi), fref["recv_idx"][:M])
    np.testing.assert_array_equal(host(fw).view(np.uint32), fref["recv_w"][:M].view(np.uint32))
    np.testing.assert_array_equal(host(fs), fref["recv_src"][:M])


def test_send_takes_every_valid_node_slot():
    # k = 2 over 8 nodes: 2 waves per token, rows naming up to 8 nodes
    T, H, E, k, R, N = 400, 64, 32, 2, 16, 8
    print(f"\ncase: caller-built node_slot T={T} k={k} N={N}", flush=True)
    rng = np.random.default_rng(7)
    idx, w, x = _inputs(rng, T, H, E, k)
    ns, _, counts = _column_slots(rng, T, N, 0.6, True)
    assert (ns >= 0).sum(axis=1).max() > min(k, N)
    Tmax = T
    ref = oracle.hook_dispatch_send(x, idx, w, ns, Tmax)
    sx = torch.full((N, Tmax, H), 3.0, dtype=torch.bfloat16, device="cuda")
    si = torch.full((N, Tmax, k), -9, dtype=torch.int64, device="cuda")
    sw = torch.full((N, Tmax, k), -9.0, dtype=torch.float32, device="cuda")
    ss = torch.full((N, Tmax), -9, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_send(_dev(x.view(np.int16), torch.bfloat16), _dev(idx), _dev(w), _dev(ns),
                        stage_x=sx, stage_topk_idx=si, stage_topk_weights=sw, stage_src=ss,
                        error_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    for n in range(N):
        c = int(counts[n])
        np.testing.assert_array_equal(host(sx[n, :c]), ref["stage_x"][n, :c])
        np.testing.assert_array_equal(host(si[n, :c]), ref["stage_idx"][n, :c])
        np.testing.assert_array_equal(host(sw[n, :c]).view(np.uint32), ref["stage_w"][n, :c].view(np.uint32))
        np.testing.assert_array_equal(host(ss[n, :c]), ref["stage_src"][n, :c])
        assert bool((ss[n, c:] == -9).all())
