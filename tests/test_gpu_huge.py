"""Buffers past 2^31 16-byte words: a batch of 320 000 tokens (hidden 7168, 256 experts,
top-8, 64 ranks on 8 nodes). Its receive rows in use, its expert-major rows and the
highest rows of its per-node staging buffer all lie past 2^31 128-bit words (32 GiB),
so every row address of dispatch, the permute, the two-phase calls and combine must be
formed in 64 bits.

The oracle cannot copy 35 GB of rows in seconds, so the checks are:
  - every layout output in full;
  - every receive / expert-major row's routing, weight and source in full, and the first
    8 channels of every row, against the oracle run on x narrowed to those channels
    (routing never depends on the hidden size);
  - a sample of whole rows (random, the first and last rows, and the rows around the
    2^31-word boundary) against x[source] from the oracle's own source ids;
  - combine: the first 8 channels of every output row against the oracle on the narrowed
    rows, and whole rows of sampled tokens against the oracle run on those tokens alone
    (a token's combined row depends on nothing but its own routed rows).
x is `hidden_rows_indexed` (each row names its token), so a misplaced row shows."""
import numpy as np
import pytest
import torch

import oracle
import combine_ep_get_03_amd as ep
from combine_ep_get_03_amd import workloads as W
from combine_ep_get_03_amd.buffers import LayoutBuffers
from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

from gpu_util import SENT_I64, SENT_U16, fill_sentinels, host

pytestmark = pytest.mark.gpu

T, H, E, K, R, N, P = 320_000, 7168, 256, 8, 64, 8, 32
V = H // 8               # 128-bit words per row
NARROW = 8
WORD_LIMIT = 1 << 31


@pytest.fixture(scope="module")
def big():
    if torch.cuda.get_device_properties(0).total_memory < (160 << 30):
        pytest.skip("needs a GPU with at least 160 GiB")
    print(f"\ncase: huge batch T={T} H={H} E={E} k={K} R={R} N={N}: drawing inputs", flush=True)
    rng = np.random.default_rng(20241)
    idx = W.routing_uniform(rng, T, E, K)
    w = W.gate_weights(rng, T, K)
    prob = rng.random((T, N, P), dtype=np.float32)
    x = W.hidden_rows_indexed(T, H)
    lay = oracle.layout(idx, E, R, N)
    return dict(idx=idx, w=w, prob=prob, x=x, lay=lay, xn=np.ascontiguousarray(x[:, :NARROW]))


def _rows_to_check(n_rows: int, rng) -> np.ndarray:
    """Random rows, the first and last ones, and those around the 2^31-word boundary."""
    b = WORD_LIMIT // V
    pick = set(rng.choice(n_rows, 384, replace=False).tolist())
    pick |= {0, 1, n_rows - 1, n_rows - 2}
    pick |= {r for r in range(b - 3, b + 4) if 0 <= r < n_rows}
    return np.array(sorted(pick), dtype=np.int64)


def _gather_rows(t: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    return host(t.index_select(0, torch.from_numpy(rows).to(t.device)).contiguous())


def _narrow(t: torch.Tensor, n: int) -> np.ndarray:
    return host(t[:n, :NARROW].contiguous())


def _token_sample(rng) -> np.ndarray:
    return np.array(sorted(set(rng.choice(T, 128, replace=False).tolist()) | {0, T - 1}),
                    dtype=np.int64)


@pytest.mark.parametrize("form", ["counts", "preprocess"])
def test_path_rows_past_2_31_words(big, form):
    """Both step forms: the counts path (ep_layout_counts + ep_dispatch_layout) and the
    preprocess path (ep_dispatch_preprocess + ep_dispatch)."""
    lay, x, idx, w = big["lay"], big["x"], big["idx"], big["w"]
    M = int(lay["rank_offset"][-1])
    assert M * V > WORD_LIMIT
    print(f"case: huge path ({form}) M={M} ({M * V / WORD_LIMIT:.2f} x 2^31 words)", flush=True)
    b = DeviceBatch.from_host(idx, w, x, big["prob"])
    path = Path(T, H, E, K, R, N, P, T)
    fill_sentinels(path)
    path.step_counts(b) if form == "counts" else path.step_preprocess(b)
    torch.cuda.synchronize()
    L = path.layout_buf
    assert int(host(L.error_flag)[0]) == 0
    for name, t in (("count_r", L.num_tokens_per_rank), ("count_n", L.num_tokens_per_node),
                    ("count_e", L.num_tokens_per_expert), ("in_rank", L.is_token_in_rank),
                    ("rank_offset", L.rank_offset), ("expert_offset", L.expert_offset),
                    ("token_slot", L.token_slot)):
        np.testing.assert_array_equal(host(t), lay[name], err_msg=name)

    if "d" not in big:
        big["d"] = oracle.dispatch(big["xn"], idx, w, E, R, lay["token_slot"], M)
    d = big["d"]
    r = path.recv
    np.testing.assert_array_equal(_narrow(r.recv_x, M), d["recv_x"])
    np.testing.assert_array_equal(host(r.recv_topk_idx[:M]), d["recv_idx"])
    np.testing.assert_array_equal(host(r.recv_topk_weights[:M]).view(np.uint32),
                                  d["recv_w"].view(np.uint32))
    np.testing.assert_array_equal(host(r.recv_src_idx[:M]), d["recv_src"])
    rng = np.random.default_rng(5)
    rows = _rows_to_check(M, rng)
    np.testing.assert_array_equal(_gather_rows(r.recv_x, rows), x[d["recv_src"][rows]])
    # rows past M are not written
    tail = np.array([M, M + 1, path.cap - 1], dtype=np.int64)
    assert np.all(_gather_rows(r.recv_x, tail) == SENT_U16)
    assert np.all(host(r.recv_topk_idx[M:M + 2]) == SENT_I64)

    np.testing.assert_array_equal(host(path.prob_dest_major).view(np.uint32),
                                  oracle.restripe_prob(big["prob"], T).view(np.uint32))

    # combine of the dispatched rows
    np.testing.assert_array_equal(_narrow(path.out, T),
                                  oracle.combine(d["recv_x"], lay["token_slot"], R))
    ts = _token_sample(rng)
    sl = oracle.layout(idx[ts], E, R, N)
    sd = oracle.dispatch(x[ts], idx[ts], w[ts], E, R, sl["token_slot"], int(sl["rank_offset"][-1]))
    want = oracle.combine(sd["recv_x"], sl["token_slot"], R)
    np.testing.assert_array_equal(_gather_rows(path.out, ts), want)
    del path, b
    torch.cuda.empty_cache()


def test_permute_rows_past_2_31_words(big):
    x, idx, w = big["x"], big["idx"], big["w"]
    rows = T * K
    assert rows * V > WORD_LIMIT
    print(f"case: huge permute rows={rows}", flush=True)
    b = DeviceBatch.from_host(idx, w, x, big["prob"][:1])
    lbe = LayoutBuffers.alloc(T, E, R, N, k_expert_slots=K)
    lbe.compute(b.topk_idx, E, R, N)
    es = oracle.expert_slots(idx, E)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(lbe.expert_slot), es)
    px = torch.empty((rows, H), dtype=torch.bfloat16, device="cuda")
    pw = torch.empty(rows, dtype=torch.float32, device="cuda")
    ps = torch.empty(rows, dtype=torch.int32, device="cuda")
    ep.ep_dispatch_permute(b.x, b.topk_weights, lbe.expert_slot, perm_x=px, perm_weights=pw,
                           perm_src_idx=ps, error_flag=lbe.error_flag)
    torch.cuda.synchronize()
    assert int(host(lbe.error_flag)[0]) == 0
    want = oracle.dispatch_permute(big["xn"], idx, w, es, rows)
    np.testing.assert_array_equal(_narrow(px, rows), want["perm_x"])
    np.testing.assert_array_equal(host(pw).view(np.uint32), want["perm_w"].view(np.uint32))
    np.testing.assert_array_equal(host(ps), want["perm_src"])
    sample = _rows_to_check(rows, np.random.default_rng(6))
    np.testing.assert_array_equal(_gather_rows(px, sample), x[want["perm_src"][sample]])
    del px, pw, ps, lbe, b
    torch.cuda.empty_cache()


def test_two_phase_rows_past_2_31_words(big):
    lay, x, idx, w = big["lay"], big["x"], big["idx"], big["w"]
    M = int(lay["rank_offset"][-1])
    ns = oracle.node_slots(idx, E, R, N)
    routed = int((ns >= 0).sum())
    # staged rows sit at n * Tmax + slot: the last node's rows pass the boundary
    top = max(n * T + int(ns[:, n].max()) for n in range(N))
    assert (top + 1) * V > WORD_LIMIT
    print(f"case: huge two-phase routed={routed} M={M} top staged row {top}", flush=True)
    b = DeviceBatch.from_host(idx, w, x, big["prob"][:1])
    path = Path(T, H, E, K, R, N, P, T, node_slots=True)
    fill_sentinels(path)
    path.layout(b)
    hook = path.dispatch_send(b)
    hook()
    torch.cuda.synchronize()
    assert int(host(path.error_flag)[0]) == 0
    np.testing.assert_array_equal(host(path.layout_buf.node_slot), ns)
    if "d" not in big:
        big["d"] = oracle.dispatch(big["xn"], idx, w, E, R, lay["token_slot"], M)
    d = big["d"]
    r = path.recv
    np.testing.assert_array_equal(_narrow(r.recv_x, M), d["recv_x"])
    np.testing.assert_array_equal(host(r.recv_topk_idx[:M]), d["recv_idx"])
    np.testing.assert_array_equal(host(r.recv_src_idx[:M]), d["recv_src"])
    rng = np.random.default_rng(7)
    rows = _rows_to_check(M, rng)
    np.testing.assert_array_equal(_gather_rows(r.recv_x, rows), x[d["recv_src"][rows]])
    # staged rows: node n's row s holds x of the token staged there
    stage_rows = _rows_to_check(N * T, rng)
    st_src = host(path.stage.stage_src.reshape(-1)).astype(np.int64)
    ns_flat = np.full(N * T, -1, np.int64)
    tt, nn = np.nonzero(ns >= 0)
    ns_flat[nn * T + ns[tt, nn]] = tt
    np.testing.assert_array_equal(st_src[ns_flat >= 0], ns_flat[ns_flat >= 0])
    live = stage_rows[ns_flat[stage_rows] >= 0]
    np.testing.assert_array_equal(_gather_rows(path.stage.stage_x.reshape(N * T, H), live),
                                  x[ns_flat[live]])

    chook = path.combine_send(b)
    chook()
    torch.cuda.synchronize()
    assert int(host(path.error_flag)[0]) == 0
    stage = oracle.hook_combine_send(d["recv_x"], lay["token_slot"], R, ns, T)
    np.testing.assert_array_equal(_narrow(path.out, T), oracle.hook_combine_recv(stage, ns))
    ts = _token_sample(rng)
    sl = oracle.layout(idx[ts], E, R, N)
    sns = oracle.node_slots(idx[ts], E, R, N)
    sd = oracle.dispatch(x[ts], idx[ts], w[ts], E, R, sl["token_slot"], int(sl["rank_offset"][-1]))
    sst = oracle.hook_combine_send(sd["recv_x"], sl["token_slot"], R, sns, len(ts))
    np.testing.assert_array_equal(_gather_rows(path.out, ts), oracle.hook_combine_recv(sst, sns))
    del path, b
    torch.cuda.empty_cache()
