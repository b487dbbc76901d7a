"""Pins for the oracle's bf16 rounding and combine.

* bf16 round-to-nearest-even against torch's conversion (a library routine) and
  against a nearest-by-distance choice made in float64;
* combine against exact sums (small-integer partials), the round-trip closed
  form out = bf16(c_t * x_t) with c_t the token's rank count, the single-rank
  case, and an fp64 sum within the fp32 accumulation error bound.
"""
import numpy as np
import pytest
import torch

from combine_ep_get_03_amd import workloads as W


def torch_bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def nearest_even_by_distance(a):
    """Pick the closer of the two neighbouring bf16 values in float64; on a tie
    the one with an even last bit."""
    a = np.asarray(a, np.float32)
    u = a.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)                     # truncation toward zero
    hi = lo + 1
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = a.astype(np.float64)
    dlo, dhi = np.abs(x - f(lo)), np.abs(f(hi) - x)
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo & 1) == 1))
    return np.where(pick_hi, hi, lo).astype(np.uint16)


def test_bf16_rounding_vs_torch_and_distance(orc):
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),    # subnormals
        rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    a = a[np.isfinite(a)]
    # exact ties: low half exactly 0x8000, both parities
    ties = ((rng.integers(0, 0x7F80, 5000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, np.float32([0.0, -0.0, 1.0, 3.3895314e38, -3.3895314e38])])
    got = orc.f32_to_bf16(a)
    np.testing.assert_array_equal(got, torch_bf16(a))
    finite = np.abs(a) < 3.3e38
    np.testing.assert_array_equal(got[finite], nearest_even_by_distance(a[finite]))


def test_bf16_special_values(orc):
    inf = np.float32(np.inf)
    got = orc.f32_to_bf16(np.float32([inf, -inf, np.nan, 3.4028235e38]))
    assert got[0] == 0x7F80 and got[1] == 0xFF80
    assert (got[2] & 0x7F80) == 0x7F80 and (got[2] & 0x7F) != 0 and (got[2] & 0x40)
    assert got[3] == 0x7F80  # FLT_MAX rounds up to +inf


def _routed(cfg):
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    return inp


def test_small_integer_partials_are_exact(orc):
    """Partials in {-4..4} sum exactly in fp32 and the sum fits bf16 exactly."""
    cfg = W.CONFIGS["dsv3"].with_(T=300, H=40)
    inp = _routed(cfg)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    vals = np.random.default_rng(5).integers(-4, 5, size=(M, cfg.H)).astype(np.float32)
    partial = torch_bf16(vals)
    out = orc.combine(partial, lay["token_slot"], cfg.R)
    s = lay["token_slot"]
    exact = np.zeros((cfg.T, cfg.H), np.float64)
    for t in range(cfg.T):
        for r in range(cfg.R):
            if s[t, r] >= 0:
                exact[t] += vals[s[t, r]]
    np.testing.assert_array_equal(out, torch_bf16(exact.astype(np.float32)))


@pytest.mark.parametrize("name,kw", [("large", dict(T=512, H=256)), ("dsv3", dict(T=256, H=128)),
                                     ("tiny", {})])
def test_round_trip_closed_form(orc, name, kw):
    """partial = dispatched rows: sum over ranks = c_t * x_t, exact in fp32 (8 significant
    bits times c_t <= 8 needs at most 11), so out = bf16(c_t * x_t) bit for bit."""
    cfg = W.CONFIGS[name].with_(**kw)
    inp = _routed(cfg)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    d = orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"],
                     cfg.cap)
    out = orc.combine(d["recv_x"], lay["token_slot"], cfg.R)
    c = (lay["token_slot"] >= 0).sum(1).astype(np.float32)
    xf = orc.bf16_to_f32(inp.x)
    np.testing.assert_array_equal(out, torch_bf16(c[:, None] * xf))


def test_single_rank_returns_partial(orc):
    T, H = 64, 32
    slot = np.arange(T, dtype=np.int32)[::-1].copy().reshape(T, 1)
    partial = torch_bf16(np.random.default_rng(9).standard_normal((T, H)))
    out = orc.combine(partial, slot, 1)
    np.testing.assert_array_equal(out, partial[slot[:, 0]])


def test_random_partials_within_fp32_bound(orc):
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    out = orc.combine(inp.partials, lay["token_slot"], cfg.R)
    s = lay["token_slot"]
    pf = orc.bf16_to_f32(inp.partials).astype(np.float64)
    S = np.zeros((cfg.T, cfg.H))
    A = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        rows = s[t][s[t] >= 0]
        S[t] = pf[rows].sum(0)
        A[t] = np.abs(pf[rows]).sum(0)
    m = (s >= 0).sum(1)[:, None]
    got = orc.bf16_to_f32(out).astype(np.float64)
    bound = (m - 1) * 2.0**-24 * A + 2.0**-8 * np.abs(got) + 1e-45
    assert np.all(np.abs(got - S) <= bound)


def test_no_rank_gives_positive_zero(orc):
    slot = np.array([[-1, -1], [0, -1]], np.int32)
    partial = np.array([[0x3F80, 0xBF80]], np.uint16)
    out = orc.combine(partial, slot, 2)
    assert out.tolist() == [[0, 0], [0x3F80, 0xBF80]]


def test_slot_beyond_rows_rejected(orc):
    with pytest.raises(ValueError):
        orc.combine(np.zeros((2, 4), np.uint16), np.array([[2]], np.int32), 1)
