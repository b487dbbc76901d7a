"""Pins for the oracle's FP8 path: the e4m3 encoder against torch's float8_e4m3fn
conversion and a nearest-even choice on the e4m3 grid written from the format's
definition; quantisation invariants; FP8 dispatch against the bf16 dispatch."""
import numpy as np
import pytest
import torch

from combine_ep_get_03_amd import workloads as W


def grid_values():
    """Every finite e4m3 value from the format definition: bias 7, 3 mantissa bits,
    exponent field 0 subnormal, field 15 with mantissa 7 reserved for NaN."""
    vals = {}
    for code in range(256):
        s, ef, m = code >> 7, (code >> 3) & 15, code & 7
        if ef == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0**-6 if ef == 0 else (1 + m / 8.0) * 2.0**(ef - 7)
        vals[code] = -v if s else v
    return vals


def nearest_even(v, vals):
    """Nearest finite e4m3 value (ties to the even code), saturated at +-448."""
    codes = np.array(sorted(vals, key=lambda c: (vals[c], c)))
    grid = np.array([vals[c] for c in codes])
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.astype(np.float64)):
        x = min(max(x, -448.0), 448.0)
        d = np.abs(grid - x)
        best = np.flatnonzero(d == d.min())
        cands = codes[best]
        if any(grid[b] == 0.0 for b in best):
            # the zero codes are even, so any tie with zero goes to zero, which keeps
            # the input's sign (-0 is code 0x80)
            out[i] = 0x80 if np.signbit(x) else 0x00
            continue
        if len(cands) > 1:
            cands = [c for c in cands if (c & 1) == 0]
        out[i] = cands[0]
    return out


def test_grid_has_the_formats_landmarks():
    vals = grid_values()
    assert max(vals.values()) == 448.0 and vals[0x7E] == 448.0
    assert vals[0x08] == 2.0**-6 and vals[0x01] == 2.0**-9 and vals[0x38] == 1.0
    assert len(vals) == 254


def test_e4m3_vs_torch(orc):
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(-463.9, 463.9, 200000).astype(np.float32),
        (rng.standard_normal(100000) * 2.0**rng.integers(-14, 8, 100000)).astype(np.float32),
        np.float32([0.0, -0.0, 448.0, -448.0, 464.0, -464.0, 2**-9, 2**-10, 3 * 2**-11]),
    ])
    # exact midpoints between neighbouring grid values (ties)
    g = np.array(sorted(set(abs(x) for x in grid_values().values())))
    mids = ((g[1:] + g[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.f32_to_e4m3(v), want)


def test_e4m3_vs_grid_nearest_even(orc):
    rng = np.random.default_rng(1)
    vals = grid_values()
    g = np.array(sorted(set(abs(x) for x in vals.values())))
    mids = (g[1:] + g[:-1]) / 2
    v = np.concatenate([rng.uniform(-500, 500, 3000), mids, -mids, g, -g,
                        rng.uniform(-2**-5, 2**-5, 2000), [1000.0, -1e6]]).astype(np.float32)
    np.testing.assert_array_equal(orc.f32_to_e4m3(v), nearest_even(v, vals))


def test_decode_matches_grid(orc):
    vals = grid_values()
    dec = orc.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    for c, v in vals.items():
        assert dec[c] == np.float32(v)
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])


def test_quantize_invariants(orc):
    cfg = W.CONFIGS["dsv3"].with_(T=200)
    x = W.make_inputs(cfg, with_partials=False, with_prob=False).x
    x = x.copy()
    x[7, 128:256] = 0                           # an all-zero group
    codes, scales = orc.quantize_fp8(x)
    xf = orc.bf16_to_f32(x).astype(np.float64).reshape(cfg.T, -1, 128)
    amax = np.abs(xf).max(axis=2)
    deq = orc.e4m3_to_f32(codes).astype(np.float64).reshape(cfg.T, -1, 128)
    # scale = amax / 448 in fp32; zero groups get 1
    np.testing.assert_array_equal(scales, np.where(amax > 0, (amax.astype(np.float32) / np.float32(448)), 1).astype(np.float32))
    # the group maximum lands on +-448
    nz = amax > 0
    assert np.all(np.abs(deq).max(axis=2)[nz] == 448.0)
    assert np.all(codes.reshape(cfg.T, -1, 128)[~nz] == 0)
    # reconstruction within half an e4m3 step (relative 2^-4 for normals, 2^-10 absolute
    # in scaled units for subnormals)
    recon = deq * scales[:, :, None].astype(np.float64)
    err = np.abs(recon - xf)
    bound = np.maximum(np.abs(xf) * 2.0**-4, 2.0**-10 * scales[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantize_rejects_ragged_hidden(orc):
    with pytest.raises(ValueError):
        orc.quantize_fp8(np.zeros((2, 100), np.uint16))


@pytest.mark.parametrize("name", ["tiny", "dsv3", "skewed"])
def test_fp8_dispatch_is_quantize_then_permute(orc, name):
    cfg = W.CONFIGS[name].with_(T=300)
    inp = W.make_inputs(cfg, with_partials=False, with_prob=False)
    lay = orc.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    d = orc.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], cfg.cap)
    f = orc.dispatch_fp8(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], cfg.cap)
    codes, scales = orc.quantize_fp8(inp.x)
    src = d["recv_src"][:M]
    np.testing.assert_array_equal(f["recv_codes"][:M], codes[src])
    np.testing.assert_array_equal(f["recv_scales"][:M], scales[src])
    for key in ("recv_idx", "recv_w", "recv_src"):
        np.testing.assert_array_equal(f[key][:M], d[key][:M])
    assert not f["recv_codes"][M:].any()
    # FP8 rows carry H + 4 H / 128 bytes instead of 2 H
    assert f["recv_codes"].shape[1] + 4 * f["recv_scales"].shape[1] == cfg.H + cfg.H // 32
