"""The measurement helpers behind the bench's yardsticks move exactly the bytes they
claim: the copy writes dst[:n] = src[:n] and nothing past it, the fan writes the XOR of
its input slabs into every output slab and nothing past them, and the spread writes into
each output chunk the XOR of its input chunks under the region mapping. The copy and the
fan are checked at sizes that end inside a block's share and in a whole number of
blocks."""
import numpy as np
import pytest
import torch

import combine_ep_get_03_amd as ep

pytestmark = pytest.mark.gpu

SENT = 0x6B


def _rand_bytes(n, seed):
    g = np.random.default_rng(seed)
    return torch.from_numpy(g.integers(0, 256, n, dtype=np.uint8)).cuda()


# 16 KiB is one copy block's share (256 threads x 4 words of 16 bytes)
@pytest.mark.parametrize("nbytes", [16, 16 * 255, 16 * 1024, 16 * 1025 + 16 * 7,
                                    16 * 1024 * 37 + 48, (64 << 20) + 16])
def test_copy_moves_exactly_n_bytes(nbytes):
    print(f"\ncase: ep_hbm_copy {nbytes} bytes", flush=True)
    src = _rand_bytes(nbytes + 4096, nbytes)
    dst = torch.full((nbytes + 4096,), SENT, dtype=torch.uint8, device="cuda")
    ep.ep_hbm_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert bool((dst[nbytes:] == SENT).all())


def test_copy_of_zero_bytes_writes_nothing():
    src = _rand_bytes(64, 1)
    dst = torch.full((64,), SENT, dtype=torch.uint8, device="cuda")
    ep.ep_hbm_copy(src, dst, 0)
    torch.cuda.synchronize()
    assert bool((dst == SENT).all())


@pytest.mark.parametrize("fan_in,fan_out", [(7, 1), (8, 1), (1, 7), (1, 8), (2, 1), (1, 2),
                                            (1, 1), (4, 3), (4, 8), (12, 1), (9, 2), (16, 1)])
@pytest.mark.parametrize("slab", [16 * 3001, 16 * 1024 * 3])
def test_fan_writes_the_xor_of_its_slabs(fan_in, fan_out, slab):
    print(f"\ncase: ep_hbm_fan {fan_in}:{fan_out} slab {slab}", flush=True)
    src = _rand_bytes(fan_in * slab, fan_in * 31 + fan_out + slab)
    dst = torch.full((fan_out * slab + 4096,), SENT, dtype=torch.uint8, device="cuda")
    ep.ep_hbm_fan(src, dst, slab, fan_in, fan_out)
    torch.cuda.synchronize()
    s = src.cpu().numpy().reshape(fan_in, slab)
    want = np.bitwise_xor.reduce(s, axis=0)
    d = dst.cpu().numpy()
    for j in range(fan_out):
        np.testing.assert_array_equal(d[j * slab:(j + 1) * slab], want, err_msg=f"slab {j}")
    assert bool((d[fan_out * slab:] == SENT).all())


@pytest.mark.parametrize("fan_in,regions,nchunks", [(7, 32, 64), (8, 32, 64), (7, 7, 48),
                                                    (8, 8, 48), (1, 1, 5), (3, 1, 7),
                                                    (5, 64, 64), (7, 28, 4)])
def test_spread_writes_the_xor_of_its_chunks(fan_in, regions, nchunks):
    print(f"\ncase: ep_hbm_spread fan_in {fan_in} regions {regions} chunks {nchunks}", flush=True)
    C = ep.EP_HBM_SPREAD_CHUNK_BYTES
    out_bytes = nchunks * C
    src = _rand_bytes(fan_in * out_bytes, fan_in * 131 + regions + nchunks)
    dst = torch.full((out_bytes + 4096,), SENT, dtype=torch.uint8, device="cuda")
    ep.ep_hbm_spread(src, dst, out_bytes, fan_in, regions)
    torch.cuda.synchronize()
    # input chunk j is chunk j // regions of region j % regions
    s = src.cpu().numpy().reshape(regions, fan_in * nchunks // regions, C)
    want = np.zeros((nchunks, C), dtype=np.uint8)
    for b in range(nchunks):
        for q in range(fan_in):
            j = fan_in * b + q
            want[b] ^= s[j % regions, j // regions]
    d = dst.cpu().numpy()
    np.testing.assert_array_equal(d[:out_bytes].reshape(nchunks, C), want)
    assert bool((d[out_bytes:] == SENT).all())
