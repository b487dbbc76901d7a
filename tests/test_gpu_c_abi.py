"""The C ABI driven from plain C (tests/c_abi/ep_c_smoke.c): device buffers from the
HIP runtime, the path on one stream as the four calls and as the counts path
(ep_layout_counts, ep_dispatch_layout, ep_combine), every output compared bit for bit with
the oracle inside the program."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_matches_the_oracle():
    exe = os.path.join(HERE, "c_abi", "ep_c_smoke")
    if not os.path.exists(exe):
        import __graft_entry__

        __graft_entry__._build_c_consumer()
    print("\ncase: C ABI program (T=256, H=1024, E=16, top-4, R=4, N=2)", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0
    assert "four calls ok" in r.stdout and "counts path ok" in r.stdout
    assert "one launch ok" in r.stdout
