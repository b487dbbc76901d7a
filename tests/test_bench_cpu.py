"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the algorithmic
byte counts (cross-checked against the sizes of the arrays each call reads and writes),
the counter-traffic lookup and its source-hash guard, and the CPU-baseline record."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from combine_ep_get_03_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_zero_steps_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--steps" in r.stderr and r.stdout == ""


def _nbytes(*arrays):
    return sum(a.nbytes for a in arrays)


def test_algorithmic_bytes_match_the_arrays_each_call_touches():
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg)
    lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
    M = int(lay["rank_offset"][-1])
    d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R, lay["token_slot"], M)
    rs = oracle.restripe_prob(inp.prob, cfg.Tmax)
    out = oracle.combine(inp.partials, lay["token_slot"], cfg.R)
    alg = bench.algorithmic_bytes(cfg, M)
    # layout: reads the ids; writes the bitmap, the slots, the three count vectors and the
    # error flag (the offsets are prefix sums of the counts, not counted again)
    assert alg["layout"] == _nbytes(inp.topk_idx, lay["in_rank"], lay["token_slot"],
                                    lay["count_r"], lay["count_n"], lay["count_e"],
                                    lay["error_flag"])
    # dispatch: reads x, ids, weights and slots; writes M receive rows with their metadata
    assert alg["dispatch"] == _nbytes(inp.x, inp.topk_idx, inp.topk_weights, lay["token_slot"],
                                      d["recv_x"], d["recv_idx"], d["recv_w"], d["recv_src"])
    # restripe: the T*N*P words in, the same words out (rows past T are not written)
    assert alg["restripe"] == inp.prob.nbytes + rs[:, :cfg.T].nbytes
    # combine: reads the slots and M partial rows, writes T output rows
    assert alg["combine"] == lay["token_slot"].nbytes + inp.partials[:M].nbytes + out.nbytes


def test_measured_traffic_is_guarded_by_the_source_hash(tmp_path, monkeypatch):
    assert bench.measured_traffic("dispatch", "no_such_workload") is None
    h = hashlib.sha256()
    for f in bench.KERNEL_SOURCES["dispatch"]:
        with open(os.path.join(ROOT, "combine_ep_get_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "dsv3_hbm_counters.md").write_text(
        f"traffic dispatch bytes_per_launch=123456 sources_sha256={h.hexdigest()[:16]}\n")
    assert bench.measured_traffic("dispatch", "dsv3") == 123456
    assert bench.measured_traffic("dispatch", "large") is None
    (tmp_path / "large_hbm_counters.md").write_text(
        "traffic dispatch bytes_per_launch=123456 sources_sha256=0000000000000000\n")
    assert bench.measured_traffic("dispatch", "large") is None


@pytest.mark.parametrize("workload", ["dsv3", "skewed", "large"])
def test_committed_counters_agree_with_the_algorithmic_bytes(workload):
    # Where a committed counter summary matches today's sources, its calibrated bytes per
    # launch are within 2% of what the kernel is expected to move. Combine: its algorithmic
    # bytes. Dispatch: its algorithmic bytes plus one more fetch of what a token's waves
    # read (row, routing and slot row), because a top-8 token's waves fill two 256-thread
    # blocks, which the hardware places on two XCDs, and each XCD's L2 fetches them.
    cfg = W.CONFIGS[workload]
    inp = W.make_inputs(cfg, with_x=False)
    M = int(oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)["rank_offset"][-1])
    second_fetch = cfg.T * cfg.H * 2 + cfg.T * cfg.k * 12 + cfg.T * cfg.R * 4
    assert min(cfg.k, cfg.R) == 8  # two blocks of four waves per token
    extra = {"dispatch": second_fetch, "combine": 0}
    checked = 0
    for k in ("dispatch", "combine"):
        v = bench.measured_traffic(k, workload)
        if v is None:
            continue
        want = bench.algorithmic_bytes(cfg, M)[k] + extra[k]
        assert 0.98 * want <= v <= 1.02 * want, (k, v, want)
        checked += 1
    if checked == 0:
        pytest.skip(f"{workload}: no counter summary matches the current kernel sources")


def test_cpu_baseline_record():
    cfg = W.CONFIGS["tiny"]
    inp = W.make_inputs(cfg)
    rec = bench.cpu_baseline(cfg, inp, 0.05)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s" and rec["cores"] == 1
    assert rec["value"] > 0 and "tiny" in rec["sample"] and rec["ms_per_step"] > 0
    M = int(oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)["rank_offset"][-1])
    assert np.isclose(rec["value"], 2 * M * cfg.H * 2 / (rec["ms_per_step"] * 1e-3) / 1e9, rtol=0.01)
