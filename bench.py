"""Benchmark of the single-GPU EP dispatch/combine path on one MI355X.

One step = the whole path on one batch: ep_dispatch_preprocess (the layout and the
restripe of prob in one call) -> ep_dispatch -> ep_combine, enqueued on one stream. The K
timed steps run as one HIP graph of K steps. The same step as one call per step
(ep_get_layout -> ep_dispatch -> ep_restripe_prob -> ep_combine) is timed beside it.
Inputs are seeded synthetic data already resident in HBM when the timed region starts.
Prints one JSON line.

value = dispatch+combine algorithm GB/s over the whole step: (2 * M * H * 2 bytes) / step
time, where M = number of (token, rank) pairs (each token's row counted once per
destination rank, the pages' "algorithm bandwidth" taken at rank granularity).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine algorithm GB/s and tokens/s on 1 MI355X; % of HBM roofline"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's CPU time for the baseline")
    ap.add_argument("--copy-gib", default="2,4",
                    help="comma-separated copy sizes in GiB; the best rate is the yardstick")
    ap.add_argument("--small-batches", action="store_true",
                    help="also time the whole step at 256 and 1024 tokens of the same shape")
    ap.add_argument("--flush-gib", type=float, default=1.0,
                    help="scratch written before each cold launch (evicts L2 and the 256 MB "
                         "Infinity Cache)")
    return ap.parse_args()


def algorithmic_bytes(cfg, M: int) -> dict:
    """Minimum bytes each kernel must move (reads + writes)."""
    T, H, k, R, N, P, E = cfg.T, cfg.H, cfg.k, cfg.R, cfg.N, cfg.P, cfg.E
    return {
        "layout": T * k * 8 + T * R * (1 + 4) + (R + N + E + 1) * 4,
        "dispatch": T * H * 2 + T * k * 12 + T * R * 4 + M * (2 * H + 12 * k + 4),
        "restripe": 2 * T * N * P * 4,
        "combine": T * R * 4 + M * H * 2 + T * H * 2,
        # the counts path: the counting pass with the restripe in one launch, then the
        # dispatch that also writes the slot table, the bitmap and the rank, node and expert
        # counts and offsets
        "layout_counts": T * k * 8 + 2 * T * N * P * 4,
        "dispatch_layout": (T * H * 2 + T * k * 12 + M * (2 * H + 12 * k + 4) +
                            T * R * (1 + 4) + (2 * R + 1 + N + 2 * E + 1) * 4),
    }


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"dispatch": ["ep_internal.hpp", "dispatch_rows.hpp", "dispatch.hip"],
                  "combine": ["ep_internal.hpp", "combine.hip"]}


def counters_file(workload: str) -> str:
    return os.path.join(PROFILES, f"{workload}_hbm_counters.md")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary of this workload
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel of known size), or None when no
    summary covers the workload or the kernel's sources changed since the counters were
    taken."""
    import hashlib

    path = counters_file(workload)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_ep_get_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel:
                fields = dict(p.split("=", 1) for p in parts[2:])
                if fields.get("sources_sha256") == h.hexdigest()[:16]:
                    return int(fields["bytes_per_launch"])
    return None


def copy_bandwidth(torch, ep, sizes_gib):
    """The library's 128-bit copy kernel and torch's device copy at each size (all far
    above the 256 MB Infinity Cache), read+write bytes; the caller takes the best."""
    res = {}
    for gib in sizes_gib:
        res.update(_copy_at(torch, ep, gib))
    return res


def _copy_at(torch, ep, gib: float):
    n = int(gib * (1 << 30)) // 16 * 16
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    res = {}
    tag = f"{gib:g}GiB"
    for name, fn in ((f"ep_hbm_copy_{tag}", lambda: ep.ep_hbm_copy(a, b)),
                     (f"torch_copy_{tag}", lambda: b.copy_(a))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        res[name] = 2 * n / (ms * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(cfg, inp, seconds: float) -> dict:
    """The CPU oracle on this host, single thread, whole step on the same batch;
    repeated until `seconds` of CPU time (at least three times). `value` is taken at the
    median step time."""
    import statistics

    import oracle

    times = []
    M = None
    while len(times) < 3 or sum(times) < seconds:
        t0 = time.perf_counter()
        lay = oracle.layout(inp.topk_idx, cfg.E, cfg.R, cfg.N)
        d = oracle.dispatch(inp.x, inp.topk_idx, inp.topk_weights, cfg.E, cfg.R,
                            lay["token_slot"], cfg.cap)
        oracle.restripe_prob(inp.prob, cfg.Tmax)
        partial = d["recv_x"] if inp.partials is None else inp.partials
        oracle.combine(partial, lay["token_slot"], cfg.R)
        times.append(time.perf_counter() - t0)
        M = int(lay["rank_offset"][-1])
        del d
    s = statistics.median(times)
    return {"value": round(2 * M * cfg.H * 2 / s / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(times)} whole steps (layout+dispatch+restripe+combine) of the "
                      f"{cfg.name} batch, median {s * 1e3:.1f} ms each, single-threaded C oracle "
                      f"incl. its output allocation; host {cpu_model()}, nproc {os.cpu_count()}",
            "ms_per_step": round(s * 1e3, 2),
            "ms_per_step_min_max": [round(min(times) * 1e3, 2), round(max(times) * 1e3, 2)],
            "host_cpu": cpu_model(), "nproc": os.cpu_count()}


def launch_distribution(torch, ep, calls: dict, reps: int, flush_gib: float) -> dict:
    """Time of single launches, `reps` of each call: an event pair around one launch, and
    before it on the same stream a cushion long enough that the host has queued the events
    and the launch by the time the GPU reaches them (so host launch cost stays outside the
    pair). Warm: the cushion is a ~100 us spin that touches no memory, so what the previous
    launch left in L2 and the Infinity Cache stays there. Cold: the cushion is a copy
    through `flush_gib` GiB of scratch, which evicts both. Median, p10 and p90 in us; the
    floor is the same measurement around a 16-byte copy (event and dispatch latency that
    every single-launch figure includes)."""
    import numpy as np

    stream = torch.cuda.current_stream()
    # spin cycles per microsecond of the sleep kernel, measured here
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cyc = 1 << 22
    torch.cuda._sleep(cyc)
    s0.record(stream)
    torch.cuda._sleep(cyc)
    s1.record(stream)
    torch.cuda.synchronize()
    spin = max(1, int(cyc / max(s0.elapsed_time(s1) * 1e3, 1.0) * 100.0))
    nflush = int(flush_gib * (1 << 30)) // 32 * 16
    scratch = torch.empty(2 * nflush, dtype=torch.uint8, device="cuda")
    scratch.fill_(0)
    tiny = torch.zeros(32, dtype=torch.uint8, device="cuda")

    def cushion(cold):
        if cold:
            ep.ep_hbm_copy(scratch[:nflush], scratch[nflush:])
        else:
            torch.cuda._sleep(spin)

    def sample(fn, cold):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        fn()
        torch.cuda.synchronize()
        for a, b_ in ev:
            cushion(cold)
            a.record(stream)
            fn()
            b_.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b_) * 1e3 for a, b_ in ev])
        return {"median_us": round(float(np.median(us)), 2),
                "p10_us": round(float(np.percentile(us, 10)), 2),
                "p90_us": round(float(np.percentile(us, 90)), 2)}

    out = {"reps": reps, "flush_bytes": 2 * nflush,
           "event_floor_us": sample(lambda: ep.ep_hbm_copy(tiny[:16], tiny[16:]), False)["median_us"]}
    for mode, cold in (("warm", False), ("cold", True)):
        out[mode] = {n: sample(fn, cold) for n, fn in calls.items()}
    del scratch, tiny
    torch.cuda.empty_cache()
    return out


def hook_section(torch, cfg, b, args, timed, M: int) -> dict:
    """Two-phase dispatch/combine: each phase's average launch time (a graph of K launches),
    send + receive (the pages' hook-mode kernel time), and the send phase overlapped with
    a 4096 x 4096 x 4096 bf16 GEMM on a second stream against the two run back to back."""
    from combine_ep_get_03_amd.pipeline import Path

    hp = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax, node_slots=True)
    hp.layout(b)
    torch.cuda.synchronize()
    routed = int(hp.layout_buf.num_tokens_per_node.sum().item())
    holder = {}

    def d_send():
        holder["d"] = hp.dispatch_send(b)

    def c_send():
        holder["c"] = hp.combine_send(b)

    d_send()
    holder["d"]()
    c_send()
    res = {}
    for n, fn in (("dispatch_send", d_send), ("dispatch_recv", lambda: holder["d"]()),
                  ("combine_send", c_send), ("combine_recv", lambda: holder["c"]())):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                fn()
        g.replay()
        res[n] = timed(g.replay, 1) / args.steps
        del g
    if int(hp.error_flag.item()) != 0:
        raise RuntimeError("device error flag in the two-phase calls")
    T, H, k, N, R = cfg.T, cfg.H, cfg.k, cfg.N, cfg.R
    row = 2 * H + 12 * k + 4
    alg = {"dispatch_send": T * H * 2 + T * k * 12 + T * N * 4 + routed * row,
           "dispatch_recv": routed * row + routed * (R // N) * 4 + N * 4 + M * row,
           "combine_send": T * R * 4 + T * N * 4 + M * 2 * H + routed * 2 * H,
           "combine_recv": T * N * 4 + routed * 2 * H + T * 2 * H}

    # Overlap: K iterations of the send phase on one stream and the GEMM on another,
    # against the two run back to back. The send's stream has a hardware queue of its own
    # (HIP spreads plain streams over a few queues in turn, and two streams on one queue
    # run their kernels one after the other). The send runs on the full grid and on a
    # budget of SEND_BUDGET workgroups, which leaves room for the GEMM on every CU.
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    w = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(4096, 4096, device="cuda", dtype=torch.bfloat16)
    comm, comm_handle = dedicated_queue_stream(torch)
    comp = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def gemm():
        torch.matmul(a, w, out=c)

    for _ in range(3):
        gemm()
    gemm_ms = timed(gemm, args.steps)

    def send_alone(budget):
        with torch.cuda.stream(comm):
            hp.dispatch_send(b, stream=comm, num_workgroups=budget)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(comm)
            for _ in range(args.steps):
                hp.dispatch_send(b, stream=comm, num_workgroups=budget)
            e1.record(comm)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def overlapped(reps, budget):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(main)
        comm.wait_stream(main)
        comp.wait_stream(main)
        for _ in range(reps):
            with torch.cuda.stream(comm):
                hp.dispatch_send(b, stream=comm, num_workgroups=budget)
            with torch.cuda.stream(comp):
                gemm()
        main.wait_stream(comm)
        main.wait_stream(comp)
        s1.record(main)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    ov = {"gemm_4096_bf16_us": round(gemm_ms * 1e3, 2), "send_stream": "own hardware queue"}
    for tag, budget in (("full_grid", 0), (f"{SEND_BUDGET}_workgroups", SEND_BUDGET)):
        send_ms = send_alone(budget)
        overlapped(3, budget)
        ov_ms = min(overlapped(args.steps, budget) for _ in range(3))
        ov[tag] = {"send_us": round(send_ms * 1e3, 2),
                   "serial_us": round((gemm_ms + send_ms) * 1e3, 2),
                   "send_with_gemm_on_two_streams_us": round(ov_ms * 1e3, 2),
                   "ratio_to_serial": round(ov_ms / (gemm_ms + send_ms), 4)}
    if int(hp.error_flag.item()) != 0:
        raise RuntimeError("device error flag in the overlapped send phases")
    torch.cuda.synchronize()
    destroy_stream(comm_handle)
    out = {n: {"avg_us": round(res[n] * 1e3, 2), "alg_bytes": alg[n],
               "hbm_gbps": round(alg[n] / (res[n] * 1e-3) / 1e9, 1)} for n in res}
    out["routed_token_node_pairs"] = routed
    out["dispatch_send_plus_recv_us"] = round((res["dispatch_send"] + res["dispatch_recv"]) * 1e3, 2)
    out["combine_send_plus_recv_us"] = round((res["combine_send"] + res["combine_recv"]) * 1e3, 2)
    out["overlap"] = ov
    del hp, a, w, c
    torch.cuda.empty_cache()
    return out


SEND_BUDGET = 512  # workgroups of the budgeted send phase: two per CU


def _hip_runtime():
    """The HIP runtime library torch has loaded (the library's calls go through the same)."""
    import ctypes

    with open("/proc/self/maps") as fh:
        path = next(l.split()[-1] for l in fh if "libamdhip64" in l)
    return ctypes.CDLL(path)


def dedicated_queue_stream(torch):
    """A stream with a hardware queue of its own: HIP gives each CU-masked stream its own
    queue; the mask here enables every CU. Returns (torch stream, raw handle)."""
    import ctypes

    hip = _hip_runtime()
    ncu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    words = (ncu + 31) // 32
    mask = (ctypes.c_uint32 * words)()
    for i in range(ncu):
        mask[i // 32] |= 1 << (i % 32)
    h = ctypes.c_void_p()
    hip.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                 ctypes.c_uint32,
                                                 ctypes.POINTER(ctypes.c_uint32)]
    rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), words, mask)
    if rc != 0:
        raise RuntimeError(f"hipExtStreamCreateWithCUMask returned {rc}")
    return torch.cuda.ExternalStream(h.value), h.value


def destroy_stream(handle) -> None:
    import ctypes

    hip = _hip_runtime()
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy(ctypes.c_void_p(handle))


def restripe_page_shape(torch, W, ep, steps: int, timed, flush_gib: float) -> dict:
    """The restripe at the shape its page measures, prob [4096][8][128] -> [8][4096][128]:
    the average of K back-to-back launches (warm: the 33.6 MB stay in the 256 MB Infinity
    Cache between launches), right after the yardsticks and again after 200 ms of idle,
    and single launches after a spin (warm) and after a flush of `flush_gib` GiB (cold)."""
    c = W.CONFIGS["restripe"]
    inp = W.make_inputs(c, with_x=False)
    prob = torch.from_numpy(inp.prob).cuda()
    out = torch.empty((c.N, c.Tmax, c.P), dtype=torch.float32, device="cuda")
    fn = lambda: ep.ep_restripe_prob(prob, out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    g.replay()
    ms = timed(g.replay, 1) / steps
    # The same graph after the GPU has idled: for some 30-100 ms after sustained HBM
    # traffic (the bench's yardsticks run just before) short launches run slower.
    torch.cuda.synchronize()
    time.sleep(0.2)
    ms_idle = timed(g.replay, 1) / steps
    del g
    dist = launch_distribution(torch, ep, {"restripe": fn}, steps, flush_gib)
    alg = 2 * c.T * c.N * c.P * 4
    res = {"shape": f"[{c.T}][{c.N}][{c.P}] -> [{c.N}][{c.Tmax}][{c.P}]", "alg_bytes": alg,
           "back_to_back_avg_us": round(ms * 1e3, 2),
           "back_to_back_hbm_gbps": round(alg / (ms * 1e-3) / 1e9, 1),
           "back_to_back_after_200ms_idle_avg_us": round(ms_idle * 1e3, 2),
           "single_launch_warm_median_us": dist["warm"]["restripe"]["median_us"],
           "single_launch_cold_median_us": dist["cold"]["restripe"]["median_us"],
           "event_floor_us": dist["event_floor_us"]}
    del prob, out
    torch.cuda.empty_cache()
    return res


def mix_yardstick(torch, ep, cfg, M: int, avg: dict, alg: dict, steps: int, timed) -> dict:
    """What HBM sustains for the read/write mix of each big kernel, with every access a
    sequential stream (ep_hbm_fan on slabs of T*H*2 bytes): F slabs reduced into one for the
    combine (F = 7 and 8 around its M/T reads per write), one slab written F times for the
    dispatch. The time at F = M/T is interpolated between the two. For the combine the
    same fan-in is also timed with its reads spread over R sequential streams, one per
    rank's block of the receive buffer (ep_hbm_spread, when T*H*2 splits into whole
    chunks over the R regions)."""
    slab = cfg.T * cfg.H * 2
    src = torch.empty(8 * slab, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(8 * slab, dtype=torch.uint8, device="cuda")
    t = {}

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        g.replay()
        ms = timed(g.replay, 1) / steps
        del g
        return ms
    for fi, fo in ((7, 1), (8, 1), (1, 7), (1, 8)):
        t[(fi, fo)] = graph_of(lambda: ep.ep_hbm_fan(src, dst, slab, fi, fo))
    chunk = ep.EP_HBM_SPREAD_CHUNK_BYTES
    spread_ok = slab % chunk == 0 and all((F * (slab // chunk)) % cfg.R == 0 for F in (7, 8))
    if spread_ok:
        for F in (7, 8):
            t[("spread", F)] = graph_of(lambda: ep.ep_hbm_spread(src, dst, slab, F, cfg.R))
    del src, dst
    torch.cuda.empty_cache()
    f = M / cfg.T
    out = {"slab_bytes": slab, "reads_per_write": round(f, 4)}
    for name, lo, hi in (("combine", (7, 1), (8, 1)), ("dispatch", (1, 7), (1, 8))):
        ms = t[lo] + (f - 7) * (t[hi] - t[lo])
        moved = (f + 1) * slab
        out[name] = {"fan_7_us": round(t[lo] * 1e3, 2), "fan_8_us": round(t[hi] * 1e3, 2),
                     "yardstick_us_at_mix": round(ms * 1e3, 2),
                     "yardstick_gbps": round(moved / (ms * 1e-3) / 1e9, 1),
                     "kernel_us": round(avg[name] * 1e3, 2),
                     "kernel_hbm_gbps": round(alg[name] / (avg[name] * 1e-3) / 1e9, 1),
                     "kernel_frac_of_yardstick": round((alg[name] / avg[name]) /
                                                       (moved / ms), 4)}
    if spread_ok:
        lo, hi = t[("spread", 7)], t[("spread", 8)]
        ms = lo + (f - 7) * (hi - lo)
        moved = (f + 1) * slab
        out["combine"]["spread_over_ranks"] = {
            "regions": cfg.R, "chunk_bytes": chunk,
            "fan_7_us": round(lo * 1e3, 2), "fan_8_us": round(hi * 1e3, 2),
            "yardstick_us_at_mix": round(ms * 1e3, 2),
            "yardstick_gbps": round(moved / (ms * 1e-3) / 1e9, 1),
            "kernel_frac_of_yardstick": round((alg["combine"] / avg["combine"]) / (moved / ms), 4)}
    else:
        out["combine"]["spread_over_ranks"] = None
    return out


def small_batches(torch, W, DeviceBatch, Path, cfg, steps: int, timed) -> dict:
    """The whole step at decode-sized batches of the same shape (64, 256 and 1024 tokens),
    timed like the headline step (one graph of K steps); seeded inputs of their own. Up to
    256 tokens Path.step is ep_layout_dispatch + ep_combine; the counts path's step (three
    launches) is timed beside it there, and its outputs checked equal."""
    def graph_ms(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fn()
        g.replay()
        ms = timed(g.replay, 1) / steps
        del g
        return ms

    out = {}
    for T in (64, 256, 1024):
        c = cfg.with_(T=T, Tmax=T, name=f"{cfg.name}_T{T}")
        inp = W.make_inputs(c)
        b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
        p = Path(c.T, c.H, c.E, c.k, c.R, c.N, c.P, c.Tmax)
        p.step(b)
        torch.cuda.synchronize()
        M = int(p.layout_buf.rank_offset[-1].item())
        ms = graph_ms(lambda: p.step(b))
        if int(p.error_flag.item()) != 0:
            raise RuntimeError(f"device error flag at T={T}")
        one = p.counts_path and T <= 256
        r = {"step_us": round(ms * 1e3, 2),
             "step": "ep_layout_dispatch + ep_combine" if one else "the counts path",
             "M_token_rank_pairs": M,
             "algorithm_gbps": round(2 * M * c.H * 2 / (ms * 1e-3) / 1e9, 1),
             "tokens_per_s": round(T / (ms * 1e-3), 1)}
        if one:
            ref = (p.out.clone(), p.recv.recv_x[:M].clone(), p.prob_dest_major[:, :T].clone())
            # per call, each a graph of K launches of that call alone
            r["layout_dispatch_us"] = round(graph_ms(lambda: p.layout_dispatch(b)) * 1e3, 2)
            r["combine_us"] = round(graph_ms(lambda: p.combine(b)) * 1e3, 2)
            r["counts_path_layout_counts_us"] = round(graph_ms(lambda: p.layout_counts(b)) * 1e3, 2)
            r["counts_path_dispatch_layout_us"] = round(
                graph_ms(lambda: p.dispatch_layout(b)) * 1e3, 2)
            r["counts_path_step_us"] = round(graph_ms(lambda: p.step_counts(b)) * 1e3, 2)
            torch.cuda.synchronize()
            if not (torch.equal(ref[0], p.out) and torch.equal(ref[1], p.recv.recv_x[:M]) and
                    torch.equal(ref[2], p.prob_dest_major[:, :T])):
                raise RuntimeError(f"the counts path's step differs at T={T}")
        out[f"T{T}"] = r
        del p, b
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py needs --steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU and uses no collectives.", file=sys.stderr)
        sys.exit(2)

    import torch

    import __graft_entry__

    __graft_entry__._ensure_built()
    import combine_ep_get_03_amd as ep
    from combine_ep_get_03_amd import workloads as W
    from combine_ep_get_03_amd.buffers import LayoutBuffers
    from combine_ep_get_03_amd.pipeline import DeviceBatch, Path

    cfg = W.CONFIGS[args.config]
    print(f"bench: generating {cfg}", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg)
    torch.cuda.set_device(0)
    # every launch and event of the bench goes to one dedicated stream (default priority)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    b = DeviceBatch.from_host(inp.topk_idx, inp.topk_weights, inp.x, inp.prob, inp.partials)
    path = Path(cfg.T, cfg.H, cfg.E, cfg.k, cfg.R, cfg.N, cfg.P, cfg.Tmax)

    copy_bw = copy_bandwidth(torch, ep, [float(g) for g in args.copy_gib.split(",")])
    print(f"bench: copy bandwidth {copy_bw}", file=sys.stderr, flush=True)

    # one eager step whose outputs every graph replay is checked against (also with W = 0)
    path.step(b)
    for _ in range(args.warmup):
        path.step(b)
    torch.cuda.synchronize()
    if int(path.error_flag.item()) != 0:
        raise RuntimeError(f"device error flag {int(path.error_flag.item())}")
    M = int(path.layout_buf.rank_offset[-1].item())

    names = ["layout", "dispatch", "restripe", "combine"]
    calls = [path.layout, path.dispatch, path.restripe, path.combine]
    if path.counts_path:
        names += ["layout_counts", "dispatch_layout"]
        calls += [path.layout_counts, path.dispatch_layout]
    # every element of these is written by each step (receive rows beyond M are not)
    lb = path.layout_buf
    outputs = [lb.num_tokens_per_rank, lb.num_tokens_per_node, lb.num_tokens_per_expert,
               lb.is_token_in_rank, lb.rank_offset, lb.expert_offset, lb.token_slot,
               path.recv.recv_x[:M], path.recv.recv_topk_idx[:M],
               path.recv.recv_topk_weights[:M], path.recv.recv_src_idx[:M],
               path.prob_dest_major[:, :cfg.T], path.out]
    eager_ref = [t.clone() for t in outputs]

    def timed(fn, reps):
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(stream)
        for _ in range(reps):
            fn()
        s1.record(stream)
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / reps

    # The step is captured once into a HIP graph and replayed, so the host issues one
    # call per step; the replay must reproduce the eager outputs bit for bit.
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        path.step(b)
    for t in outputs:
        t.view(torch.uint8).fill_(0xA5)
    g_step.replay()
    torch.cuda.synchronize()
    for t, r in zip(outputs, eager_ref):
        if not torch.equal(t.view(torch.uint8), r.view(torch.uint8)):
            raise RuntimeError("graph replay differs from the eager step")
    # The K timed steps are captured back to back into one graph as well, so the host
    # issues one call for all of them and no per-replay launch gap falls between steps;
    # its replay must also leave the eager outputs.
    g_k = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_k):
        for _ in range(args.steps):
            path.step(b)
    for t in outputs:
        t.view(torch.uint8).fill_(0xA5)
    g_k.replay()
    torch.cuda.synchronize()
    for t, r in zip(outputs, eager_ref):
        if not torch.equal(t.view(torch.uint8), r.view(torch.uint8)):
            raise RuntimeError("the K-step graph's replay differs from the eager step")
    for _ in range(args.warmup):
        g_step.replay()

    # Timed region: K whole steps (one replay of the K-step graph), events at both ends.
    ms_step = timed(g_k.replay, 1) / args.steps
    ms_step_replays = timed(g_step.replay, args.steps)
    ms_step_eager = timed(lambda: path.step(b), args.steps)
    del g_k
    # the same K steps with one call per step of the path (no fused layout + restripe)
    g_sep = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_sep):
        for _ in range(args.steps):
            path.step_separate(b)
    for t in outputs:
        t.view(torch.uint8).fill_(0xA5)
    g_sep.replay()
    torch.cuda.synchronize()
    for t, r in zip(outputs, eager_ref):
        if not torch.equal(t.view(torch.uint8), r.view(torch.uint8)):
            raise RuntimeError("the one-call-per-step graph differs from the eager step")
    ms_step_sep = timed(g_sep.replay, 1) / args.steps
    del g_sep
    # the same K steps on the preprocess path (layout and restripe in one call, then
    # ep_dispatch), when the step itself is the counts path
    ms_step_pre = None
    if path.counts_path:
        g_pre = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pre):
            for _ in range(args.steps):
                path.step_preprocess(b)
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        g_pre.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, eager_ref):
            if not torch.equal(t.view(torch.uint8), r.view(torch.uint8)):
                raise RuntimeError("the preprocess-path graph differs from the eager step")
        ms_step_pre = timed(g_pre.replay, 1) / args.steps
        del g_pre

    # Each call's average launch duration: one graph of K back-to-back launches of that
    # call alone, replayed between two events on the launch stream.
    avg = {}
    for n, fn in zip(names, calls):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                fn(b)
        g.replay()
        avg[n] = timed(g.replay, 1) / args.steps
        del g
    # FP8 dispatch (same routing, e4m3 payload + per-128-channel scales), when H allows it
    fp8 = None
    if cfg.H % 128 == 0:
        codes = torch.empty((path.cap, cfg.H), dtype=torch.uint8, device="cuda")
        scales = torch.empty((path.cap, cfg.H // 128), dtype=torch.float32, device="cuda")
        r = path.recv

        def fp8_call():
            ep.ep_dispatch_fp8(b.x, b.topk_idx, b.topk_weights, cfg.E, cfg.R,
                               path.layout_buf.token_slot, recv_x_fp8=codes, recv_scales=scales,
                               recv_topk_idx=r.recv_topk_idx, recv_topk_weights=r.recv_topk_weights,
                               recv_src_idx=r.recv_src_idx, error_flag=path.error_flag)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                fp8_call()
        g.replay()
        fp8_ms = timed(g.replay, 1) / args.steps
        del g
        fb = (cfg.T * cfg.H * 2 + cfg.T * cfg.k * 12 + cfg.T * cfg.R * 4 +
              M * (cfg.H + 4 * (cfg.H // 128) + 12 * cfg.k + 4))
        fp8 = {"avg_us": round(fp8_ms * 1e3, 2), "alg_bytes": fb,
               "hbm_gbps": round(fb / (fp8_ms * 1e-3) / 1e9, 1),
               "algorithm_gbps": round(M * (cfg.H + 4 * (cfg.H // 128)) / (fp8_ms * 1e-3) / 1e9, 1),
               "tokens_per_s": round(cfg.T / (fp8_ms * 1e-3), 1)}
        del codes, scales
    # Dispatch + permute: layout with expert-major slots, then the rows straight into
    # expert-major order (k rows per token)
    permute = None
    if cfg.k <= ep.EP_EXPERT_SLOT_MAX_K:
        lbe = LayoutBuffers.alloc(cfg.T, cfg.E, cfg.R, cfg.N, k_expert_slots=cfg.k)
        px = torch.empty((cfg.T * cfg.k, cfg.H), dtype=torch.bfloat16, device="cuda")
        pw = torch.empty(cfg.T * cfg.k, dtype=torch.float32, device="cuda")
        ps = torch.empty(cfg.T * cfg.k, dtype=torch.int32, device="cuda")

        def layout_e():
            lbe.compute(b.topk_idx, cfg.E, cfg.R, cfg.N)

        def permute_call():
            ep.ep_dispatch_permute(b.x, b.topk_weights, lbe.expert_slot, perm_x=px,
                                   perm_weights=pw, perm_src_idx=ps, error_flag=lbe.error_flag)
        perm_calls = [("layout_with_expert_slots", layout_e), ("dispatch_permute", permute_call)]
        # the counts path's form (R <= 64, T <= 16384): the count launch with each pair's
        # in-block expert rank, then the permute forming the rows itself; checked bit-equal
        counts_form = cfg.R <= ep.EP_COUNTS_MAX_RANKS and cfg.T <= 16384
        if counts_form:
            ws = torch.zeros(ep.ep_layout_counts_workspace_bytes(cfg.T, cfg.E, cfg.R, cfg.N),
                             dtype=torch.uint8, device="cuda")
            er = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
            es2 = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
            px2, pw2, ps2 = torch.empty_like(px), torch.empty_like(pw), torch.empty_like(ps)
            flag2 = torch.zeros(1, dtype=torch.int32, device="cuda")

            def counts_e():
                ep.ep_layout_counts(b.topk_idx, cfg.E, cfg.R, cfg.N, error_flag=flag2,
                                    workspace=ws, expert_rank=er)

            def permute_layout_call():
                ep.ep_dispatch_permute_layout(b.x, b.topk_idx, b.topk_weights, cfg.E, cfg.R,
                                              cfg.N, expert_rank=er, perm_x=px2, workspace=ws,
                                              perm_weights=pw2, perm_src_idx=ps2,
                                              expert_slot=es2, error_flag=flag2)
            perm_calls += [("layout_counts_with_expert_ranks", counts_e),
                           ("dispatch_permute_layout", permute_layout_call)]
        res = {}
        for n, fn in perm_calls:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(args.steps):
                    fn()
            g.replay()
            res[n] = timed(g.replay, 1) / args.steps
            del g
        if int(lbe.error_flag.item()) != 0:
            raise RuntimeError("device error flag in dispatch+permute")
        rows = cfg.T * cfg.k
        pb = cfg.T * cfg.H * 2 + rows * (4 + 4) + rows * (2 * cfg.H + 8)
        permute = {"layout_with_expert_slots_us": round(res["layout_with_expert_slots"] * 1e3, 2),
                   "dispatch_permute_us": round(res["dispatch_permute"] * 1e3, 2),
                   "alg_bytes": pb,
                   "hbm_gbps": round(pb / (res["dispatch_permute"] * 1e-3) / 1e9, 1)}
        if counts_form:
            n_rows = int((lbe.expert_slot >= 0).sum().item())
            if (int(flag2.item()) != 0 or not torch.equal(es2, lbe.expert_slot)
                    or not torch.equal(px2[:n_rows], px[:n_rows])
                    or not torch.equal(ps2[:n_rows], ps[:n_rows])):
                raise RuntimeError("the counts path's permute differs from ep_dispatch_permute")
            permute["counts_path"] = {
                "layout_counts_with_expert_ranks_us":
                    round(res["layout_counts_with_expert_ranks"] * 1e3, 2),
                "dispatch_permute_layout_us": round(res["dispatch_permute_layout"] * 1e3, 2),
                "both_us": round((res["layout_counts_with_expert_ranks"] +
                                  res["dispatch_permute_layout"]) * 1e3, 2)}
            del ws, er, es2, px2, pw2, ps2
        del px, pw, ps, lbe
    # Sparse restripe: layout with per-node slots, then only the routed (token, node)
    # slices packed per node (the dense restripe copies all T*N of them)
    lbn = LayoutBuffers.alloc(cfg.T, cfg.E, cfg.R, cfg.N, node_slots=True)
    sp_out = torch.empty((cfg.N, cfg.Tmax, cfg.P), dtype=torch.float32, device="cuda")

    def layout_n():
        lbn.compute(b.topk_idx, cfg.E, cfg.R, cfg.N)

    def sparse_call():
        ep.ep_restripe_prob_sparse(b.prob, lbn.node_slot, sp_out, error_flag=lbn.error_flag)
    res = {}
    for n, fn in (("layout_with_node_slots", layout_n), ("restripe_sparse", sparse_call)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(args.steps):
                fn()
        g.replay()
        res[n] = timed(g.replay, 1) / args.steps
        del g
    if int(lbn.error_flag.item()) != 0:
        raise RuntimeError("device error flag in sparse restripe")
    routed = int(lbn.num_tokens_per_node.sum().item())
    sb = cfg.T * cfg.N * 4 + 2 * routed * cfg.P * 4
    sparse = {"layout_with_node_slots_us": round(res["layout_with_node_slots"] * 1e3, 2),
              "restripe_sparse_us": round(res["restripe_sparse"] * 1e3, 2),
              "routed_token_node_pairs": routed, "alg_bytes": sb,
              "hbm_gbps": round(sb / (res["restripe_sparse"] * 1e-3) / 1e9, 1)}
    del sp_out, lbn
    hook = hook_section(torch, cfg, b, args, timed, M)
    alg = algorithmic_bytes(cfg, M)
    mix = mix_yardstick(torch, ep, cfg, M, avg, alg, args.steps, timed)
    restripe_page = restripe_page_shape(torch, W, ep, args.steps, timed, args.flush_gib)
    small = (small_batches(torch, W, DeviceBatch, Path, cfg, args.steps, timed)
             if args.small_batches else None)
    dist_calls = {n: (lambda fn=fn: fn(b)) for n, fn in zip(names, calls)}
    dist_calls["step_graph"] = g_step.replay
    dist = launch_distribution(torch, ep, dist_calls, args.steps, args.flush_gib)
    if int(path.error_flag.item()) != 0:
        raise RuntimeError(f"device error flag {int(path.error_flag.item())}")

    payload = 2 * M * cfg.H * 2
    value = payload / (ms_step * 1e-3) / 1e9
    dom = max(("dispatch", "combine"), key=lambda n: avg[n])
    achieved = alg[dom] / (avg[dom] * 1e-3) / 1e9
    best_copy = max(copy_bw.values())
    kernels = {n: {"avg_us": round(avg[n] * 1e3, 2), "alg_bytes": alg[n],
                   "hbm_gbps": round(alg[n] / (avg[n] * 1e-3) / 1e9, 1),
                   "frac_of_copy": round(alg[n] / (avg[n] * 1e-3) / 1e9 / best_copy, 4)}
               for n in names}
    dc_ms = avg["dispatch"] + avg["combine"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_one_graph_replay_each": round(ms_step_replays, 4),
        "ms_per_step_eager_launches": round(ms_step_eager, 4),
        "ms_per_step_one_call_per_step": round(ms_step_sep, 4),
        "ms_per_step_preprocess_path": None if ms_step_pre is None else round(ms_step_pre, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} top-{cfg.k} "
                               f"{cfg.routing} R={cfg.R} simulated ranks N={cfg.N} nodes "
                               f"P={cfg.P} Tmax={cfg.Tmax}, seed {cfg.seed}",
                   "M_token_rank_pairs": M, "global_batch": cfg.T, "parallelism": "none"},
        "tokens_per_s": round(cfg.T / (ms_step * 1e-3), 1),
        "dispatch_combine": {"ms": round(dc_ms, 4),
                             "algorithm_gbps": round(payload / (dc_ms * 1e-3) / 1e9, 1),
                             "hbm_gbps": round((alg["dispatch"] + alg["combine"]) /
                                               (dc_ms * 1e-3) / 1e9, 1),
                             "frac_of_copy": round((alg["dispatch"] + alg["combine"]) /
                                                   (dc_ms * 1e-3) / 1e9 / best_copy, 4),
                             "tokens_per_s": round(cfg.T / (dc_ms * 1e-3), 1)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom, cfg.name),
                     "alg_bytes_per_launch": alg[dom], "avg_launch_us": round(avg[dom] * 1e3, 2)},
        "copy_bandwidth_gbps": {k: round(v, 1) for k, v in copy_bw.items()},
        "mix_yardstick": mix,
        "restripe_page_shape": restripe_page,
        "dispatch_fp8": fp8,
        "dispatch_permute": permute,
        "restripe_sparse": sparse,
        "hook": hook,
        "kernels": kernels,
        "launch_distribution": dist,
        "small_batches": small,
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
