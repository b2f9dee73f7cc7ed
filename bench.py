#!/usr/bin/env python3
"""Routed tokens/s of one masked-top-k MXFP4 MoE layer on one MI355X.

A step is one pass of the whole layer over one batch of tokens already
resident in HBM: moe_route (router logits, demand picks, masked top-k,
renormalisation, bucketing by slot, MXFP4 activations, and the demand
histogram update) followed by moe_experts_forward (grouped SwiGLU experts on
MXFP4 arena slots and the fixed-order weighted combine).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all]

Prints one JSON line.  Inputs are seeded synthetic workloads (fixtures/).  The
line's `value` is the decode batch (8 tokens, hidden 4096, 256 experts, top-8,
SwiGLU intermediate 2048, 166 resident + 64 hot-ring slots, Zipf-skewed
router): the memory-bound half of the metric.  With the default
`--workload all` the same line carries, under "workloads", a block for each
other workload, with its own time per step, roofline and CPU-oracle baseline:
  prefill  2048 tokens of the same model (memory-bound at this size)
  long     8192 tokens, hidden 6144, 192 experts (the matrix-bound half)
  arena40  40 layers x 256 experts sharing one 6666-slot arena, 32 tokens a
           layer call: demand accumulated over 512 steps, the 5 % re-plan (333
           slot swaps), then 8 more steps.
Layer workloads rotate over 4 token batches and 4 copies of the arena so the
256 MB Infinity Cache cannot serve expert bytes reused from a previous step.
The decode, prefill and long blocks also time, under "act_mxfp6", the
activation-format variant (activation and h rows in MXFP6, same weights);
--no-act-mxfp6 leaves that leg out.

Timing: W warmup steps, then K steps between two events on the launch stream
(no other instrumentation) give `ms_per_step`.  A second run of the K steps
takes the start and end of the dominant kernel -- the grouped gate/up GEMM,
2/3 of the expert bytes and flops -- from its own dispatch, for the roofline:
achieved = algorithmic bytes (or, above the MXFP4 ridge, flops) per launch /
mean launch time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4, vendor figure
METRIC = "routed tokens/s per MoE layer; % peak HBM GB/s (decode), % MXFP4 MFMA (prefill)"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "resident_expert_routing_amd", "csrc", "experts.hip")
LAYER_WORKLOADS = ("decode", "prefill", "long", "tiny")
ARENA40_DEMAND_STEPS = 512     # steps of demand before the re-plan
ARENA40_AFTER_STEPS = 8        # steps run on the re-planned arena
RING_SLOTS, RING_PER_STEP, RING_STEPS = 64, 8, 32   # the hot ring's cost measurement


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill", "long", "tiny", "arena40"])
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak microbenchmarks (for profiler runs)")
    ap.add_argument("--no-act-mxfp6", action="store_true",
                    help="skip the MXFP6 activation-row leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (to scale HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))


def gateup_kernel_name(T: int, k: int, H: int, I: int) -> str:
    """The gate/up kernel moe_experts_forward launches for this batch shape."""
    tiled = T * k >= 2048 and H % 512 == 0 and I % 512 == 0
    return "gateup_pipe" if tiled else "gateup_kernel"


def gateup_bytes_per_slot(H: int, I: int) -> int:
    return 2 * I * (H // 2 + H // 32)


def expert_bytes(H: int, I: int) -> int:
    return 3 * H * I // 2 + 3 * H * I // 32


def row_bytes(K: int) -> int:
    return (K // 2 + K // 32 + 15) // 16 * 16


def row6_bytes(K: int) -> int:
    """An MXFP6 activation row: 24 code bytes and a scale byte per 32 elements."""
    return (K // 32 * 25 + 15) // 16 * 16


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per gate/up launch from the committed rocprofv3 PMC summary
    (profiles/<kernel>_<workload>_pmc.json).

    Returns None if there is no summary or the kernel source changed since."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        p = json.load(f)
    if p.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return p.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(lay, k: int, tokens: int | None = None, what: str | None = None):
    """The oracle (numpy float64) on one layer call, timed on the host cores.
    tokens: run the layer on the first `tokens` rows of the batch only (a
    bounded sample of a large chunk); tokens/s is per token either way."""
    from oracle import moe
    blas = blas_threads()
    cfg = lay.cfg
    sc = lay.slot_content()
    x = lay.x_bits if tokens is None else lay.x_bits[:tokens]
    t0 = time.perf_counter()
    moe.layer(x, lay.w_router, lay.bias, lay.expert_slot, k,
              lambda s: lay.content_bytes(sc[s]), cfg.H, cfg.I)
    dt = time.perf_counter() - t0
    T = x.shape[0]
    what = what or f"one full {cfg.name} layer call"
    return {"value": T / dt, "unit": "tokens/s", "cores": int(blas), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{what} ({T} tokens: float64 router, softmax, top-k, masked top-k, "
                      f"demand, MXFP4 decode of every used expert, SwiGLU, combine) in "
                      f"{dt:.2f} s; numpy elementwise on 1 thread, BLAS on {blas}",
            "seconds": dt}


_PEAKS = {}


def achievable_peak(bound: str, dev) -> dict:
    """The device's achievable peak for the roofline's bound, measured once per
    run with the library's microbenchmarks: an 8 GiB read (32x the Infinity
    Cache, 16-byte loads, four in flight per thread; three launches back to
    back, so the launch ramps weigh little) or a loop of the MXFP4 32x32x64
    instruction; the best of the repetitions."""
    if bound in _PEAKS:
        return _PEAKS[bound]
    import torch
    from resident_expert_routing_amd import binding as B
    mk = lambda: torch.cuda.Event(enable_timing=True)
    best = 0.0
    if bound == "hbm":
        n, grid, back = 8 << 30, 8192, 3
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        sink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
        for _ in range(3):
            e0, e1 = mk(), mk()
            e0.record()
            for _ in range(back):
                B.check(B.moe_test_stream_read(src, n, sink, grid), "moe_test_stream_read")
            e1.record()
            torch.cuda.synchronize()
            best = max(best, back * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        del src
        _PEAKS[bound] = {"achievable_peak": best, "achievable_how": "moe_test_stream_read: 3 "
                         "reads of 8 GiB back to back, best of 3"}
        return _PEAKS[bound]
    _PEAKS[bound] = {"achievable_peak": mfma_loop_rate(dev, 0),
                     "achievable_how": "moe_test_mfma_loop: 32x32x64 MXFP4 instruction, 8 chains "
                     "per wave, best of 6 launches"}
    return _PEAKS[bound]


def mfma_loop_rate(dev, act_format: int) -> float:
    """TFLOP/s of the 32x32x64 block-scaled instruction loop, E2M1 A operands
    and E2M1 (0) or E2M3 (1) B operands; best of 6 launches."""
    import torch
    from resident_expert_routing_amd import binding as B
    mk = lambda: torch.cuda.Event(enable_timing=True)
    iters, grid = 1000, 1024
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    flops = grid * 4 * iters * 8 * 2.0 * 32 * 32 * 64
    best = 0.0
    for _ in range(6):
        e0, e1 = mk(), mk()
        e0.record()
        B.check(B.moe_test_mfma_loop(iters, sink, grid, act_format=act_format),
                "moe_test_mfma_loop")
        e1.record()
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def gateup_roofline(gu_us: float, gu_bytes: float, gu_flops: float, args, dev) -> dict:
    """Roofline of the gate/up kernel: memory-bound below the MXFP4 ridge (peak
    flops / peak bytes), matrix-bound above it."""
    ridge = MXFP4_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if gu_flops / gu_bytes > ridge:
        roof = {"bound": "mfma", "achieved": gu_flops / (gu_us * 1e-6) / 1e12,
                "peak": MXFP4_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": gu_bytes / (gu_us * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if not args.no_peaks:
        roof.update(achievable_peak(roof["bound"], dev))
        roof["achievable_frac"] = roof["achieved"] / roof["achievable_peak"]
    return roof


def act_mxfp6_timing(name, T, H, E, k, I, S, xs, w_router, bias, expert_slot, arenas, hist, U,
                     stream, steps: int, warmup: int, args, dev) -> dict:
    """The activation-format variant on the same inputs: activation and h rows
    in MXFP6 (E2M3), weights unchanged; every batch size on the small-batch
    kernels.  Same step and timing protocol as the MXFP4 line."""
    import numpy as np
    import torch
    from resident_expert_routing_amd import binding as B
    from resident_expert_routing_amd import runtime as R
    nrot = len(arenas)
    buf = R.LayerBuffers(T, H, E, k, I, S, dev, act_format=B.MOE_ACT_MXFP6)

    def step(i, ev_e=None):
        j = i % nrot
        R.route(buf, xs[j], w_router, bias, expert_slot, stream, hist_row=hist)
        R.experts(buf, arenas[j].ptr(), arenas[j].stride, stream, ev_e)

    for i in range(warmup):
        step(i)
    mk = lambda: torch.cuda.Event(enable_timing=True)
    start, end = mk(), mk()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ev = [(mk(), mk()) for _ in range(steps)]
    for a_, b_ in ev:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        step(i, [None, ev[i][0], ev[i][1], None, None])
    torch.cuda.synchronize()
    gu_us = float(np.mean([a_.elapsed_time(b_) for a_, b_ in ev])) * 1e3
    A = T * k
    u_steps = [U[i % nrot] for i in range(steps)]
    gu_bytes = float(np.mean([u * gateup_bytes_per_slot(H, I) for u in u_steps])) \
        + T * row6_bytes(H) + A * row6_bytes(I)
    roof = gateup_roofline(gu_us, gu_bytes, 4.0 * H * I * A, args, dev)
    kernel = "gateup_pipe6" if gateup_kernel_name(T, k, H, I) == "gateup_pipe" else "gateup_kernel6"
    out = {"value": T * steps / (total_ms * 1e-3), "unit": "tokens/s", "steps": steps,
           "ms_per_step": total_ms / steps, "dtype": "mxfp4 weights x mxfp6 activations",
           "roofline": {**roof, "kernel": kernel,
                        "traffic": traffic_from_profile(kernel, name),
                        "algo_bytes_per_launch": gu_bytes,
                        "algo_flops_per_launch": 4.0 * H * I * A, "mean_launch_us": gu_us}}
    if not args.no_peaks:   # the instruction's rate with E2M3 against E2M1 B operands
        out["mfma_loop_tflops"] = {"e2m1_x_e2m1": mfma_loop_rate(dev, 0),
                                   "e2m1_x_e2m3": mfma_loop_rate(dev, 1)}
    log(f"  MXFP6 activations: {total_ms / steps * 1e3:.1f} us/step, gate/up {gu_us:.1f} us "
        f"({roof['frac']:.3f} of peak {roof['unit']})")
    return out


def hot_read_timing(lay, x, w_router, bias, arena, buf, E, stream, reps: int = 11):
    """Layer calls of the long chunk with the hot read (route, pick the heaviest
    miss, copy its 20 MB from page-locked host memory into the coldest arena
    expert's slot on a side stream, route again, experts after the copy) and
    without it, each timed on the host around the call with a synchronisation;
    the copy alone is timed with events on the side stream.  Never part of
    `value`: the copy crosses PCIe."""
    import numpy as np
    import torch
    from resident_expert_routing_amd import binding as B
    from resident_expert_routing_amd import runtime as R

    dev = x.device
    es0 = lay.expert_slot.astype(np.int32)
    hist = torch.zeros(E, dtype=torch.float64, device=dev)
    es0_dev = torch.from_numpy(es0).to(dev)
    es = es0_dev.clone()
    n_arena = lay.extra["n_resident"]
    pins = R.PinnedCopies()
    # one reader for every call, as a serving loop keeps one per layer (its
    # stream, events and page-locked buffers are made once, outside the timing)
    hot = R.HotReader(es0, n_arena, dev)
    hot.pins = pins

    def plain():
        es.copy_(es0_dev)   # the table as the chunk found it (also before each hot call)
        R.route(buf, x, w_router, bias, es, stream, hist_row=hist)
        R.experts(buf, arena.ptr(), arena.stride, stream)

    def with_hot():
        es.copy_(es0_dev)
        hot.es[:] = es0
        picked = R.layer_step_hot(buf, x, w_router, bias, es, hist, arena, hot, lay.expert_bytes,
                                  stream)
        return picked, hot

    picked, hot = with_hot()    # warm: makes the page-locked copy of the loaded expert
    torch.cuda.synchronize()
    if picked is None:
        return {"loaded": None, "note": "no pick with a share of at least 0.2 in this chunk"}
    times = {"plain": [], "hot": []}
    for _ in range(reps):
        for kind, fn in (("plain", plain), ("hot", with_hot)):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            times[kind].append(time.perf_counter() - t0)
    # the copy alone, timed on the side stream
    hot = R.HotReader(es0, n_arena, dev)
    hot.pins = pins
    src = hot.pinned(picked[0], lay.expert_bytes)   # the copy made above
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    slot = int(es0[picked[1]])
    with torch.cuda.stream(hot.side):
        e0.record(hot.side)
    B.check(B.arena_load_slot(arena.mem, arena.stride, arena.S, slot, src, arena.slot_bytes,
                              hot.side, None), "arena_load_slot")
    with torch.cuda.stream(hot.side):
        e1.record(hot.side)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1)
    # put the evicted expert's bytes back, so the arena is as the bench found it
    arena.upload(lambda s: lay.content_bytes(lay.slot_content()[s]), slots=[slot])
    torch.cuda.synchronize()
    return {"loaded": int(picked[0]), "evicted": int(picked[1]), "slot": slot,
            "bytes_h2d": int(arena.slot_bytes),
            "ms_layer_with_hot_read": 1e3 * float(np.median(times["hot"])),
            "ms_layer_without": 1e3 * float(np.median(times["plain"])),
            "ms_copy": copy_ms, "GB_per_s_copy": arena.slot_bytes / (copy_ms * 1e-3) / 1e9,
            "timing": "host clock around each call with synchronisations (median of "
                      f"{reps}); the copy alone with events on the side stream"}


def layer_workload(name: str, args, dev, steps: int, warmup: int) -> dict:
    """One layer workload (decode, prefill, long, tiny): times, roofline, layer
    figures, and the CPU oracle's rate on the host."""
    import numpy as np
    import torch
    import fixtures
    from resident_expert_routing_amd import runtime as R

    base = fixtures.make_layer(name)
    cfg = base.cfg
    T, H, E, k, I, S = base.x_bits.shape[0], cfg.H, cfg.E, cfg.k, cfg.I, base.S
    nrot = max(1, args.rotate)
    log(f"workload {name}: T={T} H={H} E={E} k={k} I={I} S={S}")

    # ---- inputs resident in HBM ----
    layers = [base] + [fixtures.make_layer(name, x_stream=i) for i in range(1, nrot)]
    xs = [torch.from_numpy(l.x_bits.view(np.int16)).to(dev) for l in layers]
    w_router = torch.from_numpy(base.w_router).to(dev)
    bias = torch.from_numpy(base.bias).to(dev)
    expert_slot = torch.from_numpy(base.expert_slot.astype(np.int32)).to(dev)
    sc = base.slot_content()
    arenas = []
    for i in range(nrot):
        a = R.Arena(S, H, I, dev)
        a.upload(lambda s: base.content_bytes(sc[s]))
        arenas.append(a)
    log(f"{nrot} arena copies of {S} slots uploaded")
    buf = R.LayerBuffers(T, H, E, k, I, S, dev)
    hist = torch.zeros(E, dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, ev_e=None):
        j = i % nrot
        # demand is accumulated inside moe_route (same result as moe_demand_accumulate)
        R.route(buf, xs[j], w_router, bias, expert_slot, stream, hist_row=hist)
        R.experts(buf, arenas[j].ptr(), arenas[j].stride, stream, ev_e)

    # distinct slots used by each rotation's routing (deterministic)
    U = []
    for j in range(nrot):
        step(j)
        torch.cuda.synchronize()
        off = buf.slot_offsets.cpu().numpy()
        U.append(int(np.count_nonzero(np.diff(off))))
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- the timed steps ----
    K = steps
    mk = lambda: torch.cuda.Event(enable_timing=True)
    start, end = mk(), mk()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    log(f"{name}: timed {K} steps: {ms_step * 1e3:.1f} us/step")

    # ---- the dominant kernel, timed from its own dispatch ----
    ev = [(mk(), mk()) for _ in range(K)]
    for a_, b_ in ev:
        a_.record(stream)   # torch creates the HIP event on first record
        b_.record(stream)
    torch.cuda.synchronize()
    r0, r1 = mk(), mk()
    r0.record(stream)
    for i in range(K):
        step(i, [None, ev[i][0], ev[i][1], None, None])
    r1.record(stream)
    torch.cuda.synchronize()
    gu_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in ev]))
    ms_step_ev = r0.elapsed_time(r1) / K

    # ---- routing alone (router, selection, demand, bucketing, MXFP4 rows) ----
    q0, q1 = mk(), mk()
    torch.cuda.synchronize()
    q0.record(stream)
    for i in range(K):
        R.route(buf, xs[i % nrot], w_router, bias, expert_slot, stream, hist_row=hist)
    q1.record(stream)
    torch.cuda.synchronize()
    route_us = q0.elapsed_time(q1) * 1e3 / K

    A = T * k
    u_steps = [U[i % nrot] for i in range(K)]
    gu_bytes = float(np.mean([u * gateup_bytes_per_slot(H, I) for u in u_steps])) \
        + T * row_bytes(H) + A * row_bytes(I)
    gu_flops = 4.0 * H * I * A
    roof = gateup_roofline(gu_ms * 1e3, gu_bytes, gu_flops, args, dev)
    layer_bytes = float(np.mean([u * expert_bytes(H, I) for u in u_steps])) + H * E * 4 \
        + 2 * T * H * 2
    layer_gbs = layer_bytes / (ms_step * 1e-3) / 1e9
    flops = 6.0 * H * I * A
    block = {
        "value": T * K / (total_ms * 1e-3), "unit": "tokens/s", "steps": K, "warmup": warmup,
        "ms_per_step": ms_step,
        "config": {"workload": f"{name}: T={T} H={H} E={E} k={k} I={I} "
                               f"resident={cfg.resident} ring={cfg.ring} S={S}",
                   "T": T, "H": H, "E": E, "k": k, "I": I, "S": S, "rotate": nrot,
                   "zipf_beta": base.beta},
        "roofline": {**roof, "kernel": gateup_kernel_name(T, k, H, I),
                     "traffic": traffic_from_profile(gateup_kernel_name(T, k, H, I), name),
                     "algo_bytes_per_launch": gu_bytes,
                     "algo_flops_per_launch": gu_flops, "mean_launch_us": gu_ms * 1e3,
                     "ms_per_step_with_these_events": ms_step_ev},
        "layer": {"algo_bytes_per_step": layer_bytes, "GB_per_s": layer_gbs,
                  "hbm_frac": layer_gbs / HBM_PEAK_GBS, "distinct_slots_used": U,
                  "assignments_per_s": A * K / (total_ms * 1e-3),
                  "mxfp4_tflops": flops / (ms_step * 1e-3) / 1e12,
                  "mxfp4_frac": flops / (ms_step * 1e-3) / 1e12 / MXFP4_PEAK_TFLOPS,
                  "routing_us_per_call": route_us, "wall_s": wall},
    }
    log(f"{name}: gate/up {gu_ms * 1e3:.1f} us, {roof['achieved']:.0f} {roof['unit']} "
        f"({roof['frac']:.3f} of peak); layer {layer_gbs:.0f} GB/s, "
        f"{block['layer']['mxfp4_frac']:.3f} of MXFP4; routing {route_us:.1f} us")
    if name == "long":
        block["hot_read"] = hot_read_timing(base, xs[0], w_router, bias, arenas[0], buf, E,
                                            stream)
    if name in ("decode", "prefill", "long") and not args.no_act_mxfp6:
        block["act_mxfp6"] = act_mxfp6_timing(name, T, H, E, k, I, S, xs, w_router, bias,
                                              expert_slot, arenas, hist, U, stream, K,
                                              min(warmup, 5), args, dev)
    del arenas
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"{name}: timing the CPU oracle")
        if name == "long":   # bounded sample: the first 1024 tokens of the chunk
            block["cpu_baseline"] = cpu_baseline(
                base, k, tokens=1024, what="the first 1024 tokens of the 8192-token chunk")
        else:
            block["cpu_baseline"] = cpu_baseline(base, k)
    return block


def arena40_workload(args, dev, warmup: int) -> dict:
    """40 layers x 256 experts sharing one 6666-slot arena, T=32 tokens a layer
    call.  Demand accumulates over 512 steps (each step: every layer on that
    step's own tokens), then the 5 % re-plan (333 slot swaps through
    arena_load_slot, timed on its own), then 8 more steps on the new tables.
    The first `warmup` of the 512 steps are untimed."""
    import numpy as np
    import torch
    import fixtures
    from resident_expert_routing_amd import runtime as R

    model = fixtures.make_arena_model("arena40")
    cfg = model.cfg
    L, T, H, E, k, I, S = model.L, cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, model.S
    S_all = S + RING_SLOTS     # the hot ring's entries sit on top of the arena's slots
    n_steps = ARENA40_DEMAND_STEPS
    log(f"arena40: {L} layers, T={T} H={H} E={E} k={k} I={I}, {S} shared slots "
        f"+ {RING_SLOTS} ring entries")
    sa = R.SharedArena(S_all, H, I, model.expert_slot_table(), dev)
    t0 = time.perf_counter()
    sa.upload(model.pair_bytes)
    log(f"arena of {S * sa.arena.stride / 1e9:.1f} GB uploaded in {time.perf_counter() - t0:.1f} s")
    ws = [torch.from_numpy(l.w_router).to(dev) for l in model.layers]
    bs = [torch.from_numpy(l.bias).to(dev) for l in model.layers]
    n_x = n_steps + ARENA40_AFTER_STEPS + RING_STEPS
    xs = torch.from_numpy(np.stack([model.tokens(s).view(np.int16) for s in range(n_x)])).to(dev)
    buf = R.LayerBuffers(T, H, E, k, I, S_all, dev)
    stream = torch.cuda.current_stream(dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)

    def step(s, gu_events=None):
        for l in range(L):
            R.route(buf, xs[s], ws[l], bs[l], sa.table[l], stream, hist_row=sa.hist[l])
            R.experts(buf, sa.arena.ptr(), sa.arena.stride, stream,
                      None if gu_events is None else [None, *gu_events[l], None, None])

    # distinct slots of every layer call of the first 4 steps (deterministic)
    used = []
    for s in range(4):
        for l in range(L):
            R.route(buf, xs[s], ws[l], bs[l], sa.table[l], stream)
            torch.cuda.synchronize()
            used.append(int(np.count_nonzero(np.diff(buf.slot_offsets.cpu().numpy()))))
    U = float(np.mean(used))

    sa.hist.zero_()
    for s in range(warmup):
        step(s)
    K = n_steps - warmup
    e0, e1 = mk(), mk()
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(warmup, n_steps):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_layer_us = ms * 1e3 / (K * L)
    log(f"arena40: {K} timed steps, {per_layer_us:.1f} us per layer call")

    # the gate/up kernel of every layer call of 4 steps (the first 4 step's tokens, whose
    # distinct slots were counted above), from its own dispatch
    gu_ev = [[(mk(), mk()) for _ in range(L)] for _ in range(4)]
    for st in gu_ev:
        for a_, b_ in st:
            a_.record(stream)
            b_.record(stream)
    torch.cuda.synchronize()
    hist_keep = sa.hist.clone()
    for s in range(4):
        step(s, gu_ev[s])
    torch.cuda.synchronize()
    sa.hist.copy_(hist_keep)        # these 4 steps are not part of the 512
    gu_us = float(np.mean([a_.elapsed_time(b_) for st in gu_ev for a_, b_ in st])) * 1e3
    gu_bytes = U * gateup_bytes_per_slot(H, I) + T * row_bytes(H) + T * k * row_bytes(I)
    roof = gateup_roofline(gu_us, gu_bytes, 4.0 * H * I * T * k, args, dev)

    be = expert_bytes(H, I)
    algo = U * be + H * E * 4 + 2 * T * H * 2   # per layer call, mean over the layer calls
    n_swap = S // 20
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    ev, ld = sa.replan(k, n_swap, model.pair_bytes, stream)
    torch.cuda.synchronize()
    replan_s = time.perf_counter() - r0
    moved = sum(1 for (le, _), (ll, _) in zip(ev, ld) if le != ll)
    a0, a1 = mk(), mk()
    a0.record(stream)
    for s in range(n_steps, n_steps + ARENA40_AFTER_STEPS):   # the layers on the new tables
        step(s)
    a1.record(stream)
    torch.cuda.synchronize()
    after_us = a0.elapsed_time(a1) * 1e3 / (ARENA40_AFTER_STEPS * L)
    ring_block = hot_ring_cost(model, sa, buf, ws, bs, xs, n_steps + ARENA40_AFTER_STEPS, S,
                               stream, dev)
    block = {
        "value": T / (per_layer_us * 1e-6), "unit": "tokens/s",
        "steps": K, "warmup": warmup, "ms_per_step": ms / K,
        "config": {"workload": f"arena40: {L} layers x E={E}, T={T} per layer call, H={H} "
                               f"k={k} I={I}, {S} shared slots; demand over {n_steps} steps, "
                               f"re-plan of {n_swap} swaps, {ARENA40_AFTER_STEPS} steps after",
                   "layers": L, "T": T, "S": S},
        "roofline": {**roof, "kernel": gateup_kernel_name(T, k, H, I),
                     "traffic": traffic_from_profile(gateup_kernel_name(T, k, H, I), "arena40"),
                     "algo_bytes_per_launch": gu_bytes, "mean_launch_us": gu_us,
                     "launches": 4 * L},
        "layer": {"us_per_layer_call": per_layer_us, "distinct_slots_per_call": U,
                  "algo_bytes_per_call": algo,
                  "GB_per_s": algo / (per_layer_us * 1e-6) / 1e9,
                  "hbm_frac": algo / (per_layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                  "us_per_layer_call_after_replan": after_us},
        "replan": {"demand_steps": n_steps, "swaps": len(ev), "cross_layer_swaps": moved,
                   "bytes_h2d": len(ev) * sa.arena.slot_bytes, "seconds": replan_s,
                   "GB_per_s_h2d": len(ev) * sa.arena.slot_bytes / replan_s / 1e9},
        "hot_ring": ring_block,
    }
    log(f"arena40: gate/up {gu_us:.1f} us ({roof['frac']:.3f} of peak); layer "
        f"{block['layer']['GB_per_s']:.0f} GB/s; re-plan {len(ev)} swaps in {replan_s:.3f} s; "
        f"{after_us:.1f} us per layer call after it")
    del sa
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("arena40: timing the CPU oracle on one layer call")
        lay = model.layers[0]
        lay.x_bits = model.tokens(0)
        block["cpu_baseline"] = cpu_baseline(
            lay, k, what="one of the 40 layer calls of a step (layer 0, its own resident set)")
    return block


def hot_ring_cost(model, sa, buf, ws, bs, xs, s0, ring_slot0, stream, dev) -> dict:
    """Decode steps with the asynchronous hot ring against the same steps
    without it (TideLM README, "How adaptive expert loading works", item 3,
    DeepSeek bullet: the pages report the ring's decode cost as a rate with
    and without it).  Both runs start from the same tables and tokens; with
    the ring, each step's heaviest misses are planned on the device after the
    step, copied into ring entries on a side stream while the next step runs,
    and routable from the step after.  Timed with events on the layer stream
    around RING_STEPS steps (the host waits for a plan one step behind, so the
    GPU never idles for it)."""
    import torch
    from resident_expert_routing_amd import runtime as R
    L = model.L
    mk = lambda: torch.cuda.Event(enable_timing=True)
    table_keep = sa.table.clone()
    hist_keep = sa.hist.clone()

    def run(with_ring):
        sa.table.copy_(table_keep)
        ring = R.HotRing(sa, ring_slot0, RING_SLOTS, RING_PER_STEP, model.pair_bytes, dev) \
            if with_ring else None
        torch.cuda.synchronize()
        e0, e1 = mk(), mk()
        e0.record(stream)
        for i in range(RING_STEPS):
            if ring:
                ring.before_step(i, stream)
            for l in range(L):
                R.route(buf, xs[s0 + i], ws[l], bs[l], sa.table[l], stream, hist_row=sa.hist[l],
                        delta=ring.delta_row(l) if ring else None)
                R.experts(buf, sa.arena.ptr(), sa.arena.stride, stream)
            if ring:
                ring.after_step(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (RING_STEPS * L)
        # assignments the last step's last layer sent to ring slots (a sample of the effect)
        routed_ring = int((buf.sel_slot >= ring_slot0).sum())
        out = {"us_per_layer_call": us, "tokens_per_s": xs.shape[1] / (us * 1e-6)}
        if ring:
            out.update({"picks": ring.n_picks,
                        "bytes_h2d": ring.bytes_copied,
                        "last_layer_assignments_on_ring_slots": routed_ring})
        return out

    off = run(False)
    on = run(True)
    sa.table.copy_(table_keep)
    sa.hist.copy_(hist_keep)
    torch.cuda.synchronize()
    log(f"hot ring: {on['us_per_layer_call']:.1f} us per layer call with it, "
        f"{off['us_per_layer_call']:.1f} without ({on['picks']} picks, "
        f"{on['bytes_h2d'] / 1e9:.2f} GB copied)")
    return {"ring_entries": RING_SLOTS, "picks_per_step": RING_PER_STEP, "steps": RING_STEPS,
            "on": on, "off": off,
            "rate_ratio_on_over_off": off["us_per_layer_call"] / on["us_per_layer_call"]}


def prepack(names) -> None:
    """Pack every expert content the chosen workloads upload, before the GPU
    is touched (the packer runs in worker processes)."""
    import fixtures
    for name in names:
        if name == "arena40":
            fixtures.make_arena_model("arena40").prepack()
        else:
            fixtures.make_layer(name).prepack()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this layer build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    names = ["decode", "prefill", "long", "arena40"] if args.workload == "all" else [args.workload]
    log(f"packing expert contents for {', '.join(names)}")
    prepack(names)

    import torch
    import resident_expert_routing_amd  # noqa: F401  (loads libmoe_arena.so; fails loudly)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    blocks = {}
    for name in names:
        if name == "arena40":
            blocks[name] = arena40_workload(args, dev, min(args.warmup, 10))
        elif name == names[0]:
            blocks[name] = layer_workload(name, args, dev, args.steps, args.warmup)
        else:   # the other layer workloads: 20 timed steps (the protocol's count for them)
            blocks[name] = layer_workload(name, args, dev, min(args.steps, 20),
                                          min(args.warmup, 5))
    head = blocks[names[0]]
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": head["warmup"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": head["config"],
    }
    for key in ("roofline", "layer", "replan", "hot_read", "act_mxfp6", "cpu_baseline"):
        if key in head:
            result[key] = head[key]
    if len(names) > 1:
        result["workloads"] = {n: blocks[n] for n in names[1:]}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
