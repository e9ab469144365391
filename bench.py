#!/usr/bin/env python3
"""Benchmark of the Muon hot path on one MI355X.

A step is one whole Muon hot-path pass over the GPT-2 124M hidden-matrix set
(12 layers x 768x2304, 768x768, 768x3072, 3072x768; synthetic rank-16 plus
noise gradients and N(0, 0.1^2) momentum buffers, seed 1): one
muon_momentum_ns5_batched call, i.e. Nesterov momentum on all 48 gradients
fused with the first pass of the norm, then NS5 of every momentum output with
one launch per product and NS5 step over all 48 matrices.  Inputs are
resident in HBM before the timed region.  The call is captured once in a HIP
graph, and the timed steps are replays of it (every kernel of the step runs
in each replay; the host enqueues nothing between them).

Printed (one JSON line on stdout):
  value          nominal NS5 flops of the step, sum of 5 (4 m^2 n + 2 m^3),
                 divided by the measured step time (momentum included), TFLOP/s
  ms_per_step    the step time (graph replays)
  eager_ms_per_step  the same step called from the host K times
  roofline       the dominant kernel (the a X + B X product of NS5 steps 1-4)
                 timed with HIP events around each of its launches, against
                 the bf16 dense MFMA peak
  momentum       the stand-alone momentum kernel (16 bytes per element) against
                 HBM
  ns5_4096       NS5 of one 4096x4096 matrix (U diag(s) V^T, seed 3)
  apply_step     the same step with the parameter update p <- p - lr * O
                 fused into the last epilogue (muon_momentum_ns5_apply_batched)
  f32_iteration  the same 48 matrices through the iteration carried in float32
                 (muon_newton_schulz_f32_batched), against the float32 matrix
                 peak, and its time over the bf16 NS5 of the same matrices
  single_64x128  one 64x128 Muon step (momentum + NS5) and its 128x64
                 transpose, microseconds per call (one launch each)
  gpt2_1p5b      the GPT-2 1.5B hidden set (192 matrices, 48 layers x 1600x4800,
                 1600x1600, 1600x6400, 6400x1600), one fused Muon step
  extreme_aspect eight 2048x8192 and eight 8192x2048 matrices, one batched NS5
  polar_svd      U V^T of the 48 124M momentum outputs through an SVD on the
                 GPU (block one-sided Jacobi), against NS5 of the same matrices
  cpu_baseline   the CPU oracle on a bounded sample of the same step
  cpu_samples    the CPU oracle on samples of the other workloads, scaled to
                 their whole size

Every NS5 rate is given twice: on the nominal flops 5 (4 m^2 n + 2 m^3) of
the metric, and on the symmetry-aware minimum 5 (3 m^2 n + m^3) (X X^T and
A A are symmetric, so half of each is a mirror); the kernels compute upper
tiles only, so the second is the closer measure of the matrix cores' work.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "NS5 TFLOP/s (bf16) & % MFMA peak; ms per GPT-2-124M-shaped Muon step"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
PEAK_F32_TFLOPS = 157.3     # MI355X dense float32 matrix-core peak (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--skip-cpu-baseline", action="store_true")
    p.add_argument("--skip-square", action="store_true", help="skip the 4096x4096 NS5 line")
    p.add_argument("--skip-extras", action="store_true", help="only the timed step (for profiling)")
    p.add_argument("--only", choices=["square_4096", "extreme_aspect", "gpt2_1p5b", "single_64x128", "polar_svd"],
                   help="time only this workload (for profiling its kernels); prints its line alone")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device-to-device copy of COPY_BYTES bytes (10 times), the reference "
                        "kernel whose FETCH_SIZE / WRITE_SIZE readings scale the traffic counters")
    return p.parse_args()


COPY_BYTES = 1 << 30

# HBM-side traffic of the dominant kernel per launch, from two rocprofv3 --pmc
# runs over `MUON_SPLIT=0 bench.py --steps 2 --warmup 1 --skip-extras` (the
# step on one stream, so that it runs the launch over all 48 matrices;
# FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), scaled by what the same
# counters read for
# the 1 GiB copy of `bench.py --copy-calibration` (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0).  Valid only for the kernel sources it was measured with:
# reported as null once their hash differs (the summary is
# profiles/gpt2_124m_step_traffic.md).
TRAFFIC = {
    "sources_sha256": "92a53af61601dedb3f47ab6e6169f8fbe05ee69c9094b972eafb90972c317dd9",
    "fetch_bytes": 285517379,
    "write_bytes": 169869312,
}
TRAFFIC_SOURCES = ("newton_schulz_09_amd/csrc/gemm.hip", "newton_schulz_09_amd/csrc/api.hip",
                   "newton_schulz_09_amd/csrc/internal.hpp", "newton_schulz_09_amd/csrc/common.hpp")


def sources_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    if TRAFFIC["sources_sha256"] is None or TRAFFIC["sources_sha256"] != sources_hash():
        return None
    return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]


def copy_calibration(torch):
    """A plain copy of a known size: 1 GiB read + 1 GiB written per launch."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(10):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / 10
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "ms": round(ms, 4),
                      "GB/s (read+write)": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}), flush=True)


def time_step(run, steps, torch):
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def capture_step(st, torch):
    """The step captured once in a HIP graph: the kernels of one
    muon_momentum_ns5_batched call (its side streams forked from and joined
    into the capturing stream by events), so that a replay runs the whole
    step with no host work between its launches.  One untimed step on the
    capturing stream first (library set-up stays out of the capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.fused_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.fused_step()
    torch.cuda.synchronize()
    return graph


def time_dominant_kernel(st, steps, torch):
    """Second timed pass: the same steps, with HIP events recorded by the
    library around every a X + B X launch of NS5 steps 1-4, each launch over
    all 48 matrices: the kernel measured alone (the library's measurement
    hook keeps the whole batch on the caller's stream; the timed step runs
    every product as three launches of 16 matrices on three streams, whose
    durations overlap other work)."""
    max_pairs = 4 * (st.steps - 1)      # room for several launch groups
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * max_pairs)] for _ in range(steps)]
    for evs in events:                  # create the underlying HIP events
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    recorded = []
    for s in range(steps):
        st.fused_step(events=events[s])
        recorded.append(st.last_recorded())
    torch.cuda.synchronize()
    total_ms, launches = 0.0, 0
    for s in range(steps):
        for p in range(recorded[s]):
            total_ms += events[s][2 * p].elapsed_time(events[s][2 * p + 1])
            launches += 1
    groups_per_call = recorded[0] // (st.steps - 1)
    if groups_per_call != 1:
        raise RuntimeError(f"expected one launch group for the step, got {groups_per_call}")
    flops_per_launch = sum(2.0 * min(r, c) ** 2 * max(r, c) for r, c in st.shapes)
    avg_ms = total_ms / launches
    achieved = flops_per_launch / (avg_ms * 1e-3) / 1e12
    return {
        "bound": "mfma",
        "kernel": "k_gemm_nt<256, 256, 64, 2, 2, 4, GEMM_BX> (256x256 tiles, 8 waves): X' = a X + B X of NS5 steps 1-4, one launch over all "
                  "48 matrices, measured alone (the step runs it as three concurrent launches of 16)",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(),
        "launches": launches,
        "avg_launch_us": round(avg_ms * 1e3, 2),
        "flops_per_launch": flops_per_launch,
    }


def time_momentum(st, steps, torch):
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.momentum()
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        st.momentum()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    gbs = st.momentum_bytes() / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "bytes": st.momentum_bytes()}


def time_apply_step(st, steps, torch, lr=0.02):
    st.apply_step(lr)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        st.apply_step(lr)
    stop.record()
    torch.cuda.synchronize()
    return {"ms": round(start.elapsed_time(stop) / steps, 4), "lr": lr}


def time_square(torch, muon, workloads, reps=10):
    G, _, _, _ = workloads.square_4096()
    g = torch.from_numpy(G).cuda()
    out = torch.empty_like(g)
    ms = _timed(torch, lambda: muon.ns5(g, out), reps, warm=3)
    res = {"ms": round(ms, 4)}
    res.update(_rates(muon.ns5_flops(4096, 4096), sym_min_flops(4096, 4096), ms))
    return res


def time_f32_iteration(st, torch, muon, reps=3):
    """The same 48 matrices through the iteration carried in float32
    (muon_newton_schulz_f32_batched: no bf16 anywhere, float32 MFMA products),
    next to NS5 of the same matrices in bf16 (muon_ns5_batched), both on the
    momentum outputs already in HBM."""
    st.momentum()   # u = g + mu buf: real values (constant operands would flatter the matrix cores)
    outs = [torch.empty_like(u) for u in st.us]
    ws = torch.empty(muon.f32_workspace_size(st.shapes), dtype=torch.uint8, device=st.device)
    timings = {}
    for name, fn in (("f32", lambda: muon.newton_schulz_f32(st.us, outs, workspace=ws)),
                     ("bf16", lambda: muon.ns5_batched(st.us, outs, workspace=st.workspace))):
        fn()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        timings[name] = start.elapsed_time(stop) / reps
    tf = st.nominal_ns5_flops() / (timings["f32"] * 1e-3) / 1e12
    return {"ms": round(timings["f32"], 3), "TFLOP/s": round(tf, 2), "pct_f32_mfma_peak": round(100 * tf / PEAK_F32_TFLOPS, 2),
            "bf16_ns5_ms": round(timings["bf16"], 4), "f32_over_bf16": round(timings["f32"] / timings["bf16"], 2)}


def sym_min_flops(rows, cols, steps=5):
    """Symmetry-aware minimum NS5 flops, 5 (3 m^2 n + m^3): the upper half of
    X X^T (m^2 n) and of A A (m^3), and all of B X (2 m^2 n)."""
    m, n = min(rows, cols), max(rows, cols)
    return steps * (3 * m * m * n + m ** 3)


def _rates(nominal, symmin, ms):
    tf = nominal / (ms * 1e-3) / 1e12
    tf_min = symmin / (ms * 1e-3) / 1e12
    return {"TFLOP/s": round(tf, 2), "pct_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "TFLOP/s_symmetric_min": round(tf_min, 2),
            "pct_mfma_peak_symmetric_min": round(100 * tf_min / PEAK_BF16_TFLOPS, 2)}


def _timed(torch, fn, reps, warm=2, settle_ms=100.0):
    """Mean ms per call of `fn` over `reps` calls, after an untimed warm-up
    of at least `warm` calls and `settle_ms` of GPU time: the clocks take some
    tens of ms of matrix work to settle after other work or idle time (one
    4096^2 NS5 measured 1.55 ms over its first 10 calls, 1.41 ms from the
    20th on)."""
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(warm):
        fn()
    stop.record()
    torch.cuda.synchronize()
    per_call = start.elapsed_time(stop) / max(warm, 1)
    for _ in range(math.ceil(max(0.0, settle_ms - per_call * warm) / max(per_call, 1e-3))):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / reps


def time_single_64x128(torch, muon, workloads, reps=200):
    """The 64x128 matrix and its 128x64 transpose: one Muon step each
    (muon_momentum_ns5_batched on one matrix), microseconds per call."""
    G, buf = workloads.single_64x128()
    res = {}
    for name, M, B in (("64x128", G, buf), ("128x64", G.T, buf.T)):
        g = torch.from_numpy(M.copy()).cuda()
        b = torch.from_numpy(B.copy()).cuda()
        o = torch.empty_like(g)
        ms = _timed(torch, lambda: muon.ns5_batched([g], [o], bufs=[b]), reps, warm=5)
        res[f"us_per_call_{name}"] = round(ms * 1e3, 2)
    g2 = [torch.from_numpy(G.copy()).cuda(), torch.from_numpy(G.T.copy()).cuda()]
    b2 = [torch.zeros_like(x) for x in g2]
    o2 = [torch.empty_like(x) for x in g2]
    res["us_per_call_both_batched"] = round(_timed(torch, lambda: muon.ns5_batched(g2, o2, bufs=b2), reps, 5) * 1e3, 2)
    return res


def time_gpt2_1p5b(torch, muon, step, workloads, reps=5):
    """One fused Muon step over the GPT-2 1.5B hidden set (192 matrices)."""
    t0 = time.time()
    items = workloads.gpt2_1p5b()
    st = step.MuonStep([it[2].shape for it in items], device="cuda:0")
    for k, (_, _, G, buf) in enumerate(items):
        st.grads[k].copy_(torch.from_numpy(G))
        st.bufs[k].copy_(torch.from_numpy(buf))
    del items
    torch.cuda.synchronize()
    log(f"gpt2-1.5b inputs ready in {time.time() - t0:.1f} s")
    ms = _timed(torch, st.fused_step, reps)
    res = {"ms_per_step": round(ms, 3), "matrices": len(st.shapes), "nominal_ns5_flops": st.nominal_ns5_flops(),
           "momentum_bytes": st.momentum_bytes()}
    res.update(_rates(st.nominal_ns5_flops(), sum(sym_min_flops(r, c) for r, c in st.shapes), ms))
    del st
    torch.cuda.empty_cache()
    return res


def time_extreme_aspect(torch, muon, workloads, reps=5):
    """Eight 2048x8192 and eight 8192x2048 matrices in one muon_ns5_batched
    call (pure NS5, no momentum)."""
    items = workloads.extreme_aspect()
    Gs = [torch.from_numpy(it[0]).cuda() for it in items]
    shapes = [tuple(g.shape) for g in Gs]
    del items
    outs = [torch.empty_like(g) for g in Gs]
    ws = torch.empty(muon.batched_workspace_size(shapes), dtype=torch.uint8, device="cuda")
    ms = _timed(torch, lambda: muon.ns5_batched(Gs, outs, workspace=ws), reps)
    nominal = sum(muon.ns5_flops(r, c) for r, c in shapes)
    res = {"ms": round(ms, 3), "matrices": len(shapes), "nominal_ns5_flops": nominal}
    res.update(_rates(nominal, sum(sym_min_flops(r, c) for r, c in shapes), ms))
    return res


def time_polar_svd(st, torch, muon, reps=2):
    """U V^T of the 48 GPT-2 124M momentum outputs through an SVD on the GPU
    (muon_polar_svd_grouped, one call per shape class), next to NS5 of the
    same matrices (one muon_ns5_batched call): how much slower the SVD route
    is, the claim of the Muon section."""
    st.momentum()   # u = g + mu buf in HBM: the matrices both routes orthogonalise
    classes = {}
    for k, shape in enumerate(st.shapes):
        classes.setdefault(shape, []).append(st.us[k])
    outs = {sh: [torch.empty_like(t) for t in v] for sh, v in classes.items()}
    ws = torch.empty(max(muon.polar_svd_workspace_size(*sh, len(v)) for sh, v in classes.items()),
                     dtype=torch.uint8, device=st.device)
    svd_ms = _timed(torch, lambda: [muon.polar_svd_grouped(v, outs[sh], workspace=ws) for sh, v in classes.items()],
                    reps, warm=1)
    ns5_ms = _timed(torch, lambda: muon.ns5_batched(st.us, st.outs, workspace=st.workspace), 10, warm=2)
    return {"svd_ms": round(svd_ms, 2), "ns5_ms": round(ns5_ms, 4), "svd_over_ns5": round(svd_ms / ns5_ms, 1),
            "matrices": len(st.shapes), "method": "block one-sided Jacobi, float32 storage, float64 arithmetic, "
                                                  "at most 16 sweeps, all matrices of a shape class per launch"}


def _loaded_step(torch, step, workloads):
    items = workloads.gpt2_124m()
    st = step.MuonStep([it[2].shape for it in items], device="cuda:0")
    for k, (_, _, G, buf) in enumerate(items):
        st.grads[k].copy_(torch.from_numpy(G))
        st.bufs[k].copy_(torch.from_numpy(buf))
    return st


def cpu_samples(workloads):
    """The oracle on bounded samples of the other workloads, each scaled to
    its whole size: the 64x128 step and its transpose whole (median of 3);
    the 4096x4096 NS5 from its normalisation and one step, scaled to five
    steps; one matrix of each of the four GPT-2 1.5B shape classes
    (momentum + NS5), scaled by 48; one 2048x8192 and one 8192x2048 matrix
    (NS5), scaled by 8."""
    import oracle
    res = {}
    G, buf = workloads.single_64x128()
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        for M, B in ((G, buf), (G.T, buf.T)):
            _, u = oracle.momentum_nesterov(M, B, 0.95)
            oracle.ns5(u)
        runs.append(time.perf_counter() - t0)
    res["single_64x128_ms"] = round(sorted(runs)[1] * 1e3, 2)
    G, _, _, _ = workloads.square_4096()
    t0 = time.perf_counter()
    oracle.ns5(G, steps=0)
    t_norm = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.ns5(G, steps=1)
    t_one = time.perf_counter() - t0
    res["square_4096_s"] = round(t_norm + 5 * (t_one - t_norm), 1)
    res["square_4096_sample"] = (f"the normalisation alone ({t_norm:.1f} s) and with one NS5 step ({t_one:.1f} s): "
                                 f"normalisation + 5 steps")
    t0 = time.perf_counter()
    for si in range(4):
        _, _, G, buf = workloads.gpt_hidden_set(workloads.GPT2_1P5B_SHAPES, 1, 4, only_shape=si)[0]
        _, u = oracle.momentum_nesterov(G, buf, 0.95)
        oracle.ns5(u)
    dt = time.perf_counter() - t0
    res["gpt2_1p5b_s_per_step"] = round(dt * workloads.GPT2_1P5B_LAYERS, 1)
    res["gpt2_1p5b_sample"] = f"layer 0, one matrix per shape class: {dt:.1f} s, x 48 layers"
    t0 = time.perf_counter()
    for it in workloads.extreme_aspect(indices=[0, 8]):
        oracle.ns5(it[0])
    dt = time.perf_counter() - t0
    res["extreme_aspect_s"] = round(dt * 8, 1)
    res["extreme_aspect_sample"] = f"matrices 0 (2048x8192) and 8 (8192x2048): {dt:.1f} s, x 8"
    return res


def cpu_baseline(items):
    """The oracle, as it stands, on the whole step (all 48 matrices: momentum
    then NS5), timed on this host's cores."""
    import threadpoolctl

    import oracle
    flops = sum(oracle.ns5_nominal_flops(*it[2].shape) for it in items)
    t0 = time.perf_counter()
    for _, _, G, buf in items:
        _, u = oracle.momentum_nesterov(G, buf, 0.95)
        oracle.ns5(u)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole GPT-2 124M step (48 matrices, momentum + NS5) once: {flops:.4g} nominal NS5 "
                      f"flops in {dt:.1f} s, {dt * 1e3:.0f} ms per step (float64 BLAS matmuls on {threads} "
                      "threads, bf16 rounding in numpy)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the Muon hot path here has no multi-GPU path "
              "(see the sharding design); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    from newton_schulz_09_amd import muon, step, workloads

    if args.only:
        fn = {"square_4096": lambda: time_square(torch, muon, workloads),
              "extreme_aspect": lambda: time_extreme_aspect(torch, muon, workloads),
              "gpt2_1p5b": lambda: time_gpt2_1p5b(torch, muon, step, workloads),
              "single_64x128": lambda: time_single_64x128(torch, muon, workloads),
              "polar_svd": lambda: time_polar_svd(_loaded_step(torch, step, workloads), torch, muon)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return

    t0 = time.time()
    items = workloads.gpt2_124m()
    st = step.MuonStep([it[2].shape for it in items], device="cuda:0")
    for k, (_, _, G, buf) in enumerate(items):
        st.grads[k].copy_(torch.from_numpy(G))
        st.bufs[k].copy_(torch.from_numpy(buf))
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s: {len(items)} matrices, {st.total} floats per buffer")

    for _ in range(args.warmup):
        st.fused_step()
    torch.cuda.synchronize()
    eager_ms = time_step(st.fused_step, args.steps, torch)
    log(f"step, called from the host: {eager_ms:.4f} ms")
    graph = capture_step(st, torch)
    for _ in range(args.warmup):
        graph.replay()
    ms = time_step(graph.replay, args.steps, torch)
    flops = st.nominal_ns5_flops()
    value = flops / (ms * 1e-3) / 1e12
    log(f"step, replayed from a HIP graph: {ms:.4f} ms, {value:.1f} TFLOP/s nominal NS5")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gpt2_124m_hidden_set",
            "matrices": len(items),
            "layers": 12,
            "shapes": ["768x2304", "768x768", "768x3072", "3072x768"],
            "mu": 0.95,
            "ns5_steps": 5,
            "eps": 1e-7,
            "nominal_ns5_flops": flops,
            "launch": "one muon_momentum_ns5_batched call per step, captured once in a HIP graph and replayed",
        },
        "eager_ms_per_step": round(eager_ms, 4),
        "pct_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
    }
    symmin = sum(sym_min_flops(r, c) for r, c in st.shapes)
    res["pct_mfma_peak_symmetric_min"] = round(100 * symmin / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)
    props = torch.cuda.get_device_properties(0)
    res["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                     "compute_units": props.multi_processor_count, "hbm_gib": round(props.total_memory / 2**30, 1)}
    if not args.skip_extras:
        res["roofline"] = time_dominant_kernel(st, args.steps, torch)
        log(f"dominant kernel: {res['roofline']}")
        res["momentum"] = time_momentum(st, args.steps, torch)
        log(f"momentum: {res['momentum']}")
        res["apply_step"] = time_apply_step(st, args.steps, torch)
        log(f"apply step: {res['apply_step']}")
        res["f32_iteration"] = time_f32_iteration(st, torch, muon)
        log(f"float32 iteration: {res['f32_iteration']}")
        res["polar_svd"] = time_polar_svd(st, torch, muon)
        log(f"polar svd: {res['polar_svd']}")
        if not args.skip_square:
            res["ns5_4096"] = time_square(torch, muon, workloads)
            log(f"ns5 4096: {res['ns5_4096']}")
        res["single_64x128"] = time_single_64x128(torch, muon, workloads)
        log(f"64x128: {res['single_64x128']}")
        res["extreme_aspect"] = time_extreme_aspect(torch, muon, workloads)
        log(f"extreme aspect: {res['extreme_aspect']}")

        del st
        torch.cuda.empty_cache()
        res["gpt2_1p5b"] = time_gpt2_1p5b(torch, muon, step, workloads)
        log(f"gpt2 1.5b: {res['gpt2_1p5b']}")
        if not args.skip_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline(items)
            log(f"cpu baseline: {res['cpu_baseline']}")
            res["cpu_samples"] = cpu_samples(workloads)
            log(f"cpu samples: {res['cpu_samples']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
