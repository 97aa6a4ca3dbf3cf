"""Benchmark of the MI355X Muon / Dimuon optimizer step.

One step = one pass of the whole hot path (momentum, conditioning, Frobenius
normalisation, Newton-Schulz iterations, post-scale, weight update) over one
batch of matrices whose inputs are already resident in HBM.

Default workload: the LoRA batch (64 pairs of 8 x 4096 and 4096 x 8, fp32
master weights, Dimuon).  Its 84 MB per step would fit the 256 MiB Infinity
Cache, so independent buffer sets are rotated until the bytes resident across
the rotation are at least twice that cache.  The GPT-2, square
4096^2 and MoE batches are measured as well and reported under
"workloads".

Prints one JSON line.  Rank 0 only; one GPU (`--gpus` above 1 is refused).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}

# HBM bytes per launch of the thin-path kernels on the LoRA batch, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch), FETCH_SIZE scaled by 2.0 and WRITE_SIZE by 1.0: what the same
# counters read for a 256 MiB device-to-device copy (--copy-probe).  Valid only
# for the kernel sources they were taken on (sha256 of thin_kernel.hip and
# common.h); the figures and the commands are in
# profiles/k_thin_lora_batch_64x8x4096.md.
THIN_SOURCES = ("dimuon_newton_schulz_amd/csrc/thin_kernel.hip", "dimuon_newton_schulz_amd/csrc/common.h")
MEASURED_TRAFFIC = {
    "sources_sha256": "e35e3c4802044f21fb56a03786e5766071f0f5d903b32c8d9217c7ef0e710aeb",
    "k_thin_a": {"fetch_kib": 17684.7, "write_kib": 19012.0},
    "k_thin_b": {"fetch_kib": 18036.1, "write_kib": 18468.0},
}
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0

# The same counters for the combine kernel of the GEMM workloads (one
# iteration before the last, on the tiles those iterations use; a product
# with a tail launch lists both launches), plus the matrix-core counters of
# that kernel: bf16 MFMA busy cycles over the active cycles of the 1024 SIMDs
# (GRBM_GUI_ACTIVE summed over the 8 XCDs, divided by 8), and the clock those
# active cycles imply.  Each workload was counted on its own inputs.  Valid
# only for the GEMM and planner sources they were taken on; figures and
# commands in profiles/gemm_counters_gpt2_square_moe.md.
GEMM_SOURCES = ("dimuon_newton_schulz_amd/csrc/gemm_kernels.hip", "dimuon_newton_schulz_amd/csrc/api.hip",
                "dimuon_newton_schulz_amd/csrc/common.h")
MEASURED_GEMM = {
    "sources_sha256": "cf7e0845c718b4c011d8f77514d35717d007443866948b486c52999ccee92a78",
    "gpt2_small_12x4_bf16": {"fetch_kib": [134273.6, 5270.3], "write_kib": [163840.1, 2048.0],
                             "mfma_busy_frac": 0.363, "clock_ghz": 2.17},
    "square_8x4096x4096_bf16": {"fetch_kib": [786652.0], "write_kib": [262231.2],
                                "mfma_busy_frac": 0.573, "clock_ghz": 1.94},
    "moe_64x(2048x1408+1408x2048)_bf16": {"fetch_kib": [968372.0], "write_kib": [786466.5],
                                          "mfma_busy_frac": 0.475, "clock_ghz": 1.92},
}


def sources_sha(rels):
    import hashlib
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_gemm(workload):
    """Counter figures of a GEMM workload's combine (HBM bytes per iteration,
    matrix-core busy fraction), or None if the sources changed since."""
    rec = MEASURED_GEMM.get(workload)
    if rec is None or sources_sha(GEMM_SOURCES) != MEASURED_GEMM["sources_sha256"]:
        return None
    nbytes = sum(f * FETCH_SCALE + w * WRITE_SCALE for f, w in zip(rec["fetch_kib"], rec["write_kib"])) * 1024
    return {"traffic": int(round(nbytes)), "mfma_busy_frac": rec["mfma_busy_frac"], "clock_ghz": rec["clock_ghz"]}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter runs, or None if the
    kernel sources changed since they were taken."""
    rec = MEASURED_TRAFFIC.get(kernel)
    if rec is None or sources_sha(THIN_SOURCES) != MEASURED_TRAFFIC["sources_sha256"]:
        return None
    return int(round((rec["fetch_kib"] * FETCH_SCALE + rec["write_kib"] * WRITE_SCALE) * 1024))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--variant", default=None, choices=[None, "muon", "dimuon"])
    ap.add_argument("--extra", default="c3:muon,c4:dimuon,c4:muon,c5:dimuon,c4:muon:f32",
                    help="comma list of config:variant[:ns dtype] measured besides the main one, or 'none'")
    ap.add_argument("--extra-steps", type=int, default=10)
    ap.add_argument("--sets", type=int, default=0,
                    help="buffer sets rotated (0: automatic, enough that the rotation's resident bytes "
                         "exceed twice the 256 MiB Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-toy", action="store_true", help="skip the 4 x 16 toy's column-share report")
    ap.add_argument("--graph", action="store_true",
                    help="time the plans replaying their launch sequences as HIP graphs")
    ap.add_argument("--ns-dtype", default=None, choices=[None, "bf16", "f32"],
                    help="precision of the Newton-Schulz products (default: the workload's)")
    ap.add_argument("--next", action="store_true",
                    help="turn on the extensions together: Nesterov input, decoupled weight decay 0.01, a "
                         "per-iteration coefficient schedule and a per-matrix update scale of 0.5")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="bytes of a plain device-to-device copy run once before the workload "
                         "(calibrates HBM byte counters against a known size)")
    return ap.parse_args()


_BUILT = {}


def make_workload(name, device, variant=None):
    """The configuration's batch on the device.  The square set (32 float64
    QRs on the host) is built once per process and shared by its variants;
    every measurement steps clones of the tensors."""
    import workloads as W
    if name in _BUILT:
        wl = _BUILT[name]
    elif name == "c1":
        wl = W.lora_toy(seed=0, device=device)
    elif name == "c2":
        wl = W.lora_batch(device=device)
    elif name == "c3":
        wl = W.gpt2_hidden(device=device)
    elif name == "c4":
        wl = W.square_batch(device=device, variant=variant or "dimuon")
        _BUILT[name] = wl
    else:
        wl = W.moe_experts(device=device)
    if variant:
        wl.variant = variant
    return wl


def algorithmic(wl, is_thin):
    """Per-step algorithmic work.  Thin path: the bytes the step must move
    (read G and M_{t-1}, write M_t, read and write W: 20 B per f32 element);
    a two-pass step splits them as pass A (G, M_{t-1}, M_t) and pass B (W
    read and write).  Pass B's second read of M_t, the energy cache, the
    factors and the Gram partials are not counted.  MFMA path: NS flops
    (symmetric products counted once)."""
    size = {"f32": 4, "bf16": 2}
    per_elem = size[wl.g_dtype] + 2 * size[wl.mom_dtype] + 2 * size[wl.w_dtype]
    per_a = size[wl.g_dtype] + 2 * size[wl.mom_dtype]
    per_b = 2 * size[wl.w_dtype]
    a_bytes = b_bytes = gram = poly = comb = 0
    for m in wl.mats:
        rows, cols = m.shape
        k, n = min(rows, cols), max(rows, cols)
        if is_thin(rows, cols):
            a_bytes += rows * cols * per_a
            b_bytes += rows * cols * per_b
        else:
            gram += k * k * n
            poly += k ** 3
            comb += 2 * k * k * n
    return {"thin_a_bytes": a_bytes, "thin_b_bytes": b_bytes, "thin_bytes": a_bytes + b_bytes,
            "gram_flops": gram, "poly_flops": poly, "comb_flops": comb,
            "hbm_bytes_min": sum(m.shape[0] * m.shape[1] for m in wl.mats) * per_elem,
            "input_bytes": sum(m.shape[0] * m.shape[1] for m in wl.mats) * (size[wl.g_dtype] + size[wl.mom_dtype]
                                                                            + size[wl.w_dtype])}


def is_thin(m, n):
    """Same rule as the library's planner: Gram side <= 32."""
    return min(m, n) <= 32


# Buffer-set rotation: enough independent sets (W, G, M and workspace each)
# that the bytes resident across the rotation are at least twice the 256 MiB
# Infinity Cache, so that no step finds its operands left in it by the last.
ROTATION_TARGET_BYTES = 2 * 256 * 2 ** 20
MAX_SETS = 64


# The extensions' settings for --next.  The schedule keeps the quintic's
# coefficients for the first iterations and ends on the classical
# Newton-Schulz quintic (15/8, -10/8, 3/8); the values only steer the
# arithmetic, the cost is the same for any schedule.
NEXT_SETTINGS = {"nesterov": True, "weight_decay": 0.01, "update_scale": 0.5,
                 "coeff_schedule": [(3.4445, -4.7750, 2.0315)] * 4 + [(1.875, -1.25, 0.375)]}


def measure(wl, steps, warmup, sets=0, ns_dtype=None, graph=False, next_features=False):
    import torch
    import dimuon_newton_schulz_amd as D

    cfg = D.StepConfig(lr=wl.lr, momentum=wl.mu, ns_steps=wl.ns_steps, w_dtype=wl.w_dtype,
                       g_dtype=wl.g_dtype, mom_dtype=wl.mom_dtype, ns_dtype=ns_dtype or wl.ns_dtype)
    scale = 1.0
    if next_features:
        cfg.nesterov = NEXT_SETTINGS["nesterov"]
        cfg.weight_decay = NEXT_SETTINGS["weight_decay"]
        cfg.coeff_schedule = NEXT_SETTINGS["coeff_schedule"][:wl.ns_steps]
        scale = NEXT_SETTINGS["update_scale"]
    dimuon = wl.variant == "dimuon"
    plans = []

    def new_plan():
        params = [D.Param(w=m.w.clone(), g=m.g.clone(), mom=m.m_prev.clone(), update_scale=scale) for m in wl.mats]
        plans.append(D.Plan(params, cfg, dimuon=dimuon))

    new_plan()
    # Bytes one set keeps resident: W, G, M and the plan's workspace.
    per_set = algorithmic(wl, is_thin)["input_bytes"] + plans[0].workspace.numel()
    if sets <= 0:
        sets = min(MAX_SETS, max(1, -(-ROTATION_TARGET_BYTES // per_set)))
    while len(plans) < sets:
        new_plan()
    if graph:
        for p in plans:
            p.set_graph(True)
    torch.cuda.synchronize()
    # With graphs, every plan first runs its eager step and captures both of
    # its states before the timed region.
    for i in range(warmup + (3 * sets if graph else 0)):
        plans[i % sets].step()
    torch.cuda.synchronize()

    # Timed region: K steps, HIP events around it on the library's stream.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        plans[i % sets].step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps

    # Same K steps again with one HIP event after every kernel launch (the
    # library's launch-event hook), for per-kernel durations.
    lib = D.load_library()
    per_step = 64
    n_ev = per_step * steps
    import ctypes
    events = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in events:
        e.record()
    torch.cuda.synchronize()
    handles = (ctypes.c_void_p * n_ev)(*[e.cuda_event for e in events])
    kinds = (ctypes.c_int32 * n_ev)()
    counts = []
    hs = ctypes.sizeof(ctypes.c_void_p)
    for i in range(steps):
        base = i * per_step
        lib.muon_set_launch_events(ctypes.cast(ctypes.addressof(handles) + base * hs, ctypes.c_void_p),
                                   ctypes.cast(ctypes.addressof(kinds) + base * 4,
                                               ctypes.POINTER(ctypes.c_int32)), per_step)
        plans[i % sets].step()
        counts.append(lib.muon_set_launch_events(None, None, 0))
    torch.cuda.synchronize()
    # Each event marker between two launches delays the next dispatch; the
    # marker overhead per launch is the instrumented step time minus the
    # plain one, spread over the step's launches, and is taken off each
    # kernel's event interval.
    hooked = sum(events[i * per_step].elapsed_time(events[i * per_step + counts[i] - 1]) for i in range(steps))
    launches = sum(counts) - steps
    overhead = max(0.0, hooked - ms * steps) / max(launches, 1)
    per_kind = {}
    for i in range(steps):
        base = i * per_step
        for j in range(1, counts[i]):
            kind = D.LAUNCH_KINDS[kinds[base + j]]
            dt = max(events[base + j - 1].elapsed_time(events[base + j]) - overhead, 0.0)
            tot, n = per_kind.get(kind, (0.0, 0))
            per_kind[kind] = (tot + dt, n + 1)
    for p in plans:
        p.close()
    del plans
    torch.cuda.empty_cache()
    return cfg, ms, per_kind, overhead, sets, per_set


THIN_KERNELS = {"thin_a": "k_thin_a", "thin_b": "k_thin_b", "thin": "k_thin_step"}


def roofline_for(wl, cfg, per_kind, work, steps):
    """Dominant kernel (largest total time) and its achieved rate."""
    kind = max(per_kind, key=lambda k: per_kind[k][0])
    tot_ms, launches = per_kind[kind]
    avg_ms = tot_ms / launches
    if kind in THIN_KERNELS:
        nbytes = work[kind + "_bytes"]
        achieved = nbytes / (avg_ms * 1e-3) / 1e9
        name = THIN_KERNELS[kind]
        traffic = measured_traffic(name)
        out = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
               "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
               "kernel": name, "avg_launch_ms": round(avg_ms, 5), "bytes_per_launch": nbytes}
        if traffic is not None:
            out["traffic_over_algorithmic"] = round(traffic / nbytes, 3)
        return kind, out
    flops = {"combine": work["comb_flops"], "gram": work["gram_flops"], "poly": work["poly_flops"]}.get(kind)
    if flops is None:
        # a streaming kernel dominates: report bytes of one pass
        achieved = work["hbm_bytes_min"] / (avg_ms * 1e-3) / 1e9
        return kind, {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None, "kernel": kind,
                      "avg_launch_ms": round(avg_ms, 5)}
    # A product may take two launches per iteration (a partial last round of
    # big tiles runs as 128 x 128 tiles): the rate is the product's flops over
    # its launches' time, per iteration.
    peak = PEAK_TFLOPS[cfg.ns_dtype]
    iters = steps * max(cfg.ns_steps, 1)
    per_iter = launches / iters
    achieved = flops * iters / (tot_ms * 1e-3) / 1e12
    names = {"combine": "k_combine_bf16", "gram": "k_syrk_bf16", "poly": "k_syrk_bf16"}
    out = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
           "frac": round(achieved / peak, 4), "traffic": None,
           "kernel": names[kind] if cfg.ns_dtype == "bf16" else names[kind].replace("bf16", "f32"),
           "avg_launch_ms": round(avg_ms, 5), "launches_per_iteration": round(per_iter, 3)}
    if per_iter == 1:
        out["flops_per_launch"] = flops
    else:
        out["flops_per_iteration"] = flops
    # (The committed counter figures are those of the bf16 products.)
    counted = measured_gemm(wl.name) if kind == "combine" and cfg.ns_dtype == "bf16" else None
    if counted is not None:
        out["traffic"] = counted["traffic"]
        if per_iter != 1:
            out["traffic_basis"] = "per iteration (all launches of the product)"
        out["counters"] = {"mfma_busy_frac": counted["mfma_busy_frac"], "clock_ghz": counted["clock_ghz"],
                           "source": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE"}
    return kind, out


def host_sample(name, variant):
    """Host copy of a representative slice of the workload for the oracle:
    the whole batch when it is small (the toy, the LoRA batch), otherwise one
    matrix of each shape (one GPT-2 layer, one square matrix, one MoE
    expert's up and down matrices)."""
    import workloads as W
    if name == "c1":
        wl = W.lora_toy(seed=0)
    elif name == "c2":
        wl = W.lora_batch()
    elif name == "c3":
        wl = W.gpt2_hidden(layers=1)
    elif name == "c4":
        wl = W.square_batch(count=1)
    else:
        wl = W.moe_experts(experts=1)
    wl.variant = variant
    return wl


def blas_info():
    """BLAS library numpy calls, its version and thread count."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"vendor": i.get("internal_api"), "version": i.get("version"),
                        "threads": int(i.get("num_threads", 1))}
    except Exception:  # pragma: no cover
        pass
    return {"vendor": "unknown", "version": None, "threads": None}


def cpu_baseline(wl_host, full_count, seconds, threads=None):
    """The oracle as it stands, on host cores, over a bounded sample of the
    batch: whole passes over the sample's matrices until `seconds` have
    elapsed (one pass when 0).  `threads` limits the BLAS threads (1 for the
    single-thread figure); the oracle's own code is single-threaded numpy."""
    import contextlib
    import oracle as O
    limit = contextlib.nullcontext()
    if threads is not None:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(threads)
    fn = O.dimuon_step if wl_host.variant == "dimuon" else O.muon_step
    mats = [(m.w.double().numpy(), m.g.double().numpy(), m.m_prev.double().numpy()) for m in wl_host.mats]
    with limit:
        blas = blas_info()
        done = 0
        t0 = time.perf_counter()
        while True:
            w, g, mp = mats[done % len(mats)]
            fn(w, g, mp, lr=wl_host.lr, mu=wl_host.mu, mom_dtype=wl_host.mom_dtype, w_dtype=wl_host.w_dtype)
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds and done % len(mats) == 0:
                break
    per_matrix = el / done
    steps_per_s = 1.0 / (per_matrix * full_count)
    return {"value": round(steps_per_s, 6 if steps_per_s > 1e-3 else 9), "unit": "steps/s",
            "cores": int(blas["threads"] or 1), "host_cpus": os.cpu_count(), "blas": blas, "kind": "oracle",
            "sample": f"{done} matrix steps over {len(mats)} distinct matrices of {wl_host.name} "
                      f"({wl_host.variant}) in {el:.1f} s (float64 numpy, BLAS threads {blas['threads']}); "
                      f"steps/s = 1 / (mean seconds per matrix x {full_count} matrices of the batch)"}


TOY_SEEDS = 32


def top4_share(o):
    """Share of the squared step in the four largest-scale columns (the last
    four of the toy's geometric column grid)."""
    col = (o ** 2).sum(0)
    return float(col[-4:].sum() / col.sum())


def toy_report(dev):
    """The 4 x 16 LoRA toy's report ("Dimuon: LoRA 에 맞춰 다시 짠 Muon",
    the toy with sixteen input columns of scale 0.1 .. 10): the share of the
    squared step in the four largest-scale columns and sigma_max / sigma_min
    of the step, for Muon and Dimuon, from the GPU path over seeded draws.
    The pages' figures (one unknown seed, a different orthogonaliser) are
    carried beside them as context."""
    import numpy as np
    import torch
    import dimuon_newton_schulz_amd as D
    import workloads as W

    wls = [W.lora_toy(seed=s, device=dev) for s in range(TOY_SEEDS)]
    wl0 = wls[0]
    cfg = D.StepConfig(lr=wl0.lr, momentum=wl0.mu, w_dtype=wl0.w_dtype, g_dtype=wl0.g_dtype,
                       mom_dtype=wl0.mom_dtype, ns_dtype=wl0.ns_dtype)
    out = {"workload": wl0.name, "seeds": TOY_SEEDS, "ns_dtype": wl0.ns_dtype}
    shares = {}
    for variant in ("muon", "dimuon"):
        params = [D.Param(w=wl.mats[0].w.clone(), g=wl.mats[0].g.clone(), mom=wl.mats[0].m_prev.clone(),
                          o_out=torch.empty(wl.mats[0].w.shape, dtype=torch.float32, device=dev)) for wl in wls]
        (D.dimuon_step if variant == "dimuon" else D.muon_step)(params, cfg)
        torch.cuda.synchronize()
        os_ = [p.o_out.double().cpu().numpy() for p in params]
        sh = [top4_share(o) for o in os_]
        sv = [np.linalg.svd(o, compute_uv=False) for o in os_]
        ratio = [float(v[0] / v[-1]) for v in sv]
        shares[variant] = sh
        out[variant] = {"top4_share_seed0": round(sh[0], 4), "top4_share_median": round(float(np.median(sh)), 4),
                        "sigma_ratio_seed0": round(ratio[0], 3), "sigma_ratio_median": round(float(np.median(ratio)), 3)}
    out["dimuon_below_muon_fraction"] = sum(d < m for d, m in zip(shares["dimuon"], shares["muon"])) / TOY_SEEDS
    g0 = wl0.mats[0].g.double().cpu().numpy()
    out["adam_first_step_top4_share"] = round(top4_share(np.sign(g0)), 4)
    out["pages_context"] = {"muon_polar_express_top4_share": 0.71, "dimuon_top4_share": 0.19,
                            "dimuon_sigma_ratio": 5.41, "adam_first_step_top4_share": 0.25}
    return out


_T0 = time.perf_counter()


def progress(msg):
    """One line per phase on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.perf_counter() - _T0:6.1f} s] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(matrices are independent and would shard by ownership across GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    import dimuon_newton_schulz_amd as D

    D.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    variant = args.variant or ("muon" if args.config == "c3" else "dimuon")
    progress(f"building {args.config} ({variant})")
    wl = make_workload(args.config, dev, variant)
    work = algorithmic(wl, is_thin)
    full_count = wl.count
    progress(f"timing {wl.name}: {args.warmup} warmup + {args.steps} steps")
    cfg, ms, per_kind, overhead, sets, per_set = measure(wl, args.steps, args.warmup, args.sets, ns_dtype=args.ns_dtype,
                                                         graph=args.graph, next_features=args.next)
    kind, roof = roofline_for(wl, cfg, per_kind, work, args.steps)
    total_flops = 5 * (work["gram_flops"] + work["poly_flops"] + work["comb_flops"])
    dtype = "f32" if (wl.w_dtype == "f32" and all(is_thin(*m.shape) for m in wl.mats)) else cfg.ns_dtype
    out = {
        "metric": "Muon/Dimuon steps/s per matrix batch",
        "value": round(1000.0 / ms, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "variant": wl.variant, "matrices": wl.count,
                   "ns_dtype": cfg.ns_dtype, "ns_steps": cfg.ns_steps, "buffer_sets": sets,
                   "launches": "hip graph" if args.graph else "stream", "parallelism": "single-gpu",
                   **({"extensions": {k: (f"{len(v)} rows" if k == "coeff_schedule" else v)
                                      for k, v in NEXT_SETTINGS.items()}} if args.next else {})},
        "matrices_per_s": round(wl.count * 1000.0 / ms, 1),
        "rotation_resident_bytes": sets * per_set,
        "step_gbs_algorithmic": round(work["hbm_bytes_min"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac_algorithmic": round(work["hbm_bytes_min"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roof,
        "kernel_ms_per_step": {k: round(v[0] / args.steps, 5) for k, v in sorted(per_kind.items())},
        "event_marker_overhead_ms": round(overhead, 5),
    }
    if total_flops:
        out["ns_tflops_algorithmic"] = round(total_flops / (ms * 1e-3) / 1e12, 2)
    # The other thin pass (two-pass step): its own fraction beside the dominant one's.
    for k in THIN_KERNELS:
        if k in per_kind and k != kind:
            tot, n = per_kind[k]
            b = work[k + "_bytes"]
            gbs = b / (tot / n * 1e-3) / 1e9
            out.setdefault("other_thin_kernels", {})[THIN_KERNELS[k]] = {
                "achieved": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": b,
                "avg_launch_ms": round(tot / n, 5)}
    del wl
    torch.cuda.empty_cache()

    extras = []
    if args.extra != "none":
        for item in args.extra.split(","):
            name, var, ns = (item.split(":") + ["", ""])[:3]
            progress(f"building and timing {item}")
            wl2 = make_workload(name, dev, var or None)
            w2 = algorithmic(wl2, is_thin)
            cfg2, ms2, pk2, _, sets2, _ = measure(wl2, args.extra_steps, 2, args.sets, ns_dtype=ns or args.ns_dtype,
                                                  graph=args.graph, next_features=args.next)
            k2, roof2 = roofline_for(wl2, cfg2, pk2, w2, args.extra_steps)
            tf = 5 * (w2["gram_flops"] + w2["poly_flops"] + w2["comb_flops"])
            rec = {"workload": wl2.name, "variant": wl2.variant, "ns_dtype": cfg2.ns_dtype, "matrices": wl2.count,
                   "steps": args.extra_steps, "buffer_sets": sets2, "ms_per_step": round(ms2, 4),
                   "steps_per_s": round(1000.0 / ms2, 3),
                   "matrices_per_s": round(wl2.count * 1000.0 / ms2, 1),
                   "ns_tflops_algorithmic": round(tf / (ms2 * 1e-3) / 1e12, 2) if tf else None,
                   "roofline": roof2,
                   "kernel_ms_per_step": {k: round(v[0] / args.extra_steps, 4) for k, v in sorted(pk2.items())}}
            extras.append((name, rec))
            del wl2
            torch.cuda.empty_cache()
    if not args.no_toy:
        progress("toy report")
        out["toy_report"] = toy_report(dev)

    if not args.no_cpu_baseline:
        progress("oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(host_sample(args.config, variant), full_count, args.cpu_seconds)
        # Single-thread figures for the two small configurations.
        single = {}
        for name in ("c1", "c2"):
            hs = host_sample(name, "dimuon")
            count = 128 if name == "c2" else 1
            single[name] = cpu_baseline(hs, count, min(args.cpu_seconds, 6.0), threads=1)
        out["cpu_baseline"]["single_thread"] = single
        # The larger sets: one pass over one matrix of each shape, scaled to the batch.
        counts = {"c3": 48, "c4": 8, "c5": 128}
        samples = {}
        for name, rec in extras:
            if name not in counts:
                continue
            key = (name, rec["variant"])
            if key not in samples:
                progress(f"oracle on one matrix of each shape of {name}")
                samples[key] = cpu_baseline(host_sample(name, rec["variant"]), counts[name], 0.0)
            rec["cpu_baseline"] = samples[key]
    out["workloads"] = [rec for _, rec in extras]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
