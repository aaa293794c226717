#!/usr/bin/env python3
"""Benchmark of the single-layer MoE training hot path on one MI355X.

One step = moe_dispatch_build + moe_ffn_forward + moe_ffn_backward on one
batch of synthetic inputs already resident in HBM.  Prints one JSON line:
routed tokens/s (L per step time), per-kernel times from HIP events recorded
by the library on the launch stream, the roofline of the dominant kernel,
the dispatch builder's HBM roofline, and the CPU oracle timed on a bounded
sample of the same workload.  The router-logit gradient (optional output of
the backward) is not part of the step; it is timed separately afterwards
(`router_grad`: its kernel and the extra time of the dG kernel that feeds it).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5]
       python bench.py --study memory|dispatch-e|skew   (extra measurements,
       one JSON line per point, instead of the step benchmark)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from token_dispatch_expert_amd import binding as B  # noqa: E402
from token_dispatch_expert_amd import workloads as W  # noqa: E402
from token_dispatch_expert_amd.layer import MoELayerBuffers  # noqa: E402

PEAK_TFLOPS = {W.BF16: 2500.0, W.F32: 157.3}   # dense MFMA peaks of MI355X
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_flops(cfg):
    """Algorithmic flops of ONE launch of each GEMM kernel."""
    L, d, h, K, R = cfg.L, cfg.d, cfg.h, cfg.K, cfg.R
    nproj = 2 if cfg.act == W.SWIGLU else 1
    return {
        "ffn_f1_gather_glu": 2 * R * d * h * nproj,
        "ffn_f2_down_combine": 2 * L * h * d,          # one slot pass: L routes
        "ffn_b1_dgrad_glu": 2 * R * d * h,
        "ffn_b0_dw2": 2 * R * h * d,
        "ffn_b2_dw13": 2 * R * d * h * nproj,
        "ffn_b3_dx": 2 * L * d * h * nproj,            # one slot pass
    }


def mask_words(E):
    """64-bit expert-mask words per token of the bit-form map: 1 for E <= 64,
    else the smallest power of two P >= 2 with 64 P >= E."""
    if E <= 64:
        return 1
    P = 2
    while 64 * P < E:
        P *= 2
    return P


def dispatch_bytes(cfg):
    """Algorithmic HBM bytes of one dispatch build, for the map representation
    the library uses at this shape.

    Always: logits read once (4LE), the four L*K int32/float32 outputs
    token_expert_indices, gates, expert_token_indices, token_index_map written
    once (16LK), and the offsets (4(E+1)).
    E <= 1024 and K <= 8 (bit-form map): each token's expert mask (W words of
    8 bytes) and each 64-token part's per-expert column (E/8 bytes per token)
    written once and read once; per-part counts (int32 per expert and part)
    written and read, 256-token tile bases written and read.
    Otherwise (byte map, K > 8): E bytes per token written once and read once."""
    L, E, K = cfg.L, cfg.E, cfg.K
    b = 4 * L * E + 16 * L * K + 4 * (E + 1)
    if E <= 1024 and K <= 8:
        tiles = -(-L // 256)
        parts = 4 * tiles
        b += (2 * 8 * mask_words(E) * L + 2 * 8 * E * parts + 2 * 4 * E * parts
              + 2 * 4 * E * tiles)
    else:
        b += 2 * L * E
    return b


def dispatch_bytes_byte_map(cfg):
    """Bytes of one dispatch build in the method's own layout with a one-byte
    token-expert map entry: logits read (4LE), the map written once and read
    twice (count, then scan and scatter: 3LE), the four L*K outputs (16LK) and
    the offsets.  Reported beside the implemented layout's figure, which
    moves fewer bytes for E <= 64 (bit masks)."""
    L, E, K = cfg.L, cfg.E, cfg.K
    return 4 * L * E + 3 * L * E + 16 * L * K + 4 * (E + 1)


def source_hash(timer):
    """Hash of the sources a timer's kernels are built from (their .hip file
    and the shared headers), so that counters stay valid for kernels that did
    not change."""
    src = "ffn.hip" if timer.startswith("ffn_") else "dispatch.hip"
    h = hashlib.sha256()
    for f in (src, "moe_device.h", "moe_internal.h"):
        with open(os.path.join(ROOT, "token_dispatch_expert_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


ROCPROF_NAMES = {   # library timer name -> kernel symbol base names in rocprofv3 output (first found)
    "ffn_f1_gather_glu": ("f1_gather_glu",),
    "ffn_f2_down_combine": ("f2_down_combine",),
    "ffn_b1_dgrad_glu": ("b1_dgrad_glu",),
    "ffn_b0_dw2": ("b0_dw2",),
    "ffn_b2_dw13": ("b2_dw13",),
    "ffn_b3_dx": ("b3_dx",),
    # E == 64 with aligned rows and L >= 64, else E <= 64 (k1_route_wide_mask beyond 64)
    "dispatch_route_map": ("k1_route_mask64", "k1_route_mask"),
    "dispatch_scatter": ("k3_scatter_mask",),
}


def _counter_means(csv_path, counter):
    import csv
    import re
    sums, counts = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")
            name = re.sub(r"<.*", "", name).split("::")[-1]
            sums[name] = sums.get(name, 0.0) + float(r["Counter_Value"])
            counts[name] = counts.get(name, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def record_traffic(dirs, workload):
    """Write profiles/traffic.json from four rocprofv3 --pmc runs (csv output
    directories): FETCH_SIZE and WRITE_SIZE of bench.py, and the same two
    counters of `bench.py --copy-calibration 1024` (a plain copy of known
    size, used to scale the counters to bytes)."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    csvf = lambda d: os.path.join(d, "run_counter_collection.csv")  # noqa: E731
    copy_bytes = 1024 << 20
    cf = max(_counter_means(csvf(cfetch_dir), "FETCH_SIZE").values())
    cw = max(_counter_means(csvf(cwrite_dir), "WRITE_SIZE").values())
    fscale, wscale = copy_bytes / cf, copy_bytes / cw
    fetch = _counter_means(csvf(fetch_dir), "FETCH_SIZE")
    write = _counter_means(csvf(write_dir), "WRITE_SIZE")
    p = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(p)) if os.path.exists(p) else {}
    ent = {}
    for timer, syms in ROCPROF_NAMES.items():
        sym = next((n for n in syms if n in fetch and n in write), None)
        if sym is not None:
            ent[timer] = {"source_hash": source_hash(timer),
                          "fetch_bytes_per_launch": fetch[sym] * fscale,
                          "write_bytes_per_launch": write[sym] * wscale,
                          "bytes_per_launch": fetch[sym] * fscale + write[sym] * wscale}
    rec[workload] = ent
    rec["_scale"] = {"fetch_size_bytes_per_unit": fscale, "write_size_bytes_per_unit": wscale,
                     "reference": "plain device copy of 1 GiB"}
    with open(p, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(ent, indent=1))


def measured_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(kernel)
    if not ent or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def router_grad_bytes(cfg):
    """Algorithmic HBM bytes of the router-logit gradient: the dG kernel's
    per-route partials written and read (4 R ceil(h/256)), token_index_map,
    token_expert_indices and gates read (12 L K), dlogits written (4 L E)."""
    nN = -(-cfg.h // 256)
    return 2 * 4 * cfg.R * nN + 12 * cfg.L * cfg.K + 4 * cfg.L * cfg.E


def time_router_grad(cfg, buf, inp, per_kernel, reps=2):
    """forward + backward with dlogits requested, `reps` times, timed per kernel."""
    buf.dlogits = torch.empty(cfg.L, cfg.E, dtype=torch.float32, device=buf.device)
    torch.cuda.synchronize()
    B.profile_reset()
    B.profile_enable(True)
    for _ in range(reps):
        buf.forward(inp["x"], inp["W1"], inp["W3"], inp["W2"])
        buf.backward(inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    B.profile_enable(False)
    st = B.profile_read()
    buf.dlogits = None
    kn, kms = st.get("router_grad", (0, 0.0))
    b1n, b1ms = st.get("ffn_b1_dgrad_glu", (0, 0.0))
    k_ms = kms / max(kn, 1)
    b1_with = b1ms / max(b1n, 1)
    b1_without = per_kernel.get("ffn_b1_dgrad_glu", {}).get("avg_launch_ms", 0.0)
    nbytes = router_grad_bytes(cfg)
    return {"kernel_ms": k_ms, "dgrad_kernel_ms_with": b1_with,
            "dgrad_kernel_ms_without": b1_without,
            "extra_ms_per_step": k_ms + b1_with - b1_without,
            "bytes": nbytes,
            "kernel_gbs": (nbytes - 4 * cfg.R * -(-cfg.h // 256)) / (k_ms / 1e3) / 1e9 if k_ms > 0 else None}


def _emit(d):
    print(json.dumps(d), flush=True)


def study_memory(cfg, seed, dev, steps=3):
    """Device memory and step time of one layer step, with G kept between
    the two GEMMs of each pass (default) and with G formed in [L, h] pieces
    (MOE_FLAG_RECOMPUTE_G): what the method keeps between forward and
    backward (A, B), the transient buffers, the measured peak (torch's
    allocator holds every buffer), and, for scale, the two (L*K, d) buffers
    a materialising layer keeps (routed copy of x, per-route expert output)."""
    es = 2 if cfg.dtype == W.BF16 else 4
    inp = W.make_inputs(cfg, seed, dev)
    torch.cuda.synchronize()
    for recompute in (False, True):
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        m_inputs = torch.cuda.memory_allocated(dev)
        buf = MoELayerBuffers(cfg, dev, recompute_g=recompute)
        torch.cuda.synchronize()
        m_buffers = torch.cuda.memory_allocated(dev)
        buf.step(inp)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev)
        B.profile_reset()
        B.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            buf.step(inp)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        B.profile_enable(False)
        st = B.profile_read()
        _emit({"study": "memory", "workload": cfg.name,
               "mode": "G formed in L-row pieces" if recompute else "G kept",
               "checkpoint_bytes": cfg.R * cfg.h * (2 if cfg.act == W.SWIGLU else 1) * es,
               "transient_G_bytes": (cfg.L if recompute else cfg.R) * cfg.h * es,
               "workspace_bytes": int(buf.ws.numel()),
               "inputs_bytes": int(m_inputs),
               "layer_buffers_bytes": int(m_buffers - m_inputs),
               "peak_allocated_bytes": int(peak),
               "ms_per_step": ms,
               "kernels_ms": {k: v[1] / steps for k, v in st.items()},
               "materialising_layer_extra_bytes": 2 * cfg.R * cfg.d * es})
        del buf


def time_builds(buf, logits, reps=50):
    """ms per dispatch build: `reps` builds back to back between two HIP
    events on the stream the builds run on (kernels and the gaps between
    them, without the per-launch event pairs of the kernel timers)."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    buf.build(logits)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        buf.build(logits)
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def study_dispatch_e(cfg, seed, dev, reps=20):
    """Dispatch build time and HBM rate over E at the workload's L and K."""
    for E in (8, 16, 32, 64, 128, 256, 512, 1024):
        if E < cfg.K:
            continue
        c = W.MoEConfig(f"{cfg.name}-E{E}", cfg.L, cfg.d, cfg.h, E, cfg.K, cfg.act, cfg.dtype)
        logits = W.make_logits(c, seed, dev)
        buf = MoELayerBuffers(W.small_config(c.L, 8, 8, E, c.K), dev)
        buf.build(logits)
        torch.cuda.synchronize()
        B.profile_reset()
        B.profile_enable(True)
        for _ in range(reps):
            buf.build(logits)
        torch.cuda.synchronize()
        B.profile_enable(False)
        st = B.profile_read()
        ms_ev = sum(v[1] for k, v in st.items() if k.startswith("dispatch_")) / reps
        ms = time_builds(buf, logits, reps)
        nb = dispatch_bytes(c)
        _emit({"study": "dispatch-e", "L": c.L, "E": E, "K": c.K, "ms_per_build": ms,
               "ms_per_build_kernel_events": ms_ev,
               "bytes_per_build": nb, "GB/s": nb / (ms / 1e3) / 1e9,
               "map": f"bit-form, {mask_words(E)} mask word(s) per token" if c.K <= 8 else "byte",
               "kernels_ms": {k: v[1] / reps for k, v in st.items()}})
        del buf, logits
        torch.cuda.empty_cache()


def study_skew(cfg, seed, dev, steps=3):
    """Layer step time over the skew of expert loads: logits N(0,1) plus
    2 log(w_e), w_e proportional to (e+1)^-s."""
    import math
    c = W.MoEConfig(f"{cfg.name}-L{cfg.L // 4}", cfg.L // 4, cfg.d, cfg.h, cfg.E, cfg.K,
                    cfg.act, cfg.dtype)
    inp = W.make_inputs(c, seed, dev)
    base = inp["logits"].clone()
    buf = MoELayerBuffers(c, dev)
    for s in (0.0, 0.6, 1.0, 1.2, 1.5):
        w = [(r + 1) ** (-s) for r in range(c.E)]
        tot = sum(w)
        bias = torch.tensor([2.0 * math.log(x / tot) for x in w], dtype=torch.float32, device=dev)
        inp["logits"] = base + bias
        buf.step(inp)
        torch.cuda.synchronize()
        load = torch.diff(buf.offsets.long()).cpu()
        B.profile_reset()
        B.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(steps):
            buf.step(inp)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        B.profile_enable(False)
        st = B.profile_read()
        _emit({"study": "skew", "workload": c.name, "zipf_s": s, "ms_per_step": ms,
               "routed_tokens_per_s": c.L / (ms / 1e3),
               "expert_load_max": int(load.max()), "expert_load_min": int(load.min()),
               "kernels_ms": {k: v[1] / steps for k, v in st.items()}})


def cpu_baseline(cfg, inp, budget_s=15.0):
    """The oracle, untuned, on a bounded prefix sample of the same workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 0) for i in info] or [0])
    except Exception:  # noqa: BLE001
        threads = 0
    if threads <= 0:
        threads = int(os.environ.get("OPENBLAS_NUM_THREADS")
                      or os.environ.get("OMP_NUM_THREADS") or os.cpu_count())

    W1 = inp["W1"].float().cpu().numpy()
    W3 = inp["W3"].float().cpu().numpy() if inp["W3"] is not None else None
    W2 = inp["W2"].float().cpu().numpy()

    def run(n):
        z = inp["logits"][:n].cpu().numpy()
        x = inp["x"][:n].float().cpu().numpy()
        dy = inp["dy"][:n].float().cpu().numpy()
        t0 = time.perf_counter()
        tei, gates = oracle.route(z, cfg.K)
        eti, off, tim = oracle.build_indices(tei, cfg.E)
        oracle.ffn_forward(x, W1, W3, W2, eti, off, tim, gates, cfg.act)
        oracle.ffn_backward(dy, x, W1, W3, W2, eti, off, tim, gates, cfg.act)
        return time.perf_counter() - t0

    n = min(256, cfg.L)
    t = run(n)
    while t < budget_s / 2 and n < cfg.L:     # grow the sample to ~budget_s
        n = min(cfg.L, max(n * 2, int(n * budget_s / max(t, 1e-3))))
        t = run(n)
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} tokens of the workload (same d, h, E, K, weights), "
                      f"dispatch + forward + backward in float64 numpy, {t:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--recompute-g", action="store_true",
                    help="MOE_FLAG_RECOMPUTE_G: G formed from A, B in [L, h] pieces, no [L*K, h] buffer")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scale reference "
                         "for rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--study", choices=("memory", "dispatch-e", "skew"),
                    help="memory: analytic and measured device memory of one step; dispatch-e: "
                         "dispatch build time over E at fixed L and K; skew: layer step time "
                         "over the Zipf skew of the router logits")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write profiles/traffic.json from rocprofv3 --pmc csv output directories "
                         "and exit (no GPU needed)")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.record_traffic, W.CONFIGS[args.config].name)
        return

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X here "
              "and has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    cfg = W.CONFIGS[args.config]
    seed = args.config if args.seed is None else args.seed
    dev = torch.device("cuda:0")
    if args.study:
        {"memory": study_memory, "dispatch-e": study_dispatch_e, "skew": study_skew}[args.study](
            cfg, seed, dev)
        return
    log(f"[bench] {cfg.name}: generating inputs on {torch.cuda.get_device_name(0)}")
    inp = W.make_inputs(cfg, seed, dev)
    buf = MoELayerBuffers(cfg, dev, recompute_g=args.recompute_g)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        buf.step(inp)
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    B.profile_reset()
    B.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        buf.step(inp)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    B.profile_enable(False)
    stats = B.profile_read()
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")

    ms_step = elapsed * 1e3 / args.steps
    kflops = kernel_flops(cfg)
    per_kernel = {k: {"launches_per_step": n / args.steps, "ms_per_step": ms / args.steps,
                      "avg_launch_ms": ms / max(n, 1)} for k, (n, ms) in stats.items()}
    gemm = {k: v for k, v in per_kernel.items() if k in kflops}
    dom = max(gemm, key=lambda k: gemm[k]["ms_per_step"])
    avg_s = gemm[dom]["avg_launch_ms"] / 1e3
    achieved = kflops[dom] / avg_s / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    for k, v in per_kernel.items():
        if k in kflops:
            v["tflops"] = kflops[k] / (v["avg_launch_ms"] / 1e3) / 1e12
    gemm_ms = sum(v["ms_per_step"] for v in gemm.values())
    total_flops = sum(kflops[k] * gemm[k]["launches_per_step"] for k in gemm)

    disp_keys = ("dispatch_route_map", "dispatch_expert_scan", "dispatch_scatter")
    disp_ms_ev = sum(per_kernel[k]["ms_per_step"] for k in disp_keys if k in per_kernel)
    disp_ms = time_builds(buf, inp["logits"])
    disp_gbs = dispatch_bytes(cfg) / (disp_ms / 1e3) / 1e9 if disp_ms > 0 else None

    traffic = measured_traffic(dom, cfg.name)
    out = {
        "metric": "routed tokens/sec (MoE layer fwd+bwd, 1 GPU)",
        "value": cfg.L / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == W.BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "L": cfg.L, "d": cfg.d, "h": cfg.h, "E": cfg.E,
                   "K": cfg.K, "act": "swiglu" if cfg.act == W.SWIGLU else "silu",
                   "seed": seed, "parallelism": "none (1 GPU)",
                   "g_buffer": "[L, h] pieces" if args.recompute_g else "kept"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                     "flops_per_launch": kflops[dom],
                     "avg_launch_ms": gemm[dom]["avg_launch_ms"]},
        "roofline_dispatch": {"bound": "hbm", "achieved": disp_gbs, "peak": PEAK_HBM_GBS,
                              "unit": "GB/s",
                              "frac": (disp_gbs / PEAK_HBM_GBS) if disp_gbs else None,
                              "bytes_per_build": dispatch_bytes(cfg), "ms_per_build": disp_ms,
                              "timing": "50 builds back to back between two HIP events",
                              "ms_per_build_kernel_events": disp_ms_ev},
        "roofline_by_kernel": {
            k: {"bound": "mfma", "achieved": v["tflops"], "peak": peak, "unit": "TFLOP/s",
                "frac": v["tflops"] / peak, "traffic": measured_traffic(k, cfg.name),
                "flops_per_launch": kflops[k], "avg_launch_ms": v["avg_launch_ms"]}
            for k, v in gemm.items()},
        "assignments_per_s": cfg.R / (ms_step / 1e3),
        "gemm_tflops_all": total_flops / (gemm_ms / 1e3) / 1e12,
        "kernels": per_kernel,
    }
    out["router_grad"] = time_router_grad(cfg, buf, inp, per_kernel)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
