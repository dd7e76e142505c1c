#!/usr/bin/env python3
"""Benchmark of the structured-grid stencil sweeps on one MI355X.

    python bench.py [--steps K] [--warmup W] [--dtype f64|f32] [--quick]

One benchmark step = one full run of the 4096x4096 explicit five-point
diffusion workload: 1000 sweeps from a seeded interior uniform [0,1) field
with zero edges, alpha 0.1, in the production mapping (temporal blocking).
Inputs are resident in HBM before the timed region starts.  K steps are timed
with HIP events on the stream the kernels run on (torch's current stream) and
with the host clock around synchronisations.

Prints ONE JSON line with:
  value       interior cell updates per second (the cell-var rate; nvar = 1),
  roofline    the dominant kernel (the marching sweep) against MI355X peaks:
              algorithmic bytes per launch (one read of the grid, one write of
              its interior) over the kernel's average launch time, and its
              arithmetic (7 operations per interior cell per fused step) over
              the vector-ALU peak; `bound` names the tighter one;
  cpu_baseline  the CPU oracle (single thread) on a bounded sample of the
              same workload, timed on this host;
  kernels     per-kernel figures for the other workloads (pack along x/y/z,
              flux difference and its fused SSPRK stage, the 2D workload, the
              page's three loop layouts, the resident small-grid map,
              FP32, a 16-byte copy for reference), each as time, cell-var
              updates/s and GB/s of minimal traffic with the MALL flushed
              before every single-pass repetition.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "cell-var updates/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# Vector ALU peak for the stencil's adds and multiplies, from the published
# vector rates (an FMA counts as two operations there, one here):
#   FP64 78.6 TFLOP/s = 256 CUs x 64 lanes x 2 x 2.4 GHz -> 39.3 T operations/s,
#   FP32 157.3 TFLOP/s = 256 CUs x 128 lanes x 2 x 2.4 GHz -> 78.6 T operations/s
# (plain FP32 adds and multiplies issue faster than FP64 ones on gfx950).
ALU_PEAK_TOPS = {"f64": 256 * 64 * 2.4e9 / 1e12, "f32": 256 * 128 * 2.4e9 / 1e12}
FLOPS_PER_UPDATE = 7  # W+E, +S, +N, 4*C, -, alpha*t, C+
PROFILE_COUNTERS = ROOT / "profiles" / "diffusion_march_counters.json"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--dtype", choices=["f64", "f32"], default="f64")
    p.add_argument("--time-block", type=int, default=None)
    p.add_argument("--tile-rows", type=int, default=None)
    p.add_argument("--quick", action="store_true", help="headline only: skip the per-kernel table")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-steps", type=int, default=1000,
                   help="sweeps of the CPU-baseline sample (same grid; 1000 = one full step, ~11 s)")
    p.add_argument("--kernels", default="all",
                   help="comma-separated sections of the per-kernel table: copy, diffusion "
                        "(4096^2), small (64^2 and the size sweep), fields (eight fields per call), "
                        "large (16384^2), pack, flux, 2d (4800x1200 flux and packs), or all")
    p.add_argument("--ref-copy", action="store_true",
                   help="first run one 1 GiB copy (1 GiB read + 1 GiB written) as a known-size "
                        "reference for profiler byte counters")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def host_cpu_model() -> str:
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "host CPU"


def source_hash(path: Path) -> str:
    """Hash of a source's code: lines with their // comments removed, blank
    lines dropped, so that edits to comments alone keep recorded counters."""
    code = []
    for line in path.read_text().splitlines():
        i = line.find("//")
        line = (line[:i] if i >= 0 else line).rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the sweeps have no "
                          "multi-GPU path", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from structured_grid_cfd_amd import binding, inputs, launch_config

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    binding.load()
    dtype = np.float64 if args.dtype == "f64" else np.float32
    es = 8 if args.dtype == "f64" else 4
    cfg = launch_config.diffusion(args.dtype)
    if args.time_block is not None:
        cfg["time_block"] = args.time_block
        cfg["map"] = "temporal" if args.time_block > 1 else cfg["map"]
    if args.tile_rows is not None:
        cfg["tile_rows"] = args.tile_rows

    if args.ref_copy:
        n = 128 * 1024 * 1024
        src = torch.ones((1, 1, 1, n), dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        binding.field_pack(src, 0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- headline: 4096^2, 1000 sweeps per step -----------------
    c = inputs.uniform_4096(dtype)
    nx, ny, sweeps = c["nx"], c["ny"], c["steps"]
    u = torch.from_numpy(c["u"]).cuda()
    v = torch.from_numpy(c["v"]).cuda()
    stream = torch.cuda.current_stream()
    launches = binding.stencil_diffuse2d_launches(sweeps, cfg["map"], cfg["time_block"])

    def step():
        binding.stencil_diffuse2d(u, v, nx, c["alpha"], sweeps, cfg["map"], cfg["time_block"],
                                  cfg["tile_rows"], stream)

    log(f"headline {nx}x{ny} {args.dtype} {sweeps} sweeps/step, {cfg}, {launches} launches/step")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    updates = (nx - 2) * (ny - 2) * sweeps * args.steps
    value = updates / gpu_s
    ms_per_step = gpu_s / args.steps * 1e3
    log(f"headline: {ms_per_step:.3f} ms/step (host clock {wall / args.steps * 1e3:.3f}), "
        f"{value:.4e} cell-updates/s")

    # roofline of the marching kernel: every launch moves one read of the grid
    # and one write of its interior; its arithmetic is 7 ops per interior cell
    # per fused sweep.
    n_launch = launches * args.steps
    avg_launch_s = gpu_s / n_launch
    bytes_per_launch = (nx * ny + (nx - 2) * (ny - 2)) * es
    sweeps_per_launch = sweeps / launches
    hbm_gbs = bytes_per_launch / avg_launch_s / 1e9
    alu_tops = FLOPS_PER_UPDATE * (nx - 2) * (ny - 2) * sweeps_per_launch / avg_launch_s / 1e12
    alu_peak = ALU_PEAK_TOPS[args.dtype]
    hbm_frac, alu_frac = hbm_gbs / HBM_PEAK_GBS, alu_tops / alu_peak
    traffic = None
    if PROFILE_COUNTERS.exists():
        prof = json.loads(PROFILE_COUNTERS.read_text())
        src = ROOT / "structured_grid_cfd_amd" / "csrc" / "diffuse2d.hip"
        key = f"{args.dtype}_T{cfg['time_block']}"
        if prof.get("source_sha") == source_hash(src) and key in prof.get("per_launch_bytes", {}):
            traffic = prof["per_launch_bytes"][key]
    kernel_name = "k_march<%s, TS=%g>" % ("double" if es == 8 else "float", sweeps_per_launch)
    if hbm_frac >= alu_frac:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(hbm_frac, 4), "traffic": traffic}
    else:
        roofline = {"bound": "alu", "achieved": round(alu_tops, 2), "peak": round(alu_peak, 2),
                    "unit": "TFLOP/s", "frac": round(alu_frac, 4), "traffic": traffic}
    # The single-sweep bound: a kernel that reads the grid and writes it once
    # per sweep can do at most HBM peak / (bytes per cell per sweep) updates/s.
    single_sweep_bound = HBM_PEAK_GBS * 1e9 / (2 * es)
    roofline.update({"single_sweep_hbm_bound_cu_s": single_sweep_bound,
                     "value_over_single_sweep_bound": round(value / single_sweep_bound, 3)})
    roofline.update({"kernel": kernel_name, "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "launches_timed": n_launch, "bytes_per_launch": bytes_per_launch,
                     "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_frac, 4),
                     "alu_tflops": round(alu_tops, 2), "alu_frac": round(alu_frac, 4)})

    # ---------------- CPU oracle baseline (bounded sample) ------------------
    cpu = None
    if not args.no_cpu:
        import oracle
        uc, vc = c["u"].copy(), c["v"].copy()
        # pinned to one core of this process's set for the duration of the call
        allowed = os.sched_getaffinity(0)
        core = min(allowed)
        log(f"cpu baseline: oracle, {args.cpu_steps} sweeps of the same grid, one thread on core {core}")
        os.sched_setaffinity(0, {core})
        try:
            t = time.perf_counter()
            oracle.diffuse2d(uc, vc, nx, c["alpha"], args.cpu_steps)
            dt = time.perf_counter() - t
        finally:
            os.sched_setaffinity(0, allowed)
        cpu = {"value": (nx - 2) * (ny - 2) * args.cpu_steps / dt, "unit": "cell-var updates/s",
               "cores": 1, "kind": "oracle",
               "sample": f"{nx}x{ny} {args.dtype}, {args.cpu_steps} of the {sweeps} sweeps of one "
                         f"step, single-threaded C oracle pinned to one core ({dt:.1f} s on "
                         f"{host_cpu_model()}, {len(allowed)} of {os.cpu_count()} host cores "
                         f"available to the process)"}
        log(f"cpu baseline: {cpu['value']:.4e} cell-updates/s in {dt:.1f} s")

    kernels = None
    if not args.quick:
        del u, v
        torch.cuda.empty_cache()
        kernels = measure_all(log, set(args.kernels.split(",")))

    line = {
        "metric": METRIC, "value": value, "unit": "cell-var updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": f"2D five-point diffusion {nx}x{ny} {args.dtype.upper()}, "
                               f"{sweeps} sweeps per step, alpha 0.1, zero edges, interior "
                               f"uniform [0,1) seed 1002",
                   "map": cfg["map"], "time_block": cfg["time_block"],
                   "tile_rows": cfg["tile_rows"], "launches_per_step": launches,
                   "parallelism": "single GPU"},
        "achieved_hbm_gbs_minimal": round(hbm_gbs, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Per-kernel table (secondary figures; the JSON line's `kernels` object)
# ---------------------------------------------------------------------------

def measure_all(log, sections=frozenset({"all"})) -> dict:
    import torch

    from structured_grid_cfd_amd import binding, inputs, launch_config

    def want(name):
        return "all" in sections or name in sections

    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")  # 1 GiB

    def flush():
        # Reading 1 GiB evicts the 256 MB MALL and the L2s; a write would leave
        # dirty lines whose write-back then overlaps the timed kernel.
        flush_buf.sum()

    def timed(fn, reps, do_flush):
        out = []
        for _ in range(reps):
            if do_flush:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / 1e3)
        return out

    def entry(times, work, nbytes, extra=None):
        med = statistics.median(times)
        d = {"ms": round(med * 1e3, 4), "ms_min": round(min(times) * 1e3, 4),
             "cellvar_per_s": float("%.4e" % (work / med)),
             "gbs_minimal": round(nbytes / med / 1e9, 1),
             "hbm_frac": round(nbytes / med / 1e9 / HBM_PEAK_GBS, 4)}
        if extra:
            d.update(extra)
        return d

    res = {}
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731

    if want("copy"):
        # reference: a 16-byte-vector copy of 1 GiB (the x pack of one variable)
        n = 128 * 1024 * 1024
        src = torch.empty((1, 1, 1, n), dtype=torch.float64, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        binding.field_pack(src, 0, out=dst)
        t = timed(lambda: binding.field_pack(src, 0, out=dst), 5, True)
        res["copy_1GiB_dwordx4"] = entry(t, n, 2 * n * 8)
        log("copy", res["copy_1GiB_dwordx4"])
        del src, dst

    if want("diffusion"):
        # diffusion, 4096^2: production in both precisions, the page layouts, time blocks
        for dt_name, dt in (("f64", np.float64), ("f32", np.float32)):
            es = 8 if dt_name == "f64" else 4
            c = inputs.uniform_4096(dt)
            nx, ny = c["nx"], c["ny"]
            per_sweep = (nx * ny + (nx - 2) * (ny - 2)) * es
            u0, v0 = dev(c["u"]), dev(c["v"])
            u, v = u0.clone(), v0.clone()
            cells = (nx - 2) * (ny - 2)

            def run(m, tb, sweeps, rows=0):
                binding.stencil_diffuse2d(u, v, nx, 0.1, sweeps, m, tb, rows, stream)

            cfg = launch_config.diffusion(dt_name)
            run(cfg["map"], cfg["time_block"], 1000, cfg["tile_rows"])
            t = timed(lambda: run(cfg["map"], cfg["time_block"], 1000, cfg["tile_rows"]), 3, False)
            L = binding.stencil_diffuse2d_launches(1000, cfg["map"], cfg["time_block"])
            res[f"diffusion_4096_{dt_name}_1000sweeps_production"] = entry(
                t, cells * 1000, per_sweep * L,
                {"map": cfg["map"], "time_block": cfg["time_block"], "launches": L,
                 "note": "gbs_minimal counts one grid read + write per launch"})
            log(dt_name, "production", res[f"diffusion_4096_{dt_name}_1000sweeps_production"])
            for m in ("collapse_branch", "contig", "strided", "tiled"):
                sw = 100
                run(m, 1, 2)
                t = timed(lambda: run(m, 1, sw), 3, False)
                res[f"diffusion_4096_{dt_name}_{m}"] = entry(t, cells * sw, per_sweep * sw,
                                                             {"sweeps": sw})
                log(dt_name, m, res[f"diffusion_4096_{dt_name}_{m}"])
            for tb in (2, 3, 4, 6, 8, 10, 12):
                sw = 240
                run("temporal", tb, sw)
                t = timed(lambda: run("temporal", tb, sw), 3, False)
                L = binding.stencil_diffuse2d_launches(sw, "temporal", tb)
                res[f"diffusion_4096_{dt_name}_temporal_T{tb}"] = entry(
                    t, cells * sw, per_sweep * L, {"sweeps": sw, "launches": L})
                log(dt_name, "T", tb, res[f"diffusion_4096_{dt_name}_temporal_T{tb}"])
            del u, v, u0, v0
            torch.cuda.empty_cache()

    if want("small"):
        # 64x64 impulse, 32 sweeps: launch/latency bound.  Production is the
        # resident map (all sweeps in one workgroup); the depth-8 march beside it.
        c = inputs.impulse_64()
        u, v = dev(c["u"]), dev(c["v"])
        t = timed(lambda: binding.stencil_diffuse2d(u, v, 64, 0.1, 32, "temporal", 8, 0, stream), 10, False)
        res["diffusion_64_f64_32sweeps_march"] = entry(t, 62 * 62 * 32, (64 * 64 + 62 * 62) * 8 *
                                                       binding.stencil_diffuse2d_launches(32, "temporal", 8),
                                                       {"map": "temporal", "time_block": 8})
        cfg = launch_config.diffusion("f64", 64, 64)
        t = timed(lambda: binding.stencil_diffuse2d(u, v, 64, 0.1, 32, cfg["map"], cfg["time_block"], 0, stream),
                  10, False)
        res["diffusion_64_f64_32sweeps_resident"] = entry(t, 62 * 62 * 32, (64 * 64 + 62 * 62) * 8,
                                                          {"map": cfg["map"], "launches": 1})

        # size sweep, FP64 production map, 100 sweeps: where the small-grid
        # latency floor gives way to throughput
        for n in (128, 256, 512, 1024, 2048):
            cfg = launch_config.diffusion("f64", n, n)
            uu, vv = (dev(a) for a in inputs.uniform_grid(n, n, 1100 + n, np.float64))
            fn = lambda: binding.stencil_diffuse2d(uu, vv, n, 0.1, 100, cfg["map"], cfg["time_block"], 0, stream)  # noqa: E731
            fn()
            t = timed(fn, 5, False)
            res[f"diffusion_{n}_f64_100sweeps"] = entry(
                t, (n - 2) ** 2 * 100, (n * n + (n - 2) ** 2) * 8 *
                binding.stencil_diffuse2d_launches(100, cfg["map"], cfg["time_block"]),
                {"time_block": cfg["time_block"]})
            del uu, vv

    if want("fields"):
        # eight fields of one grid: one multi-field call (shared launches)
        # against eight single-field calls, 100 sweeps each, production depth
        for n in (256, 1024):
            cfg = launch_config.diffusion("f64", n, n)
            pairs = [inputs.uniform_grid(n, n, 2100 + k, np.float64) for k in range(8)]
            us = [dev(p0) for p0, _ in pairs]
            vs = [dev(p1) for _, p1 in pairs]
            L = binding.stencil_diffuse2d_launches(100, cfg["map"], cfg["time_block"])
            work = 8 * (n - 2) ** 2 * 100
            nbytes = 8 * (n * n + (n - 2) ** 2) * 8 * L

            def multi():
                binding.stencil_diffuse2d_fields(us, vs, n, 0.1, 100, cfg["map"], cfg["time_block"], 0,
                                                 stream)

            def separate():
                for k in range(8):
                    binding.stencil_diffuse2d(us[k], vs[k], n, 0.1, 100, cfg["map"], cfg["time_block"],
                                              0, stream)

            multi(); separate()
            res[f"diffusion_fields_8x{n}_f64_100sweeps"] = entry(
                timed(multi, 5, False), work, nbytes, {"time_block": cfg["time_block"], "launches": L})
            res[f"diffusion_8_calls_{n}_f64_100sweeps"] = entry(
                timed(separate, 5, False), work, nbytes, {"time_block": cfg["time_block"], "launches": 8 * L})
            log("fields", n, res[f"diffusion_fields_8x{n}_f64_100sweeps"], res[f"diffusion_8_calls_{n}_f64_100sweeps"])
            del us, vs
        # eight 64^2 fields, 32 sweeps, resident map: one workgroup per field
        c = inputs.impulse_64()
        us = [dev(c["u"]) for _ in range(8)]
        vs = [dev(c["v"]) for _ in range(8)]
        work = 8 * 62 * 62 * 32
        nbytes = 8 * (64 * 64 + 62 * 62) * 8

        def rmulti():
            binding.stencil_diffuse2d_fields(us, vs, 64, 0.1, 32, "resident", 1, 0, stream)

        def rseparate():
            for k in range(8):
                binding.stencil_diffuse2d(us[k], vs[k], 64, 0.1, 32, "resident", 1, 0, stream)

        rmulti(); rseparate()
        res["diffusion_fields_8x64_f64_32sweeps_resident"] = entry(timed(rmulti, 10, False), work, nbytes,
                                                                   {"map": "resident", "launches": 1})
        res["diffusion_8_calls_64_f64_32sweeps_resident"] = entry(timed(rseparate, 10, False), work, nbytes,
                                                                  {"map": "resident", "launches": 8})
        log("fields resident", res["diffusion_fields_8x64_f64_32sweeps_resident"],
            res["diffusion_8_calls_64_f64_32sweeps_resident"])
        del us, vs

    if want("large"):
        # 16384^2 FP32, 200 sweeps
        c = inputs.uniform_16384_f32()
        u, v = dev(c["u"]), dev(c["v"])
        del c
        cfg = launch_config.diffusion("f32")
        nx = ny = 16384
        binding.stencil_diffuse2d(u, v, nx, 0.1, 8, cfg["map"], cfg["time_block"], 0, stream)
        t = timed(lambda: binding.stencil_diffuse2d(u, v, nx, 0.1, 200, cfg["map"], cfg["time_block"],
                                                    cfg["tile_rows"], stream), 2, False)
        L = binding.stencil_diffuse2d_launches(200, cfg["map"], cfg["time_block"])
        res["diffusion_16384_f32_200sweeps_production"] = entry(
            t, (nx - 2) * (ny - 2) * 200, (nx * ny + (nx - 2) * (ny - 2)) * 4 * L,
            {"launches": L, "time_block": cfg["time_block"]})
        log("16384", res["diffusion_16384_f32_200sweeps_production"])
        t = timed(lambda: binding.stencil_diffuse2d(u, v, nx, 0.1, 10, "tiled", 1, 0, stream), 2, False)
        res["diffusion_16384_f32_tiled_single_sweep"] = entry(
            t, (nx - 2) * (ny - 2) * 10, (nx * ny + (nx - 2) * (ny - 2)) * 4 * 10, {"sweeps": 10})
        log("16384 tiled", res["diffusion_16384_f32_tiled_single_sweep"])
        del u, v
        torch.cuda.empty_cache()

    if want("pack"):
        # pack, 8 x 201^3
        f = dev(inputs.fields_201cubed())
        nvar, nz, ny_, nx_ = f.shape
        cv = nvar * nx_ * ny_ * nz
        out = torch.empty(cv, dtype=torch.float64, device="cuda")
        for d, dn in enumerate("xyz"):
            for m in ("tiled", "per_cell", "per_cellvar"):
                binding.field_pack(f, d, out=out, map=m)
                t = timed(lambda: binding.field_pack(f, d, out=out, map=m), 5, True)
                res[f"pack_201cubed_x8_{dn}_{m}"] = entry(t, cv, 16 * cv)
                log("pack", dn, m, res[f"pack_201cubed_x8_{dn}_{m}"])
        del f, out
        torch.cuda.empty_cache()

    if want("flux"):
        # flux difference, 7 x 201x101x101
        fi = inputs.faces_201x101x101()
        args = (dev(fi.fx), dev(fi.fy), dev(fi.fz), dev(fi.dx), dev(fi.dy), dev(fi.dz))
        nvar, nxc, nyc, nzc = fi.shape
        cv = nvar * nxc * nyc * nzc
        nbytes = 8 * (fi.fx.size + fi.fy.size + fi.fz.size + cv + nxc + nyc + nzc)
        rhs = torch.empty(cv, dtype=torch.float64, device="cuda").view(nvar, nzc, nyc, nxc)
        for m in ("tiled", "per_cell", "per_cellvar"):
            binding.flux_diff3d(*args, rhs=rhs, map=m)
            t = timed(lambda: binding.flux_diff3d(*args, rhs=rhs, map=m), 5, True)
            res[f"flux_201x101x101_x7_{m}"] = entry(t, cv, nbytes)
            log("flux", m, res[f"flux_201x101x101_x7_{m}"])
        # one SSPRK stage fused with it: reads q0 and q, writes q' instead of rhs
        q0 = dev(inputs.normal_fields(nvar, nxc, nyc, nzc, 1060))
        qs = dev(inputs.normal_fields(nvar, nxc, nyc, nzc, 1061))
        qo = torch.empty_like(qs)
        sbytes = nbytes + 2 * 8 * cv
        for m in ("tiled", "per_cell", "per_cellvar"):
            binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo, map=m)
            t = timed(lambda: binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo, map=m), 5, True)
            res[f"flux_stage_201x101x101_x7_{m}"] = entry(
                t, cv, sbytes, {"note": "a separate update pass would add one write and one read of rhs"})
            log("flux stage", m, res[f"flux_stage_201x101x101_x7_{m}"])
        del args, rhs, q0, qs, qo
        torch.cuda.empty_cache()

    if want("2d"):
        # 2D workload, 6 x 4800x1200: flux difference and packs along x, y
        fi = inputs.faces_4800x1200()
        args = (dev(fi.fx), dev(fi.fy), None, dev(fi.dx), dev(fi.dy), None)
        nvar, nxc, nyc, _ = fi.shape
        cv = nvar * nxc * nyc
        nbytes = 8 * (fi.fx.size + fi.fy.size + cv + nxc + nyc)
        rhs = torch.empty(cv, dtype=torch.float64, device="cuda").view(nvar, 1, nyc, nxc)
        for m in ("tiled", "per_cell", "per_cellvar"):
            binding.flux_diff3d(*args, rhs=rhs, map=m)
            t = timed(lambda: binding.flux_diff3d(*args, rhs=rhs, map=m), 5, True)
            res[f"flux2d_4800x1200_x6_{m}"] = entry(t, cv, nbytes)
            log("flux2d", m, res[f"flux2d_4800x1200_x6_{m}"])
        q0 = dev(inputs.normal_fields(nvar, nxc, nyc, 1, 1062))
        qs = dev(inputs.normal_fields(nvar, nxc, nyc, 1, 1063))
        qo = torch.empty_like(qs)
        sbytes = nbytes + 2 * 8 * cv
        binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo)
        t = timed(lambda: binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo), 5, True)
        res["flux_stage2d_4800x1200_x6_tiled"] = entry(t, cv, sbytes)
        log("flux2d stage", res["flux_stage2d_4800x1200_x6_tiled"])
        del args, rhs, q0, qs, qo
        f = dev(inputs.fields_4800x1200())
        out = torch.empty(cv, dtype=torch.float64, device="cuda")
        for d, dn in ((0, "x"), (1, "y")):
            for m in ("tiled", "per_cell", "per_cellvar"):
                binding.field_pack(f, d, out=out, map=m)
                t = timed(lambda: binding.field_pack(f, d, out=out, map=m), 5, True)
                res[f"pack2d_4800x1200_x6_{dn}_{m}"] = entry(t, cv, 16 * cv)
                log("pack2d", dn, m, res[f"pack2d_4800x1200_x6_{dn}_{m}"])
        del f, out
        torch.cuda.empty_cache()
    del flush_buf
    return res


if __name__ == "__main__":
    main()
