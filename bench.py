#!/usr/bin/env python3
"""Benchmark of the structured-grid stencil sweeps on one MI355X.

    python bench.py [--steps K] [--warmup W] [--quick] [--no-cpu]

One benchmark step = one pass over the large 2D workload, every part in its
production mapping:
  * the conservative flux difference of 6 FP64 fields on a 4800x1200 grid
    (x and y faces normal(0,1), widths U[0.5,1.5)/n, seed 1005), and
  * the x and y packs of 6 FP64 fields of 4800x1200 (normal(0,1), seed 1050),
  * 200 sweeps of the explicit five-point diffusion on a 16384x16384 FP32
    grid (interior uniform [0,1), zero edges, alpha 0.1, seed 1006).
Inputs are resident in HBM before the timed region starts.  K steps are timed
with HIP events on the stream the library launches on (torch's current
stream), and with the host clock around synchronisations.

Prints ONE JSON line with:
  value       cell-var updates per second over the timed steps: diffusion
              counts interior cells x sweeps, the flux difference and each
              pack count fields x cells;
  roofline    the dominant kernel (the FP32 marching sweep, depth 10), its
              average launch duration from HIP events around the sweeps of
              every timed step: algorithmic bytes per launch (one read of the
              grid, one write of its interior) against HBM peak, and its
              arithmetic (7 operations of the definition per interior cell per
              fused sweep) against the vector-ALU peak; `bound` is the ALU for
              fused depths of five and more, HBM below;
  cpu_baseline  the CPU oracle (one thread, pinned) on a bounded sample of
              the same workload, timed on this host;
  kernels     per-kernel figures for every workload (the 64x64 impulse, the
              4096^2 diffusion in both precisions and all mappings, the 201^3
              packs, the 201x101x101 flux difference, the large workload's
              parts, the resident and multi-field maps, a 16-byte copy for
              reference), each with the oracle's time on one pinned host core
              beside the GPU's.
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
# Vector-ALU peaks in operations per second, one operation being one lane of
# one VALU instruction (an FMA is one operation, two flops).  A SIMD issues a
# 64-lane VALU instruction per 4 cycles, and gfx950 can issue two FP32 VALU
# instructions in one 4-cycle slot (the profiler counts such slots as
# SQ_ACTIVE_INST_VALU2): 256 CUs x 4 SIMDs x 16 lanes x 2 x 2.4 GHz =
# 78.6 T operations/s for FP32, the published 157.3 TFLOP/s counted with FMAs
# as two flops; FP64 issues one per slot, 39.3 T operations/s (78.6 TFLOP/s).
# The five-point update is 7 operations of its definition per interior cell
# and sweep (W+E, +S, +N, 4*C, -, alpha*t, C+).
ALU_PEAK_TOPS = {"f64": 256 * 4 * 16 * 2.4e9 / 1e12, "f32": 256 * 4 * 16 * 2 * 2.4e9 / 1e12}
OPS_PER_UPDATE = 7
PROFILE_COUNTERS = ROOT / "profiles" / "diffusion_march_counters.json"

# The pages' own figures for related work on other hardware: context for the
# report, not targets (other kernels, other machines, whole solvers).
CONTEXT = {
    "mfc_h200_grind_time_ns_per_gp_eq_rhs": {
        "value": [0.416, 0.379], "hardware": "NVIDIA H200, 1 GPU, FP64",
        "what": "MFC whole-solver grind time before and after collapsing only the spatial loops of "
                "the per-variable kernels (3D_performance_test, 201^3); the changed kernels ran "
                "40-49% shorter",
        "source": "MFC pull request 2087, Performance"},
    "mallard_a100_teno_smooth": {
        "value_tbs": 0.8, "peak_tbs": 1.94, "frac": 0.42,
        "hardware": "NVIDIA A100-SXM4-80GB, FP64",
        "what": "Mallard's TENO5 smoothness pass on a 1024^2 grid, achieved bandwidth",
        "source": "Mallard documentation, Design: single-GPU performance and parallel scaling, "
                  "Baseline (main)"},
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--time-block", type=int, default=None,
                   help="depth of the diffusion part (default: the production setting)")
    p.add_argument("--tile-rows", type=int, default=None)
    p.add_argument("--quick", action="store_true", help="headline only: skip the per-kernel table")
    p.add_argument("--no-cpu", action="store_true", help="skip every CPU oracle timing")
    p.add_argument("--cpu-sweeps", type=int, default=40,
                   help="sweeps of the 16384^2 grid in the CPU-baseline sample (of the step's 200)")
    p.add_argument("--kernels", default="all",
                   help="comma-separated sections of the per-kernel table: copy, diffusion "
                        "(4096^2; prod4096 for its production runs only), small (64^2 and the size "
                        "sweep), fields (eight fields per call), "
                        "large (16384^2 single sweeps), pack, flux, 2d (4800x1200 flux and packs), "
                        "or all")
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


def on_one_core(fn, reps=1):
    """Run ``fn`` ``reps`` times with the calling thread pinned to one core of
    the process's set; returns (median seconds, all seconds, core, cores
    available).  Only the call itself is inside the clock."""
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        ts = []
        for _ in range(reps):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
    finally:
        os.sched_setaffinity(0, allowed)
    return statistics.median(ts), ts, core, len(allowed)


def cpu_entry(fn, work, reps, sample):
    """The oracle's time on one pinned host core for ``work`` cell-var updates."""
    med, ts, _, avail = on_one_core(fn, reps)
    return {"s": round(med, 4), "reps": reps, "cellvar_per_s": float("%.4e" % (work / med)),
            "cores": 1, "sample": sample,
            "host": f"{host_cpu_model()}, {avail} of {os.cpu_count()} host cores available"}


def counted_traffic(key: str):
    """HBM bytes per launch of the marching kernel from the recorded profiler
    counters, or None once diffuse2d.hip's code has changed since."""
    if not PROFILE_COUNTERS.exists():
        return None
    prof = json.loads(PROFILE_COUNTERS.read_text())
    src = ROOT / "structured_grid_cfd_amd" / "csrc" / "diffuse2d.hip"
    if prof.get("source_sha") != source_hash(src):
        return None
    return prof.get("per_launch_bytes", {}).get(key)


# ---------------------------------------------------------------------------
# The large 2D workload: the benchmark step
# ---------------------------------------------------------------------------

class LargeWorkload:
    """Device-resident inputs and outputs of one benchmark step."""

    def __init__(self, cfg):
        import torch

        from structured_grid_cfd_amd import inputs

        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        self.fi = inputs.faces_4800x1200()
        self.fields = inputs.fields_4800x1200()
        self.nvar, self.pnx, self.pny, _ = self.fi.shape
        self.flux_args = (dev(self.fi.fx), dev(self.fi.fy), None, dev(self.fi.dx), dev(self.fi.dy), None)
        cv = self.nvar * self.pnx * self.pny
        self.cellvars = cv
        self.rhs = torch.empty(cv, dtype=torch.float64, device="cuda").view(self.nvar, 1, self.pny, self.pnx)
        self.fd = dev(self.fields)
        self.pack_x = torch.empty(cv, dtype=torch.float64, device="cuda")
        self.pack_y = torch.empty(cv, dtype=torch.float64, device="cuda")
        self.grid = inputs.uniform_16384_f32()
        self.nx, self.ny, self.sweeps = self.grid["nx"], self.grid["ny"], self.grid["steps"]
        self.alpha = self.grid["alpha"]
        self.u = dev(self.grid["u"])
        self.v = dev(self.grid["v"])
        self.cfg = cfg
        self.flux_bytes = 8 * (self.fi.fx.size + self.fi.fy.size + cv + self.pnx + self.pny)
        self.pack_bytes = 16 * cv
        self.cells = (self.nx - 2) * (self.ny - 2)
        self.launch_bytes = (self.nx * self.ny + self.cells) * 4

    @property
    def units(self):
        """Cell-var updates of one step."""
        return 3 * self.cellvars + self.cells * self.sweeps

    def step(self, stream, ev=None):
        from structured_grid_cfd_amd import binding
        binding.flux_diff3d(*self.flux_args, rhs=self.rhs, map="tiled", stream=stream)
        binding.field_pack(self.fd, 0, out=self.pack_x, map="tiled", stream=stream)
        binding.field_pack(self.fd, 1, out=self.pack_y, map="tiled", stream=stream)
        if ev is not None:
            ev[0].record(stream)
        binding.stencil_diffuse2d(self.u, self.v, self.nx, self.alpha, self.sweeps, self.cfg["map"],
                                  self.cfg["time_block"], self.cfg["tile_rows"], stream)
        if ev is not None:
            ev[1].record(stream)


def cpu_baseline_large(cpu_sweeps: int):
    """The oracle on a bounded sample of the benchmark step: the flux
    difference and both packs of the 4800x1200 workload in full, and
    ``cpu_sweeps`` of the 200 sweeps of the 16384^2 grid."""
    import oracle
    from structured_grid_cfd_amd import inputs

    fi = inputs.faces_4800x1200()
    fields = inputs.fields_4800x1200()
    g = inputs.uniform_16384_f32()
    nvar, pnx, pny, _ = fi.shape
    u, v = g["u"].copy(), g["v"].copy()

    def run():
        oracle.flux_diff(fi.fx, fi.fy, None, fi.dx, fi.dy, None)
        oracle.field_pack(fields, 0)
        oracle.field_pack(fields, 1)
        oracle.diffuse2d(u, v, g["nx"], g["alpha"], cpu_sweeps)

    med, _, core, avail = on_one_core(run, 1)
    work = 3 * nvar * pnx * pny + (g["nx"] - 2) * (g["ny"] - 2) * cpu_sweeps
    return {"value": work / med, "unit": "cell-var updates/s", "cores": 1, "kind": "oracle",
            "sample": f"flux difference and x/y packs of 6 x 4800x1200 FP64 in full, plus "
                      f"{cpu_sweeps} of the 200 sweeps of the 16384^2 FP32 grid; single-threaded "
                      f"C oracle pinned to core {core} ({med:.1f} s on {host_cpu_model()}, "
                      f"{avail} of {os.cpu_count()} host cores available to the process)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the sweeps have no "
                          "multi-GPU path", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from structured_grid_cfd_amd import binding, launch_config

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    binding.load()
    cfg = launch_config.diffusion("f32", 16384, 16384)
    if args.time_block is not None:
        cfg["time_block"] = args.time_block
        cfg["map"] = "temporal" if args.time_block > 1 else "tiled"
    if args.tile_rows is not None:
        cfg["tile_rows"] = args.tile_rows

    if args.ref_copy:
        n = 128 * 1024 * 1024
        src = torch.ones((1, 1, 1, n), dtype=torch.float64, device="cuda")
        dst = torch.empty_like(src)
        binding.field_pack(src, 0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- headline: the large 2D workload ------------------------
    w = LargeWorkload(cfg)
    units = w.units
    stream = torch.cuda.current_stream()
    launches = binding.stencil_diffuse2d_launches(w.sweeps, cfg["map"], cfg["time_block"])
    log(f"headline: 6 x 4800x1200 flux + x/y packs, {w.nx}x{w.ny} f32 {w.sweeps} sweeps, {cfg}, "
        f"{launches} diffusion launches per step")
    for _ in range(args.warmup):
        w.step(stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    e0.record(stream)
    for k in range(args.steps):
        w.step(stream, dev_ev[k])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = e0.elapsed_time(e1) / 1e3
    diff_s = sum(a.elapsed_time(b) for a, b in dev_ev) / 1e3
    value = w.units * args.steps / gpu_s
    ms_per_step = gpu_s / args.steps * 1e3
    step_bytes = w.flux_bytes + 2 * w.pack_bytes + w.launch_bytes * launches
    log(f"headline: {ms_per_step:.3f} ms/step (host clock {wall / args.steps * 1e3:.3f}; diffusion "
        f"{diff_s / args.steps * 1e3:.3f}), {value:.4e} cell-var updates/s")

    # roofline of the marching kernel: its launches' time from the events
    # around the sweeps of every timed step
    n_launch = launches * args.steps
    avg_launch_s = diff_s / n_launch
    sweeps_per_launch = w.sweeps / launches
    hbm_gbs = w.launch_bytes / avg_launch_s / 1e9
    alu_tops = OPS_PER_UPDATE * w.cells * sweeps_per_launch / avg_launch_s / 1e12
    alu_peak = ALU_PEAK_TOPS["f32"]
    hbm_frac, alu_frac = hbm_gbs / HBM_PEAK_GBS, alu_tops / alu_peak
    traffic = counted_traffic(f"f32_16384_T{cfg['time_block']}") if cfg["map"] == "temporal" else None
    kernel_name = "k_march<float, %d, ...>" % (cfg["time_block"] if cfg["map"] == "temporal" else 1)
    # Fused depths of five and more are bound by vector-ALU issue (the VALU
    # counters of the marching kernel show the SIMDs issuing in about 90% of
    # their cycles); one and two sweeps per launch by HBM.
    fused = cfg["map"] == "temporal" and cfg["time_block"] >= 5
    if not fused:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(hbm_frac, 4), "traffic": traffic}
    else:
        roofline = {"bound": "alu", "achieved": round(alu_tops, 2), "peak": round(alu_peak, 2),
                    "unit": "T operations/s (7 per update)", "frac": round(alu_frac, 4),
                    "traffic": traffic}
    # A kernel that reads the grid and writes it once per sweep can do at most
    # HBM peak / (8 bytes per FP32 cell per sweep) updates/s.
    single_sweep_bound = HBM_PEAK_GBS * 1e9 / 8
    diff_rate = w.cells * w.sweeps * args.steps / diff_s
    roofline.update({"kernel": kernel_name, "avg_launch_us": round(avg_launch_s * 1e6, 3),
                     "launches_timed": n_launch, "bytes_per_launch": w.launch_bytes,
                     "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_frac, 4),
                     "alu_tops": round(alu_tops, 2), "alu_frac": round(alu_frac, 4),
                     "diffusion_cell_updates_per_s": float("%.4e" % diff_rate),
                     "single_sweep_hbm_bound_cu_s": single_sweep_bound,
                     "diffusion_over_single_sweep_bound": round(diff_rate / single_sweep_bound, 3),
                     "share_of_step": round(diff_s / gpu_s, 4)})

    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle on the large workload's sample ({args.cpu_sweeps} sweeps)")
        cpu = cpu_baseline_large(args.cpu_sweeps)
        log(f"cpu baseline: {cpu['value']:.4e} cell-var updates/s")

    kernels = None
    if not args.quick:
        del w
        torch.cuda.empty_cache()
        kernels = measure_all(log, set(args.kernels.split(",")), cpu=not args.no_cpu)

    line = {
        "metric": METRIC, "value": value, "unit": "cell-var updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": "large 2D sweep: conservative flux difference and x/y packs of 6 "
                               "FP64 fields on 4800x1200 (seeds 1005, 1050), plus 200 sweeps of "
                               "FP32 five-point diffusion on 16384x16384 (alpha 0.1, zero edges, "
                               "interior uniform [0,1), seed 1006)",
                   "units_per_step": units,
                   "diffusion": {"map": cfg["map"], "time_block": cfg["time_block"],
                                 "tile_rows": cfg["tile_rows"], "launches_per_step": launches,
                                 "dtype": "f32"},
                   "flux_and_packs": {"map": "tiled", "dtype": "f64"},
                   "parallelism": "single GPU"},
        "achieved_hbm_gbs_minimal": round(step_bytes / (gpu_s / args.steps) / 1e9, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "context": CONTEXT,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Per-kernel table (secondary figures; the JSON line's `kernels` object)
# ---------------------------------------------------------------------------

def measure_all(log, sections=frozenset({"all"}), cpu=True) -> dict:
    import torch

    import oracle
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

    def timed_group(fns, reps, do_flush):
        """Time several variants of one workload, rotating their order on
        every repetition so that no variant always runs first or last."""
        names = list(fns)
        out = {k: [] for k in names}
        for r in range(reps):
            for i in range(len(names)):
                k = names[(i + r) % len(names)]
                out[k].extend(timed(fns[k], 1, do_flush))
        return out

    copy_gbs = []  # the reference copy's bandwidth, once measured

    def entry(times, work, nbytes, extra=None, ops=None):
        """Median time, rate, minimal-byte bandwidth (also as a fraction of
        the measured reference copy's); with `ops` = (operations per unit of
        work, dtype) also the fraction of the vector-ALU peak."""
        med = statistics.median(times)
        d = {"ms": round(med * 1e3, 4), "ms_min": round(min(times) * 1e3, 4),
             "ms_max": round(max(times) * 1e3, 4),
             "reps": len(times), "cellvar_per_s": float("%.4e" % (work / med)),
             "gbs_minimal": round(nbytes / med / 1e9, 1),
             "hbm_frac": round(nbytes / med / 1e9 / HBM_PEAK_GBS, 4)}
        if copy_gbs:
            d["of_copy"] = round(nbytes / med / 1e9 / copy_gbs[0], 4)
        if ops:
            d["alu_frac"] = round(ops[0] * work / med / 1e12 / ALU_PEAK_TOPS[ops[1]], 4)
        if extra:
            d.update(extra)
        return d

    res = {}
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731

    if want("copy"):
        # reference: a 16-byte-vector copy of 2 GiB (the x pack of one
        # variable); every later entry also reports its bandwidth against it
        n = 256 * 1024 * 1024
        src = torch.empty((1, 1, 1, n), dtype=torch.float64, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        binding.field_pack(src, 0, out=dst)
        t = timed(lambda: binding.field_pack(src, 0, out=dst), 10, True)
        res["copy_2GiB_dwordx4"] = entry(t, n, 2 * n * 8)
        copy_gbs.append(res["copy_2GiB_dwordx4"]["gbs_minimal"])
        log("copy", res["copy_2GiB_dwordx4"])
        del src, dst
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
        extra = {"map": cfg["map"], "launches": 1}
        if cpu:
            extra["oracle"] = cpu_entry(lambda: oracle.diffuse2d_result(c["u"], 64, 0.1, 32), 62 * 62 * 32, 3,
                                        "the whole workload")
        res["diffusion_64_f64_32sweeps_resident"] = entry(t, 62 * 62 * 32, (64 * 64 + 62 * 62) * 8, extra)
        log("64^2", res["diffusion_64_f64_32sweeps_resident"])

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

    if want("diffusion") or want("prod4096"):
        # diffusion, 4096^2: production in both precisions, the page layouts, time
        # blocks (section prod4096: the production runs only)
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

            cfg = launch_config.diffusion(dt_name, nx, ny)
            run(cfg["map"], cfg["time_block"], 1000, cfg["tile_rows"])
            t = timed(lambda: run(cfg["map"], cfg["time_block"], 1000, cfg["tile_rows"]), 5, False)
            L = binding.stencil_diffuse2d_launches(1000, cfg["map"], cfg["time_block"])
            extra = {"map": cfg["map"], "time_block": cfg["time_block"], "launches": L,
                     "note": "gbs_minimal counts one grid read + write per launch"}
            if cpu:
                uc = c["u"].copy()
                vc = c["v"].copy()
                extra["oracle"] = cpu_entry(lambda: oracle.diffuse2d(uc, vc, nx, 0.1, 100), cells * 100, 3,
                                            "100 of the 1000 sweeps of the same grid")
            res[f"diffusion_4096_{dt_name}_1000sweeps_production"] = entry(t, cells * 1000, per_sweep * L, extra,
                                                                           ops=(OPS_PER_UPDATE, dt_name))
            log(dt_name, "production", res[f"diffusion_4096_{dt_name}_1000sweeps_production"])
            if not want("diffusion"):
                del u, v, u0, v0
                torch.cuda.empty_cache()
                continue
            maps = ("collapse_branch", "contig", "strided", "tiled")
            sw = 100
            for m in maps:
                run(m, 1, 2)
            tg = timed_group({m: (lambda m=m: run(m, 1, sw)) for m in maps}, 3, False)
            for m in maps:
                res[f"diffusion_4096_{dt_name}_{m}"] = entry(tg[m], cells * sw, per_sweep * sw,
                                                             {"sweeps": sw})
                log(dt_name, m, res[f"diffusion_4096_{dt_name}_{m}"])
            depths = (2, 3, 4, 6, 8, 10, 12)
            sw = 240
            for tb in depths:
                run("temporal", tb, sw)
            tg = timed_group({tb: (lambda tb=tb: run("temporal", tb, sw)) for tb in depths}, 3, False)
            for tb in depths:
                L = binding.stencil_diffuse2d_launches(sw, "temporal", tb)
                res[f"diffusion_4096_{dt_name}_temporal_T{tb}"] = entry(
                    tg[tb], cells * sw, per_sweep * L, {"sweeps": sw, "launches": L}, ops=(OPS_PER_UPDATE, dt_name))
                log(dt_name, "T", tb, res[f"diffusion_4096_{dt_name}_temporal_T{tb}"])
            del u, v, u0, v0
            torch.cuda.empty_cache()

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
            tg = timed_group({"multi": multi, "separate": separate}, 5, False)
            res[f"diffusion_fields_8x{n}_f64_100sweeps"] = entry(
                tg["multi"], work, nbytes, {"time_block": cfg["time_block"], "launches": L})
            res[f"diffusion_8_calls_{n}_f64_100sweeps"] = entry(
                tg["separate"], work, nbytes, {"time_block": cfg["time_block"], "launches": 8 * L})
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
        tg = timed_group({"multi": rmulti, "separate": rseparate}, 10, False)
        res["diffusion_fields_8x64_f64_32sweeps_resident"] = entry(tg["multi"], work, nbytes,
                                                                   {"map": "resident", "launches": 1})
        res["diffusion_8_calls_64_f64_32sweeps_resident"] = entry(tg["separate"], work, nbytes,
                                                                  {"map": "resident", "launches": 8})
        log("fields resident", res["diffusion_fields_8x64_f64_32sweeps_resident"],
            res["diffusion_8_calls_64_f64_32sweeps_resident"])
        del us, vs

    if want("large"):
        # 16384^2 FP32: the production 200 sweeps (also the headline's
        # diffusion part) and single sweeps, the memory-bound depth 1
        c = inputs.uniform_16384_f32()
        u, v = dev(c["u"]), dev(c["v"])
        del c
        cfg = launch_config.diffusion("f32", 16384, 16384)
        nx = ny = 16384
        per_sweep = (nx * ny + (nx - 2) * (ny - 2)) * 4
        binding.stencil_diffuse2d(u, v, nx, 0.1, 8, cfg["map"], cfg["time_block"], 0, stream)
        t = timed(lambda: binding.stencil_diffuse2d(u, v, nx, 0.1, 200, cfg["map"], cfg["time_block"],
                                                    cfg["tile_rows"], stream), 5, False)
        L = binding.stencil_diffuse2d_launches(200, cfg["map"], cfg["time_block"])
        res["diffusion_16384_f32_200sweeps_production"] = entry(
            t, (nx - 2) * (ny - 2) * 200, per_sweep * L, {"launches": L, "time_block": cfg["time_block"]},
            ops=(OPS_PER_UPDATE, "f32"))
        log("16384", res["diffusion_16384_f32_200sweeps_production"])
        t = timed(lambda: binding.stencil_diffuse2d(u, v, nx, 0.1, 10, "tiled", 1, 0, stream), 5, False)
        res["diffusion_16384_f32_tiled_single_sweep"] = entry(
            t, (nx - 2) * (ny - 2) * 10, per_sweep * 10, {"sweeps": 10})
        log("16384 tiled", res["diffusion_16384_f32_tiled_single_sweep"])
        del u, v
        torch.cuda.empty_cache()

    if want("pack"):
        # pack, 8 x 201^3
        fh = inputs.fields_201cubed()
        f = dev(fh)
        nvar, nz, ny_, nx_ = f.shape
        cv = nvar * nx_ * ny_ * nz
        out = torch.empty(cv, dtype=torch.float64, device="cuda")
        for d, dn in enumerate("xyz"):
            maps = ("tiled", "per_cell", "per_cellvar")
            for m in maps:
                binding.field_pack(f, d, out=out, map=m)
            tg = timed_group({m: (lambda m=m: binding.field_pack(f, d, out=out, map=m)) for m in maps}, 10, True)
            for m in maps:
                extra = None
                if cpu and m == "tiled":
                    extra = {"oracle": cpu_entry(lambda: oracle.field_pack(fh, d), cv, 3, "the whole workload")}
                res[f"pack_201cubed_x8_{dn}_{m}"] = entry(tg[m], cv, 16 * cv, extra)
                log("pack", dn, m, res[f"pack_201cubed_x8_{dn}_{m}"])
        del f, out, fh
        torch.cuda.empty_cache()

    if want("flux"):
        # flux difference, 7 x 201x101x101
        fi = inputs.faces_201x101x101()
        args = (dev(fi.fx), dev(fi.fy), dev(fi.fz), dev(fi.dx), dev(fi.dy), dev(fi.dz))
        nvar, nxc, nyc, nzc = fi.shape
        cv = nvar * nxc * nyc * nzc
        nbytes = 8 * (fi.fx.size + fi.fy.size + fi.fz.size + cv + nxc + nyc + nzc)
        rhs = torch.empty(cv, dtype=torch.float64, device="cuda").view(nvar, nzc, nyc, nxc)
        maps = ("tiled", "per_cell", "per_cellvar")
        for m in maps:
            binding.flux_diff3d(*args, rhs=rhs, map=m)
        tg = timed_group({m: (lambda m=m: binding.flux_diff3d(*args, rhs=rhs, map=m)) for m in maps}, 10, True)
        for m in maps:
            extra = None
            if cpu and m == "tiled":
                extra = {"oracle": cpu_entry(lambda: oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz),
                                             cv, 3, "the whole workload")}
            res[f"flux_201x101x101_x7_{m}"] = entry(tg[m], cv, nbytes, extra)
            log("flux", m, res[f"flux_201x101x101_x7_{m}"])
        # one SSPRK stage fused with it: reads q0 and q, writes q' instead of rhs
        q0 = dev(inputs.normal_fields(nvar, nxc, nyc, nzc, 1060))
        qs = dev(inputs.normal_fields(nvar, nxc, nyc, nzc, 1061))
        qo = torch.empty_like(qs)
        sbytes = nbytes + 2 * 8 * cv
        for m in maps:
            binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo, map=m)
        tg = timed_group({m: (lambda m=m: binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo, map=m))
                          for m in maps}, 10, True)
        for m in maps:
            res[f"flux_stage_201x101x101_x7_{m}"] = entry(
                tg[m], cv, sbytes, {"note": "a separate update pass would add one write and one read of rhs"})
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
        maps = ("tiled", "per_cell", "per_cellvar")
        for m in maps:
            binding.flux_diff3d(*args, rhs=rhs, map=m)
        tg = timed_group({m: (lambda m=m: binding.flux_diff3d(*args, rhs=rhs, map=m)) for m in maps}, 10, True)
        for m in maps:
            extra = None
            if cpu and m == "tiled":
                extra = {"oracle": cpu_entry(lambda: oracle.flux_diff(fi.fx, fi.fy, None, fi.dx, fi.dy, None),
                                             cv, 3, "the whole workload")}
            res[f"flux2d_4800x1200_x6_{m}"] = entry(tg[m], cv, nbytes, extra)
            log("flux2d", m, res[f"flux2d_4800x1200_x6_{m}"])
        q0 = dev(inputs.normal_fields(nvar, nxc, nyc, 1, 1062))
        qs = dev(inputs.normal_fields(nvar, nxc, nyc, 1, 1063))
        qo = torch.empty_like(qs)
        sbytes = nbytes + 2 * 8 * cv
        binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo)
        t = timed(lambda: binding.flux_stage3d(*args, q0, qs, 0.75, 0.25, 1e-3, out=qo), 10, True)
        res["flux_stage2d_4800x1200_x6_tiled"] = entry(t, cv, sbytes)
        log("flux2d stage", res["flux_stage2d_4800x1200_x6_tiled"])
        del args, rhs, q0, qs, qo
        fh = inputs.fields_4800x1200()
        f = dev(fh)
        out = torch.empty(cv, dtype=torch.float64, device="cuda")
        for d, dn in ((0, "x"), (1, "y")):
            for m in maps:
                binding.field_pack(f, d, out=out, map=m)
            tg = timed_group({m: (lambda m=m: binding.field_pack(f, d, out=out, map=m)) for m in maps}, 10, True)
            for m in maps:
                extra = None
                if cpu and m == "tiled":
                    extra = {"oracle": cpu_entry(lambda: oracle.field_pack(fh, d), cv, 3, "the whole workload")}
                res[f"pack2d_4800x1200_x6_{dn}_{m}"] = entry(tg[m], cv, 16 * cv, extra)
                log("pack2d", dn, m, res[f"pack2d_4800x1200_x6_{dn}_{m}"])
        del f, out, fh
        torch.cuda.empty_cache()
    del flush_buf
    return res


if __name__ == "__main__":
    main()
