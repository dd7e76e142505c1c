"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Every output element is compared bit for bit.

* Diffusion, 4096^2 FP64 and FP32 for 1000 steps: the production settings
  against the oracle run on the whole grid (about 11-15 s of one host core
  per precision), and every mapping, the production depth included, against
  one another at the full step count; plus all mappings against the oracle
  at a few steps.
* Diffusion, 16384^2 FP32 for 200 steps: the production settings against the
  oracle on every cell, the oracle run on bands of rows in parallel threads
  (each band holds its rows' whole domain of dependence, so a band's cut edge
  cannot reach them: ``oracle.diffuse2d_rows``, pinned against the whole-grid
  oracle on the CPU), and against the single-step map over the whole grid.
* Pack (8 x 201^3 along x/y/z), flux difference (7 x 201x101x101), and the
  2D workload (6 x 4800x1200 flux difference and x/y packs): whole outputs.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_bitwise, dev, host, require_gpu, say
from structured_grid_cfd_amd import binding, inputs, launch_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _run(u0, v0, nx, alpha, steps, cfg):
    u, v = dev(u0), dev(v0)
    in_v = binding.stencil_diffuse2d(u, v, nx, alpha, steps, cfg["map"], cfg["time_block"],
                                     cfg["tile_rows"])
    torch.cuda.synchronize()
    out = host(v if in_v else u)
    del u, v
    torch.cuda.empty_cache()
    return out


def _oracle_in_bands(u0, nx, alpha, steps, band_rows, workers=8):
    """The whole-grid oracle result, assembled from bands of rows computed in
    parallel threads (the oracle's C code runs outside the interpreter lock)."""
    ny = u0.shape[0]
    out = np.empty_like(u0)
    edges = list(range(0, ny, band_rows)) + [ny]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(oracle.diffuse2d_rows, u0, nx, alpha, steps, j0, j1): (j0, j1)
                for j0, j1 in zip(edges[:-1], edges[1:])}
        for f in cf.as_completed(futs):
            j0, j1 = futs[f]
            out[j0:j1] = f.result()
    return out


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_diffusion_4096_1000_steps_whole_grid(dt):
    """The production settings (temporal blocking, depth 10 in FP64 and 12 in
    FP32) after the full 1000 steps, every cell against the oracle run on the
    whole grid."""
    c = inputs.uniform_4096(np.float64 if dt == "f64" else np.float32)
    cfg = launch_config.diffusion(dt, c["nx"], c["ny"])
    assert cfg["map"] == "temporal" and cfg["time_block"] == (10 if dt == "f64" else 12)
    say("uniform_4096 production, whole grid", dt, cfg)
    got = _run(c["u"], c["v"], c["nx"], c["alpha"], c["steps"], cfg)
    assert np.all(np.isfinite(got)) and got.min() >= 0 and got.max() < 1
    say("uniform_4096 oracle, whole grid", dt)
    ref = oracle.diffuse2d_result(c["u"], c["nx"], c["alpha"], c["steps"])
    assert_bitwise(got, ref, f"uniform_4096 {dt} production vs oracle")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_diffusion_4096_all_maps_whole_grid_few_steps(dt):
    c = inputs.uniform_4096(np.float64 if dt == "f64" else np.float32, steps=6)
    ref = oracle.diffuse2d_result(c["u"], c["nx"], 0.1, 6)
    for m, tb in [("collapse_branch", 1), ("contig", 1), ("strided", 1), ("tiled", 1),
                  ("temporal", 3), ("temporal", 6)]:
        say("uniform_4096 6 steps", dt, m, tb)
        got = _run(c["u"], c["v"], c["nx"], 0.1, 6, {"map": m, "time_block": tb, "tile_rows": 0})
        assert_bitwise(got, ref, f"uniform_4096 {m} T={tb}")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_diffusion_4096_all_maps_agree_at_1000_steps(dt):
    """The three page layouts and this library's sweeps, the production
    depths 10 and 12 among them, return one bit pattern after the full 1000
    steps."""
    c = inputs.uniform_4096(np.float64 if dt == "f64" else np.float32)
    first = None
    for m, tb in [("temporal", 10), ("temporal", 12), ("temporal", 8), ("tiled", 1), ("contig", 1),
                  ("collapse_branch", 1), ("strided", 1), ("temporal", 5)]:
        say("uniform_4096 1000 steps", dt, m, tb)
        got = _run(c["u"], c["v"], c["nx"], 0.1, c["steps"], {"map": m, "time_block": tb, "tile_rows": 0})
        if first is None:
            first = got
        else:
            assert_bitwise(got, first, f"{m} T={tb} vs temporal 10")


def test_diffusion_16384_fp32_200_steps_whole_grid():
    """16384^2 FP32 after 200 steps in the production settings: every cell
    against the oracle (run on bands of rows) and against the single-step
    map."""
    c = inputs.uniform_16384_f32()
    cfg = launch_config.diffusion("f32", c["nx"], c["ny"])
    say("uniform_16384_f32 production, whole grid", cfg)
    got = _run(c["u"], c["v"], c["nx"], c["alpha"], c["steps"], cfg)
    assert got.min() >= 0 and got.max() < 1
    say("uniform_16384_f32 single-step map, whole grid")
    tiled = _run(c["u"], c["v"], c["nx"], c["alpha"], c["steps"],
                 {"map": "tiled", "time_block": 1, "tile_rows": 0})
    assert_bitwise(got, tiled, "uniform_16384_f32 production vs single-step map")
    del tiled
    say("uniform_16384_f32 oracle in bands of 2048 rows")
    ref = _oracle_in_bands(c["u"], c["nx"], c["alpha"], c["steps"], 2048)
    assert_bitwise(got, ref, "uniform_16384_f32 production vs oracle")


@pytest.mark.parametrize("direction", [0, 1, 2])
def test_pack_8_fields_201cubed(direction):
    f = inputs.fields_201cubed()
    ref = oracle.field_pack(f, direction)
    fd = dev(f)
    for m in ["tiled", "per_cell", "per_cellvar"]:
        say("fields_201cubed pack", direction, m)
        out = binding.field_pack(fd, direction, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(out), ref, f"fields_201cubed dir={direction} {m}")
        del out


def test_flux_7_fields_201x101x101():
    fi = inputs.faces_201x101x101()
    ref = oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz)
    args = (dev(fi.fx), dev(fi.fy), dev(fi.fz), dev(fi.dx), dev(fi.dy), dev(fi.dz))
    for m in ["tiled", "per_cell", "per_cellvar"]:
        say("faces_201x101x101 flux", m)
        rhs = binding.flux_diff3d(*args, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(rhs), ref, f"faces_201x101x101 {m}")


def test_2d_flux_and_packs_4800x1200():
    fi = inputs.faces_4800x1200()
    ref = oracle.flux_diff(fi.fx, fi.fy, None, fi.dx, fi.dy, None)
    args = (dev(fi.fx), dev(fi.fy), None, dev(fi.dx), dev(fi.dy), None)
    for m in ["tiled", "per_cell", "per_cellvar"]:
        say("4800x1200 flux", m)
        rhs = binding.flux_diff3d(*args, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(rhs), ref, f"4800x1200 flux {m}")
    f = inputs.fields_4800x1200()
    fd = dev(f)
    for direction in (0, 1):
        pref = oracle.field_pack(f, direction)
        for m in ["tiled", "per_cell", "per_cellvar"]:
            say("4800x1200 pack", direction, m)
            out = binding.field_pack(fd, direction, map=m)
            torch.cuda.synchronize()
            assert_bitwise(host(out), pref, f"4800x1200 pack dir={direction} {m}")


def test_flux_stage_201x101x101_and_4800x1200():
    """The SSPRK stage fused with the flux difference on the 7 x 201x101x101
    and 6 x 4800x1200 workloads, in the benchmark's launch configuration."""
    for fi in (inputs.faces_201x101x101(), inputs.faces_4800x1200()):
        nvar, nx, ny, nz = fi.shape
        g = np.random.Generator(np.random.PCG64(1099))
        q0 = g.standard_normal((nvar, nz, ny, nx))
        q = g.standard_normal((nvar, nz, ny, nx))
        ref = oracle.flux_stage(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz, q0, q, 1.0 / 3.0, 2.0 / 3.0, 1e-3)
        say("flux stage full size", fi.shape)
        out = binding.flux_stage3d(dev(fi.fx), dev(fi.fy), dev(fi.fz) if fi.fz is not None else None,
                                   dev(fi.dx), dev(fi.dy), dev(fi.dz) if fi.dz is not None else None,
                                   dev(q0), dev(q), 1.0 / 3.0, 2.0 / 3.0, 1e-3, map=launch_config.FLUX["map"])
        torch.cuda.synchronize()
        assert_bitwise(host(out), ref, f"stage {fi.shape}")
        del out
        torch.cuda.empty_cache()
