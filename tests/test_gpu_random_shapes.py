"""GPU parity on seeded random shapes: every entry point against the CPU
oracle, bit for bit, over cases drawn from a fixed seed per case.

Diffusion: grid sizes 3..400 on each side (a third of them up to 24),
padded leading dimensions with a NaN sentinel in the padding, element
offsets of the base pointers, dirty edge rings, both precisions, every map
(the page layouts, TILED, TEMPORAL at depths 1..12 with automatic or explicit
tile heights, RESIDENT where the grid fits), 0..40 steps and several alpha.
Several fields per call: 1..5 fields through the marching and resident maps.
Pack / unpack: 1..6 fields of 1..70 cells per side, every direction and map.
Flux difference and the fused SSPRK stage: 1..5 fields, 2D and 3D, every
map, stage outputs fresh or in place of q or q0.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_bitwise, dev, host, require_gpu, say
from structured_grid_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu

N_DIFFUSION, N_FIELDS, N_PACK, N_FLUX = 160, 24, 60, 60


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _rng(tag, case):
    return np.random.Generator(np.random.PCG64(91000 + 1000 * tag + case))


def _side(g):
    return int(g.integers(3, 25)) if g.random() < 1 / 3 else int(g.integers(3, 401))


def _diffusion_case(case):
    g = _rng(1, case)
    nx, ny = _side(g), _side(g)
    dtype = np.float64 if g.random() < 0.5 else np.float32
    pad = int(g.choice([0, 0, 1, 3, 17]))
    ld = nx + pad
    maps = ["temporal", "temporal", "temporal", "tiled", "collapse_branch", "contig", "strided"]
    if nx <= 64 and ny <= 128:
        maps += ["resident", "resident"]
    m = str(g.choice(maps))
    tb = int(g.integers(1, 13)) if m == "temporal" else 1
    rows = int(g.integers(1, ny + 1)) if m in ("tiled", "temporal") and g.random() < 0.3 else 0
    steps = 0 if g.random() < 0.05 else int(g.integers(1, 41))
    alpha = float(g.choice([0.1, 0.25, 0.05, 0.2, 0.125]))
    offset = int(g.integers(1, 3)) if g.random() < 0.2 else 0
    return nx, ny, ld, dtype, m, tb, rows, steps, alpha, offset, g


@pytest.mark.parametrize("case", range(N_DIFFUSION))
def test_random_diffusion(case):
    nx, ny, ld, dtype, m, tb, rows, steps, alpha, offset, g = _diffusion_case(case)
    u0, v0 = inputs.uniform_grid(nx, ny, 50000 + case, dtype, ld=ld, pad_value=np.nan)
    # dirty edge rings in both buffers: the sweeps treat them as 0
    for a in (u0, v0):
        a[0, :nx] = g.random(nx)
        a[-1, :nx] = g.random(nx)
        a[:, 0] = g.random(ny)
        a[:, nx - 1] = g.random(ny)
    say("random diffusion", case, (nx, ny, ld), dtype.__name__, m, tb, rows, steps, alpha, offset)
    # element offset of both bases: slices of larger buffers
    n = ny * ld
    ub = torch.full((n + offset,), float("nan"), dtype=torch.float64 if dtype == np.float64 else torch.float32,
                    device="cuda")
    vb = torch.full_like(ub, float("nan"))
    ub[offset:] = dev(u0).reshape(-1)
    vb[offset:] = dev(v0).reshape(-1)
    u = ub[offset:].view(ny, ld)
    v = vb[offset:].view(ny, ld)
    in_v = binding.stencil_diffuse2d(u, v, nx, alpha, steps, m, tb, rows)
    torch.cuda.synchronize()
    uh, vh = host(u), host(v)
    got = vh if in_v else uh
    ru, rv = u0.copy(), v0.copy()
    ref_in_v = oracle.diffuse2d(ru, rv, nx, alpha, steps)
    ref = rv if ref_in_v else ru
    assert in_v == ref_in_v == (steps % 2 == 1)
    assert_bitwise(got[:, :nx], ref[:, :nx], f"case {case}")
    assert np.all(np.isnan(uh[:, nx:])) and np.all(np.isnan(vh[:, nx:])), "padding touched"
    assert np.isnan(host(ub[:offset])).all() and np.isnan(host(vb[:offset])).all(), "bytes before the base touched"


@pytest.mark.parametrize("case", range(N_FIELDS))
def test_random_fields(case):
    g = _rng(2, case)
    nvar = int(g.integers(1, 6))
    dtype = np.float64 if g.random() < 0.5 else np.float32
    if g.random() < 0.3:
        nx, ny, m, tb = int(g.integers(3, 65)), int(g.integers(3, 129)), "resident", 1
    else:
        nx, ny = _side(g), _side(g)
        m = "temporal" if g.random() < 0.75 else "tiled"
        tb = int(g.integers(1, 13)) if m == "temporal" else 1
    ld = nx + int(g.choice([0, 0, 5]))
    steps = int(g.integers(1, 31))
    say("random fields", case, nvar, (nx, ny, ld), dtype.__name__, m, tb, steps)
    pairs = [inputs.uniform_grid(nx, ny, 60000 + 10 * case + k, dtype, ld=ld, pad_value=np.nan) for k in range(nvar)]
    us = [dev(a) for a, _ in pairs]
    vs = [dev(b) for _, b in pairs]
    in_v = binding.stencil_diffuse2d_fields(us, vs, nx, 0.1, steps, m, tb)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(pairs):
        ru, rv = a.copy(), b.copy()
        ref_in_v = oracle.diffuse2d(ru, rv, nx, 0.1, steps)
        assert in_v == ref_in_v
        got = host(vs[k] if in_v else us[k])
        assert_bitwise(got[:, :nx], (rv if ref_in_v else ru)[:, :nx], f"case {case} field {k}")


@pytest.mark.parametrize("case", range(N_PACK))
def test_random_pack_unpack(case):
    g = _rng(3, case)
    nvar = int(g.integers(1, 7))
    nx, ny, nz = (int(g.integers(1, 71)) for _ in range(3))
    d = int(g.integers(0, 3))
    m = str(g.choice(["tiled", "tiled", "per_cell", "per_cellvar"]))
    say("random pack", case, nvar, (nx, ny, nz), d, m)
    f = inputs.normal_fields(nvar, nx, ny, nz, 70000 + case)
    fd = dev(f)
    out = binding.field_pack(fd, d, map=m)
    torch.cuda.synchronize()
    ref = oracle.field_pack(f, d)
    assert_bitwise(host(out), ref, f"pack case {case}")
    back = binding.field_unpack(dev(ref), nx, ny, nz, d, map=m)
    torch.cuda.synchronize()
    assert_bitwise(host(back), oracle.field_unpack(ref, nx, ny, nz, d), f"unpack case {case}")
    assert_bitwise(host(back), f, f"round trip case {case}")


@pytest.mark.parametrize("case", range(N_FLUX))
def test_random_flux_and_stage(case):
    g = _rng(4, case)
    nvar = int(g.integers(1, 6))
    two_d = g.random() < 0.35
    nx, ny = int(g.integers(1, 51)), int(g.integers(1, 51))
    nz = 1 if two_d else int(g.integers(1, 51))
    m = str(g.choice(["tiled", "tiled", "per_cell", "per_cellvar"]))
    say("random flux", case, nvar, (nx, ny, nz), "2D" if two_d else "3D", m)
    fi = inputs.normal_faces(nvar, nx, ny, nz, 80000 + case, two_d=two_d)
    args = (dev(fi.fx), dev(fi.fy), dev(fi.fz) if fi.fz is not None else None, dev(fi.dx), dev(fi.dy),
            dev(fi.dz) if fi.dz is not None else None)
    rhs = binding.flux_diff3d(*args, map=m)
    torch.cuda.synchronize()
    assert_bitwise(host(rhs), oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz), f"flux case {case}")
    q0 = g.standard_normal((nvar, nz, ny, nx))
    q = g.standard_normal((nvar, nz, ny, nx))
    a, b = [(0.0, 1.0), (0.75, 0.25), (1.0 / 3.0, 2.0 / 3.0)][int(g.integers(0, 3))]
    dt = float(g.uniform(1e-4, 1e-2))
    where = str(g.choice(["fresh", "q", "q0"]))
    ref = oracle.flux_stage(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz, q0, q, a, b, dt)
    q0d, qd = dev(q0), dev(q)
    out = {"fresh": None, "q": qd, "q0": q0d}[where]
    got = binding.flux_stage3d(*args, q0d, qd, a, b, dt, out=out, map=m)
    torch.cuda.synchronize()
    assert_bitwise(host(got), ref, f"stage case {case} ({where})")
