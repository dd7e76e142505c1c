"""GPU parity of field_pack / field_unpack / flux_diff3d against the CPU
oracle, bitwise (a pack is a bit copy; the flux difference has one rounding
per operation and correctly rounded reciprocals on both sides).

Shapes span several 64x64 transpose tiles with ragged edges, unit extents on
every axis, up to the maximum variable count, and variables that are slices
of one tensor (so their base addresses are not 16-byte aligned)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_bitwise, dev, host, require_gpu, say
from structured_grid_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu

MAPS = ["per_cell", "per_cellvar", "tiled"]
SHAPES = [  # nvar, nx, ny, nz
    (3, 67, 45, 23), (2, 130, 129, 3), (1, 1, 1, 1), (4, 1, 50, 70), (3, 70, 1, 65),
    (2, 66, 70, 1), (5, 1, 1, 99), (2, 99, 1, 1), (1, 1, 77, 1), (32, 9, 8, 7), (3, 200, 3, 129)]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


@pytest.mark.parametrize("nvar,nx,ny,nz", SHAPES)
@pytest.mark.parametrize("direction", [0, 1, 2])
def test_pack_and_unpack(nvar, nx, ny, nz, direction):
    f = inputs.normal_fields(nvar, nx, ny, nz, seed=nvar + nx + ny + nz)
    ref = oracle.field_pack(f, direction)
    fd = dev(f)  # one tensor: the variables are slices with odd offsets
    for m in MAPS:
        say("pack", nvar, nx, ny, nz, direction, m)
        out = binding.field_pack(fd, direction, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(out), ref, f"pack dir={direction} {m}")
        say("unpack", nvar, nx, ny, nz, direction, m)
        back = binding.field_unpack(out, nx, ny, nz, direction, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(back), f, f"unpack dir={direction} {m}")


@pytest.mark.parametrize("direction", [0, 1, 2])
def test_pack_separate_allocations_and_distinct_values(direction):
    nvar, nx, ny, nz = 4, 131, 70, 66
    f = inputs.distinct_fields(nvar, nx, ny, nz)
    ref = oracle.field_pack(f, direction)
    fl = [dev(f[v]) for v in range(nvar)]
    for m in MAPS:
        say("pack separate", direction, m)
        out = binding.field_pack(fl, direction, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(out), ref, f"pack {m}")


def test_pack_rejects_aliasing():
    f = torch.zeros(2, 4, 4, 4, dtype=torch.float64, device="cuda")
    with pytest.raises(binding.SGCError):
        binding.field_pack(f, 0, out=f.view(-1)[:128].view(2, 4, 4, 4))


FLUX_SHAPES = [  # nvar, nx, ny, nz, two_d
    (3, 67, 45, 23, False), (2, 130, 129, 3, False), (1, 1, 1, 1, False), (4, 1, 50, 70, False),
    (3, 70, 1, 65, False), (2, 66, 70, 1, False), (5, 300, 1, 1, False), (32, 9, 8, 7, False),
    (3, 257, 33, 300, False), (2, 513, 71, 1, True), (6, 48, 120, 1, True), (1, 1, 1, 1, True),
    (3, 1, 90, 1, True), (2, 90, 1, 1, True)]


def _flux_case(nvar, nx, ny, nz, two_d, seed):
    fi = inputs.normal_faces(nvar, nx, ny, nz, seed, two_d)
    ref = oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz)
    return fi, ref


@pytest.mark.parametrize("nvar,nx,ny,nz,two_d", FLUX_SHAPES)
def test_flux_difference(nvar, nx, ny, nz, two_d):
    fi, ref = _flux_case(nvar, nx, ny, nz, two_d, seed=7 * nvar + nx + ny + nz)
    fx, fy = dev(fi.fx), dev(fi.fy)
    fz = dev(fi.fz) if fi.fz is not None else None
    dx, dy = dev(fi.dx), dev(fi.dy)
    dz = dev(fi.dz) if fi.dz is not None else None
    for m in MAPS:
        say("flux", nvar, nx, ny, nz, two_d, m)
        rhs = binding.flux_diff3d(fx, fy, fz, dx, dy, dz, map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(rhs), ref, f"flux {m}")


def test_flux_reciprocal_is_correctly_rounded():
    """Widths chosen where 1/d is hard to round (mantissas near the tie
    region); the GPU's FP64 division must agree with the host's bit for bit."""
    nvar, nx, ny, nz = 1, 257, 3, 2
    fi, _ = _flux_case(nvar, nx, ny, nz, False, seed=99)
    g = np.random.Generator(np.random.PCG64(5))
    fi.dx[:] = 1.0 + g.integers(0, 2 ** 52, nx).astype(np.float64) * 2.0 ** -52
    fi.dx[:8] = [3.0, 7.0, 1.0 / 3.0, 0.1, 49.0, 1e-300, 1e300, 2.0 ** -1022]
    fi.fx[:] = 1.0
    fi.fx[..., 0] = 2.0
    ref = oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz)
    for m in MAPS:
        rhs = binding.flux_diff3d(dev(fi.fx), dev(fi.fy), dev(fi.fz), dev(fi.dx), dev(fi.dy),
                                  dev(fi.dz), map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(rhs), ref, f"reciprocal {m}")


def test_flux_separate_allocations():
    nvar, nx, ny, nz = 3, 120, 61, 40
    fi, ref = _flux_case(nvar, nx, ny, nz, False, seed=3)
    fx = [dev(fi.fx[v]) for v in range(nvar)]
    fy = [dev(fi.fy[v]) for v in range(nvar)]
    fz = [dev(fi.fz[v]) for v in range(nvar)]
    for m in MAPS:
        rhs = binding.flux_diff3d(fx, fy, fz, dev(fi.dx), dev(fi.dy), dev(fi.dz), map=m)
        torch.cuda.synchronize()
        assert_bitwise(host(rhs), ref, f"flux separate {m}")


def test_pack_and_flux_on_a_nonblocking_stream_are_deterministic():
    """Work enqueued on a side stream lands there (the caller synchronises
    that stream only) and repeated runs give the same bits."""
    f = inputs.normal_fields(5, 67, 41, 19, 911)
    fi = inputs.normal_faces(5, 67, 41, 19, 912)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        fd = dev(f)
        args = [dev(a) for a in (fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz)]
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            packs = [binding.field_pack(fd, d, stream=s) for d in (0, 1, 2)]
            rhs = binding.flux_diff3d(*args, stream=s)
        s.synchronize()
        outs.append([host(p) for p in packs] + [host(rhs)])
    for d in (0, 1, 2):
        assert_bitwise(outs[0][d].reshape(-1), oracle.field_pack(f, d).reshape(-1), f"stream pack {d}")
    assert_bitwise(outs[0][3], oracle.flux_diff(fi.fx, fi.fy, fi.fz, fi.dx, fi.dy, fi.dz), "stream flux")
    for a, b in zip(outs[0], outs[1]):
        assert_bitwise(a, b, "determinism")
