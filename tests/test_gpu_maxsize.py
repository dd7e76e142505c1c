"""GPU parity at the largest arrays the ABI accepts, where every 32-bit
index, row offset and launch-grid computation runs at its limit.

Diffusion: ld * ny just under 2^31 elements (FP32, 46341 x 46340, 8.6 GB per
buffer), every map, and two such fields in one multi-field launch.

The grid is too large to fill from the random generator in a test, so it is
the hashed grid of ``inputs.hashed_window``: interior (a_i + b_j) / 2 from
hashed column and row terms.  The device copy is built from the same two
float32 operations on a and b (checked against host windows), the result is
read back only at sampled cells, and each sampled cell is compared bit for bit
with the oracle run on the sub-grid that holds its whole domain of dependence.

Flux difference and the fused SSPRK stage: one variable on 1289^3 cells,
every face array at 2.14e9 elements; sampled cells against the oracle's
one-cell problem.

Pack: nvar * nx * ny * nz just under 2^31 (2 FP64 fields of 1290 x 1290 x
645, 8.6 GB each).  The packed arrays are checked on the device against the
fields' axis permutation (the definition of the y and z orders, a property
that holds at any size; the oracle pins the same permutation on small
arrays), and unpacking must return the fields bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import require_gpu, say
from structured_grid_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu

NX, NY = 46341, 46340
assert NX * NY <= 2 ** 31 - 1 < NX * (NY + 1)


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def grid():
    a, b = inputs.hashed_parts(NX, NY, np.float32, salt=2031)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    u0 = torch.empty(NY, NX, dtype=torch.float32, device="cuda")
    rows = 4096
    for j0 in range(0, NY, rows):
        blk = u0[j0:j0 + rows]
        torch.add(bd[j0:j0 + rows, None], ad[None, :], out=blk)
        blk.mul_(0.5)
    u0[0].zero_()
    u0[-1].zero_()
    u0[:, 0].zero_()
    u0[:, -1].zero_()
    torch.cuda.synchronize()
    for i0, i1, j0, j1 in [(0, 40, 0, 30), (NX - 37, NX, NY - 29, NY), (20000, 20050, 30000, 30010)]:
        want = inputs.hashed_window(a, b, i0, i1, j0, j1)
        got = u0[j0:j1, i0:i1].cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (i0, j0)
    yield a, b, u0
    del u0
    torch.cuda.empty_cache()


def _oracle_cell(a, b, i, j, alpha, steps):
    r = steps + 1
    i0, i1 = max(0, i - r), min(NX, i + r + 1)
    j0, j1 = max(0, j - r), min(NY, j + r + 1)
    sub = inputs.hashed_window(a, b, i0, i1, j0, j1)
    return oracle.diffuse2d_result(sub, i1 - i0, alpha, steps)[j - j0, i - i0]


@pytest.mark.parametrize("m,tb,steps", [("temporal", 10, 10), ("temporal", 2, 2), ("temporal", 12, 12),
                                        ("tiled", 1, 1), ("collapse_branch", 1, 2), ("contig", 1, 1),
                                        ("strided", 1, 1)])
def test_diffusion_at_the_element_limit(grid, m, tb, steps):
    a, b, u0 = grid
    say("max size", m, tb, steps, NX, NY)
    u = u0.clone()
    v = torch.empty_like(u)
    in_v = binding.stencil_diffuse2d(u, v, NX, 0.1, steps, m, tb)
    torch.cuda.synchronize()
    assert in_v == (steps % 2 == 1)
    res = v if in_v else u
    g = np.random.Generator(np.random.PCG64(2032))
    pts = [(1, 1), (NX - 2, NY - 2), (1, NY - 2), (NX - 2, 1), (NX // 2, NY - 2), (NX - 2, NY // 2),
           (0, NY - 1), (NX - 1, NY - 1), (NX - 1, 0)]
    pts += [(int(g.integers(1, NX - 1)), int(g.integers(NY - 200, NY - 1))) for _ in range(6)]
    pts += [(int(g.integers(1, NX - 1)), int(g.integers(1, NY - 1))) for _ in range(6)]
    for i, j in pts:
        got = np.float32(res[j, i].item())
        ref = np.float32(_oracle_cell(a, b, i, j, 0.1, steps))
        assert got.view(np.uint32) == ref.view(np.uint32), (m, i, j, got, ref)
    del u, v
    torch.cuda.empty_cache()


def _device_grid(a, b):
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    u = torch.empty(b.size, a.size, dtype=torch.float32, device="cuda")
    for j0 in range(0, b.size, 4096):
        blk = u[j0:j0 + 4096]
        torch.add(bd[j0:j0 + 4096, None], ad[None, :], out=blk)
        blk.mul_(0.5)
    u[0].zero_()
    u[-1].zero_()
    u[:, 0].zero_()
    u[:, -1].zero_()
    return u


def test_two_fields_at_the_element_limit():
    """Two 46341 x 46340 FP32 fields stepped in the same depth-10 launch of
    the multi-field march: sampled cells of each against the oracle."""
    parts = [inputs.hashed_parts(NX, NY, np.float32, salt=2050 + k) for k in range(2)]
    us = [_device_grid(a, b) for a, b in parts]
    vs = [torch.empty_like(u) for u in us]
    say("max size, two fields")
    in_v = binding.stencil_diffuse2d_fields(us, vs, NX, 0.1, 10, "temporal", 10)
    torch.cuda.synchronize()
    assert not in_v
    g = np.random.Generator(np.random.PCG64(2052))
    pts = [(1, 1), (NX - 2, NY - 2), (NX // 2, NY - 2)]
    pts += [(int(g.integers(1, NX - 1)), int(g.integers(1, NY - 1))) for _ in range(6)]
    for k, (a, b) in enumerate(parts):
        for i, j in pts:
            got = np.float32(us[k][j, i].item())
            ref = np.float32(_oracle_cell(a, b, i, j, 0.1, 10))
            assert got.view(np.uint32) == ref.view(np.uint32), (k, i, j, got, ref)
    del us, vs
    torch.cuda.empty_cache()


PNVAR, PNX, PNY, PNZ = 2, 1290, 1290, 645
assert PNVAR * PNX * PNY * PNZ <= 2 ** 31 - 1


@pytest.mark.parametrize("m", ["tiled", "per_cell", "per_cellvar"])
def test_pack_roundtrip_at_the_element_limit(m):
    a, b = inputs.hashed_parts(PNX, PNVAR * PNZ * PNY, np.float64, salt=2033)
    f = (torch.from_numpy(b).cuda()[:, None] + torch.from_numpy(a).cuda()[None, :]).mul_(0.5)
    f = f.view(PNVAR, PNZ, PNY, PNX)
    for direction, perm in ((1, (0, 1, 3, 2)), (2, (0, 3, 2, 1))):
        say("max pack", m, direction)
        packed = binding.field_pack(f, direction, map=m)
        torch.cuda.synchronize()
        want = f.permute(*perm)
        assert torch.equal(packed.view(want.shape).view(torch.int64), want.contiguous().view(torch.int64))
        del want
        back = binding.field_unpack(packed, PNX, PNY, PNZ, direction, map=m)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int64), f.view(torch.int64))
        del packed, back
        torch.cuda.empty_cache()
    del f
    torch.cuda.empty_cache()


def test_x_pack_copy_at_the_limit_with_mismatched_phase():
    """One FP64 field of 2^31 - 2 elements (42966 x 49981) copied by the x
    pack into an output whose address differs from the field's by 8 bytes
    modulo 16, so the copy takes its 8-byte path up to the last chunk, which
    starts 512 elements before 2^31 (a bound checked without overflowing
    32-bit arithmetic); then back.  The element before the output stays
    untouched."""
    nx, ny = 42966, 49981
    assert nx * ny == 2 ** 31 - 2
    a, b = inputs.hashed_parts(nx, ny, np.float64, salt=2034)
    f = (torch.from_numpy(b).cuda()[:, None] + torch.from_numpy(a).cuda()[None, :]).mul_(0.5)
    f = f.view(1, 1, ny, nx)
    buf = torch.full((nx * ny + 1,), 7.25, dtype=torch.float64, device="cuda")
    out = buf[1:].view(1, 1, ny, nx)
    say("max x pack, mismatched phase")
    binding.field_pack(f, 0, out=out, map="tiled")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int64), f.view(torch.int64))
    assert buf[0].item() == 7.25
    back = torch.empty_like(f)
    binding.field_unpack(out, nx, ny, 1, 0, fields=back, map="tiled")
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int64), f.view(torch.int64))
    del f, buf, out, back
    torch.cuda.empty_cache()


# The flux entry points bound (nx+1)(ny+1)(nz+1), which covers every face
# array, by 2^31 - 1: 1290^3 = 2^31 - 794648.
FNX, FNY, FNZ = 1289, 1289, 1289
assert (FNX + 1) * (FNY + 1) * (FNZ + 1) <= 2 ** 31 - 1


def _hashed_device(rows, cols, salt):
    a, b = inputs.hashed_parts(cols, rows, np.float64, salt=salt)
    t = (torch.from_numpy(b).cuda()[:, None] + torch.from_numpy(a).cuda()[None, :]).mul_(0.5)
    return t, a, b


@pytest.mark.parametrize("m", ["tiled", "per_cell", "per_cellvar"])
def test_flux_difference_at_the_element_limit(m):
    """One variable on 1289^3 cells: face arrays of 2.14e9 elements and
    (nx+1)(ny+1)(nz+1) at 99.96% of the entry point's 2^31 - 1 bound (17 GB
    per array).  Sampled cells are compared bit for bit with the
    oracle run on the one-cell problem made of that cell's six faces and
    three widths (a cell's value depends on nothing else)."""
    fx, ax, bx = _hashed_device(FNZ * FNY, FNX + 1, 2035)
    fy, ay, by = _hashed_device(FNZ * (FNY + 1), FNX, 2036)
    fz, az, bz = _hashed_device((FNZ + 1) * FNY, FNX, 2037)
    g = np.random.Generator(np.random.PCG64(2038))
    dx, dy, dz = (g.uniform(0.5, 1.5, n) / n for n in (FNX, FNY, FNZ))
    say("max flux", m)
    rhs = binding.flux_diff3d(fx.view(1, FNZ, FNY, FNX + 1), fy.view(1, FNZ, FNY + 1, FNX),
                              fz.view(1, FNZ + 1, FNY, FNX), torch.from_numpy(dx).cuda(),
                              torch.from_numpy(dy).cuda(), torch.from_numpy(dz).cuda(), map=m)
    torch.cuda.synchronize()
    face = lambda a, b, row, col: (b[row] + a[col]) * 0.5  # noqa: E731 -- the device's two operations
    pts = [(0, 0, 0), (FNX - 1, FNY - 1, FNZ - 1), (FNX - 1, 0, FNZ - 1), (0, FNY - 1, FNZ - 1)]
    pts += [tuple(int(g.integers(0, n)) for n in (FNX, FNY, FNZ)) for _ in range(12)]
    for j, k, l in pts:
        cfx = np.array([face(ax, bx, k + FNY * l, j), face(ax, bx, k + FNY * l, j + 1)]).reshape(1, 1, 1, 2)
        cfy = np.array([face(ay, by, k + (FNY + 1) * l, j),
                        face(ay, by, k + 1 + (FNY + 1) * l, j)]).reshape(1, 1, 2, 1)
        cfz = np.array([face(az, bz, k + FNY * l, j), face(az, bz, k + FNY * (l + 1), j)]).reshape(1, 2, 1, 1)
        ref = oracle.flux_diff(cfx, cfy, cfz, dx[j:j + 1], dy[k:k + 1], dz[l:l + 1])[0, 0, 0, 0]
        got = rhs[0, l, k, j].item()
        assert np.float64(got).view(np.uint64) == np.float64(ref).view(np.uint64), (m, j, k, l, got, ref)
    del fx, fy, fz, rhs
    torch.cuda.empty_cache()


def test_flux_stage_at_the_element_limit():
    """The SSPRK stage fused with the flux difference on the same 1289^3
    problem, q updated in place: sampled cells against the oracle's one-cell
    stage."""
    fx, ax, bx = _hashed_device(FNZ * FNY, FNX + 1, 2039)
    fy, ay, by = _hashed_device(FNZ * (FNY + 1), FNX, 2040)
    fz, az, bz = _hashed_device((FNZ + 1) * FNY, FNX, 2041)
    q0, aq0, bq0 = _hashed_device(FNZ * FNY, FNX, 2042)
    q, aq, bq = _hashed_device(FNZ * FNY, FNX, 2043)
    g = np.random.Generator(np.random.PCG64(2044))
    dx, dy, dz = (g.uniform(0.5, 1.5, n) / n for n in (FNX, FNY, FNZ))
    a, b, dt = 0.75, 0.25, 0.0125
    say("max flux stage")
    q4 = q.view(1, FNZ, FNY, FNX)
    binding.flux_stage3d(fx.view(1, FNZ, FNY, FNX + 1), fy.view(1, FNZ, FNY + 1, FNX),
                         fz.view(1, FNZ + 1, FNY, FNX), torch.from_numpy(dx).cuda(),
                         torch.from_numpy(dy).cuda(), torch.from_numpy(dz).cuda(),
                         q0.view(1, FNZ, FNY, FNX), q4, a, b, dt, out=q4, map="tiled")
    torch.cuda.synchronize()
    face = lambda a_, b_, row, col: (b_[row] + a_[col]) * 0.5  # noqa: E731 -- the device's two operations
    pts = [(0, 0, 0), (FNX - 1, FNY - 1, FNZ - 1), (FNX - 1, 0, FNZ - 1)]
    pts += [tuple(int(g.integers(0, n)) for n in (FNX, FNY, FNZ)) for _ in range(10)]
    for j, k, l in pts:
        cfx = np.array([face(ax, bx, k + FNY * l, j), face(ax, bx, k + FNY * l, j + 1)]).reshape(1, 1, 1, 2)
        cfy = np.array([face(ay, by, k + (FNY + 1) * l, j),
                        face(ay, by, k + 1 + (FNY + 1) * l, j)]).reshape(1, 1, 2, 1)
        cfz = np.array([face(az, bz, k + FNY * l, j), face(az, bz, k + FNY * (l + 1), j)]).reshape(1, 2, 1, 1)
        cq0 = np.array([face(aq0, bq0, k + FNY * l, j)]).reshape(1, 1, 1, 1)
        cq = np.array([face(aq, bq, k + FNY * l, j)]).reshape(1, 1, 1, 1)
        ref = oracle.flux_stage(cfx, cfy, cfz, dx[j:j + 1], dy[k:k + 1], dz[l:l + 1], cq0, cq, a, b, dt)
        got = q4[0, l, k, j].item()
        assert np.float64(got).view(np.uint64) == np.float64(ref[0, 0, 0, 0]).view(np.uint64), (j, k, l)
    del fx, fy, fz, q0, q, q4
    torch.cuda.empty_cache()
