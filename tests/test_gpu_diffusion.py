"""GPU parity of stencil_diffuse2d against the CPU oracle, element by element
and bitwise (both sides compute without contraction in the same order, so
exactly one result is correct).

Cases: the 64x64 impulse workload; the Qiita Part 3 validation matrix (31x27,
steps 7/8/31/32, FP32 and FP64, every mapping; section 10); ragged sizes that
span several strips and row tiles with partial last strips/tiles; padded
leading dimensions; unaligned base pointers; dirty input edges; zero steps;
several alpha values; every time block 1..12 including blocks that do not
divide the step count; explicit tile heights down to one row.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (assert_bitwise, dev, gpu_diffuse, host, oracle_diffuse, require_gpu,
                         say)
from structured_grid_cfd_amd import binding, inputs

pytestmark = pytest.mark.gpu

PAGE_MAPS = ["collapse_branch", "contig", "strided"]
ALL_MAPS = [(m, 1) for m in PAGE_MAPS + ["tiled", "resident"]] + [("temporal", t) for t in range(1, 13)]
DT = {"f64": np.float64, "f32": np.float32}


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _check(u0, v0, nx, alpha, steps, m, tb=1, rows=0, what=""):
    say(what, m, tb, rows, u0.shape, u0.dtype, steps)
    got, in_v, uh, vh = gpu_diffuse(u0, v0, nx, alpha, steps, m, tb, rows)
    ref, ref_in_v = oracle_diffuse(u0, v0, nx, alpha, steps)
    assert in_v == ref_in_v == (steps % 2 == 1)
    assert_bitwise(got[:, :nx], ref[:, :nx], f"{what} {m} T={tb} rows={rows}")
    # padding columns of both buffers untouched
    assert_bitwise(uh[:, nx:], u0[:, nx:], "u padding")
    assert_bitwise(vh[:, nx:], v0[:, nx:], "v padding")
    return got


@pytest.mark.parametrize("m,tb", ALL_MAPS)
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_impulse_64x64_32_steps(m, tb, dt):
    cfg = inputs.impulse_64(DT[dt])
    got = _check(cfg["u"], cfg["v"], 64, cfg["alpha"], cfg["steps"], m, tb, what="impulse_64")
    # the impulse spreads from its cell, which stays the largest, and no
    # value turns negative (alpha <= 1/4)
    assert got.max() == got[32, 32] and got.min() == 0


@pytest.mark.parametrize("m,tb", ALL_MAPS)
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_rounding_ties_and_unfused_products(m, tb, dt):
    """The two one-step closed forms that fix the rounding order (the oracle
    pins them by hand), planted at interior and edge-adjacent cells of a
    zero grid: a tie in ((W + E) + S) + N that only the left-to-right order
    resolves to 1 - h, and an update c + alpha*t whose product must be
    rounded before the sum."""
    dtype = DT[dt]
    nx, ny = (60, 90) if m == "resident" else (301, 203)
    h = float(np.finfo(dtype).eps) / 2
    tie_cells = [(2, 2), (nx // 2, ny // 2), (nx - 2, ny - 3), (min(65, nx // 3), 2), (nx - 2, 2)]
    u = np.zeros((ny, nx), dtype=dtype)
    for i, j in tie_cells:
        u[j, i - 1], u[j - 1, i], u[j + 1, i] = 1.0, h, -h
    got = _check(u, np.zeros_like(u), nx, 1.0, 1, m, tb, what="sum-order ties")
    for i, j in tie_cells:
        assert got[j, i] == dtype(1.0 - h), (i, j)

    p = 30 if dtype == np.float64 else 12
    t = 1.0 + 2.0 ** -(p + 1)
    prod_cells = [(2, 1), (nx // 2, ny // 2), (nx - 2, ny - 2), (min(64, nx // 3), 5)]
    u = np.zeros((ny, nx), dtype=dtype)
    for i, j in prod_cells:
        u[j, i], u[j, i - 1] = -1.0, t - 4.0
    got = _check(u, np.zeros_like(u), nx, 1.0 + 2.0 ** -p, 1, m, tb, what="unfused products")
    for i, j in prod_cells:
        assert float(got[j, i]) == 2.0 ** -p + 2.0 ** -(p + 1), (i, j)


@pytest.mark.parametrize("steps", [7, 8, 31, 32])
@pytest.mark.parametrize("m,tb", [(m, 1) for m in PAGE_MAPS + ["tiled", "resident"]] + [("temporal", 4), ("temporal", 12)])
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_page_validation_matrix_31x27(steps, m, tb, dt):
    u, v = inputs.page_impulse_grid(31, 27, DT[dt])
    _check(u, v, 31, 0.1, steps, m, tb, what="31x27")


RAGGED = [  # nx, ny, ld, seed
    (257, 131, 257, 1), (1000, 37, 1000, 2), (3, 3, 3, 3), (3, 40, 3, 4), (40, 3, 40, 5),
    (130, 130, 132, 6), (125, 66, 128, 7), (511, 19, 516, 8), (64, 64, 64, 9), (250, 250, 250, 10),
    (248, 77, 248, 11), (124, 200, 124, 12), (1031, 97, 1040, 13)]


@pytest.mark.parametrize("nx,ny,ld,seed", RAGGED)
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_ragged_grids_every_map(nx, ny, ld, seed, dt):
    """Padding columns hold a NaN sentinel: any read of them would poison the
    result, any write would change them."""
    u, v = inputs.uniform_grid(nx, ny, seed, DT[dt], ld=ld, pad_value=np.nan)
    for steps in (1, 5, 13):
        for m, tb in [(m, 1) for m in PAGE_MAPS + ["tiled"]] + [("temporal", t) for t in (2, 3, 5, 8, 12)]:
            _check(u, v, nx, 0.1, steps, m, tb, what=f"ragged {nx}x{ny} ld={ld}")


@pytest.mark.parametrize("rows", [1, 2, 5, 16, 33])
@pytest.mark.parametrize("tb", [1, 4, 9, 12])
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_explicit_tile_rows(rows, tb, dt):
    u, v = inputs.uniform_grid(300, 90, 21, DT[dt])
    m = "tiled" if tb == 1 else "temporal"
    _check(u, v, 300, 0.1, 17, m, tb, rows, what="tile_rows")


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned_base_pointer(dt, offset):
    """Buffers starting off a 16-byte boundary take the element-wise path."""
    nx, ny = 203, 71
    u0, v0 = inputs.uniform_grid(nx, ny, 31, DT[dt])
    ref, _ = oracle_diffuse(u0, v0, nx, 0.1, 9)
    for m, tb in [("tiled", 1), ("temporal", 3), ("temporal", 8), ("contig", 1)]:
        say("unaligned", dt, offset, m, tb)
        ub = torch.zeros(nx * ny + offset, dtype=torch.float64 if dt == "f64" else torch.float32,
                         device="cuda")
        vb = torch.zeros_like(ub)
        u = ub[offset:].view(ny, nx)
        v = vb[offset:].view(ny, nx)
        u.copy_(dev(u0))
        v.copy_(dev(v0))
        in_v = binding.stencil_diffuse2d(u, v, nx, 0.1, 9, m, tb)
        torch.cuda.synchronize()
        assert_bitwise(host(v if in_v else u), ref, f"unaligned {m}")
        assert host(ub[:offset]).tolist() == [0] * offset


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_dirty_input_edges_are_zeroed(dt):
    nx, ny = 150, 47
    u0, v0 = inputs.uniform_grid(nx, ny, 41, DT[dt])
    u0[0, :] = 5
    u0[:, 0] = -2
    u0[-1, :] = 3
    u0[:, nx - 1] = 7
    u0[:, 59] = 7  # the east edge when the resident map runs the first 60 columns
    v0[:] = 11
    for m, tb in ALL_MAPS:
        n = 60 if m == "resident" else nx  # the resident map takes at most 64 columns
        got = _check(u0, v0, n, 0.1, 6, m, tb, what="dirty edges")
        assert np.all(got[0, :n] == 0) and np.all(got[:, 0] == 0)
        assert np.all(got[-1, :n] == 0) and np.all(got[:, n - 1] == 0)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_zero_steps(dt):
    u0, v0 = inputs.uniform_grid(33, 21, 5, DT[dt])
    u0[0, 3] = 9
    for m, tb in [("tiled", 1), ("temporal", 5), ("collapse_branch", 1)]:
        got, in_v, _, _ = gpu_diffuse(u0, v0, 33, 0.1, 0, m, tb)
        assert not in_v
        ref, _ = oracle_diffuse(u0, v0, 33, 0.1, 0)
        assert_bitwise(got, ref, "zero steps")


@pytest.mark.parametrize("nx,ny,ld", [(3, 3, 3), (5, 7, 8), (31, 27, 31), (64, 64, 64), (64, 128, 64),
                                      (17, 100, 20), (64, 65, 70), (63, 128, 63), (40, 3, 40)])
@pytest.mark.parametrize("steps", [1, 2, 7, 32, 33])
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_resident_small_grids(nx, ny, ld, steps, dt):
    """One workgroup runs every step: the result is the oracle's, and the
    other buffer holds the state one step earlier, as alternating sweeps
    leave it (zero ring included); padding columns are untouched."""
    u0, v0 = inputs.uniform_grid(nx, ny, 70 + nx + ny, DT[dt], ld=ld, pad_value=np.nan)
    got = _check(u0, v0, nx, 0.1, steps, "resident", what=f"resident {nx}x{ny}")
    _, in_v, uh, vh = gpu_diffuse(u0, v0, nx, 0.1, steps, "resident")
    other = uh if in_v else vh
    before, _ = oracle_diffuse(u0, v0, nx, 0.1, steps - 1)
    assert_bitwise(other[:, :nx], before[:, :nx], "resident: previous state")
    assert_bitwise(got[:, :nx], _check(u0, v0, nx, 0.1, steps, "temporal", 8)[:, :nx], "resident vs march")


def test_resident_rejects_large_grids():
    u = torch.zeros(129, 64, dtype=torch.float64, device="cuda")
    v = torch.zeros_like(u)
    with pytest.raises(binding.SGCError):
        binding.stencil_diffuse2d(u, v, 64, 0.1, 4, "resident")
    w = torch.zeros(10, 65, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.SGCError):
        binding.stencil_diffuse2d(w, torch.zeros_like(w), 65, 0.1, 4, "resident")


@pytest.mark.parametrize("alpha", [0.05, 0.25, 0.3, 1.0 / 3.0])
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_other_alphas(alpha, dt):
    u, v = inputs.uniform_grid(97, 83, 51, DT[dt])
    for m, tb in [("collapse_branch", 1), ("tiled", 1), ("temporal", 6), ("temporal", 11)]:
        _check(u, v, 97, alpha, 10, m, tb, what=f"alpha={alpha}")


def test_subnormal_tail_fp32():
    """The impulse's far tail goes subnormal in FP32 after ~38 steps; no
    flush-to-zero on the GPU side either."""
    u, v = inputs.impulse_grid(120, 120, 60, 60, np.float32)
    for m, tb in [("tiled", 1), ("temporal", 8), ("contig", 1)]:
        got = _check(u, v, 120, 0.1, 50, m, tb, what="fp32 subnormals")
    tiny = got[(got > 0) & (got < np.finfo(np.float32).tiny)]
    assert tiny.size > 0


def test_nonblocking_stream_and_determinism():
    u0, v0 = inputs.uniform_grid(700, 301, 61, np.float64)
    s = torch.cuda.Stream()
    outs = []
    for _ in range(2):
        u, v = dev(u0), dev(v0)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            in_v = binding.stencil_diffuse2d(u, v, 700, 0.1, 23, "temporal", 7, 0, s)
        s.synchronize()
        outs.append(host(v if in_v else u))
    ref, _ = oracle_diffuse(u0, v0, 700, 0.1, 23)
    assert_bitwise(outs[0], ref, "stream")
    assert_bitwise(outs[1], outs[0], "determinism")


def test_invalid_arguments_raise_before_launch():
    u = torch.zeros(10, 10, dtype=torch.float64, device="cuda")
    with pytest.raises(binding.SGCError):
        binding.stencil_diffuse2d(u, u, 10, 0.1, 1, "tiled")
    v = torch.zeros(10, 10, dtype=torch.float64, device="cuda")
    with pytest.raises(binding.SGCError):
        binding.stencil_diffuse2d(u, v, 10, 0.1, 1, "temporal", 13)
    with pytest.raises(binding.SGCError):
        binding.stencil_diffuse2d(u, v, 11, 0.1, 1, "tiled")  # ld < nx
    torch.cuda.synchronize()
    assert float(u.abs().sum()) == 0.0 and float(v.abs().sum()) == 0.0
