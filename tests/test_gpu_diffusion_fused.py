"""GPU parity of the marching sweep's fused form, which every tile takes: it
computes t - 4c through one fused multiply-add (the same rounding while 4c is
finite), holds the boundary columns at 0 through a zero coefficient and the
boundary rows through skipped levels, and falls back to the separate form
with per-cell masks when a tile's inputs are large enough for 4c to
overflow, or hold NaN or infinity.

Grids are large enough for many tiles away from every edge; magnitudes cover
the ordinary range, values near the largest the fused form accepts, the
subnormal range, and cells that force the fallback, in an interior tile and
in tiles on each edge and corner.  Every result is compared
with the oracle bit for bit (NaN positions only, where inf - inf occurs).
"""
import numpy as np
import pytest

from gpu_helpers import (assert_bitwise, assert_bitwise_nan, gpu_diffuse, oracle_diffuse,
                         require_gpu, say)
from structured_grid_cfd_amd import inputs

pytestmark = pytest.mark.gpu

DT = {"f64": np.float64, "f32": np.float32}
NX, NY = 650, 520


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _signed(dt, seed, scale_exp):
    """Interior uniform [-1, 1) times 2**scale_exp (an exact scaling)."""
    u, v = inputs.uniform_grid(NX, NY, seed, DT[dt])
    w = u.copy()
    w[1:-1, 1:NX - 1] = np.ldexp(u[1:-1, 1:NX - 1] * 2 - 1, scale_exp).astype(DT[dt])
    return w, v


def _run(u, v, steps, tb, rows, what, nan_ok=False):
    say(what, u.dtype, tb, rows, steps)
    got, in_v, _, _ = gpu_diffuse(u, v, NX, 0.1, steps, "temporal", tb, rows)
    ref, ref_in_v = oracle_diffuse(u, v, NX, 0.1, steps)
    assert in_v == ref_in_v
    (assert_bitwise_nan if nan_ok else assert_bitwise)(got[:, :NX], ref[:, :NX], what)
    return ref


@pytest.mark.parametrize("rows", [0, 16])
@pytest.mark.parametrize("tb", [2, 5, 8, 10, 12])
@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_interior_tiles(dt, tb, rows):
    u, v = inputs.uniform_grid(NX, NY, 71, DT[dt])
    _run(u, v, 2 * tb + 3, tb, rows, "interior")


@pytest.mark.parametrize("dt,exp", [("f64", 1000), ("f64", -1000), ("f64", -1070),
                                    ("f32", 105), ("f32", -120), ("f32", -140)])
def test_extreme_magnitudes(dt, exp):
    """Signed values scaled to 2**exp: close to the largest inputs the fused
    form takes at depth 8 (2**1000 in FP64 and 2**105 in FP32 pass the check),
    and deep into the subnormal range, where 4c must still be exact."""
    u, v = _signed(dt, 72, exp)
    _run(u, v, 16, 8, 16, f"2^{exp}")


PLACES = {"interior": (NY // 2, NX // 2), "left": (NY // 2, 1), "right": (NY // 2, NX - 2),
          "bottom": (1, NX // 3), "top": (NY - 2, NX // 3), "corner": (NY - 2, 1)}


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["overflow", "nan", "inf"])
@pytest.mark.parametrize("place", list(PLACES))
def test_fallback_cells(dt, kind, place):
    """A cell whose 4c overflows (centre 2**(emax-1), interior neighbours half
    that: the separate form gives -inf where the fused one stays finite), a
    NaN, or an infinity, placed in an interior tile or in a tile on an edge
    or corner: the tile must be recomputed in the separate form."""
    u, v = inputs.uniform_grid(NX, NY, 73, DT[dt])
    j, i = PLACES[place]
    big = np.ldexp(1.0, 1022 if dt == "f64" else 126)
    if kind == "overflow":
        u[j, i] = big
        for jj, ii in ((j, i - 1), (j, i + 1), (j - 1, i), (j + 1, i)):
            if 1 <= jj <= NY - 2 and 1 <= ii <= NX - 2:
                u[jj, ii] = big / 2
    elif kind == "nan":
        u[j, i] = np.nan
    else:
        u[j, i] = -np.inf
    for tb, rows in [(8, 16), (5, 0), (12, 24)]:
        ref = _run(u, v, 2 * tb, tb, rows, f"fallback {kind} {place}", nan_ok=True)
        assert not np.isfinite(ref).all()


# ---------------------------------------------------------------------------
# The resident map's fast form (fused t - 4c, zero coefficient on cells it
# never updates) and its separate form, chosen once per workgroup from the
# largest input magnitude, the step count and alpha.
# ---------------------------------------------------------------------------

def _resident(u, v, nx, alpha, steps, what):
    say("resident", what, u.dtype, u.shape, alpha, steps)
    got, in_v, uh, vh = gpu_diffuse(u, v, nx, alpha, steps, "resident")
    ref, ref_in_v = oracle_diffuse(u, v, nx, alpha, steps)
    assert in_v == ref_in_v
    assert_bitwise_nan(got[:, :nx], ref[:, :nx], what)
    before, _ = oracle_diffuse(u, v, nx, alpha, steps - 1)
    assert_bitwise_nan((uh if in_v else vh)[:, :nx], before[:, :nx], what + " (previous state)")
    return ref


def _signed_small(dt, nx, ny, seed, scale_exp):
    u, v = inputs.uniform_grid(nx, ny, seed, DT[dt])
    w = u.copy()
    w[1:-1, 1:nx - 1] = np.ldexp(u[1:-1, 1:nx - 1] * 2 - 1, scale_exp).astype(DT[dt])
    return w, v


@pytest.mark.parametrize("nx,ny", [(60, 60), (64, 100)])
@pytest.mark.parametrize("dt,exp,alpha,steps", [
    ("f64", 1000, 0.1, 33),     # fast: the bound for alpha <= 1/4 barely grows
    ("f64", 1018, 0.1, 33),     # fast, just below 2^1019
    ("f64", 1000, 1.0, 10),     # separate: growth 7 per step leaves a limit near 2^991
    ("f64", 980, 1.0, 10),      # fast again
    ("f64", -1070, 0.3, 7),     # subnormal, fast
    ("f32", 120, 0.1, 200),     # fast
    ("f32", 124, 0.1, 5),       # separate (above 2^123)
    ("f32", -140, 0.1, 9),      # subnormal, fast
    ("f32", 100, -0.1, 40),     # negative alpha, growth 1.8: separate
])
def test_resident_magnitudes(nx, ny, dt, exp, alpha, steps):
    u, v = _signed_small(dt, nx, ny, 74 + nx, exp)
    _resident(u, v, nx, alpha, steps, f"2^{exp} alpha {alpha}")


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("kind", ["overflow", "nan", "inf"])
@pytest.mark.parametrize("place", [(30, 30), (1, 1), (58, 62), (1, 40)])
def test_resident_separate_form_cells(dt, kind, place):
    """A cell whose 4c overflows, a NaN or an infinity anywhere in the grid
    (interior, next to a corner or an edge): the workgroup takes the
    separate form, and edge cells stay 0 next to NaN and infinite values."""
    nx, ny = 64, 60
    u, v = inputs.uniform_grid(nx, ny, 75, DT[dt])
    j, i = place
    big = np.ldexp(1.0, 1022 if dt == "f64" else 126)
    if kind == "overflow":
        u[j, i] = big
        for jj, ii in ((j, i - 1), (j, i + 1), (j - 1, i), (j + 1, i)):
            if 1 <= jj <= ny - 2 and 1 <= ii <= nx - 2:
                u[jj, ii] = big / 2
    elif kind == "nan":
        u[j, i] = np.nan
    else:
        u[j, i] = -np.inf
    ref = _resident(u, v, nx, 0.1, 6, f"separate {kind} {place}")
    assert not np.isfinite(ref).all()
    assert (ref[0, :] == 0).all() and (ref[:, 0] == 0).all() and (ref[:, nx - 1] == 0).all()
