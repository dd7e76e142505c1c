"""Pins of the CPU oracle's 2D five-point diffusion against what the pages and
the mathematics fix (no GPU needed).

Sources: Qiita "Fortran 2018でGPUを高速化する Part 3", section 3 (update,
alpha = 0.1, fixed-zero edges, alpha <= 1/4), section 5.4 (u/v alternation and
where the result lands), section 8.2 (printed FP32-vs-FP64 comparison),
Appendix A ``diffusion_common`` (impulse position, bound checks).
"""
import json
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import oracle
from structured_grid_cfd_amd import inputs

GOLDEN = Path(__file__).resolve().parent / "golden"
DTYPES = [np.float64, np.float32]


def test_printed_fp32_vs_fp64_example():
    """Section 8.2 prints max abs 3.949045e-9, rel L2 1.138846e-7, mass diff
    1.036993e-7 over 837 cells with 0 failures.  Matching all three to the
    printed 7 digits fixes left-to-right summation without contraction."""
    g = json.loads((GOLDEN / "qiita_p3_fp32_vs_fp64_31x27.json").read_text())
    nx, ny, steps = g["nx"], g["ny"], g["steps"]
    i1, j1 = g["impulse_1based"]
    assert (i1, j1) == ((nx + 1) // 2, (ny + 1) // 2)
    u64, _ = inputs.impulse_grid(nx, ny, i1, j1, np.float64)
    u32, _ = inputs.impulse_grid(nx, ny, i1, j1, np.float32)
    r64 = oracle.diffuse2d_result(u64, nx, g["alpha"], steps)
    r32 = oracle.diffuse2d_result(u32, nx, g["alpha"], steps)
    d = oracle.deviation(r64, r32, g["atol"], g["rtol"])
    for got, key in ((d.largest, "max_abs"), (d.l2_ratio, "relative_l2"),
                     (d.total_shift, "mass_difference")):
        assert f"{got:.6e}" == f"{g[key]:.6e}", (key, got, g[key])
    assert d.n == g["cells"]
    assert d.outside_band == g["failures"]


def test_printed_example_discriminates_summation_order():
    """The printed numbers are not reproduced by the obvious alternative
    (pairwise (W+E)+(S+N)); written here with numpy so the check does not go
    through the oracle's C code."""
    g = json.loads((GOLDEN / "qiita_p3_fp32_vs_fp64_31x27.json").read_text())

    def pairwise(dtype):
        u, v = inputs.page_impulse_grid(g["nx"], g["ny"], dtype)
        a, four = dtype(g["alpha"]), dtype(4)
        for _ in range(g["steps"]):
            c = u[1:-1, 1:-1]
            t = (u[1:-1, :-2] + u[1:-1, 2:]) + (u[:-2, 1:-1] + u[2:, 1:-1])
            v[1:-1, 1:-1] = c + a * (t - four * c)
            u, v = v, u
        return u

    d = oracle.deviation(pairwise(np.float64), pairwise(np.float32), 1e-6, 1e-4)
    assert f"{d.largest:.6e}" != f"{g['max_abs']:.6e}"


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_step_from_unit_impulse(dtype):
    """One step of the section 3 update from a unit cell: centre 1 - 4*alpha
    = 0.6, each of the four neighbours alpha = 0.1, everything else 0."""
    u, v = inputs.impulse_grid(9, 7, 5, 4, dtype)
    in_v = oracle.diffuse2d(u, v, 9, 0.1, 1)
    assert in_v
    r = v
    assert r[3, 4] == dtype(0.6)
    for (j, i) in [(3, 3), (3, 5), (2, 4), (4, 4)]:
        assert r[j, i] == dtype(0.1)
    mask = np.ones_like(r, dtype=bool)
    mask[3, 4] = False
    for (j, i) in [(3, 3), (3, 5), (2, 4), (4, 4)]:
        mask[j, i] = False
    assert np.all(r[mask] == 0)


def test_two_steps_closed_form():
    """Two steps = the kernel K = 0.6 + 0.1(x + 1/x + y + 1/y) squared:
    centre 0.40, distance-1 cells 0.12, (+-2,0)/(0,+-2) cells 0.01, diagonal
    cells 0.02.  FP64 results within 2 ulp of these."""
    u, v = inputs.impulse_grid(11, 11, 6, 6, np.float64)
    r = oracle.diffuse2d_result(u, 11, 0.1, 2)
    c = (5, 5)
    expect = {(0, 0): 0.40, (1, 0): 0.12, (-1, 0): 0.12, (0, 1): 0.12, (0, -1): 0.12,
              (2, 0): 0.01, (-2, 0): 0.01, (0, 2): 0.01, (0, -2): 0.01,
              (1, 1): 0.02, (1, -1): 0.02, (-1, 1): 0.02, (-1, -1): 0.02}
    seen = np.zeros_like(r, dtype=bool)
    for (dj, di), val in expect.items():
        got = r[c[0] + dj, c[1] + di]
        assert abs(got - val) <= 2 * np.spacing(val), (dj, di, got, val)
        seen[c[0] + dj, c[1] + di] = True
    assert np.all(r[~seen] == 0)
    assert abs(r.sum() - 1.0) < 1e-15


@pytest.mark.parametrize("steps", [7, 8, 31, 32])
@pytest.mark.parametrize("dtype", DTYPES)
def test_result_buffer_follows_step_parity(steps, dtype):
    """Section 5.4: odd steps u -> v, even steps v -> u; the final value is in
    v after an odd number of steps and in u after an even number.  The other
    buffer holds the previous step, so one more step from it reproduces the
    result."""
    u, v = inputs.page_impulse_grid(31, 27, dtype)
    in_v = oracle.diffuse2d(u, v, 31, 0.1, steps)
    assert in_v == (steps % 2 == 1)
    res, prev = (v, u) if in_v else (u, v)
    again = oracle.diffuse2d_result(prev, 31, 0.1, 1)
    assert np.array_equal(again, res)


def test_mirror_symmetry():
    """Four-fold symmetry of an impulse before the front reaches an edge: the
    mirror in i is bitwise exact (W+E = E+W); the mirror in j and the
    transpose hold to rounding."""
    n, steps = 41, 19
    u, _ = inputs.impulse_grid(n, n, 21, 21, np.float64)
    r = oracle.diffuse2d_result(u, n, 0.1, steps)
    assert np.array_equal(r, r[:, ::-1])
    assert np.max(np.abs(r - r[::-1, :])) < 1e-16
    assert np.max(np.abs(r - r.T)) < 1e-16
    assert r[20, 20] == r.max()


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_order_closed_form(dtype):
    """One step on values chosen so that the order of the four additions
    shows in the last bit.  With h half an ulp of 1, W = 1, S = h (row
    j - 1), N = -h (row j + 1), C = 0 and alpha = 1, the page's expression
    read left to right gives ((1 + 0) + h) + (-h): 1 + h is a tie and rounds
    to the even 1, then 1 - h is exact, so v = 1 - h.  Adding N before S, or
    (W + E) + (S + N), or the vertical pair first all give exactly 1."""
    h = float(np.finfo(dtype).eps) / 2
    u = np.zeros((5, 5), dtype=dtype)
    u[2, 1] = 1.0    # W of cell (i, j) = (2, 2)
    u[1, 2] = h      # S
    u[3, 2] = -h     # N
    r = oracle.diffuse2d_result(u, 5, 1.0, 1)
    assert r[2, 2] == dtype(1.0 - h)


@pytest.mark.parametrize("dtype,p", [(np.float64, 30), (np.float32, 12)])
def test_update_rounds_product_then_sum(dtype, p):
    """c + alpha * t rounds the product before the sum (no fused multiply-
    add).  With alpha = 1 + 2^-p, t = 1 + 2^-(p+1) and c = -1, the exact
    product is 1 + 2^-p + 2^-(p+1) + 2^-(2p+1); its last term is below half
    an ulp of 1, so the rounded product drops it and v = 2^-p + 2^-(p+1)
    exactly, where a fused form would keep 2^-(2p+1).  t comes from
    W = t - 4 (representable) at the cell (2, 1) of a 4 x 3 grid whose other
    neighbours are edge cells."""
    t = 1.0 + 2.0 ** -(p + 1)
    u = np.zeros((3, 4), dtype=dtype)
    u[1, 2] = -1.0      # C
    u[1, 1] = t - 4.0   # W
    assert float(u[1, 1]) == t - 4.0
    r = oracle.diffuse2d_result(u, 4, 1.0 + 2.0 ** -p, 1)
    assert float(r[1, 2]) == 2.0 ** -p + 2.0 ** -(p + 1)


@pytest.mark.parametrize("dtype", DTYPES)
def test_maximum_principle_random(dtype):
    """With alpha <= 1/4 each update is a convex combination of
    non-negative values, so 0 <= result <= max(initial) (Appendix A's bound
    checks are the tolerant form of this)."""
    u, _ = inputs.uniform_grid(67, 45, seed=7, dtype=dtype)
    top = u.max()
    r = oracle.diffuse2d_result(u, 67, 0.1, 25)
    assert r.min() >= 0 and r.max() <= top
    assert np.all(np.isfinite(r))


def test_mass_balance_identity():
    """Summing the update over interior cells telescopes: the total changes
    only through flux into the fixed-zero edges,
    M(t+1) = M(t) - alpha * sum_c b(c) u_c(t), b(c) = number of edge
    neighbours of interior cell c."""
    nx, ny = 40, 33
    u, _ = inputs.uniform_grid(nx, ny, seed=11, dtype=np.float64)
    b = np.zeros((ny, nx))
    b[1, 1:-1] += 1
    b[-2, 1:-1] += 1
    b[1:-1, 1] += 1
    b[1:-1, -2] += 1
    m0 = u.sum()
    r = oracle.diffuse2d_result(u, nx, 0.1, 1)
    predicted = m0 - 0.1 * (b * u).sum()
    assert abs(r.sum() - predicted) < 1e-12 * m0


def test_impulse_mass_conserved_until_edges():
    """For the 64x64 impulse workload the total stays 1 while the front has
    not reached the cells next to the edges (the leak after that is far
    below FP64 resolution for 32 steps)."""
    cfg = inputs.impulse_64()
    import math
    for steps in (10, 30, 32):
        r = oracle.diffuse2d_result(cfg["u"], 64, 0.1, steps)
        assert abs(math.fsum(r.ravel().tolist()) - 1.0) < 1e-14


def _exact_steps(u0, nx, ny, alpha, steps):
    """Exact rational arithmetic of the section 3 update (zero edges)."""
    a = Fraction(alpha)
    cur = [[Fraction(float(u0[j, i])) if 0 < i < nx - 1 and 0 < j < ny - 1 else Fraction(0)
            for i in range(nx)] for j in range(ny)]
    for _ in range(steps):
        nxt = [[Fraction(0)] * nx for _ in range(ny)]
        for j in range(1, ny - 1):
            for i in range(1, nx - 1):
                c = cur[j][i]
                lap = cur[j][i - 1] + cur[j][i + 1] + cur[j - 1][i] + cur[j + 1][i] - 4 * c
                nxt[j][i] = c + a * lap
        cur = nxt
    return cur


@pytest.mark.parametrize("nx,ny,steps", [(5, 5, 3), (8, 7, 6), (6, 9, 5), (3, 4, 2)])
@pytest.mark.parametrize("dtype", DTYPES)
def test_bruteforce_exact_rational(nx, ny, steps, dtype):
    """Tiny grids against exact rationals (alpha = the working-precision value
    of 0.1): every cell within a few rounding units of the exact value."""
    u, _ = inputs.uniform_grid(nx, ny, seed=nx * 100 + ny, dtype=dtype)
    alpha_w = float(dtype(0.1))
    exact = _exact_steps(u, nx, ny, alpha_w, steps)
    r = oracle.diffuse2d_result(u, nx, 0.1, steps)
    eps = float(np.finfo(dtype).eps)
    bound = 6 * steps * eps * max(1.0, float(u.max()))
    for j in range(ny):
        for i in range(nx):
            assert abs(float(r[j, i]) - float(exact[j][i])) <= bound, (i, j)


def test_leading_dimension_padding_untouched():
    """With ld > nx the padding columns are never read or written, and the
    logical result equals the unpadded one bitwise."""
    nx, ny, ld = 13, 9, 16
    u, v = inputs.uniform_grid(nx, ny, seed=3, dtype=np.float64, ld=ld, pad_value=np.nan)
    up, _ = inputs.uniform_grid(nx, ny, seed=3, dtype=np.float64)
    in_v = oracle.diffuse2d(u, v, nx, 0.1, 5)
    ref = oracle.diffuse2d_result(up, nx, 0.1, 5)
    res = v if in_v else u
    assert np.array_equal(res[:, :nx], ref)
    assert np.all(np.isnan(u[:, nx:])) and np.all(np.isnan(v[:, nx:]))


def test_nonzero_input_edges_are_zeroed():
    """Edges are fixed at 0 in both buffers; values a caller leaves in the
    input edge ring do not enter the update."""
    nx, ny = 10, 8
    u, _ = inputs.uniform_grid(nx, ny, seed=5, dtype=np.float64)
    dirty = u.copy()
    dirty[0, :] = 7.0
    dirty[:, 0] = -3.0
    dirty[-1, :] = 2.0
    dirty[:, nx - 1] = 9.0
    a = oracle.diffuse2d_result(u, nx, 0.1, 3)
    b = oracle.diffuse2d_result(dirty, nx, 0.1, 3)
    assert np.array_equal(a, b)


def test_zero_steps_is_identity_with_zero_edges():
    u, _ = inputs.uniform_grid(9, 9, seed=1, dtype=np.float32)
    r = oracle.diffuse2d_result(u, 9, 0.1, 0)
    assert np.array_equal(r, u)


@pytest.mark.parametrize("dtype", DTYPES)
def test_sub_grid_helpers_equal_the_whole_grid(dtype):
    """The cell window and the row band that the full-size GPU tests use to
    reach single cells and whole bands of large grids return exactly the
    whole-grid oracle's bits: a cut edge lies farther than the step count from
    every kept cell.  Bands that touch the grid's first or last row, bands in
    the middle, and windows at corners, edges and the interior."""
    nx, ny, steps = 37, 61, 9
    u0, _ = inputs.uniform_grid(nx, ny, 4242, dtype, ld=40)
    whole = oracle.diffuse2d_result(u0, nx, 0.1, steps)
    as_bits = lambda a: np.ascontiguousarray(a).view(np.uint64 if dtype == np.float64 else np.uint32)  # noqa: E731
    edges = list(range(0, ny, 7)) + [ny]
    for j0, j1 in zip(edges[:-1], edges[1:]):
        got = oracle.diffuse2d_rows(u0, nx, 0.1, steps, j0, j1)
        assert np.array_equal(as_bits(got[:, :nx]), as_bits(whole[j0:j1, :nx])), (j0, j1)
    for i, j in [(1, 1), (nx - 2, ny - 2), (1, ny // 2), (nx // 2, 1), (18, 30), (nx - 2, 11)]:
        got = oracle.diffuse2d_window(u0, nx, 0.1, steps, i, j)
        assert as_bits(np.asarray(got)) == as_bits(whole[j, i]), (i, j)
