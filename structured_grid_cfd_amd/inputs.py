"""Seeded synthetic inputs for the stencil sweeps.

This module only draws and lays out input arrays; it holds none of the
methods' arithmetic, so both the HIP path's tests/benchmark and the CPU oracle
can consume the very same host arrays.

Generator: ``numpy.random.Generator(PCG64(seed))``, one stream per array
family, values drawn in storage order (first Fortran index fastest, variable
slowest).  Uniform [0, 1) values are drawn directly in the working precision;
normal values are float64 standard normals.

Workloads (grid shapes follow the examples named in MFC pull request 2087,
"Performance" table, and the diffusion setup of Qiita "Fortran 2018でGPUを
高速化する Part 3", section 3 and Appendix A ``diffusion_common``):

* ``impulse_64`` 64x64 FP64, impulse 1 at (33, 33) 1-based, 32 steps.
* ``uniform_4096`` 4096x4096 FP64/FP32, interior uniform [0,1), 1000 steps.
* ``fields_201cubed`` 8 fields of 201^3 FP64, normal(0,1), pack along x/y/z.
* ``faces_201x101x101`` 7 fields on 201x101x101, faces normal(0,1), spacings
  U[0.5,1.5)/n.
* ``faces_4800x1200`` / ``fields_4800x1200`` 6 fields on 4800x1200 (2D flux
  difference + x/y packs).
* ``uniform_16384_f32`` 16384x16384 FP32 diffusion for 200 steps.

Seeds: 1002 (4096^2), 1003 (201^3 fields), 1004 (201x101x101 faces), 1005
and 1050 (4800x1200 faces and fields), 1006 (16384^2); the impulse draws none.

Array conventions match ``oracle`` and the binding: a 2D grid u(nx, ny) with
leading dimension ld is a ``(ny, ld)`` array; a field f(j,k,l) is
``(nz, ny, nx)``; faces Fx/Fy/Fz are ``(nz, ny, nx+1)``, ``(nz, ny+1, nx)``,
``(nz+1, ny, nx)``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 1000


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# 2D diffusion grids
# ---------------------------------------------------------------------------

def impulse_grid(nx: int, ny: int, i1: int, j1: int, dtype=np.float64, ld: int | None = None):
    """Zero grid with a unit value at 1-based cell (i1, j1); returns (u, v)."""
    ld = nx if ld is None else ld
    u = np.zeros((ny, ld), dtype=dtype)
    v = np.zeros((ny, ld), dtype=dtype)
    u[j1 - 1, i1 - 1] = 1
    return u, v


def page_impulse_grid(nx: int, ny: int, dtype=np.float64):
    """The pages' default start: unit value at ((nx+1)/2, (ny+1)/2), integer
    division, 1-based (Qiita Part 3, Appendix A, ``set_initial_condition``)."""
    return impulse_grid(nx, ny, (nx + 1) // 2, (ny + 1) // 2, dtype)


def uniform_grid(nx: int, ny: int, seed: int, dtype=np.float64, ld: int | None = None,
                 pad_value: float = 0.0):
    """Edges 0, interior (nx-2)(ny-2) values uniform [0,1) in storage order.

    Padding columns [nx, ld) are filled with ``pad_value`` (tests use a NaN
    sentinel to prove no kernel touches them).  Returns (u, v) with v = 0 in
    the logical region and ``pad_value`` in the padding.
    """
    ld = nx if ld is None else ld
    g = rng(seed)
    inner = g.random((ny - 2) * (nx - 2), dtype=dtype).reshape(ny - 2, nx - 2)
    u = np.full((ny, ld), pad_value, dtype=dtype)
    u[:, :nx] = 0
    u[1:-1, 1:nx - 1] = inner
    v = np.full((ny, ld), pad_value, dtype=dtype)
    v[:, :nx] = 0
    return u, v


def _hash_unit(n: int, mult: int, salt: int) -> np.ndarray:
    """n values k/2^24 in [0, 1) from a multiplicative hash of 0..n-1."""
    idx = np.arange(n, dtype=np.uint64) + np.uint64(salt)
    return ((idx * np.uint64(mult)) >> np.uint64(40)).astype(np.float64) / float(1 << 24)


def hashed_parts(nx: int, ny: int, dtype=np.float64, salt: int = 0):
    """Column and row terms (a, b) of ``hashed_grid``: a and b hash the
    column and row indices with different multipliers, rounded to dtype."""
    a = _hash_unit(nx, 0x9E3779B97F4A7C15, salt).astype(dtype)
    b = _hash_unit(ny, 0xC2B2AE3D27D4EB4F, salt).astype(dtype)
    return a, b


def hashed_window(a: np.ndarray, b: np.ndarray, i0: int, i1: int, j0: int, j1: int) -> np.ndarray:
    """Rows [j0, j1) and columns [i0, i1) of the grid with interior value
    (a_i + b_j) / 2 (each operation rounded in the dtype of a and b) and
    edges 0.  The whole grid is the window over every row and column, for
    sizes of about 2^31 cells that the random generator would take minutes
    to fill; a device copy of the same grid comes from the same two
    operations on a and b."""
    nx, ny = a.size, b.size
    w = np.add(b[j0:j1, None], a[None, i0:i1])
    w *= a.dtype.type(0.5)
    if j0 == 0:
        w[0, :] = 0
    if j1 == ny:
        w[-1, :] = 0
    if i0 == 0:
        w[:, 0] = 0
    if i1 == nx:
        w[:, -1] = 0
    return w


# ---------------------------------------------------------------------------
# 3D per-variable fields and face fluxes
# ---------------------------------------------------------------------------

def normal_fields(nvar: int, nx: int, ny: int, nz: int, seed: int) -> np.ndarray:
    """nvar SoA fields, normal(0,1), shape (nvar, nz, ny, nx)."""
    return rng(seed).standard_normal((nvar, nz, ny, nx), dtype=np.float64)


def distinct_fields(nvar: int, nx: int, ny: int, nz: int) -> np.ndarray:
    """f_var[idx] = idx + N*var: every element distinct (a permutation probe)."""
    n = nx * ny * nz
    return np.arange(nvar * n, dtype=np.float64).reshape(nvar, nz, ny, nx)


@dataclass
class FluxInputs:
    fx: np.ndarray            # (nvar, nz, ny, nx+1)
    fy: np.ndarray            # (nvar, nz, ny+1, nx)
    fz: np.ndarray | None     # (nvar, nz+1, ny, nx) or None (2D)
    dx: np.ndarray            # (nx,)
    dy: np.ndarray            # (ny,)
    dz: np.ndarray | None     # (nz,) or None (2D)

    @property
    def shape(self):
        nvar, nz, ny, nxp1 = self.fx.shape
        return nvar, nxp1 - 1, ny, nz


def normal_faces(nvar: int, nx: int, ny: int, nz: int, seed: int, two_d: bool = False) -> FluxInputs:
    """Face fluxes normal(0,1) per variable; widths d = U[0.5, 1.5)/n per axis.

    Draw order: Fx for all variables, then Fy, then Fz, then dx, dy, dz.
    """
    g = rng(seed)
    fx = g.standard_normal((nvar, nz, ny, nx + 1), dtype=np.float64)
    fy = g.standard_normal((nvar, nz, ny + 1, nx), dtype=np.float64)
    fz = None if two_d else g.standard_normal((nvar, nz + 1, ny, nx), dtype=np.float64)
    dx = g.uniform(0.5, 1.5, nx) / nx
    dy = g.uniform(0.5, 1.5, ny) / ny
    dz = None if two_d else g.uniform(0.5, 1.5, nz) / nz
    return FluxInputs(fx, fy, fz, dx, dy, dz)


# ---------------------------------------------------------------------------
# The workloads
# ---------------------------------------------------------------------------

UNIFORM_4096_N, UNIFORM_4096_STEPS = 4096, 1000
FIELDS_201_NVAR, FIELDS_201_N = 8, 201
FACES_201_NVAR, FACES_201_SHAPE = 7, (201, 101, 101)
PLANE_4800_NVAR, PLANE_4800_SHAPE = 6, (4800, 1200)
UNIFORM_16384_N, UNIFORM_16384_STEPS = 16384, 200
ALPHA = 0.1


def impulse_64(dtype=np.float64):
    """64x64, impulse at (33,33) 1-based, alpha 0.1, 32 steps."""
    u, v = impulse_grid(64, 64, 33, 33, dtype)
    return dict(u=u, v=v, nx=64, ny=64, alpha=ALPHA, steps=32)


def uniform_4096(dtype=np.float64, steps: int = UNIFORM_4096_STEPS):
    u, v = uniform_grid(UNIFORM_4096_N, UNIFORM_4096_N, SEED_BASE + 2, dtype)
    return dict(u=u, v=v, nx=UNIFORM_4096_N, ny=UNIFORM_4096_N, alpha=ALPHA, steps=steps)


def fields_201cubed():
    return normal_fields(FIELDS_201_NVAR, FIELDS_201_N, FIELDS_201_N, FIELDS_201_N, SEED_BASE + 3)


def faces_201x101x101():
    nx, ny, nz = FACES_201_SHAPE
    return normal_faces(FACES_201_NVAR, nx, ny, nz, SEED_BASE + 4)


def faces_4800x1200():
    nx, ny = PLANE_4800_SHAPE
    return normal_faces(PLANE_4800_NVAR, nx, ny, 1, SEED_BASE + 5, two_d=True)


def fields_4800x1200():
    nx, ny = PLANE_4800_SHAPE
    # A second stream of the same workload's seed family, kept apart from the faces.
    return normal_fields(PLANE_4800_NVAR, nx, ny, 1, SEED_BASE + 50)


def uniform_16384_f32(steps: int = UNIFORM_16384_STEPS):
    u, v = uniform_grid(UNIFORM_16384_N, UNIFORM_16384_N, SEED_BASE + 6, np.float32)
    return dict(u=u, v=v, nx=UNIFORM_16384_N, ny=UNIFORM_16384_N, alpha=ALPHA, steps=steps)
