"""CPU oracle for the structured-grid stencil sweeps -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and never falls back to it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C built with
``-O2 -ffp-contract=off``); this module only builds it with gcc and marshals
numpy arrays.  It shares no code with the HIP library.

Array conventions (all numpy, C-contiguous):

* 2D grid ``u(nx, ny)`` column-major with leading dimension ``ld``: a numpy
  array of shape ``(ny, ld)``; logical columns are ``[:, :nx]``.
* field ``f_var(j, k, l)``: numpy shape ``(nz, ny, nx)``; nvar fields stacked
  as ``(nvar, nz, ny, nx)``.
* packed output: x -> ``(nvar, nz, ny, nx)``, y -> ``(nvar, nz, nx, ny)``,
  z -> ``(nvar, nx, ny, nz)`` (first Fortran index last in numpy).
* faces per variable: Fx ``(nz, ny, nx+1)``, Fy ``(nz, ny+1, nx)``,
  Fz ``(nz+1, ny, nx)``; rhs ``(nvar, nz, ny, nx)``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import time
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB = _HERE / "liboracle.so"

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
             "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = False) -> Path:
    """Compile oracle.c into liboracle.so with gcc (contraction off)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        subprocess.run(["gcc", *GCC_FLAGS, str(_SRC), "-o", str(tmp)], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(str(build()))
        i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
        for name in ("oracle_diffuse2d_f64", "oracle_diffuse2d_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, vp, i64, i64, i64, dbl, i64]
            fn.restype = ctypes.c_int
        lib.oracle_field_pack.argtypes = [vp, i32, i64, i64, i64, i32, vp]
        lib.oracle_field_pack.restype = ctypes.c_int
        lib.oracle_field_unpack.argtypes = [vp, i32, i64, i64, i64, i32, vp]
        lib.oracle_field_unpack.restype = ctypes.c_int
        lib.oracle_flux_diff.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
        lib.oracle_flux_stage.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, i32,
                                          i64, i64, i64, vp]
        lib.oracle_flux_stage.restype = ctypes.c_int
        lib.oracle_flux_diff.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _ptr_table(arrs) -> ctypes.Array:
    tab = (ctypes.c_void_p * len(arrs))()
    for n, a in enumerate(arrs):
        tab[n] = _ptr(a)
    return tab


# ---------------------------------------------------------------------------
# 2D five-point diffusion
# ---------------------------------------------------------------------------

def diffuse2d(u: np.ndarray, v: np.ndarray, nx: int, alpha: float, steps: int) -> bool:
    """Advance ``steps`` five-point sweeps in place on the ping-pong pair.

    ``u`` and ``v`` are ``(ny, ld)`` float32 or float64 arrays.  Both edge
    rings are zeroed first.  Returns True if the result is in ``v`` (odd step
    count), False if it is in ``u``.
    """
    assert u.shape == v.shape and u.dtype == v.dtype and u.ndim == 2
    ny, ld = u.shape
    assert 3 <= nx <= ld and ny >= 3 and steps >= 0
    lib = _load()
    fn = lib.oracle_diffuse2d_f64 if u.dtype == np.float64 else lib.oracle_diffuse2d_f32
    assert u.dtype in (np.float64, np.float32)
    return bool(fn(_ptr(u), _ptr(v), nx, ny, ld, float(alpha), int(steps)))


def diffuse2d_result(u0: np.ndarray, nx: int, alpha: float, steps: int) -> np.ndarray:
    """Copying convenience: run from ``u0`` with ``v`` = 0, return the result grid."""
    u = np.array(u0, copy=True, order="C")
    v = np.zeros_like(u)
    return v if diffuse2d(u, v, nx, alpha, steps) else u


def diffuse2d_window(u0: np.ndarray, nx: int, alpha: float, steps: int,
                     i: int, j: int) -> float:
    """Value of cell (i, j) of the full-grid result, computed on a sub-grid.

    After ``steps`` sweeps a cell depends only on cells within Manhattan
    distance ``steps``.  The sub-grid keeps every such cell; where it is cut
    inside the grid the cut ring lies more than ``steps`` away from (i, j), so
    the artificial zero edge the oracle puts there cannot reach it.
    """
    ny = u0.shape[0]
    r = steps + 1
    i0, i1 = max(0, i - r), min(nx, i + r + 1)
    j0, j1 = max(0, j - r), min(ny, j + r + 1)
    sub = np.ascontiguousarray(u0[j0:j1, i0:i1])
    # Grid edges that survive in the window are real edges; cut sides become
    # window edges that the oracle zeroes, which is harmless (see above).
    res = diffuse2d_result(sub, i1 - i0, alpha, steps)
    return res[j - j0, i - i0]


def diffuse2d_rows(u0: np.ndarray, nx: int, alpha: float, steps: int, j0: int, j1: int) -> np.ndarray:
    """Rows ``[j0, j1)`` of the full-grid result, computed on a band of rows.

    The same domain-of-dependence argument as :func:`diffuse2d_window`: the
    band keeps every row within ``steps`` of the requested ones, and a cut
    edge of the band lies more than ``steps`` rows away from them, so its
    artificial zero never reaches them.  Columns are not cut.  The returned
    array is ``(j1 - j0, ld)``.
    """
    ny = u0.shape[0]
    assert 0 <= j0 < j1 <= ny
    r = steps + 1
    b0, b1 = max(0, j0 - r), min(ny, j1 + r)
    band = np.ascontiguousarray(u0[b0:b1])
    res = diffuse2d_result(band, nx, alpha, steps)
    return res[j0 - b0:j1 - b0]


# ---------------------------------------------------------------------------
# Directional pack / unpack
# ---------------------------------------------------------------------------

PACK_SHAPE = {0: lambda nx, ny, nz: (nz, ny, nx),
              1: lambda nx, ny, nz: (nz, nx, ny),
              2: lambda nx, ny, nz: (nx, ny, nz)}


def field_pack(fields: np.ndarray, direction: int) -> np.ndarray:
    """Pack ``fields`` of shape (nvar, nz, ny, nx) along x (0), y (1) or z (2)."""
    assert fields.dtype == np.float64 and fields.ndim == 4
    nvar, nz, ny, nx = fields.shape
    fl = [np.ascontiguousarray(fields[v]) for v in range(nvar)]
    out = np.empty((nvar,) + PACK_SHAPE[direction](nx, ny, nz), dtype=np.float64)
    rc = _load().oracle_field_pack(_ptr_table(fl), nvar, nx, ny, nz, direction, _ptr(out))
    assert rc == 0
    return out


def field_unpack(packed: np.ndarray, nx: int, ny: int, nz: int, direction: int) -> np.ndarray:
    """Inverse of :func:`field_pack`; returns (nvar, nz, ny, nx)."""
    nvar = packed.shape[0]
    out = np.empty((nvar, nz, ny, nx), dtype=np.float64)
    fl = [out[v] for v in range(nvar)]
    rc = _load().oracle_field_unpack(_ptr(np.ascontiguousarray(packed)), nvar, nx, ny, nz,
                                     direction, _ptr_table(fl))
    assert rc == 0
    return out


# ---------------------------------------------------------------------------
# Conservative flux difference
# ---------------------------------------------------------------------------

def flux_diff(fx, fy, fz, dx, dy, dz) -> np.ndarray:
    """rhs (nvar, nz, ny, nx) from per-variable face arrays.

    ``fx`` (nvar, nz, ny, nx+1), ``fy`` (nvar, nz, ny+1, nx), ``fz``
    (nvar, nz+1, ny, nx) or None for the 2D form (then nz must be 1).
    """
    nvar, nz, ny, nxp1 = fx.shape
    nx = nxp1 - 1
    assert fy.shape == (nvar, nz, ny + 1, nx)
    if fz is not None:
        assert fz.shape == (nvar, nz + 1, ny, nx)
    else:
        assert nz == 1
    fxl = [np.ascontiguousarray(fx[v]) for v in range(nvar)]
    fyl = [np.ascontiguousarray(fy[v]) for v in range(nvar)]
    fzl = [np.ascontiguousarray(fz[v]) for v in range(nvar)] if fz is not None else None
    dx = np.ascontiguousarray(dx, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    rhs = np.empty((nvar, nz, ny, nx), dtype=np.float64)
    if fz is not None:
        dz = np.ascontiguousarray(dz, dtype=np.float64)
        fz_tab, dz_p = _ptr_table(fzl), _ptr(dz)
    else:
        fz_tab, dz_p = None, None
    rc = _load().oracle_flux_diff(_ptr_table(fxl), _ptr_table(fyl), fz_tab,
                                  _ptr(dx), _ptr(dy), dz_p, nvar, nx, ny, nz, _ptr(rhs))
    assert rc == 0
    return rhs


def flux_stage(fx, fy, fz, dx, dy, dz, q0, q, a: float, b: float, dt: float,
               out: np.ndarray | None = None) -> np.ndarray:
    """One SSPRK stage q' = a*q0 + b*(q + dt*rhs) on the flux difference rhs.

    ``q0``, ``q`` (and ``out``) are (nvar, nz, ny, nx); ``out`` may be ``q``
    or ``q0`` (updated in place).  Faces and spacings as for :func:`flux_diff`.
    """
    nvar, nz, ny, nxp1 = fx.shape
    nx = nxp1 - 1
    assert q0.shape == (nvar, nz, ny, nx) and q.shape == (nvar, nz, ny, nx)
    fxl = [np.ascontiguousarray(fx[v]) for v in range(nvar)]
    fyl = [np.ascontiguousarray(fy[v]) for v in range(nvar)]
    fzl = [np.ascontiguousarray(fz[v]) for v in range(nvar)] if fz is not None else None
    if out is None:
        out = np.empty((nvar, nz, ny, nx), dtype=np.float64)
    assert out.flags.c_contiguous and q0.flags.c_contiguous and q.flags.c_contiguous
    dx = np.ascontiguousarray(dx, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    if fz is not None:
        dz = np.ascontiguousarray(dz, dtype=np.float64)
        fz_tab, dz_p = _ptr_table(fzl), _ptr(dz)
    else:
        fz_tab, dz_p = None, None
    rc = _load().oracle_flux_stage(_ptr_table(fxl), _ptr_table(fyl), fz_tab, _ptr(dx), _ptr(dy), dz_p,
                                   _ptr_table([q0[v] for v in range(nvar)]),
                                   _ptr_table([q[v] for v in range(nvar)]), float(a), float(b),
                                   float(dt), nvar, nx, ny, nz, _ptr_table([out[v] for v in range(nvar)]))
    assert rc == 0
    return out


# ---------------------------------------------------------------------------
# How far one field lies from another (Qiita "Fortran 2018でGPUを高速化する
# Part 3", section 8: the per-cell acceptance band atol + rtol*|reference|;
# section 8.1: the largest error, the error's L2 norm relative to the
# reference's, the difference of the totals, and the cells outside the band).
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Deviation:
    """A candidate field measured against a reference field, in float64."""
    largest: float      # max over cells of |candidate - reference|
    l2_ratio: float     # ||candidate - reference||_2 / ||reference||_2
    total_shift: float  # sum(candidate) - sum(reference)
    outside_band: int   # cells with |candidate - reference| > atol + rtol*|reference|
    n: int              # cells compared


def deviation(reference: np.ndarray, candidate: np.ndarray, atol: float, rtol: float) -> Deviation:
    """Measure ``candidate`` against ``reference`` over every cell.

    Both are widened to float64 first.  The L2 ratio needs a reference that
    is not identically zero.  The total shift is the sum of the per-cell
    differences, which equals the difference of the two totals.
    """
    ref = np.asarray(reference, dtype=np.float64).reshape(-1)
    cand = np.asarray(candidate, dtype=np.float64).reshape(-1)
    if ref.shape != cand.shape:
        raise ValueError("reference and candidate hold different numbers of cells")
    diff = cand - ref
    size = np.abs(diff)
    ref_norm = float(np.linalg.norm(ref))
    if ref_norm == 0.0:
        raise ValueError("the L2 ratio is undefined for an all-zero reference")
    band = atol + rtol * np.abs(ref)
    return Deviation(largest=float(size.max(initial=0.0)),
                     l2_ratio=float(np.linalg.norm(diff)) / ref_norm,
                     total_shift=float(np.sum(diff)),
                     outside_band=int((size > band).sum()),
                     n=int(ref.size))


def timed(fn, *args, **kw):
    """(result, seconds) of one call, wall clock around the compute only."""
    t0 = time.perf_counter()
    out = fn(*args, **kw)
    return out, time.perf_counter() - t0
