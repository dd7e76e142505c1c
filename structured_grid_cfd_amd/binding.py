"""Thin ctypes binding to libsgc.so (declared in include/sgc.h).

Argument marshalling only: torch supplies device memory and streams, every
step of the sweeps runs in the library's HIP kernels.  There is no CPU path:
if the library has not been built, or no GPU is present, the calls raise.

Layouts (numpy/torch C-order view of the Fortran-order arrays):

* 2D grid u(nx, ny), leading dimension ld: tensor ``(ny, ld)``.
* field f(j,k,l): ``(nz, ny, nx)``; nvar fields ``(nvar, nz, ny, nx)``.
* packed: x ``(nvar, nz, ny, nx)``, y ``(nvar, nz, nx, ny)``,
  z ``(nvar, nx, ny, nz)``.
* faces: Fx ``(nvar, nz, ny, nx+1)``, Fy ``(nvar, nz, ny+1, nx)``,
  Fz ``(nvar, nz+1, ny, nx)``; rhs ``(nvar, nz, ny, nx)``.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path
from typing import Sequence

import torch

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libsgc.so"
HEADER = PKG.parent / "include" / "sgc.h"

DIFF_MAPS = {"collapse_branch": 0, "contig": 1, "strided": 2, "tiled": 3, "temporal": 4,
             "resident": 5}
VAR_MAPS = {"per_cell": 0, "per_cellvar": 1, "tiled": 2}
DIRS = {"x": 0, "y": 1, "z": 2, 0: 0, 1: 1, 2: 2}
STATUS = {0: "SGC_OK", 1: "SGC_EINVAL", 2: "SGC_ENULL", 3: "SGC_EDTYPE", 4: "SGC_EALIAS",
          5: "SGC_ERANGE", 6: "SGC_EHIP"}
MAX_NVAR = 32
MAX_TIME_BLOCK = 12


class SGCError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libsgc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it first (python -m structured_grid_cfd_amd.build)")
    lib = ctypes.CDLL(str(LIB_PATH))
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.stencil_diffuse2d.argtypes = [vp, vp, i32, i64, i64, i64, dbl, i64, i32, i32, vp,
                                      ctypes.POINTER(i32)]
    lib.stencil_diffuse2d.restype = ctypes.c_int
    lib.stencil_diffuse2d_ex.argtypes = [vp, vp, i32, i64, i64, i64, dbl, i64, i32, i32, i32, vp,
                                         ctypes.POINTER(i32)]
    lib.stencil_diffuse2d_ex.restype = ctypes.c_int
    lib.stencil_diffuse2d_fields.argtypes = [vp, vp, i32, i32, i64, i64, i64, dbl, i64, i32, i32, i32,
                                             vp, vp]
    lib.stencil_diffuse2d_fields.restype = ctypes.c_int
    lib.stencil_diffuse2d_launches.argtypes = [i64, i32, i32]
    lib.stencil_diffuse2d_launches.restype = i64
    lib.field_pack.argtypes = [vp, i32, i64, i64, i64, i32, vp, i32, vp]
    lib.field_pack.restype = ctypes.c_int
    lib.field_unpack.argtypes = [vp, i32, i64, i64, i64, i32, vp, i32, vp]
    lib.field_unpack.restype = ctypes.c_int
    lib.flux_diff3d.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, vp, i32, vp]
    lib.flux_diff3d.restype = ctypes.c_int
    lib.flux_stage3d.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, i32, i64, i64, i64,
                                 vp, i32, vp]
    lib.flux_stage3d.restype = ctypes.c_int
    lib.sgc_last_error.argtypes = []
    lib.sgc_last_error.restype = ctypes.c_char_p
    lib.sgc_abi_version.argtypes = []
    lib.sgc_abi_version.restype = i32
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/sgc.h declares."""
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*SGC_API\s+(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text,
                      flags=re.M)


def last_error() -> str:
    return load().sgc_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise SGCError(rc, last_error())


def _stream_ptr(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev_ptr(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _table(ts: Sequence[torch.Tensor]):
    tab = (ctypes.c_void_p * len(ts))()
    for k, t in enumerate(ts):
        tab[k] = _dev_ptr(t)
    return tab


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float64:
        return 1
    if t.dtype == torch.float32:
        return 0
    raise ValueError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
# five-point diffusion
# ---------------------------------------------------------------------------

def stencil_diffuse2d(u: torch.Tensor, v: torch.Tensor, nx: int, alpha: float, steps: int,
                      map: str | int = "temporal", time_block: int = 1, tile_rows: int = 0,
                      stream=None) -> bool:
    """Run ``steps`` sweeps on the (ny, ld) pair; returns True if the result is in v.

    ``tile_rows`` 0 calls the C entry point ``stencil_diffuse2d`` (automatic
    tile height); any other value calls ``stencil_diffuse2d_ex`` with it.
    """
    if u.shape != v.shape or u.dtype != v.dtype or u.dim() != 2:
        raise ValueError("u and v must be 2D tensors of one shape and dtype")
    ny, ld = u.shape
    m = DIFF_MAPS[map] if isinstance(map, str) else int(map)
    res = ctypes.c_int32(-1)
    if int(tile_rows) == 0:
        rc = load().stencil_diffuse2d(_dev_ptr(u), _dev_ptr(v), _dtype_code(u), nx, ny, ld,
                                      float(alpha), int(steps), m, int(time_block),
                                      _stream_ptr(stream), ctypes.byref(res))
    else:
        rc = load().stencil_diffuse2d_ex(_dev_ptr(u), _dev_ptr(v), _dtype_code(u), nx, ny, ld,
                                         float(alpha), int(steps), m, int(time_block),
                                         int(tile_rows), _stream_ptr(stream), ctypes.byref(res))
    _check(rc)
    return bool(res.value)


def stencil_diffuse2d_ex(u: torch.Tensor, v: torch.Tensor, nx: int, alpha: float, steps: int,
                         map: str | int = "temporal", time_block: int = 1, tile_rows: int = 0,
                         stream=None) -> bool:
    """``stencil_diffuse2d_ex``: the sweeps with an explicit tile height."""
    if u.shape != v.shape or u.dtype != v.dtype or u.dim() != 2:
        raise ValueError("u and v must be 2D tensors of one shape and dtype")
    ny, ld = u.shape
    m = DIFF_MAPS[map] if isinstance(map, str) else int(map)
    res = ctypes.c_int32(-1)
    rc = load().stencil_diffuse2d_ex(_dev_ptr(u), _dev_ptr(v), _dtype_code(u), nx, ny, ld,
                                     float(alpha), int(steps), m, int(time_block), int(tile_rows),
                                     _stream_ptr(stream), ctypes.byref(res))
    _check(rc)
    return bool(res.value)


def stencil_diffuse2d_fields(us, vs, nx: int, alpha: float, steps: int, map: str | int = "temporal",
                             time_block: int = 1, tile_rows: int = 0, stream=None) -> bool:
    """The sweeps of :func:`stencil_diffuse2d` on several (ny, ld) pairs of one
    shape and dtype in shared launches; returns True if every result is in its v."""
    ul, vl = _as_list(us), _as_list(vs)
    if not ul or len(ul) != len(vl):
        raise ValueError("us and vs must be non-empty and of one length")
    ny, ld = ul[0].shape
    for t in ul + vl:
        if t.dim() != 2 or tuple(t.shape) != (ny, ld) or t.dtype != ul[0].dtype:
            raise ValueError("every field must be a 2D tensor of one shape and dtype")
    m = DIFF_MAPS[map] if isinstance(map, str) else int(map)
    res = ctypes.c_int32(-1)
    rc = load().stencil_diffuse2d_fields(_table(ul), _table(vl), len(ul), _dtype_code(ul[0]), nx, ny,
                                         ld, float(alpha), int(steps), m, int(time_block),
                                         int(tile_rows), _stream_ptr(stream), ctypes.byref(res))
    _check(rc)
    return bool(res.value)


def stencil_diffuse2d_launches(steps: int, map: str | int, time_block: int = 1) -> int:
    m = DIFF_MAPS[map] if isinstance(map, str) else int(map)
    return int(load().stencil_diffuse2d_launches(int(steps), m, int(time_block)))


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------

def packed_shape(nvar: int, nx: int, ny: int, nz: int, direction) -> tuple:
    d = DIRS[direction]
    return (nvar,) + {0: (nz, ny, nx), 1: (nz, nx, ny), 2: (nx, ny, nz)}[d]


def _as_list(fields) -> list:
    if isinstance(fields, torch.Tensor):
        return [fields[k] for k in range(fields.shape[0])]
    return list(fields)


def field_pack(fields, direction, out: torch.Tensor | None = None, map: str | int = "tiled",
               stream=None) -> torch.Tensor:
    """Pack nvar fields (each (nz, ny, nx) float64) along x, y or z."""
    fl = _as_list(fields)
    nz, ny, nx = fl[0].shape
    nvar = len(fl)
    d = DIRS[direction]
    if out is None:
        out = torch.empty(packed_shape(nvar, nx, ny, nz, d), dtype=torch.float64, device=fl[0].device)
    for t in fl:
        if t.dtype != torch.float64 or tuple(t.shape) != (nz, ny, nx):
            raise ValueError("fields must be float64 tensors of one shape")
    if out.numel() != nvar * nx * ny * nz or out.dtype != torch.float64:
        raise ValueError("out has the wrong size or dtype")
    m = VAR_MAPS[map] if isinstance(map, str) else int(map)
    _check(load().field_pack(_table(fl), nvar, nx, ny, nz, d, _dev_ptr(out), m, _stream_ptr(stream)))
    return out


def field_unpack(packed: torch.Tensor, nx: int, ny: int, nz: int, direction, fields=None,
                 map: str | int = "tiled", stream=None):
    """Inverse of :func:`field_pack`; returns the (nvar, nz, ny, nx) fields."""
    nvar = packed.shape[0]
    d = DIRS[direction]
    if fields is None:
        fields = torch.empty((nvar, nz, ny, nx), dtype=torch.float64, device=packed.device)
    fl = _as_list(fields)
    if packed.numel() != nvar * nx * ny * nz or packed.dtype != torch.float64:
        raise ValueError("packed has the wrong size or dtype")
    m = VAR_MAPS[map] if isinstance(map, str) else int(map)
    _check(load().field_unpack(_dev_ptr(packed), nvar, nx, ny, nz, d, _table(fl), m,
                               _stream_ptr(stream)))
    return fields


# ---------------------------------------------------------------------------
# flux difference
# ---------------------------------------------------------------------------

def flux_diff3d(fx, fy, fz, dx: torch.Tensor, dy: torch.Tensor, dz: torch.Tensor | None,
                rhs: torch.Tensor | None = None, map: str | int = "tiled",
                stream=None) -> torch.Tensor:
    """rhs (nvar, nz, ny, nx) from per-variable faces; fz=None is the 2D form."""
    fxl, fyl = _as_list(fx), _as_list(fy)
    fzl = _as_list(fz) if fz is not None else None
    nvar = len(fxl)
    nz, ny, nxp1 = fxl[0].shape
    nx = nxp1 - 1
    if rhs is None:
        rhs = torch.empty((nvar, nz, ny, nx), dtype=torch.float64, device=fxl[0].device)
    if rhs.numel() != nvar * nx * ny * nz:
        raise ValueError("rhs has the wrong size")
    for t in fxl:
        if tuple(t.shape) != (nz, ny, nx + 1):
            raise ValueError("fx entries must be (nz, ny, nx+1)")
    for t in fyl:
        if tuple(t.shape) != (nz, ny + 1, nx):
            raise ValueError("fy entries must be (nz, ny+1, nx)")
    if fzl is not None:
        for t in fzl:
            if tuple(t.shape) != (nz + 1, ny, nx):
                raise ValueError("fz entries must be (nz+1, ny, nx)")
    m = VAR_MAPS[map] if isinstance(map, str) else int(map)
    rc = load().flux_diff3d(_table(fxl), _table(fyl), _table(fzl) if fzl is not None else None,
                            _dev_ptr(dx), _dev_ptr(dy), _dev_ptr(dz) if dz is not None else None,
                            nvar, nx, ny, nz, _dev_ptr(rhs), m, _stream_ptr(stream))
    _check(rc)
    return rhs


def flux_stage3d(fx, fy, fz, dx: torch.Tensor, dy: torch.Tensor, dz: torch.Tensor | None,
                 q0, q, a: float, b: float, dt: float, out=None, map: str | int = "tiled",
                 stream=None):
    """One SSPRK stage q' = a*q0 + b*(q + dt*rhs) fused with the flux difference.

    q0, q and out are nvar fields of (nz, ny, nx) float64 (a stacked tensor or
    a list); out defaults to a new (nvar, nz, ny, nx) tensor and may be q or
    q0 (updated in place).  Faces and spacings as for :func:`flux_diff3d`.
    """
    fxl, fyl = _as_list(fx), _as_list(fy)
    fzl = _as_list(fz) if fz is not None else None
    nvar = len(fxl)
    nz, ny, nxp1 = fxl[0].shape
    nx = nxp1 - 1
    q0l, ql = _as_list(q0), _as_list(q)
    if out is None:
        out = torch.empty((nvar, nz, ny, nx), dtype=torch.float64, device=fxl[0].device)
    outl = _as_list(out)
    for name, lst in (("q0", q0l), ("q", ql), ("out", outl)):
        if len(lst) != nvar:
            raise ValueError(f"{name} must hold {nvar} fields")
        for t in lst:
            if t.dtype != torch.float64 or tuple(t.shape) != (nz, ny, nx):
                raise ValueError(f"{name} fields must be float64 (nz, ny, nx)")
    m = VAR_MAPS[map] if isinstance(map, str) else int(map)
    rc = load().flux_stage3d(_table(fxl), _table(fyl), _table(fzl) if fzl is not None else None,
                             _dev_ptr(dx), _dev_ptr(dy), _dev_ptr(dz) if dz is not None else None,
                             _table(q0l), _table(ql), float(a), float(b), float(dt), nvar, nx, ny, nz,
                             _table(outl), m, _stream_ptr(stream))
    _check(rc)
    return out
