"""The C-ABI library without a GPU: it loads, exports exactly what
include/sgc.h declares, and its host-side logic (launch counting, argument
validation before any enqueue) behaves as documented.  No call here reaches a
kernel launch: every validation case fails before the library touches HIP."""
import ctypes
import subprocess

import pytest

from structured_grid_cfd_amd import binding as b

EXPECTED = ["stencil_diffuse2d", "stencil_diffuse2d_ex", "stencil_diffuse2d_fields", "stencil_diffuse2d_launches", "field_pack", "field_unpack",
            "flux_diff3d", "flux_stage3d", "sgc_last_error", "sgc_abi_version"]


@pytest.fixture(scope="module")
def lib():
    if not b.LIB_PATH.exists():
        from structured_grid_cfd_amd import build
        build.build()
    return b.load()


def test_header_declares_the_abi():
    assert sorted(b.header_functions()) == sorted(EXPECTED)


def test_exports_every_declared_symbol(lib):
    for name in b.header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", str(b.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.split() and ln.split()[-2] == "T"}
    public = {s for s in exported if not s.startswith("_")}
    assert public == set(EXPECTED)


def test_abi_version(lib):
    assert lib.sgc_abi_version() == 1
    assert b.last_error() == ""


@pytest.mark.parametrize("steps,tb,expect", [
    (0, 4, 0), (1, 4, 1), (2, 4, 2), (4, 4, 2), (5, 4, 3), (8, 4, 2), (1000, 8, 126),
    (1000, 12, 84), (32, 8, 4), (7, 12, 1), (8, 12, 2), (31, 12, 3), (32, 12, 4), (3, 2, 3)])
def test_temporal_launch_count_parity(lib, steps, tb, expect):
    """Launch count L = ceil(steps/T), plus one when its parity differs from
    the step count's, so the alternating launches end in v iff steps is odd."""
    L = b.stencil_diffuse2d_launches(steps, "temporal", tb)
    assert L == expect
    assert L % 2 == steps % 2
    assert L <= steps or steps == 0
    if steps:
        assert -(-steps // L) <= tb


def test_launch_count_other_maps(lib):
    for m in ("collapse_branch", "contig", "strided", "tiled"):
        assert b.stencil_diffuse2d_launches(17, m, 99) == 17
    assert b.stencil_diffuse2d_launches(17, "resident", 99) == 1
    assert b.stencil_diffuse2d_launches(0, "resident", 1) == 0
    assert b.stencil_diffuse2d_launches(-1, "tiled", 1) == -1
    assert b.stencil_diffuse2d_launches(5, "temporal", 0) == -1
    assert b.stencil_diffuse2d_launches(5, "temporal", 13) == -1
    assert b.stencil_diffuse2d_launches(5, 9, 1) == -1


U, V = 0x10000, 0x90000  # fake, never dereferenced: every call below fails validation


@pytest.mark.parametrize("args,code,msg", [
    ((0, V, 1, 8, 8, 8, 0.1, 1, 3, 1, 0), 2, "non-NULL"),
    ((U, V, 7, 8, 8, 8, 0.1, 1, 3, 1, 0), 3, "dtype"),
    ((U, V, 1, 2, 8, 8, 0.1, 1, 3, 1, 0), 1, ">= 3"),
    ((U, V, 1, 8, 2, 8, 0.1, 1, 3, 1, 0), 1, ">= 3"),
    ((U, V, 1, 8, 8, 7, 0.1, 1, 3, 1, 0), 1, "ld"),
    ((U, V, 1, 8, 8, 8, 0.1, -1, 3, 1, 0), 1, "steps"),
    ((U, V, 1, 8, 8, 8, float("nan"), 1, 3, 1, 0), 1, "finite"),
    ((U, V, 1, 8, 8, 8, float("inf"), 1, 3, 1, 0), 1, "finite"),
    ((U, V, 1, 8, 8, 8, 0.1, 1, 6, 1, 0), 1, "map"),
    ((U, V, 1, 8, 8, 8, 0.1, 1, 4, 0, 0), 1, "time_block"),
    ((U, V, 1, 8, 8, 8, 0.1, 1, 4, 13, 0), 5, "time_block"),
    ((U, V, 1, 8, 8, 8, 0.1, 1, 3, 1, 9), 1, "tile_rows"),
    ((U, V, 1, 8, 8, 8, 0.1, 1, 3, 1, -1), 1, "tile_rows"),
    ((U, V, 1, 70000, 70000, 70000, 0.1, 1, 3, 1, 0), 5, "2^31"),
    ((U, V, 0, 46341, 46341, 46341, 0.1, 1, 4, 10, 0), 5, "2^31"),       # ld*ny = 2^31 + 4634
    ((U, U + 8, 0, 46341, 46340, 46341, 0.1, 1, 4, 10, 0), 4, "overlap"),  # 2^31 - 41708: in range
    ((U, V, 1, 65, 8, 65, 0.1, 1, 5, 1, 0), 5, "64 columns"),
    ((U, V, 1, 8, 129, 8, 0.1, 1, 5, 1, 0), 5, "128 rows"),
    ((U, V, 1, 8, 8, 8, 0.1, 1 << 31, 5, 1, 0), 5, "2^31-1 steps"),
    ((U, U + 8 * 63, 1, 8, 8, 8, 0.1, 1, 3, 1, 0), 4, "overlap"),
    ((U + 4, V, 1, 8, 8, 8, 0.1, 1, 3, 1, 0), 1, "aligned"),
    ((U, V + 2, 0, 8, 8, 8, 0.1, 1, 3, 1, 0), 1, "aligned"),
    ((U, U + 4 * 63, 0, 8, 8, 8, 0.1, 1, 3, 1, 0), 4, "overlap"),
])
def test_diffuse_validation(lib, args, code, msg):
    """stencil_diffuse2d_ex (explicit tile height), and the same case through
    stencil_diffuse2d, whose argument list has no tile height: every case
    whose error does not come from the tile height fails the same way, and
    neither writes the result flag on an error."""
    res = ctypes.c_int32(-7)
    rc = lib.stencil_diffuse2d_ex(*args, None, ctypes.byref(res))
    assert rc == code
    assert msg in b.last_error()
    assert res.value == -7
    if msg != "tile_rows":
        rc = lib.stencil_diffuse2d(*args[:10], None, ctypes.byref(res))
        assert rc == code
        assert msg in b.last_error()
        assert res.value == -7


def _declared_params(name):
    import re
    text = re.sub(r"/\*.*?\*/", "", b.HEADER.read_text(), flags=re.S)
    m = re.search(r"SGC_API\s+int\s+" + name + r"\s*\((.*?)\);", text, flags=re.S)
    return [re.split(r"[\s*]+", p.strip())[-1] for p in m.group(1).split(",")]


def test_diffuse_signature_is_the_surveyed_one():
    """stencil_diffuse2d takes (u, v, dtype, nx, ny, ld, alpha, steps, map,
    time_block, stream, result_is_v): a caller written to that list passes
    its stream and result pointer in the right places; the tile height is
    only in stencil_diffuse2d_ex."""
    assert _declared_params("stencil_diffuse2d") == [
        "u", "v", "dtype", "nx", "ny", "ld", "alpha", "steps", "map", "time_block", "stream",
        "result_is_v"]
    assert _declared_params("stencil_diffuse2d_ex") == [
        "u", "v", "dtype", "nx", "ny", "ld", "alpha", "steps", "map", "time_block", "tile_rows",
        "stream", "result_is_v"]
    assert len(b.load().stencil_diffuse2d.argtypes) == 12
    assert len(b.load().stencil_diffuse2d_ex.argtypes) == 13


def test_diffuse_surveyed_form_reaches_the_result_pointer(lib):
    """A NULL stream and a result pointer in the surveyed positions: a
    validation error (ld < nx) is reported without touching the flag, and a
    valid zero-size request is impossible without a GPU, so the flag is
    checked on the error path only."""
    res = ctypes.c_int32(-3)
    assert lib.stencil_diffuse2d(U, V, 1, 8, 8, 7, 0.1, 3, 4, 10, None, ctypes.byref(res)) == 1
    assert "ld" in b.last_error() and res.value == -3


def _tab(*ptrs):
    t = (ctypes.c_void_p * len(ptrs))()
    for k, p in enumerate(ptrs):
        t[k] = p
    return t


def test_pack_validation(lib):
    f = _tab(U, U + 0x1000)
    assert lib.field_pack(f, 0, 4, 4, 4, 0, V, 2, None) == 1
    assert lib.field_pack(f, 33, 4, 4, 4, 0, V, 2, None) == 1
    assert lib.field_pack(None, 2, 4, 4, 4, 0, V, 2, None) == 2
    assert lib.field_pack(_tab(U, 0), 2, 4, 4, 4, 0, V, 2, None) == 2
    assert "entry 1" in b.last_error()
    assert lib.field_pack(f, 2, 4, 4, 4, 0, None, 2, None) == 2
    assert lib.field_pack(f, 2, 4, 4, 4, 3, V, 2, None) == 1
    assert lib.field_pack(f, 2, 4, 4, 4, 0, V, 3, None) == 1
    assert lib.field_pack(f, 2, 0, 4, 4, 0, V, 2, None) == 1
    assert lib.field_pack(f, 2, 2000, 2000, 1000, 0, V, 2, None) == 5
    assert lib.field_pack(f, 2, 1290, 1290, 646, 0, V, 2, None) == 5     # 2 * 1290^2 * 646 > 2^31 - 1
    assert lib.field_pack(f, 2, 1290, 1290, 645, 0, U + 8, 2, None) == 4  # in range, then the alias
    # out overlapping field 1
    assert lib.field_pack(f, 2, 4, 4, 4, 0, U + 0x1000 + 8, 2, None) == 4
    assert lib.field_unpack(V, 2, 4, 4, 4, 1, _tab(U, U + 8), 2, None) == 4
    assert lib.field_unpack(U + 16, 2, 4, 4, 4, 1, _tab(U, U + 0x1000), 2, None) == 4
    assert lib.field_unpack(None, 2, 4, 4, 4, 1, f, 2, None) == 2


def test_flux_validation(lib):
    fx, fy, fz = _tab(U), _tab(U + 0x1000), _tab(U + 0x2000)
    d = U + 0x3000
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 4, 4, 4, V, 5, None) == 1
    assert lib.flux_diff3d(None, fy, fz, d, d, d, 1, 4, 4, 4, V, 2, None) == 2
    assert lib.flux_diff3d(fx, fy, fz, d, d, None, 1, 4, 4, 4, V, 2, None) == 2
    assert lib.flux_diff3d(fx, fy, None, d, d, d, 1, 4, 4, 4, V, 2, None) == 2
    assert lib.flux_diff3d(fx, fy, None, d, d, None, 1, 4, 4, 4, V, 2, None) == 1
    assert "nz == 1" in b.last_error()
    assert lib.flux_diff3d(fx, fy, fz, 0, d, d, 1, 4, 4, 4, V, 2, None) == 2
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 4, 4, 4, None, 2, None) == 2
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 4, 4, 4, U + 0x1000, 2, None) == 4
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 3000, 3000, 3000, V, 2, None) == 5
    # the size bound: (nx+1)(ny+1)(nz+1) and nvar*nx*ny*nz at most 2^31 - 1
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 1290, 1290, 1290, V, 2, None) == 5  # 1291^3
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 1289, 1289, 1289, U, 2, None) == 4  # 1290^3: passes, then the alias
    fx2, fy2, fz2 = _tab(U, U + 0x800), _tab(U + 0x1000, U + 0x1800), _tab(U + 0x2000, U + 0x2800)
    assert lib.flux_diff3d(fx2, fy2, fz2, d, d, d, 2, 1289, 1289, 1289, V, 2, None) == 5  # 2 * 1289^3
    assert lib.flux_diff3d(fx, fy, fz, d, d, d, 1, 4, 4, 4, V + 4, 2, None) == 1
    assert lib.flux_diff3d(_tab(U + 2), fy, fz, d, d, d, 1, 4, 4, 4, V, 2, None) == 1


def test_stage_validation(lib):
    fx, fy, fz = _tab(U), _tab(U + 0x1000), _tab(U + 0x2000)
    d = U + 0x3000
    q0, q = _tab(V), _tab(V + 0x1000)
    def call(qout, a=0.75, b=0.25, dt=0.1, m=2, q0t=q0, qt=q, fzt=fz, dzp=d, n=(4, 4, 4)):
        return lib.flux_stage3d(fx, fy, fzt, d, d, dzp, q0t, qt, a, b, dt, 1, *n, qout, m, None)
    assert call(None) == 2
    assert call(_tab(0)) == 2
    assert call(_tab(V + 0x3000), q0t=None) == 2
    assert call(_tab(V + 0x3000), a=float("nan")) == 1 and "finite" in b.last_error()
    assert call(_tab(V + 0x3000), dt=float("inf")) == 1
    assert call(_tab(V + 0x3000), m=5) == 1
    assert call(_tab(V + 0x3000), fzt=None) == 2          # dz given without fz
    assert call(_tab(V + 0x3000), fzt=None, dzp=None) == 1  # 2D form needs nz == 1
    assert call(_tab(U + 0x1000)) == 4                     # qout on fy
    assert call(_tab(d)) == 4                              # qout on the spacings
    assert call(_tab(V + 8)) == 4                          # qout straddles q0
    assert call(_tab(V + 0x1000 + 8)) == 4                 # qout straddles q
    assert call(_tab(V + 4)) == 1                          # misaligned
    assert call(_tab(V + 0x3000), n=(3000, 3000, 3000)) == 5


def test_fields_validation(lib):
    """stencil_diffuse2d_fields: every field's pointers and every pair of the
    2*nvar buffers are checked, and only the marching maps are accepted."""
    u, v = _tab(U, U + 0x1000), _tab(V, V + 0x1000)
    base = (1, 8, 8, 8, 0.1, 1, 4, 2, 0)  # f64, nx, ny, ld, alpha, steps, TEMPORAL, time_block, rows

    def call(uu, vv, n, *rest):
        return lib.stencil_diffuse2d_fields(uu, vv, n, *rest, None, None)

    assert call(None, v, 2, *base) == 2 and "non-NULL" in b.last_error()
    assert call(u, v, 0, *base) == 1 and "nvar" in b.last_error()
    assert call(u, v, 33, *base) == 1 and "nvar" in b.last_error()
    assert call(u, v, 2, 7, 8, 8, 8, 0.1, 1, 4, 2, 0) == 3                     # dtype
    assert call(u, v, 2, 1, 8, 8, 7, 0.1, 1, 4, 2, 0) == 1                     # ld < nx
    assert call(u, v, 2, 1, 8, 8, 8, 0.1, 1, 4, 13, 0) == 5                    # time_block
    for m in (0, 1, 2, 6):                                                     # page maps, unknown
        assert call(u, v, 2, 1, 8, 8, 8, 0.1, 1, m, 1, 0) == 1 and "map" in b.last_error()
    assert call(u, v, 2, 1, 65, 8, 65, 0.1, 1, 5, 1, 0) == 5 and "64 columns" in b.last_error()
    assert call(u, v, 2, 1, 8, 129, 8, 0.1, 1, 5, 1, 0) == 5 and "128 rows" in b.last_error()
    assert call(u, v, 2, 1, 8, 8, 8, 0.1, 1 << 31, 5, 1, 0) == 5 and "2^31-1" in b.last_error()
    assert call(_tab(U, 0), v, 2, *base) == 2 and "entry 1" in b.last_error()
    assert call(_tab(U, U + 0x1004), v, 2, *base) == 1 and "aligned" in b.last_error()
    assert call(_tab(U, U + 8 * 63), v, 2, *base) == 4 and "overlap" in b.last_error()  # u[0], u[1]
    assert call(u, _tab(V, U + 8 * 7), 2, *base) == 4                          # v[1] on u[0]
    assert call(u, _tab(V, V), 2, *base) == 4                                  # v[0] is v[1]


def test_last_error_is_per_call(lib):
    lib.stencil_diffuse2d(0, 0, 1, 8, 8, 8, 0.1, 1, 3, 1, None, None)
    assert b.last_error() != ""
    assert b.stencil_diffuse2d_launches(3, "tiled", 1) == 3
    # a later failing call replaces the message
    lib.field_pack(None, 1, 1, 1, 1, 0, V, 0, None)
    assert "fields table" in b.last_error()


def test_production_launch_settings():
    """The production settings per grid size and precision: the resident map
    for grids of at most 64 x 128 cells; FP64 marches at depth 8 below 2^24
    cells and 10 from there up; FP32 at 8 below 2^22, 10 up to 2^24, 12 up to
    2^26 and 10 beyond (what the benchmark and the full-size parity tests
    run)."""
    from structured_grid_cfd_amd import launch_config as lc
    assert lc.diffusion("f64", 64, 64)["map"] == "resident"
    assert lc.diffusion("f32", 64, 128)["map"] == "resident"
    assert lc.diffusion("f64", 65, 64) == {"map": "temporal", "time_block": 8, "tile_rows": 0}
    assert lc.diffusion("f64", 64, 129)["time_block"] == 8
    assert lc.diffusion("f64", 4095, 4095)["time_block"] == 8
    assert lc.diffusion("f64", 4096, 4096) == {"map": "temporal", "time_block": 10, "tile_rows": 0}
    assert lc.diffusion("f64", 16384, 16384)["time_block"] == 10
    assert lc.diffusion("f32") == {"map": "temporal", "time_block": 10, "tile_rows": 0}
    # FP32: 8 below 2^22 cells, 10 up to 2^24, 12 up to 2^26, 10 beyond
    assert lc.diffusion("f32", 2047, 2048)["time_block"] == 8
    assert lc.diffusion("f32", 2048, 2048)["time_block"] == 10
    assert lc.diffusion("f32", 4095, 4096)["time_block"] == 10
    assert lc.diffusion("f32", 4096, 4096) == {"map": "temporal", "time_block": 12, "tile_rows": 0}
    assert lc.diffusion("f32", 8191, 8192)["time_block"] == 12
    assert lc.diffusion("f32", 8192, 8192)["time_block"] == 10
    assert lc.diffusion("f32", 16384, 16384)["time_block"] == 10
    assert lc.diffusion("f32", 64, 128)["map"] == "resident"
    for nx, ny in ((64, 64), (300, 200), (4096, 4096)):
        c = lc.diffusion("f64", nx, ny)
        assert b.stencil_diffuse2d_launches(32, c["map"], c["time_block"]) >= 1
