"""GPU parity of stencil_diffuse2d_fields: several fields of one shape stepped
in shared marching launches.  Every field must come out bit for bit as the
oracle steps it on its own, and as a single-field call steps it: the fields
only share launches, never values.  Cases: 1..32 fields, ragged grids with a
NaN sentinel in the padding columns, the TILED map and TEMPORAL depths 3..12,
odd and even step counts, zero steps, an overflowing cell in one field only
(that field's tiles fall back to the separate form, the others stay fused),
and eight 1024^2 fields at the production depth."""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_bitwise, assert_bitwise_nan, dev, host, oracle_diffuse, require_gpu, say
from structured_grid_cfd_amd import binding, inputs, launch_config

pytestmark = pytest.mark.gpu

DT = {"f64": np.float64, "f32": np.float32}


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def _fields(nf, nx, ny, ld, dt, seed, pad=np.nan):
    return [inputs.uniform_grid(nx, ny, seed + k, DT[dt], ld=ld, pad_value=pad) for k in range(nf)]


def _run_fields(pairs, nx, steps, m, tb, rows=0):
    us = [dev(u) for u, _ in pairs]
    vs = [dev(v) for _, v in pairs]
    in_v = binding.stencil_diffuse2d_fields(us, vs, nx, 0.1, steps, m, tb, rows)
    torch.cuda.synchronize()
    return [host(v if in_v else u) for u, v in zip(us, vs)], in_v


def _check_against_oracle(pairs, nx, steps, m, tb, what, nan_ok=False, rows=0):
    got, in_v = _run_fields(pairs, nx, steps, m, tb, rows)
    for k, (u0, v0) in enumerate(pairs):
        ref, ref_in_v = oracle_diffuse(u0, v0, nx, 0.1, steps)
        assert in_v == ref_in_v
        (assert_bitwise_nan if nan_ok else assert_bitwise)(got[k][:, :nx], ref[:, :nx], f"{what} field {k}")
        if got[k].shape[1] > nx:  # padding columns keep their sentinel bits
            w = np.uint64 if got[k].dtype == np.float64 else np.uint32
            assert np.array_equal(got[k][:, nx:].view(w), u0[:, nx:].view(w)), f"{what} field {k} padding"
    return got


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("nf", [1, 3, 7])
@pytest.mark.parametrize("nx,ny,ld", [(257, 131, 260), (96, 70, 96), (1031, 97, 1040)])
@pytest.mark.parametrize("m,tb", [("tiled", 1), ("temporal", 3), ("temporal", 5), ("temporal", 8),
                                  ("temporal", 10), ("temporal", 12)])
def test_fields_match_the_oracle(dt, nf, nx, ny, ld, m, tb):
    pairs = _fields(nf, nx, ny, ld, dt, 1500 + nx)
    for steps in (2 * tb + 1, 2 * tb):
        say("fields", dt, nf, nx, ny, ld, m, tb, steps)
        _check_against_oracle(pairs, nx, steps, m, tb, f"{nf} fields {nx}x{ny} {m} T={tb} S={steps}")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_fields_equal_single_field_calls(dt):
    nx, ny, ld = 300, 211, 304
    pairs = _fields(5, nx, ny, ld, dt, 1600)
    for m, tb, steps, rows in (("temporal", 10, 23, 0), ("temporal", 7, 14, 9), ("tiled", 1, 3, 0)):
        say("fields vs single", dt, m, tb, steps, rows)
        got, _ = _run_fields(pairs, nx, steps, m, tb, rows)
        for k, (u0, v0) in enumerate(pairs):
            u, v = dev(u0), dev(v0)
            in_v = binding.stencil_diffuse2d(u, v, nx, 0.1, steps, m, tb, rows)
            torch.cuda.synchronize()
            assert_bitwise(got[k], host(v if in_v else u), f"field {k} {m} T={tb}")


@pytest.mark.parametrize("dt", ["f64", "f32"])
@pytest.mark.parametrize("nf", [1, 4, 32])
@pytest.mark.parametrize("nx,ny,ld", [(64, 64, 64), (37, 128, 40), (5, 7, 8), (64, 65, 64)])
def test_resident_fields(dt, nf, nx, ny, ld):
    """One workgroup per field: each field as the oracle steps it, and the
    other buffer one step earlier, as for a single field."""
    pairs = _fields(nf, nx, ny, ld, dt, 2300 + nx + ny)
    for steps in (1, 8, 33):
        say("resident fields", dt, nf, nx, ny, ld, steps)
        us = [dev(u) for u, _ in pairs]
        vs = [dev(v) for _, v in pairs]
        in_v = binding.stencil_diffuse2d_fields(us, vs, nx, 0.1, steps, "resident")
        torch.cuda.synchronize()
        for k, (u0, v0) in enumerate(pairs):
            ref, ref_in_v = oracle_diffuse(u0, v0, nx, 0.1, steps)
            before, _ = oracle_diffuse(u0, v0, nx, 0.1, steps - 1)
            assert in_v == ref_in_v
            assert_bitwise(host(vs[k] if in_v else us[k])[:, :nx], ref[:, :nx], f"resident field {k}")
            assert_bitwise(host(us[k] if in_v else vs[k])[:, :nx], before[:, :nx], f"resident field {k} prev")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_resident_fields_choose_their_form_each(dt):
    """The fast or separate form is chosen per workgroup, that is per field:
    a NaN in one field and values too large for the fast form in another
    leave the ordinary fields beside them on the fast form, and every field
    is the oracle's."""
    nx, ny = 64, 90
    pairs = _fields(4, nx, ny, nx, dt, 2400)
    big = np.ldexp(1.0, 1021 if dt == "f64" else 125)
    pairs[1][0][40, 30] = np.nan
    pairs[2][0][20:23, 10:13] = big
    steps = 9
    say("resident fields, mixed forms", dt)
    us = [dev(u) for u, _ in pairs]
    vs = [dev(v) for _, v in pairs]
    in_v = binding.stencil_diffuse2d_fields(us, vs, nx, 0.1, steps, "resident")
    torch.cuda.synchronize()
    for k, (u0, v0) in enumerate(pairs):
        ref, _ = oracle_diffuse(u0, v0, nx, 0.1, steps)
        assert_bitwise_nan(host(vs[k] if in_v else us[k])[:, :nx], ref[:, :nx], f"resident field {k}")


def test_resident_fields_reject_large_grids():
    us = [torch.zeros(129, 8, dtype=torch.float64, device="cuda") for _ in range(2)]
    vs = [torch.zeros_like(t) for t in us]
    with pytest.raises(binding.SGCError) as e:
        binding.stencil_diffuse2d_fields(us, vs, 8, 0.1, 4, "resident")
    assert e.value.code == 5


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_max_fields_small_grid(dt):
    pairs = _fields(32, 37, 29, 37, dt, 1700)
    say("32 fields", dt)
    _check_against_oracle(pairs, 37, 21, "temporal", 10, "32 fields")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_zero_steps_zeroes_every_u_ring(dt):
    nx, ny = 40, 30
    pairs = _fields(3, nx, ny, nx, dt, 1800)
    for u0, _ in pairs:
        u0[0, :] = 3
        u0[:, 0] = 4
    got, in_v = _run_fields(pairs, nx, 0, "temporal", 8)
    assert not in_v
    for k, (u0, _) in enumerate(pairs):
        ref = u0.copy()
        ref[0, :nx] = ref[-1, :nx] = 0
        ref[:, 0] = ref[:, nx - 1] = 0
        assert_bitwise(got[k][:, :nx], ref[:, :nx], f"zero steps field {k}")


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_one_field_overflows(dt):
    nx, ny = 400, 300
    pairs = _fields(4, nx, ny, nx, dt, 1900, pad=0.0)
    u0 = pairs[2][0]
    big = np.ldexp(1.0, 1022 if dt == "f64" else 126)
    j, i = ny // 2, 1  # next to the left boundary: an edge tile
    u0[j, i] = big
    u0[j, i + 1] = u0[j - 1, i] = u0[j + 1, i] = big / 2
    say("one field overflows", dt)
    got = _check_against_oracle(pairs, nx, 20, "temporal", 10, "overflow in field 2", nan_ok=True)
    assert not np.isfinite(got[2]).all() and all(np.isfinite(got[k]).all() for k in (0, 1, 3))


def test_eight_fields_1024_production_depth():
    n = 1024
    cfg = launch_config.diffusion("f64", n, n)
    pairs = _fields(8, n, n, n, "f64", 2000, pad=0.0)
    say("8 x 1024^2", cfg)
    _check_against_oracle(pairs, n, 100, cfg["map"], cfg["time_block"], "8 x 1024^2 100 sweeps")
