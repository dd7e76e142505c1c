"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from structured_grid_cfd_amd import binding


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU (torch.cuda.is_available() is False)")
    binding.load()


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Bit pattern view (so NaN sentinels and signed zeros compare exactly)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint64 if a.dtype == np.float64 else np.uint32)


def assert_bitwise(got: np.ndarray, ref: np.ndarray, what: str = ""):
    gb, rb = bits(got), bits(ref)
    if not np.array_equal(gb, rb):
        bad = np.argwhere(gb != rb)
        first = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} of {gb.size} elements differ; first at {first}: "
            f"got {got[first]!r} expected {ref[first]!r}")


def gpu_diffuse(u0, v0, nx, alpha, steps, map, time_block=1, tile_rows=0, stream=None):
    """Run the HIP path on copies; returns (result, in_v, u_after, v_after)."""
    u, v = dev(u0), dev(v0)
    in_v = binding.stencil_diffuse2d(u, v, nx, alpha, steps, map, time_block, tile_rows, stream)
    torch.cuda.synchronize()
    uh, vh = host(u), host(v)
    return (vh if in_v else uh), in_v, uh, vh


def oracle_diffuse(u0, v0, nx, alpha, steps):
    u, v = u0.copy(), v0.copy()
    in_v = oracle.diffuse2d(u, v, nx, alpha, steps)
    return (v if in_v else u), in_v


def assert_bitwise_nan(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """Bitwise equality where every NaN counts as equal to every NaN: the sign
    and payload of a NaN made by inf - inf are the platform's choice, not the
    definition's (x86 and gfx950 differ), so only NaN positions are compared."""
    gn, rn = np.isnan(got), np.isnan(ref)
    if not np.array_equal(gn, rn):
        bad = np.argwhere(gn != rn)
        first = tuple(bad[0])
        raise AssertionError(f"{what}: NaN positions differ at {len(bad)} elements; first at "
                             f"{first}: got {got[first]!r} expected {ref[first]!r}")
    assert_bitwise(np.where(gn, 0, got).astype(got.dtype), np.where(rn, 0, ref).astype(ref.dtype), what)
