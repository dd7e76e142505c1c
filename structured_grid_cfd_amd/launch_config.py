"""Launch settings of the production path: the maps, time block and tile
shapes that the benchmark times and the full-size parity tests check."""

# Five-point diffusion: temporal blocking, automatic tile rows.  Depth 10 on
# grids of 4096^2 and up (whole-workload timings on MI355X, 1000 sweeps of
# 4096^2 and 200 of 16384^2: FP64 depth 10 beat 8 by 2% and 11%, FP32 depth
# 10 beat 8 and 12); depth 8 below, where each launch is latency bound and
# the shallower march finishes sooner (9-20% faster at 128^2-2048^2).
DIFFUSION = {"map": "temporal", "time_block": 10, "tile_rows": 0}
DIFFUSION_F32 = {"map": "temporal", "time_block": 10, "tile_rows": 0}
SMALL_GRID_CELLS = 8 * 1024 * 1024  # below this, depth 8

# Per-variable field kernels.
PACK = {"map": "tiled"}
FLUX = {"map": "tiled"}


def diffusion(dtype_name: str, nx: int | None = None, ny: int | None = None) -> dict:
    """Production diffusion settings for a dtype, and for a grid size if given."""
    cfg = dict(DIFFUSION_F32 if dtype_name in ("f32", "float32") else DIFFUSION)
    if nx is not None and ny is not None and nx * ny < SMALL_GRID_CELLS:
        cfg["time_block"] = 8
    return cfg
