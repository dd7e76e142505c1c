"""Launch settings of the production path: the maps, time block and tile
shapes that the benchmark times and the full-size parity tests check."""

# Five-point diffusion: temporal blocking, automatic tile rows.  The depth
# depends on the grid size and precision (whole-workload timings on MI355X,
# 240-400 sweeps, depths 6-12):
#   FP64: depth 8 below 2^24 cells, 10 from 4096^2 up (10 ahead of 8 and 12
#     by 3-17% from 4096^2 to 12288^2; between 2048^2 and 3072^2 depths 8
#     and 10 came within 7% of each other, either way round).
#   FP32: depth 8 below 2^22 cells; 10 from 2048^2 (13-23% ahead of 8 at
#     2048^2-3072^2); 12 from 4096^2 (2^24 cells) up to 2^26 (3-15% ahead of
#     10 at 4096^2, 6144^2 and 7168^2, launches there being short enough for
#     their fixed start and finish to matter); 10 from 8192^2 up (7-8% ahead
#     of 12 at 8192^2, 12288^2 and 16384^2).
#   grids of at most 64 x 128 cells: the resident map, every sweep in one
#     launch (64^2 FP64, 32 sweeps: 17.6 us against 32 us for the depth-8
#     march; 16^2 x 8: 8.6 against 23; 64^2 x 1000: 0.44 against ~0.75 ms).
# Below 2^22 cells launches are latency bound and depths 6-8 come within
# about 10% of each other.
DIFFUSION = {"map": "temporal", "time_block": 10, "tile_rows": 0}
DIFFUSION_F32 = {"map": "temporal", "time_block": 10, "tile_rows": 0}
SMALL_GRID_CELLS = 1 << 24  # FP64 below this (FP32 below 2^22): depth 8
RESIDENT_MAX_NX, RESIDENT_MAX_NY = 64, 128

# Per-variable field kernels.
PACK = {"map": "tiled"}
FLUX = {"map": "tiled"}


def diffusion(dtype_name: str, nx: int | None = None, ny: int | None = None) -> dict:
    """Production diffusion settings for a dtype, and for a grid size if given."""
    f32 = dtype_name in ("f32", "float32")
    cfg = dict(DIFFUSION_F32 if f32 else DIFFUSION)
    if nx is not None and ny is not None:
        cells = nx * ny
        if nx <= RESIDENT_MAX_NX and ny <= RESIDENT_MAX_NY:
            cfg.update(map="resident", time_block=1)
        elif f32:
            if cells < 1 << 22:
                cfg["time_block"] = 8
            elif (1 << 24) <= cells < (1 << 26):
                cfg["time_block"] = 12
        elif cells < SMALL_GRID_CELLS:
            cfg["time_block"] = 8
    return cfg
