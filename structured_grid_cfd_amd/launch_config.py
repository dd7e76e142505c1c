"""Launch settings of the production path: the maps, time block and tile
shapes that the benchmark times and the full-size parity tests check."""

# Five-point diffusion: temporal blocking, automatic tile rows.  The depth
# grows with the grid (whole-workload timings on MI355X, FP64): launches on
# grids below 4096^2 take depth 8, large ones depth 10.
#   below 2^24 cells: depth 8.  Small launches are latency bound (about 6 us
#     each whatever the depth up to ~512^2), so depths 6-8 trade launch count
#     against per-launch time and none wins everywhere (within 10% of each
#     other at 64^2-1024^2, 32-840 sweeps); at 1280^2-3072^2 depth 8 is best
#     or within 4%, and 5% ahead of 10 at 3072^2.
#   from 2^24 cells (4096^2) up: depth 10 (4096^2 1000 sweeps: ahead of 8 by
#     1-2% in FP64; 16384^2 FP32 200 sweeps: ahead of 8 and 12).
#   grids of at most 64 x 128 cells: the resident map, every sweep in one
#     launch (64^2 FP64, 32 sweeps: 17.6 us against 32 us for the depth-8
#     march; 16^2 x 8: 8.6 against 23; 64^2 x 1000: 0.44 against ~0.75 ms).
DIFFUSION = {"map": "temporal", "time_block": 10, "tile_rows": 0}
DIFFUSION_F32 = {"map": "temporal", "time_block": 10, "tile_rows": 0}
SMALL_GRID_CELLS = 1 << 24  # below this, depth 8
RESIDENT_MAX_NX, RESIDENT_MAX_NY = 64, 128

# Per-variable field kernels.
PACK = {"map": "tiled"}
FLUX = {"map": "tiled"}


def diffusion(dtype_name: str, nx: int | None = None, ny: int | None = None) -> dict:
    """Production diffusion settings for a dtype, and for a grid size if given."""
    cfg = dict(DIFFUSION_F32 if dtype_name in ("f32", "float32") else DIFFUSION)
    if nx is not None and ny is not None:
        if nx <= RESIDENT_MAX_NX and ny <= RESIDENT_MAX_NY:
            cfg.update(map="resident", time_block=1)
        elif nx * ny < SMALL_GRID_CELLS:
            cfg["time_block"] = 8
    return cfg
