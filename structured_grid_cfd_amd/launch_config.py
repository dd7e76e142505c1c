"""Launch settings of the production path: the maps, time block and tile
shapes that the benchmark times and the full-size parity tests check."""

# Five-point diffusion: temporal blocking (8 sweeps per launch in FP64, 10 in
# FP32, the fastest depths measured on MI355X), automatic tile rows.
DIFFUSION = {"map": "temporal", "time_block": 8, "tile_rows": 0}
DIFFUSION_F32 = {"map": "temporal", "time_block": 10, "tile_rows": 0}

# Per-variable field kernels.
PACK = {"map": "tiled"}
FLUX = {"map": "tiled"}


def diffusion(dtype_name: str) -> dict:
    return dict(DIFFUSION_F32 if dtype_name in ("f32", "float32") else DIFFUSION)
