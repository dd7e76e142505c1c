"""Launch settings of the production path: the maps, time block and tile
shapes that the benchmark times and the full-size parity tests check."""

# Five-point diffusion: temporal blocking, 10 sweeps per launch, automatic
# tile rows.  Whole-workload timings on MI355X (1000 sweeps of 4096^2, 200 of
# 16384^2): FP64 depth 10 beat 8 by 2% and 11%, FP32 depth 10 beat 8 and 12.
DIFFUSION = {"map": "temporal", "time_block": 10, "tile_rows": 0}
DIFFUSION_F32 = {"map": "temporal", "time_block": 10, "tile_rows": 0}

# Per-variable field kernels.
PACK = {"map": "tiled"}
FLUX = {"map": "tiled"}


def diffusion(dtype_name: str) -> dict:
    return dict(DIFFUSION_F32 if dtype_name in ("f32", "float32") else DIFFUSION)
