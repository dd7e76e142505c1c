// sgc_internal.h -- shared declarations of the HIP kernel launchers behind
// the C ABI in include/sgc.h.  Internal to libsgc.so; gfx950 only.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <string>

#include "../../include/sgc.h"

namespace sgc {

// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const std::string &msg);

// Launch-status check after an enqueue: SGC_EHIP with the runtime's message.
int check_launch(const char *what);

// Resident workgroups of `kernel` per CU (for `block_threads`-thread
// workgroups) and the device's CU count, queried once per device and cached
// in `cache` (one cache per kernel).
constexpr int kMaxDevices = 64;
struct SlotCache {
    std::atomic<int> per_cu[kMaxDevices];
    std::atomic<int> cus[kMaxDevices];
};
int resident_slots(const void *kernel, int block_threads, SlotCache &cache, int *per_cu, int *cus);

// Workgroups are dealt to the 8 XCDs of the chip round-robin (block b runs on
// XCD b % 8).  This maps the hardware block index to a logical index such that
// each XCD receives one contiguous range of logical blocks, so neighbouring
// tiles, which share halo rows/columns and partial cache lines, meet in the
// same 4 MB L2.  A bijection on [0, nb).
__device__ __forceinline__ int xcd_remap(int b, int nb) {
    const int q = nb >> 3, r = nb & 7;
    const int x = b & 7, m = b >> 3;
    return x * q + (x < r ? x : r) + m;
}

// Raw buffer descriptors (gfx9 layout: 48-bit base, stride 0, byte range,
// config word 0x00020000).  Accesses are range-checked by the hardware
// against the descriptor: a load outside [0, bytes) returns 0 and a store
// outside it is dropped.  Kernels use this to mask elements without branching
// around memory instructions (branches there make the compiler wait for every
// outstanding load before continuing, serialising the memory pipeline).
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset no descriptor covers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// POL: cache policy bits of gfx950 buffer instructions (1 = sc0, 2 = nt:
// the line is not expected to be re-read, 16 = sc1).
template <int POL = 0>
__device__ __forceinline__ double buf_load_f64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
}
template <int POL = 0>
__device__ __forceinline__ void buf_store_f64(double x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, off, 0, POL);
}

// ---- diffusion (diffuse2d.hip) --------------------------------------------
struct DiffPlan {
    int nx, ny, ld;
    int time_block;  // TEMPORAL only
    int tile_rows;   // 0 = automatic
};
int diffuse_zero_ring(void *buf, int dtype, int nx, int ny, int ld, hipStream_t s);
// All `steps` steps of grids of at most 64 x 128 cells in one launch, one
// workgroup per field: field k's result in dst[k], the state one step earlier
// in prev[k] (SGC_ERANGE if larger).
struct ResidentFields {
    const void *src[SGC_MAX_NVAR];
    void *dst[SGC_MAX_NVAR];
    void *prev[SGC_MAX_NVAR];
};
int diffuse_resident_fields(const ResidentFields &f, int n, int dtype, const DiffPlan &p,
                            double alpha, int steps, hipStream_t s);
int diffuse_sweep(const void *src, void *dst, int dtype, const DiffPlan &p,
                  double alpha, int map, int steps_in_launch, hipStream_t s);
// Several fields of the same shape stepped in the same marching launches
// (maps TILED and TEMPORAL): field f reads src[f] and writes dst[f].
struct FieldPairs {
    const void *src[SGC_MAX_NVAR];
    void *dst[SGC_MAX_NVAR];
    int n;
};
int diffuse_sweep_fields(const FieldPairs &f, int dtype, const DiffPlan &p, double alpha, int map,
                         int steps_in_launch, hipStream_t s);

// ---- per-variable field kernels (field_pack.hip, flux_diff.hip) ------------
struct PtrTable {
    const double *p[SGC_MAX_NVAR];
};
int pack_launch(const PtrTable &fields, int nvar, int nx, int ny, int nz, int dir,
                double *out, int map, hipStream_t s);
int unpack_launch(const double *packed, int nvar, int nx, int ny, int nz, int dir,
                  const PtrTable &fields, int map, hipStream_t s);
// SSPRK stage fused with the flux difference: q' = a*q0 + b*(q + dt*rhs).
struct StageArgs {
    PtrTable q0, q, qout;  // qout entries are written (the table holds them const)
    double a, b, dt;
};
// rhs != nullptr: write the flux difference; st != nullptr: the stage instead.
int flux_launch(const PtrTable &fx, const PtrTable &fy, const PtrTable *fz,
                const double *dx, const double *dy, const double *dz, int nvar,
                int nx, int ny, int nz, double *rhs, const StageArgs *st, int map,
                hipStream_t s);

}  // namespace sgc
