// abi.hip -- the extern "C" entry points of libsgc.so (include/sgc.h):
// argument validation on the host before any enqueue, then dispatch to the
// HIP kernel launchers.  Allocates nothing and keeps no pointers.
#include <cmath>
#include <cstdio>
#include <string>

#include "sgc_internal.h"

namespace sgc {

namespace {
thread_local std::string g_last_error;

constexpr int64_t kMaxElems = 2147483647LL;  // 32-bit element indices in kernels

bool misaligned(const void *p, int64_t elem_bytes) {
    return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)elem_bytes) != 0;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

std::string fmt(const char *f, long long x) {
    char buf[256];
    std::snprintf(buf, sizeof buf, f, x);
    return buf;
}

int clear() {
    g_last_error.clear();
    return SGC_OK;
}

// Number of kernel launches, and the steps each fuses, for a TEMPORAL call:
// L = ceil(steps / T), bumped by one when its parity differs from the step
// count's, so that alternating launches u->v, v->u, ... end in v exactly when
// `steps` is odd; the steps are then spread as evenly as possible (each
// launch fuses at most T).  L never exceeds `steps`.
int64_t temporal_launches(int64_t steps, int64_t tb) {
    if (steps == 0) return 0;
    int64_t L = (steps + tb - 1) / tb;
    if ((L & 1) != (steps & 1)) L += 1;
    return L;
}
}  // namespace

int fail(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

int check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(SGC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return SGC_OK;
}

int resident_slots(const void *kernel, int block_threads, SlotCache &cache, int *per_cu, int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(SGC_EHIP, "hipGetDevice failed");
    if (dev >= 0 && dev < kMaxDevices) {
        const int p = cache.per_cu[dev].load(std::memory_order_relaxed);
        const int c = cache.cus[dev].load(std::memory_order_relaxed);
        if (p > 0 && c > 0) {
            *per_cu = p;
            *cus = c;
            return SGC_OK;
        }
    }
    int p = 0, c = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&p, kernel, block_threads, 0);
    if (e != hipSuccess) return fail(SGC_EHIP, std::string("occupancy query: ") + hipGetErrorString(e));
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(SGC_EHIP, std::string("CU count query: ") + hipGetErrorString(e));
    if (p < 1 || c < 1) return fail(SGC_EHIP, "a kernel cannot be resident on this device");
    if (dev >= 0 && dev < kMaxDevices) {
        cache.per_cu[dev].store(p, std::memory_order_relaxed);
        cache.cus[dev].store(c, std::memory_order_relaxed);
    }
    *per_cu = p;
    *cus = c;
    return SGC_OK;
}

}  // namespace sgc

using namespace sgc;

namespace {

int check_dims(const char *fn, int32_t nvar, int64_t nx, int64_t ny, int64_t nz) {
    if (nvar < 1 || nvar > SGC_MAX_NVAR)
        return fail(SGC_EINVAL, std::string(fn) + fmt(": nvar must be in 1..%lld", SGC_MAX_NVAR));
    if (nx < 1 || ny < 1 || nz < 1) return fail(SGC_EINVAL, std::string(fn) + ": nx, ny, nz must be >= 1");
    if (nx >= kMaxElems || ny >= kMaxElems || nz >= kMaxElems)
        return fail(SGC_ERANGE, std::string(fn) + ": an extent exceeds 2^31-2");
    return SGC_OK;
}

int check_table(const char *fn, const char *name, const double *const *tab, int32_t nvar) {
    if (tab == nullptr) return fail(SGC_ENULL, std::string(fn) + ": " + name + " table is NULL");
    for (int32_t k = 0; k < nvar; ++k) {
        if (tab[k] == nullptr)
            return fail(SGC_ENULL, std::string(fn) + ": " + name + fmt(" entry %lld is NULL", k));
        if (misaligned(tab[k], 8))
            return fail(SGC_EINVAL, std::string(fn) + ": " + name + fmt(" entry %lld is not 8-byte aligned", k));
    }
    return SGC_OK;
}

int check_ptr(const char *fn, const char *name, const double *p) {
    if (p == nullptr) return fail(SGC_ENULL, std::string(fn) + ": " + name + " is NULL");
    if (misaligned(p, 8)) return fail(SGC_EINVAL, std::string(fn) + ": " + name + " is not 8-byte aligned");
    return SGC_OK;
}

// Faces, spacings and extents of a flux call (the 2D form has fz == dz == NULL
// and nz == 1).
int check_flux_inputs(const char *fn, const double *const *fx, const double *const *fy,
                      const double *const *fz, const double *dx, const double *dy, const double *dz,
                      int32_t nvar, int64_t nx, int64_t ny, int64_t nz) {
    int rc;
    if ((rc = check_dims(fn, nvar, nx, ny, nz))) return rc;
    if ((rc = check_table(fn, "fx", fx, nvar))) return rc;
    if ((rc = check_table(fn, "fy", fy, nvar))) return rc;
    if (fz != nullptr && (rc = check_table(fn, "fz", fz, nvar))) return rc;
    if ((rc = check_ptr(fn, "dx", dx))) return rc;
    if ((rc = check_ptr(fn, "dy", dy))) return rc;
    if ((fz == nullptr) != (dz == nullptr))
        return fail(SGC_ENULL, std::string(fn) + ": fz and dz must both be given or both be NULL");
    if (dz != nullptr && (rc = check_ptr(fn, "dz", dz))) return rc;
    if (fz == nullptr && nz != 1) return fail(SGC_EINVAL, std::string(fn) + ": the 2D form (fz NULL) needs nz == 1");
    if ((nx + 1) * (ny + 1) > kMaxElems / (nz + 1) || nx * ny * nz > kMaxElems / nvar)
        return fail(SGC_ERANGE, std::string(fn) + ": an array exceeds 2^31-1 elements");
    return SGC_OK;
}

// An output region must not overlap any face or spacing array.
int check_output_vs_flux_inputs(const char *fn, const char *name, const void *out, int64_t obytes,
                                const double *const *fx, const double *const *fy, const double *const *fz,
                                const double *dx, const double *dy, const double *dz, int32_t nvar,
                                int64_t nx, int64_t ny, int64_t nz) {
    const int64_t nfx = (nx + 1) * ny * nz, nfy = nx * (ny + 1) * nz, nfz = nx * ny * (nz + 1);
    for (int32_t k = 0; k < nvar; ++k) {
        if (overlaps(out, obytes, fx[k], nfx * 8)) return fail(SGC_EALIAS, std::string(fn) + ": " + name + " overlaps fx");
        if (overlaps(out, obytes, fy[k], nfy * 8)) return fail(SGC_EALIAS, std::string(fn) + ": " + name + " overlaps fy");
        if (fz && overlaps(out, obytes, fz[k], nfz * 8))
            return fail(SGC_EALIAS, std::string(fn) + ": " + name + " overlaps fz");
    }
    if (overlaps(out, obytes, dx, nx * 8) || overlaps(out, obytes, dy, ny * 8) ||
        (dz && overlaps(out, obytes, dz, nz * 8)))
        return fail(SGC_EALIAS, std::string(fn) + ": " + name + " overlaps a spacing array");
    return SGC_OK;
}

void flux_tables(const double *const *fx, const double *const *fy, const double *const *fz, int32_t nvar,
                 PtrTable &tx, PtrTable &ty, PtrTable &tz) {
    for (int32_t k = 0; k < nvar; ++k) {
        tx.p[k] = fx[k];
        ty.p[k] = fy[k];
        if (fz) tz.p[k] = fz[k];
    }
}

// The scalar arguments every diffusion entry point shares, with `fn` naming
// the entry point in the messages.
int check_diffusion_args(const char *fn, int32_t dtype, int64_t nx, int64_t ny, int64_t ld,
                         double alpha, int64_t steps, int32_t map, int32_t time_block,
                         int32_t tile_rows) {
    const std::string f(fn);
    if (dtype != SGC_F32 && dtype != SGC_F64)
        return fail(SGC_EDTYPE, f + fmt(": unknown dtype %lld", dtype));
    if (nx < 3 || ny < 3) return fail(SGC_EINVAL, f + ": nx and ny must be >= 3");
    if (ld < nx) return fail(SGC_EINVAL, f + ": ld must be >= nx");
    if (steps < 0) return fail(SGC_EINVAL, f + ": steps must be >= 0");
    if (!std::isfinite(alpha)) return fail(SGC_EINVAL, f + ": alpha must be finite");
    if (map < SGC_DIFF_COLLAPSE_BRANCH || map > SGC_DIFF_RESIDENT)
        return fail(SGC_EINVAL, f + fmt(": unknown map %lld", map));
    if (map == SGC_DIFF_TEMPORAL) {
        if (time_block < 1) return fail(SGC_EINVAL, f + ": time_block must be >= 1");
        if (time_block > SGC_MAX_TIME_BLOCK)
            return fail(SGC_ERANGE, f + fmt(": time_block above %lld", SGC_MAX_TIME_BLOCK));
    }
    if (map == SGC_DIFF_TILED || map == SGC_DIFF_TEMPORAL) {
        if (tile_rows < 0 || tile_rows > ny)
            return fail(SGC_EINVAL, f + ": tile_rows must be 0 (auto) or 1..ny");
    }
    if (ld > kMaxElems / ny) return fail(SGC_ERANGE, f + ": ld*ny exceeds 2^31-1 elements");
    return SGC_OK;
}

// The march's launch sequence for `steps` sweeps of the fields in `fwd`
// (u -> v; `back` is v -> u): TILED takes one sweep per launch, TEMPORAL the
// launch schedule of temporal_launches (the steps spread evenly, an even or
// odd launch count so that the result lands in v iff steps is odd).  The
// march treats the edge ring as 0 on read and writes it as 0.
int march_steps(const FieldPairs &fwd, const FieldPairs &back, int32_t dtype, const DiffPlan &p,
                double alpha, int64_t steps, int32_t map, int32_t time_block, hipStream_t s) {
    int rc = SGC_OK;
    if (map == SGC_DIFF_TILED) {
        for (int64_t k = 1; k <= steps; ++k)
            if ((rc = diffuse_sweep_fields((k & 1) ? fwd : back, dtype, p, alpha, map, 1, s))) return rc;
        return SGC_OK;
    }
    const int64_t L = temporal_launches(steps, time_block);
    const int64_t base = steps / L, extra = steps % L;
    for (int64_t k = 0; k < L; ++k) {
        const int ts = (int)(base + (k < extra ? 1 : 0));
        if ((rc = diffuse_sweep_fields((k & 1) == 0 ? fwd : back, dtype, p, alpha, map, ts, s))) return rc;
    }
    return SGC_OK;
}

// The resident map for the fields (u[k], v[k]): one workgroup per field, all
// steps in one launch; the result lands in v iff steps is odd and the other
// buffer ends one step earlier.
int resident_steps(void *const *u, void *const *v, int32_t n, int32_t dtype, const DiffPlan &p,
                   double alpha, int64_t steps, hipStream_t s) {
    const bool odd = (steps & 1) != 0;
    ResidentFields r{};
    for (int32_t k = 0; k < n; ++k) {
        r.src[k] = u[k];
        r.dst[k] = odd ? v[k] : u[k];
        r.prev[k] = odd ? u[k] : v[k];
    }
    return diffuse_resident_fields(r, n, dtype, p, alpha, (int)steps, s);
}

}  // namespace

extern "C" {

const char *sgc_last_error(void) { return g_last_error.c_str(); }

int32_t sgc_abi_version(void) { return SGC_ABI_VERSION; }

int64_t stencil_diffuse2d_launches(int64_t steps, int32_t map, int32_t time_block) {
    if (steps < 0) return -1;
    switch (map) {
    case SGC_DIFF_COLLAPSE_BRANCH:
    case SGC_DIFF_CONTIG:
    case SGC_DIFF_STRIDED:
    case SGC_DIFF_TILED:
        return steps;
    case SGC_DIFF_TEMPORAL:
        if (time_block < 1 || time_block > SGC_MAX_TIME_BLOCK) return -1;
        return temporal_launches(steps, time_block);
    case SGC_DIFF_RESIDENT:
        return steps > 0 ? 1 : 0;
    default:
        return -1;
    }
}

int stencil_diffuse2d_ex(void *u, void *v, int32_t dtype, int64_t nx, int64_t ny, int64_t ld,
                         double alpha, int64_t steps, int32_t map, int32_t time_block,
                         int32_t tile_rows, void *stream, int32_t *result_is_v) {
    clear();
    if (u == nullptr || v == nullptr) return fail(SGC_ENULL, "stencil_diffuse2d: u and v must be non-NULL");
    int rc = check_diffusion_args("stencil_diffuse2d", dtype, nx, ny, ld, alpha, steps, map, time_block,
                                  tile_rows);
    if (rc) return rc;
    const int64_t es = dtype == SGC_F64 ? 8 : 4;
    const int64_t bytes = ld * ny * es;
    if (misaligned(u, es) || misaligned(v, es))
        return fail(SGC_EINVAL, "stencil_diffuse2d: u and v must be aligned to their element size");
    if (overlaps(u, bytes, v, bytes)) return fail(SGC_EALIAS, "stencil_diffuse2d: u and v overlap");

    hipStream_t s = static_cast<hipStream_t>(stream);
    DiffPlan p{(int)nx, (int)ny, (int)ld, time_block, tile_rows};
    if (steps == 0) {
        rc = diffuse_zero_ring(u, dtype, p.nx, p.ny, p.ld, s);
        if (rc) return rc;
    } else if (map == SGC_DIFF_COLLAPSE_BRANCH || map == SGC_DIFF_CONTIG || map == SGC_DIFF_STRIDED) {
        // The page layouts read the edge ring as the Dirichlet value: start
        // from zero rings in both buffers, as the pages' initial condition does.
        if ((rc = diffuse_zero_ring(u, dtype, p.nx, p.ny, p.ld, s))) return rc;
        if ((rc = diffuse_zero_ring(v, dtype, p.nx, p.ny, p.ld, s))) return rc;
        for (int64_t k = 1; k <= steps; ++k) {
            const bool odd = (k & 1) != 0;
            rc = diffuse_sweep(odd ? u : v, odd ? v : u, dtype, p, alpha, map, 1, s);
            if (rc) return rc;
        }
    } else if (map == SGC_DIFF_RESIDENT) {
        if (steps > 0x7fffffffLL) return fail(SGC_ERANGE, "stencil_diffuse2d: resident sweep takes at most 2^31-1 steps");
        if ((rc = resident_steps(&u, &v, 1, dtype, p, alpha, steps, s))) return rc;
    } else {  // TILED, TEMPORAL
        FieldPairs fwd{}, back{};
        fwd.n = back.n = 1;
        fwd.src[0] = u;
        fwd.dst[0] = v;
        back.src[0] = v;
        back.dst[0] = u;
        if ((rc = march_steps(fwd, back, dtype, p, alpha, steps, map, time_block, s))) return rc;
    }
    if (result_is_v) *result_is_v = (int32_t)(steps & 1);
    return SGC_OK;
}

// The automatic tile height of the marching maps.
int stencil_diffuse2d(void *u, void *v, int32_t dtype, int64_t nx, int64_t ny, int64_t ld,
                      double alpha, int64_t steps, int32_t map, int32_t time_block, void *stream,
                      int32_t *result_is_v) {
    return stencil_diffuse2d_ex(u, v, dtype, nx, ny, ld, alpha, steps, map, time_block, 0, stream,
                                result_is_v);
}

int stencil_diffuse2d_fields(void *const *u, void *const *v, int32_t nvar, int32_t dtype, int64_t nx,
                             int64_t ny, int64_t ld, double alpha, int64_t steps, int32_t map,
                             int32_t time_block, int32_t tile_rows, void *stream,
                             int32_t *result_is_v) {
    clear();
    const char *fn = "stencil_diffuse2d_fields";
    if (u == nullptr || v == nullptr)
        return fail(SGC_ENULL, "stencil_diffuse2d_fields: the u and v tables must be non-NULL");
    if (nvar < 1 || nvar > SGC_MAX_NVAR)
        return fail(SGC_EINVAL, fmt("stencil_diffuse2d_fields: nvar must be 1..%lld", SGC_MAX_NVAR));
    int rc = check_diffusion_args(fn, dtype, nx, ny, ld, alpha, steps, map, time_block, tile_rows);
    if (rc) return rc;
    if (map != SGC_DIFF_TILED && map != SGC_DIFF_TEMPORAL && map != SGC_DIFF_RESIDENT)
        return fail(SGC_EINVAL,
                    "stencil_diffuse2d_fields: map must be SGC_DIFF_TILED, SGC_DIFF_TEMPORAL or SGC_DIFF_RESIDENT");
    if (map == SGC_DIFF_RESIDENT && (nx > 64 || ny > 128))
        return fail(SGC_ERANGE, "stencil_diffuse2d_fields: the resident map takes grids of at most 64 columns and 128 rows");
    if (map == SGC_DIFF_RESIDENT && steps > 0x7fffffffLL)
        return fail(SGC_ERANGE, "stencil_diffuse2d_fields: the resident map takes at most 2^31-1 steps");
    const int64_t es = dtype == SGC_F64 ? 8 : 4;
    const int64_t bytes = ld * ny * es;
    for (int32_t k = 0; k < nvar; ++k) {
        if (u[k] == nullptr || v[k] == nullptr)
            return fail(SGC_ENULL, fmt("stencil_diffuse2d_fields: u or v entry %lld is NULL", k));
        if (misaligned(u[k], es) || misaligned(v[k], es))
            return fail(SGC_EINVAL, fmt("stencil_diffuse2d_fields: field %lld is not aligned to its element size", k));
    }
    // No two of the 2*nvar buffers may overlap.
    for (int32_t a = 0; a < 2 * nvar; ++a) {
        const void *pa = a < nvar ? u[a] : v[a - nvar];
        for (int32_t b = a + 1; b < 2 * nvar; ++b) {
            const void *pb = b < nvar ? u[b] : v[b - nvar];
            if (overlaps(pa, bytes, pb, bytes))
                return fail(SGC_EALIAS, fmt("stencil_diffuse2d_fields: buffer %lld", a) + fmt(" overlaps buffer %lld (u entries first, then v)", b));
        }
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    DiffPlan p{(int)nx, (int)ny, (int)ld, time_block, tile_rows};
    FieldPairs fwd{}, back{};
    fwd.n = back.n = nvar;
    for (int32_t k = 0; k < nvar; ++k) {
        fwd.src[k] = u[k];
        fwd.dst[k] = v[k];
        back.src[k] = v[k];
        back.dst[k] = u[k];
    }
    if (steps == 0) {
        for (int32_t k = 0; k < nvar; ++k)
            if ((rc = diffuse_zero_ring(u[k], dtype, p.nx, p.ny, p.ld, s))) return rc;
    } else if (map == SGC_DIFF_RESIDENT) {
        if ((rc = resident_steps(u, v, nvar, dtype, p, alpha, steps, s))) return rc;
    } else {  // TILED, TEMPORAL
        if ((rc = march_steps(fwd, back, dtype, p, alpha, steps, map, time_block, s))) return rc;
    }
    if (result_is_v) *result_is_v = (int32_t)(steps & 1);
    return SGC_OK;
}

int field_pack(const double *const *fields, int32_t nvar, int64_t nx, int64_t ny, int64_t nz,
               int32_t dir, double *out, int32_t map, void *stream) {
    clear();
    int rc;
    if ((rc = check_dims("field_pack", nvar, nx, ny, nz))) return rc;
    if ((rc = check_table("field_pack", "fields", fields, nvar))) return rc;
    if ((rc = check_ptr("field_pack", "out", out))) return rc;
    if (dir < SGC_DIR_X || dir > SGC_DIR_Z) return fail(SGC_EINVAL, "field_pack: dir must be 0, 1 or 2");
    if (map < SGC_VAR_PER_CELL || map > SGC_VAR_TILED) return fail(SGC_EINVAL, "field_pack: unknown map");
    if (nx * ny > kMaxElems / nz || nx * ny * nz > kMaxElems / nvar)
        return fail(SGC_ERANGE, "field_pack: nvar*nx*ny*nz exceeds 2^31-1 elements");
    const int64_t n = nx * ny * nz;
    for (int32_t k = 0; k < nvar; ++k)
        if (overlaps(out, n * nvar * 8, fields[k], n * 8))
            return fail(SGC_EALIAS, fmt("field_pack: out overlaps field %lld", k));
    PtrTable t{};
    for (int32_t k = 0; k < nvar; ++k) t.p[k] = fields[k];
    return pack_launch(t, nvar, (int)nx, (int)ny, (int)nz, dir, out, map, static_cast<hipStream_t>(stream));
}

int field_unpack(const double *packed, int32_t nvar, int64_t nx, int64_t ny, int64_t nz, int32_t dir,
                 double *const *fields, int32_t map, void *stream) {
    clear();
    int rc;
    if ((rc = check_dims("field_unpack", nvar, nx, ny, nz))) return rc;
    if ((rc = check_ptr("field_unpack", "packed", packed))) return rc;
    if ((rc = check_table("field_unpack", "fields", fields, nvar))) return rc;
    if (dir < SGC_DIR_X || dir > SGC_DIR_Z) return fail(SGC_EINVAL, "field_unpack: dir must be 0, 1 or 2");
    if (map < SGC_VAR_PER_CELL || map > SGC_VAR_TILED) return fail(SGC_EINVAL, "field_unpack: unknown map");
    if (nx * ny > kMaxElems / nz || nx * ny * nz > kMaxElems / nvar)
        return fail(SGC_ERANGE, "field_unpack: nvar*nx*ny*nz exceeds 2^31-1 elements");
    const int64_t n = nx * ny * nz;
    for (int32_t k = 0; k < nvar; ++k) {
        if (overlaps(packed, n * nvar * 8, fields[k], n * 8))
            return fail(SGC_EALIAS, fmt("field_unpack: field %lld overlaps packed", k));
        for (int32_t m = 0; m < k; ++m)
            if (overlaps(fields[m], n * 8, fields[k], n * 8))
                return fail(SGC_EALIAS, fmt("field_unpack: field %lld overlaps an earlier field", k));
    }
    PtrTable t{};
    for (int32_t k = 0; k < nvar; ++k) t.p[k] = fields[k];
    return unpack_launch(packed, nvar, (int)nx, (int)ny, (int)nz, dir, t, map,
                         static_cast<hipStream_t>(stream));
}

int flux_diff3d(const double *const *fx, const double *const *fy, const double *const *fz,
                const double *dx, const double *dy, const double *dz, int32_t nvar, int64_t nx,
                int64_t ny, int64_t nz, double *rhs, int32_t map, void *stream) {
    clear();
    int rc;
    if ((rc = check_flux_inputs("flux_diff3d", fx, fy, fz, dx, dy, dz, nvar, nx, ny, nz))) return rc;
    if ((rc = check_ptr("flux_diff3d", "rhs", rhs))) return rc;
    if (map < SGC_VAR_PER_CELL || map > SGC_VAR_TILED) return fail(SGC_EINVAL, "flux_diff3d: unknown map");
    const int64_t n = nx * ny * nz;
    if ((rc = check_output_vs_flux_inputs("flux_diff3d", "rhs", rhs, n * nvar * 8, fx, fy, fz, dx, dy, dz,
                                          nvar, nx, ny, nz)))
        return rc;
    PtrTable tx{}, ty{}, tz{};
    flux_tables(fx, fy, fz, nvar, tx, ty, tz);
    return flux_launch(tx, ty, fz ? &tz : nullptr, dx, dy, dz, nvar, (int)nx, (int)ny, (int)nz, rhs,
                       nullptr, map, static_cast<hipStream_t>(stream));
}

int flux_stage3d(const double *const *fx, const double *const *fy, const double *const *fz,
                 const double *dx, const double *dy, const double *dz, const double *const *q0,
                 const double *const *q, double a, double b, double dt, int32_t nvar, int64_t nx,
                 int64_t ny, int64_t nz, double *const *qout, int32_t map, void *stream) {
    clear();
    int rc;
    if ((rc = check_flux_inputs("flux_stage3d", fx, fy, fz, dx, dy, dz, nvar, nx, ny, nz))) return rc;
    if ((rc = check_table("flux_stage3d", "q0", q0, nvar))) return rc;
    if ((rc = check_table("flux_stage3d", "q", q, nvar))) return rc;
    if ((rc = check_table("flux_stage3d", "qout", qout, nvar))) return rc;
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(dt))
        return fail(SGC_EINVAL, "flux_stage3d: a, b and dt must be finite");
    if (map < SGC_VAR_PER_CELL || map > SGC_VAR_TILED) return fail(SGC_EINVAL, "flux_stage3d: unknown map");
    const int64_t fb = nx * ny * nz * 8;  // bytes per field
    for (int32_t k = 0; k < nvar; ++k) {
        if ((rc = check_output_vs_flux_inputs("flux_stage3d", "qout", qout[k], fb, fx, fy, fz, dx, dy, dz,
                                              nvar, nx, ny, nz)))
            return rc;
        for (int32_t m = 0; m < nvar; ++m) {
            if (m != k && overlaps(qout[k], fb, qout[m], fb))
                return fail(SGC_EALIAS, "flux_stage3d: two qout fields overlap");
            // q' may replace q or q0 of its own variable in place, nothing else
            const bool same_var = m == k;
            if (overlaps(qout[k], fb, q[m], fb) && !(same_var && qout[k] == q[m]))
                return fail(SGC_EALIAS, "flux_stage3d: qout overlaps a q field other than its own");
            if (overlaps(qout[k], fb, q0[m], fb) && !(same_var && qout[k] == q0[m]))
                return fail(SGC_EALIAS, "flux_stage3d: qout overlaps a q0 field other than its own");
        }
    }
    PtrTable tx{}, ty{}, tz{};
    flux_tables(fx, fy, fz, nvar, tx, ty, tz);
    StageArgs st{};
    for (int32_t k = 0; k < nvar; ++k) {
        st.q0.p[k] = q0[k];
        st.q.p[k] = q[k];
        st.qout.p[k] = qout[k];
    }
    st.a = a;
    st.b = b;
    st.dt = dt;
    return flux_launch(tx, ty, fz ? &tz : nullptr, dx, dy, dz, nvar, (int)nx, (int)ny, (int)nz, nullptr,
                       &st, map, static_cast<hipStream_t>(stream));
}

}  // extern "C"
