/*
 * sgc.h -- C ABI of libsgc.so: structured-grid stencil sweeps on AMD MI355X
 * (gfx950), hand-written HIP kernels behind plain C entry points.
 *
 * Every entry point:
 *   - takes plain device pointers (memory the caller allocated on the current
 *     HIP device, e.g. torch tensors' data_ptr()), host integers and a HIP
 *     stream passed as `void *` (a hipStream_t; NULL = the null stream);
 *   - validates every argument on the host BEFORE enqueuing anything, so an
 *     error return leaves every buffer untouched;
 *   - only enqueues work on `stream` and returns; results are valid once the
 *     caller synchronises that stream;
 *   - allocates nothing and keeps no pointer after it returns (the caller owns
 *     all memory); host pointer tables are copied into the kernel arguments;
 *   - returns SGC_OK (0) or an sgc_status code, with a message available from
 *     sgc_last_error() on the calling thread.  Faults during execution surface
 *     at the caller's synchronisation.  The library never aborts.
 *
 * Indices are 32-bit inside the kernels: every array an entry point touches
 * must hold at most 2^31 - 1 elements (SGC_ERANGE otherwise).
 *
 * Pages defining the operations (cited by title and section):
 *   [Q3]  Qiita, "Fortran 2018でGPUを高速化する Part 3 - GPUカーネルのメモリ
 *         アクセスとFP32・FP64を比較する".
 *   [MFC] MFC pull request 2087, "SCC26: Collapse only spatial loops in
 *         per-variable GPU kernels".
 */
#ifndef SGC_H
#define SGC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI are the only ones libsgc.so exports. */
#define SGC_API __attribute__((visibility("default")))

#define SGC_ABI_VERSION 1
#define SGC_MAX_NVAR 32        /* variables per call (pointer tables by value) */
#define SGC_MAX_TIME_BLOCK 12  /* steps fused per launch by SGC_DIFF_TEMPORAL  */

typedef enum sgc_status {
    SGC_OK = 0,
    SGC_EINVAL = 1, /* a size, mode or value is outside its documented range */
    SGC_ENULL = 2,  /* a required pointer (or pointer-table entry) is NULL   */
    SGC_EDTYPE = 3, /* unknown dtype code                                    */
    SGC_EALIAS = 4, /* an output overlaps an input or the other buffer       */
    SGC_ERANGE = 5, /* an array exceeds 2^31 - 1 elements, time_block > max, or
                       a row too long for the marching maps (see below)         */
    SGC_EHIP = 6    /* the HIP runtime refused a launch (message has details) */
} sgc_status;

typedef enum sgc_dtype { SGC_F32 = 0, SGC_F64 = 1 } sgc_dtype;

/* Thread mappings of the five-point sweep.  The first three are the loop
 * layouts [Q3] section 5 compares; the last two are this library's own. */
typedef enum sgc_diff_map {
    SGC_DIFF_COLLAPSE_BRANCH = 0, /* one thread per cell of the flattened grid,
                                     edge cells written 0 by a branch ([Q3] 5.1) */
    SGC_DIFF_CONTIG = 1,          /* workgroup per row j, lanes along i,
                                     interior only ([Q3] 5.2)                   */
    SGC_DIFF_STRIDED = 2,         /* workgroup per column i, lanes along j,
                                     interior only ([Q3] 5.3)                   */
    SGC_DIFF_TILED = 3,           /* one step per launch: each wave marches a
                                     column strip along j with 16-byte row loads
                                     and a three-row register window            */
    SGC_DIFF_TEMPORAL = 4,        /* time_block steps per launch: the march
                                     keeps one window per time level and
                                     recomputes the halo, one HBM read and
                                     write per launch                           */
    SGC_DIFF_RESIDENT = 5         /* small grids (nx <= 64, ny <= 128): one
                                     workgroup holds the grid in registers and
                                     runs every step in a single launch         */
} sgc_diff_map;

/* Variable-loop mappings of the per-variable field kernels ([MFC] Changes and
 * "Why this is faster"). */
typedef enum sgc_var_map {
    SGC_VAR_PER_CELL = 0,    /* one thread per cell, spatial index math once,
                                variables in a loop inside the thread        */
    SGC_VAR_PER_CELLVAR = 1, /* one thread per (variable, cell): the flattened
                                four-level index decomposed per thread       */
    SGC_VAR_TILED = 2        /* this library's own: 16-byte streaming copies,
                                LDS-tiled transposes, plane-marching pencils */
} sgc_var_map;

typedef enum sgc_dir { SGC_DIR_X = 0, SGC_DIR_Y = 1, SGC_DIR_Z = 2 } sgc_dir;

/*
 * stencil_diffuse2d -- explicit 2D five-point diffusion with u/v alternation
 * ([Q3] section 3: v(i,j) = u(i,j) + alpha*(u(i-1,j) + u(i+1,j) + u(i,j-1) +
 * u(i,j+1) - 4*u(i,j)), edges fixed at 0; section 5.4: odd steps read u and
 * write v, even steps read v and write u).
 *
 *   u, v        device buffers of ld*ny elements of `dtype` each, column-major
 *               (element (i, j), 0-based, at [i + ld*j]); must not overlap.
 *               u holds the initial field.  Both are read and written.
 *   dtype       SGC_F32 or SGC_F64 (the arithmetic precision too).
 *   nx, ny      grid extents, each >= 3.  ld >= nx is the leading dimension;
 *               columns [nx, ld) are never read or written.
 *   alpha       finite; rounded once to `dtype`.  alpha <= 1/4 keeps the update
 *               a convex combination but is not required.
 *   steps       >= 0.  0 only zeroes u's edge ring (the result is u).
 *   map         an sgc_diff_map.
 *   time_block  steps fused per launch for SGC_DIFF_TEMPORAL, 1 ..
 *               SGC_MAX_TIME_BLOCK (SGC_ERANGE above); ignored by other maps.
 *   stream      hipStream_t or NULL.
 *   result_is_v optional out (host): 1 if the result is in v, 0 if in u.
 *
 * The marching maps (SGC_DIFF_TILED, SGC_DIFF_TEMPORAL) choose their tile
 * height automatically here (stencil_diffuse2d_ex takes it explicitly).  They
 * address each wave's rows through a window of 2^30 bytes, so where a single
 * tile row would not fit (rows of ~45 MB or more) they return SGC_ERANGE
 * before enqueueing anything, and the page maps still apply.
 *
 * SGC_DIFF_RESIDENT returns SGC_ERANGE for grids wider than 64 or taller
 * than 128 cells, or for more than 2^31 - 1 steps, before enqueueing
 * anything; it leaves the state one step before the result in the other
 * buffer.
 *
 * Semantics: the edge ring (i = 0, nx-1 or j = 0, ny-1) is treated as 0 in
 * both buffers whatever the caller stored there, and the result buffer's ring
 * holds zeros on return.  The result is in v if `steps` is odd, in u if even,
 * for every map.  The other buffer holds an unspecified earlier state.  Each
 * interior cell is computed as c + alpha*((((W + E) + S) + N) - 4*c) with one
 * rounding per operation, so all maps return the same bits.  (The marching
 * and resident maps form t - 4*c with a fused multiply-add only where that
 * rounds exactly like the separate subtraction, i.e. while 4*c is finite;
 * see diffuse2d.hip.)
 */
SGC_API int stencil_diffuse2d(void *u, void *v, int32_t dtype, int64_t nx, int64_t ny,
                              int64_t ld, double alpha, int64_t steps, int32_t map,
                              int32_t time_block, void *stream, int32_t *result_is_v);

/*
 * stencil_diffuse2d_ex -- stencil_diffuse2d with the marching maps' tile
 * height given by the caller (the same operation, results and errors; the
 * tile height changes only how the work is split into waves):
 *
 *   tile_rows   rows per wave tile for SGC_DIFF_TILED / SGC_DIFF_TEMPORAL;
 *               0 chooses automatically (what stencil_diffuse2d does);
 *               otherwise 1 .. ny (SGC_EINVAL outside 0 .. ny).  Ignored by
 *               the other maps.  Tiles are at most
 *               2^30 / (ld * element size) - 2*time_block - 8 rows (larger
 *               values are clamped to that).
 */
SGC_API int stencil_diffuse2d_ex(void *u, void *v, int32_t dtype, int64_t nx, int64_t ny,
                                 int64_t ld, double alpha, int64_t steps, int32_t map,
                                 int32_t time_block, int32_t tile_rows, void *stream,
                                 int32_t *result_is_v);

/*
 * stencil_diffuse2d_fields -- the same sweeps applied to nvar independent
 * fields of one shape in the same marching launches.  Field f is stepped
 * exactly as stencil_diffuse2d(u[f], v[f], ...) would step it, bit for bit;
 * the fields only share the launches (their tiles run side by side, so a
 * small grid with several fields pays each launch's latency once).  [Mallard]
 * "Design: single-GPU performance and parallel scaling", the reacting-flow
 * changes: stencil kernels take all variables in one pass over the stencil;
 * here all fields share each launch.
 *
 *   u, v        host arrays of nvar device buffers; each buffer as u / v of
 *               stencil_diffuse2d (ld*ny elements of `dtype`).  No two of the
 *               2*nvar buffers may overlap (SGC_EALIAS).
 *   nvar        1 .. SGC_MAX_NVAR.
 *   map         SGC_DIFF_TILED, SGC_DIFF_TEMPORAL or SGC_DIFF_RESIDENT
 *               (SGC_EINVAL otherwise); RESIDENT runs one workgroup per field
 *               with stencil_diffuse2d's limits (SGC_ERANGE beyond them) and
 *               leaves each field's state one step earlier in its other buffer.
 *   the rest    as stencil_diffuse2d, for every field; the result is in
 *               v[f] for every f if `steps` is odd, in u[f] if even.
 * Errors are detected before anything is enqueued, as for stencil_diffuse2d.
 */
SGC_API int stencil_diffuse2d_fields(void *const *u, void *const *v, int32_t nvar, int32_t dtype,
                                     int64_t nx, int64_t ny, int64_t ld, double alpha,
                                     int64_t steps, int32_t map, int32_t time_block,
                                     int32_t tile_rows, void *stream, int32_t *result_is_v);

/*
 * stencil_diffuse2d_launches -- number of sweep-kernel launches a
 * stencil_diffuse2d call with these arguments enqueues (not counting the
 * one-off edge-ring initialisation of the interior-only page maps), or -1 if
 * the arguments are invalid.  Host-only; touches no device.
 */
SGC_API int64_t stencil_diffuse2d_launches(int64_t steps, int32_t map,
                                   int32_t time_block);

/*
 * field_pack -- directional pack of nvar SoA fields ([MFC] Changes: the WENO
 * input pack v_rs_weno(j,k,l,i) = v_vf(i)%sf(j,k,l); the y and z orders
 * transpose the first index with the second or third).
 *
 *   fields  HOST array of nvar DEVICE pointers; field v holds nx*ny*nz
 *           doubles, column-major f(j,k,l) at [j + nx*(k + ny*l)].
 *   nvar    1 .. SGC_MAX_NVAR.   nx, ny, nz >= 1.
 *   dir     SGC_DIR_X: out(j,k,l,v) dims (nx,ny,nz,nvar)
 *           SGC_DIR_Y: out(k,j,l,v) dims (ny,nx,nz,nvar)
 *           SGC_DIR_Z: out(l,k,j,v) dims (nz,ny,nx,nvar), first index fastest.
 *   out     device, nvar*nx*ny*nz doubles; must not overlap any field.
 *   map     an sgc_var_map.
 * A bit copy: every map returns identical bytes.
 */
SGC_API int field_pack(const double *const *fields, int32_t nvar, int64_t nx,
               int64_t ny, int64_t nz, int32_t dir, double *out, int32_t map,
               void *stream);

/*
 * field_unpack -- inverse of field_pack: the directional copies from the
 * packed layout back into the nvar fields ([MFC] Changes: the directional
 * flux copies of the Riemann-solver finalisation).  Arguments as field_pack
 * with the roles of input and output exchanged: `packed` (device, read) and
 * `fields` (HOST array of nvar DEVICE pointers, written; must not overlap
 * `packed` or each other).
 */
SGC_API int field_unpack(const double *packed, int32_t nvar, int64_t nx, int64_t ny,
                 int64_t nz, int32_t dir, double *const *fields, int32_t map,
                 void *stream);

/*
 * flux_diff3d -- conservative flux difference ([MFC] Changes: the x/y/z flux
 * differences, with the inverse grid spacing formed outside the variable
 * loop):
 *   rhs(j,k,l,v) = ((Fx(j) - Fx(j+1))*(1/dx[j]) + (Fy(k) - Fy(k+1))*(1/dy[k]))
 *                  + (Fz(l) - Fz(l+1))*(1/dz[l])
 * summed in that order, each reciprocal a correctly rounded FP64 division.
 *
 *   fx, fy, fz  HOST arrays of nvar DEVICE pointers to per-variable face
 *               arrays, column-major: Fx (nx+1,ny,nz), Fy (nx,ny+1,nz),
 *               Fz (nx,ny,nz+1).  fz == NULL selects the 2D form: nz must be
 *               1, there is no z term and dz must be NULL too.
 *   dx, dy, dz  device cell widths, nx / ny / nz doubles.
 *   nvar        1 .. SGC_MAX_NVAR.   nx, ny, nz >= 1, with (nx+1)(ny+1)(nz+1)
 *               (a bound on every face array) and nvar*nx*ny*nz at most
 *               2^31 - 1 (SGC_ERANGE otherwise).
 *   rhs         device, (nx,ny,nz,nvar) doubles, j fastest; must not overlap
 *               any input.
 *   map         an sgc_var_map.
 * Every map returns identical bits.
 */
SGC_API int flux_diff3d(const double *const *fx, const double *const *fy,
                const double *const *fz, const double *dx, const double *dy,
                const double *dz, int32_t nvar, int64_t nx, int64_t ny,
                int64_t nz, double *rhs, int32_t map, void *stream);

/*
 * flux_stage3d -- one SSPRK stage fused with the flux difference (Mallard
 * documentation, "Design: single-GPU performance and parallel scaling":
 * Hardware and method -- time steps are SSPRK3, three stages -- and the
 * Baseline tables, where each stage computes a right-hand side and applies
 * an axpby update).  The pages give no stage formula; this is the Shu-Osher
 * form, per cell and variable
 *   q'(j,k,l,v) = a*q0 + b*(q + dt*rhs)
 * with rhs exactly as flux_diff3d computes it, evaluated t = dt*rhs;
 * t = q + t; t = b*t; s = a*q0; q' = s + t (one rounding each).  SSPRK3 uses
 * (a, b) = (0, 1), (3/4, 1/4), (1/3, 2/3).  rhs is never stored.
 *
 *   fx .. dz, nvar, nx, ny, nz   as flux_diff3d.
 *   q0, q       HOST arrays of nvar DEVICE pointers, each field nx*ny*nz
 *               doubles, j fastest (the stage's base state and its input).
 *   a, b, dt    finite.
 *   qout        HOST array of nvar DEVICE pointers, written.  qout[v] may be
 *               the same pointer as q[v] or q0[v] (updated in place); it must
 *               not otherwise overlap any input or another output.
 *   map         an sgc_var_map.
 * Every map returns identical bits.  Errors as flux_diff3d (SGC_EALIAS for a
 * disallowed overlap), all before anything is enqueued.
 */
SGC_API int flux_stage3d(const double *const *fx, const double *const *fy,
                         const double *const *fz, const double *dx, const double *dy,
                         const double *dz, const double *const *q0, const double *const *q,
                         double a, double b, double dt, int32_t nvar, int64_t nx, int64_t ny,
                         int64_t nz, double *const *qout, int32_t map, void *stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
SGC_API const char *sgc_last_error(void);

/* SGC_ABI_VERSION of the loaded library. */
SGC_API int32_t sgc_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGC_H */
