/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the structured-grid
 * stencil sweeps (2D five-point diffusion, directional field packing and the
 * conservative flux difference).
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and
 * the benchmark's CPU-baseline leg may load or call this code.  It shares no
 * source, header, table or helper with the HIP library and must never be used
 * as a fallback for it.
 *
 * Build (see oracle/__init__.py):
 *     gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC oracle.c
 * Contraction is off so that every operation below is exactly one IEEE-754
 * round-to-nearest in its declared type, in the order written.
 *
 * Pages followed (cited by title and section):
 *   [Q3]  Qiita, "Fortran 2018でGPUを高速化する Part 3 - GPUカーネルのメモリ
 *         アクセスとFP32・FP64を比較する": section 3 (five-point update,
 *         alpha = 0.1, edges fixed at 0), section 4 (first index contiguous),
 *         section 5.4 (u -> v on odd steps, v -> u on even steps; the result is
 *         in v after an odd number of steps), section 6.1 (alpha is the literal
 *         0.1 in the working precision), Appendix A "src/cpu_reference.f90"
 *         (j outer, i inner, edge branch in every cell).
 *   [MFC] MFC pull request 2087, "SCC26: Collapse only spatial loops in
 *         per-variable GPU kernels": Changes (the WENO input pack
 *         v_rs_weno(j,k,l,i) = v_vf(i)%sf(j,k,l); the x/y/z flux differences;
 *         inverse grid spacing formed once per cell).
 *   [Mallard] Mallard documentation, "Design: single-GPU performance and
 *         parallel scaling": Hardware and method (time steps are SSPRK3, three
 *         stages) and the Baseline tables (per stage a right-hand side, a
 *         division by the cell volume and an axpby update).
 *
 * Readings taken where the pages are silent:
 *   - evaluation order of the five-point sum is left to right,
 *     ((((W + E) + S) + N) - 4*C), then C + alpha*t, no fused multiply-add;
 *   - both buffers' edge rings are zeroed before the first step;
 *   - the y and z packs are out(k,j,l,var) and out(l,k,j,var), first index
 *     contiguous;
 *   - the flux difference is rhs = (F_lo - F_hi) * (1/d) per direction, summed
 *     in the order x, y, z; cell j's low face is face j, its high face j+1;
 *   - the SSPRK stage, for which the pages give no formula, is the Shu-Osher
 *     form q' = a*q0 + b*(q + dt*rhs) with (a, b) = (0, 1), (3/4, 1/4),
 *     (1/3, 2/3), evaluated as t = dt*rhs; t = q + t; t = b*t; s = a*q0;
 *     q' = s + t, one rounding each.
 *
 * Every function is pinned by the tests named test_oracle_*: the pages'
 * printed comparison, hand-worked closed forms, exact rationals on tiny
 * inputs, permutation and telescoping identities; a mutation test checks
 * that planted mistakes fail them.
 */
#include <stddef.h>
#include <stdlib.h>
#include <stdint.h>

/* ------------------------------------------------------------------------ */
/* 2D five-point explicit diffusion ([Q3] sections 3, 5.4; Appendix A).     */
/* Arrays are column-major u(nx, ny) with leading dimension ld >= nx:       */
/* element (i, j), 0-based, lives at u[i + ld*j].                           */
/* ------------------------------------------------------------------------ */

static void zero_ring_f64(double *a, int64_t nx, int64_t ny, int64_t ld)
{
    for (int64_t i = 0; i < nx; ++i) {
        a[i] = 0.0;
        a[i + ld * (ny - 1)] = 0.0;
    }
    for (int64_t j = 0; j < ny; ++j) {
        a[ld * j] = 0.0;
        a[(nx - 1) + ld * j] = 0.0;
    }
}

static void zero_ring_f32(float *a, int64_t nx, int64_t ny, int64_t ld)
{
    for (int64_t i = 0; i < nx; ++i) {
        a[i] = 0.0f;
        a[i + ld * (ny - 1)] = 0.0f;
    }
    for (int64_t j = 0; j < ny; ++j) {
        a[ld * j] = 0.0f;
        a[(nx - 1) + ld * j] = 0.0f;
    }
}

/* One sweep src -> dst over every cell: edge cells get 0, interior cells the
 * five-point update.  Returns nothing; dst never aliases src. */
static void sweep_f64(const double *src, double *dst, int64_t nx, int64_t ny,
                      int64_t ld, double a)
{
    const double four = 4.0;
    for (int64_t j = 0; j < ny; ++j) {
        for (int64_t i = 0; i < nx; ++i) {
            const int64_t p = i + ld * j;
            if (i == 0 || i == nx - 1 || j == 0 || j == ny - 1) {
                dst[p] = 0.0;
            } else {
                const double c = src[p];
                double t = src[p - 1] + src[p + 1]; /* W + E          */
                t = t + src[p - ld];                /* + S  (j - 1)   */
                t = t + src[p + ld];                /* + N  (j + 1)   */
                t = t - four * c;                   /* - 4 C          */
                dst[p] = c + a * t;
            }
        }
    }
}

static void sweep_f32(const float *src, float *dst, int64_t nx, int64_t ny,
                      int64_t ld, float a)
{
    const float four = 4.0f;
    for (int64_t j = 0; j < ny; ++j) {
        for (int64_t i = 0; i < nx; ++i) {
            const int64_t p = i + ld * j;
            if (i == 0 || i == nx - 1 || j == 0 || j == ny - 1) {
                dst[p] = 0.0f;
            } else {
                const float c = src[p];
                float t = src[p - 1] + src[p + 1];
                t = t + src[p - ld];
                t = t + src[p + ld];
                t = t - four * c;
                dst[p] = c + a * t;
            }
        }
    }
}

/* Runs `steps` sweeps with u/v alternation and returns 1 if the result is in
 * v (odd step count), 0 if it is in u.  alpha is rounded once to the working
 * precision, as the page's literal 0.1 of kind rk is. */
int oracle_diffuse2d_f64(double *u, double *v, int64_t nx, int64_t ny,
                         int64_t ld, double alpha, int64_t steps)
{
    zero_ring_f64(u, nx, ny, ld);
    zero_ring_f64(v, nx, ny, ld);
    for (int64_t s = 1; s <= steps; ++s) {
        if (s % 2 == 1)
            sweep_f64(u, v, nx, ny, ld, alpha);
        else
            sweep_f64(v, u, nx, ny, ld, alpha);
    }
    return (int)(steps % 2);
}

int oracle_diffuse2d_f32(float *u, float *v, int64_t nx, int64_t ny,
                         int64_t ld, double alpha, int64_t steps)
{
    const float a = (float)alpha;
    zero_ring_f32(u, nx, ny, ld);
    zero_ring_f32(v, nx, ny, ld);
    for (int64_t s = 1; s <= steps; ++s) {
        if (s % 2 == 1)
            sweep_f32(u, v, nx, ny, ld, a);
        else
            sweep_f32(v, u, nx, ny, ld, a);
    }
    return (int)(steps % 2);
}

/* ------------------------------------------------------------------------ */
/* Directional pack of nvar SoA fields ([MFC] Changes: the WENO input pack). */
/* Field f_var(j,k,l) is column-major (j fastest) with nx*ny*nz elements.    */
/*   dir 0 (x): out(j,k,l,var)   dims (nx,ny,nz,nvar)                        */
/*   dir 1 (y): out(k,j,l,var)   dims (ny,nx,nz,nvar)                        */
/*   dir 2 (z): out(l,k,j,var)   dims (nz,ny,nx,nvar)                        */
/* The output's first index is contiguous.  A pure copy: no arithmetic.     */
/* ------------------------------------------------------------------------ */

int oracle_field_pack(const double *const *fields, int32_t nvar, int64_t nx,
                      int64_t ny, int64_t nz, int32_t dir, double *out)
{
    if (dir < 0 || dir > 2)
        return 1;
    for (int32_t var = 0; var < nvar; ++var) {
        const double *f = fields[var];
        for (int64_t l = 0; l < nz; ++l)
            for (int64_t k = 0; k < ny; ++k)
                for (int64_t j = 0; j < nx; ++j) {
                    const double x = f[j + nx * (k + ny * l)];
                    int64_t o;
                    if (dir == 0)
                        o = j + nx * (k + ny * (l + nz * (int64_t)var));
                    else if (dir == 1)
                        o = k + ny * (j + nx * (l + nz * (int64_t)var));
                    else
                        o = l + nz * (k + ny * (j + nx * (int64_t)var));
                    out[o] = x;
                }
    }
    return 0;
}

/* Inverse of oracle_field_pack: scatter the packed array back to the nvar
 * fields (the directional copies back out of the packed layout). */
int oracle_field_unpack(const double *packed, int32_t nvar, int64_t nx,
                        int64_t ny, int64_t nz, int32_t dir,
                        double *const *fields)
{
    if (dir < 0 || dir > 2)
        return 1;
    for (int32_t var = 0; var < nvar; ++var) {
        double *f = fields[var];
        for (int64_t l = 0; l < nz; ++l)
            for (int64_t k = 0; k < ny; ++k)
                for (int64_t j = 0; j < nx; ++j) {
                    int64_t o;
                    if (dir == 0)
                        o = j + nx * (k + ny * (l + nz * (int64_t)var));
                    else if (dir == 1)
                        o = k + ny * (j + nx * (l + nz * (int64_t)var));
                    else
                        o = l + nz * (k + ny * (j + nx * (int64_t)var));
                    f[j + nx * (k + ny * l)] = packed[o];
                }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Conservative flux difference ([MFC] Changes: x/y/z flux differences with */
/* the inverse spacing formed outside the variable loop).                   */
/* Per variable, face arrays are column-major:                              */
/*   Fx (nx+1, ny, nz), Fy (nx, ny+1, nz), Fz (nx, ny, nz+1).               */
/* Cell widths dx[nx], dy[ny], dz[nz].  rhs is (nx, ny, nz, nvar).          */
/* fz == NULL selects the 2D form (nz must be 1, no z term, dz unused).     */
/* ------------------------------------------------------------------------ */

int oracle_flux_diff(const double *const *fx, const double *const *fy,
                     const double *const *fz, const double *dx,
                     const double *dy, const double *dz, int32_t nvar,
                     int64_t nx, int64_t ny, int64_t nz, double *rhs)
{
    if (fz == NULL && nz != 1)
        return 1;
    for (int32_t var = 0; var < nvar; ++var) {
        for (int64_t l = 0; l < nz; ++l)
            for (int64_t k = 0; k < ny; ++k)
                for (int64_t j = 0; j < nx; ++j) {
                    const double ix = 1.0 / dx[j];
                    const double iy = 1.0 / dy[k];
                    double r = (fx[var][j + (nx + 1) * (k + ny * l)] -
                                fx[var][(j + 1) + (nx + 1) * (k + ny * l)]) *
                               ix;
                    r = r + (fy[var][j + nx * (k + (ny + 1) * l)] -
                             fy[var][j + nx * ((k + 1) + (ny + 1) * l)]) *
                                iy;
                    if (fz != NULL) {
                        const double iz = 1.0 / dz[l];
                        r = r + (fz[var][j + nx * (k + ny * l)] -
                                 fz[var][j + nx * (k + ny * (l + 1))]) *
                                    iz;
                    }
                    rhs[j + nx * (k + ny * (l + nz * (int64_t)var))] = r;
                }
    }
    return 0;
}

/*
 * One SSPRK stage on the flux difference ([Mallard] Hardware and method,
 * Baseline): per cell and variable, r is the flux difference of
 * oracle_flux_diff, then qout = a*q0 + b*(q + dt*r) in the order
 * t = dt*r; t = q + t; t = b*t; s = a*q0; qout = s + t.  q0, q and qout are
 * tables of nvar fields of nx*ny*nz doubles (j fastest).  qout may be q or q0
 * (each cell is read before it is written).  Returns 0, or 1 for a 2D call
 * with nz != 1, 2 if the scratch rhs cannot be allocated.
 */
int oracle_flux_stage(const double *const *fx, const double *const *fy,
                      const double *const *fz, const double *dx,
                      const double *dy, const double *dz,
                      const double *const *q0, const double *const *q,
                      double a, double b, double dt, int32_t nvar,
                      int64_t nx, int64_t ny, int64_t nz, double *const *qout)
{
    const int64_t n = nx * ny * nz;
    double *rhs = (double *)malloc((size_t)(n * nvar) * sizeof(double));
    if (rhs == NULL)
        return 2;
    const int rc = oracle_flux_diff(fx, fy, fz, dx, dy, dz, nvar, nx, ny, nz, rhs);
    if (rc != 0) {
        free(rhs);
        return rc;
    }
    for (int32_t var = 0; var < nvar; ++var)
        for (int64_t c = 0; c < n; ++c) {
            double t = dt * rhs[c + n * var];
            t = q[var][c] + t;
            t = b * t;
            const double s = a * q0[var][c];
            qout[var][c] = s + t;
        }
    free(rhs);
    return 0;
}
