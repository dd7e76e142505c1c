// flux_diff.hip -- conservative flux difference over nvar fields, gfx950.
//
// Operation (MFC pull request 2087, "SCC26: Collapse only spatial loops in
// per-variable GPU kernels", Changes: the x/y/z flux-difference loops, with
// the inverse grid spacing computed outside the variable loop):
//   rhs(j,k,l,v) = ((Fx(j)-Fx(j+1))*(1/dx[j]) + (Fy(k)-Fy(k+1))*(1/dy[k]))
//                  + (Fz(l)-Fz(l+1))*(1/dz[l])
// with one rounding per operation, no fused multiply-add, and each reciprocal
// a correctly rounded FP64 division, so every mapping returns the same bits.
// Three variable mappings:
//   * PER_CELLVAR -- one thread per (var, cell), index decomposition and the
//     three reciprocals per thread (the page's "before");
//   * PER_CELL -- one thread per cell, reciprocals once, variables looped
//     inside (the page's "after");
//   * TILED -- one thread per (j, k) column marching a run of l planes: the
//     high z face of plane l is kept in a register as the low face of plane
//     l+1; 1/dx and 1/dy are formed once per thread, i.e. per column of one
//     variable over one run of planes (two planes on most grids), and 1/dz
//     once per plane per workgroup (in LDS).  Forming them once per column
//     for every variable (one workgroup per column block and run, variables
//     in turn) or over longer runs measured slower: the kernel is bound by
//     the loads it keeps in flight, not by the divisions.  Each workgroup
//     handles one variable and the
//     workgroups are ordered variable-major, so at any time the chip streams
//     the five arrays of about one variable: streaming many arrays at once
//     (all variables per thread) measured 10-13% slower on MI355X.  The 2D
//     form marches along k instead, treating Fy as the marched face.
//
// Stage variant (flux_stage3d): the same right-hand side r feeds one SSPRK
// stage in the same thread, q' = a*q0 + b*(q + dt*r) (Mallard documentation,
// "Design: single-GPU performance and parallel scaling": SSPRK3 time steps
// with a right-hand side and an axpby update per stage; the Shu-Osher stage
// form is this library's reading), evaluated t = dt*r; t = q + t; t = b*t;
// s = a*q0; q' = s + t with one rounding each.  r never goes to memory: per
// cell and variable the fused pass reads q0 and q and writes q' instead of
// writing r and re-reading it for a separate update.
#include "sgc_internal.h"

namespace sgc {
namespace {

struct FluxArgs {
    PtrTable fx, fy, fz;
    const double *dx, *dy, *dz;
    double *rhs;
    int nvar, nx, ny, nz;
    StageArgs st;  // stage variant only
};

__device__ __forceinline__ double face_term(double lo, double hi, double inv) {
#pragma clang fp contract(off)
    return (lo - hi) * inv;
}

__device__ __forceinline__ double add(double a, double b) {
#pragma clang fp contract(off)
    return a + b;
}

// q' = a*q0 + b*(q + dt*r), one rounding per operation in this order.
__device__ __forceinline__ double stage(double r, double q0, double q, const StageArgs &st) {
#pragma clang fp contract(off)
    double t = st.dt * r;
    t = q + t;
    t = st.b * t;
    const double s = st.a * q0;
    return s + t;
}

// Output of variable v at flat cell index cell (j + nx*(k + ny*l)): the rhs
// entry, or the stage update of the state.  The state pointers may alias each
// other (q' in place of q or q0); each cell is read before it is written, by
// the same thread.
template <bool STAGE>
__device__ __forceinline__ void put(const FluxArgs &g, int v, long n, long cell, double r) {
    if (STAGE) {
        double *out = const_cast<double *>(g.st.qout.p[v]);
        out[cell] = stage(r, g.st.q0.p[v][cell], g.st.q.p[v][cell], g.st);
    } else {
        g.rhs[cell + (long)v * n] = r;
    }
}

// One thread per cell; variables looped inside the thread.
template <bool HAS_Z, bool STAGE>
__global__ __launch_bounds__(256) void k_flux_per_cell(FluxArgs g) {
    const int n = g.nx * g.ny * g.nz;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int j = idx % g.nx;
    const int t = idx / g.nx;
    const int k = t % g.ny;
    const int l = t / g.ny;
    const double ix = 1.0 / g.dx[j];
    const double iy = 1.0 / g.dy[k];
    const double iz = HAS_Z ? 1.0 / g.dz[l] : 0.0;
    const int ox = j + (g.nx + 1) * (k + g.ny * l);
    const int oy = j + g.nx * (k + (g.ny + 1) * l);
    const int sz = g.nx * g.ny;
    for (int v = 0; v < g.nvar; ++v) {
        double r = face_term(g.fx.p[v][ox], g.fx.p[v][ox + 1], ix);
        r = add(r, face_term(g.fy.p[v][oy], g.fy.p[v][oy + g.nx], iy));
        if (HAS_Z) r = add(r, face_term(g.fz.p[v][idx], g.fz.p[v][idx + sz], iz));
        put<STAGE>(g, v, n, idx, r);
    }
}

// One thread per (var, cell): everything recomputed per thread.
template <bool HAS_Z, bool STAGE>
__global__ __launch_bounds__(256) void k_flux_per_cellvar(FluxArgs g) {
    const int n = g.nx * g.ny * g.nz;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n * g.nvar) return;
    const int j = idx % g.nx;
    int t = idx / g.nx;
    const int k = t % g.ny;
    t /= g.ny;
    const int l = t % g.nz;
    const int v = t / g.nz;
    const double ix = 1.0 / g.dx[j];
    const double iy = 1.0 / g.dy[k];
    const int ox = j + (g.nx + 1) * (k + g.ny * l);
    const int oy = j + g.nx * (k + (g.ny + 1) * l);
    const int oc = j + g.nx * (k + g.ny * l);
    double r = face_term(g.fx.p[v][ox], g.fx.p[v][ox + 1], ix);
    r = add(r, face_term(g.fy.p[v][oy], g.fy.p[v][oy + g.nx], iy));
    if (HAS_Z) {
        const double iz = 1.0 / g.dz[l];
        r = add(r, face_term(g.fz.p[v][oc], g.fz.p[v][oc + g.nx * g.ny], iz));
    }
    put<STAGE>(g, v, n, oc, r);
}

// Column pencils marching the slowest axis.  View (nxv, nyv, nzv): the 3D
// form is (nx, ny, nz) with y and z terms; the 2D form is (nx, 1, ny) whose
// marched face array is Fy and whose widths along the march are dy (there is
// no separate y term), giving the same sum x + y as the definition.
constexpr int kMaxPlanes = 256;

struct PencilArgs {
    FluxArgs g;
    int nxv, nyv, nzv;
    int planes;       // planes per workgroup run
    int col_blocks;   // workgroups across the nxv*nyv columns
    int runs;         // plane runs along the marched axis
    int per_var;      // workgroups per variable (a multiple of 8)
};


template <bool HAS_Y, bool STAGE>
__global__ __launch_bounds__(256) void k_flux_pencil(PencilArgs a) {
    __shared__ double iz_s[kMaxPlanes];
    const FluxArgs &g = a.g;
    // Variable-major block order, dispatched as is: the resident blocks of
    // every XCD work on one variable's arrays at a time.
    const int per_var = a.per_var;  // col_blocks * runs rounded up to a multiple of 8
    const int b = blockIdx.x;
    const int v = b / per_var;
    const int rem = xcd_remap(b - v * per_var, per_var);
    if (rem >= a.col_blocks * a.runs) return;
    const int lb = rem / a.col_blocks;
    const int cb = rem - lb * a.col_blocks;
    const int l0 = lb * a.planes;
    const int l1 = min(l0 + a.planes, a.nzv);
    const double *__restrict__ dzv = HAS_Y ? g.dz : g.dy;
    if ((int)threadIdx.x < l1 - l0) iz_s[threadIdx.x] = 1.0 / dzv[l0 + threadIdx.x];
    __syncthreads();
    const int ncols = a.nxv * a.nyv;
    const int c = cb * 256 + threadIdx.x;
    if (c >= ncols) return;
    const int j = c % a.nxv;
    const int k = c / a.nxv;
    const double ix = 1.0 / g.dx[j];
    const double iy = HAS_Y ? 1.0 / g.dy[k] : 0.0;
    const int sx = (a.nxv + 1) * a.nyv;  // Fx plane size
    const int sy = a.nxv * (a.nyv + 1);  // Fy plane size
    const int sc = ncols;                // cell / marched-face plane size
    const int n = sc * a.nzv;
    const int ox = c + k;                // j + (nxv+1)*k
    const double *__restrict__ FX = g.fx.p[v];
    const double *__restrict__ FY = g.fy.p[v];
    const double *__restrict__ FZ = HAS_Y ? g.fz.p[v] : g.fy.p[v];

    double zlo = FZ[c + sc * l0];
    for (int l = l0; l < l1; ++l) {
        const double xl = FX[ox + sx * l];
        const double xh = FX[ox + sx * l + 1];
        double yl = 0.0, yh = 0.0;
        if (HAS_Y) {
            yl = FY[c + sy * l];
            yh = FY[c + sy * l + a.nxv];
        }
        const double zh = FZ[c + sc * (l + 1)];
        double r = face_term(xl, xh, ix);
        if (HAS_Y) r = add(r, face_term(yl, yh, iy));
        r = add(r, face_term(zlo, zh, iz_s[l - l0]));
        put<STAGE>(g, v, n, c + (long)sc * l, r);
        zlo = zh;
    }
}

// Waves over the grid: the plane run per thread is chosen so the launch has
// about this many, which in practice means the shortest runs (two planes) on
// the grids measured: more waves, more loads in flight, and the z faces of a
// run boundary are the only ones read twice.
constexpr int kTargetWaves = 262144;

template <bool STAGE>
int flux_launch_t(const FluxArgs &g, bool has_z, int map, hipStream_t s) {
    const long n = (long)g.nx * g.ny * g.nz;
    if (map == SGC_VAR_PER_CELL) {
        const dim3 grid((unsigned)((n + 255) / 256));
        if (has_z) hipLaunchKernelGGL((k_flux_per_cell<true, STAGE>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_flux_per_cell<false, STAGE>), grid, dim3(256), 0, s, g);
        return check_launch("flux difference, one thread per cell");
    }
    if (map == SGC_VAR_PER_CELLVAR) {
        const dim3 grid((unsigned)((n * g.nvar + 255) / 256));
        if (has_z) hipLaunchKernelGGL((k_flux_per_cellvar<true, STAGE>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_flux_per_cellvar<false, STAGE>), grid, dim3(256), 0, s, g);
        return check_launch("flux difference, one thread per (var, cell)");
    }
    if (map != SGC_VAR_TILED) return fail(SGC_EINVAL, "unknown variable map");
    PencilArgs a;
    a.g = g;
    if (has_z) {
        a.nxv = g.nx; a.nyv = g.ny; a.nzv = g.nz;
    } else {
        a.nxv = g.nx; a.nyv = 1; a.nzv = g.ny;
    }
    const long ncols = (long)a.nxv * a.nyv;
    a.col_blocks = (int)((ncols + 255) / 256);
    const long waves_per_run = (ncols + 63) / 64;
    long runs = (kTargetWaves + waves_per_run * g.nvar - 1) / (waves_per_run * g.nvar);
    if (runs < 1) runs = 1;
    int planes = (int)((a.nzv + runs - 1) / runs);
    planes = planes < 2 ? 2 : planes;
    planes = planes > kMaxPlanes ? kMaxPlanes : planes;
    planes = planes > a.nzv ? a.nzv : planes;
    a.planes = planes;
    a.runs = (a.nzv + planes - 1) / planes;
    a.per_var = ((a.col_blocks * a.runs + 7) / 8) * 8;
    const long blocks = (long)a.per_var * g.nvar;
    if (has_z) hipLaunchKernelGGL((k_flux_pencil<true, STAGE>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_flux_pencil<false, STAGE>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return check_launch("flux difference, column pencils");
}

}  // namespace

int flux_launch(const PtrTable &fx, const PtrTable &fy, const PtrTable *fz, const double *dx,
                const double *dy, const double *dz, int nvar, int nx, int ny, int nz, double *rhs,
                const StageArgs *st, int map, hipStream_t s) {
    FluxArgs g{};
    g.fx = fx;
    g.fy = fy;
    if (fz) g.fz = *fz;
    g.dx = dx;
    g.dy = dy;
    g.dz = dz;
    g.rhs = rhs;
    g.nvar = nvar;
    g.nx = nx;
    g.ny = ny;
    g.nz = nz;
    if (st) g.st = *st;
    const bool has_z = fz != nullptr;
    return st ? flux_launch_t<true>(g, has_z, map, s) : flux_launch_t<false>(g, has_z, map, s);
}

}  // namespace sgc
