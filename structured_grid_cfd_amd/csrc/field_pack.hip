// field_pack.hip -- directional pack of nvar SoA fields into one 4D array,
// and its inverse, for gfx950.
//
// Operation (MFC pull request 2087, "SCC26: Collapse only spatial loops in
// per-variable GPU kernels", Changes): v_rs_weno(j,k,l,i) = v_vf(i)%sf(j,k,l)
// for the x direction; the y and z directions exchange the first index with
// the second (out(k,j,l,var)) or the third (out(l,k,j,var)).  Three variable
// mappings:
//   * PER_CELLVAR -- one thread per (var, cell): the flattened
//     (var, l, k, j) index decomposed per thread, as a four-level collapse
//     does (the page's "before");
//   * PER_CELL -- one thread per cell, index math once, variables looped
//     inside the thread (the page's "after");
//   * TILED -- x: 16-byte streaming copies per variable (the x pack is a
//     concatenation); y/z: 64x64 tiles transposed through LDS so that both the
//     read and the write side move whole 512-byte row segments.
#include "sgc_internal.h"

namespace sgc {
namespace {

struct PackArgs {
    PtrTable f;             // field pointers (written when unpacking)
    const double *packed;   // unpack source
    double *out;            // pack destination
    int nvar, nx, ny, nz;
};

template <int DIR>
__device__ __forceinline__ int packed_index(int j, int k, int l, int nx, int ny, int nz) {
    if (DIR == 0) return j + nx * (k + ny * l);
    if (DIR == 1) return k + ny * (j + nx * l);
    return l + nz * (k + ny * j);
}

// One thread per cell; the variable loop runs inside the thread.
template <int DIR, bool UNPACK>
__global__ __launch_bounds__(256) void k_pack_per_cell(PackArgs g) {
    const int n = g.nx * g.ny * g.nz;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int j = idx % g.nx;
    const int t = idx / g.nx;
    const int k = t % g.ny;
    const int l = t / g.ny;
    const int o = packed_index<DIR>(j, k, l, g.nx, g.ny, g.nz);
    for (int v = 0; v < g.nvar; ++v) {
        if (UNPACK)
            const_cast<double *>(g.f.p[v])[idx] = g.packed[o + v * n];
        else
            g.out[o + v * n] = g.f.p[v][idx];
    }
}

// One thread per (var, cell): the flattened index decomposed into all four
// loop indices by every thread.
template <int DIR, bool UNPACK>
__global__ __launch_bounds__(256) void k_pack_per_cellvar(PackArgs g) {
    const int n = g.nx * g.ny * g.nz;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= n * g.nvar) return;
    const int j = idx % g.nx;
    int t = idx / g.nx;
    const int k = t % g.ny;
    t /= g.ny;
    const int l = t % g.nz;
    const int v = t / g.nz;
    const int o = packed_index<DIR>(j, k, l, g.nx, g.ny, g.nz) + v * n;
    const int c = j + g.nx * (k + g.ny * l);
    if (UNPACK)
        const_cast<double *>(g.f.p[v])[c] = g.packed[o];
    else
        g.out[o] = g.f.p[v][c];
}

// x direction, TILED: per variable a straight copy of n doubles.  Each block
// copies `chunk` elements; when source and destination share their 16-byte
// phase, one peeled element aligns both and the body moves 16-byte vectors,
// four in flight per thread.
template <bool UNPACK>
__global__ __launch_bounds__(256) void k_copy_x(PackArgs g, int chunk) {
    typedef double d2 __attribute__((ext_vector_type(2)));
    const int v = blockIdx.y;
    const int n = g.nx * g.ny * g.nz;
    const double *__restrict__ src = UNPACK ? g.packed + (long)v * n : g.f.p[v];
    double *__restrict__ dst = UNPACK ? const_cast<double *>(g.f.p[v]) : g.out + (long)v * n;
    const int b0 = blockIdx.x * chunk;
    if (b0 >= n) return;
    const int b1 = min(b0 + chunk, n);
    const int tid = threadIdx.x;
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src + b0), da = reinterpret_cast<uintptr_t>(dst + b0);
    if (((sa ^ da) & 15) != 0) {  // phases differ: 8-byte copies
        for (int i = b0 + tid; i < b1; i += 256) dst[i] = src[i];
        return;
    }
    int h = b0 + ((sa & 15) ? 1 : 0);
    if (h > b1) h = b1;
    if (tid < h - b0) dst[b0 + tid] = src[b0 + tid];
    const int nvec = (b1 - h) >> 1;
    const d2 *__restrict__ s2 = reinterpret_cast<const d2 *>(src + h);
    d2 *__restrict__ t2 = reinterpret_cast<d2 *>(dst + h);
    int i = tid;
    for (; i + 3 * 256 < nvec; i += 4 * 256) {
        const d2 a0 = s2[i], a1 = s2[i + 256], a2 = s2[i + 512], a3 = s2[i + 768];
        t2[i] = a0;
        t2[i + 256] = a1;
        t2[i + 512] = a2;
        t2[i + 768] = a3;
    }
    for (; i < nvec; i += 256) t2[i] = s2[i];
    if (((b1 - h) & 1) && tid == 0) dst[b1 - 1] = src[b1 - 1];
}

// Generic batched transpose through LDS.  in(x, y) = in_base[x + y*s_in]
// (x contiguous), out(x, y) = out_base[y + x*s_out] (y contiguous).  One
// 64x64 tile per workgroup of four waves: each wave reads 16 row segments of
// 64 contiguous x, then writes 16 segments of 64 contiguous y.
struct TransArgs {
    PtrTable f;
    const double *packed;
    double *out;
    int X, Y;          // extents of the contiguous input / output indices
    int s_in, s_out;   // strides of the other index on each side
    int P;             // planes per variable
    int p_in, p_out;   // plane offsets on each side
    int v_in, v_out;   // variable offsets on the packed side
    int nvar;
};

template <bool UNPACK>
__global__ __launch_bounds__(256) void k_transpose(TransArgs g) {
    __shared__ double tile[64][65];
    const int ntx = (g.X + 63) >> 6, nty = (g.Y + 63) >> 6;
    int t = xcd_remap(blockIdx.x, gridDim.x);
    const int tx = t % ntx;
    t /= ntx;
    const int ty = t % nty;
    t /= nty;
    const int p = t % g.P;
    const int v = t / g.P;
    const double *__restrict__ in =
        UNPACK ? g.packed + v * g.v_in + p * g.p_in : g.f.p[v] + p * g.p_in;
    double *__restrict__ out =
        UNPACK ? const_cast<double *>(g.f.p[v]) + p * g.p_out : g.out + v * g.v_out + p * g.p_out;
    const int x0 = tx << 6, y0 = ty << 6;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const bool xin = x0 + lane < g.X;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int yy = w + 4 * i;
        if (xin && y0 + yy < g.Y) tile[yy][lane] = in[(x0 + lane) + (y0 + yy) * g.s_in];
    }
    __syncthreads();
    const bool yin = y0 + lane < g.Y;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int xx = w + 4 * i;
        if (yin && x0 + xx < g.X) out[(y0 + lane) + (x0 + xx) * g.s_out] = tile[lane][xx];
    }
}

// How the TILED map moves one variable.  With every extent > 1, y pairs j
// with k and z pairs j with l.  Unit extents collapse the permutation:
//   y, nx or ny == 1       -> identity (out k + ny*(j + nx*l) = j + nx*(k + ny*l))
//   z, nz == 1             -> the y transpose of the (j, k) plane
//   z, nx == 1             -> a (k, l) transpose; identity when ny == 1 too
enum class Layout { Copy, PairJK, PairJL, PairKL };

Layout tiled_layout(int dir, int nx, int ny, int nz) {
    if (dir == SGC_DIR_X) return Layout::Copy;
    if (dir == SGC_DIR_Y || nz == 1) return (nx == 1 || ny == 1) ? Layout::Copy : Layout::PairJK;
    if (nx == 1) return ny == 1 ? Layout::Copy : Layout::PairKL;
    return Layout::PairJL;
}

template <bool UNPACK>
int launch_transpose(const PackArgs &a, Layout lay, hipStream_t s) {
    TransArgs g{};
    g.f = a.f;
    g.packed = a.packed;
    g.out = a.out;
    g.nvar = a.nvar;
    const int nx = a.nx, ny = a.ny, nz = a.nz;
    const int n = nx * ny * nz;
    // Field side f(j,k,l) at j + nx*k + nx*ny*l; packed side per packed_index.
    // fX/fY: extents of the field-contiguous and the paired index; fS / pS:
    // stride of the other index on the field / packed side; P planes with
    // offsets fP / pP.
    int fX, fY, fS, pS, P, fP, pP;
    if (lay == Layout::PairJK) {  // field (j,k) per l -> packed (k,j) per l
        fX = nx; fY = ny; fS = nx; pS = ny; P = nz; fP = nx * ny; pP = nx * ny;
    } else if (lay == Layout::PairJL) {  // field (j,l) per k -> packed (l,j) per k
        fX = nx; fY = nz; fS = nx * ny; pS = nz * ny; P = ny; fP = nx; pP = nz;
    } else {  // PairKL (nx == 1): field (k,l) at k + ny*l -> packed (l,k) at l + nz*k
        fX = ny; fY = nz; fS = ny; pS = nz; P = 1; fP = 0; pP = 0;
    }
    if (!UNPACK) {  // read the field (x contiguous), write packed (y contiguous)
        g.X = fX; g.Y = fY; g.s_in = fS; g.s_out = pS;
        g.P = P; g.p_in = fP; g.p_out = pP; g.v_in = 0; g.v_out = n;
    } else {        // read packed (its contiguous index is x), write the field
        g.X = fY; g.Y = fX; g.s_in = pS; g.s_out = fS;
        g.P = P; g.p_in = pP; g.p_out = fP; g.v_in = n; g.v_out = 0;
    }
    const long tiles = (long)((g.X + 63) / 64) * ((g.Y + 63) / 64) * g.P * g.nvar;
    if (tiles > 0x7fffffffL) return fail(SGC_ERANGE, "transpose grid too large");
    hipLaunchKernelGGL((k_transpose<UNPACK>), dim3((unsigned)tiles), dim3(256), 0, s, g);
    return check_launch("pack transpose");
}

template <bool UNPACK>
int launch_pack(const PackArgs &g, int dir, int map, hipStream_t s) {
    const int n = g.nx * g.ny * g.nz;
    if (map == SGC_VAR_PER_CELL) {
        const dim3 grid((n + 255) / 256);
        if (dir == 0) hipLaunchKernelGGL((k_pack_per_cell<0, UNPACK>), grid, dim3(256), 0, s, g);
        else if (dir == 1) hipLaunchKernelGGL((k_pack_per_cell<1, UNPACK>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_pack_per_cell<2, UNPACK>), grid, dim3(256), 0, s, g);
        return check_launch("pack, one thread per cell");
    }
    if (map == SGC_VAR_PER_CELLVAR) {
        const dim3 grid((unsigned)(((long)n * g.nvar + 255) / 256));
        if (dir == 0) hipLaunchKernelGGL((k_pack_per_cellvar<0, UNPACK>), grid, dim3(256), 0, s, g);
        else if (dir == 1) hipLaunchKernelGGL((k_pack_per_cellvar<1, UNPACK>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((k_pack_per_cellvar<2, UNPACK>), grid, dim3(256), 0, s, g);
        return check_launch("pack, one thread per (var, cell)");
    }
    if (map == SGC_VAR_TILED) {
        const Layout lay = tiled_layout(dir, g.nx, g.ny, g.nz);
        if (lay == Layout::Copy) {
            const int chunk = 8192;
            const dim3 grid((n + chunk - 1) / chunk, g.nvar);
            hipLaunchKernelGGL((k_copy_x<UNPACK>), grid, dim3(256), 0, s, g, chunk);
            return check_launch("pack, streaming copy");
        }
        return launch_transpose<UNPACK>(g, lay, s);
    }
    return fail(SGC_EINVAL, "unknown variable map");
}

}  // namespace

int pack_launch(const PtrTable &fields, int nvar, int nx, int ny, int nz, int dir, double *out, int map,
                hipStream_t s) {
    PackArgs g{};
    g.f = fields;
    g.packed = nullptr;
    g.out = out;
    g.nvar = nvar;
    g.nx = nx;
    g.ny = ny;
    g.nz = nz;
    return launch_pack<false>(g, dir, map, s);
}

int unpack_launch(const double *packed, int nvar, int nx, int ny, int nz, int dir, const PtrTable &fields,
                  int map, hipStream_t s) {
    PackArgs g{};
    g.f = fields;
    g.packed = packed;
    g.out = nullptr;
    g.nvar = nvar;
    g.nx = nx;
    g.ny = ny;
    g.nz = nz;
    return launch_pack<true>(g, dir, map, s);
}

}  // namespace sgc
