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
//   * TILED -- x: 16-byte streaming copies per variable (the x
//     pack is a concatenation); y/z: balanced tiles of at most 64x64
//     transposed through LDS so that both the read and the write side move
//     contiguous row segments.
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

// x direction (and the identity cases), TILED: per variable a straight copy
// of n doubles.  Each workgroup moves one chunk of kChunkVec 16-byte vectors,
// one per thread, through buffer descriptors spanning the chunk (the last
// chunk's tail falls outside them).  Loads are non-temporal (nothing re-reads
// the source) and stores carry the sc1 scope bit: on MI355X that pairing
// streamed a 1 GiB copy at 7.4 TB/s against 6.5 with default policies and
// 7.2 with non-temporal loads alone, and one vector per thread beat four.
// (Non-temporal stores, and sc1 stores on the transposes and the march,
// measured slower.)  When source and destination share their 16-byte phase,
// element 0 is peeled (if needed) so both are aligned; otherwise the chunk
// falls back to 8-byte copies.
constexpr int kChunkVec = 256;
constexpr int kStreamLoadPolicy = 2;    // nt
constexpr int kStreamStorePolicy = 16;  // sc1

template <bool UNPACK>
__global__ __launch_bounds__(256) void k_copy(PackArgs g, int chunks_per_var) {
    // Variable-major: all XCDs copy one variable at a time, each a contiguous
    // range of its chunks (chunks_per_var is a multiple of 8; chunks past the
    // variable's end copy nothing).
    const int v = blockIdx.x / chunks_per_var;
    const int chunk = xcd_remap(blockIdx.x - v * chunks_per_var, chunks_per_var);
    const int n = g.nx * g.ny * g.nz;
    const double *__restrict__ src = UNPACK ? g.packed + (long)v * n : g.f.p[v];
    double *__restrict__ dst = UNPACK ? const_cast<double *>(g.f.p[v]) : g.out + (long)v * n;
    const int tid = threadIdx.x;
    const uintptr_t sa = reinterpret_cast<uintptr_t>(src), da = reinterpret_cast<uintptr_t>(dst);
    if (((sa ^ da) & 15) != 0) {  // phases differ: 8-byte copies, two per chunk vector
        constexpr int U8 = 2 * kChunkVec / 256;
        const int e0 = chunk * 2 * kChunkVec;
        double t[U8];
        if (e0 <= n - 2 * kChunkVec) {  // whole chunk in range (no overflow for n near 2^31)
#pragma unroll
            for (int u = 0; u < U8; ++u) t[u] = __builtin_nontemporal_load(src + e0 + u * 256 + tid);
#pragma unroll
            for (int u = 0; u < U8; ++u) *(dst + e0 + u * 256 + tid) = t[u];
            return;
        }
#pragma unroll
        for (int u = 0; u < U8; ++u) {
            const int i = e0 + u * 256 + tid;
            t[u] = i < n ? __builtin_nontemporal_load(src + i) : 0.0;
        }
#pragma unroll
        for (int u = 0; u < U8; ++u) {
            const int i = e0 + u * 256 + tid;
            if (i < n) *(dst + i) = t[u];
        }
        return;
    }
    const int h = (sa & 15) ? 1 : 0;  // peeled head element
    const int nvec = (n - h) >> 1;
    if (chunk == 0 && tid == 0) {
        if (h) dst[0] = src[0];
        if ((n - h) & 1) dst[n - 1] = src[n - 1];
    }
    const int c0 = chunk * kChunkVec;
    if (c0 >= nvec) return;
    const uint32_t bytes = (uint32_t)min(kChunkVec, nvec - c0) * 16u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + h + 2 * (long)c0, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dst + h + 2 * (long)c0, bytes);
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    constexpr int U = kChunkVec / 256;
    i32x4 t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) t[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(tid + u * 256) * 16u, 0, kStreamLoadPolicy);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(t[u], rd, (uint32_t)(tid + u * 256) * 16u, 0, kStreamStorePolicy);
}

// Generic batched transpose through LDS.  in(x, y) = in_base[x + y*s_in]
// (x contiguous), out(x, y) = out_base[y + x*s_out] (y contiguous).  Tiles of
// TX x TY (each at most 64) split X and Y into equal parts, so no tile is a
// thin remainder that costs a full tile's time for a few elements (201 =
// 4 x 51 rather than 3 x 64 + 9).  One tile per workgroup of four waves: the
// waves read rows of TX contiguous x, then write rows of TY contiguous y.
struct TransArgs {
    PtrTable f;
    const double *packed;
    double *out;
    int X, Y;          // extents of the contiguous input / output indices
    int TX, TY;        // tile extents (<= 64)
    int ntx, nty;      // tiles along X and Y
    int s_in, s_out;   // strides of the other index on each side
    int P;             // planes per variable
    int p_in, p_out;   // plane offsets on each side
    int v_in, v_out;   // variable offsets on the packed side
    int nvar;
    int per_var;       // workgroups per variable (tiles rounded up to a multiple of 8)
};

template <bool UNPACK>
__global__ __launch_bounds__(256) void k_transpose(TransArgs g) {
    // The tile in LDS, sized to this launch's tiles: TY rows of TX values at
    // an odd stride (in doubles), so that reading a column touches 32
    // different bank pairs per half-wave.  Smaller tiles leave room for more
    // workgroups per CU (201 = 4 x 51: 20.8 KB, seven per CU, against four
    // for a padded 64 x 64 tile).
    extern __shared__ double tile[];
    const int ts = g.TX | 1;
    // Variable-major: all XCDs work on one variable's planes at a time, each
    // on a contiguous range of its tiles.
    const int per_var = g.per_var;  // ntx * nty * P rounded up to a multiple of 8
    const int v = blockIdx.x / per_var;
    int t = xcd_remap(blockIdx.x - v * per_var, per_var);
    if (t >= g.ntx * g.nty * g.P) return;  // padding workgroup (uniform exit, before the barrier)
    const int tx = t % g.ntx;
    t /= g.ntx;
    const int ty = t % g.nty;
    const int p = t / g.nty;
    const int x0 = tx * g.TX, y0 = ty * g.TY;
    const int w = min(g.TX, g.X - x0), h = min(g.TY, g.Y - y0);
    const double *in = (UNPACK ? g.packed + v * g.v_in : g.f.p[v]) + p * g.p_in + x0 + y0 * g.s_in;
    double *out = (UNPACK ? const_cast<double *>(g.f.p[v]) : g.out + v * g.v_out) + p * g.p_out +
                  y0 + x0 * g.s_out;
    // Descriptors span exactly this tile's rows; elements outside the tile
    // get an out-of-range offset, so every load and store below is issued
    // unconditionally (all sixteen loads are in flight before the first use).
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in, (uint32_t)(w + (h - 1) * g.s_in) * 8u);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out, (uint32_t)(h + (w - 1) * g.s_out) * 8u);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    double val[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int yy = wv + 4 * i;
        const uint32_t off = (lane < w && yy < h) ? (uint32_t)(lane + yy * g.s_in) * 8u : kOutOfRange;
        val[i] = buf_load_f64<2>(rin, off);  // each element is read once: non-temporal
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (wv + 4 * i < g.TY && lane < g.TX) tile[(wv + 4 * i) * ts + lane] = val[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int xx = wv + 4 * i;
        const uint32_t off = (lane < h && xx < w) ? (uint32_t)(lane + xx * g.s_out) * 8u : kOutOfRange;
        buf_store_f64(lane < h && xx < w ? tile[lane * ts + xx] : 0.0, rout, off);
    }
}

// Equal split of n into ceil(n / 64) parts of at most 64.
inline int balanced_tile(int n) {
    const int parts = (n + 63) / 64;
    return (n + parts - 1) / parts;
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
    // Buffer offsets inside one tile must stay below 2^31.
    if ((long)64 * (g.s_in + 1) * 8 >= (1L << 31) || (long)64 * (g.s_out + 1) * 8 >= (1L << 31))
        return -1;
    g.TX = balanced_tile(g.X);
    g.TY = balanced_tile(g.Y);
    g.ntx = (g.X + g.TX - 1) / g.TX;
    g.nty = (g.Y + g.TY - 1) / g.TY;
    const long per_var = (((long)g.ntx * g.nty * g.P + 7) / 8) * 8;
    const long tiles = per_var * g.nvar;
    if (tiles > 0x7fffffffL) return fail(SGC_ERANGE, "transpose grid too large");
    g.per_var = (int)per_var;
    const size_t lds = (size_t)g.TY * (size_t)(g.TX | 1) * sizeof(double);
    hipLaunchKernelGGL((k_transpose<UNPACK>), dim3((unsigned)tiles), dim3(256), lds, s, g);
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
            const long chunks = ((long)n + 2L * kChunkVec - 1) / (2L * kChunkVec);
            const long per_var = ((chunks + 7) / 8) * 8;  // a multiple of 8 for the XCD remap
            const long blocks = per_var * g.nvar;
            if (blocks > 0x7fffffffL) return fail(SGC_ERANGE, "copy grid too large");
            hipLaunchKernelGGL((k_copy<UNPACK>), dim3((unsigned)blocks), dim3(256), 0, s, g, (int)per_var);
            return check_launch("pack, streaming copy");
        }
        const int rc = launch_transpose<UNPACK>(g, lay, s);
        if (rc != -1) return rc;
        // Strides too large for 32-bit tile offsets: one thread per cell.
        return launch_pack<UNPACK>(g, dir, SGC_VAR_PER_CELL, s);
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
