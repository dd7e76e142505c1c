// diffuse2d.hip -- explicit 2D five-point diffusion sweeps for gfx950.
//
// Operation (Qiita "Fortran 2018でGPUを高速化する Part 3", section 3):
//   v(i,j) = u(i,j) + alpha*(u(i-1,j) + u(i+1,j) + u(i,j-1) + u(i,j+1) - 4u(i,j))
// on interior cells, edges fixed at 0, column-major storage with i contiguous
// (section 4).  Thread mappings:
//   * k_collapse_branch, k_contig, k_strided -- the three loop layouts of
//     section 5.1-5.3 (flattened grid with an edge branch; workgroup per row
//     with lanes along i; workgroup per column with lanes along j);
//   * k_march<T, TS, KV, ...> -- this library's sweep: one wave owns a strip
//     of 64*K columns (K = 2 doubles, or 4 floats at depths 1-2 and 2 floats
//     from depth 3: one 16- or 8-byte load per lane and row) and marches
//     along a tile of rows, keeping a three-row register window per time
//     level.  West/east neighbours cross lanes with DPP wave shifts,
//     north/south come from the window, so every input row is read from
//     memory exactly once and every output row written once per launch.
//     TS > 1 fuses TS time steps in one launch (temporal blocking): the strip
//     carries a halo of TS columns on each side and the tile TS extra rows
//     above and below, recomputed redundantly.  (Section 5.4 leaves fusion
//     across steps out, since one that ignored the neighbour dependencies
//     would be wrong; the halo carries exactly those dependencies.)  Every
//     cell of a level is produced by the same expression as a single step,
//     so all mappings give identical bits.  Memory goes through raw buffer
//     instructions whose range check supplies the zero rows and drops stores
//     outside the wave's rows, so the loop has no branches around memory and
//     its prefetch waits stay partial.  A launch may step several fields of one shape: tile t
//     belongs to field t / field_tiles.
//   * k_resident<T, R, W> -- grids of at most 64 x 128 cells held in the
//     registers of one workgroup of W waves (R rows each) for every step of
//     the call, one workgroup per field.
#include <climits>
#include <cmath>

#include "sgc_internal.h"

namespace sgc {
namespace {

// c + a*((((W + E) + S) + N) - 4c): left-to-right sum, one rounding per
// operation, no fused multiply-add (fused c + a*t would change the bits).
template <typename T>
__device__ __forceinline__ T five_point(T w, T e, T s, T n, T c, T a) {
#pragma clang fp contract(off)
    T t = w + e;
    t = t + s;
    t = t + n;
    t = t - T(4) * c;
    return c + a * t;
}

// The same bits through one fused multiply-add.  Scaling by 4 is exact
// whenever the product is finite, so fma(-4, c, t) rounds t - 4c once exactly
// as the separate subtraction does (signed zeros and subnormals included);
// valid only while |4c| stays below the overflow threshold, which the march
// checks on every tile it computes this way.
__device__ __forceinline__ float fma_op(float x, float y, float z) { return __builtin_fmaf(x, y, z); }
__device__ __forceinline__ double fma_op(double x, double y, double z) { return __builtin_fma(x, y, z); }
template <typename T>
__device__ __forceinline__ T five_point_fused(T w, T e, T s, T n, T c, T a) {
#pragma clang fp contract(off)
    T t = w + e;
    t = t + s;
    t = t + n;
    t = fma_op(T(-4), c, t);
    return c + a * t;
}

// ---------------------------------------------------------------------------
// The pages' three loop layouts
// ---------------------------------------------------------------------------

// Section 5.1: collapse(2) over all cells; edge cells get 0 through a branch.
template <typename T>
__global__ __launch_bounds__(256) void k_collapse_branch(const T *__restrict__ src,
                                                         T *__restrict__ dst, int nx,
                                                         int ny, int ld, T a) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= nx * ny) return;
    const int j = idx / nx;
    const int i = idx - j * nx;
    const int p = i + ld * j;
    T out = T(0);
    if (!(i == 0 || i == nx - 1 || j == 0 || j == ny - 1))
        out = five_point(src[p - 1], src[p + 1], src[p - ld], src[p + ld], src[p], a);
    dst[p] = out;
}

// Section 5.2: one workgroup per interior row j, lanes along i (contiguous).
template <typename T>
__global__ __launch_bounds__(256) void k_contig(const T *__restrict__ src, T *__restrict__ dst,
                                                int nx, int ny, int ld, T a) {
    const int j = 1 + blockIdx.x;
    for (int i = 1 + threadIdx.x; i < nx - 1; i += 256) {
        const int p = i + ld * j;
        dst[p] = five_point(src[p - 1], src[p + 1], src[p - ld], src[p + ld], src[p], a);
    }
}

// Section 5.3: one workgroup per interior column i, lanes along j (stride ld).
template <typename T>
__global__ __launch_bounds__(256) void k_strided(const T *__restrict__ src, T *__restrict__ dst,
                                                 int nx, int ny, int ld, T a) {
    const int i = 1 + blockIdx.x;
    for (int j = 1 + threadIdx.x; j < ny - 1; j += 256) {
        const int p = i + ld * j;
        dst[p] = five_point(src[p - 1], src[p + 1], src[p - ld], src[p + ld], src[p], a);
    }
}

// Zero the edge ring (rows 0 and ny-1, columns 0 and nx-1) of one buffer.
template <typename T>
__global__ __launch_bounds__(256) void k_zero_ring(T *__restrict__ g, int nx, int ny, int ld) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < nx)
        g[t] = T(0);
    else if (t < 2 * nx)
        g[(t - nx) + ld * (ny - 1)] = T(0);
    else if (t < 2 * nx + ny)
        g[ld * (t - 2 * nx)] = T(0);
    else if (t < 2 * nx + 2 * ny)
        g[(nx - 1) + ld * (t - 2 * nx - ny)] = T(0);
}

// ---------------------------------------------------------------------------
// Marching strip sweep with optional temporal blocking
// ---------------------------------------------------------------------------

// The vector one lane loads per row, VN elements.  FP64 uses two (16 bytes).
// FP32 uses four (16 bytes) for one or two fused steps, which are memory
// bound and stream better with 16-byte accesses, and two (8 bytes) for
// deeper fusion: twice the strips means fewer row tiles for the same wave
// count, and the taller tiles save more recomputed halo rows than the extra
// halo columns cost (measured +3-8% at 4096^2..16384^2, +35% at 2048^2;
// 8-byte vectors were 8-10% slower at one or two steps).
template <typename T> constexpr int lane_elems(int ts) {
    return sizeof(T) == 8 ? 2 : (ts <= 2 ? 4 : 2);
}
template <typename T, int VN> struct LaneVec {
    static constexpr int V = VN;
    typedef T type __attribute__((ext_vector_type(VN)));
};

// DPP wavefront shifts by one lane (GFX9 dpp_ctrl 0x138 wave_shr:1 and 0x130
// wave_shl:1) with bound_ctrl set: shr gives lane l the value of lane l-1,
// shl the value of lane l+1, and the lane without a source receives 0.  Those
// lanes only ever feed halo columns that the march discards.
__device__ __forceinline__ float wave_shr1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_shl1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x130, 0xf, 0xf, true));
}
__device__ __forceinline__ double wave_shr1(double x) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), 0x138, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), 0x138, 0xf, 0xf, true);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_shl1(double x) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), 0x130, 0xf, 0xf, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), 0x130, 0xf, 0xf, true);
    return __hiloint2double(hi, lo);
}

// Memory goes through raw buffer descriptors (sgc_internal.h): the march
// points each wave's load descriptor at exactly the interior rows it may read
// and its store descriptor at exactly the rows it owns, so boundary rows, halo
// rows and discarded lanes need no branches around memory operations.
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Loads one VN-element lane vector into x[at .. at+VN).
template <int POL, int VN, typename T, int K>
__device__ __forceinline__ void buf_load_vec(T (&x)[K], int at, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef typename LaneVec<T, VN>::type VT;
    VT y;
    if constexpr (sizeof(VT) == 16)
        y = __builtin_bit_cast(VT, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL));
    else
        y = __builtin_bit_cast(VT, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
#pragma unroll
    for (int e = 0; e < VN; ++e) x[at + e] = y[e];
}
template <int POL>
__device__ __forceinline__ float buf_load_elem(float *, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POL));
}
template <int POL>
__device__ __forceinline__ double buf_load_elem(double *, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
}
// Stores x[at .. at+VN) as one lane vector.
template <int POL, int VN, typename T, int K>
__device__ __forceinline__ void buf_store_vec(const T (&x)[K], int at, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef typename LaneVec<T, VN>::type VT;
    VT y;
#pragma unroll
    for (int e = 0; e < VN; ++e) y[e] = x[at + e];
    if constexpr (sizeof(VT) == 16)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, y), r, off, 0, POL);
    else
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, y), r, off, 0, POL);
}
template <int POL>
__device__ __forceinline__ void buf_store_elem(float x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(x), r, off, 0, POL);
}
template <int POL>
__device__ __forceinline__ void buf_store_elem(double x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, off, 0, POL);
}

struct MarchArgs {
    const void *src[SGC_MAX_NVAR];  // per field
    void *dst[SGC_MAX_NVAR];
    int nx, ny, ld;
    int nstrips;      // strips across the grid (OW output columns each)
    int field_tiles;  // nstrips * row tiles: the tiles of one field
    int ntiles;       // fields * field_tiles; tile t is field t / field_tiles
    int tile_rows;  // output rows per tile
    double alpha;
    double fuse_limit;  // fused form allowed while sum |input| stays below this
    int balance;        // waves lower their issue priority as they progress
};

// Strip geometry for KV lane vectors per lane: K = KV*V columns per lane,
// 64*K per wave; the halo is TS columns rounded up to whole vectors.
template <typename T, int KV> constexpr int march_k(int ts) { return KV * lane_elems<T>(ts); }
template <typename T, int KV> constexpr int march_halo(int ts) {
    return ((ts + lane_elems<T>(ts) - 1) / lane_elems<T>(ts)) * lane_elems<T>(ts);
}
template <typename T, int KV> constexpr int march_out_width(int ts) {
    return 64 * march_k<T, KV>(ts) - 2 * march_halo<T, KV>(ts);
}

// One wave's march over output rows [row_out0, row_out1) and output columns
// [col_out0, col_out0 + OW).
// VEC: rows aligned to the lane vector, KV vector accesses per lane and row.
// LPOL/SPOL: cache policy bits of the loads/stores (2 = non-temporal).
// FUSED: cells use five_point_fused, and the lane adds up |x| over every value
// it loads; the return value is true when that sum is not below `limit` (or is
// NaN), in which case the stored results may differ from the separate form
// and the caller recomputes the tile with FUSED off.
// Boundary handling, for tiles some of whose computed cells lie on or outside
// the grid's edge: EF (with FUSED) as described below; EDGE (the separate
// form's fallback) forces every such cell to 0 with per-cell row/column masks.
// Interior tiles take neither and run without masks.
// balance: the wave lowers its issue priority as it progresses (below).
template <typename T, int TS, int KV, bool VEC, bool EDGE, bool DOWN, int LPOL, int SPOL, bool FUSED,
          int EF = 0>
__device__ __forceinline__ bool march(const T *__restrict__ src, T *__restrict__ dst, int nx,
                                      int ny, int ld, T a, T limit, int lane, int col_out0,
                                      int row_out0, int row_out1, bool balance) {
    constexpr int V = lane_elems<T>(TS);
    constexpr int K = march_k<T, KV>(TS);
    constexpr int HALO = march_halo<T, KV>(TS);
    constexpr int OW = march_out_width<T, KV>(TS);
    constexpr int ES = (int)sizeof(T);

    const int c0 = col_out0 - HALO + lane * K;  // first column this lane holds
    bool colin[K];                              // column is an interior column
#pragma unroll
    for (int e = 0; e < K; ++e) colin[e] = (EDGE || (EF & 1)) ? (c0 + e >= 1 && c0 + e <= nx - 2) : true;
    // Fused form on the grid's edge (EF, with FUSED): bit 1, the strip holds
    // column 0 or nx-1: loads of non-interior columns are masked to 0 and the
    // two boundary columns take the coefficient 0 instead of alpha (c = 0 and
    // t finite, which the overflow guard ensures, so c + 0*t is +0 exactly);
    // columns beyond the boundary only ever feed the boundary column.  Bit 2,
    // the tile reaches row 0 or ny-1: a level's row that is a boundary row or
    // lies outside the grid is not computed but held at 0.
    T ae[K];
#pragma unroll
    for (int e = 0; e < K; ++e) ae[e] = ((EF & 1) && (c0 + e == 0 || c0 + e == nx - 1)) ? T(0) : a;

    // DOWN marches from the top of the tile to its bottom (rows decreasing);
    // vertically adjacent tiles march in opposite directions so that the halo
    // rows they share are read by both at about the same time, while they are
    // still in L2.
    constexpr int DR = DOWN ? -1 : 1;        // row step of the march
    const int r_first = DOWN ? row_out1 - 1 + TS : row_out0 - TS;  // first input row
    const int nit = row_out1 - row_out0 + 2 * TS;
    const int nit3 = ((nit + 2) / 3) * 3;    // three-phase unrolled loop

    // Load descriptor: the interior rows this wave may read.
    const int lr0 = max(1, row_out0 - TS);
    const int lr1 = min(ny - 2, row_out1 - 1 + TS);
    const __amdgpu_buffer_rsrc_t rin =
        make_rsrc(src + (long)lr0 * ld, lr1 >= lr0 ? (uint32_t)(lr1 - lr0 + 1) * (uint32_t)ld * ES : 0u);
    // Store descriptor: the rows this wave owns.
    const __amdgpu_buffer_rsrc_t rout =
        make_rsrc(dst + (long)row_out0 * ld, (uint32_t)(row_out1 - row_out0) * (uint32_t)ld * ES);
    const uint32_t row_bytes = (uint32_t)ld * ES;
    // Byte offsets within a row.  Cells this lane must not store (halo
    // columns, columns past nx) get an offset outside every descriptor.
    uint32_t st_off[K];
#pragma unroll
    for (int e = 0; e < K; ++e) {
        const int c = c0 + e;
        st_off[e] = (c >= col_out0 && c < col_out0 + OW && c < nx) ? (uint32_t)c * ES : kOutOfRange;
    }
    uint32_t st_vec[KV];  // whole-vector stores (interior strips)
#pragma unroll
    for (int v = 0; v < KV; ++v) {
        const int c = c0 + v * V;
        st_vec[v] = (c >= col_out0 && c < col_out0 + OW) ? (uint32_t)c * ES : kOutOfRange;
    }

    T win[TS][3][K];  // win[s][slot][e]: level-s rows, slot = row phase mod 3
    T pre[3][K];      // level-0 rows in flight, three rows ahead
#pragma unroll
    for (int s = 0; s < TS; ++s)
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int e = 0; e < K; ++e) win[s][p][e] = T(0);

    T checksum = T(0);  // FUSED: sum of |x| over the lane's loads

    // Row r of the input: rows outside [lr0, lr1] read as 0 through the
    // descriptor range (also rows 0 and ny-1, which are edge rows).  Columns
    // left of column 0 (the first strip's left halo) give wrapped offsets
    // outside the descriptor and read 0 as well (they are masked anyway).
    // That relies on no lane holding columns on both sides of column 0: the
    // compiler may merge a lane's adjacent loads into one wider access, and
    // the range check of such an access does not wrap, so a merged access
    // starting left of column 0 also reads 0 for the columns from 0 on.
    // The halo is a whole number of lane widths (asserted in k_march), so a
    // lane's columns are all left of column 0 or none are.
    auto load_row = [&](T (&x)[K], int r) {
        const uint32_t roff = (uint32_t)(r - lr0) * row_bytes;
        if (VEC) {
#pragma unroll
            for (int v = 0; v < KV; ++v)
                buf_load_vec<LPOL, V>(x, v * V, rin, roff + (uint32_t)(c0 + v * V) * ES);
        } else {
#pragma unroll
            for (int e = 0; e < K; ++e)
                x[e] = buf_load_elem<LPOL>((T *)nullptr, rin, roff + (uint32_t)(c0 + e) * ES);
        }
        if (EDGE || (EF & 1)) {
#pragma unroll
            for (int e = 0; e < K; ++e) x[e] = colin[e] ? x[e] : T(0);
        }
        if (FUSED) {
#pragma unroll
            for (int e = 0; e < K; ++e) checksum = checksum + __builtin_fabs(x[e]);
        }
    };

#pragma unroll
    for (int p = 0; p < 3; ++p) load_row(pre[p], r_first + DR * p);

    auto step = [&](auto phase, int it) {
        constexpr int P = decltype(phase)::value;
        constexpr int PC = (P + 2) % 3;  // previous row (centre for the next level)
        constexpr int PO = (P + 1) % 3;  // row before that
        // Rows q-1 (south) and q+1 (north) of the level below: marching up the
        // newest row is north, marching down it is south.
        constexpr int PSOUTH = DOWN ? P : PO;
        constexpr int PNORTH = DOWN ? PO : P;
        const int r = r_first + DR * it;
#pragma unroll
        for (int e = 0; e < K; ++e) win[0][P][e] = pre[P][e];
        load_row(pre[P], r + DR * 3);
        T out[K];
#pragma unroll
        for (int e = 0; e < K; ++e) out[e] = T(0);
#pragma unroll
        for (int s = 1; s <= TS; ++s) {
            if ((EF & 2) && it >= 2 * s && !(r - DR * s >= 1 && r - DR * s <= ny - 2)) {
                if (s < TS) {
#pragma unroll
                    for (int e = 0; e < K; ++e) win[s < TS ? s : 0][P][e] = T(0);
                }
            } else if (it >= 2 * s) {  // level s row r - DR*s depends only on loaded rows
                const int q = r - DR * s;
                const bool rowin = !EDGE || (q >= 1 && q <= ny - 2);
                const T wl = wave_shr1(win[s - 1][PC][K - 1]);
                const T er = wave_shl1(win[s - 1][PC][0]);
                T res[K];
#pragma unroll
                for (int e = 0; e < K; ++e) {
                    const T w = e == 0 ? wl : win[s - 1][PC][e - 1];
                    const T ee = e == K - 1 ? er : win[s - 1][PC][e + 1];
                    T val = FUSED ? five_point_fused(w, ee, win[s - 1][PSOUTH][e], win[s - 1][PNORTH][e],
                                                     win[s - 1][PC][e], (EF & 1) ? ae[e] : a)
                                  : five_point(w, ee, win[s - 1][PSOUTH][e], win[s - 1][PNORTH][e],
                                               win[s - 1][PC][e], a);
                    if (EDGE) val = (colin[e] && rowin) ? val : T(0);
                    res[e] = val;
                }
#pragma unroll
                for (int e = 0; e < K; ++e) {
                    if (s < TS)
                        win[s < TS ? s : 0][P][e] = res[e];
                    else
                        out[e] = res[e];
                }
            }
        }
        // Row r - DR*TS of the last level; rows outside [row_out0, row_out1)
        // and discarded cells fall outside the store descriptor and are dropped.
        const uint32_t qoff = (uint32_t)(r - DR * TS - row_out0) * row_bytes;
        if (VEC && !EDGE && !(EF & 1)) {
#pragma unroll
            for (int v = 0; v < KV; ++v) buf_store_vec<SPOL, V>(out, v * V, rout, qoff + st_vec[v]);
        } else {
#pragma unroll
            for (int e = 0; e < K; ++e) buf_store_elem<SPOL>(out[e], rout, qoff + st_off[e]);
        }
    };

    // Issue priority falls as the march nears its end: 3 for the first half
    // of the rows, then 2, 1 and 0 from 1/2, 3/4 and 7/8 of the way.  The
    // SIMD's arbiter otherwise favours its oldest wave, which then finishes
    // well ahead of the others and leaves the last one to run alone at a
    // fraction of the VALU rate for the end of the launch; with falling
    // priority, waves that are ahead yield to those behind and the waves of
    // a SIMD finish close together.  The host turns this off (`balance`) for
    // the memory-bound shallow depths and for launches with fewer than two
    // waves per SIMD, which keep the default priority.
    // One compare per iteration: `next` is the iteration of the next drop.
    // Only depths of five and up ever balance; shallower marches compile
    // without the check.
    constexpr bool kBalanced = TS >= 5;
    constexpr int kTop = 3;
    int prio = kTop;
    int stage = 0;
    int next = (kBalanced && balance) ? nit3 / 2 : INT_MAX;
    if (kBalanced && balance) __builtin_amdgcn_s_setprio(kTop);
    for (int it = 0; it < nit3; it += 3) {
        if (kBalanced && it >= next) {
            ++stage;
            prio = prio > 0 ? prio - 1 : 0;
            if (prio == 2) __builtin_amdgcn_s_setprio(2);
            else if (prio == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            next = stage == 1 ? nit3 * 3 / 4 : (stage == 2 ? nit3 * 7 / 8 : INT_MAX);
        }
        step(std::integral_constant<int, 0>{}, it);
        step(std::integral_constant<int, 1>{}, it + 1);
        step(std::integral_constant<int, 2>{}, it + 2);
    }
    return FUSED && !(checksum < limit);
}

// One tile in the fused form, with the boundary handling its position needs
// (EF above; edge tiles then cost about what interior tiles do, so no SIMD
// holding one finishes late).  A wave whose inputs could push 4c past the
// overflow threshold recomputes its tile in the separate form with per-cell
// masks (same stores, now with the definition's bits).
template <typename T, int TS, int KV, bool VEC, bool DOWN, int LPOL, int SPOL>
__device__ __forceinline__ void march_tile(const T *src, T *dst, const MarchArgs &g, T a, T limit,
                                           int lane, bool cols_in, bool rows_in, bool bal,
                                           int col_out0, int row_out0, int row_out1) {
    bool redo;
    if (cols_in && rows_in)
        redo = march<T, TS, KV, VEC, false, DOWN, LPOL, SPOL, true, 0>(
            src, dst, g.nx, g.ny, g.ld, a, limit, lane, col_out0, row_out0, row_out1, bal);
    else if (rows_in)
        redo = march<T, TS, KV, VEC, false, DOWN, LPOL, SPOL, true, 1>(
            src, dst, g.nx, g.ny, g.ld, a, limit, lane, col_out0, row_out0, row_out1, bal);
    else
        redo = march<T, TS, KV, VEC, false, DOWN, LPOL, SPOL, true, 3>(
            src, dst, g.nx, g.ny, g.ld, a, limit, lane, col_out0, row_out0, row_out1, bal);
    if (__any(redo))
        march<T, TS, KV, VEC, true, DOWN, LPOL, SPOL, false>(src, dst, g.nx, g.ny, g.ld, a, limit, lane,
                                                            col_out0, row_out0, row_out1, bal);
}

template <typename T, int TS, int KV, bool VEC, int LPOL, int SPOL>
__global__ __launch_bounds__(256) void k_march(MarchArgs g) {
    constexpr int K = march_k<T, KV>(TS);
    constexpr int HALO = march_halo<T, KV>(TS);
    constexpr int OW = march_out_width<T, KV>(TS);
    static_assert(OW > 0, "time block too deep for the strip width");
    static_assert(HALO % K == 0, "a lane must not hold columns on both sides of column 0");
    const int lane = threadIdx.x & 63;
    // The wave index is uniform across the wave; saying so keeps the tile
    // coordinates, and the buffer descriptors built from them, in SGPRs.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = xcd_remap(blockIdx.x, gridDim.x) * 4 + wave;
    if (tile >= g.ntiles) return;  // whole wave leaves; the kernel has no barriers
    const int field = tile / g.field_tiles;
    const int ftile = tile - field * g.field_tiles;
    const int strip = ftile % g.nstrips;
    const int rtile = ftile / g.nstrips;
    const int col_out0 = strip * OW;
    const int row_out0 = rtile * g.tile_rows;
    const int row_out1 = min(row_out0 + g.tile_rows, g.ny);
    const T *src = static_cast<const T *>(g.src[field]);
    T *dst = static_cast<T *>(g.dst[field]);
    const T a = T(g.alpha);
    const int span0 = col_out0 - HALO;  // first column of the strip
    // Rows formed at any level lie within [row_out0 - TS - 2, row_out1 + TS + 1]
    // (the three-phase loop may run two rows past the last needed one).
    const bool cols_in = span0 >= 1 && span0 + 64 * K <= g.nx - 1;
    const bool rows_in = row_out0 - TS - 2 >= 1 && row_out1 + TS + 2 <= g.ny - 2;
    const T limit = T(g.fuse_limit);
    const bool bal = g.balance != 0;
    if (rtile & 1)
        march_tile<T, TS, KV, VEC, true, LPOL, SPOL>(src, dst, g, a, limit, lane, cols_in, rows_in, bal,
                                                     col_out0, row_out0, row_out1);
    else
        march_tile<T, TS, KV, VEC, false, LPOL, SPOL>(src, dst, g, a, limit, lane, cols_in, rows_in, bal,
                                                      col_out0, row_out0, row_out1);
}

// ---------------------------------------------------------------------------
// Resident sweep for small grids: every step in one launch
// ---------------------------------------------------------------------------

// A grid of at most 64 columns and W*R rows lives in the registers of one
// workgroup of W waves (sixteen, or eight for tall FP32 grids): lane i holds
// column i, wave w holds rows [w*R, w*R + R).  West/east neighbours cross lanes with DPP; north/south
// come from the lane's own rows, except at a wave's first and last row, whose
// neighbours are the adjacent waves' last and first rows: each step every
// wave publishes those two rows in LDS (two slot sets used alternately, so
// one barrier per step suffices) and reads its neighbours'.  Ring cells and
// cells outside the grid hold 0 and are never updated.  On return `dst`
// holds the state after `steps` steps and `prev` the state one step earlier,
// as alternating sweeps would leave them; both include the zero ring.
// `src` may equal `dst` or `prev`: all reads of `src` precede the first
// barrier, all writes follow it.
constexpr int kResidentWaves = 16;
constexpr int kResidentCols = 64;

// Fast form: when every loaded value is finite and below `fast_limit`, no
// value, partial sum or product of any step can overflow (the host bounds the
// growth over all steps), so t - 4c takes one fused multiply-add (exact while
// 4c is finite) and cells that are never updated take the coefficient 0
// instead of a select (c = 0 and t finite give c + 0*t = +0).  Otherwise the
// separate form with per-cell masks runs.  The choice is made once per
// workgroup, before the first step.
template <typename T, int R, int W = kResidentWaves>
__global__ __launch_bounds__(1024) void k_resident(ResidentFields f, int nx, int ny, int ld, T a,
                                                   int steps, T fast_limit) {
    // One workgroup per field.
    const T *src = static_cast<const T *>(f.src[blockIdx.x]);
    T *dst = static_cast<T *>(f.dst[blockIdx.x]);
    T *prev = static_cast<T *>(f.prev[blockIdx.x]);
    __shared__ T edge[2][W][2][kResidentCols];  // [slot set][wave][first, last row][lane]
    const int i = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j0 = w * R;
    const bool colin = i >= 1 && i <= nx - 2;
    T val[R];
    bool upd[R];
    bool small = true;  // every value this lane holds is finite and below fast_limit
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = j0 + r;
        upd[r] = colin && j >= 1 && j <= ny - 2;
        val[r] = upd[r] ? src[i + (long)ld * j] : T(0);
        small = small && __builtin_fabs(val[r]) < fast_limit;  // false for NaN
    }
    const bool fast = __syncthreads_and(small) != 0;  // uniform across the workgroup
    T ae[R];
#pragma unroll
    for (int r = 0; r < R; ++r) ae[r] = upd[r] ? a : T(0);

    auto run = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        for (int s = 0; s < steps; ++s) {
            const int set = s & 1;
            edge[set][w][0][i] = val[0];
            edge[set][w][1][i] = val[R - 1];
            __syncthreads();
            const T below = w > 0 ? edge[set][w - 1][1][i] : T(0);                   // row j0 - 1
            const T above = w < W - 1 ? edge[set][w + 1][0][i] : T(0);  // row j0 + R
            if (s == steps - 1) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int j = j0 + r;
                    if (i < nx && j < ny) prev[i + (long)ld * j] = val[r];
                }
            }
            T nv[R];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const T c = val[r];
                const T west = wave_shr1(c);
                const T east = wave_shl1(c);
                const T south = r == 0 ? below : val[r - 1];
                const T north = r == R - 1 ? above : val[r + 1];
                if (FAST)
                    nv[r] = five_point_fused(west, east, south, north, c, ae[r]);
                else
                    nv[r] = upd[r] ? five_point(west, east, south, north, c, a) : T(0);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) val[r] = nv[r];
        }
    };
    if (fast)
        run(std::true_type{});
    else
        run(std::false_type{});
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int j = j0 + r;
        if (i < nx && j < ny) dst[i + (long)ld * j] = val[r];
    }
}

// ---------------------------------------------------------------------------
// Host-side launch selection
// ---------------------------------------------------------------------------

// Launch shape (chosen from sweeps on MI355X): vectors per lane, cache
// policies, and the tile height.
constexpr int kLoadPolicy = 0;   // cache policy bits of the march's loads
constexpr int kStorePolicy = 0;  // ... and of its stores
// One lane vector per lane: two (wider strips, half the halo) cost more
// registers than they save and measured slower at every depth.
template <typename T> constexpr int vectors_per_lane(int) { return 1; }

// Tile height for fused depths of five or more.  Such a launch is bound by
// vector-ALU issue, and a SIMD holding w resident waves takes about
// w x (rows + 2*TS + 3) row steps divided by the efficiency of w resident
// waves.  Tile counts just above a multiple of the SIMD count put one more
// wave on some SIMDs, or start a short extra round, and sweeps show those
// 10-30% slower; so each candidate takes the lowest height whose tile count
// fits w waves per SIMD exactly, for w = 1..occupancy (one round) and for
// whole rounds of `occupancy` waves, and the cheapest candidate wins.  The
// efficiency of w resident waves relative to a full SIMD fits (w/occupancy)^0.7
// in sweeps over 2048^2..16384^2 grids at depths 8-10 in FP64 and FP32 on
// MI355X (waves with falling issue priority, as the march sets it): one
// full round beat every partial one.  Tiles taller than 160 rows measured up
// to 4% slower at 16384^2, beyond the on-package cache, and at most 1%
// faster at 8192^2, so taller candidates are left out.
constexpr double kOccupancyExponent = 0.7;
constexpr long kMaxTileRows = 160;

long march_tile_rows(long ny, long nstrips, int ts, int occupancy, long simds, long max_rows) {
    const long cap = max_rows < kMaxTileRows ? max_rows : kMaxTileRows;
    double best = 0.0;
    long best_rows = -1;
    auto consider = [&](long waves_per_simd, double eff) {
        const long row_tiles = waves_per_simd * simds / nstrips;
        if (row_tiles < 1) return;
        const long rows = (ny + row_tiles - 1) / row_tiles;
        if (rows > cap) return;
        const double cost = (double)waves_per_simd * (double)(rows + 2 * ts + 3) / eff;
        if (best_rows < 0 || cost < best) {
            best = cost;
            best_rows = rows;
        }
    };
    for (int w = 1; w <= occupancy; ++w)
        consider(w, std::pow((double)w / (double)occupancy, kOccupancyExponent));
    // Whole rounds: the fewest that bring the height under the cap (more
    // rounds only add halo rows).
    const long slots = (long)occupancy * simds;
    const long row_tiles_needed = (ny + cap - 1) / cap;
    long rounds = (row_tiles_needed * nstrips + slots - 1) / slots;
    if (rounds < 2) rounds = 2;
    consider(rounds * occupancy, 1.0);
    return best_rows > 0 ? best_rows : cap;
}

// Largest sum of |input| over a wave's loads for which no level of a TS-deep
// fused launch can bring 4c near overflow.  One level grows the largest
// magnitude by at most 1 + 8|alpha| exactly, times the rounding of its six
// operations (1 + 2^-16 covers FP32 and FP64); inputs below the limit keep
// |c| <= 2^(emax-2) (2^1021, 2^125) at every level, so 4c and the partial
// sums stay finite.  A NaN or infinite alpha gives 0: never fused.
template <typename T> double march_fuse_limit(double alpha, int ts) {
    const double growth = (1.0 + 8.0 * __builtin_fabs(alpha)) * (1.0 + 0x1p-16);
    double lim = sizeof(T) == 8 ? 0x1p1021 : 0x1p125;
    for (int i = 0; i < ts; ++i) lim /= growth;
    return lim > 0.0 ? lim : 0.0;
}

// Largest |input| for which the resident kernel's fast form is exact over
// `steps` steps: every value then stays below 2^(emax-4) (2^1019, 2^123), so
// 4c, the partial sums and t (at most 8 times the largest value) stay finite
// and a never-updated cell keeps c + 0*t = +0.  In exact arithmetic a step
// is v = (1 - 4a) c + a (W + E + S + N), so the largest magnitude grows by at
// most g = |1 - 4a| + 4|a| (1 for 0 <= a <= 1/4); the six roundings add less
// than 41 (|a| + 1) units of roundoff u of the old largest magnitude, taken
// here as 64 (|a| + 1) u.  0 (never fast) when the bound underflows.
template <typename T> double resident_fast_limit(double alpha, int steps) {
    const double a = __builtin_fabs(alpha);
    const double u = sizeof(T) == 8 ? 0x1p-53 : 0x1p-24;
    const double growth = __builtin_fabs(1.0 - 4.0 * alpha) + 4.0 * a + 64.0 * (a + 1.0) * u;
    const double lim = (sizeof(T) == 8 ? 0x1p1019 : 0x1p123) * std::pow(growth, -(double)steps);
    return lim > 0.0 ? lim : 0.0;
}

template <typename T, int TS, int KV>
int launch_march_kv(const FieldPairs &f, const DiffPlan &p, double alpha, hipStream_t s) {
    MarchArgs g{};
    for (int k = 0; k < f.n; ++k) {
        g.src[k] = f.src[k];
        g.dst[k] = f.dst[k];
    }
    g.nx = p.nx;
    g.ny = p.ny;
    g.ld = p.ld;
    g.alpha = alpha;
    g.fuse_limit = march_fuse_limit<T>(alpha, TS);
    const int ow = march_out_width<T, KV>(TS);
    g.nstrips = (p.nx + ow - 1) / ow;
    // Strips of all fields: the tile model sees the fields side by side.
    const long strips_all = (long)g.nstrips * f.n;
    // Keep every descriptor within 2^30 bytes and every offset a wave can
    // form (its rows plus the halo and prefetch rows around them) below
    // 2^30, so that offsets outside a wave's rows, and the out-of-range
    // marker added to any of them, never land back inside a descriptor.
    const long row_bytes = (long)p.ld * (long)sizeof(T);
    const long max_rows = (1L << 30) / row_bytes - 2 * TS - 8;
    if (max_rows < 1) return fail(SGC_ERANGE, "grid rows too wide for the marching sweep");
    constexpr uintptr_t VB = sizeof(T) * lane_elems<T>(TS);
    bool vec = ((uintptr_t)p.ld * sizeof(T)) % VB == 0;
    for (int k = 0; k < f.n; ++k)
        vec = vec && reinterpret_cast<uintptr_t>(f.src[k]) % VB == 0 &&
              reinterpret_cast<uintptr_t>(f.dst[k]) % VB == 0;
    auto kernel = vec ? k_march<T, TS, KV, true, kLoadPolicy, kStorePolicy>
                      : k_march<T, TS, KV, false, kLoadPolicy, kStorePolicy>;
    // A 256-thread workgroup puts one wave on each SIMD of a CU, so resident
    // workgroups per CU is also resident waves per SIMD.
    static SlotCache cache[2];
    int per_cu = 0, cus = 0;
    const int rc = resident_slots(reinterpret_cast<const void *>(kernel), 256, cache[vec], &per_cu, &cus);
    if (rc != SGC_OK) return rc;
    long rows = p.tile_rows;
    if (rows <= 0) {
        const long model_rows = march_tile_rows(p.ny, strips_all, TS, per_cu, 4L * cus, max_rows);
        if (TS <= 2) {
            rows = 4;  // memory bound: many short tiles in flight
        } else if (TS == 3) {
            rows = 8;
        } else if (TS == 4) {
            // Between memory and ALU bound: about 8192 tiles of 16 to 128 rows.
            rows = max(16L, min((long)p.ny * strips_all / 8192, 128L));
        } else {
            rows = model_rows;
        }
        // A grid too small to fill one round of resident waves at the fixed
        // heights is latency bound: each launch lasts as long as one wave's
        // march, so it takes the model's height (the shortest tiles that
        // spread the grid over the resident waves) instead.
        const long tiles = strips_all * ((p.ny + rows - 1) / rows);
        if (TS <= 4 && tiles < (long)per_cu * 4L * cus) rows = min(rows, model_rows);
    }
    rows = min(rows, (long)p.ny);
    rows = min(rows, max_rows);
    g.tile_rows = (int)rows;
    const long field_tiles = (long)g.nstrips * ((p.ny + rows - 1) / rows);
    const long ntiles = field_tiles * f.n;
    if (ntiles > 0x7fffffffL - 3) return fail(SGC_ERANGE, "too many tiles");
    g.field_tiles = (int)field_tiles;
    g.ntiles = (int)ntiles;
    // Progress balancing pays where the march is bound by VALU issue (depth
    // five and up) and the SIMDs hold two or more waves; the memory-bound
    // shallow depths measured 5-13% slower with it.
    g.balance = (TS >= 5 && ntiles >= 2L * 4L * cus) ? 1 : 0;
    const int blocks = (int)((ntiles + 3) / 4);
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, s, g);
    return check_launch("diffusion march kernel");
}

template <typename T, int TS>
int launch_march_ts(const FieldPairs &f, const DiffPlan &p, double alpha, hipStream_t s) {
    return launch_march_kv<T, TS, vectors_per_lane<T>(TS)>(f, p, alpha, s);
}

template <typename T>
int launch_march(const FieldPairs &f, const DiffPlan &p, double alpha, int ts, hipStream_t s) {
    switch (ts) {
#define SGC_TS_CASE(n) \
    case n: return launch_march_ts<T, n>(f, p, alpha, s);
        SGC_TS_CASE(1) SGC_TS_CASE(2) SGC_TS_CASE(3) SGC_TS_CASE(4)
        SGC_TS_CASE(5) SGC_TS_CASE(6) SGC_TS_CASE(7) SGC_TS_CASE(8)
        SGC_TS_CASE(9) SGC_TS_CASE(10) SGC_TS_CASE(11) SGC_TS_CASE(12)
#undef SGC_TS_CASE
    default: return fail(SGC_ERANGE, "time block out of range");
    }
}
static_assert(SGC_MAX_TIME_BLOCK == 12, "launch_march instantiates 1..12");

template <typename T>
int sweep_t(const void *src, void *dst, const DiffPlan &p, double alpha, int map, int ts,
            hipStream_t s) {
    const T *in = static_cast<const T *>(src);
    T *out = static_cast<T *>(dst);
    const T a = T(alpha);
    switch (map) {
    case SGC_DIFF_COLLAPSE_BRANCH: {
        const long n = (long)p.nx * p.ny;
        hipLaunchKernelGGL((k_collapse_branch<T>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           in, out, p.nx, p.ny, p.ld, a);
        return check_launch("collapse-branch sweep");
    }
    case SGC_DIFF_CONTIG:
        hipLaunchKernelGGL((k_contig<T>), dim3(p.ny - 2), dim3(256), 0, s, in, out, p.nx, p.ny, p.ld, a);
        return check_launch("contiguous-lane sweep");
    case SGC_DIFF_STRIDED:
        hipLaunchKernelGGL((k_strided<T>), dim3(p.nx - 2), dim3(256), 0, s, in, out, p.nx, p.ny, p.ld, a);
        return check_launch("strided-lane sweep");
    case SGC_DIFF_TILED:
    case SGC_DIFF_TEMPORAL: {
        FieldPairs f{};
        f.src[0] = src;
        f.dst[0] = dst;
        f.n = 1;
        return launch_march<T>(f, p, alpha, map == SGC_DIFF_TILED ? 1 : ts, s);
    }
    default:
        return fail(SGC_EINVAL, "unknown diffusion map");
    }
}

}  // namespace

int diffuse_zero_ring(void *buf, int dtype, int nx, int ny, int ld, hipStream_t s) {
    const int n = 2 * nx + 2 * ny;
    const dim3 grid((n + 255) / 256);
    if (dtype == SGC_F64)
        hipLaunchKernelGGL((k_zero_ring<double>), grid, dim3(256), 0, s, static_cast<double *>(buf), nx,
                           ny, ld);
    else
        hipLaunchKernelGGL((k_zero_ring<float>), grid, dim3(256), 0, s, static_cast<float *>(buf), nx,
                           ny, ld);
    return check_launch("edge-ring zeroing");
}

template <typename T>
int resident_t(const ResidentFields &f, int n, const DiffPlan &p, double alpha, int steps,
               hipStream_t s) {
    const T a = T(alpha);
    const T lim = T(resident_fast_limit<T>(alpha, steps));
    // Sixteen waves of four or eight rows; FP32 grids taller than 64 rows run
    // faster as eight waves of sixteen rows (fewer waves at the barrier; the
    // VALU work per step is smaller than in FP64), FP64 ones slower.
    if (p.ny <= kResidentWaves * 4) {
        hipLaunchKernelGGL((k_resident<T, 4>), dim3(n), dim3(1024), 0, s, f, p.nx, p.ny, p.ld, a, steps, lim);
    } else {
        if constexpr (sizeof(T) == 4)  // (the FP64 form of this shape is never built)
            hipLaunchKernelGGL((k_resident<T, 16, 8>), dim3(n), dim3(512), 0, s, f, p.nx, p.ny, p.ld, a, steps, lim);
        else
            hipLaunchKernelGGL((k_resident<T, 8>), dim3(n), dim3(1024), 0, s, f, p.nx, p.ny, p.ld, a, steps, lim);
    }
    return check_launch("diffusion resident sweep");
}

int diffuse_resident_fields(const ResidentFields &f, int n, int dtype, const DiffPlan &p,
                            double alpha, int steps, hipStream_t s) {
    if (p.nx > kResidentCols || p.ny > kResidentWaves * 8)
        return fail(SGC_ERANGE, "resident sweep: the grid must fit 64 columns and 128 rows");
    if (n < 1 || n > SGC_MAX_NVAR) return fail(SGC_EINVAL, "field count out of range");
    if (dtype == SGC_F64) return resident_t<double>(f, n, p, alpha, steps, s);
    return resident_t<float>(f, n, p, alpha, steps, s);
}

int diffuse_sweep(const void *src, void *dst, int dtype, const DiffPlan &p, double alpha, int map,
                  int steps_in_launch, hipStream_t s) {
    if (dtype == SGC_F64) return sweep_t<double>(src, dst, p, alpha, map, steps_in_launch, s);
    return sweep_t<float>(src, dst, p, alpha, map, steps_in_launch, s);
}

int diffuse_sweep_fields(const FieldPairs &f, int dtype, const DiffPlan &p, double alpha, int map,
                         int steps_in_launch, hipStream_t s) {
    if (f.n < 1 || f.n > SGC_MAX_NVAR) return fail(SGC_EINVAL, "field count out of range");
    if (map != SGC_DIFF_TILED && map != SGC_DIFF_TEMPORAL)
        return fail(SGC_EINVAL, "several fields per launch need the TILED or TEMPORAL map");
    const int ts = map == SGC_DIFF_TILED ? 1 : steps_in_launch;
    if (dtype == SGC_F64) return launch_march<double>(f, p, alpha, ts, s);
    return launch_march<float>(f, p, alpha, ts, s);
}

}  // namespace sgc
