// HIP kernels (gfx950 / CDNA4) and launchers of the multi-LoRA add-on.
//
// shrink  v[row][j] = sum_k x[row][k] A^T[s][j][k]      (Punica summary, "The SGMV Operator")
// expand  y[row][c] += scale[s] sum_j v[row][j] B[s][j][c]
//
// Both kernels run over a flat work-list of tiles (a tile = up to 64 consecutive rows
// of one segment, or one row in the per-row-slot form) instead of binding the adapter
// to a grid dimension, so segments of 1 to thousands of rows share one launch.  A
// workgroup is 4 wavefronts (256 lanes); workgroup ids are remapped so that the 8
// XCDs (which take workgroups round-robin) each own a contiguous range of work
// items, keeping the x rows and weights that neighbouring items share in one L2.
//
// Shrink.  Its output is only r wide, so parallelism comes from splitting the
// rank-rows of a tile over workgroups (jw rank-rows each) and d_in over the 4
// wavefronts of a workgroup.  The 4 partial sums are added in LDS in wavefront order:
// no cross-workgroup reduction, no atomics, no workspace, and the result does not
// depend on scheduling.
//   - few rows (< 8, the decode case): fp16 dot2 (v_dot2_f32_f16) on 16-byte
//     coalesced loads of x rows and A^T rank-rows, both contiguous in d_in.
//   - 8..64 rows: v_mfma_f32_16x16x32_f16, one 16-rank slice per workgroup; both
//     operands load straight from global memory (x rows and A^T rank-rows give each
//     lane 8 consecutive k values).
// Expand.  A workgroup owns 512 output columns of one tile.
//   - few rows: each wavefront reads a quarter of the rank-rows of B (16-byte loads,
//     contiguous in d_out), the quarters are added in LDS, and one fp32 -> fp16
//     rounding updates y.
//   - 8..64 rows: B[0:r][512 columns] is staged in LDS once and reused by every
//     16-row slice; the product D^T = B^T (s v)^T runs on v_mfma_f32_16x16x16_f16
//     with s*v split into fp16 hi + lo/2048 parts (two MFMAs) so that v keeps ~22
//     bits; the accumulator starts from y, and each lane updates 4 consecutive y
//     elements of one row.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "lora_internal.hpp"

namespace lora {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

struct WeightsDev {
    int32_t num_slots, d_in, d_out, r_max;
    const int32_t *rank;
    const float *scale;
    const uint16_t *a_t, *b;        // dense
    const uint16_t *pool;           // paged
    int64_t num_pages;
    int32_t page_elems;
    const int32_t *page_table;
    int64_t pt_entries;
    const int64_t *a_pt_off, *b_pt_off;
};

struct TileSrc {
    const lora_tile *tiles;   // segment form
    const int32_t *row_map;   // segment form, may be NULL
    int32_t n_pos;
    const int32_t *idx;       // per-row form
};

struct ShrinkArgs {
    float *v;
    int64_t ldv;
    const uint16_t *x;
    int64_t ldx;
    int32_t n_rows, n_tiles;
    TileSrc ts;
    WeightsDev w;
    int32_t jw, n_jg, grid;
};

struct ExpandArgs {
    uint16_t *y;
    int64_t ldy;
    const float *v;
    int64_t ldv;
    int32_t n_rows, n_tiles, n_cchunks, grid;
    int32_t mfma;  // the launch may contain MFMA tiles (LDS holds a B chunk)
    TileSrc ts;
    WeightsDev w;
};

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerPass = 4;
constexpr int kCols = 512;           // expand columns per workgroup
constexpr int kBStride = kCols;      // LDS row stride of the staged B chunk (halves)

struct TileInfo {
    int32_t slot, pos0, nrows, rank;
};

// Contiguous work ranges per XCD: workgroup b runs on XCD b % 8; grid % 8 == 0.
__device__ inline int work_item(int b, int grid) { return (b & 7) * (grid >> 3) + (b >> 3); }

// Resolves work tile `t`; rank 0 means "nothing to do" (no adapter, rank 0, or a
// slot outside the descriptor).
template <bool PERROW>
__device__ inline TileInfo load_tile(const TileSrc &ts, const WeightsDev &w, int t)
{
    TileInfo ti;
    if (PERROW) {
        ti.slot = ts.idx[t];
        ti.pos0 = t;
        ti.nrows = 1;
    } else {
        const lora_tile tl = ts.tiles[t];
        ti.slot = tl.slot;
        ti.pos0 = tl.pos0;
        ti.nrows = min(tl.nrows, LORA_MAX_TILE_ROWS);
    }
    ti.rank = 0;
    if (ti.slot >= 0 && ti.slot < w.num_slots && ti.nrows > 0) ti.rank = min(w.rank[ti.slot], w.r_max);
    return ti;
}

// Row of position `pos`, or -1 when it falls outside the row map or the row range.
template <bool PERROW>
__device__ inline int row_of(const TileSrc &ts, int pos, int n_rows)
{
    int row = pos;
    if (!PERROW && ts.row_map) row = (pos >= 0 && pos < ts.n_pos) ? ts.row_map[pos] : -1;
    return (row >= 0 && row < n_rows) ? row : -1;
}

// Address of elements e .. e+7 of rank-row j of A^T[s] (IS_B false) or B[s];
// NULL when a page-table entry or page id is out of range.
template <bool PAGED, bool IS_B>
__device__ inline const uint16_t *rank_row_ptr(const WeightsDev &w, int s, int j, int e)
{
    const int d = IS_B ? w.d_out : w.d_in;
    if (!PAGED) {
        const uint16_t *base = IS_B ? w.b : w.a_t;
        return base + ((int64_t)s * w.r_max + j) * d + e;
    } else {
        const int P = w.page_elems;
        const int64_t off = (IS_B ? w.b_pt_off[s] : w.a_pt_off[s]) + (int64_t)j * (d / P) + e / P;
        if (off < 0 || off >= w.pt_entries) return nullptr;
        const int64_t page = w.page_table[off];
        if (page < 0 || page >= w.num_pages) return nullptr;
        return w.pool + page * P + (e % P);
    }
}

__device__ inline uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ inline h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }

// fp32 += dot of 8 fp16 pairs (v_dot2_f32_f16; fp16 products are exact in fp32).
__device__ inline float dot8(uint4 a, uint4 b, float acc)
{
    acc = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), acc, false);
    acc = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), acc, false);
    return acc;
}

__device__ inline float h2f(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ inline uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

__device__ inline float wave_sum(float s)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    return s;
}

// ------------------------------------------------------------------------ shrink
// Rows without an MFMA tile: workgroup = one tile x rank-rows [j0, j1);
// RJ rank-rows per pass, d_in striped over all 256 lanes (16 bytes each).
template <bool PAGED, bool PERROW, int RJ>
__device__ void shrink_valu(const ShrinkArgs &a, const TileInfo &ti, int j0, int j1, float *red)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_oct = a.w.d_in >> 3;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    for (int rg = 0; rg < ti.nrows; rg += kRowsPerPass) {
        int rows[kRowsPerPass];
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
            rows[q] = (rg + q < ti.nrows) ? row_of<PERROW>(a.ts, ti.pos0 + rg + q, a.n_rows) : -1;
        for (int jb = j0; jb < j1; jb += RJ) {
            float acc[kRowsPerPass][RJ];
#pragma unroll
            for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
                for (int jj = 0; jj < RJ; ++jj) acc[q][jj] = 0.f;
            // two octets per lane per iteration keep more loads in flight
            for (int o = tid; o < n_oct; o += 2 * kThreads) {
                const int o2 = o + kThreads;
                const bool in2 = o2 < n_oct;
                uint4 xv[kRowsPerPass], xw[kRowsPerPass], av[RJ], aw[RJ];
#pragma unroll
                for (int q = 0; q < kRowsPerPass; ++q) {
                    const uint16_t *xr = a.x + (int64_t)(rows[q] < 0 ? 0 : rows[q]) * a.ldx;
                    xv[q] = rows[q] >= 0 ? load16(xr + 8 * o) : z4;
                    xw[q] = (rows[q] >= 0 && in2) ? load16(xr + 8 * o2) : z4;
                }
#pragma unroll
                for (int jj = 0; jj < RJ; ++jj) {
                    av[jj] = aw[jj] = z4;
                    if (jb + jj < j1) {
                        const uint16_t *p = rank_row_ptr<PAGED, false>(a.w, ti.slot, jb + jj, 8 * o);
                        if (p) av[jj] = load16(p);
                        if (in2) {
                            const uint16_t *p2 = rank_row_ptr<PAGED, false>(a.w, ti.slot, jb + jj, 8 * o2);
                            if (p2) aw[jj] = load16(p2);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
                    for (int jj = 0; jj < RJ; ++jj) acc[q][jj] = dot8(xw[q], aw[jj], dot8(xv[q], av[jj], acc[q][jj]));
            }
#pragma unroll
            for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
                for (int jj = 0; jj < RJ; ++jj) {
                    const float s = wave_sum(acc[q][jj]);
                    if (lane == 0) red[wave * kRowsPerPass * RJ + q * RJ + jj] = s;
                }
            __syncthreads();
            if (tid < kRowsPerPass * RJ) {
                const int q = tid / RJ, jj = tid - q * RJ;
                // wavefront order: the same sum for every launch of this shape
                const float s = red[tid] + red[kRowsPerPass * RJ + tid] + red[2 * kRowsPerPass * RJ + tid] +
                                red[3 * kRowsPerPass * RJ + tid];
                if (rows[q] >= 0 && jb + jj < j1) a.v[(int64_t)rows[q] * a.ldv + jb + jj] = s;
            }
            __syncthreads();
        }
    }
}

// 8..64 rows: MFMA 16x16x32 over (16-row slices) x (16 rank slice j0..j0+15); the 4
// wavefronts take interleaved 32-wide k-steps and their sums are added in LDS.
template <bool PAGED, bool PERROW>
__device__ void shrink_mfma(const ShrinkArgs &a, const TileInfo &ti, int j0, float *red)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;       // operand row/col, k-group of the lane
    const int MT = (ti.nrows + 15) >> 4;
    const int r = ti.rank;
    const int jcol = j0 + li;                        // this lane's rank column (B operand)
    int xrow[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rr = 16 * mt + li;
        xrow[mt] = (mt < MT && rr < ti.nrows) ? row_of<PERROW>(a.ts, ti.pos0 + rr, a.n_rows) : -1;
    }
    f4_t acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = f4_t{0.f, 0.f, 0.f, 0.f};
    const int d_in = a.w.d_in;
    const int steps = (d_in + 31) >> 5;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    for (int s = wave; s < steps; s += kWaves) {
        const int k = 32 * s + 8 * lg;
        const bool kin = k < d_in;
        uint4 bq = z4;
        if (kin && jcol < r) {
            const uint16_t *p = rank_row_ptr<PAGED, false>(a.w, ti.slot, jcol, k);
            if (p) bq = load16(p);
        }
        const h8_t bop = __builtin_bit_cast(h8_t, bq);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt >= MT) break;
            const uint4 xq = (kin && xrow[mt] >= 0) ? load16(a.x + (int64_t)xrow[mt] * a.ldx + k) : z4;
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xq), bop, acc[mt], 0, 0, 0);
        }
    }
    // D layout: lane holds rows 4*lg + e of the slice, rank column li.
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave * 1024 + mt * 256 + (4 * lg + e) * 16 + li] = acc[mt][e];
    __syncthreads();
    for (int o = tid; o < MT * 256; o += kThreads) {
        const int mt = o >> 8, i = (o >> 4) & 15, j = o & 15;
        const int rr = 16 * mt + i, col = j0 + j;
        if (rr >= ti.nrows || col >= a.w.r_max) continue;
        const int row = row_of<PERROW>(a.ts, ti.pos0 + rr, a.n_rows);
        if (row < 0) continue;
        const float s = red[o] + red[1024 + o] + red[2048 + o] + red[3072 + o];
        a.v[(int64_t)row * a.ldv + col] = col < r ? s : 0.f;
    }
}

template <bool PAGED, bool PERROW, int RJ>
__global__ __launch_bounds__(kThreads) void lora_shrink_kernel(ShrinkArgs a)
{
    __shared__ float red[kWaves * 1024];
    const int wi = work_item(blockIdx.x, a.grid);
    const int tile = wi / a.n_jg;
    if (tile >= a.n_tiles) return;
    const int jg = wi - tile * a.n_jg;
    const TileInfo ti = load_tile<PERROW>(a.ts, a.w, tile);
    if (ti.rank <= 0) return;
    const int j0 = jg * a.jw;
    const int jend = min(j0 + a.jw, a.w.r_max);
    if (j0 >= jend) return;
    if (!PERROW && ti.nrows >= kMfmaMinRows && a.jw == 16 && j0 < ti.rank) {
        shrink_mfma<PAGED, PERROW>(a, ti, j0, red);
        return;
    }
    // columns rank .. r_max-1 of the tile's rows are zero
    const int z0 = max(j0, ti.rank);
    if (z0 < jend) {
        const int zc = jend - z0;
        for (int e = threadIdx.x; e < ti.nrows * zc; e += kThreads) {
            const int row = row_of<PERROW>(a.ts, ti.pos0 + e / zc, a.n_rows);
            if (row >= 0) a.v[(int64_t)row * a.ldv + z0 + e % zc] = 0.f;
        }
    }
    const int j1 = min(jend, ti.rank);
    if (j0 < j1) shrink_valu<PAGED, PERROW, RJ>(a, ti, j0, j1, red);
}

// ------------------------------------------------------------------------ expand
template <bool PAGED, bool PERROW>
__device__ void expand_valu(const ExpandArgs &a, const TileInfo &ti, int c0, float *red)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = c0 + 8 * lane;
    const bool cin = c < a.w.d_out;
    const int r = ti.rank;
    const float sc = a.w.scale[ti.slot];
    for (int rg = 0; rg < ti.nrows; rg += kRowsPerPass) {
        int rows[kRowsPerPass];
        float sv[kRowsPerPass];  // lane j holds scale * v[row][j]
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q) {
            rows[q] = (rg + q < ti.nrows) ? row_of<PERROW>(a.ts, ti.pos0 + rg + q, a.n_rows) : -1;
            sv[q] = (rows[q] >= 0 && lane < r) ? sc * a.v[(int64_t)rows[q] * a.ldv + lane] : 0.f;
        }
        float acc[kRowsPerPass][8];
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
        // wavefront w takes rank-rows w, w+4, ...; four of them per pass in flight
        for (int jb = wave; jb < r; jb += 4 * kWaves) {
            uint4 bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = jb + u * kWaves;
                bv[u] = make_uint4(0, 0, 0, 0);
                if (cin && j < r) {
                    const uint16_t *p = rank_row_ptr<PAGED, true>(a.w, ti.slot, j, c);
                    if (p) bv[u] = load16(p);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = jb + u * kWaves;
                if (j >= r) break;
                const uint32_t bw[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
                float bf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bf[2 * e] = h2f((uint16_t)(bw[e] & 0xffff));
                    bf[2 * e + 1] = h2f((uint16_t)(bw[e] >> 16));
                }
#pragma unroll
                for (int q = 0; q < kRowsPerPass; ++q) {
                    const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv[q]), j));
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[q][e] = __builtin_fmaf(s, bf[e], acc[q][e]);
                }
            }
        }
        // red[wave][q][e][lane]
#pragma unroll
        for (int q = 0; q < kRowsPerPass; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[((wave * kRowsPerPass + q) * 8 + e) * 64 + lane] = acc[q][e];
        __syncthreads();
        {
            const int q = wave;  // wavefront q updates row q of the pass
            if (rows[q] >= 0 && cin) {
                uint16_t *yp = a.y + (int64_t)rows[q] * a.ldy + c;
                const uint4 yv = load16(yp);
                const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
                uint32_t out[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    float d[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int e = 2 * e2 + h;
                        d[h] = red[((0 * kRowsPerPass + q) * 8 + e) * 64 + lane] +
                               red[((1 * kRowsPerPass + q) * 8 + e) * 64 + lane] +
                               red[((2 * kRowsPerPass + q) * 8 + e) * 64 + lane] +
                               red[((3 * kRowsPerPass + q) * 8 + e) * 64 + lane];
                    }
                    const float lo = h2f((uint16_t)(yw[e2] & 0xffff)) + d[0];
                    const float hi = h2f((uint16_t)(yw[e2] >> 16)) + d[1];
                    out[e2] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
                }
                *reinterpret_cast<uint4 *>(yp) = make_uint4(out[0], out[1], out[2], out[3]);
            }
        }
        __syncthreads();
    }
}

// 8..64 rows: B chunk in LDS (row k at a column rotation of 8 * ((k >> 2) & 3)
// halves, so the 4 k-groups of a wavefront read different banks), then per 16-row
// slice D^T[cols][rows] = B^T (s v)^T with hi/lo fp16 operands.
template <bool PAGED, bool PERROW>
__device__ void expand_mfma(const ExpandArgs &a, const TileInfo &ti, int c0, uint16_t *lds_b)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int r = ti.rank;
    const int rk = (r + 15) & ~15;  // ranks padded to the 16-wide k-step
    // stage B[0:rk][c0:c0+512] (zeros past the rank or past d_out)
    for (int o = tid; o < rk * (kCols / 8); o += kThreads) {
        const int k = o >> 6, oc = (o & 63) * 8;
        uint4 q = make_uint4(0, 0, 0, 0);
        if (k < r && c0 + oc < a.w.d_out) {
            const uint16_t *p = rank_row_ptr<PAGED, true>(a.w, ti.slot, k, c0 + oc);
            if (p) q = load16(p);
        }
        const int pc = (oc + 8 * ((k >> 2) & 3)) & (kCols - 1);
        *reinterpret_cast<uint4 *>(lds_b + k * kBStride + pc) = q;
    }
    __syncthreads();
    const float sc = a.w.scale[ti.slot];
    const int MT = (ti.nrows + 15) >> 4;
    const int cw = c0 + 128 * wave;  // this wavefront's 128 columns = 8 slices of 16
    for (int mt = 0; mt < MT; ++mt) {
        const int rr = 16 * mt + li;
        const int row = rr < ti.nrows ? row_of<PERROW>(a.ts, ti.pos0 + rr, a.n_rows) : -1;
        f4_t acc_hi[8], acc_lo[8];
        // accumulator starts from y: lane holds y[row][cw + 16 nt + 4 lg + e]
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int col = cw + 16 * nt + 4 * lg;
            acc_lo[nt] = f4_t{0.f, 0.f, 0.f, 0.f};
            if (row >= 0 && col < a.w.d_out) {
                const uint2 yq = *reinterpret_cast<const uint2 *>(a.y + (int64_t)row * a.ldy + col);
                acc_hi[nt] = f4_t{h2f((uint16_t)(yq.x & 0xffff)), h2f((uint16_t)(yq.x >> 16)),
                                  h2f((uint16_t)(yq.y & 0xffff)), h2f((uint16_t)(yq.y >> 16))};
            } else {
                acc_hi[nt] = f4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        for (int kb = 0; kb < rk; kb += 16) {
            // B operand of the MFMA: (s v)^T, lane holds ranks kb + 4 lg .. +3 of its row
            const int j = kb + 4 * lg;
            float4 vq = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row >= 0 && j < r) vq = *reinterpret_cast<const float4 *>(a.v + (int64_t)row * a.ldv + j);
            const float sv[4] = {sc * vq.x, sc * vq.y, sc * vq.z, sc * vq.w};
            h4_t vhi, vlo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float m = (j + e < r) ? sv[e] : 0.f;
                const _Float16 h = (_Float16)m;
                vhi[e] = h;
                vlo[e] = (_Float16)((m - (float)h) * 2048.f);
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                // A operand: B^T, lane holds column cw + 16 nt + li, ranks j .. j+3
                const int lc = 128 * wave + 16 * nt + li;
                h4_t bop;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = j + e;
                    const int pc = (lc + 8 * ((k >> 2) & 3)) & (kCols - 1);
                    bop[e] = __builtin_bit_cast(_Float16, lds_b[k * kBStride + pc]);
                }
                acc_hi[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(bop, vhi, acc_hi[nt], 0, 0, 0);
                acc_lo[nt] = __builtin_amdgcn_mfma_f32_16x16x16f16(bop, vlo, acc_lo[nt], 0, 0, 0);
            }
        }
        if (row < 0) continue;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int col = cw + 16 * nt + 4 * lg;
            if (col >= a.w.d_out) continue;
            uint16_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = f2h(acc_hi[nt][e] + acc_lo[nt][e] * (1.f / 2048.f));
            *reinterpret_cast<uint2 *>(a.y + (int64_t)row * a.ldy + col) =
                make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        }
    }
}

template <bool PAGED, bool PERROW>
__global__ __launch_bounds__(kThreads) void lora_expand_kernel(ExpandArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int wi = work_item(blockIdx.x, a.grid);
    const int tile = wi / a.n_cchunks;
    if (tile >= a.n_tiles) return;
    const int cch = wi - tile * a.n_cchunks;
    const TileInfo ti = load_tile<PERROW>(a.ts, a.w, tile);
    if (ti.rank <= 0) return;
    if (!PERROW && a.mfma && ti.nrows >= kMfmaMinRows)
        expand_mfma<PAGED, PERROW>(a, ti, cch * kCols, reinterpret_cast<uint16_t *>(smem));
    else
        expand_valu<PAGED, PERROW>(a, ti, cch * kCols, reinterpret_cast<float *>(smem));
}

// ------------------------------------------------------------------------ launchers
// Event pair attached to this thread's next kernel launch (lora_set_launch_events).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

template <typename Kernel, typename Args>
void launch(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const Args &a)
{
    if (t_ev_start || t_ev_stop) {
        hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0, a);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, a);
    }
}

WeightsDev to_dev(const lora_weights *w)
{
    WeightsDev d;
    d.num_slots = w->num_slots;
    d.d_in = w->d_in;
    d.d_out = w->d_out;
    d.r_max = w->r_max;
    d.rank = w->rank;
    d.scale = w->scale;
    d.a_t = static_cast<const uint16_t *>(w->a_t);
    d.b = static_cast<const uint16_t *>(w->b);
    d.pool = static_cast<const uint16_t *>(w->pool);
    d.num_pages = w->num_pages;
    d.page_elems = w->page_elems;
    d.page_table = w->page_table;
    d.pt_entries = w->pt_entries;
    d.a_pt_off = w->a_pt_off;
    d.b_pt_off = w->b_pt_off;
    return d;
}

int launch_status(const char *what)
{
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LORA_E_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return LORA_OK;
}

int check_rows_arg(const void *p, int64_t ld, int32_t need, int32_t mult, const char *name)
{
    if (!p) return fail(LORA_E_NULL, "%s is NULL", name);
    if (!aligned16(p)) return fail(LORA_E_ALIGN, "%s must be 16-byte aligned", name);
    if (ld < need) return fail(LORA_E_SHAPE, "leading dimension of %s = %lld < %d", name, (long long)ld, need);
    if (ld % mult) return fail(LORA_E_ALIGN, "leading dimension of %s = %lld is not a multiple of %d", name,
                               (long long)ld, mult);
    return LORA_OK;
}

int check_segments(const lora_segments *seg)
{
    if (!seg) return fail(LORA_E_NULL, "segments descriptor is NULL");
    if (seg->n_tiles < 0 || seg->n_pos < 0) return fail(LORA_E_SHAPE, "n_tiles = %d, n_pos = %d", seg->n_tiles, seg->n_pos);
    if (seg->max_rows < 0 || seg->max_rows > LORA_MAX_TILE_ROWS)
        return fail(LORA_E_SHAPE, "max_rows = %d outside 0..%d", seg->max_rows, LORA_MAX_TILE_ROWS);
    if (seg->n_tiles > 0 && !seg->tiles) return fail(LORA_E_NULL, "tiles is NULL");
    if (seg->tiles && !aligned16(seg->tiles)) return fail(LORA_E_ALIGN, "tiles must be 16-byte aligned");
    return LORA_OK;
}

inline int32_t pad8(int64_t g) { return (int32_t)((g + 7) & ~int64_t(7)); }

template <bool PERROW>
int shrink_impl(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx, int32_t n_rows,
                const lora_weights *w, TileSrc ts, int32_t n_tiles, int32_t max_rows)
{
    int st = check_weights_desc(w);
    if (st) return st;
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0 || n_tiles == 0) return LORA_OK;
    if ((st = check_rows_arg(v, ldv, w->r_max, 4, "v"))) return st;
    if ((st = check_rows_arg(x, ldx, w->d_in, 8, "x"))) return st;
    const int32_t jw = plan_shrink_jw(n_tiles, w->r_max, max_rows);
    ShrinkArgs a;
    a.v = v;
    a.ldv = ldv;
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.n_rows = n_rows;
    a.n_tiles = n_tiles;
    a.ts = ts;
    a.w = to_dev(w);
    a.jw = jw;
    a.n_jg = (w->r_max + jw - 1) / jw;
    a.grid = pad8((int64_t)n_tiles * a.n_jg);
    const dim3 grid((unsigned)a.grid), block(kThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool paged = w->layout == LORA_LAYOUT_PAGED;
    if (jw == 1) {
        if (paged) launch(lora_shrink_kernel<true, PERROW, 1>, grid, block, 0, s, a);
        else launch(lora_shrink_kernel<false, PERROW, 1>, grid, block, 0, s, a);
    } else if (jw == 2) {
        if (paged) launch(lora_shrink_kernel<true, PERROW, 2>, grid, block, 0, s, a);
        else launch(lora_shrink_kernel<false, PERROW, 2>, grid, block, 0, s, a);
    } else {
        if (paged) launch(lora_shrink_kernel<true, PERROW, 4>, grid, block, 0, s, a);
        else launch(lora_shrink_kernel<false, PERROW, 4>, grid, block, 0, s, a);
    }
    return launch_status("shrink");
}

template <bool PERROW>
int expand_impl(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv, int32_t n_rows,
                const lora_weights *w, TileSrc ts, int32_t n_tiles, int32_t max_rows)
{
    int st = check_weights_desc(w);
    if (st) return st;
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0 || n_tiles == 0) return LORA_OK;
    if ((st = check_rows_arg(y, ldy, w->d_out, 8, "y"))) return st;
    if ((st = check_rows_arg(v, ldv, w->r_max, 4, "v"))) return st;
    ExpandArgs a;
    a.y = static_cast<uint16_t *>(y);
    a.ldy = ldy;
    a.v = v;
    a.ldv = ldv;
    a.n_rows = n_rows;
    a.n_tiles = n_tiles;
    a.n_cchunks = (w->d_out + kCols - 1) / kCols;
    a.grid = pad8((int64_t)n_tiles * a.n_cchunks);
    a.mfma = (!PERROW && max_rows >= kMfmaMinRows) ? 1 : 0;
    a.ts = ts;
    a.w = to_dev(w);
    const size_t lds_valu = (size_t)kWaves * kRowsPerPass * 8 * 64 * sizeof(float);
    const size_t lds_mfma = a.mfma ? (size_t)((w->r_max + 15) & ~15) * kBStride * sizeof(uint16_t) : 0;
    const size_t lds = std::max(lds_valu, lds_mfma);
    const dim3 grid((unsigned)a.grid), block(kThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (w->layout == LORA_LAYOUT_PAGED)
        launch(lora_expand_kernel<true, PERROW>, grid, block, lds, s, a);
    else
        launch(lora_expand_kernel<false, PERROW>, grid, block, lds, s, a);
    return launch_status("expand");
}

TileSrc seg_src(const lora_segments *seg)
{
    TileSrc ts{};
    ts.tiles = seg->tiles;
    ts.row_map = seg->row_map;
    ts.n_pos = seg->n_pos;
    return ts;
}

TileSrc row_src(const int32_t *idx)
{
    TileSrc ts{};
    ts.idx = idx;
    return ts;
}

inline int32_t seg_max_rows(const lora_segments *seg) { return seg->max_rows > 0 ? seg->max_rows : LORA_MAX_TILE_ROWS; }

}  // namespace

int32_t plan_shrink_jw(int32_t n_tiles, int32_t r_max, int32_t max_rows)
{
    if (max_rows >= kMfmaMinRows) return 16;
    // Smallest rank-row group that keeps the grid near kTargetGroups workgroups.
    int32_t jw = 1;
    while (jw < 4 && (int64_t)n_tiles * ((r_max + jw - 1) / jw) > kTargetGroups) jw *= 2;
    return jw;
}

}  // namespace lora

using namespace lora;

extern "C" {

int lora_set_launch_events(void *start_event, void *stop_event)
{
    clear_error();
    t_ev_start = static_cast<hipEvent_t>(start_event);
    t_ev_stop = static_cast<hipEvent_t>(stop_event);
    return LORA_OK;
}

int lora_sgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx, int32_t n_rows,
                     const lora_weights *w, const lora_segments *seg)
{
    clear_error();
    int st = check_segments(seg);
    if (st) return st;
    return shrink_impl<false>(stream, v, ldv, x, ldx, n_rows, w, seg_src(seg), seg->n_tiles, seg_max_rows(seg));
}

int lora_sgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv, int32_t n_rows,
                     const lora_weights *w, const lora_segments *seg)
{
    clear_error();
    int st = check_segments(seg);
    if (st) return st;
    return expand_impl<false>(stream, y, ldy, v, ldv, n_rows, w, seg_src(seg), seg->n_tiles, seg_max_rows(seg));
}

int lora_bgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx, const int32_t *idx,
                     int32_t n_rows, const lora_weights *w)
{
    clear_error();
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    return shrink_impl<true>(stream, v, ldv, x, ldx, n_rows, w, row_src(idx), n_rows, 1);
}

int lora_bgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv, const int32_t *idx,
                     int32_t n_rows, const lora_weights *w)
{
    clear_error();
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    return expand_impl<true>(stream, y, ldy, v, ldv, n_rows, w, row_src(idx), n_rows, 1);
}

int lora_bgmv(void *stream, void *y, int64_t ldy, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
              const lora_weights *w, float *v, int64_t ldv)
{
    clear_error();
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    // Check both halves before launching either.
    int st = check_weights_desc(w);
    if (st) return st;
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0) return LORA_OK;
    if ((st = check_rows_arg(y, ldy, w->d_out, 8, "y"))) return st;
    if ((st = check_rows_arg(v, ldv, w->r_max, 4, "v"))) return st;
    st = shrink_impl<true>(stream, v, ldv, x, ldx, n_rows, w, row_src(idx), n_rows, 1);
    if (st) return st;
    return expand_impl<true>(stream, y, ldy, v, ldv, n_rows, w, row_src(idx), n_rows, 1);
}

}  // extern "C"
