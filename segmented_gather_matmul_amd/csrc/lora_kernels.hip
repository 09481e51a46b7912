// HIP kernels (gfx950 / CDNA4) and launchers of the multi-LoRA add-on.
//
// shrink  v[row][j] = sum_k x[row][k] A^T[s][j][k]      (Punica summary, "The SGMV Operator")
// expand  y[row][c] += scale[s] sum_j v[row][j] B[s][j][c]
//
// Work decomposition.  Both kernels run over a flat work-list of tiles (a tile = up to
// 64 consecutive rows of one segment, or one row in the per-row-slot form) instead of
// binding the adapter to a grid dimension, so segments of 1 to thousands of rows share
// one launch.  One launch may also serve up to LORA_MAX_PROJ projections that share
// the batch (q/k/v, gate/up): each work item is (tile, projection, slice), and the items
// of one tile are consecutive (tile-major), except in the VALU expand, whose items are
// slice-major so that the tiles of one adapter reuse each chunk of its B.  A workgroup
// is 4 wavefronts (256 lanes); workgroup ids are remapped so that each of the 8 XCDs
// (which take workgroups round-robin) owns a contiguous range of items, so the x row and
// v row of a tile stay in one L2.
//
// Shrink.  The output is only r wide, so parallelism comes from splitting rank-rows
// over workgroups and d_in over the wavefronts of a workgroup; the partial sums are
// added in LDS in wavefront order.  No cross-workgroup reduction, no atomics, no
// workspace, and results do not depend on scheduling or on the work split.
//   - tiles of < 8 rows (decode): fp16 dot2 (v_dot2_f32_f16) on 16-byte coalesced
//     loads of x rows and A^T rank-rows, both contiguous in d_in, many in flight;
//   - tiles of 8..64 rows: v_mfma_f32_16x16x32_f16 over 16-rank slices, up to four of
//     them (across the launch's projections) sharing each read of the tile's x rows;
//     16 wavefronts split d_in, which goes through LDS in 512-column chunks; a single
//     slice on 64-row tiles (one projection of rank <= 16) takes the wave-staged kernel
//     instead: two 32-row workgroups per tile, four wavefronts that each stage their own
//     128-column chunks through LDS, with no barrier in the k loop.  Every MFMA shrink
//     sums each element in the same order, so all give the same bits.
// Expand.  A workgroup owns 512 output columns of one tile (256 in the MFMA kernel at
// ranks above 32).
//   - tiles of < 8 rows: each wavefront loads its quarter of the rank-rows of B once
//     (16-byte loads, contiguous in d_out, all in flight together), the quarters are
//     added in LDS, and one fp32 -> fp16 rounding updates y;
//   - tiles of 8..64 rows: each wavefront holds its columns of every rank-row of B in
//     registers and runs v_mfma_f32_16x16x16_f16 on s v (fp16 hi + lo/2048 parts, ~22
//     bits kept) x B, one 16-row block after another, the next block's y and v
//     requested before the current block's products; B is read once per tile, y and v
//     move in whole lines, and nothing passes through LDS.
// The per-row and the segment forms of decode batches also run both steps in one launch,
// the shrink's workgroups handing v to the expand's (lora_handoff_kernel).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "lora_internal.hpp"

// No floating-point contraction anywhere in the kernels: whether the compiler fused a
// multiply and an add (or rounded an fp32 product straight to fp16) depended on the
// template instance, so one projection's result could differ in the last bit between a
// single-projection launch and a launch serving several.  Every fused operation is an
// explicit __builtin_fmaf.
#pragma clang fp contract(off)

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

struct ProjDev {
    WeightsDev w;
    float *v;        // shrink output / expand input
    int64_t ldv;
    uint16_t *y;     // expand output
    int64_t ldy;
    int32_t slices;  // shrink: rank groups; expand: 512-column chunks
};

struct TileSrc {
    const lora_tile *tiles;   // segment form, tile list (NULL: the offsets below)
    const int32_t *row_map;   // segment form, may be NULL
    int32_t n_pos;
    const int32_t *idx;       // per-row form
    const int32_t *seg_ptr;   // segment form, offsets: [n_seg + 1]
    const int32_t *seg_slot;  // [n_seg]
    int32_t n_seg, tile_rows;
};

// The one-launch form that hands v from the shrink's workgroups to the expand's
// (lora_handoff_kernel): the grid holds the shrink's work items (laid out as in a
// shrink launch: per_tile, off, p[].slices) and then the expand's.
struct HandoffDev {
    uint32_t *work;                    // caller's workspace: kHandoffWords per (row, projection)
    int32_t n_shrink;                  // workgroups of the shrink part
    int32_t e_per_tile;                // expand items per row
    int32_t e_off[LORA_MAX_PROJ];      // first expand item of projection p within a row's items
    int32_t e_slices[LORA_MAX_PROJ];   // 512-column chunks of projection p
    int32_t polls;                     // polls before an expand workgroup computes v itself
};

struct Args {
    const uint16_t *x;  // shrink input
    int64_t ldx;
    int32_t n_rows, n_tiles, n_proj, per_tile, grid;
    int32_t jw;         // shrink: rank-rows per workgroup
    int32_t off[LORA_MAX_PROJ];  // first slice of projection p within a tile's items
    TileSrc ts;
    ProjDev p[LORA_MAX_PROJ];
    HandoffDev ho;
};

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowsPerPass = 4;     // rows per pass of the VALU kernels (segment form)
constexpr int kCols = 512;           // expand columns per workgroup
constexpr int kMfmaShrinkThreads = 1024;  // 16 wavefronts split d_in in the MFMA shrink

// The kernel arguments, read through a pointer that comes out of one scalar load per
// 64-byte line of them, all issued before a single wait: every argument read that
// follows hits the scalar cache.  Without it the reads miss one line after another at
// the start of a launch, each a round trip to L2 or memory, and the compiler hoists
// them ahead of any load of its own that does not feed their address.
__device__ inline const Args &touched_args()
{
    static_assert(sizeof(Args) > 11 * 64 && sizeof(Args) <= 12 * 64, "12 lines of kernel arguments");
    auto ka = __builtin_amdgcn_kernarg_segment_ptr();
    int t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11;
    asm volatile(
        "s_load_dword %0, %12, 0x0\n\t"
        "s_load_dword %1, %12, 0x40\n\t"
        "s_load_dword %2, %12, 0x80\n\t"
        "s_load_dword %3, %12, 0xc0\n\t"
        "s_load_dword %4, %12, 0x100\n\t"
        "s_load_dword %5, %12, 0x140\n\t"
        "s_load_dword %6, %12, 0x180\n\t"
        "s_load_dword %7, %12, 0x1c0\n\t"
        "s_load_dword %8, %12, 0x200\n\t"
        "s_load_dword %9, %12, 0x240\n\t"
        "s_load_dword %10, %12, 0x280\n\t"
        "s_load_dword %11, %12, 0x2c0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=s"(t0), "=s"(t1), "=s"(t2), "=s"(t3), "=s"(t4), "=s"(t5), "=s"(t6), "=s"(t7), "=s"(t8), "=s"(t9),
          "=s"(t10), "=s"(t11), "+s"(ka));
    typedef const __attribute__((address_space(4))) Args args_t;
    return *(const Args *)(args_t *)ka;
}

// touched_args for an argument block that starts OFF bytes into the kernel arguments
// (after leading scalar arguments): one scalar load per 64-byte line it spans.
template <int OFF>
__device__ inline const Args &touched_args_at()
{
    static_assert(OFF % 8 == 0 && OFF + sizeof(Args) <= 13 * 64, "13 lines of kernel arguments");
    auto ka = __builtin_amdgcn_kernarg_segment_ptr();
    int t0, t1, t2, t3, t4, t5, t6, t7, t8, t9, t10, t11, t12;
    asm volatile(
        "s_load_dword %0, %13, 0x0\n\t"
        "s_load_dword %1, %13, 0x40\n\t"
        "s_load_dword %2, %13, 0x80\n\t"
        "s_load_dword %3, %13, 0xc0\n\t"
        "s_load_dword %4, %13, 0x100\n\t"
        "s_load_dword %5, %13, 0x140\n\t"
        "s_load_dword %6, %13, 0x180\n\t"
        "s_load_dword %7, %13, 0x1c0\n\t"
        "s_load_dword %8, %13, 0x200\n\t"
        "s_load_dword %9, %13, 0x240\n\t"
        "s_load_dword %10, %13, 0x280\n\t"
        "s_load_dword %11, %13, 0x2c0\n\t"
        "s_load_dword %12, %13, 0x300\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=s"(t0), "=s"(t1), "=s"(t2), "=s"(t3), "=s"(t4), "=s"(t5), "=s"(t6), "=s"(t7), "=s"(t8), "=s"(t9),
          "=s"(t10), "=s"(t11), "=s"(t12), "+s"(ka));
    typedef const __attribute__((address_space(4))) Args args_t;
    typedef const __attribute__((address_space(4))) char bytes_t;
    return *(const Args *)(args_t *)((bytes_t *)ka + OFF);
}

// The kernel arguments as a kernel reads them: through touched_args with dense weights;
// with paged weights directly (there the touch measured slower: the kernels' extra
// registers cost a wavefront per SIMD).
template <bool TOUCH>
__device__ inline const Args &kernel_args(const Args &param)
{
    if constexpr (TOUCH) return touched_args();
    else return param;
}

// Contiguous work ranges per XCD: workgroup b runs on XCD b % 8; grid % 8 == 0.
__device__ inline int work_item(int b, int grid) { return (b & 7) * (grid >> 3) + (b >> 3); }

// Projection of slice `r` of a tile's items (uniform over the workgroup).
__device__ inline int proj_of(const Args &a, int r)
{
    int p = 0;
#pragma unroll
    for (int q = 1; q < LORA_MAX_PROJ; ++q) p += (q < a.n_proj && r >= a.off[q]) ? 1 : 0;
    return p;
}

// Row of position `pos`, or -1 when it falls outside the row map or the row range.
template <bool PERROW>
__device__ inline int row_of(const TileSrc &ts, int pos, int n_rows)
{
    int row = pos;
    if (!PERROW && ts.row_map) row = (pos >= 0 && pos < ts.n_pos) ? ts.row_map[pos] : -1;
    return (row >= 0 && row < n_rows) ? row : -1;
}

// Rank-row j of A^T[s] (IS_B false) or B[s] in the dense layout.
template <bool IS_B>
__device__ inline const uint16_t *dense_row(const WeightsDev &w, int s, int j)
{
    const int d = IS_B ? w.d_out : w.d_in;
    return (IS_B ? w.b : w.a_t) + ((int64_t)s * w.r_max + j) * d;
}

// Paged layout: first entry of slot s's A^T (IS_B false) or B rank-rows in the page table.
template <bool IS_B>
__device__ inline int64_t pt_base(const WeightsDev &w, int s)
{
    return IS_B ? w.b_pt_off[s] : w.a_pt_off[s];
}

// Page-table entry for page-index q (element q*P) of rank-row j, unchecked (-1 when
// the entry lies outside the table).  page_ok() checks the id once it has arrived, so
// a wavefront can have all its page-table loads in flight before it uses any.
template <bool IS_B>
__device__ inline int page_entry(const WeightsDev &w, int64_t ptb, int j, int q)
{
    const int d = IS_B ? w.d_out : w.d_in;
    const int64_t off = ptb + (int64_t)j * (d / w.page_elems) + q;
    return (off >= 0 && off < w.pt_entries) ? w.page_table[off] : -1;
}

__device__ inline int page_ok(const WeightsDev &w, int pg) { return (pg >= 0 && pg < w.num_pages) ? pg : -1; }

template <bool IS_B>
__device__ inline int page_id(const WeightsDev &w, int64_t ptb, int j, int q)
{
    return page_ok(w, page_entry<IS_B>(w, ptb, j, q));
}

__device__ inline const uint16_t *page_ptr(const WeightsDev &w, int pg, int within)
{
    return w.pool + (int64_t)pg * w.page_elems + within;
}

constexpr int kPageCache = 4096;  // page ids a shrink workgroup keeps in LDS

// Page ids of A^T rank-rows [j0, j1) of slot s, all pages, into LDS (one round trip
// for the whole workgroup).  Returns false, and caches nothing, when they do not fit.
template <int NTHREADS>
__device__ inline bool cache_a_pages(const WeightsDev &w, int s, int j0, int j1, int *cache)
{
    const int npg = w.d_in / w.page_elems;
    const int n = (j1 - j0) * npg;
    if (n > kPageCache) return false;
    const int64_t ptb = pt_base<false>(w, s);
    for (int t = threadIdx.x; t < n; t += NTHREADS) cache[t] = page_id<false>(w, ptb, j0 + t / npg, t % npg);
    __syncthreads();
    return true;
}

// Element k..k+7 of A^T rank-row j through the LDS page cache (or the page table when
// the cache was not filled); NULL for an out-of-range page.
__device__ inline const uint16_t *a_paged(const WeightsDev &w, const int *cache, bool cached, int64_t ptb, int j0,
                                          int j, int k)
{
    const int P = w.page_elems, q = k / P;
    const int pg = cached ? cache[(j - j0) * (w.d_in / P) + q] : page_id<false>(w, ptb, j, q);
    return pg >= 0 ? page_ptr(w, pg, k - q * P) : nullptr;
}

__device__ inline uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// A non-temporal (streaming) 16-byte load, for data read once per launch that dwarfs the
// caches: prefill's x rows in the MFMA shrinks and y in the expand of tall tiles.  Kept
// at normal priority, those streams evict the weights the next tiles reuse and fill the
// memory-side cache with lines that the next launch must first write back or displace;
// streamed, the 7B prefill layer measured 609 -> 554 us (its shrinks 1.2-1.8x faster).
__device__ inline uint4 load16_nt(const uint16_t *p)
{
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// SW, a template flag of the per-row VALU and hand-off kernels: the adapters' dense A^T and
// B rows are read with streaming loads (lora_set_stream_weights: a batch whose rows all
// use distinct adapters reads every weight row once).
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

// One lane-shuffling step of wave_sum: x from the lane that DPP control CTRL names, in the
// rows of ROWS (bit i = lanes 16i..16i+15); 0 in the other rows.
template <int CTRL, int ROWS>
__device__ inline float dpp_take(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

constexpr int kDppSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;     // row_ror:4
constexpr int kDppRor8 = 0x128;     // row_ror:8
constexpr int kDppBcast15 = 0x142;  // row_bcast:15 (lane 15 of each row into the next row)
constexpr int kDppBcast31 = 0x143;  // row_bcast:31 (lane 31 into rows 2 and 3)

// Sum over the 64 lanes of a wavefront, returned to every lane.  Data-parallel-primitive
// moves instead of LDS permutes: within each row of 16 lanes, partners 1 and 2 apart,
// then 4 and 8 apart (rotations), so every lane of a row holds the row's sum; then row 0
// is added into row 1 and row 2 into row 3, and rows 0 + 1 into row 3.  Lane 63 ends
// with the total, in an order fixed by this sequence alone.
__device__ inline float wave_sum(float s)
{
    s += dpp_take<kDppSwap1, 0xF>(s);
    s += dpp_take<kDppSwap2, 0xF>(s);
    s += dpp_take<kDppRor4, 0xF>(s);
    s += dpp_take<kDppRor8, 0xF>(s);
    s += dpp_take<kDppBcast15, 0xA>(s);
    s += dpp_take<kDppBcast31, 0xC>(s);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, s), 63));
}

// ------------------------------------------------------------------------ tiles from offsets
// The segment form given as offsets (no tile list): each workgroup finds its own tile
// t of the cut lora_build_tiles makes (segment g of len rows -> ceil(len / T) tiles of
// near-equal height, in segment order) from seg_ptr and seg_slot, and keeps it in LDS
// for tile_head.

// This workgroup's tile (offsets form).
__device__ inline lora_tile &wg_tile()
{
    __shared__ lora_tile t;
    return t;
}

// Tile t of the offsets form into wg_tile(), or slot -1 when the batch has fewer tiles.
// The whole workgroup (NT threads) scans NT segments at a time: each lane loads one
// segment's offsets and slot, counts its tiles, and a prefix sum over the workgroup
// (shuffles within a wavefront, then the wavefront totals in LDS) gives every segment's
// first tile; the lane whose range holds t writes the tile.  Offsets are clamped to the
// positions (the row map's length seg_ptr[n_seg] with a row map, else n_rows), so any
// device values stay in bounds.  The scan stops at the chunk that holds t.
template <int NT>
__device__ void derive_tile(const TileSrc &ts, int n_rows, int t)
{
    constexpr int W = NT / 64;
    __shared__ int wave_total[W];
    lora_tile &out = wg_tile();
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = max(ts.tile_rows, 1);
    const int lim = ts.row_map ? min(n_rows, max(ts.seg_ptr[ts.n_seg], 0)) : n_rows;
    if (tid == 0) out = lora_tile{-1, 0, 0, -1};
    int base = 0;  // tiles of the segments before this chunk
    for (int g0 = 0; g0 < ts.n_seg && base <= t; g0 += NT) {
        const int g = g0 + tid;
        int nt = 0, p0 = 0, len = 0, slot = -1;
        if (g < ts.n_seg) {
            p0 = min(max(ts.seg_ptr[g], 0), lim);
            const int p1 = min(max(ts.seg_ptr[g + 1], p0), lim);
            slot = ts.seg_slot[g];
            len = p1 - p0;
            nt = (slot >= 0 && len > 0) ? (len + T - 1) / T : 0;
        }
        int inc = nt;  // inclusive prefix sum over the wavefront
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(inc, d);
            if (lane >= d) inc += u;
        }
        if (lane == 63) wave_total[wave] = inc;
        __syncthreads();
        int first = base + inc - nt, total = base;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const int s = wave_total[w];
            first += w < wave ? s : 0;
            total += s;
        }
        if (nt > 0 && t >= first && t < first + nt) {
            const int q = t - first, rows = len / nt, rem = len - rows * nt;
            out = lora_tile{slot, p0 + q * rows + min(q, rem), rows + (q < rem ? 1 : 0), g};
        }
        base = total;
        __syncthreads();  // wave_total is rewritten by the next chunk
    }
    __syncthreads();
}

// Every segment-form kernel calls this first (all threads, after uniform early exits):
// in the offsets form (OFFS) it finds the workgroup's tile; with a tile list it does
// nothing.  The two forms are separate kernel instances: the scan's barriers, even in a
// branch a tile-list launch never takes, keep the compiler from moving the kernel's first
// loads ahead of it (the paged 70B layer measured 8 % slower with one instance for both).
template <bool PERROW, bool OFFS, int NT>
__device__ inline void prepare_tile(const TileSrc &ts, int n_rows, int t)
{
    if constexpr (!PERROW && OFFS) derive_tile<NT>(ts, n_rows, t);
}

// ------------------------------------------------------------------------ common head
// Slot and rows of work tile `t`.  The slot's rank is read separately: the dense
// layout holds r_max rank-rows per slot, so loads of rank-rows below r_max are in
// bounds and can be issued before the rank arrives (rows at or past the rank are
// masked out of every result); the paged layout reads only rank-rows below the rank.
struct TileHead {
    int32_t slot, pos0, nrows;
    bool valid;
};

// The head of a tile record already read (its slot checked against this projection).
__device__ inline TileHead head_of(const lora_tile &tl, const WeightsDev &w)
{
    TileHead th;
    th.slot = tl.slot;
    th.pos0 = tl.pos0;
    th.nrows = min(tl.nrows, LORA_MAX_TILE_ROWS);
    th.valid = th.slot >= 0 && th.slot < w.num_slots && th.nrows > 0;
    return th;
}

template <bool PERROW, bool OFFS>
__device__ inline TileHead tile_head(const TileSrc &ts, const WeightsDev &w, int t)
{
    TileHead th;
    if (PERROW) {
        th.slot = ts.idx[t];
        th.pos0 = t;
        th.nrows = 1;
    } else {
        lora_tile tl;
        if constexpr (!OFFS) {
            tl = ts.tiles[t];
        } else {
            // uniform over the workgroup: kept in scalar registers like the tile list's
            const lora_tile &w = wg_tile();
            tl = lora_tile{__builtin_amdgcn_readfirstlane(w.slot), __builtin_amdgcn_readfirstlane(w.pos0),
                           __builtin_amdgcn_readfirstlane(w.nrows), 0};
        }
        th.slot = tl.slot;
        th.pos0 = tl.pos0;
        th.nrows = min(tl.nrows, LORA_MAX_TILE_ROWS);
    }
    th.valid = th.slot >= 0 && th.slot < w.num_slots && th.nrows > 0;
    return th;
}

__device__ inline int slot_rank(const WeightsDev &w, int slot) { return max(0, min(w.rank[slot], w.r_max)); }

// Work item of this workgroup: tile, projection and slice within the projection.
struct Item {
    int tile, p, slice;
    bool ok;
};

__device__ inline Item work(const Args &a)
{
    Item it;
    const int wi = work_item(blockIdx.x, a.grid);
    it.tile = wi / a.per_tile;
    const int sl = wi - it.tile * a.per_tile;
    it.p = proj_of(a, sl);
    it.slice = sl - a.off[it.p];
    it.ok = it.tile < a.n_tiles && it.slice < a.p[it.p].slices;
    return it;
}

// The VALU expand's work item: slice-major (all tiles of one 512-column chunk, then the
// next chunk), so the tiles of one adapter read each chunk of its B one after another
// (an L2 hit after the first) instead of each tile sweeping all of B.  Tile-major, a
// rank-64, 28672-wide B (3.7 MB per tile, about one XCD's L2) was read from HBM 1.6 times.
__device__ inline Item work_by_slice(const Args &a)
{
    Item it;
    const int wi = work_item(blockIdx.x, a.grid);
    const int sl = wi / max(a.n_tiles, 1);
    it.tile = wi - sl * max(a.n_tiles, 1);
    const int slc = min(sl, a.per_tile - 1);
    it.p = proj_of(a, slc);
    it.slice = sl - a.off[it.p];
    it.ok = sl < a.per_tile && it.tile < a.n_tiles && it.slice < a.p[it.p].slices;
    return it;
}

// ------------------------------------------------------------------------ shrink
// Operands of one half-pair of the VALU shrink: octet o of x for NR rows and of A^T for
// RJ rank-rows [jb, jb + RJ), zero past the end of d_in, for rows < 0 and for rank-rows
// at or past jload.
struct ShrinkSrc {
    const WeightsDev &w;
    const uint16_t *x;
    int64_t ldx;
    int slot, jb, jload, j0, n_oct;
    int64_t ptb;
    const int *pcache;
    bool cached;
};

template <int NR, int RJ>
struct ShrinkHalf {
    uint4 x[NR], a[RJ];
};

// CACHED (paged weights only): the page ids come from the workgroup's LDS page cache,
// else from the page table.  Paged rank-rows first resolve all their page ids, then issue
// every data load unconditionally (page 0, which always exists, stands in for a rank-row
// that needs none) and mask the results: loads under per-lane branches were issued one
// page-id round trip apart.
// NT: streaming loads of dense A^T rank-rows (the SW flag of the kernels).
template <bool PAGED, bool CACHED, int NR, int RJ, bool NT = false>
__device__ inline ShrinkHalf<NR, RJ> load_half(const ShrinkSrc &s, const int (&rows)[NR], int o)
{
    ShrinkHalf<NR, RJ> h;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    const bool in = o < s.n_oct;
#pragma unroll
    for (int q = 0; q < NR; ++q) h.x[q] = (in && rows[q] >= 0) ? load16(s.x + (int64_t)rows[q] * s.ldx + 8 * o) : z4;
    if constexpr (!PAGED) {
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) {
            const int j = s.jb + jj;
            h.a[jj] = (in && j < s.jload) ? (NT ? load16_nt(dense_row<false>(s.w, s.slot, j) + 8 * o)
                                                 : load16(dense_row<false>(s.w, s.slot, j) + 8 * o))
                                          : z4;
        }
    } else {
        const int P = s.w.page_elems, k = 8 * o, q = k / P, within = k - q * P, npg = s.w.d_in / P;
        int pg[RJ];
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) {
            const int j = s.jb + jj;
            const bool need = in && j < s.jload;
            if constexpr (CACHED) {
                // entry 0 exists whenever the cache was filled; read unconditionally, then masked
                const int e = s.pcache[need ? (j - s.j0) * npg + q : 0];
                pg[jj] = need ? e : -1;
            } else {
                pg[jj] = need ? page_id<false>(s.w, s.ptb, j, q) : -1;
            }
        }
        uint4 t[RJ];
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) t[jj] = load16(page_ptr(s.w, max(pg[jj], 0), within));
#pragma unroll
        for (int jj = 0; jj < RJ; ++jj) h.a[jj] = pg[jj] >= 0 ? t[jj] : z4;
    }
    return h;
}

__device__ inline uint32_t *handoff_row(const HandoffDev &ho, int row, int p);

// The VALU shrink's sums over halves [0, h_end) of octet pairs for NR rows and RJ
// rank-rows: D halves (whole pairs) are requested together, then summed in order.
template <bool PAGED, bool CACHED, int NR, int RJ, int D, bool NT = false>
__device__ inline void shrink_halves(const ShrinkSrc &src, const int (&rows)[NR], int n_half, int h_end,
                                     float (&acc)[NR][RJ])
{
    const int tid = threadIdx.x;
    for (int h0 = 0; h0 < h_end; h0 += D) {
        ShrinkHalf<NR, RJ> hf[D];
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (d == 0 || h0 + d < n_half) hf[d] = load_half<PAGED, CACHED, NR, RJ, NT>(src, rows, tid + kThreads * (h0 + d));
#pragma unroll
        for (int d = 0; d < D; ++d) {
            // a pair runs when its first octet exists; its second term may be zero
            const int h = h0 + d;
            if (h < n_half && tid + kThreads * (h & ~1) < src.n_oct) {
#pragma unroll
                for (int q = 0; q < NR; ++q)
#pragma unroll
                    for (int jj = 0; jj < RJ; ++jj) acc[q][jj] = dot8(hf[d].x[q], hf[d].a[jj], acc[q][jj]);
            }
        }
    }
}

// Where a VALU shrink puts v: the v buffer; a workgroup's own LDS row (indexed by
// rank-row, per-row form); or the v buffer and the launch's hand-off row.
enum class VSink { Global, Lds, Handoff };

// VALU shrink.  Workgroup = one tile x rank-rows [j0, j0 + jw); NR rows and RJ
// rank-rows per pass; d_in striped over the 256 lanes, 16 bytes per lane per load.
// Lane l sums octets l, l + 256, l + 512, ... of d_in in that order, the octets taken
// in pairs (o, o + 256) with a zero second term when o + 256 is past the end; then the
// wavefront's lanes are added by wave_sum and the 4 wavefronts in order.  The
// loads of several halves of pairs (256 octets each, about 16 loads per lane) are
// issued together before any is summed, so a long d_in costs few round trips.
// shrink_valu_item runs one work item.  It returns true when it stored v (a valid
// tile whose slot has a non-zero rank), the same for every thread of the workgroup.
// DH: halves of octet pairs in flight together (0: about 16 loads per lane); it changes
// the batching of the loads, not the order of any sum.  only_rg >= 0: only the pass over
// the tile's rows [only_rg, only_rg + NR).
template <bool PAGED, bool PERROW, int RJ, int NR, VSink SINK, int DH = 0, bool OFFS = false, bool SW = false>
__device__ inline bool shrink_valu_item(const Args &a, const Item &it, float *red, int *pcache, float *vlds,
                                        int only_rg = -1, bool use_known = false, lora_tile known = lora_tile{})
{
    // halves in flight together: about 16 loads per lane, an even count (whole pairs)
    constexpr int D = DH > 0 ? DH : (16 / (NR + RJ)) & ~1 ? (16 / (NR + RJ)) & ~1 : 2;
    const ProjDev pd = a.p[it.p];  // by value: the fields stay in registers
    const int j0 = it.slice * a.jw;
    const int jend = min(j0 + a.jw, pd.w.r_max);
    const TileHead th = use_known ? head_of(known, pd.w) : tile_head<PERROW, OFFS>(a.ts, pd.w, it.tile);
    if (!th.valid || j0 >= jend) return false;
    const int rank = slot_rank(pd.w, th.slot);
    const int jload = PAGED ? min(jend, rank) : jend;
    bool cached = false;
    int64_t ptb = 0;
    if (PAGED) {
        ptb = pt_base<false>(pd.w, th.slot);
        if (j0 < jload) cached = cache_a_pages<kThreads>(pd.w, th.slot, j0, jload, pcache);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_oct = pd.w.d_in >> 3;
    const int n_half = 2 * ((n_oct + 2 * kThreads - 1) / (2 * kThreads));  // halves of octet pairs, even
    for (int rg = only_rg < 0 ? 0 : only_rg; rg < th.nrows; rg += NR) {
        int rows[NR];
#pragma unroll
        for (int q = 0; q < NR; ++q)
            rows[q] = (rg + q < th.nrows) ? row_of<PERROW>(a.ts, th.pos0 + rg + q, a.n_rows) : -1;
        for (int jb = j0; jb < jend; jb += RJ) {
            float acc[NR][RJ];
#pragma unroll
            for (int q = 0; q < NR; ++q)
#pragma unroll
                for (int jj = 0; jj < RJ; ++jj) acc[q][jj] = 0.f;
            const ShrinkSrc src{pd.w, a.x, a.ldx, th.slot, jb, jload, j0, n_oct, ptb, pcache, cached};
            // D halves (whole pairs) are requested together, then summed in order.  Paged
            // weights: rank-rows at or past the slot's rank (known here) need neither x nor
            // A; their sums stay zero, as the loop would leave them.
            const int h_end = (!PAGED || jb < jload) ? n_half : 0;
            if (!PAGED || cached) shrink_halves<PAGED, true, NR, RJ, D, SW>(src, rows, n_half, h_end, acc);
            else shrink_halves<PAGED, false, NR, RJ, D>(src, rows, n_half, h_end, acc);
#pragma unroll
            for (int q = 0; q < NR; ++q)
#pragma unroll
                for (int jj = 0; jj < RJ; ++jj) {
                    const float s = wave_sum(acc[q][jj]);
                    if (lane == 0) red[wave * NR * RJ + q * RJ + jj] = s;
                }
            __syncthreads();
            if (tid < NR * RJ && rank > 0) {
                const int q = tid / RJ, jj = tid - q * RJ, j = jb + jj;
                int row = rows[0];  // rows[q] without a dynamically indexed register array
#pragma unroll
                for (int qq = 1; qq < NR; ++qq) row = q == qq ? rows[qq] : row;
                // wavefront order: the same sum for every launch of this shape
                const float s = red[tid] + red[NR * RJ + tid] + red[2 * NR * RJ + tid] + red[3 * NR * RJ + tid];
                if (row >= 0 && j < jend) {
                    const float vj = j < rank ? s : 0.f;
                    float *dst = pd.v + (int64_t)row * pd.ldv + j;
                    if constexpr (SINK == VSink::Lds) vlds[q * LORA_MAX_RANK + j] = vj;
                    else *dst = vj;
                    if constexpr (SINK == VSink::Handoff) {
                        uint32_t hv = ~__builtin_bit_cast(uint32_t, vj);
                        if (hv == 0) hv = ~0x7FC00000u;  // zero stays "not yet"
                        __hip_atomic_store(handoff_row(a.ho, row, it.p) + j, hv, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
            __syncthreads();
        }
        if (only_rg >= 0) break;
    }
    return rank > 0;
}

template <bool PAGED, bool PERROW, int RJ, int NR, bool OFFS, bool SW = false>
__global__ __launch_bounds__(kThreads) void lora_shrink_valu_kernel(Args args)
{
    const Args &a = kernel_args<!PAGED>(args);
    __shared__ float red[kWaves * NR * RJ];
    __shared__ int pcache[PAGED ? kPageCache : 1];
    const Item it = work(a);
    if (!it.ok) return;
    prepare_tile<PERROW, OFFS, kThreads>(a.ts, a.n_rows, it.tile);
    shrink_valu_item<PAGED, PERROW, RJ, NR, VSink::Global, 0, OFFS, SW>(a, it, red, pcache, nullptr);
}

// Rank slices of an MFMA shrink workgroup: slices g0 .. g0 + NS - 1 of the launch's
// slice list, each with its projection, first rank-row, the slot's rank and validity.
template <int NS>
struct MfmaSlices {
    int sp[NS], sj0[NS], srank[NS];
    bool sok[NS];
};

template <int NS>
__device__ inline MfmaSlices<NS> mfma_slices(const Args &a, int slot, int g0)
{
    MfmaSlices<NS> m;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const int sl = g0 + q;
        m.sp[q] = proj_of(a, min(sl, a.per_tile - 1));
        m.sj0[q] = 16 * (sl - a.off[m.sp[q]]);
        const WeightsDev &w = a.p[m.sp[q]].w;
        m.sok[q] = sl < a.per_tile && slot < w.num_slots && m.sj0[q] < w.r_max;
        m.srank[q] = m.sok[q] ? slot_rank(w, slot) : 0;
    }
    return m;
}

// The MFMA shrinks' last step: every wavefront's 16x16 accumulators go to LDS and are
// added in wavefront order, one rank slice at a time; columns at or past the rank are
// written as 0.  red holds W * MTX * 256 floats.
template <int MTX, int NS>
__device__ inline void mfma_shrink_store(const Args &a, const TileHead &th, const MfmaSlices<NS> &m, int MT,
                                         const f4_t (&acc)[NS][MTX], float *red)
{
    constexpr int W = kMfmaShrinkThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
    // D layout: lane holds rows 4*lg + e of the slice, rank column li.
#pragma unroll
    for (int q = 0; q < NS; ++q) {
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave * (MTX * 256) + mt * 256 + (4 * lg + e) * 16 + li] = acc[q][mt][e];
        __syncthreads();
        if (m.sok[q] && m.srank[q] > 0) {
            const ProjDev &pd = a.p[m.sp[q]];
            for (int o = tid; o < MT * 256; o += kMfmaShrinkThreads) {
                const int mt = o >> 8, i = (o >> 4) & 15, j = o & 15;
                const int rr = 16 * mt + i, col = m.sj0[q] + j;
                if (rr >= th.nrows || col >= pd.w.r_max) continue;
                const int row = row_of<false>(a.ts, th.pos0 + rr, a.n_rows);
                if (row < 0) continue;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) s += red[w * (MTX * 256) + o];
                pd.v[(int64_t)row * pd.ldv + col] = col < m.srank[q] ? s : 0.f;
            }
        }
        __syncthreads();
    }
}

// MFMA shrink for tiles of up to 64 rows: v_mfma_f32_16x16x32_f16 over (16-row
// slices) x (16-rank slices).  A workgroup takes NS consecutive rank slices of the
// launch's slice list (projection by projection), so the projections of one launch
// share each read of the tile's x rows.  16 wavefronts take interleaved 32-wide
// k-steps, U of them in flight each, and their sums are added in LDS in wavefront
// order, one rank slice at a time.  Neither NS nor MTX changes the order in which any
// element is summed, so every split gives the same bits.
template <bool PAGED, int MTX, int NS, bool OFFS>
__global__ __launch_bounds__(kMfmaShrinkThreads) void lora_shrink_mfma_kernel(Args args)
{
    const Args &a = kernel_args<!PAGED>(args);
    constexpr int W = kMfmaShrinkThreads / 64;
    // k-steps in flight per wavefront: ~16 loads, or one step when the accumulators are large
    constexpr int U = MTX * NS >= 12 ? 1 : 16 / (MTX + NS);
    __shared__ float red[W * 1024];
    __shared__ int pcache[PAGED ? kPageCache : 1];
    const int wi = work_item(blockIdx.x, a.grid);
    const int groups = (a.per_tile + NS - 1) / NS;
    const int tile = wi / groups, g0 = (wi - tile * groups) * NS;
    if (tile >= a.n_tiles) return;
    prepare_tile<false, OFFS, kMfmaShrinkThreads>(a.ts, a.n_rows, tile);
    const TileHead th = tile_head<false, OFFS>(a.ts, a.p[0].w, tile);
    if (th.slot < 0 || th.nrows <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;       // operand row/col, k-group of the lane
    // this workgroup's rank slices, and this lane's A^T rank-row in each
    const MfmaSlices<NS> m = mfma_slices<NS>(a, th.slot, g0);
    const int *sp = m.sp, *sj0 = m.sj0, *srank = m.srank;
    const bool *sok = m.sok;
    const uint16_t *arow[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const WeightsDev &w = a.p[sp[q]].w;
        const int jcol = sj0[q] + li;
        arow[q] = (!PAGED && sok[q] && jcol < w.r_max) ? dense_row<false>(w, th.slot, jcol) : nullptr;
    }
    // paged weights: one rank slice per workgroup (NS == 1), its descriptor by value
    const WeightsDev w0 = a.p[sp[0]].w;
    bool cached = false;
    int64_t ptb = 0;
    if (PAGED) {
        ptb = sok[0] ? pt_base<false>(w0, th.slot) : 0;
        const int j1 = min(sj0[0] + 16, srank[0]);
        if (sok[0] && sj0[0] < j1) cached = cache_a_pages<kMfmaShrinkThreads>(w0, th.slot, sj0[0], j1, pcache);
    }
    // the tile's rows 16 * MTX at a time (one block for the tile heights the launch was
    // planned for; the row height is only a hint)
    for (int m0 = 0; m0 < th.nrows; m0 += 16 * MTX) {
    const TileHead tb{th.slot, th.pos0 + m0, th.nrows - m0, th.valid};
    const int MT = min((tb.nrows + 15) >> 4, MTX);
    int xrow[MTX];
#pragma unroll
    for (int mt = 0; mt < MTX; ++mt) {
        const int rr = 16 * mt + li;
        xrow[mt] = (mt < MT && rr < tb.nrows) ? row_of<false>(a.ts, tb.pos0 + rr, a.n_rows) : -1;
    }
    f4_t acc[NS][MTX];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) acc[q][mt] = f4_t{0.f, 0.f, 0.f, 0.f};
    const int d_in = a.p[0].w.d_in;
    const int steps = (d_in + 31) >> 5;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    for (int s0 = wave; s0 < steps; s0 += W * U) {
        uint4 bq[U][NS], xq[U][MTX];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = 32 * (s0 + W * u) + 8 * lg;
            const bool kin = k < d_in;
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                bq[u][q] = z4;
                if (!kin) continue;
                if (!PAGED) {
                    if (arow[q]) bq[u][q] = load16(arow[q] + k);
                } else if (sok[q] && sj0[q] + li < srank[q]) {
                    const uint16_t *p = a_paged(w0, pcache, cached, ptb, sj0[q], sj0[q] + li, k);
                    if (p) bq[u][q] = load16(p);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MTX; ++mt)
                xq[u][mt] = (kin && xrow[mt] >= 0) ? load16(a.x + (int64_t)xrow[mt] * a.ldx + k) : z4;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const h8_t bop = __builtin_bit_cast(h8_t, bq[u][q]);
#pragma unroll
                for (int mt = 0; mt < MTX; ++mt)
                    acc[q][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xq[u][mt]), bop,
                                                                        acc[q][mt], 0, 0, 0);
            }
    }
    mfma_shrink_store<MTX, NS>(a, tb, m, MT, acc, red);
    }
}

// The dense MFMA shrink with x and A^T staged through LDS.  Work item, operand values
// and accumulation order are those of lora_shrink_mfma_kernel (wavefront w owns k-steps
// w, w + 16, ... and applies them in that order; the sums are added in LDS in wavefront
// order), so the two give the same bits; only the data movement differs.  Each
// 512-column chunk (one k-step per wavefront) of the tile's x rows and of the slices'
// A^T rank-rows is loaded one whole 1 KB row per wavefront load (full cache lines,
// where the operand layout would fetch 64 bytes from each of 16 rows), written to LDS,
// and the MFMA operands are read from LDS while the next chunk's loads are in flight.
constexpr int kStageCols = 512;               // columns per chunk: 16 k-steps of 32
constexpr int kStageStride = kStageCols + 8;  // halves per staged row; the pad puts the 16
                                              // rows an operand read touches in distinct banks

__host__ __device__ constexpr int stage_rows(int mtx, int ns) { return 16 * (mtx + ns); }

__host__ __device__ constexpr size_t stage_lds_bytes(int mtx, int ns)
{
    // the staged chunk, or the wavefronts' accumulators once the k loop is done
    return (size_t)stage_rows(mtx, ns) * kStageStride * 2 > (size_t)(kMfmaShrinkThreads / 64) * mtx * 256 * 4
               ? (size_t)stage_rows(mtx, ns) * kStageStride * 2
               : (size_t)(kMfmaShrinkThreads / 64) * mtx * 256 * 4;
}

// Octet k .. k+7 of every staged row this wavefront loads; zero past d_in or for rows
// without a source.  The wavefront's first nx staged rows are x rows, read once per
// launch and loaded streaming; the A^T rank-rows after them, which the adapter's other
// tiles read again, keep normal loads (measured 0.25 % faster per 7B prefill layer than
// streaming them too).
template <int RPW>
__device__ inline void stage_load(const uint16_t *const (&src)[RPW], int k, int d_in, uint4 (&st)[RPW], int nx)
{
    const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
        st[i] = (src[i] && k < d_in) ? (i < nx ? load16_nt(src[i] + k) : load16(src[i] + k)) : z4;
}

template <int MTX, int NS, bool OFFS>
__global__ __launch_bounds__(kMfmaShrinkThreads) void lora_shrink_mfma_staged_kernel(Args args)
{
    const Args &a = kernel_args<true>(args);
    constexpr int W = kMfmaShrinkThreads / 64;
    constexpr int XR = 16 * MTX, ROWS = stage_rows(MTX, NS);
    constexpr int RPW = (ROWS + W - 1) / W;  // staged rows per wavefront: rows wave, wave + W, ...
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t *stg = reinterpret_cast<uint16_t *>(smem);  // [ROWS][kStageStride]
    float *red = reinterpret_cast<float *>(smem);        // reused after the k loop
    const int wi = work_item(blockIdx.x, a.grid);
    // work item: (tile, group of NS rank slices)
    const int groups = (a.per_tile + NS - 1) / NS;
    const int tile = wi / groups, g0 = (wi - tile * groups) * NS;
    if (tile >= a.n_tiles) return;
    prepare_tile<false, OFFS, kMfmaShrinkThreads>(a.ts, a.n_rows, tile);
    const TileHead th = tile_head<false, OFFS>(a.ts, a.p[0].w, tile);
    if (th.slot < 0 || th.nrows <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const MfmaSlices<NS> m = mfma_slices<NS>(a, th.slot, g0);
    // The tile's rows XR at a time (one block for the tile heights the launch was planned
    // for; the row height is only a hint).
    for (int m0 = 0; m0 < th.nrows; m0 += XR) {
    const TileHead tb{th.slot, th.pos0 + m0, th.nrows - m0, th.valid};
    const int MT = min((tb.nrows + 15) >> 4, MTX);
    // staged row r: x row r of the block (r < XR), else A^T rank-row of slice (r - XR) / 16
    const uint16_t *src[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int r = i * W + wave;
        src[i] = nullptr;
        if (r < XR) {
            const int row = r < tb.nrows ? row_of<false>(a.ts, tb.pos0 + r, a.n_rows) : -1;
            if (row >= 0) src[i] = a.x + (int64_t)row * a.ldx;
        } else if (r < ROWS) {
            const int q = (r - XR) >> 4, j = m.sj0[q] + ((r - XR) & 15);
            const WeightsDev &w = a.p[m.sp[q]].w;
            if (m.sok[q] && j < w.r_max) src[i] = dense_row<false>(w, th.slot, j);
        }
    }
    f4_t acc[NS][MTX];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) acc[q][mt] = f4_t{0.f, 0.f, 0.f, 0.f};
    const int d_in = a.p[0].w.d_in;
    const int chunks = (d_in + kStageCols - 1) / kStageCols;
    const int kc = 32 * wave + 8 * lg;  // this lane's operand columns within a chunk
    const int nx = (XR - wave + W - 1) / W;  // staged rows i < nx of this wavefront are x rows
    uint4 st[RPW];
    stage_load<RPW>(src, 8 * lane, d_in, st, nx);
    for (int ck = 0; ck < chunks; ++ck) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int r = i * W + wave;
            if (r < ROWS) *reinterpret_cast<uint4 *>(stg + r * kStageStride + 8 * lane) = st[i];
        }
        __syncthreads();
        if (ck + 1 < chunks) stage_load<RPW>(src, (ck + 1) * kStageCols + 8 * lane, d_in, st, nx);
        h8_t bop[NS];
#pragma unroll
        for (int q = 0; q < NS; ++q) bop[q] = *reinterpret_cast<const h8_t *>(stg + (XR + 16 * q + li) * kStageStride + kc);
#pragma unroll
        for (int mt = 0; mt < MTX; ++mt) {
            if (mt < MT) {
                const h8_t xop = *reinterpret_cast<const h8_t *>(stg + (16 * mt + li) * kStageStride + kc);
#pragma unroll
                for (int q = 0; q < NS; ++q)
                    acc[q][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, bop[q], acc[q][mt], 0, 0, 0);
            }
        }
        __syncthreads();
    }
    mfma_shrink_store<MTX, NS>(a, tb, m, MT, acc, red);
    }
}

// MFMA shrink with four wavefronts and no barrier inside the k loop, for RB workgroups
// of 16 * MTX rows per tile and NS rank slices per workgroup (the planner launches it for
// a single slice on 64-row tiles: MTX 2, RB 2, NS 1).  Wavefront w takes the 128-column
// chunks w, w + 4, w + 8, ... of d_in.  Each chunk's x rows and the slices' A^T
// rank-rows are loaded as 256-byte row spans (four rows per load instruction), written
// to the wavefront's own LDS region (16-byte groups XOR-swizzled by row, so both the
// row-span writes and the operand reads spread over the banks) and read back in the
// MFMA operand layout while the next chunk's loads are in flight.  A chunk holds the
// 32-wide k-steps 4c .. 4c+3 of d_in; k-step kk is accumulated into class kk mod 16
// (classes 4w .. 4w+3 in wavefront w), in ascending kk, and the 16 classes are added in
// LDS in class order.  That is the summation order of the other MFMA shrinks (16
// wavefronts, wavefront w owning k-steps w, w + 16, ...), so every MFMA shrink gives the
// same bits.  Against the staged kernel it drops the two workgroup barriers per chunk,
// each of which waits for the slowest of the chunk's row loads.
constexpr int kWaveChunk = 128;                      // columns per chunk: 4 k-steps
constexpr int kWaveBlock = 16 * kWaveChunk / 8;      // 16-byte groups of one staged 16-row block

__host__ __device__ constexpr size_t wave_lds_bytes(int mtx, int ns)
{
    // the wavefronts' staged blocks, or the 16 classes' sums (16 * mtx KB) after the k loop
    return (size_t)kWaves * (mtx + ns) * kWaveBlock * 16;
}

// v where c holds, else zero.  A value select: `c ? v : z` of two lvalues is an lvalue
// that clang forms by selecting between their addresses, which puts both in scratch.
__device__ inline uint4 keep_if(bool c, uint4 v) { return c ? v : make_uint4(0, 0, 0, 0); }

// Rows of block positions r[i] (relative to pos0) as row_of gives them, -1 for positions
// at or past nrows: every row-map read is issued unconditionally (at a clamped index)
// before any is used, so a lane's lookups take one round trip, not one each.
template <int N>
__device__ inline void rows_of_block(const TileSrc &ts, int n_rows, int pos0, int nrows, int (&r)[N])
{
    if (ts.row_map && ts.n_pos > 0) {
        const int last = ts.n_pos - 1;
        int v[N];
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = ts.row_map[min(max(pos0 + r[i], 0), last)];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int pos = pos0 + r[i];
            r[i] = (r[i] < nrows && pos >= 0 && pos < ts.n_pos) ? v[i] : -1;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) r[i] = (!ts.row_map && r[i] < nrows) ? pos0 + r[i] : -1;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = (r[i] >= 0 && r[i] < n_rows) ? r[i] : -1;
}

template <int MTX, int NS, int RB, bool OFFS>
__global__ __launch_bounds__(kThreads) void lora_shrink_mfma_wave_kernel(Args args)
{
    const Args &a = kernel_args<true>(args);
    constexpr int NB = MTX + NS;  // staged blocks per wavefront: x row blocks, then A^T per slice
    extern __shared__ __align__(16) unsigned char smem[];
    const int wi = work_item(blockIdx.x, a.grid);
    const int groups = (a.per_tile + NS - 1) / NS;
    const int tile = wi / (groups * RB), rem = wi - tile * (groups * RB);
    const int rbk = RB == 1 ? 0 : rem / groups, g0 = (rem - rbk * groups) * NS;
    if (tile >= a.n_tiles) return;
    prepare_tile<false, OFFS, kThreads>(a.ts, a.n_rows, tile);
    const TileHead th = tile_head<false, OFFS>(a.ts, a.p[0].w, tile);
    if (th.slot < 0 || th.nrows <= 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
    uint4 *const my = reinterpret_cast<uint4 *>(smem) + wave * NB * kWaveBlock;
    float *const red = reinterpret_cast<float *>(smem);  // [16 classes][MTX][256], after the k loop
    const MfmaSlices<NS> m = mfma_slices<NS>(a, th.slot, g0);
    const int d_in = a.p[0].w.d_in;
    const int nct = (d_in + kWaveChunk - 1) / kWaveChunk;
    const int nc = (nct - wave + kWaves - 1) / kWaves;  // chunks wave, wave + 4, ...
    // this lane loads 16-byte group li of rows 4i + lg (i = 0..3) of every staged block;
    // past d_in it reloads the last group in range and the chunk masks it to zero
    const int lim = d_in - 8 - 8 * li;
    const bool tail = nct * kWaveChunk > d_in;
    // A^T rank-rows past r_max or of a slice without work: x row 0 stands in, masked to zero
    const uint16_t *ap[NS][4];
    bool aok[NS][4];
    bool amask = false;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        const WeightsDev &w = a.p[m.sp[q]].w;
        amask |= !(m.sok[q] && m.sj0[q] + 16 <= w.r_max);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = m.sj0[q] + 4 * i + lg;
            aok[q][i] = m.sok[q] && j < w.r_max;
            ap[q][i] = (aok[q][i] ? dense_row<false>(w, th.slot, j) : a.x) + 8 * li;
        }
    }
    // The tile's rows 16 * MTX at a time: block rbk of every RB (one block per workgroup
    // for the planned tile height; the row height is only a hint).
    for (int m0 = rbk * 16 * MTX; m0 < th.nrows; m0 += RB * 16 * MTX) {
        const int pos0 = th.pos0 + m0, nrows = th.nrows - m0;
        const int MT = min((nrows + 15) >> 4, MTX);
        // Rows of this lane's x loads (rows 16b + 4i + lg of the block) and of its v stores
        // (rows 16b + tid / 16), all row-map reads in flight together.  Rows past the tile or
        // without a source load x row 0; their results are not stored.
        int rows[5 * MTX];
#pragma unroll
        for (int b = 0; b < MTX; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rows[4 * b + i] = 16 * b + 4 * i + lg;
            rows[4 * MTX + b] = 16 * b + (tid >> 4);
        }
        rows_of_block<5 * MTX>(a.ts, a.n_rows, pos0, nrows, rows);
        const uint16_t *xp[MTX][4];
#pragma unroll
        for (int b = 0; b < MTX; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) xp[b][i] = a.x + (int64_t)max(rows[4 * b + i], 0) * a.ldx + 8 * li;
        auto load = [&](int jc, uint4 (&X)[MTX][4], uint4 (&A)[NS][4]) __attribute__((always_inline)) {
            const int k = min((kWaves * jc + wave) * kWaveChunk, lim);
#pragma unroll
            for (int b = 0; b < MTX; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[b][i] = load16_nt(xp[b][i] + k);
#pragma unroll
            for (int q = 0; q < NS; ++q)
#pragma unroll
                for (int i = 0; i < 4; ++i) A[q][i] = load16(ap[q][i] + k);
        };
        f4_t acc[MTX][NS][4];
#pragma unroll
        for (int b = 0; b < MTX; ++b)
#pragma unroll
            for (int q = 0; q < NS; ++q)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc[b][q][s] = f4_t{0.f, 0.f, 0.f, 0.f};
        // valid: false for the pipeline's reload past this wavefront's last chunk
        auto process = [&](int jc, bool valid, uint4 (&X)[MTX][4], uint4 (&A)[NS][4]) __attribute__((always_inline)) {
            const int k = (kWaves * jc + wave) * kWaveChunk + 8 * li;
            if (tail && k - 8 * li + kWaveChunk > d_in) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int b = 0; b < MTX; ++b) X[b][i] = keep_if(k < d_in, X[b][i]);
#pragma unroll
                    for (int q = 0; q < NS; ++q) A[q][i] = keep_if(k < d_in, A[q][i]);
                }
            }
            if (amask) {
#pragma unroll
                for (int q = 0; q < NS; ++q)
#pragma unroll
                    for (int i = 0; i < 4; ++i) A[q][i] = keep_if(aok[q][i], A[q][i]);
            }
            if (!valid) {  // zero products, and no Inf or NaN of x times 0
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int b = 0; b < MTX; ++b) X[b][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int q = 0; q < NS; ++q) A[q][i] = make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * i + lg, o = 16 * r + (li ^ r);
#pragma unroll
                for (int b = 0; b < MTX; ++b) my[b * kWaveBlock + o] = X[b][i];
#pragma unroll
                for (int q = 0; q < NS; ++q) my[(MTX + q) * kWaveBlock + o] = A[q][i];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int o = 16 * li + ((4 * s + lg) ^ li);
                h8_t bop[NS];
#pragma unroll
                for (int q = 0; q < NS; ++q) bop[q] = __builtin_bit_cast(h8_t, my[(MTX + q) * kWaveBlock + o]);
#pragma unroll
                for (int b = 0; b < MTX; ++b) {
                    const h8_t xop = __builtin_bit_cast(h8_t, my[b * kWaveBlock + o]);
#pragma unroll
                    for (int q = 0; q < NS; ++q)
                        acc[b][q][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, bop[q], acc[b][q][s], 0, 0, 0);
                }
            }
        };
        // two chunks in flight: the next one's loads are issued before this one is
        // processed (the scheduling barriers keep the compiler from sinking them)
        if (nc > 0) {
            uint4 X0[MTX][4], A0[NS][4], X1[MTX][4], A1[NS][4];
            load(0, X0, A0);
            for (int jc = 0; jc < nc; jc += 2) {
                load(min(jc + 1, nc - 1), X1, A1);
                __builtin_amdgcn_sched_barrier(0);
                process(jc, true, X0, A0);
                load(min(jc + 2, nc - 1), X0, A0);
                __builtin_amdgcn_sched_barrier(0);
                process(min(jc + 1, nc - 1), jc + 1 < nc, X1, A1);
            }
        }
        __syncthreads();  // every wavefront is done with its staged blocks
        // the classes' sums, one rank slice at a time; columns at or past the rank are 0
#pragma unroll
        for (int q = 0; q < NS; ++q) {
#pragma unroll
            for (int b = 0; b < MTX; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        red[((kWaves * wave + s) * MTX + b) * 256 + (4 * lg + e) * 16 + li] = acc[b][q][s][e];
            __syncthreads();
            if (m.sok[q] && m.srank[q] > 0) {
                const ProjDev &pd = a.p[m.sp[q]];
                const int col = m.sj0[q] + (tid & 15);
#pragma unroll
                for (int b = 0; b < MTX; ++b) {
                    const int o = tid + 256 * b, row = rows[4 * MTX + b];
                    if (b >= MT || row < 0 || col >= pd.w.r_max) continue;
                    float sum = 0.f;
#pragma unroll
                    for (int cl = 0; cl < 16; ++cl) sum += red[cl * MTX * 256 + o];
                    pd.v[(int64_t)row * pd.ldv + col] = col < m.srank[q] ? sum : 0.f;
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------------------ expand
// Rank-rows j = w + 4 u, u0 <= u < u0 + RU, that wavefront w of a 256-lane group loads
// for its 8 columns at c: B[slot][j][c .. c+7], zero where j >= jlim or the columns
// are out of range.  Paged weights resolve all page ids first; the data loads are then
// issued unconditionally (page 0, which always exists, stands in for a missing entry)
// and masked, because a load under a per-lane branch is sunk by the compiler next to
// its conditional use and waited on alone.
// Paged part of load_b_octets: the first N of the RU entries (the rest zero).  Every
// load is issued, in bounds (page 0 stands in for a missing or invalid entry) and
// without a branch, then masked: all N loads are in flight together.
template <int N, int RU>
__device__ inline void load_b_paged(const WeightsDev &w, int slot, int jlim, int wave, int u0, int c, bool cin,
                                    uint4 *bv)
{
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    const int P = w.page_elems, q = c / P, within = c - q * P;
    const int64_t ptb = pt_base<true>(w, slot);
    int pg[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int j = wave + kWaves * (u0 + u);
        pg[u] = (cin && j < jlim) ? page_entry<true>(w, ptb, j, q) : -1;
    }
    uint4 t[N];
#pragma unroll
    for (int u = 0; u < N; ++u) t[u] = load16(page_ptr(w, max(page_ok(w, pg[u]), 0), within));
#pragma unroll
    for (int u = 0; u < N; ++u) bv[u] = page_ok(w, pg[u]) >= 0 ? t[u] : z4;
#pragma unroll
    for (int u = N; u < RU; ++u) bv[u] = z4;
    // keep the loads here: otherwise each is sunk next to its (conditional) use and waited on alone
#pragma unroll
    for (int u = 0; u < RU; ++u) asm volatile("" : "+v"(bv[u].x), "+v"(bv[u].y), "+v"(bv[u].z), "+v"(bv[u].w));
}

// Rank-rows j = w + 4 u, u0 <= u < u0 + RU, that wavefront w of a 256-lane group loads
// for its 8 columns at c: B[slot][j][c .. c+7], zero where j >= jlim or the columns
// are out of range.  Paged weights resolve all page ids first, then issue only as many
// data loads as the rank needs (a quarter, half or all of RU, picked once per
// wavefront), unconditionally and masked, because a load under a per-lane branch is
// sunk by the compiler next to its conditional use and waited on alone.
template <bool PAGED, int RU, bool NT = false>
__device__ inline void load_b_octets(const WeightsDev &w, int slot, int jlim, int wave, int u0, int c, bool cin,
                                     uint4 *bv)
{
    if (!PAGED) {
        const uint4 z4 = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < RU; ++u) {
            const int j = wave + kWaves * (u0 + u);
            bv[u] = (cin && j < jlim) ? (NT ? load16_nt(dense_row<true>(w, slot, j) + c) : load16(dense_row<true>(w, slot, j) + c)) : z4;
        }
    } else if constexpr (RU >= 8) {
        // entries this wavefront needs: rank-rows wave + 4 u below jlim, from u0 on
        const int need = (jlim - wave + kWaves - 1) / kWaves - u0;
        if (need <= RU / 4) load_b_paged<RU / 4, RU>(w, slot, jlim, wave, u0, c, cin, bv);
        else if (need <= RU / 2) load_b_paged<RU / 2, RU>(w, slot, jlim, wave, u0, c, cin, bv);
        else load_b_paged<RU, RU>(w, slot, jlim, wave, u0, c, cin, bv);
    } else {
        load_b_paged<RU, RU>(w, slot, jlim, wave, u0, c, cin, bv);
    }
}

// VALU expand.  Workgroup = one tile x 512 columns; wavefront w holds rank-rows
// w, w+4, ... of B (loaded once, all in flight); NR rows per pass; the four partial
// sums are added in LDS and wavefront q updates row q of the pass.
template <bool PERROW, int NR>
struct ExpandPass {
    int rows[NR];
    float sv[NR];  // lane j holds v[row][j]
    int my_row;    // row this wavefront updates

    __device__ void load(const Args &a, const ProjDev &pd, const TileHead &th, int rg)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int q = 0; q < NR; ++q)
            rows[q] = (rg + q < th.nrows) ? row_of<PERROW>(a.ts, th.pos0 + rg + q, a.n_rows) : -1;
        my_row = (wave < NR && rg + wave < th.nrows) ? row_of<PERROW>(a.ts, th.pos0 + rg + wave, a.n_rows) : -1;
#pragma unroll
        for (int q = 0; q < NR; ++q)
            sv[q] = (rows[q] >= 0 && lane < pd.w.r_max) ? pd.v[(int64_t)rows[q] * pd.ldv + lane] : 0.f;
    }

    __device__ uint4 load_y(const ProjDev &pd, int c, bool cin) const
    {
        return (my_row >= 0 && cin) ? load16(pd.y + (int64_t)my_row * pd.ldy + c) : make_uint4(0, 0, 0, 0);
    }
};

// One pass of the VALU expand on one chunk: y rows of `ps` at columns c .. c+7 of each
// lane += scale v B, with the rank-rows of B in bv (wavefront w: j = w + 4 u).
template <bool PERROW, int NR, int RU>
__device__ inline void expand_pass(const ProjDev &pd, const ExpandPass<PERROW, NR> &ps, float sc, int rank,
                                   const uint4 *bv, uint4 yv, int c, bool cin, float *red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float sv[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) sv[q] = lane < rank ? sc * ps.sv[q] : 0.f;
    float acc[NR][8];
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int j = wave + kWaves * u;
        if (j >= rank) break;
        const uint32_t bw[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
        float bf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bf[2 * e] = h2f((uint16_t)(bw[e] & 0xffff));
            bf[2 * e + 1] = h2f((uint16_t)(bw[e] >> 16));
        }
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sv[q]), j));
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = __builtin_fmaf(s, bf[e], acc[q][e]);
        }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[((wave * NR + q) * 8 + e) * 64 + lane] = acc[q][e];
    __syncthreads();
    if (ps.my_row >= 0 && cin && rank > 0) {
        const int q = wave;
        const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
        uint32_t out[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float d[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int e = 2 * e2 + h;
                d[h] = red[((0 * NR + q) * 8 + e) * 64 + lane] + red[((1 * NR + q) * 8 + e) * 64 + lane] +
                       red[((2 * NR + q) * 8 + e) * 64 + lane] + red[((3 * NR + q) * 8 + e) * 64 + lane];
            }
            const float lo = h2f((uint16_t)(yw[e2] & 0xffff)) + d[0];
            const float hi = h2f((uint16_t)(yw[e2] >> 16)) + d[1];
            out[e2] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
        }
        *reinterpret_cast<uint4 *>(pd.y + (int64_t)ps.my_row * pd.ldy + c) = make_uint4(out[0], out[1], out[2], out[3]);
    }
    __syncthreads();
}

// Wavefronts per SIMD the VALU expand is built for: 4 (at most 128 VGPRs) where that
// needs no spills.  The 2-row paged kernel at r_max 64 otherwise takes 133 VGPRs and
// keeps only 3; the 4-row paged kernel at r_max 64 would spill, so it is left alone.
template <bool PAGED, int NR, int RU>
constexpr int expand_valu_waves() { return PAGED && NR == 4 && RU == 16 ? 1 : 4; }

template <bool PAGED, bool PERROW, int NR, int RU, bool OFFS, bool SW = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(expand_valu_waves<PAGED, NR, RU>())))
void lora_expand_valu_kernel(Args args)
{
    const Args &a = kernel_args<!PAGED>(args);
    __shared__ float red[kWaves * NR * 8 * 64];
    const Item it = work_by_slice(a);
    if (!it.ok) return;
    prepare_tile<PERROW, OFFS, kThreads>(a.ts, a.n_rows, it.tile);
    const ProjDev pd = a.p[it.p];  // by value: the fields stay in registers
    const TileHead th = tile_head<PERROW, OFFS>(a.ts, pd.w, it.tile);
    if (!th.valid) return;
    const int rank = slot_rank(pd.w, th.slot);
    const int jlim = PAGED ? rank : pd.w.r_max;
    const float sc = pd.w.scale[th.slot];
    const int c = it.slice * kCols + 8 * (threadIdx.x & 63), wave = threadIdx.x >> 6;
    const bool cin = c < pd.w.d_out;
    if (th.nrows > NR) {
        // A tile taller than the launch was planned for (the row height is only a hint):
        // one row per pass, B loaded again for each.  Opaque per-pass copies of the
        // column, wavefront and rank limit keep the address arithmetic inside the loop:
        // hoisted out of it, it held ~60 VGPRs for the whole kernel and cost the planned
        // single pass half its resident wavefronts.
        for (int r = 0; r < th.nrows; ++r) {
            int cr = c, wr = wave, jr = jlim;
            asm volatile("" : "+v"(cr), "+v"(wr), "+v"(jr));
            ExpandPass<PERROW, 1> p1;
            p1.load(a, pd, th, r);
            const uint4 y1 = p1.load_y(pd, cr, cin);
            uint4 b1[RU];
            load_b_octets<PAGED, RU, SW>(pd.w, th.slot, jr, wr, 0, cr, cin, b1);
            expand_pass<PERROW, 1, RU>(pd, p1, sc, rank, b1, y1, cr, cin, red);
        }
        return;
    }
    // the tile's rows, v and y first: their loads are not queued behind B's
    ExpandPass<PERROW, NR> ps;
    ps.load(a, pd, th, 0);
    const uint4 yv = ps.load_y(pd, c, cin);
    uint4 bv[RU];
    load_b_octets<PAGED, RU, SW>(pd.w, th.slot, jlim, wave, 0, c, cin, bv);
    expand_pass<PERROW, NR, RU>(pd, ps, sc, rank, bv, yv, c, cin, red);
}

// MFMA expand for tiles of 8 to 64 rows (prefill segments, and decode batches whose rows
// share adapters): workgroup = (tile, 64 CW output columns, projection), each wavefront
// 16 CW of the columns with every rank-row, so each adapter's B is read once per tile
// (the VALU expand's 2-row tiles read it once per 2 rows) and no sums cross wavefronts.  CW (8 or 4 columns per
// lane) trades columns per workgroup for registers: 4 at ranks above 32.  Products on
// v_mfma_f32_16x16x16_f16 with A = s v (16 rows x 16 ranks, split into fp16 hi +
// lo/2048 parts: two MFMAs, ~22 bits kept) and B = the rank-rows, exact in fp16.  In
// 16-rank step s, lane (li, lg) loads rank-rows 16 s + 4 lg .. + 3 of B at its CW columns
// c .. c + CW - 1 (c = 16 CW w + CW li in the chunk) and gives MFMA m the four elements
// of column c + m, so MFMA m's output columns are c + m over the 16 lanes li; after the
// steps the lane holds rows 4 lg .. 4 lg + 3 of columns c .. c + CW - 1 and updates them
// in y (one fp16 rounding of y + the fp32 sum); each row span of 16 lanes is one or two
// whole 128-byte lines.  Each row's products
// run on s v 2^-ex with 2^ex above the row's largest |s v|, and the sum is scaled back,
// so the fp16 parts stay in fp16's normal range whatever the magnitude of v.  Every load
// is issued from an in-bounds (clamped) address and masked where its value is used, so
// a tile's loads are in flight together.  Tiles taller than 16 rows take one 16-row
// block after another with B kept in registers, the next block's v and y requested
// before the current block's products.  Work items are slice-major for tiles of up to 16
// rows (the tiles of one adapter then reuse each B chunk from L2, as in the VALU expand)
// and tile-major for taller tiles (prefill: consecutive workgroups sweep whole y rows).

// Row of position pos0 + min(i, nrows - 1) of a tile (a position inside the tile, so a
// row-map read stays in bounds), or -1 for i >= nrows or a row outside [0, n_rows).
// The per-lane read carries no branch of its own (only the uniform row-map test), so
// the compiler does not wait for every load in flight before it.
__device__ inline int tile_row(const TileSrc &ts, const TileHead &th, int i, int n_rows)
{
    const int pos = th.pos0 + min(i, th.nrows - 1);
    const bool pin = !ts.row_map || (pos >= 0 && pos < ts.n_pos);
    const int row = ts.row_map ? ts.row_map[min(max(pos, 0), max(ts.n_pos - 1, 0))] : pos;
    return (i < th.nrows && pin && row >= 0 && row < n_rows) ? row : -1;
}

// CW fp16 values (CW = 8 or 4) in 16 or 8 bytes.
template <int CW>
struct HalfVec {
    uint32_t w[CW / 2];
    __device__ uint32_t half(int m) const { return (m & 1) ? (w[m >> 1] >> 16) : (w[m >> 1] & 0xffff); }
};

// NT: a streaming load (y of tall tiles, see load16_nt).
template <int CW, bool NT = false>
__device__ inline HalfVec<CW> load_halves(const uint16_t *p)
{
    HalfVec<CW> h;
    if constexpr (CW == 8) {
        const uint4 q = NT ? load16_nt(p) : *reinterpret_cast<const uint4 *>(p);
        h.w[0] = q.x, h.w[1] = q.y, h.w[2] = q.z, h.w[3] = q.w;
    } else {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t q = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p))
                             : *reinterpret_cast<const u32x2_t *>(p);
        h.w[0] = q.x, h.w[1] = q.y;
    }
    return h;
}

// NT: a non-temporal (streaming) store.  The expand of tiles taller than 16 rows (prefill)
// reads and writes y of hundreds of MB, far beyond the L2 and memory-side caches, and
// streams both (see load16_nt; the stores alone measured 0.5 % faster per 7B prefill
// layer).  Short tiles keep normal accesses: there y is small and read again soon by the
// caller's next operation.
template <int CW, bool NT = false>
__device__ inline void store_halves(uint16_t *p, const HalfVec<CW> &h)
{
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (CW == 8) {
        const u32x4_t v{h.w[0], h.w[1], h.w[2], h.w[3]};
        if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
        else *reinterpret_cast<u32x4_t *>(p) = v;
    } else {
        const u32x2_t v{h.w[0], h.w[1]};
        if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(p));
        else *reinterpret_cast<u32x2_t *>(p) = v;
    }
}

// keep a loaded value in flight where it was issued (see the callers)
template <int CW>
__device__ inline void pin(HalfVec<CW> &h)
{
#pragma unroll
    for (int i = 0; i < CW / 2; ++i) asm volatile("" : "+v"(h.w[i]));
}

// Wavefronts per SIMD the MFMA expand is built for: four (at most 128 VGPRs) where that
// needs no spills, else three.
template <int RQ, int CW, bool TM>
constexpr int expand_mfma_waves() { return (TM && RQ > 1) || (!TM && RQ == 2) ? 3 : 4; }

template <bool PAGED, int RQ, int CW, bool TM, bool OFFS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(expand_mfma_waves<RQ, CW, TM>())))
void lora_expand_mfma_kernel(Args args)
{
    static_assert(CW == 8 || CW == 4, "columns per lane");
    constexpr int NB = 4 * RQ;  // rank-rows of B per lane: 4 in each 16-rank step
    const Args &a = kernel_args<!PAGED>(args);
    const Item it = TM ? work(a) : work_by_slice(a);
    if (!it.ok) return;
    prepare_tile<false, OFFS, kThreads>(a.ts, a.n_rows, it.tile);
    const ProjDev pd = a.p[it.p];  // by value: the fields stay in registers
    TileHead th = tile_head<false, OFFS>(a.ts, pd.w, it.tile);
    // uniform: the slot's rank, scale and B addresses come from scalar loads
    th.slot = __builtin_amdgcn_readfirstlane(th.slot);
    th.pos0 = __builtin_amdgcn_readfirstlane(th.pos0);
    th.nrows = __builtin_amdgcn_readfirstlane(th.nrows);
    if (!th.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int c = it.slice * (64 * CW) + 16 * CW * wave + CW * li;  // this lane's CW columns
    const bool cin = c < pd.w.d_out;
    const int cc = cin ? c : pd.w.d_out - CW;  // in-bounds stand-in (d_out is a multiple of 8)
    // operand row li of the first 16-row block; the rows this lane updates, 4 lg + e, are
    // the operand rows of lanes 4 lg + e
    int vr = tile_row(a.ts, th, li, a.n_rows);
    const int rank = slot_rank(pd.w, th.slot);
    const float sc = pd.w.scale[th.slot];
    const int r4 = (pd.w.r_max + 3) & ~3;  // a v row holds at least this many floats (ldv % 4 == 0)
    // B rank-rows 16 s + 4 lg + i at columns c .. c + 7.  Rank-rows below r_max are in
    // bounds (dense) or have their page-table entries checked (paged), so no load waits
    // for the rank.  Paged: page ids first (reads without a branch, so that what follows
    // waits for them alone), then v and y, then B's data.
    HalfVec<CW> bq[NB];
    int bpg[NB];
    const int P = PAGED ? pd.w.page_elems : 1, pq = cc / P, within = cc - pq * P;
    if (PAGED) {
        const int64_t ptb = pt_base<true>(pd.w, th.slot);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int j = min(16 * (k >> 2) + 4 * lg + (k & 3), pd.w.r_max - 1);
            const int64_t off = ptb + (int64_t)j * (pd.w.d_out / P) + pq;
            const bool in = off >= 0 && off < pd.w.pt_entries;
            const int e = pd.w.page_table[in ? off : 0];
            bpg[k] = in ? e : -1;
        }
    }
    float4 vq[RQ];
#pragma unroll
    for (int s = 0; s < RQ; ++s)
        vq[s] = *reinterpret_cast<const float4 *>(pd.v + (int64_t)max(vr, 0) * pd.ldv + min(16 * s + 4 * lg, r4 - 4));
    int yr[4];
    HalfVec<CW> yv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        yr[e] = __shfl(vr, 4 * lg + e);
        yv[e] = load_halves<CW, TM>(pd.y + (int64_t)max(yr[e], 0) * pd.ldy + cc);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
        if (!PAGED) {
            bpg[k] = 0;
            bq[k] = load_halves<CW>(dense_row<true>(pd.w, th.slot, min(16 * (k >> 2) + 4 * lg + (k & 3), pd.w.r_max - 1)) +
                                    cc);
        } else {
            bpg[k] = page_ok(pd.w, bpg[k]);  // page 0 stands in for a missing entry
            bq[k] = load_halves<CW>(page_ptr(pd.w, max(bpg[k], 0), within));
        }
    }
    // keep the y loads here, in flight with the others: otherwise the compiler sinks them
    // into the conditional update at the end, one more round trip after the products
#pragma unroll
    for (int e = 0; e < 4; ++e) pin<CW>(yv[e]);
    // B rank-rows at or past the rank (NaN in unfilled storage), past d_out or without a page: 0
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (!(cin && 16 * (k >> 2) + 4 * lg + (k & 3) < rank && bpg[k] >= 0))
#pragma unroll
            for (int i = 0; i < CW / 2; ++i) bq[k].w[i] = 0;
    // A rank-0 slot stores nothing (y stays as it is, bit for bit); tested as a predicate
    // at the store rather than by an early return, which the compiler would hoist above
    // the loads and so hold them back behind the rank.
    for (int m0 = 0;;) {
        // tile-major (tall tiles): the next 16-row block's rows, v and y go out before this
        // block's products (otherwise, for a tile taller than the hint, after them)
        const bool more = m0 + 16 < th.nrows;
        int vr_n = -1, yr_n[4] = {-1, -1, -1, -1};
        float4 vq_n[RQ];
        HalfVec<CW> yv_n[4];
        if (TM && more) {
            vr_n = tile_row(a.ts, th, m0 + 16 + li, a.n_rows);
#pragma unroll
            for (int s = 0; s < RQ; ++s)
                vq_n[s] = *reinterpret_cast<const float4 *>(pd.v + (int64_t)max(vr_n, 0) * pd.ldv +
                                                            min(16 * s + 4 * lg, r4 - 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yr_n[e] = __shfl(vr_n, 4 * lg + e);
                yv_n[e] = load_halves<CW, TM>(pd.y + (int64_t)max(yr_n[e], 0) * pd.ldy + cc);
            }
        }
        // row li's scale 2^ex: above max_j |s v[row][j]| (its four 16-lane groups)
        float mx = 0.f;
#pragma unroll
        for (int s = 0; s < RQ; ++s) {
            const float sv[4] = {vq[s].x, vq[s].y, vq[s].z, vq[s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (vr >= 0 && 16 * s + 4 * lg + e < rank) mx = __builtin_fmaxf(mx, __builtin_fabsf(sc * sv[e]));
        }
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        const int ex = mx > 0.f && mx <= 3.0e38f ? __builtin_amdgcn_frexp_expf(mx) : 0;
        f4_t acc[CW];
#pragma unroll
        for (int m = 0; m < CW; ++m) acc[m] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < RQ; ++s) {
            if (16 * s >= rank) break;
            const float sv[4] = {vq[s].x, vq[s].y, vq[s].z, vq[s].w};
            h4_t vhi, vlo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float m = (vr >= 0 && 16 * s + 4 * lg + e < rank) ? __builtin_ldexpf(sc * sv[e], -ex) : 0.f;
                const _Float16 hv = (_Float16)m;
                vhi[e] = hv;
                vlo[e] = (_Float16)((m - (float)hv) * 2048.f);
            }
#pragma unroll
            for (int m = 0; m < CW; ++m) {
                // column c + m of rank-rows 16 s + 4 lg .. + 3
                const uint32_t lo2 = bq[4 * s].half(m) | (bq[4 * s + 1].half(m) << 16);
                const uint32_t hi2 = bq[4 * s + 2].half(m) | (bq[4 * s + 3].half(m) << 16);
                const h4_t bop = __builtin_bit_cast(h4_t, make_uint2(lo2, hi2));
                f4_t lo = f4_t{0.f, 0.f, 0.f, 0.f};
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x16f16(vhi, bop, acc[m], 0, 0, 0);
                lo = __builtin_amdgcn_mfma_f32_16x16x16f16(vlo, bop, lo, 0, 0, 0);
                acc[m] += lo * (1.f / 2048.f);
            }
        }
        // lane (li, lg): acc[m][e] = row 4 lg + e, column c + m, in units of that row's 2^ex
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int exr = __shfl(ex, 4 * lg + e);
            if (yr[e] >= 0 && cin && rank > 0) {
                HalfVec<CW> out;
#pragma unroll
                for (int e2 = 0; e2 < CW / 2; ++e2) {
                    const float lo = h2f((uint16_t)yv[e].half(2 * e2)) + __builtin_ldexpf(acc[2 * e2][e], exr);
                    const float hi = h2f((uint16_t)yv[e].half(2 * e2 + 1)) + __builtin_ldexpf(acc[2 * e2 + 1][e], exr);
                    out.w[e2] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
                }
                store_halves<CW, TM>(pd.y + (int64_t)yr[e] * pd.ldy + c, out);
            }
        }
        if (!more) break;
        m0 += 16;
        if (TM) {
            vr = vr_n;
#pragma unroll
            for (int s = 0; s < RQ; ++s) vq[s] = vq_n[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yr[e] = yr_n[e];
                yv[e] = yv_n[e];
            }
        } else {
            vr = tile_row(a.ts, th, m0 + li, a.n_rows);
#pragma unroll
            for (int s = 0; s < RQ; ++s)
                vq[s] = *reinterpret_cast<const float4 *>(pd.v + (int64_t)max(vr, 0) * pd.ldv +
                                                          min(16 * s + 4 * lg, r4 - 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yr[e] = __shfl(vr, 4 * lg + e);
                yv[e] = load_halves<CW, TM>(pd.y + (int64_t)max(yr[e], 0) * pd.ldy + cc);
            }
        }
    }
}

// ------------------------------------------------------------------------ one launch, v handed off
// Shrink and expand in one launch, v passed from the shrink's workgroups to the
// expand's through a caller-owned workspace: the per-row form, and the segment form
// with VALU tiles (up to 4 rows).  Workgroups [0, n_shrink) run the shrink's work items
// and the rest the expand's.  The hardware hands out workgroup ids in increasing order,
// so every shrink workgroup has a CU before any expand workgroup that could wait for
// it, and shrink workgroups never wait; the waits are bounded all the same, and
// correctness does not rest on that order.
//   shrink workgroup: lora_shrink_valu_kernel's work item (same bits); besides v it
//     stores its entries into the hand-off row of each (row, projection),
//     device-coherently and bit-inverted, so that the zero of a cleared row means
//     "not yet";
//   expand workgroup: requests y and its rank-rows of B, then polls the hand-off rows
//     of its tile (wavefront q polls row q: one device-coherent load per lane, at most
//     `polls` times) until every entry is set, and runs lora_expand_valu_kernel's
//     arithmetic on them (same bits).  When the poll limit runs out it computes the
//     tile's v itself with the shrink's arithmetic (same bits again), so the result
//     never depends on scheduling;
//   a counter per (row, projection) takes every count of the launch: shrink items add
//     1 (bits 0-7) once their hand-off stores have completed, expand workgroups add
//     1 << 8 when done; whichever count completes the fixed total clears the hand-off
//     row and the counter, so the workspace is zero again when the launch ends, in any
//     order of events.  This needs every row in at most one tile, as the tile builder
//     makes them.
// A v whose bits invert to zero (one NaN pattern) is handed off as the canonical NaN.
constexpr int kHandoffWords = 128;  // per (row, projection): 64 hand-off entries, the counter on its own line

__device__ inline uint32_t *handoff_row(const HandoffDev &ho, int row, int p)
{
    return ho.work + (int64_t)kHandoffWords * (row * LORA_MAX_PROJ + p);
}

// Wavefront 0 of a workgroup adds `inc` to the (row, projection) counters of the rows
// it was given (lane q takes rows[q]; rows < 0 are skipped); a row whose count
// completes the launch's total (`need` shrink items, `e` expand workgroups) gets its
// hand-off row (r_max entries) and counter cleared.
template <int NR>
__device__ inline void handoff_count(const HandoffDev &ho, const int (&rows)[NR], int p, uint32_t inc, uint32_t need,
                                     uint32_t e, int r_max)
{
    const int lane = threadIdx.x & 63;
    int my = -1;
#pragma unroll
    for (int q = 0; q < NR; ++q) my = lane == q ? rows[q] : my;
    bool done = false;
    if (my >= 0) {
        uint32_t *cnt = handoff_row(ho, my, p) + kHandoffWords / 2;
        const uint32_t now = __hip_atomic_fetch_add(cnt, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + inc;
        done = (now & 0xFF) == need && ((now >> 8) & 0xFFFF) == e;
    }
    uint64_t m = __ballot(done);
    while (m) {
        const int q = __builtin_ctzll(m);
        m &= m - 1;
        const int row = __builtin_amdgcn_readlane(my, q);
        uint32_t *h = handoff_row(ho, row, p);
        if (lane < r_max) __hip_atomic_store(h + lane, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) __hip_atomic_store(h + kHandoffWords / 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Work item `wi` of a list with `per_tile` items per tile, projection p's from off[p].
__device__ inline Item tile_item(int wi, int per_tile, const int32_t *off, int n_proj, int n_tiles)
{
    Item it;
    it.tile = wi / per_tile;
    const int sl = wi - it.tile * per_tile;
    int p = 0;
#pragma unroll
    for (int q = 1; q < LORA_MAX_PROJ; ++q) p += (q < n_proj && sl >= off[q]) ? 1 : 0;
    it.p = p;
    it.slice = sl - off[p];
    it.ok = it.tile < n_tiles;
    return it;
}

// Rows rg .. rg + NR - 1 of a tile (-1 past its end or outside the row range).
template <bool PERROW, int NR>
__device__ inline void tile_rows(const Args &a, const TileHead &th, int rg, int (&rows)[NR])
{
#pragma unroll
    for (int q = 0; q < NR; ++q)
        rows[q] = rg + q < th.nrows ? row_of<PERROW>(a.ts, th.pos0 + rg + q, a.n_rows) : -1;
}

// The hand-off kernel takes four scalar arguments ahead of the argument block, which the
// hardware preloads into scalar registers (the library is built with kernel-argument
// preloading): the tile source (per-row slots or the tile list; NULL for the offsets
// form) and the grid layout.  With them each workgroup reads its tile's record at once,
// in parallel with the argument block instead of after it.
constexpr int kHandoffArgsOffset = 24;  // byte offset of the argument block after the four
                                        // leading arguments (8 + 3 * 4 bytes, 8-byte aligned)
static_assert(alignof(Args) == 8, "argument block alignment");

template <bool PAGED, bool PERROW, int RJ, int NR, int RU, bool OFFS, bool SW = false>
__global__ __launch_bounds__(kThreads) void lora_handoff_kernel(const void *__restrict__ pre_src, int32_t pre_n_shrink,
                                                                int32_t pre_per_tile, int32_t pre_e_per_tile, Args args)
{
    constexpr int kDH = RJ + NR == 2 ? 4 : 0;    // the shrink items' halves in flight (registers)
    __shared__ float red[kWaves * NR * 8 * 64];  // the shrink's kWaves * NR * RJ sums or the expand's
    __shared__ int pcache[PAGED ? kPageCache : 1];
    __shared__ float vrow[NR][LORA_MAX_RANK];
    __shared__ int s_ok[NR];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    // this workgroup's tile record, from the preloaded arguments (the grid holds exactly
    // n_tiles * (per_tile + e_per_tile) workgroups, so the tile exists)
    const bool have_early = pre_src != nullptr;
    lora_tile early{-1, 0, 0, -1};
    if (have_early) {
        const bool sh = b < pre_n_shrink;
        const int t = (sh ? b : b - pre_n_shrink) / (sh ? pre_per_tile : pre_e_per_tile);
        if constexpr (PERROW) early = lora_tile{static_cast<const int32_t *>(pre_src)[t], t, 1, t};
        else early = static_cast<const lora_tile *>(pre_src)[t];
    }
    const Args &a = PAGED ? args : touched_args_at<kHandoffArgsOffset>();
    // The item comes from kernel arguments read before the first branch (both parts'
    // layouts), so the slot and the projection's descriptor are one round trip later.
    const bool shrink = b < a.ho.n_shrink;
    int32_t off[LORA_MAX_PROJ];
#pragma unroll
    for (int q = 0; q < LORA_MAX_PROJ; ++q) off[q] = shrink ? a.off[q] : a.ho.e_off[q];
    const Item it = tile_item(shrink ? b : b - a.ho.n_shrink, shrink ? a.per_tile : a.ho.e_per_tile, off, a.n_proj,
                              a.n_tiles);
    if (!it.ok) return;
    prepare_tile<PERROW, OFFS, kThreads>(a.ts, a.n_rows, it.tile);
    if (shrink) {
        const bool stored = shrink_valu_item<PAGED, PERROW, RJ, NR, VSink::Handoff, kDH, OFFS, SW>(
            a, it, red, pcache, nullptr, -1, have_early, early);
        // wavefront 0 made every v store of this workgroup
        if (stored && wave == 0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the hand-off stores have completed
            const ProjDev &pd = a.p[it.p];
            const TileHead th = have_early ? head_of(early, pd.w) : tile_head<PERROW, OFFS>(a.ts, pd.w, it.tile);
            for (int rg = 0; rg < th.nrows; rg += NR) {
                int rows[NR];
                tile_rows<PERROW, NR>(a, th, rg, rows);
                handoff_count<NR>(a.ho, rows, it.p, 1u, pd.slices, a.ho.e_slices[it.p], pd.w.r_max);
            }
        }
        return;
    }
    const ProjDev pd = a.p[it.p];  // by value: the fields stay in registers
    const TileHead th = have_early ? head_of(early, pd.w) : tile_head<PERROW, OFFS>(a.ts, pd.w, it.tile);
    if (!th.valid) return;
    const int rank = slot_rank(pd.w, th.slot);
    const int jlim = PAGED ? rank : pd.w.r_max;
    const float sc = pd.w.scale[th.slot];
    const int c = it.slice * kCols + 8 * lane;
    const bool cin = c < pd.w.d_out;
    if (th.nrows > NR) {
        // A tile taller than the launch was planned for (the row height is only a hint):
        // each row's v computed here with the shrink's arithmetic, no waiting, one row at
        // a time (a cold path kept to the registers of the one-row kernels).
        for (int r = 0; r < th.nrows; ++r) {
            for (int sl = 0; sl < a.p[it.p].slices; ++sl) {
                const Item si{it.tile, it.p, sl, true};
                shrink_valu_item<PAGED, PERROW, 1, 1, VSink::Lds, 2, OFFS, SW>(a, si, red, pcache, &vrow[0][0], r, have_early,
                                                                     early);
            }
            ExpandPass<PERROW, 1> ps;
            tile_rows<PERROW, 1>(a, th, r, ps.rows);
            ps.my_row = wave == 0 ? ps.rows[0] : -1;
            const uint4 yv = ps.load_y(pd, c, cin);
            uint4 bw[RU];
            load_b_octets<PAGED, RU, SW>(pd.w, th.slot, jlim, wave, 0, c, cin, bw);
            ps.sv[0] = lane < pd.w.r_max ? vrow[0][lane] : 0.f;
            expand_pass<PERROW, 1, RU>(pd, ps, sc, rank, bw, yv, c, cin, red);
            if (wave == 0 && rank > 0)
                handoff_count<1>(a.ho, ps.rows, it.p, 1u << 8, pd.slices, a.ho.e_slices[it.p], pd.w.r_max);
        }
        return;
    }
    // the tile's rows (at most NR): y, then B, then v from the hand-off
    ExpandPass<PERROW, NR> ps;
    tile_rows<PERROW, NR>(a, th, 0, ps.rows);
    ps.my_row = ps.rows[0];  // rows[wave] without a dynamically indexed register array
#pragma unroll
    for (int q = 1; q < NR; ++q) ps.my_row = wave == q ? ps.rows[q] : ps.my_row;
    if (wave >= NR) ps.my_row = -1;
    const uint4 yv = ps.load_y(pd, c, cin);
    uint4 bv[RU];
    load_b_octets<PAGED, RU, SW>(pd.w, th.slot, jlim, wave, 0, c, cin, bv);
    // A rank-0 row's shrink items store nothing: such a workgroup neither waits nor
    // counts, and its expand writes nothing.  Tested as a predicate rather than by an
    // early return so that the loads above are not held back behind the rank.
    const bool active = rank > 0;
    {
        if (wave < NR) {
            bool ok = true;
            if (active && ps.my_row >= 0) {
                const uint32_t *h = handoff_row(a.ho, ps.my_row, it.p) + lane;
                const bool mine = lane < pd.w.r_max;
                uint32_t hv = 0;
                for (int n = 0;; ++n) {
                    hv = mine ? __hip_atomic_load(h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1u;
                    ok = __ballot(hv == 0) == 0;
                    if (ok || n >= a.ho.polls) break;
                    __builtin_amdgcn_s_sleep(8);
                }
                if (ok && mine) vrow[wave][lane] = __builtin_bit_cast(float, ~hv);
            }
            if (lane == 0) s_ok[wave] = ok;
        }
        __syncthreads();
        bool all_ok = true;
#pragma unroll
        for (int q = 0; q < NR; ++q) all_ok = all_ok && s_ok[q];
        if (!all_ok) {
            for (int sl = 0; sl < a.p[it.p].slices; ++sl) {
                const Item si{it.tile, it.p, sl, true};
                // one rank-row and one pair of halves at a time: few registers on a path
                // that only runs when the poll limit runs out
                shrink_valu_item<PAGED, PERROW, 1, NR, VSink::Lds, 2, OFFS, SW>(a, si, red, pcache, &vrow[0][0], 0, have_early,
                                                                      early);
            }
        }
#pragma unroll
        for (int q = 0; q < NR; ++q) ps.sv[q] = lane < pd.w.r_max ? vrow[q][lane] : 0.f;
        expand_pass<PERROW, NR, RU>(pd, ps, sc, rank, bv, yv, c, cin, red);
        if (wave == 0 && active)
            handoff_count<NR>(a.ho, ps.rows, it.p, 1u << 8, pd.slices, a.ho.e_slices[it.p], pd.w.r_max);
    }
}

// ------------------------------------------------------------------------ launchers
// Event pair attached to this thread's next kernel launch (lora_set_launch_events).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

// Set by lora_set_stream_weights for the calling thread: the per-row calls' rows use
// distinct adapters, so their dense weights are read with streaming loads.
thread_local int32_t t_stream_w = 0;

// A launch whose kernel takes leading scalar arguments before the argument block.
template <typename Kernel>
void launch_pre(Kernel kernel, dim3 grid, int threads, size_t lds, hipStream_t s, const void *src, int32_t n0,
                int32_t n1, int32_t n2, const Args &a)
{
    const dim3 block(threads);
    if (t_ev_start || t_ev_stop) {
        hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
        t_ev_start = t_ev_stop = nullptr;
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0, src, n0, n1, n2, a);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, src, n0, n1, n2, a);
    }
}

template <typename Kernel>
void launch(Kernel kernel, dim3 grid, int threads, size_t lds, hipStream_t s, const Args &a)
{
    const dim3 block(threads);
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
    if (seg->tiles) {
        if (seg->n_tiles < 0 || seg->n_pos < 0)
            return fail(LORA_E_SHAPE, "n_tiles = %d, n_pos = %d", seg->n_tiles, seg->n_pos);
        if (seg->max_rows < 0 || seg->max_rows > LORA_MAX_TILE_ROWS)
            return fail(LORA_E_SHAPE, "max_rows = %d outside 0..%d", seg->max_rows, LORA_MAX_TILE_ROWS);
        if (!aligned16(seg->tiles)) return fail(LORA_E_ALIGN, "tiles must be 16-byte aligned");
        return LORA_OK;
    }
    if (seg->n_tiles != 0) return fail(LORA_E_NULL, "n_tiles = %d without a tile list", seg->n_tiles);
    if (seg->n_seg < 0) return fail(LORA_E_SHAPE, "n_seg = %d", seg->n_seg);
    if (seg->tile_rows < 0 || seg->tile_rows > LORA_MAX_TILE_ROWS)
        return fail(LORA_E_SHAPE, "tile_rows = %d outside 0..%d", seg->tile_rows, LORA_MAX_TILE_ROWS);
    if (seg->n_seg > 0 && (!seg->seg_ptr || !seg->seg_slot)) return fail(LORA_E_NULL, "seg_ptr and seg_slot are required");
    return LORA_OK;
}

// How a checked segment descriptor is launched over n_rows rows: its tile source, the
// number of tiles the grid covers and the tallest tile.  The offsets form covers
// n_rows / T + n_seg tiles (an upper bound of sum ceil(len / T) over segments of at
// most n_rows positions in all); workgroups past the batch's last tile do nothing.
struct SegLaunch {
    TileSrc ts;
    int32_t n_tiles, max_rows;
};

int seg_launch(const lora_segments *seg, int32_t n_rows, SegLaunch &sl)
{
    sl.ts = TileSrc{};
    sl.ts.row_map = seg->row_map;
    if (seg->tiles) {
        sl.ts.tiles = seg->tiles;
        sl.ts.n_pos = seg->n_pos;
        sl.n_tiles = seg->n_tiles;
        sl.max_rows = seg->max_rows > 0 ? seg->max_rows : LORA_MAX_TILE_ROWS;
        return LORA_OK;
    }
    const int32_t T = seg->tile_rows > 0 ? seg->tile_rows : lora_tile_rows_for(n_rows, seg->n_seg);
    const int64_t bound = seg->n_seg > 0 ? (int64_t)std::max(n_rows, 0) / T + seg->n_seg : 0;
    if (bound > ((int64_t)1 << 28)) return fail(LORA_E_SHAPE, "%lld tiles are too many for one launch", (long long)bound);
    sl.ts.seg_ptr = seg->seg_ptr;
    sl.ts.seg_slot = seg->seg_slot;
    sl.ts.n_seg = seg->n_seg;
    sl.ts.tile_rows = T;
    sl.ts.n_pos = n_rows;
    sl.n_tiles = (int32_t)bound;
    sl.max_rows = T;
    return LORA_OK;
}

// Checks the projection list shared by shrink and expand; fills the per-projection
// parts of `a` that do not depend on the kernel.
int check_projs(int32_t n_proj, const lora_proj *proj, bool expand, Args &a, bool &paged)
{
    if (n_proj < 1 || n_proj > LORA_MAX_PROJ)
        return fail(LORA_E_SHAPE, "n_proj = %d outside 1..%d", n_proj, LORA_MAX_PROJ);
    if (!proj) return fail(LORA_E_NULL, "projection list is NULL");
    for (int32_t p = 0; p < n_proj; ++p) {
        const lora_weights *w = proj[p].w;
        int st = check_weights_desc(w);
        if (st) return st;
        if (p > 0 && w->layout != proj[0].w->layout)
            return fail(LORA_E_UNSUPPORTED, "projections of one launch must share the weight layout");
        if ((st = check_rows_arg(proj[p].v, proj[p].ldv, w->r_max, 4, "v"))) return st;
        if (expand && (st = check_rows_arg(proj[p].y, proj[p].ldy, w->d_out, 8, "y"))) return st;
        a.p[p].w = to_dev(w);
        a.p[p].v = proj[p].v;
        a.p[p].ldv = proj[p].ldv;
        a.p[p].y = static_cast<uint16_t *>(proj[p].y);
        a.p[p].ldy = proj[p].ldy;
    }
    paged = proj[0].w->layout == LORA_LAYOUT_PAGED;
    a.n_proj = n_proj;
    return LORA_OK;
}

inline int32_t pad8(int64_t g) { return (int32_t)((g + 7) & ~int64_t(7)); }

int finish_layout(Args &a, int32_t n_tiles)
{
    int32_t off = 0;
    for (int32_t p = 0; p < LORA_MAX_PROJ; ++p) {
        a.off[p] = off;
        if (p < a.n_proj) off += a.p[p].slices;
    }
    a.per_tile = off;
    const int64_t items = (int64_t)n_tiles * off;
    if (items > (int64_t)1 << 30) return fail(LORA_E_SHAPE, "launch of %lld work items is too large", (long long)items);
    a.grid = pad8(items);
    return LORA_OK;
}

// Rows per pass of the VALU kernels in the segment form: the tiles' height rounded up to
// 1, 2 or 4 (no pass computes on rows a tile does not have), unless lora_set_plan fixed it.
int rows_per_pass(int32_t max_rows)
{
    if (t_plan_nr > 0) return t_plan_nr;
    return max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : kRowsPerPass;
}

template <bool PERROW, int NR, bool OFFS>
void shrink_valu_launch(bool paged, int32_t jw, dim3 grid, hipStream_t s, const Args &a)
{
// Per-row launches with dense weights stream the weights when the caller said the rows'
// adapters are distinct (lora_set_stream_weights); SW = PERROW keeps the segment form on
// its one instance.
#define LORA_SHRINK_VALU(RJ)                                                                                   \
    (paged           ? launch(lora_shrink_valu_kernel<true, PERROW, RJ, NR, OFFS>, grid, kThreads, 0, s, a)     \
     : t_stream_w    ? launch(lora_shrink_valu_kernel<false, PERROW, RJ, NR, OFFS, PERROW>, grid, kThreads, 0, s, a) \
                     : launch(lora_shrink_valu_kernel<false, PERROW, RJ, NR, OFFS>, grid, kThreads, 0, s, a))
    if (jw == 1) LORA_SHRINK_VALU(1);
    else if (jw == 2) LORA_SHRINK_VALU(2);
    else LORA_SHRINK_VALU(4);
#undef LORA_SHRINK_VALU
}

template <bool PERROW, int NR, bool OFFS>
void expand_valu_launch(bool paged, int32_t r_max, dim3 grid, hipStream_t s, const Args &a)
{
#define LORA_EXPAND_VALU(RU)                                                                                   \
    (paged           ? launch(lora_expand_valu_kernel<true, PERROW, NR, RU, OFFS>, grid, kThreads, 0, s, a)     \
     : t_stream_w    ? launch(lora_expand_valu_kernel<false, PERROW, NR, RU, OFFS, PERROW>, grid, kThreads, 0, s, a) \
                     : launch(lora_expand_valu_kernel<false, PERROW, NR, RU, OFFS>, grid, kThreads, 0, s, a))
    if (r_max <= 16) LORA_EXPAND_VALU(4);
    else if (r_max <= 32) LORA_EXPAND_VALU(8);
    else LORA_EXPAND_VALU(16);
#undef LORA_EXPAND_VALU
}

// OFFS: the segment form given as offsets (each workgroup derives its tile).
template <bool PERROW, bool OFFS = false>
int shrink_impl(void *stream, const void *x, int64_t ldx, int32_t n_rows, TileSrc ts, int32_t n_tiles,
                int32_t max_rows, int32_t n_proj, const lora_proj *proj)
{
    Args a{};
    bool paged = false;
    int st = check_projs(n_proj, proj, false, a, paged);
    if (st) return st;
    for (int32_t p = 1; p < n_proj; ++p)
        if (proj[p].w->d_in != proj[0].w->d_in)
            return fail(LORA_E_SHAPE, "projections of one shrink launch share x: d_in %d != %d", proj[p].w->d_in,
                        proj[0].w->d_in);
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0 || n_tiles == 0) return LORA_OK;
    if ((st = check_rows_arg(x, ldx, proj[0].w->d_in, 8, "x"))) return st;
    int32_t r_max = 0;
    for (int32_t p = 0; p < n_proj; ++p) r_max = std::max(r_max, proj[p].w->r_max);
    const bool mfma = !PERROW && max_rows >= kMfmaMinRows;
    a.jw = mfma ? 16 : plan_shrink_jw(n_tiles * n_proj, r_max);
    for (int32_t p = 0; p < n_proj; ++p) a.p[p].slices = (proj[p].w->r_max + a.jw - 1) / a.jw;
    if ((st = finish_layout(a, n_tiles))) return st;
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.n_rows = n_rows;
    a.n_tiles = n_tiles;
    a.ts = ts;
    const dim3 grid((unsigned)a.grid);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mfma) {
        // rank slices per workgroup: all of the tile's (up to 4, up to 3 with 64-row tiles,
        // whose staged chunk and prefetch registers leave no room for a fourth) share one
        // read of x
        const int mtx = (max_rows + 15) / 16;
        const int ns_max = mtx > 2 ? 3 : 4;
        const int ns = paged ? 1 : (a.per_tile + (a.per_tile + ns_max - 1) / ns_max - 1) /
                                       ((a.per_tile + ns_max - 1) / ns_max);
        // A single rank slice per tile (one projection of rank <= 16) with 64-row tiles:
        // the wave-staged kernel, each tile's rows in two workgroups of 32 (the tiles alone
        // leave CUs idle); each reads the slice's A^T itself (from L2).
        const bool wave = !paged && mtx > 2 && ns == 1;
        a.grid = pad8((int64_t)n_tiles * (wave ? 2 : 1) * ((a.per_tile + ns - 1) / ns));
        const dim3 g((unsigned)a.grid);
#define LORA_SHRINK_STAGED(MTX, NS) \
    launch(lora_shrink_mfma_staged_kernel<MTX, NS, OFFS>, g, kMfmaShrinkThreads, stage_lds_bytes(MTX, NS), s, a)
        if (paged) {
            if (mtx <= 1) launch(lora_shrink_mfma_kernel<true, 1, 1, OFFS>, g, kMfmaShrinkThreads, 0, s, a);
            else if (mtx == 2) launch(lora_shrink_mfma_kernel<true, 2, 1, OFFS>, g, kMfmaShrinkThreads, 0, s, a);
            else launch(lora_shrink_mfma_kernel<true, 4, 1, OFFS>, g, kMfmaShrinkThreads, 0, s, a);
        } else if (mtx <= 1) {
            if (ns == 1) LORA_SHRINK_STAGED(1, 1);
            else if (ns == 2) LORA_SHRINK_STAGED(1, 2);
            else if (ns == 3) LORA_SHRINK_STAGED(1, 3);
            else LORA_SHRINK_STAGED(1, 4);
        } else if (mtx == 2) {
            if (ns == 1) LORA_SHRINK_STAGED(2, 1);
            else if (ns == 2) LORA_SHRINK_STAGED(2, 2);
            else if (ns == 3) LORA_SHRINK_STAGED(2, 3);
            else LORA_SHRINK_STAGED(2, 4);
        } else if (wave) {
            launch(lora_shrink_mfma_wave_kernel<2, 1, 2, OFFS>, g, kThreads, wave_lds_bytes(2, 1), s, a);
        } else {
            if (ns == 2) LORA_SHRINK_STAGED(4, 2);
            else LORA_SHRINK_STAGED(4, 3);
        }
#undef LORA_SHRINK_STAGED
    } else if constexpr (PERROW) {
        shrink_valu_launch<true, 1, false>(paged, a.jw, grid, s, a);
    } else {
        const int nr = rows_per_pass(max_rows);
        if (nr == 1) shrink_valu_launch<false, 1, OFFS>(paged, a.jw, grid, s, a);
        else if (nr == 2) shrink_valu_launch<false, 2, OFFS>(paged, a.jw, grid, s, a);
        else shrink_valu_launch<false, 4, OFFS>(paged, a.jw, grid, s, a);
    }
    return launch_status("shrink");
}

template <bool PERROW, bool OFFS = false>
int expand_impl(void *stream, int32_t n_rows, TileSrc ts, int32_t n_tiles, int32_t max_rows, int32_t n_proj,
                const lora_proj *proj)
{
    Args a{};
    bool paged = false;
    int st = check_projs(n_proj, proj, true, a, paged);
    if (st) return st;
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0 || n_tiles == 0) return LORA_OK;
    int32_t r_max = 0;
    for (int32_t p = 0; p < n_proj; ++p) r_max = std::max(r_max, proj[p].w->r_max);
    // tiles of 8 rows or more: the MFMA expand (tile-major items above 16 rows); shorter:
    // VALU (whose results the one-launch segment form reproduces bit for bit)
    const bool mfma = !PERROW && max_rows >= kMfmaMinRows;
    const bool tm = max_rows > 16;
    const int cols = mfma && r_max > 32 ? 256 : kCols;  // the MFMA expand's columns per workgroup
    for (int32_t p = 0; p < n_proj; ++p) a.p[p].slices = (proj[p].w->d_out + cols - 1) / cols;
    if ((st = finish_layout(a, n_tiles))) return st;
    a.n_rows = n_rows;
    a.n_tiles = n_tiles;
    a.ts = ts;
    const dim3 grid((unsigned)a.grid);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mfma) {
#define LORA_EXPAND_MFMA(RQ)                                                                             \
    (paged ? (tm ? launch(lora_expand_mfma_kernel<true, RQ, (RQ > 2 ? 4 : 8), true, OFFS>, grid, kThreads, 0, s, a)   \
                 : launch(lora_expand_mfma_kernel<true, RQ, (RQ > 2 ? 4 : 8), false, OFFS>, grid, kThreads, 0, s, a))  \
           : (tm ? launch(lora_expand_mfma_kernel<false, RQ, (RQ > 2 ? 4 : 8), true, OFFS>, grid, kThreads, 0, s, a)  \
                 : launch(lora_expand_mfma_kernel<false, RQ, (RQ > 2 ? 4 : 8), false, OFFS>, grid, kThreads, 0, s, a)))
        const int rq = (r_max + 15) / 16;
        if (rq == 1) LORA_EXPAND_MFMA(1);
        else if (rq == 2) LORA_EXPAND_MFMA(2);
        else if (rq == 3) LORA_EXPAND_MFMA(3);
        else LORA_EXPAND_MFMA(4);
#undef LORA_EXPAND_MFMA
    } else if constexpr (PERROW) {
        expand_valu_launch<true, 1, false>(paged, r_max, grid, s, a);
    } else {
        const int nr = rows_per_pass(max_rows);
        if (nr == 1) expand_valu_launch<false, 1, OFFS>(paged, r_max, grid, s, a);
        else if (nr == 2) expand_valu_launch<false, 2, OFFS>(paged, r_max, grid, s, a);
        else expand_valu_launch<false, 4, OFFS>(paged, r_max, grid, s, a);
    }
    return launch_status("expand");
}

TileSrc row_src(const int32_t *idx)
{
    TileSrc ts{};
    ts.idx = idx;
    return ts;
}

constexpr int32_t kHandoffPolls = 1 << 15;  // ~30 ms of polling before computing v locally
thread_local int32_t t_handoff_polls = kHandoffPolls;
constexpr int64_t kResidentGroups = 2048;   // 256 CUs x 8 workgroups of 4 wavefronts (<= 64 VGPRs)

int check_workspace(const void *work, size_t work_bytes, int32_t n_rows)
{
    if (!work) return fail(LORA_E_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(work) & 255) return fail(LORA_E_ALIGN, "workspace must be 256-byte aligned");
    if (work_bytes < lora_handoff_bytes(n_rows))
        return fail(LORA_E_SHAPE, "workspace of %zu bytes < %zu for %d rows", work_bytes, lora_handoff_bytes(n_rows),
                    n_rows);
    return LORA_OK;
}

// One launch with v handed off (lora_handoff_kernel) over n_tiles tiles of at most
// max_rows rows (the per-row form: one row per tile).  Arguments other than the
// workspace are checked by the caller; the segment form comes here with dense weights
// and tiles of fewer than kMfmaMinRows rows only.
template <bool PERROW, bool OFFS = false>
int handoff_impl(void *stream, const void *x, int64_t ldx, int32_t n_rows, TileSrc ts, int32_t n_tiles,
                 int32_t max_rows, int32_t n_proj, const lora_proj *proj, Args &a, bool paged, void *work,
                 size_t work_bytes)
{
    int st = check_workspace(work, work_bytes, n_rows);
    if (st) return st;
    int32_t r_max = 0, e_per_tile = 0;
    for (int32_t p = 0; p < n_proj; ++p) r_max = std::max(r_max, proj[p].w->r_max);
    for (int32_t p = 0; p < LORA_MAX_PROJ; ++p) {
        a.ho.e_off[p] = e_per_tile;
        a.ho.e_slices[p] = p < n_proj ? (proj[p].w->d_out + kCols - 1) / kCols : 0;
        if (a.ho.e_slices[p] > 0xFFFF)
            return fail(LORA_E_SHAPE, "d_out = %d is too wide for one launch", proj[p].w->d_out);
        e_per_tile += a.ho.e_slices[p];
    }
    a.ho.e_per_tile = e_per_tile;
    // rank-rows per shrink item: at least the separate shrink's choice, and the narrowest
    // that keeps both parts within what the CUs hold at once and gives a tile at most 8
    // shrink items, else 4 (a 7B decode o or down unit, r 16: 8 items of 2 rank-rows
    // measured 6.9 / 9.1 us against 7.4-7.9 / 9.2-9.3 with 16 of one)
    a.jw = plan_shrink_jw(n_tiles * n_proj, r_max);
    for (;; a.jw *= 2) {
        int64_t s_per_tile = 0;
        for (int32_t p = 0; p < n_proj; ++p) s_per_tile += (proj[p].w->r_max + a.jw - 1) / a.jw;
        if (a.jw >= 4 || (n_tiles * (s_per_tile + e_per_tile) <= kResidentGroups && s_per_tile <= 8)) break;
    }
    if (t_plan_jw > 0) a.jw = t_plan_jw;
    for (int32_t p = 0; p < n_proj; ++p) a.p[p].slices = (proj[p].w->r_max + a.jw - 1) / a.jw;
    if ((st = finish_layout(a, n_tiles))) return st;
    const int64_t groups = (int64_t)n_tiles * (a.per_tile + e_per_tile);
    if (groups > ((int64_t)1 << 30)) return fail(LORA_E_SHAPE, "launch of %lld workgroups is too large", (long long)groups);
    a.ho.work = static_cast<uint32_t *>(work);
    a.ho.n_shrink = n_tiles * a.per_tile;
    a.ho.polls = t_handoff_polls;
    a.grid = (int32_t)groups;
    a.x = static_cast<const uint16_t *>(x);
    a.ldx = ldx;
    a.n_rows = n_rows;
    a.n_tiles = n_tiles;
    a.ts = ts;
    const dim3 grid((unsigned)a.grid);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the preloaded leading arguments: tile source and grid layout
    const void *pre_src = PERROW ? static_cast<const void *>(ts.idx) : static_cast<const void *>(ts.tiles);
#define LORA_HANDOFF_RU(PG, RJ, NR, SW)                                                                          \
    if (r_max <= 16)                                                                                             \
        launch_pre(lora_handoff_kernel<PG, PERROW, RJ, NR, 4, OFFS, SW>, grid, kThreads, 0, s, pre_src,          \
                   a.ho.n_shrink, a.per_tile, a.ho.e_per_tile, a);                                               \
    else if (r_max <= 32)                                                                                        \
        launch_pre(lora_handoff_kernel<PG, PERROW, RJ, NR, 8, OFFS, SW>, grid, kThreads, 0, s, pre_src,          \
                   a.ho.n_shrink, a.per_tile, a.ho.e_per_tile, a);                                               \
    else                                                                                                         \
        launch_pre(lora_handoff_kernel<PG, PERROW, RJ, NR, 16, OFFS, SW>, grid, kThreads, 0, s, pre_src,         \
                   a.ho.n_shrink, a.per_tile, a.ho.e_per_tile, a)
#define LORA_HANDOFF_JW(PG, NR, SW)                          \
    if (a.jw == 1) { LORA_HANDOFF_RU(PG, 1, NR, SW); }        \
    else if (a.jw == 2) { LORA_HANDOFF_RU(PG, 2, NR, SW); }   \
    else { LORA_HANDOFF_RU(PG, 4, NR, SW); }
    if constexpr (PERROW) {
        (void)max_rows;
        if (paged) { LORA_HANDOFF_JW(true, 1, false) }
        else if (t_stream_w) { LORA_HANDOFF_JW(false, 1, true) }
        else { LORA_HANDOFF_JW(false, 1, false) }
    } else {
        const int nr = rows_per_pass(max_rows);
        if (nr == 1) { LORA_HANDOFF_JW(false, 1, false) }
        else if (nr == 2) { LORA_HANDOFF_JW(false, 2, false) }
        else { LORA_HANDOFF_JW(false, 4, false) }
    }
#undef LORA_HANDOFF_JW
#undef LORA_HANDOFF_RU
    return launch_status("shrink and expand with v handed off");
}


lora_proj one_proj(const lora_weights *w, float *v, int64_t ldv, void *y, int64_t ldy)
{
    lora_proj p;
    p.w = w;
    p.v = v;
    p.ldv = ldv;
    p.y = y;
    p.ldy = ldy;
    return p;
}

}  // namespace

thread_local int32_t t_plan_jw = 0, t_plan_nr = 0;

int32_t plan_shrink_jw(int32_t work_tiles, int32_t r_max)
{
    // The narrowest rank-row group (most workgroups in flight) that keeps the grid at
    // or below kTargetGroups.  Measured on MI355X, more and shorter workgroups beat
    // wider groups that re-read x less, and also beat longer streaming ones.
    int32_t jw = 1;
    while (jw < 4 && (int64_t)work_tiles * ((r_max + jw - 1) / jw) > kTargetGroups) jw *= 2;
    return t_plan_jw > 0 ? t_plan_jw : jw;
}

// ------------------------------------------------------------------------ hand-off without allocation
// lora_bgmv_multi_handoff_noalloc: the hand-off workspace is this file-scope array, one
// copy per GPU, instead of caller memory.  Host code never passes `scratch` itself (its
// name is a host-side stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current, and only
// that address reaches a kernel.  Every call on one GPU shares its copy; the hand-off
// protocol leaves it all zero after each call, so calls ordered on one stream may
// follow each other, while calls that may overlap on one GPU race.
constexpr int32_t kNoallocRows = LORA_NOALLOC_MAX_ROWS;
constexpr size_t kNoallocWords = (size_t)kNoallocRows * LORA_MAX_PROJ * kHandoffWords;
static __device__ __align__(256) uint32_t scratch[kNoallocWords];  // 2 MiB on every GPU

constexpr int kMaxDevices = 64;
uint32_t *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not set up)
std::mutex g_scratch_mu;

__global__ __launch_bounds__(kThreads) void lora_clear_words(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) p[i] = 0u;
}

// This device's scratch address; set up on the first call on the device: the address,
// then a clear of the whole array on `s` (a kernel, so it may be captured in a graph;
// the array starts zero anyway).
int noalloc_scratch(hipStream_t s, uint32_t *&ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LORA_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LORA_E_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(LORA_E_HIP, "hipGetSymbolAddress of the hand-off scratch: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(lora_clear_words, dim3(256), dim3(kThreads), 0, s, static_cast<uint32_t *>(p), kNoallocWords);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(LORA_E_HIP, "clearing the hand-off scratch: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<uint32_t *>(p);
    }
    ptr = g_scratch_ptr[dev];
    return LORA_OK;
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

int lora_set_stream_weights(int32_t on)
{
    clear_error();
    if (on != 0 && on != 1) return fail(LORA_E_SHAPE, "on = %d is not 0 or 1", on);
    t_stream_w = on;
    return LORA_OK;
}

int lora_set_plan(int32_t shrink_rank_rows, int32_t rows_per_pass)
{
    clear_error();
    if (shrink_rank_rows < 0 || shrink_rank_rows > LORA_MAX_RANK)
        return fail(LORA_E_SHAPE, "shrink_rank_rows = %d outside 0..%d", shrink_rank_rows, LORA_MAX_RANK);
    if (rows_per_pass != 0 && rows_per_pass != 1 && rows_per_pass != 2 && rows_per_pass != 4)
        return fail(LORA_E_SHAPE, "rows_per_pass = %d is not 0, 1, 2 or 4", rows_per_pass);
    t_plan_jw = shrink_rank_rows;
    t_plan_nr = rows_per_pass;
    return LORA_OK;
}

int lora_sgmv_shrink_multi(void *stream, const void *x, int64_t ldx, int32_t n_rows, const lora_segments *seg,
                           int32_t n_proj, const lora_proj *proj)
{
    clear_error();
    SegLaunch sl;
    int st = check_segments(seg);
    if (st || (st = seg_launch(seg, n_rows, sl))) return st;
    return sl.ts.tiles ? shrink_impl<false, false>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, sl.max_rows, n_proj, proj)
                       : shrink_impl<false, true>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, sl.max_rows, n_proj, proj);
}

int lora_sgmv_expand_multi(void *stream, int32_t n_rows, const lora_segments *seg, int32_t n_proj,
                           const lora_proj *proj)
{
    clear_error();
    SegLaunch sl;
    int st = check_segments(seg);
    if (st || (st = seg_launch(seg, n_rows, sl))) return st;
    return sl.ts.tiles ? expand_impl<false, false>(stream, n_rows, sl.ts, sl.n_tiles, sl.max_rows, n_proj, proj)
                       : expand_impl<false, true>(stream, n_rows, sl.ts, sl.n_tiles, sl.max_rows, n_proj, proj);
}

int lora_bgmv_shrink_multi(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                           int32_t n_proj, const lora_proj *proj)
{
    clear_error();
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    return shrink_impl<true>(stream, x, ldx, n_rows, row_src(idx), n_rows, 1, n_proj, proj);
}

int lora_bgmv_expand_multi(void *stream, const int32_t *idx, int32_t n_rows, int32_t n_proj, const lora_proj *proj)
{
    clear_error();
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    return expand_impl<true>(stream, n_rows, row_src(idx), n_rows, 1, n_proj, proj);
}

int lora_sgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx, int32_t n_rows,
                     const lora_weights *w, const lora_segments *seg)
{
    const lora_proj p = one_proj(w, v, ldv, nullptr, 0);
    return lora_sgmv_shrink_multi(stream, x, ldx, n_rows, seg, 1, &p);
}

int lora_sgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv, int32_t n_rows,
                     const lora_weights *w, const lora_segments *seg)
{
    const lora_proj p = one_proj(w, const_cast<float *>(v), ldv, y, ldy);
    return lora_sgmv_expand_multi(stream, n_rows, seg, 1, &p);
}

int lora_bgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx, const int32_t *idx,
                     int32_t n_rows, const lora_weights *w)
{
    const lora_proj p = one_proj(w, v, ldv, nullptr, 0);
    return lora_bgmv_shrink_multi(stream, x, ldx, idx, n_rows, 1, &p);
}

int lora_bgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv, const int32_t *idx,
                     int32_t n_rows, const lora_weights *w)
{
    const lora_proj p = one_proj(w, const_cast<float *>(v), ldv, y, ldy);
    return lora_bgmv_expand_multi(stream, idx, n_rows, 1, &p);
}

// Checks shared by the one-launch and two-launch decode entry points.
static int check_bgmv_multi(const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows, int32_t n_proj,
                            const lora_proj *proj, Args &a, bool &paged)
{
    if (n_rows > 0 && !idx) return fail(LORA_E_NULL, "idx is NULL");
    int st = check_projs(n_proj, proj, true, a, paged);
    if (st) return st;
    for (int32_t p = 1; p < n_proj; ++p)
        if (proj[p].w->d_in != proj[0].w->d_in)
            return fail(LORA_E_SHAPE, "projections of one launch share x: d_in %d != %d", proj[p].w->d_in,
                        proj[0].w->d_in);
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (n_rows == 0) return LORA_OK;
    return check_rows_arg(x, ldx, proj[0].w->d_in, 8, "x");
}

int lora_bgmv_multi(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows, int32_t n_proj,
                    const lora_proj *proj)
{
    clear_error();
    // Check everything both steps need before launching either.
    Args a{};
    bool paged = false;
    int st = check_bgmv_multi(x, ldx, idx, n_rows, n_proj, proj, a, paged);
    if (st || n_rows == 0) return st;
    st = shrink_impl<true>(stream, x, ldx, n_rows, row_src(idx), n_rows, 1, n_proj, proj);
    if (st) return st;
    return expand_impl<true>(stream, n_rows, row_src(idx), n_rows, 1, n_proj, proj);
}

size_t lora_handoff_bytes(int32_t n_rows)
{
    return n_rows > 0 ? (size_t)n_rows * LORA_MAX_PROJ * kHandoffWords * sizeof(uint32_t) : 0;
}

int lora_bgmv_multi_handoff(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                            int32_t n_proj, const lora_proj *proj, void *work, size_t work_bytes)
{
    clear_error();
    Args a{};
    bool paged = false;
    int st = check_bgmv_multi(x, ldx, idx, n_rows, n_proj, proj, a, paged);
    if (st || n_rows == 0) return st;
    return handoff_impl<true>(stream, x, ldx, n_rows, row_src(idx), n_rows, 1, n_proj, proj, a, paged, work,
                              work_bytes);
}

int lora_bgmv_multi_handoff_noalloc(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                                    int32_t n_proj, const lora_proj *proj)
{
    clear_error();
    Args a{};
    bool paged = false;
    int st = check_bgmv_multi(x, ldx, idx, n_rows, n_proj, proj, a, paged);
    if (st || n_rows == 0) return st;
    if (n_rows > kNoallocRows)
        return fail(LORA_E_SHAPE, "n_rows = %d exceeds the %d rows of the library's hand-off scratch", n_rows,
                    kNoallocRows);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *work = nullptr;
    if ((st = noalloc_scratch(s, work))) return st;
    return handoff_impl<true>(stream, x, ldx, n_rows, row_src(idx), n_rows, 1, n_proj, proj, a, paged, work,
                              kNoallocWords * sizeof(uint32_t));
}

int lora_sgmv_multi_handoff(void *stream, const void *x, int64_t ldx, int32_t n_rows, const lora_segments *seg,
                            int32_t n_proj, const lora_proj *proj, void *work, size_t work_bytes)
{
    clear_error();
    Args a{};
    bool paged = false;
    int st = check_segments(seg);
    if (st) return st;
    if ((st = check_projs(n_proj, proj, true, a, paged))) return st;
    for (int32_t p = 1; p < n_proj; ++p)
        if (proj[p].w->d_in != proj[0].w->d_in)
            return fail(LORA_E_SHAPE, "projections of one launch share x: d_in %d != %d", proj[p].w->d_in,
                        proj[0].w->d_in);
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    SegLaunch sl;
    if ((st = seg_launch(seg, n_rows, sl))) return st;
    if (n_rows == 0 || sl.n_tiles == 0) return LORA_OK;
    if ((st = check_rows_arg(x, ldx, proj[0].w->d_in, 8, "x"))) return st;
    const int32_t max_rows = sl.max_rows;
    if (paged || max_rows >= kMfmaMinRows) {
        // the two launches: the MFMA kernels' tiles and paged weights hand nothing off
        if ((st = check_workspace(work, work_bytes, n_rows))) return st;
        if (sl.ts.tiles) {
            st = shrink_impl<false, false>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj);
            return st ? st : expand_impl<false, false>(stream, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj);
        }
        st = shrink_impl<false, true>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj);
        return st ? st : expand_impl<false, true>(stream, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj);
    }
    if (sl.ts.tiles)
        return handoff_impl<false, false>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj, a, paged,
                                          work, work_bytes);
    return handoff_impl<false, true>(stream, x, ldx, n_rows, sl.ts, sl.n_tiles, max_rows, n_proj, proj, a, paged,
                                     work, work_bytes);
}

int lora_set_handoff_polls(int32_t polls)
{
    clear_error();
    t_handoff_polls = polls < 0 ? kHandoffPolls : polls;
    return LORA_OK;
}

int lora_bgmv(void *stream, void *y, int64_t ldy, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
              const lora_weights *w, float *v, int64_t ldv)
{
    const lora_proj p = one_proj(w, v, ldv, y, ldy);
    return lora_bgmv_multi(stream, x, ldx, idx, n_rows, 1, &p);
}

}  // extern "C"
