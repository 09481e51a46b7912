// Host side of the library: batch metadata (segments and the tile work-list),
// descriptor validation and error reporting.  No HIP calls here.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "lora_internal.hpp"

namespace lora {

static thread_local char g_error[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_error[0] = '\0'; }

int32_t lora_tile_rows_for(int32_t n_rows, int32_t n_seg)
{
    return n_seg > 0 && (int64_t)n_rows >= (int64_t)kLongSegment * n_seg ? LORA_MAX_TILE_ROWS : 2;
}

int check_weights_desc(const lora_weights *w)
{
    if (!w) return fail(LORA_E_NULL, "weights descriptor is NULL");
    if (w->layout != LORA_LAYOUT_DENSE && w->layout != LORA_LAYOUT_PAGED)
        return fail(LORA_E_SHAPE, "unknown layout %d", w->layout);
    if (w->num_slots < 1) return fail(LORA_E_SHAPE, "num_slots = %d (must be >= 1)", w->num_slots);
    if (w->d_in <= 0 || w->d_out <= 0 || w->d_in % 8 || w->d_out % 8)
        return fail(LORA_E_SHAPE, "d_in = %d, d_out = %d (must be positive multiples of 8)", w->d_in,
                    w->d_out);
    if (w->r_max < 1) return fail(LORA_E_SHAPE, "r_max = %d (must be >= 1)", w->r_max);
    if (w->r_max > LORA_MAX_RANK)
        return fail(LORA_E_UNSUPPORTED, "r_max = %d exceeds the supported maximum %d", w->r_max,
                    LORA_MAX_RANK);
    if (!w->rank || !w->scale) return fail(LORA_E_NULL, "rank or scale pointer is NULL");
    if (w->layout == LORA_LAYOUT_DENSE) {
        if (!w->a_t || !w->b) return fail(LORA_E_NULL, "dense layout needs a_t and b");
        if (!aligned16(w->a_t) || !aligned16(w->b))
            return fail(LORA_E_ALIGN, "a_t and b must be 16-byte aligned");
    } else {
        if (!w->pool || !w->page_table || !w->a_pt_off || !w->b_pt_off)
            return fail(LORA_E_NULL, "paged layout needs pool, page_table, a_pt_off and b_pt_off");
        if (!aligned16(w->pool)) return fail(LORA_E_ALIGN, "pool must be 16-byte aligned");
        const int32_t P = w->page_elems;
        if (P < 8 || P % 8 || w->d_in % P || w->d_out % P)
            return fail(LORA_E_SHAPE, "page_elems = %d must be a multiple of 8 dividing d_in = %d and d_out = %d",
                        P, w->d_in, w->d_out);
        if (w->num_pages < 1 || w->pt_entries < 1)
            return fail(LORA_E_SHAPE, "num_pages = %lld, pt_entries = %lld (must be >= 1)",
                        (long long)w->num_pages, (long long)w->pt_entries);
    }
    return LORA_OK;
}

}  // namespace lora

using namespace lora;

extern "C" {

const char *lora_last_error(void) { return g_error; }

const char *lora_status_str(int status)
{
    switch (status) {
    case LORA_OK: return "ok";
    case LORA_E_NULL: return "null pointer";
    case LORA_E_SHAPE: return "invalid shape";
    case LORA_E_ALIGN: return "misaligned pointer or leading dimension";
    case LORA_E_INDEX: return "index out of range";
    case LORA_E_UNSUPPORTED: return "unsupported";
    case LORA_E_HIP: return "HIP runtime error";
    case LORA_E_CAPACITY: return "output capacity too small";
    default: return "unknown status";
    }
}

int lora_abi_version(void) { return 2; }

int lora_build_segments(const int32_t *idx, int32_t n, int32_t num_slots, int32_t *row_map,
                        int32_t *seg_ptr, int32_t *seg_slot, int32_t *n_seg, int32_t *n_act)
{
    clear_error();
    if (n < 0 || num_slots < 1) return fail(LORA_E_SHAPE, "n = %d, num_slots = %d", n, num_slots);
    if (!n_seg || !n_act || !seg_ptr) return fail(LORA_E_NULL, "n_seg, n_act and seg_ptr are required");
    if (n > 0 && (!idx || !row_map || !seg_slot)) return fail(LORA_E_NULL, "idx, row_map and seg_slot are required");
    for (int32_t i = 0; i < n; ++i)
        if (idx[i] < -1 || idx[i] >= num_slots)
            return fail(LORA_E_INDEX, "idx[%d] = %d outside [-1, %d)", i, idx[i], num_slots);
    // Stable counting sort of the active rows by slot.
    std::vector<int32_t> start((size_t)num_slots + 1, 0);
    for (int32_t i = 0; i < n; ++i)
        if (idx[i] >= 0) ++start[(size_t)idx[i] + 1];
    for (int32_t s = 0; s < num_slots; ++s) start[(size_t)s + 1] += start[(size_t)s];
    std::vector<int32_t> fillpos(start.begin(), start.end() - 1);
    for (int32_t i = 0; i < n; ++i)
        if (idx[i] >= 0) row_map[fillpos[(size_t)idx[i]]++] = i;
    int32_t g = 0;
    seg_ptr[0] = 0;
    for (int32_t s = 0; s < num_slots; ++s) {
        if (start[(size_t)s + 1] > start[(size_t)s]) {
            seg_slot[g] = s;
            seg_ptr[g + 1] = start[(size_t)s + 1];
            ++g;
        }
    }
    *n_seg = g;
    *n_act = start[(size_t)num_slots];
    return LORA_OK;
}

int32_t lora_tiles_bound(int32_t n_pos, int32_t n_seg, int32_t max_tile_rows)
{
    if (n_pos < 0 || n_seg < 0 || max_tile_rows < 1) return 0;
    return (n_pos + max_tile_rows - 1) / max_tile_rows + n_seg;
}

int32_t lora_pick_tile_rows(const int32_t *seg_ptr, int32_t n_seg)
{
    int32_t longest = 0;
    for (int32_t g = 0; seg_ptr && g < n_seg; ++g) longest = std::max(longest, seg_ptr[g + 1] - seg_ptr[g]);
    // Long segments (prefill) feed the MFMA kernels 64-row tiles, which re-read each
    // adapter's A and B least; short ones (decode groups) run on the VALU kernels in
    // 2-row tiles.  Measured on MI355X, 2-row tiles are as fast as 4-row ones or faster
    // for every decode mix once the expand runs a tile in one pass (13B uniform 86 vs 92,
    // skewed 77 vs 79, identical 69 vs 69 us per layer; a 256-row batch over a
    // 2000-adapter 70B pool 426 vs 452), since shorter passes keep more wavefronts resident.
    return longest >= kLongSegment ? LORA_MAX_TILE_ROWS : 2;
}

int32_t lora_pick_expand_tile_rows(const int32_t *seg_ptr, int32_t n_seg)
{
    const int32_t base = lora_pick_tile_rows(seg_ptr, n_seg);
    if (base > 16 || !seg_ptr) return base;
    // Decode batches: 16-row tiles take the expand that reads each adapter's B once per
    // tile instead of once per 2 rows.  That pays where the tiles are well filled;
    // measured on MI355X (us per layer, expand tiles of 16 vs 2 rows): 13B identical mix
    // (one 58-row segment) 58.5 vs 68.9, skewed (30/11/9/5/1/1/1 rows) 69.4 vs 77.5; a
    // 256-row batch over 98 adapters of a 2000-adapter 70B pool (most with 1-2 rows) 430
    // vs 358.  So: 16 when the segments' 16-row tiles average at least 6 rows and the
    // tallest reaches 8 (tiles of 8 to 16 rows take that expand).
    int64_t rows = 0, tiles = 0, longest = 0;
    for (int32_t g = 0; g < n_seg; ++g) {
        const int64_t len = (int64_t)seg_ptr[g + 1] - seg_ptr[g];
        if (len <= 0) continue;
        rows += len;
        tiles += (len + 15) / 16;
        longest = std::max(longest, len);
    }
    return tiles > 0 && rows >= 6 * tiles && longest >= kMfmaMinRows ? 16 : base;
}

int lora_build_tiles(const int32_t *seg_ptr, const int32_t *seg_slot, int32_t n_seg,
                     int32_t max_tile_rows, lora_tile *tiles, int32_t tiles_cap, int32_t *n_tiles)
{
    clear_error();
    if (!n_tiles) return fail(LORA_E_NULL, "n_tiles is required");
    *n_tiles = 0;
    if (n_seg < 0) return fail(LORA_E_SHAPE, "n_seg = %d", n_seg);
    if (max_tile_rows < 1 || max_tile_rows > LORA_MAX_TILE_ROWS)
        return fail(LORA_E_SHAPE, "max_tile_rows = %d outside 1..%d", max_tile_rows, LORA_MAX_TILE_ROWS);
    if (n_seg == 0) return LORA_OK;
    if (!seg_ptr || !seg_slot) return fail(LORA_E_NULL, "seg_ptr and seg_slot are required");
    if (seg_ptr[0] < 0) return fail(LORA_E_SHAPE, "seg_ptr[0] = %d is negative", seg_ptr[0]);
    int32_t t = 0;
    for (int32_t g = 0; g < n_seg; ++g) {
        const int32_t p0 = seg_ptr[g], p1 = seg_ptr[g + 1];
        if (p1 < p0) return fail(LORA_E_SHAPE, "seg_ptr decreases at segment %d (%d > %d)", g, p0, p1);
        const int32_t len = p1 - p0;
        if (len == 0 || seg_slot[g] < 0) continue;
        const int32_t nt = (len + max_tile_rows - 1) / max_tile_rows;
        const int32_t base = len / nt, rem = len % nt;
        int32_t p = p0;
        for (int32_t q = 0; q < nt; ++q) {
            const int32_t rows = base + (q < rem ? 1 : 0);
            if (t >= tiles_cap) return fail(LORA_E_CAPACITY, "tiles_cap = %d is too small", tiles_cap);
            if (!tiles) return fail(LORA_E_NULL, "tiles is NULL");
            tiles[t] = lora_tile{seg_slot[g], p, rows, g};
            p += rows;
            ++t;
        }
    }
    *n_tiles = t;
    return LORA_OK;
}

int lora_validate_weights_host(const lora_weights *w)
{
    clear_error();
    int st = check_weights_desc(w);
    if (st) return st;
    for (int32_t s = 0; s < w->num_slots; ++s)
        if (w->rank[s] < 0 || w->rank[s] > w->r_max)
            return fail(LORA_E_SHAPE, "rank[%d] = %d outside 0..r_max = %d", s, w->rank[s], w->r_max);
    if (w->layout == LORA_LAYOUT_PAGED) {
        const int64_t P = w->page_elems, pa = w->d_in / P, pb = w->d_out / P;
        for (int32_t s = 0; s < w->num_slots; ++s) {
            const int64_t r = w->rank[s];
            if (r == 0) continue;
            const int64_t spans[2][2] = {{w->a_pt_off[s], r * pa}, {w->b_pt_off[s], r * pb}};
            for (auto &sp : spans) {
                if (sp[0] < 0 || sp[0] + sp[1] > w->pt_entries)
                    return fail(LORA_E_INDEX, "slot %d: page-table range [%lld, %lld) outside [0, %lld)", s,
                                (long long)sp[0], (long long)(sp[0] + sp[1]), (long long)w->pt_entries);
                for (int64_t e = sp[0]; e < sp[0] + sp[1]; ++e)
                    if (w->page_table[e] < 0 || w->page_table[e] >= w->num_pages)
                        return fail(LORA_E_INDEX, "page_table[%lld] = %d outside [0, %lld)", (long long)e,
                                    w->page_table[e], (long long)w->num_pages);
            }
        }
    }
    return LORA_OK;
}

// Rows of the row map used by positions [p0, p1): each in [0, n_rows) and at most once.
static int check_row_map(const int32_t *row_map, int32_t p0, int32_t p1, int32_t n_rows)
{
    std::vector<uint8_t> seen((size_t)std::max(n_rows, 0), 0);
    for (int32_t p = p0; p < p1; ++p) {
        const int32_t r = row_map[p];
        if (r < 0 || r >= n_rows) return fail(LORA_E_INDEX, "row_map[%d] = %d outside [0, %d)", p, r, n_rows);
        if (seen[(size_t)r]) return fail(LORA_E_INDEX, "row %d appears twice in row_map", r);
        seen[(size_t)r] = 1;
    }
    return LORA_OK;
}

int lora_validate_segments_host(const lora_segments *seg, int32_t n_rows, int32_t num_slots)
{
    clear_error();
    if (!seg) return fail(LORA_E_NULL, "segments descriptor is NULL");
    if (n_rows < 0) return fail(LORA_E_SHAPE, "n_rows = %d", n_rows);
    if (!seg->tiles) {
        // offsets form
        if (seg->n_seg < 0) return fail(LORA_E_SHAPE, "n_seg = %d", seg->n_seg);
        if (seg->tile_rows < 0 || seg->tile_rows > LORA_MAX_TILE_ROWS)
            return fail(LORA_E_SHAPE, "tile_rows = %d outside 0..%d", seg->tile_rows, LORA_MAX_TILE_ROWS);
        if (seg->n_tiles != 0) return fail(LORA_E_NULL, "n_tiles = %d without a tile list", seg->n_tiles);
        if (seg->n_seg == 0) return LORA_OK;
        if (!seg->seg_ptr || !seg->seg_slot) return fail(LORA_E_NULL, "seg_ptr and seg_slot are required");
        if (seg->seg_ptr[0] < 0) return fail(LORA_E_SHAPE, "seg_ptr[0] = %d is negative", seg->seg_ptr[0]);
        for (int32_t g = 0; g < seg->n_seg; ++g) {
            if (seg->seg_ptr[g + 1] < seg->seg_ptr[g])
                return fail(LORA_E_SHAPE, "seg_ptr decreases at segment %d (%d > %d)", g, seg->seg_ptr[g],
                            seg->seg_ptr[g + 1]);
            if (seg->seg_slot[g] < -1 || seg->seg_slot[g] >= num_slots)
                return fail(LORA_E_INDEX, "seg_slot[%d] = %d outside [-1, %d)", g, seg->seg_slot[g], num_slots);
        }
        const int32_t end = seg->seg_ptr[seg->n_seg];
        if (end > n_rows)
            return fail(LORA_E_INDEX, "seg_ptr[n_seg] = %d exceeds the %d rows (positions are rows or row-map entries)",
                        end, n_rows);
        return seg->row_map ? check_row_map(seg->row_map, seg->seg_ptr[0], end, n_rows) : LORA_OK;
    }
    // tile-list form
    if (seg->n_tiles < 0 || seg->n_pos < 0 || seg->max_rows < 0 || seg->max_rows > LORA_MAX_TILE_ROWS)
        return fail(LORA_E_SHAPE, "n_tiles = %d, n_pos = %d, n_rows = %d, max_rows = %d", seg->n_tiles, seg->n_pos,
                    n_rows, seg->max_rows);
    const int32_t n_pos = seg->row_map ? seg->n_pos : n_rows;
    std::vector<uint8_t> used((size_t)std::max(n_pos, 0), 0);
    for (int32_t t = 0; t < seg->n_tiles; ++t) {
        const lora_tile &tl = seg->tiles[t];
        if (tl.slot < -1 || tl.slot >= num_slots)
            return fail(LORA_E_INDEX, "tile %d: slot %d outside [-1, %d)", t, tl.slot, num_slots);
        if (tl.nrows < 1 || tl.nrows > LORA_MAX_TILE_ROWS)
            return fail(LORA_E_SHAPE, "tile %d: %d rows", t, tl.nrows);
        if (tl.pos0 < 0 || (int64_t)tl.pos0 + tl.nrows > n_pos)
            return fail(LORA_E_INDEX, "tile %d: positions [%d, %d) outside [0, %d)", t, tl.pos0,
                        tl.pos0 + tl.nrows, n_pos);
        for (int32_t p = tl.pos0; p < tl.pos0 + tl.nrows; ++p) {
            if (used[(size_t)p]) return fail(LORA_E_INDEX, "position %d is in two tiles", p);
            used[(size_t)p] = 1;
        }
    }
    return seg->row_map ? check_row_map(seg->row_map, 0, n_pos, n_rows) : LORA_OK;
}

int lora_sgmv_workspace_bytes(const lora_weights *w, int32_t n_rows, int32_t n_seg, size_t *bytes)
{
    clear_error();
    (void)w;
    if (!bytes) return fail(LORA_E_NULL, "bytes is NULL");
    *bytes = 0;
    if (n_rows < 0 || n_seg < 0) return fail(LORA_E_SHAPE, "n_rows = %d, n_seg = %d", n_rows, n_seg);
    *bytes = lora_handoff_bytes(n_rows);
    return LORA_OK;
}

}  // extern "C"
