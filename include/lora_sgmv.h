/*
 * lora_sgmv.h -- C ABI of the MI355X (gfx950) multi-LoRA add-on library.
 *
 * The operation (Punica summary, section 3.4 "The SGMV Operator: What It Computes";
 * Multi-LoRA Serving blog, "Why a mixed batch needs special kernels"):
 * every row i of a batch that carries an adapter slot s computes
 *
 *     shrink   v[i][j] = sum_k x[i][k] * A[s][k][j]                 (j < r_s, d_in -> r)
 *     expand   y[i][c] = y[i][c] + scale[s] * sum_j v[i][j] * B[s][j][c]   (r -> d_out)
 *
 * in place on the base output y.  Rows are given either as contiguous segments that
 * share one adapter (SGMV; Punica summary, "The SGMV Operator", segment offsets
 * s_0 = 0 < s_1 < ... < s_n) or with one slot per row (BGMV; Punica digest, section
 * 5.5, and the blog's reference loop, where slot -1 means "no adapter").  Each of
 * shrink and expand is one kernel launch whatever the adapter mix, including mixed
 * ranks and adapters held as scattered pages (S-LoRA summary, "Unified Paging" and
 * "Heterogeneous Batching").
 *
 * Conventions for every entry point:
 *  - Pointers documented "device" must point to GPU memory; "host" to CPU memory.
 *    All device pointers to fp16/fp32 data must be 16-byte aligned.
 *  - fp16 = IEEE binary16 (x, y, A, B); v and scale are fp32; slots, ranks and page
 *    ids are int32; page-table offsets are int64.  Matrices are row-major with the
 *    given leading dimension (in elements).
 *  - The caller owns every buffer.  The library never allocates or frees device memory,
 *    never synchronises, and keeps no state except a thread-local error message
 *    (and the thread-local diagnostics of lora_set_launch_events and lora_set_plan).
 *    Launching calls are asynchronous on `stream` (a hipStream_t; NULL = default).
 *    Inputs, outputs and metadata must stay alive until the work on `stream` ends.
 *  - Return value: LORA_OK (0) or a negative LORA_E_* code; lora_last_error() then
 *    describes the problem.  Argument checks run on the host before any launch, so
 *    a rejected call launches nothing.  Device-resident metadata (slots, ranks,
 *    row maps, page tables) is read by the kernels without a host check; an entry
 *    outside its documented range makes that tile or page a no-op instead of an
 *    out-of-bounds access.  lora_validate_*_host() check host copies fully.
 *  - An "active" row has slot s in [0, num_slots) with rank[s] > 0.  Rows that are
 *    not active keep y and v bit-identical.
 *
 * Numerics: fp16 products accumulate in fp32; v is stored in fp32; the expand adds
 * (scale[s] * v) . B to y in fp32 and rounds once to fp16 (round to nearest even).
 * Results are bit-identical from run to run for the same inputs (no float atomics);
 * different launch shapes may round differently within fp32 accumulation error.
 */
#ifndef LORA_SGMV_H
#define LORA_SGMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define LORA_OK 0
#define LORA_E_NULL (-1)        /* a required pointer is NULL */
#define LORA_E_SHAPE (-2)       /* a size or leading dimension is invalid */
#define LORA_E_ALIGN (-3)       /* a pointer or leading dimension is misaligned */
#define LORA_E_INDEX (-4)       /* a slot, row, tile or page index is out of range */
#define LORA_E_UNSUPPORTED (-5) /* valid request this library does not support (r_max > 64) */
#define LORA_E_HIP (-6)         /* the HIP runtime reported an error at launch */
#define LORA_E_CAPACITY (-7)    /* a host output array is too small */

#define LORA_LAYOUT_DENSE 0
#define LORA_LAYOUT_PAGED 1

#define LORA_MAX_RANK 64        /* largest r_max (the pages' ranks run from 8 to 64) */
#define LORA_MAX_TILE_ROWS 64   /* largest number of rows in one work tile */

/* ---------------------------------------------------------------- descriptors */
/*
 * One adapted projection (d_in -> d_out) of one layer, for all adapter slots.
 *
 * Dense layout (LORA_LAYOUT_DENSE): A is stored transposed, as rank-rows
 * (Punica digest, section 5.4, LoraWeight: A as [r][in], B as [r][out]):
 *     a_t[(s*r_max + j)*d_in  + k] = A[s][k][j]
 *     b  [(s*r_max + j)*d_out + c] = B[s][j][c]
 * Rank-rows j >= rank[s] are never read.
 *
 * Paged layout (LORA_LAYOUT_PAGED; S-LoRA summary, "Unified Paging": A is held as r
 * pages, one per column of A, and B as r pages, one per row of B, anywhere in one
 * pool).  Each rank-row is cut into d/P pages of P = page_elems elements:
 *     A[s][k][j] = pool[page_table[a_pt_off[s] + j*(d_in/P)  + k/P]*P + k%P]
 *     B[s][j][c] = pool[page_table[b_pt_off[s] + j*(d_out/P) + c/P]*P + c%P]
 * P must be a multiple of 8 that divides d_in and d_out.
 */
typedef struct lora_weights {
    int32_t layout;          /* LORA_LAYOUT_DENSE or LORA_LAYOUT_PAGED */
    int32_t num_slots;       /* number of adapter slots (>= 1) */
    int32_t d_in, d_out;     /* multiples of 8 */
    int32_t r_max;           /* 1..LORA_MAX_RANK; row stride of v must be >= r_max */
    const int32_t *rank;     /* device [num_slots], each in 0..r_max */
    const float *scale;      /* device [num_slots] (e.g. alpha / r) */
    const void *a_t;         /* dense: device fp16 [num_slots][r_max][d_in] */
    const void *b;           /* dense: device fp16 [num_slots][r_max][d_out] */
    const void *pool;        /* paged: device fp16 [num_pages][page_elems] */
    int64_t num_pages;       /* paged: pages in the pool */
    int32_t page_elems;      /* paged: P */
    const int32_t *page_table; /* paged: device [pt_entries], each in 0..num_pages-1 */
    int64_t pt_entries;      /* paged: length of page_table */
    const int64_t *a_pt_off; /* paged: device [num_slots] */
    const int64_t *b_pt_off; /* paged: device [num_slots] */
} lora_weights;

/* One work tile: `nrows` consecutive positions pos0.. of one segment, slot `slot`. */
typedef struct lora_tile {
    int32_t slot;   /* adapter slot of the segment (-1 = none) */
    int32_t pos0;   /* first position (index into row_map, or a row when row_map is NULL) */
    int32_t nrows;  /* 1..LORA_MAX_TILE_ROWS */
    int32_t seg;    /* segment the tile belongs to (informational) */
} lora_tile;

/*
 * Segment form of a batch (Punica summary, "The SGMV Operator": offsets
 * s_0 <= s_1 <= ... <= s_n, segment g = positions s_g .. s_{g+1}-1 sharing adapter
 * slot seg_slot[g]; Punica digest, section 5.4: the SGMV call takes these offsets and
 * the adapter index of each segment directly).
 *
 * Offsets form (tiles == NULL): the launch cuts every segment into
 * ceil(len / tile_rows) tiles of near-equal height itself, on the device -- each
 * workgroup finds its tile by a prefix sum over seg_ptr -- so nothing is built or
 * copied on the host and a captured graph can be replayed for a new batch written into
 * the same device arrays.  The cut equals lora_build_tiles' (same results, bit for
 * bit).  The grid covers n_rows / tile_rows + n_seg tiles, which bounds every valid
 * batch: segments may be empty, so a descriptor with a fixed capacity n_seg describes
 * every batch of at most n_seg segments.
 *   n_seg     number of segments (>= 0)
 *   seg_ptr   device int32 [n_seg + 1]: 0 <= seg_ptr[0] <= seg_ptr[1] <= ...; with
 *             row_map NULL the positions are rows, so seg_ptr[n_seg] <= n_rows; with a
 *             row map, row_map holds seg_ptr[n_seg] entries (distinct rows)
 *   seg_slot  device int32 [n_seg]: -1 = no adapter
 *   row_map   device int32 [seg_ptr[n_seg]] or NULL (position p is row p)
 *   tile_rows 1..LORA_MAX_TILE_ROWS, or 0 for the library's choice from n_rows and
 *             n_seg (64 when the segments average at least 128 rows, else 2)
 * The device arrays are read without a host check: an offset outside the positions
 * is clamped and an out-of-range slot or row makes its rows no-ops.
 *
 * Tile-list form (tiles != NULL), the precomputed fast path: the n_tiles tiles of
 * lora_build_tiles over the same segments (built once per batch on the host and
 * reused by every projection of every layer); seg_ptr, seg_slot and tile_rows are then
 * not read.  row_map as above, with n_pos = its length; max_rows = the largest nrows
 * of any tile (0 = unknown, taken as LORA_MAX_TILE_ROWS), a launch-shape hint only.
 */
typedef struct lora_segments {
    int32_t n_seg;
    const int32_t *seg_ptr;   /* device [n_seg + 1] */
    const int32_t *seg_slot;  /* device [n_seg] */
    const int32_t *row_map;   /* device, or NULL */
    int32_t tile_rows;        /* offsets form: tile height, 0 = library's choice */
    int32_t n_tiles;          /* tile-list form: number of tiles */
    const lora_tile *tiles;   /* tile-list form: device [n_tiles], 16-byte aligned; NULL = offsets form */
    int32_t n_pos;            /* tile-list form: number of positions (length of row_map) */
    int32_t max_rows;         /* tile-list form: largest nrows of any tile, 0 = unknown */
} lora_segments;

/*
 * Device workspace that the calls on a batch of n_rows rows in n_seg segments need, in
 * bytes, written to *bytes: the one-launch forms (lora_sgmv_multi_handoff,
 * lora_bgmv_multi_handoff) need lora_handoff_bytes(n_rows); the separate shrink and
 * expand launches need none (every split sum is combined inside one workgroup) and
 * take no workspace argument.  w may be NULL (the size does not depend on the
 * weights).  LORA_E_SHAPE for n_rows < 0 or n_seg < 0, LORA_E_NULL for bytes NULL.
 */
int lora_sgmv_workspace_bytes(const struct lora_weights *w, int32_t n_rows, int32_t n_seg, size_t *bytes);

/*
 * One adapted projection of a launch that serves several projections of the same
 * batch (e.g. q, k and v, which share their input x; or gate and up).
 */
typedef struct lora_proj {
    const lora_weights *w;   /* adapters of this projection */
    float *v;                /* device fp32 [n_rows][ldv], ldv >= w->r_max, ldv % 4 == 0 */
    int64_t ldv;
    void *y;                 /* expand: device fp16 [n_rows][ldy], ldy >= w->d_out, ldy % 8 == 0 */
    int64_t ldy;             /* (shrink ignores y and ldy) */
} lora_proj;

#define LORA_MAX_PROJ 4      /* projections one launch can serve */

/* ---------------------------------------------------------------- host metadata */
/*
 * Group rows by adapter (Punica summary, "Batch Layout Construction": rows that share
 * an adapter are placed consecutively and the segment offsets are built once per
 * batch, then reused by every adapted projection of every layer).
 *
 * idx      host [n]: slot of each row, -1 = no adapter.
 * row_map  host out [n]: positions -> original rows; segments in ascending slot order,
 *          rows of one segment in ascending original index; rows with -1 left out.
 * seg_ptr  host out [min(n, num_slots) + 1]: seg_ptr[0] = 0, strictly increasing.
 * seg_slot host out [min(n, num_slots)].
 * n_seg, n_act  host out: number of segments; active positions (= seg_ptr[n_seg]).
 * Returns LORA_E_INDEX if some idx is outside [-1, num_slots), LORA_E_SHAPE for
 * n < 0 or num_slots < 1, LORA_E_NULL for a missing pointer (arrays may be NULL
 * only when n == 0).  Deterministic; allocates no device memory.
 */
int lora_build_segments(const int32_t *idx, int32_t n, int32_t num_slots, int32_t *row_map,
                        int32_t *seg_ptr, int32_t *seg_slot, int32_t *n_seg, int32_t *n_act);

/* Capacity that lora_build_tiles needs for n_pos positions in n_seg segments. */
int32_t lora_tiles_bound(int32_t n_pos, int32_t n_seg, int32_t max_tile_rows);

/*
 * Tile height suited to a batch: 64 (four MFMA slices, fewest re-reads of each
 * adapter) when some segment has at least 128 rows, else 2 (short VALU tiles keep the
 * most wavefronts resident).
 * seg_ptr: host [n_seg + 1].  Any value in 1..LORA_MAX_TILE_ROWS gives the same
 * results within the stated tolerance; this only picks the faster launch shape.
 */
int32_t lora_pick_tile_rows(const int32_t *seg_ptr, int32_t n_seg);

/*
 * Tile height suited to the expand launches of a batch, whose tile list may differ
 * from the shrink's (the two are separate calls): lora_pick_tile_rows' height, except
 * 16 for batches of short segments whose 16-row tiles average at least 6 rows, one of
 * them at least 8 (tiles of 8 to 16 rows run an expand that reads each adapter's B
 * once per tile).
 * seg_ptr: host [n_seg + 1]; same tolerance statement as lora_pick_tile_rows.
 */
int32_t lora_pick_expand_tile_rows(const int32_t *seg_ptr, int32_t n_seg);

/*
 * Cut segments into the flat tile work-list the SGMV kernels run on.  Segment g
 * (positions seg_ptr[g] .. seg_ptr[g+1]-1, slot seg_slot[g]) becomes
 * ceil(len / max_tile_rows) tiles of near-equal size; empty segments and segments
 * with slot -1 produce no tile.  seg_ptr/seg_slot are host arrays (seg_ptr[0] may
 * be > 0; it must be non-decreasing).  tiles: host out [tiles_cap].
 * max_tile_rows in 1..LORA_MAX_TILE_ROWS.  Returns LORA_E_CAPACITY if tiles_cap is
 * too small (see lora_tiles_bound), LORA_E_SHAPE for decreasing offsets.
 */
int lora_build_tiles(const int32_t *seg_ptr, const int32_t *seg_slot, int32_t n_seg,
                     int32_t max_tile_rows, lora_tile *tiles, int32_t tiles_cap, int32_t *n_tiles);

/*
 * Host checks of host copies of a descriptor's device arrays.  `w` must hold host
 * pointers for rank (and, for paged layout, page_table, a_pt_off, b_pt_off); the
 * fp16 data pointers are not read.  Checks ranks against r_max, every page-table
 * range and page id, and the shape rules above.
 */
int lora_validate_weights_host(const lora_weights *w);

/* Host check of a host copy of a segment descriptor (all its arrays in host memory)
 * against n_rows and num_slots.  Tile-list form: tiles inside [0, n_pos),
 * 1..LORA_MAX_TILE_ROWS rows, slots in [-1, num_slots), no position in two tiles.
 * Offsets form: seg_ptr non-decreasing from seg_ptr[0] >= 0, seg_ptr[n_seg] <= n_rows,
 * seg_slot in [-1, num_slots), tile_rows in 0..LORA_MAX_TILE_ROWS.  Both forms: row_map
 * entries in [0, n_rows) and no row used twice. */
int lora_validate_segments_host(const lora_segments *seg, int32_t n_rows, int32_t num_slots);

/* ---------------------------------------------------------------- SGMV (segments) */
/*
 * Shrink for a segment batch (Punica summary, "The SGMV Operator"; Punica digest,
 * section 5.4, add_lora SGMV semantics).  For every active position p of every tile
 * with row = row_map ? row_map[p] : p:
 *     v[row*ldv + j] = sum_k x[row*ldx + k] * A[slot][k][j]   for j <  rank[slot]
 *     v[row*ldv + j] = 0                                      for rank[slot] <= j < r_max
 * v (device fp32 [n_rows][ldv], ldv >= r_max, ldv % 4 == 0) is overwritten there
 * and untouched elsewhere.  x: device fp16 [n_rows][ldx], ldx % 8 == 0, ldx >= d_in.
 * One launch; needs no workspace (partial sums are combined inside a workgroup).
 */
int lora_sgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx,
                     int32_t n_rows, const lora_weights *w, const lora_segments *seg);

/*
 * Expand for a segment batch: for every active position's row,
 *     y[row*ldy + c] = fp16( y[row*ldy + c] + scale[slot] * sum_{j<rank} v[row*ldv + j] * B[slot][j][c] )
 * y: device fp16 [n_rows][ldy] updated in place, ldy % 8 == 0, ldy >= d_out.
 * Reads only v[row][0:rank].  One launch; needs no workspace.
 */
int lora_sgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv,
                     int32_t n_rows, const lora_weights *w, const lora_segments *seg);

/* ---------------------------------------------------------------- BGMV (per-row slots) */
/*
 * Shrink with one slot per row (Punica digest, section 5.5, BGMV; blog reference
 * loop: slot -1 = no adapter).  idx: device int32 [n_rows].  Same v contract as
 * lora_sgmv_shrink with row = position.
 */
int lora_bgmv_shrink(void *stream, float *v, int64_t ldv, const void *x, int64_t ldx,
                     const int32_t *idx, int32_t n_rows, const lora_weights *w);

/* Expand with one slot per row; same y contract as lora_sgmv_expand. */
int lora_bgmv_expand(void *stream, void *y, int64_t ldy, const float *v, int64_t ldv,
                     const int32_t *idx, int32_t n_rows, const lora_weights *w);

/*
 * The whole add-on in decode form (Punica digest, section 5.5, BGMV; blog reference
 * loop): the result of lora_bgmv_shrink followed by lora_bgmv_expand, bit for bit.
 * v (device fp32 [n_rows][ldv]) receives the shrink result as documented above.
 * Same as lora_bgmv_multi with one projection.
 */
int lora_bgmv(void *stream, void *y, int64_t ldy, const void *x, int64_t ldx, const int32_t *idx,
              int32_t n_rows, const lora_weights *w, float *v, int64_t ldv);

/* ---------------------------------------------------------------- several projections per launch */
/*
 * The same operations for up to LORA_MAX_PROJ projections of one batch in one launch
 * each: every projection p gets exactly the result of the single-projection call
 * with (proj[p].w, proj[p].v, proj[p].y).  This cuts the launches of a transformer
 * layer from 14 to 8 (q/k/v and gate/up grouped) without changing the work.
 * All projections of one launch must use the same weight layout
 * (LORA_E_UNSUPPORTED otherwise); the shrink's projections share x, so they must
 * share d_in (LORA_E_SHAPE otherwise).  Output regions of different projections
 * must not overlap.  n_proj in 1..LORA_MAX_PROJ.
 */
int lora_sgmv_shrink_multi(void *stream, const void *x, int64_t ldx, int32_t n_rows,
                           const lora_segments *seg, int32_t n_proj, const lora_proj *proj);
int lora_sgmv_expand_multi(void *stream, int32_t n_rows, const lora_segments *seg, int32_t n_proj,
                           const lora_proj *proj);
int lora_bgmv_shrink_multi(void *stream, const void *x, int64_t ldx, const int32_t *idx,
                           int32_t n_rows, int32_t n_proj, const lora_proj *proj);
int lora_bgmv_expand_multi(void *stream, const int32_t *idx, int32_t n_rows, int32_t n_proj,
                           const lora_proj *proj);

/*
 * Shrink and expand of the decode form for up to LORA_MAX_PROJ projections sharing x:
 * lora_bgmv_shrink_multi followed by lora_bgmv_expand_multi (two launches), with the
 * arguments of both checked before either is launched.
 */
int lora_bgmv_multi(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                    int32_t n_proj, const lora_proj *proj);

/*
 * The same result as lora_bgmv_multi (bit for bit, v included) in ONE launch without
 * recomputation (Punica digest, section 5.5, BGMV; the kernel launches per layer are
 * what bounds a small decode batch): the launch's first workgroups run the shrink's
 * work items and hand each row's v to the workgroups running the expand's through
 * `work`, which poll for it while their loads of B and y are in flight.  An expand
 * workgroup that has not seen its v after a bounded number of polls computes it
 * itself, so the result does not depend on how the workgroups are scheduled.
 *   work:  caller-owned device memory of at least lora_handoff_bytes(n_rows) bytes,
 *          256-byte aligned, all zero before its first use (e.g. one hipMemset);
 *          every call leaves it all zero again when it completes.  Calls ordered on
 *          one stream (graph replays included) may share a workspace; calls that may
 *          run at the same time need their own.
 * Other arguments as for lora_bgmv_multi.  LORA_E_NULL for a NULL workspace,
 * LORA_E_ALIGN for a misaligned one, LORA_E_SHAPE when it is too small or a
 * projection's d_out exceeds 65535 * 512.  The per-row v contract is that of
 * lora_bgmv_shrink_multi; the one NaN bit pattern 0xFFFFFFFF is handed to the expand
 * as the canonical NaN (y is NaN either way).
 */
size_t lora_handoff_bytes(int32_t n_rows);   /* 0 for n_rows <= 0 */
int lora_bgmv_multi_handoff(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                            int32_t n_proj, const lora_proj *proj, void *work, size_t work_bytes);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): lora_bgmv_multi_handoff with the
 * hand-off workspace held by the library, a file-scope device array of
 * LORA_NOALLOC_MAX_ROWS rows (2 MiB) on each GPU, kept until the process ends.  Same
 * result, bit for bit.  No hipMalloc, hipFree or other allocation happens in the call.
 * The first call on a device looks up that device's copy of the array and clears it
 * with a small kernel on `stream` (recorded into the graph when `stream` is being
 * captured, where it then runs on every replay).  Every call on one GPU shares the array and leaves it all zero when
 * it completes, so calls ordered on one stream (graph replays included) may share it;
 * calls that may run at the same time on one GPU race and give wrong results.
 * LORA_E_SHAPE for n_rows > LORA_NOALLOC_MAX_ROWS (checked before anything else is done
 * on the GPU); other arguments and errors as for lora_bgmv_multi_handoff.
 */
#define LORA_NOALLOC_MAX_ROWS 1024
int lora_bgmv_multi_handoff_noalloc(void *stream, const void *x, int64_t ldx, const int32_t *idx, int32_t n_rows,
                                    int32_t n_proj, const lora_proj *proj);

/*
 * The segment form's counterpart (Punica summary, "The SGMV Operator"): the result of
 * lora_sgmv_shrink_multi followed by lora_sgmv_expand_multi, bit for bit, v included.
 * With dense weights and tiles of fewer than 8 rows (seg->max_rows, the tile heights
 * of decode batches) it is one launch that hands v over through `work` as above; with
 * taller tiles (the MFMA kernels) or paged weights it makes those two launches and
 * leaves `work` untouched.  `work` is checked (as above, for n_rows rows) either way.
 * Every row may appear in at most one tile, as lora_build_tiles makes them.  Other
 * arguments as for the two calls.
 */
int lora_sgmv_multi_handoff(void *stream, const void *x, int64_t ldx, int32_t n_rows, const lora_segments *seg,
                            int32_t n_proj, const lora_proj *proj, void *work, size_t work_bytes);

/* ---------------------------------------------------------------- adapter pool */
/*
 * Loading adapters into the paged layout (S-LoRA summary, "Unified Paging" and
 * "Adapter Loading, Prefetching, and Overlapping I/O with Computation"; Punica
 * summary, "On-Demand LoRA Weight Loading").  Pages all hold P fp16 elements, so
 * taking and returning them never fragments the pool, and an adapter's rank-rows may
 * sit in any free pages.
 *
 * Free-page list.  Its state lives in caller-owned host memory of
 * lora_pool_state_bytes(num_pages) bytes (the library keeps none).  lora_pool_alloc
 * hands out the pages of the most recent lora_pool_release first, in the order that
 * call listed them (a fresh list hands out 0, 1, 2, ...), so pages taken and returned
 * in runs of consecutive ids come back as the same runs.  Neither call is thread-safe
 * on one state.
 */
size_t lora_pool_state_bytes(int64_t num_pages);
int lora_pool_init(void *state, size_t state_bytes, int64_t num_pages);  /* num_pages in 1..2^31-1 */
/* n free page ids into pages[0..n); LORA_E_CAPACITY, taking none, if fewer are free. */
int lora_pool_alloc(void *state, int32_t n, int32_t *pages);
/* Returns n pages; LORA_E_INDEX, returning none, for an id out of range, not taken, or listed twice. */
int lora_pool_release(void *state, int32_t n, const int32_t *pages);
int64_t lora_pool_free_count(const void *state);   /* -1 for an uninitialised state */

/* Page-table entries (and pool pages) one adapter of rank r takes: r*(d_in + d_out)/P. */
int64_t lora_pool_pages_for(int32_t rank, int32_t d_in, int32_t d_out, int32_t page_elems);

/* One adapter to place into one projection's paged descriptor. */
typedef struct lora_load_job {
    const lora_weights *w;  /* host descriptor of the target (paged); its rank, scale, page_table,
                               a_pt_off and b_pt_off arrays receive the adapter */
    int32_t slot;           /* 0..num_slots-1 */
    int32_t rank;           /* 0..r_max; 0 unloads the slot (only rank[slot] is written) */
    float scale;            /* scale[slot] */
    int32_t reserved;       /* 0 */
    int64_t pt_off;         /* first of the adapter's page-table entries: A^T rank-rows
                               (rank*d_in/P entries, rank-row-major), then B (rank*d_out/P) */
    int64_t data_off;       /* byte offset in the blob of A^T [rank][d_in] followed by
                               B [rank][d_out], fp16; multiple of 16 */
    int64_t pages_off;      /* byte offset in the blob of the adapter's page ids (int32,
                               page-table order); multiple of 4 */
} lora_load_job;

/* Bytes at the start of a blob that lora_pool_load fills with its job table (a multiple of 16). */
size_t lora_pool_load_header_bytes(int32_t n_jobs);

/*
 * Places n_jobs adapters, in order on `stream`:
 *   1. writes the job table into blob[0 .. lora_pool_load_header_bytes(n_jobs));
 *   2. copies blob to staging (device, >= blob_bytes bytes, 16-byte aligned; it must not
 *      be reused before the load's kernel has finished) and the rank-rows into their
 *      pages (A^T rank-row j, page q <- elements q*P .. q*P+P-1), by one of two routes:
 *      - direct, when every page-id list lies before every job's rank-rows in the blob
 *        and the call's pages form at most 64 runs (consecutive pages of the blob to
 *        consecutive ids of one pool, across jobs too): blob[0 .. end of the last
 *        page-id list) goes to staging and each run host-to-device straight into its
 *        pool pages, by the copy engine;
 *      - staged, otherwise: all of blob goes to staging, and the kernel of step 3 also
 *        copies every page from there;
 *   3. one kernel writes page_table[pt_off + e] <- the page ids, and the slot's
 *      a_pt_off = pt_off, b_pt_off = pt_off + rank*d_in/P, rank and scale.
 * blob: host memory, 16-byte aligned, page-locked (hipHostMalloc) for the copy to be
 * asynchronous; it must stay unchanged until the copy has completed.  Every argument is
 * checked on the host before anything is issued, page ids included (read from the
 * blob): each in 0..num_pages-1 and no page named twice in the call; data and page-id
 * ranges inside the blob and after the header; page-table ranges inside pt_entries;
 * one job per (target, slot).  Pages are written in place, so a slot (and pages) being
 * loaded must not be read by work that can run at the same time: order it with an
 * event.  Page-table entries and pages of other slots are untouched.
 */
int lora_pool_load(void *stream, int32_t n_jobs, const lora_load_job *jobs, void *blob, size_t blob_bytes,
                   void *staging, size_t staging_bytes);

/* ---------------------------------------------------------------- diagnostics */
/*
 * Timing hook: attach two hipEvent_t (created by the caller; either may be NULL) to
 * the next kernel launch made by the calling thread (launched with
 * hipExtLaunchKernelGGL, which records `start_event` when the kernel starts and
 * `stop_event` when it ends, on the launch stream).  The pair is consumed by that
 * one launch; where a call makes two launches, it is the first.  Returns LORA_OK.
 */
int lora_set_launch_events(void *start_event, void *stop_event);

/*
 * Tuning hook: for the calling thread's later launches, fixes the number of rank-rows
 * each VALU shrink workgroup computes (1..64) and the number of rows each pass of the
 * segment-form VALU kernels takes (1, 2 or 4); 0 restores the library's choice.
 * Results do not depend on either, bit for bit: every element is summed in the same
 * order whatever the split.  Returns LORA_E_SHAPE for other values.  Per-thread
 * state, like the event pair.
 */
int lora_set_plan(int32_t shrink_rank_rows, int32_t rows_per_pass);

/*
 * Caller hint for the per-row calls (lora_bgmv_shrink/expand and their _multi and
 * _handoff forms) with dense weights: on = 1 when every active row of the calling
 * thread's later calls uses an adapter that no other row of the same call uses (a decode
 * batch whose requests all carry different adapters; Punica summary, the "Distinct" case
 * of the SGMV kernel schedule).  The kernels then read the A^T and B rows with streaming
 * (non-temporal) loads: each is read once, and keeping it in the caches only displaces
 * the rest (7B decode, 32 distinct adapters, one launch per unit: 35.8 -> 34.7 us per
 * layer).  With adapters shared between rows it is slower (13B Zipf 1.5 mix in the
 * per-row form: 81.5 -> 103.4), hence off (0) by default.  The segment form and paged
 * weights ignore it.  Results are bit-identical either way.  Returns LORA_E_SHAPE for
 * values other than 0 and 1.  Per-thread state, like lora_set_plan.
 */
int lora_set_stream_weights(int32_t on);

/*
 * Test hook: the number of polls an expand workgroup of lora_bgmv_multi_handoff makes
 * for its v before computing v itself, for the calling thread's later calls (0: every
 * expand workgroup computes its v; a negative value restores the default, about 30 ms
 * of polling).  Results are the same bits whatever the value.  Returns LORA_OK.
 */
int lora_set_handoff_polls(int32_t polls);

const char *lora_last_error(void);   /* message of this thread's last failed call */
const char *lora_status_str(int status);
int lora_abi_version(void);          /* 2 */

#ifdef __cplusplus
}
#endif
#endif /* LORA_SGMV_H */
