/*
 * Plain CPU reference of the multi-LoRA add-on path, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU baseline
 * leg of the benchmark may load this library.  The product path never calls it.
 * It shares no code, header or helper with the HIP library.
 *
 * What it computes (for every row i that has an adapter slot s with rank r_s > 0):
 *   v[i][j] = sum_k x[i][k] * A[s][k][j]                      j < r_s      (shrink)
 *   y[i][c] = y0[i][c] + scale[s] * sum_j v[i][j] * B[s][j][c]              (expand)
 * and y[i] = y0[i] for rows without an adapter.
 *
 * Sources (page title, section):
 *  - Punica summary, "The SGMV Operator: What It Computes": y = xW + xAB, factorised
 *    into v = xA (shrink) followed by y += vB (expand), applied per segment
 *    [s_{i-1}, s_i) of rows that share one adapter.
 *  - Punica digest, "5.4" (the add_lora SGMV semantics): rows of segment i use
 *    A stored transposed ([r][in]) and B stored [r][out].
 *  - Punica digest, "5.5" (BGMV): y[i] += x[i] A[idx[i]] B[idx[i]] * scale.
 *  - Multi-LoRA blog, "Why a mixed batch needs special kernels" (reference loop):
 *    per-slot scale alpha/r, rows with slot -1 are skipped.
 *  - S-LoRA summary, "Unified Paging": an adapter's A is held as r pages (its
 *    columns), B as r pages (its rows); pages live anywhere in one pool and are found
 *    through a page table.
 *
 * Storage read here (the same storage the GPU path reads):
 *  dense:  a_t[(s*r_max + j)*d_in + k] = A[s][k][j];   b[(s*r_max + j)*d_out + c] = B[s][j][c]
 *  paged:  A[s][k][j] = pool[page_table[a_pt_off[s] + j*(d_in/P) + k/P]*P + k%P]
 *          B[s][j][c] = pool[page_table[b_pt_off[s] + j*(d_out/P) + c/P]*P + c%P]
 * fp16 inputs are decoded bit by bit to their exact fp64 value; scale (fp32) is
 * promoted exactly.  Sums run in fp64 with k ascending, then j ascending.
 *
 * Planted mistakes for the pin tests: compiling with -DORACLE_MUTANT=<n> builds a
 * deliberately wrong variant (see mutant_* below) so a test can show that the pins
 * catch that kind of error.  The default build (no macro) is the oracle.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

typedef struct {
    int32_t layout; /* 0 = dense slot arrays, 1 = paged pool */
    int32_t num_slots, d_in, d_out, r_max;
    const int32_t *rank;   /* [num_slots] */
    const float *scale;    /* [num_slots] */
    const uint16_t *a_t;   /* dense: [num_slots][r_max][d_in]  fp16 bits */
    const uint16_t *b;     /* dense: [num_slots][r_max][d_out] fp16 bits */
    const uint16_t *pool;  /* paged: [num_pages][page_elems]   fp16 bits */
    int32_t page_elems;
    const int32_t *page_table;
    const int64_t *a_pt_off, *b_pt_off; /* [num_slots] */
} oracle_weights;

/* Exact value of an IEEE binary16 bit pattern. */
double oracle_half_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* (1024 + m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* A[s][k][j], i.e. element k of rank-row j of A^T[s]. */
static double a_elem(const oracle_weights *w, int s, int j, int k)
{
    if (w->layout == 0)
        return oracle_half_to_double(w->a_t[((size_t)s * w->r_max + j) * w->d_in + k]);
    {
        int64_t P = w->page_elems;
        int64_t entry = w->a_pt_off[s] + (int64_t)j * (w->d_in / P) + k / P;
        int64_t page = w->page_table[entry];
        return oracle_half_to_double(w->pool[page * P + k % P]);
    }
}

/* B[s][j][c]. */
static double b_elem(const oracle_weights *w, int s, int j, int c)
{
    if (w->layout == 0)
        return oracle_half_to_double(w->b[((size_t)s * w->r_max + j) * w->d_out + c]);
    {
        int64_t P = w->page_elems;
        int64_t entry = w->b_pt_off[s] + (int64_t)j * (w->d_out / P) + c / P;
        int64_t page = w->page_table[entry];
        return oracle_half_to_double(w->pool[page * P + c % P]);
    }
}

/*
 * One row of the add-on.  x_row: fp16 bits [d_in]; y0_row: fp16 bits [d_out];
 * y_row (out, fp64 [d_out]); v_row (out, fp64 [r_max], may be NULL).
 * Slot < 0 or rank 0: y_row = y0_row and v_row is left as it was.
 */
static void lora_row(const oracle_weights *w, int s, const uint16_t *x_row, const uint16_t *y0_row,
                     double *y_row, double *v_row)
{
    int d_in = w->d_in, d_out = w->d_out;
    int r = (s >= 0) ? w->rank[s] : 0;
    double v[64];
    int j, k, c;

    for (c = 0; c < d_out; ++c)
        y_row[c] = oracle_half_to_double(y0_row[c]);
    if (s < 0 || r <= 0)
        return;

    /* shrink: v_j = sum_k x_k A[k][j] */
    for (j = 0; j < r; ++j) {
        double acc = 0.0;
        for (k = 0; k < d_in; ++k) {
#if ORACLE_MUTANT == 1 /* transposed operand: reads A^T as if it were [d_in][r] */
            acc += oracle_half_to_double(x_row[k]) *
                   a_elem(w, s, (int)(((size_t)k * r + j) / d_in), (int)(((size_t)k * r + j) % d_in));
#elif ORACLE_MUTANT == 2 /* dropped term: skips the last input feature */
            if (k == d_in - 1) continue;
            acc += oracle_half_to_double(x_row[k]) * a_elem(w, s, j, k);
#else
            acc += oracle_half_to_double(x_row[k]) * a_elem(w, s, j, k);
#endif
        }
        v[j] = acc;
    }
    if (v_row) {
        for (j = 0; j < r; ++j)
            v_row[j] = v[j];
        for (j = r; j < w->r_max; ++j)
            v_row[j] = 0.0;
    }

    /* expand: y_c += scale * sum_j v_j B[j][c] */
    {
        double sc = (double)w->scale[s];
#if ORACLE_MUTANT == 3 /* wrong sign of the add-on */
        sc = -sc;
#elif ORACLE_MUTANT == 4 /* scale ignored, as in an SGMV with no scale */
        sc = 1.0;
#endif
        for (c = 0; c < d_out; ++c) {
            double acc = 0.0;
            for (j = 0; j < r; ++j) {
#if ORACLE_MUTANT == 5 /* wrong index: rank-row j read from the neighbouring slot */
                int s2 = (s + 1 < w->num_slots) ? s + 1 : s;
                acc += v[j] * b_elem(w, s2, j < w->rank[s2] ? j : 0, c);
#elif ORACLE_MUTANT == 6 /* off-by-one rank: last rank-row dropped */
                if (j == r - 1) continue;
                acc += v[j] * b_elem(w, s, j, c);
#else
                acc += v[j] * b_elem(w, s, j, c);
#endif
            }
            y_row[c] += sc * acc;
        }
    }
}

/*
 * Segment form (SGMV).  Segment g covers positions seg_ptr[g] .. seg_ptr[g+1]-1 and
 * uses slot seg_slot[g] (-1 = none).  A position p refers to row row_map[p], or to
 * row p when row_map is NULL.  Rows not covered by any segment keep y = y0.
 * y (out) fp64 [n][d_out]; v (out) fp64 [n][r_max] or NULL.
 */
int oracle_sgmv(const oracle_weights *w, int32_t n, const uint16_t *x, int64_t ldx,
                const uint16_t *y0, int64_t ldy, int32_t n_seg, const int32_t *seg_ptr,
                const int32_t *seg_slot, const int32_t *row_map, double *y, double *v,
                int32_t nthreads)
{
    int32_t i, g;
    (void)nthreads;
    for (i = 0; i < n; ++i) {
        int c;
        for (c = 0; c < w->d_out; ++c)
            y[(size_t)i * w->d_out + c] = oracle_half_to_double(y0[(size_t)i * ldy + c]);
    }
    for (g = 0; g < n_seg; ++g) {
        int32_t p0 = seg_ptr[g], p1 = seg_ptr[g + 1], p;
        int s = seg_slot[g];
#pragma omp parallel for num_threads(nthreads > 0 ? nthreads : 1) schedule(dynamic, 1) if (nthreads > 1)
        for (p = p0; p < p1; ++p) {
            int32_t row = row_map ? row_map[p] : p;
            lora_row(w, s, x + (size_t)row * ldx, y0 + (size_t)row * ldy, y + (size_t)row * w->d_out,
                     v ? v + (size_t)row * w->r_max : NULL);
        }
    }
    return 0;
}

/*
 * Per-row form (BGMV).  Row i uses slot idx[i]; idx[i] = -1 means no adapter.
 */
int oracle_bgmv(const oracle_weights *w, int32_t n, const uint16_t *x, int64_t ldx,
                const uint16_t *y0, int64_t ldy, const int32_t *idx, double *y, double *v,
                int32_t nthreads)
{
    int32_t i;
    (void)nthreads;
#pragma omp parallel for num_threads(nthreads > 0 ? nthreads : 1) schedule(dynamic, 1) if (nthreads > 1)
    for (i = 0; i < n; ++i)
        lora_row(w, idx[i], x + (size_t)i * ldx, y0 + (size_t)i * ldy, y + (size_t)i * w->d_out,
                 v ? v + (size_t)i * w->r_max : NULL);
    return 0;
}

int oracle_mutant_id(void) { return ORACLE_MUTANT; }
