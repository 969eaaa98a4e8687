/*
 * Plain CPU oracle for the head logits -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header or constant with the GPU
 * library and must never be used as a fallback for it.
 *
 * What it computes (SemBridge paper, section 5.2 "Data, Result, and Control
 * Paths": the tail output head materialises the full logits, and both the
 * full-logit plan and source projection start from that same tensor):
 *
 *     z[b][v] = sum_{h = 0 .. H-1} x[b][h] * w[h][v]
 *
 * with x and w given as bfloat16 bit patterns.  Every bf16 value is decoded
 * exactly to double (a bf16 pattern is the upper 16 bits of the float32 with
 * the same value), every product of two bf16 values is exact in double (two
 * 8-bit significands give at most 16 bits), and the sum is taken in double in
 * ascending h for every (b, v).
 *
 * The loop nest walks columns in blocks only so that each weight row segment
 * is read once from memory; that changes which (b, v) sums advance together,
 * never the order of the terms inside any one sum.  Identical weight columns
 * therefore give bit-identical logits, which the tie tests rely on.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -o liboracle.so
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Exact bf16 -> double: place the 16 bits in the top half of a float32. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

#define COL_BLOCK 512

/*
 * z[r][v] for the selected rows r = 0..nrows-1 (row index rows[r] of x, or r
 * itself when rows is NULL) and all columns v = 0..V-1.
 *   x   : bf16 bits, row-major, leading dimension ldx (elements)
 *   w   : bf16 bits, row-major [H][V], leading dimension ldw (elements)
 *   z   : double, row-major [nrows][V], leading dimension V
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int oracle_logits(const uint16_t *x, int64_t ldx, const int32_t *rows, int nrows,
                  const uint16_t *w, int64_t ldw, int H, int V,
                  double *z, int nthreads)
{
    if (!x || !w || !z || nrows < 0 || H < 0 || V < 0 || ldx < H || ldw < V)
        return -1;
    if (nrows == 0 || V == 0)
        return 0;

    /* Decode the selected hidden rows once: xd[r][h]. */
    double *xd = (double *)malloc(sizeof(double) * (size_t)nrows * (size_t)(H > 0 ? H : 1));
    if (!xd)
        return -1;
    for (int r = 0; r < nrows; ++r) {
        int64_t src = rows ? rows[r] : r;
        for (int h = 0; h < H; ++h)
            xd[(size_t)r * H + h] = bf16_to_double(x[src * ldx + h]);
    }

    int nblocks = (V + COL_BLOCK - 1) / COL_BLOCK;
    int status = 0;
    if (nthreads > 0)
        omp_set_num_threads(nthreads);

#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)nrows * COL_BLOCK);
        double *wd = (double *)malloc(sizeof(double) * COL_BLOCK);
        if (!acc || !wd) {
#pragma omp atomic write
            status = -1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int blk = 0; blk < nblocks; ++blk) {
            if (!acc || !wd)
                continue;
            int v0 = blk * COL_BLOCK;
            int nv = V - v0 < COL_BLOCK ? V - v0 : COL_BLOCK;
            for (size_t i = 0; i < (size_t)nrows * COL_BLOCK; ++i)
                acc[i] = 0.0;
            /* Ascending h: term h is added to every sum of this block before
             * term h+1 is added to any of them. */
            for (int h = 0; h < H; ++h) {
                const uint16_t *wrow = w + (int64_t)h * ldw + v0;
                for (int j = 0; j < nv; ++j)
                    wd[j] = bf16_to_double(wrow[j]);
                for (int r = 0; r < nrows; ++r) {
                    double xv = xd[(size_t)r * H + h];
                    double *a = acc + (size_t)r * COL_BLOCK;
                    for (int j = 0; j < nv; ++j)
                        a[j] = a[j] + xv * wd[j];
                }
            }
            for (int r = 0; r < nrows; ++r)
                memcpy(z + (size_t)r * V + v0, acc + (size_t)r * COL_BLOCK,
                       sizeof(double) * (size_t)nv);
        }
        free(acc);
        free(wd);
    }
    free(xd);
    return status;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int oracle_max_threads(void)
{
    return omp_get_max_threads();
}
