/*
 * tt_oracle.c -- plain, slow CPU oracle for the TT-EmbeddingBag hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header
 * or table with the GPU library and must never be used by it.
 *
 * Everything is computed in fp64 from fp32 inputs widened exactly; the build
 * uses -ffp-contract=off so every multiply and add rounds on its own.
 *
 * What is computed (sources are the pages this project follows):
 *  - "FlowTT: Exploiting Computation Flow Reuse in Irregular Tensor-Train
 *    Embedding" (paperlayer summary), sections 2.4 and 3.3: a row index is a
 *    mixed-radix number whose early (high-order) digits select the leading TT
 *    cores; rows that share those digits share the prefix intermediate.
 *  - same page, section 3.2: the forward contracts C = A.B (first two cores),
 *    then E = C.D (third core), then pools; the backward reverses it.
 *  - same page, section 4 (latency breakdown): grouping is index sorting,
 *    unique extraction, mixed-radix conversion, prefix extraction and
 *    run-length encoding, in that order.
 *  - "TT-Rec: Tensor Train Compression for Deep Learning Recommendation
 *    Models" (abstract): the operator is an EmbeddingBag over rows rebuilt
 *    from TT cores.
 *
 * Readings where the pages are silent (kept identical in the GPU library's
 * documentation):
 *  - digits are big-endian: i = (i1*n2 + i2)*n3 + i3, prefix = (i1, i2);
 *  - core k is stored row-major as [n_k][R_{k-1}][d_k][R_k], R_0 = R_3 = 1;
 *  - output column j = (j1*d2 + j2)*d3 + j3;
 *  - pooling is a sum; an empty bag pools to 0;
 *  - offsets are table-major CSR with T*B+1 entries; bag (t,b) is
 *    indices[offsets[t*B+b] .. offsets[t*B+b+1]);
 *  - the output is [B][sum_t D_t], tables concatenated in order;
 *  - grouping sorts lookups by (table, row, position) -- a stable sort by row
 *    within each table.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_INDEX (-2)
#define ORC_ERR_NOMEM (-6)

/* ---------------------------------------------------------------- decode */

/* Mixed-radix split of a row index into its three TT-core digits
 * (FlowTT summary, sections 2.4 and 3.3: shared high-order digits). */
static void decode3(int64_t i, const int32_t *n, int64_t *i1, int64_t *i2, int64_t *i3)
{
    *i3 = i % n[2];
    int64_t q = i / n[2];
    *i2 = q % n[1];
    *i1 = q / n[1];
}

int orc_decode(int64_t i, const int32_t *n, int64_t *out3)
{
    if (i < 0 || n[0] <= 0 || n[1] <= 0 || n[2] <= 0) return ORC_ERR_ARG;
    decode3(i, n, &out3[0], &out3[1], &out3[2]);
    return ORC_OK;
}

/* ------------------------------------------------------------ contraction */

/* Prefix intermediate C = A.B of FlowTT section 3.2:
 *   C[j1][j2][r2] = sum_{r1} G1[i1][0][j1][r1] * G2[i2][r1][j2][r2],
 * r1 ascending.  C is stored [d1*d2][R2]. */
static void prefix_c(const float *G1, const float *G2, const int32_t *d, const int32_t *R,
                     int64_t i1, int64_t i2, double *C)
{
    const int d1 = d[0], d2 = d[1], R1 = R[1], R2 = R[2];
    const float *g1 = G1 + i1 * (int64_t)d1 * R1;
    const float *g2 = G2 + i2 * (int64_t)R1 * d2 * R2;
    for (int j1 = 0; j1 < d1; ++j1)
        for (int j2 = 0; j2 < d2; ++j2)
            for (int r2 = 0; r2 < R2; ++r2) {
                double acc = 0.0;
                for (int r1 = 0; r1 < R1; ++r1)
                    acc += (double)g1[j1 * R1 + r1] * (double)g2[((int64_t)r1 * d2 + j2) * R2 + r2];
                C[(j1 * d2 + j2) * R2 + r2] = acc;
            }
}

/* Row E = C.D of FlowTT section 3.2:
 *   E[(j1*d2+j2)*d3 + j3] = sum_{r2} C[j1 j2][r2] * G3[i3][r2][j3][0],
 * r2 ascending. */
static void suffix_e(const double *C, const float *G3, const int32_t *d, const int32_t *R,
                     int64_t i3, double *E)
{
    const int d12 = d[0] * d[1], d3 = d[2], R2 = R[2];
    const float *g3 = G3 + i3 * (int64_t)R2 * d3;
    for (int m = 0; m < d12; ++m)
        for (int j3 = 0; j3 < d3; ++j3) {
            double acc = 0.0;
            for (int r2 = 0; r2 < R2; ++r2)
                acc += C[m * R2 + r2] * (double)g3[r2 * d3 + j3];
            E[m * d3 + j3] = acc;
        }
}

/* One embedding row rebuilt from the cores, with no reuse (TT-Rec abstract:
 * rows are reconstructed from TT cores; FlowTT 3.2 gives the order). */
int orc_row(const float *G1, const float *G2, const float *G3, const int32_t *n,
            const int32_t *d, const int32_t *R, int64_t i, double *E)
{
    int64_t i1, i2, i3;
    if (i < 0) return ORC_ERR_INDEX;
    decode3(i, n, &i1, &i2, &i3);
    if (i1 >= n[0]) return ORC_ERR_INDEX;
    double *C = (double *)malloc(sizeof(double) * (size_t)d[0] * d[1] * R[2]);
    if (!C) return ORC_ERR_NOMEM;
    prefix_c(G1, G2, d, R, i1, i2, C);
    suffix_e(C, G3, d, R, i3, E);
    free(C);
    return ORC_OK;
}

/* ------------------------------------------------------------- checking */

static int check_tables(int32_t T, const int64_t *N, const int32_t *n, const int32_t *d,
                        const int32_t *R)
{
    if (T <= 0) return ORC_ERR_ARG;
    for (int t = 0; t < T; ++t) {
        const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
        if (N[t] <= 0) return ORC_ERR_ARG;
        for (int k = 0; k < 3; ++k)
            if (nt[k] <= 0 || dt[k] <= 0) return ORC_ERR_ARG;
        if (Rt[0] != 1 || Rt[3] != 1 || Rt[1] <= 0 || Rt[2] <= 0) return ORC_ERR_ARG;
        if ((int64_t)nt[0] * nt[1] * nt[2] < N[t]) return ORC_ERR_ARG;
    }
    return ORC_OK;
}

static int check_csr(int32_t T, const int64_t *N, const int64_t *indices, const int64_t *offsets,
                     int64_t B, int64_t nnz)
{
    if (B < 0 || nnz < 0) return ORC_ERR_ARG;
    if (offsets[0] != 0 || offsets[(int64_t)T * B] != nnz) return ORC_ERR_ARG;
    for (int64_t k = 0; k < (int64_t)T * B; ++k)
        if (offsets[k + 1] < offsets[k]) return ORC_ERR_ARG;
    for (int t = 0; t < T; ++t)
        for (int64_t l = offsets[(int64_t)t * B]; l < offsets[(int64_t)(t + 1) * B]; ++l)
            if (indices[l] < 0 || indices[l] >= N[t]) return ORC_ERR_INDEX;
    return ORC_OK;
}

static int64_t sum_dims(int32_t T, const int32_t *d, int64_t *col_off)
{
    int64_t s = 0;
    for (int t = 0; t < T; ++t) {
        col_off[t] = s;
        s += (int64_t)d[3 * t] * d[3 * t + 1] * d[3 * t + 2];
    }
    return s;
}

static int max_work(int32_t T, const int32_t *d, const int32_t *R, int64_t *maxC, int64_t *maxD)
{
    *maxC = 1;
    *maxD = 1;
    for (int t = 0; t < T; ++t) {
        int64_t c = (int64_t)d[3 * t] * d[3 * t + 1] * R[4 * t + 2];
        int64_t e = (int64_t)d[3 * t] * d[3 * t + 1] * d[3 * t + 2];
        if (c > *maxC) *maxC = c;
        if (e > *maxD) *maxD = e;
    }
    return ORC_OK;
}

/* --------------------------------------------------------------- forward */

/* Pooled forward with NO reuse: every index recomputes its row, rows are
 * summed over the bag in CSR order (FlowTT 3.2: contraction, then pooling;
 * TT-Rec abstract: EmbeddingBag).  out is fp64 [nsel][sum D]; bag_sel lists
 * the bag ids b (0..B-1) to evaluate, or is NULL for all B bags. */
int orc_forward(int32_t T, const int64_t *N, const int32_t *n, const int32_t *d, const int32_t *R,
                const float *const *cores, const int64_t *indices, const int64_t *offsets,
                int64_t B, int64_t nnz, const int64_t *bag_sel, int64_t nsel, double *out,
                int32_t nthreads)
{
    int rc = check_tables(T, N, n, d, R);
    if (rc) return rc;
    rc = check_csr(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    int64_t *col_off = (int64_t *)malloc(sizeof(int64_t) * T);
    if (!col_off) return ORC_ERR_NOMEM;
    const int64_t SD = sum_dims(T, d, col_off);
    int64_t maxC, maxD;
    max_work(T, d, R, &maxC, &maxD);
    const int64_t nb = bag_sel ? nsel : B;
    for (int64_t s = 0; s < nb; ++s)
        if (bag_sel && (bag_sel[s] < 0 || bag_sel[s] >= B)) {
            free(col_off);
            return ORC_ERR_ARG;
        }
    memset(out, 0, sizeof(double) * (size_t)(nb * SD));
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel reduction(| : failed)
#endif
    {
        double *C = (double *)malloc(sizeof(double) * (size_t)maxC);
        double *E = (double *)malloc(sizeof(double) * (size_t)maxD);
        if (!C || !E) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (int64_t s = 0; s < nb; ++s) {
            if (!C || !E) continue;
            const int64_t b = bag_sel ? bag_sel[s] : s;
            for (int t = 0; t < T; ++t) {
                const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
                const int64_t Dt = (int64_t)dt[0] * dt[1] * dt[2];
                double *acc = out + s * SD + col_off[t];
                for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                    int64_t i1, i2, i3;
                    decode3(indices[l], nt, &i1, &i2, &i3);
                    prefix_c(cores[3 * t], cores[3 * t + 1], dt, Rt, i1, i2, C);
                    suffix_e(C, cores[3 * t + 2], dt, Rt, i3, E);
                    for (int64_t j = 0; j < Dt; ++j) acc[j] += E[j];
                }
            }
        }
        free(C);
        free(E);
    }
    free(col_off);
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/* -------------------------------------------------------------- grouping */

typedef struct {
    int64_t row;
    int64_t pos;
} entry_t;

static int cmp_entry(const void *a, const void *b)
{
    const entry_t *x = (const entry_t *)a, *y = (const entry_t *)b;
    if (x->row != y->row) return x->row < y->row ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* Index grouping in the stage order of FlowTT section 4 (breakdown):
 *  1. sort lookups by row within each table, ties by position (stable);
 *  2. unique extraction: runs of equal row -> uniq_row, uniq_start, inv;
 *  3. mixed-radix conversion of each unique row, prefix q = row div n3
 *     (= i1*n2 + i2, the shared high-order digits of section 3.3);
 *  4. run-length encoding of equal prefixes -> grp_prefix, grp_start.
 * Arrays are concatenated over tables in table order; ids are global.
 * Capacities: perm/inv nnz; uniq_row, grp_prefix nnz; uniq_start, grp_start
 * nnz+1; tab_* T+1.  counts[0] = U (unique rows), counts[1] = G (groups). */
int orc_grouping(int32_t T, const int64_t *N, const int32_t *n, const int64_t *indices,
                 const int64_t *offsets, int64_t B, int64_t nnz, int32_t *perm,
                 int32_t *uniq_row, int32_t *uniq_start, int32_t *inv, int32_t *grp_prefix,
                 int32_t *grp_start, int32_t *tab_uniq_start, int32_t *tab_grp_start,
                 int64_t *counts)
{
    if (T <= 0 || B < 0 || nnz < 0 || nnz > 0x7fffffffLL) return ORC_ERR_ARG;
    for (int t = 0; t < T; ++t)
        if (N[t] <= 0 || n[3 * t + 2] <= 0 || n[3 * t + 1] <= 0) return ORC_ERR_ARG;
    int rc = check_csr(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    entry_t *e = (entry_t *)malloc(sizeof(entry_t) * (size_t)(nnz > 0 ? nnz : 1));
    if (!e) return ORC_ERR_NOMEM;
    for (int64_t l = 0; l < nnz; ++l) {
        e[l].row = indices[l];
        e[l].pos = l;
    }
    /* Step 1: per table segment (positions of table t are contiguous). */
    for (int t = 0; t < T; ++t) {
        int64_t lo = offsets[(int64_t)t * B], hi = offsets[(int64_t)(t + 1) * B];
        if (hi > lo) qsort(e + lo, (size_t)(hi - lo), sizeof(entry_t), cmp_entry);
    }
    for (int64_t k = 0; k < nnz; ++k) perm[k] = (int32_t)e[k].pos;
    /* Step 2: unique rows. */
    int64_t U = 0;
    for (int t = 0; t < T; ++t) {
        int64_t lo = offsets[(int64_t)t * B], hi = offsets[(int64_t)(t + 1) * B];
        tab_uniq_start[t] = (int32_t)U;
        for (int64_t k = lo; k < hi; ++k) {
            if (k == lo || e[k].row != e[k - 1].row) {
                uniq_row[U] = (int32_t)e[k].row;
                uniq_start[U] = (int32_t)k;
                ++U;
            }
            inv[e[k].pos] = (int32_t)(U - 1);
        }
    }
    tab_uniq_start[T] = (int32_t)U;
    uniq_start[U] = (int32_t)nnz;
    /* Steps 3-4: prefix of each unique row and run-length encoding. */
    int64_t G = 0;
    for (int t = 0; t < T; ++t) {
        const int64_t n3 = n[3 * t + 2];
        tab_grp_start[t] = (int32_t)G;
        int64_t prev = -1;
        for (int64_t u = tab_uniq_start[t]; u < tab_uniq_start[t + 1]; ++u) {
            int64_t q = (int64_t)uniq_row[u] / n3;
            if (u == tab_uniq_start[t] || q != prev) {
                grp_prefix[G] = (int32_t)q;
                grp_start[G] = (int32_t)u;
                ++G;
            }
            prev = q;
        }
    }
    tab_grp_start[T] = (int32_t)G;
    grp_start[G] = (int32_t)U;
    counts[0] = U;
    counts[1] = G;
    free(e);
    return ORC_OK;
}

/* Grouped forward: the prefix intermediate C is computed once per group,
 * each unique row once from its group's C, and bags are pooled in CSR order
 * through inv (FlowTT 3.2/3.3: prefix-shared reuse).  Uses the same loops as
 * the per-index path, so in exact arithmetic and in this fp64 build the two
 * results are identical; reuse changes cost, not value (FlowTT section 4,
 * prefix-reuse ablation).  out is fp64 [B][sum D]. */
int orc_forward_grouped(int32_t T, const int64_t *N, const int32_t *n, const int32_t *d,
                        const int32_t *R, const float *const *cores, const int64_t *indices,
                        const int64_t *offsets, int64_t B, int64_t nnz, double *out)
{
    int rc = check_tables(T, N, n, d, R);
    if (rc) return rc;
    const int64_t cap = nnz > 0 ? nnz : 1;
    int32_t *perm = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *urow = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *ustart = (int32_t *)malloc(sizeof(int32_t) * (cap + 1));
    int32_t *inv = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *gpre = (int32_t *)malloc(sizeof(int32_t) * cap);
    int32_t *gstart = (int32_t *)malloc(sizeof(int32_t) * (cap + 1));
    int32_t *tu = (int32_t *)malloc(sizeof(int32_t) * (T + 1));
    int32_t *tg = (int32_t *)malloc(sizeof(int32_t) * (T + 1));
    int64_t *col_off = (int64_t *)malloc(sizeof(int64_t) * T);
    int64_t counts[2];
    double *C = NULL, *Erows = NULL;
    rc = ORC_ERR_NOMEM;
    if (!perm || !urow || !ustart || !inv || !gpre || !gstart || !tu || !tg || !col_off) goto done;
    rc = orc_grouping(T, N, n, indices, offsets, B, nnz, perm, urow, ustart, inv, gpre, gstart,
                      tu, tg, counts);
    if (rc) goto done;
    {
        int64_t maxC, maxD;
        max_work(T, d, R, &maxC, &maxD);
        const int64_t SD = sum_dims(T, d, col_off);
        const int64_t U = counts[0];
        rc = ORC_ERR_NOMEM;
        C = (double *)malloc(sizeof(double) * (size_t)maxC);
        Erows = (double *)malloc(sizeof(double) * (size_t)((U > 0 ? U : 1) * maxD));
        if (!C || !Erows) goto done;
        for (int t = 0; t < T; ++t) {
            const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
            for (int64_t g = tg[t]; g < tg[t + 1]; ++g) {
                const int64_t q = gpre[g];
                prefix_c(cores[3 * t], cores[3 * t + 1], dt, Rt, q / nt[1], q % nt[1], C);
                for (int64_t u = gstart[g]; u < gstart[g + 1]; ++u)
                    suffix_e(C, cores[3 * t + 2], dt, Rt, (int64_t)urow[u] % nt[2],
                             Erows + u * maxD);
            }
        }
        memset(out, 0, sizeof(double) * (size_t)(B * SD));
        for (int t = 0; t < T; ++t) {
            const int64_t Dt = (int64_t)d[3 * t] * d[3 * t + 1] * d[3 * t + 2];
            for (int64_t b = 0; b < B; ++b) {
                double *acc = out + b * SD + col_off[t];
                for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                    const double *E = Erows + (int64_t)inv[l] * maxD;
                    for (int64_t j = 0; j < Dt; ++j) acc[j] += E[j];
                }
            }
        }
        rc = ORC_OK;
    }
done:
    free(perm); free(urow); free(ustart); free(inv); free(gpre); free(gstart);
    free(tu); free(tg); free(col_off); free(C); free(Erows);
    return rc;
}

/* -------------------------------------------------------------- backward */

/* Gradients of L = sum(grad_out * out) with respect to every core (FlowTT
 * 3.2: the backward reverses C = A.B, E = C.D, pooling).  Per index, with
 * g = grad_out[b][table block] viewed as [d1*d2][d3] and C recomputed:
 *   dG3[i3][r2][j3]    += sum_{m} C[m][r2] g[m][j3]
 *   dC[m][r2]           = sum_{j3} g[m][j3] G3[i3][r2][j3]
 *   dG1[i1][0][j1][r1] += sum_{j2,r2} dC[j1 j2][r2] G2[i2][r1][j2][r2]
 *   dG2[i2][r1][j2][r2]+= sum_{j1} G1[i1][0][j1][r1] dC[j1 j2][r2]
 * dG are fp64 arrays shaped like the cores, overwritten (untouched slices 0).
 * sel (optional, [T*3]) restricts the work to one slice per (table, core):
 * sel[3t+k] = slice index to compute, -1 = all slices, -2 = none; lookups
 * touching no selected slice are skipped.  Tables run in parallel; each
 * table's sums are sequential in CSR order. */
int orc_backward(int32_t T, const int64_t *N, const int32_t *n, const int32_t *d, const int32_t *R,
                 const float *const *cores, const int64_t *indices, const int64_t *offsets,
                 int64_t B, int64_t nnz, const float *grad_out, const int64_t *sel,
                 double *const *dG, int32_t nthreads)
{
    int rc = check_tables(T, N, n, d, R);
    if (rc) return rc;
    rc = check_csr(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    int64_t *col_off = (int64_t *)malloc(sizeof(int64_t) * T);
    if (!col_off) return ORC_ERR_NOMEM;
    const int64_t SD = sum_dims(T, d, col_off);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < 3; ++k) {
            const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
            size_t sz = (size_t)nt[k] * Rt[k] * dt[k] * Rt[k + 1];
            memset(dG[3 * t + k], 0, sizeof(double) * sz);
        }
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int t = 0; t < T; ++t) {
        const int32_t *nt = n + 3 * t, *dt = d + 3 * t, *Rt = R + 4 * t;
        const int d1 = dt[0], d2 = dt[1], d3 = dt[2], R1 = Rt[1], R2 = Rt[2];
        const int d12 = d1 * d2;
        const float *G1 = cores[3 * t], *G2 = cores[3 * t + 1], *G3 = cores[3 * t + 2];
        double *dG1 = dG[3 * t], *dG2 = dG[3 * t + 1], *dG3 = dG[3 * t + 2];
        const int64_t s1 = sel ? sel[3 * t] : -1, s2 = sel ? sel[3 * t + 1] : -1,
                      s3 = sel ? sel[3 * t + 2] : -1;
        double *C = (double *)malloc(sizeof(double) * (size_t)d12 * R2);
        double *dC = (double *)malloc(sizeof(double) * (size_t)d12 * R2);
        if (!C || !dC) {
            failed = 1;
            free(C);
            free(dC);
            continue;
        }
        for (int64_t b = 0; b < B; ++b) {
            const float *g = grad_out + b * SD + col_off[t];
            for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                int64_t i1, i2, i3;
                decode3(indices[l], nt, &i1, &i2, &i3);
                const int w1 = (s1 == -1 || s1 == i1), w2 = (s2 == -1 || s2 == i2),
                          w3 = (s3 == -1 || s3 == i3);
                if (!w1 && !w2 && !w3) continue;
                prefix_c(G1, G2, dt, Rt, i1, i2, C);
                const float *g3 = G3 + i3 * (int64_t)R2 * d3;
                if (w3) {
                    double *o = dG3 + i3 * (int64_t)R2 * d3;
                    for (int r2 = 0; r2 < R2; ++r2)
                        for (int j3 = 0; j3 < d3; ++j3) {
                            double acc = 0.0;
                            for (int m = 0; m < d12; ++m)
                                acc += C[m * R2 + r2] * (double)g[m * d3 + j3];
                            o[r2 * d3 + j3] += acc;
                        }
                }
                if (!w1 && !w2) continue;
                for (int m = 0; m < d12; ++m)
                    for (int r2 = 0; r2 < R2; ++r2) {
                        double acc = 0.0;
                        for (int j3 = 0; j3 < d3; ++j3)
                            acc += (double)g[m * d3 + j3] * (double)g3[r2 * d3 + j3];
                        dC[m * R2 + r2] = acc;
                    }
                const float *g1 = G1 + i1 * (int64_t)d1 * R1;
                const float *g2 = G2 + i2 * (int64_t)R1 * d2 * R2;
                if (w1) {
                    double *o = dG1 + i1 * (int64_t)d1 * R1;
                    for (int j1 = 0; j1 < d1; ++j1)
                        for (int r1 = 0; r1 < R1; ++r1) {
                            double acc = 0.0;
                            for (int j2 = 0; j2 < d2; ++j2)
                                for (int r2 = 0; r2 < R2; ++r2)
                                    acc += dC[(j1 * d2 + j2) * R2 + r2] *
                                           (double)g2[((int64_t)r1 * d2 + j2) * R2 + r2];
                            o[j1 * R1 + r1] += acc;
                        }
                }
                if (w2) {
                    double *o = dG2 + i2 * (int64_t)R1 * d2 * R2;
                    for (int r1 = 0; r1 < R1; ++r1)
                        for (int j2 = 0; j2 < d2; ++j2)
                            for (int r2 = 0; r2 < R2; ++r2) {
                                double acc = 0.0;
                                for (int j1 = 0; j1 < d1; ++j1)
                                    acc += (double)g1[j1 * R1 + r1] * dC[(j1 * d2 + j2) * R2 + r2];
                                o[((int64_t)r1 * d2 + j2) * R2 + r2] += acc;
                            }
                }
            }
        }
        free(C);
        free(dC);
    }
    free(col_off);
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/* Plain SGD step of the training configuration: delta = -lr * dG. */
void orc_sgd_delta(const double *dG, int64_t count, double lr, double *delta)
{
    for (int64_t k = 0; k < count; ++k) delta[k] = -lr * dG[k];
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------ K >= 2 TT cores */

/* The general case of the same statement (FlowTT summary, section 2.4: a row
 * is rebuilt by sequential TT-core contractions; section 3.3: rows sharing
 * their leading digits share every prefix of that chain).  Each table has K
 * cores; n, d are [T][K], R is [T][K+1] with R_0 = R_K = 1; digits are
 * big-endian (i = ((i1*n2 + i2)*n3 + ...)*nK + iK) and output column
 * j = ((j1*d2 + j2)*d3 + ...)*dK + jK, the 3-core readings extended. */

#define ORC_MAXK 8

static int check_tables_k(int32_t T, int32_t K, const int64_t *N, const int32_t *n, const int32_t *d,
                          const int32_t *R)
{
    if (T <= 0 || K < 2 || K > ORC_MAXK) return ORC_ERR_ARG;
    for (int t = 0; t < T; ++t) {
        const int32_t *nt = n + K * t, *dt = d + K * t, *Rt = R + (K + 1) * t;
        if (N[t] <= 0 || Rt[0] != 1 || Rt[K] != 1) return ORC_ERR_ARG;
        int64_t prod = 1;
        for (int k = 0; k < K; ++k) {
            if (nt[k] <= 0 || dt[k] <= 0 || Rt[k + 1] <= 0) return ORC_ERR_ARG;
            prod *= nt[k];
            if (prod > ((int64_t)1 << 40)) prod = (int64_t)1 << 40;
        }
        if (prod < N[t]) return ORC_ERR_ARG;
    }
    return ORC_OK;
}

/* Digits of row i, most significant first. */
static void decode_k(int64_t i, int32_t K, const int32_t *n, int64_t *dig)
{
    for (int k = K - 1; k >= 0; --k) {
        dig[k] = i % n[k];
        i /= n[k];
    }
}

/* One step of the chain: V is [P][Rin] (row-major); the result W is
 * [P*dk][Rout] with W[p*dk + j][r] = sum_{r'} V[p][r'] * G[ik][r'][j][r],
 * r' ascending. */
static void chain_step(const double *V, int64_t P, int32_t Rin, const float *Gk, int32_t dk, int32_t Rout,
                       int64_t ik, double *Wv)
{
    const float *g = Gk + (size_t)ik * Rin * dk * Rout;
    for (int64_t p = 0; p < P; ++p)
        for (int32_t j = 0; j < dk; ++j)
            for (int32_t r = 0; r < Rout; ++r) {
                double acc = 0.0;
                for (int32_t q = 0; q < Rin; ++q) acc += V[p * Rin + q] * (double)g[((size_t)q * dk + j) * Rout + r];
                Wv[(p * dk + j) * Rout + r] = acc;
            }
}

/* Row i of a K-core table, no reuse: V_1 = G1[i1] ([d1][R1]), V_k = V_{k-1} .
 * G_k[i_k] for k = 2..K; the row is V_K ([D][1]).  work holds 2*maxP doubles
 * where maxP bounds every intermediate (product of d's times the rank). */
static void row_k(int32_t K, const int32_t *nt, const int32_t *dt, const int32_t *Rt, const float *const *G,
                  int64_t i, double *work, int64_t maxP, double *E)
{
    int64_t dig[ORC_MAXK];
    decode_k(i, K, nt, dig);
    double *V = work, *Wv = work + maxP;
    int64_t P = dt[0];
    const float *g1 = G[0] + (size_t)dig[0] * dt[0] * Rt[1];
    for (int64_t e = 0; e < P * Rt[1]; ++e) V[e] = (double)g1[e];
    for (int k = 1; k < K; ++k) {
        chain_step(V, P, Rt[k], G[k], dt[k], Rt[k + 1], dig[k], Wv);
        P *= dt[k];
        double *tmp = V;
        V = Wv;
        Wv = tmp;
    }
    for (int64_t j = 0; j < P; ++j) E[j] = V[j];
}

static int64_t maxp_k(int32_t T, int32_t K, const int32_t *d, const int32_t *R, int64_t *maxD)
{
    int64_t m = 1;
    *maxD = 1;
    for (int t = 0; t < T; ++t) {
        int64_t P = 1;
        for (int k = 0; k < K; ++k) {
            P *= d[K * t + k];
            const int64_t c = P * R[(K + 1) * t + k + 1];
            if (c > m) m = c;
        }
        if (P > *maxD) *maxD = P;
    }
    return m;
}

static int check_csr_k(int32_t T, const int64_t *N, const int64_t *indices, const int64_t *offsets, int64_t B,
                       int64_t nnz)
{
    return check_csr(T, N, indices, offsets, B, nnz);
}

/* Pooled forward of K-core tables with NO reuse (every index recomputes its
 * whole chain), bags summed in CSR order; out fp64 [B][sum D]. */
int orc_forward_k(int32_t T, int32_t K, const int64_t *N, const int32_t *n, const int32_t *d, const int32_t *R,
                  const float *const *cores, const int64_t *indices, const int64_t *offsets, int64_t B,
                  int64_t nnz, double *out, int32_t nthreads)
{
    int rc = check_tables_k(T, K, N, n, d, R);
    if (rc) return rc;
    rc = check_csr_k(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    int64_t maxD;
    const int64_t maxP = maxp_k(T, K, d, R, &maxD);
    int64_t *col_off = (int64_t *)malloc(sizeof(int64_t) * T);
    if (!col_off) return ORC_ERR_NOMEM;
    int64_t SD = 0;
    for (int t = 0; t < T; ++t) {
        col_off[t] = SD;
        int64_t D = 1;
        for (int k = 0; k < K; ++k) D *= d[K * t + k];
        SD += D;
    }
    memset(out, 0, sizeof(double) * (size_t)(B * SD));
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel reduction(| : failed)
#endif
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * maxP));
        double *E = (double *)malloc(sizeof(double) * (size_t)maxD);
        if (!work || !E) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
        for (int64_t b = 0; b < B; ++b) {
            if (!work || !E) continue;
            for (int t = 0; t < T; ++t) {
                const int32_t *nt = n + K * t, *dt = d + K * t, *Rt = R + (K + 1) * t;
                int64_t D = 1;
                for (int k = 0; k < K; ++k) D *= dt[k];
                double *acc = out + b * SD + col_off[t];
                for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                    row_k(K, nt, dt, Rt, cores + (size_t)K * t, indices[l], work, maxP, E);
                    for (int64_t j = 0; j < D; ++j) acc[j] += E[j];
                }
            }
        }
        free(work);
        free(E);
    }
    free(col_off);
    return failed ? ORC_ERR_NOMEM : ORC_OK;
}

/* Unique rows of one table's lookups and, for every prefix length m = 1..K-1,
 * the intermediate V_m computed once per distinct leading-digit prefix and
 * reused by every row that shares it (FlowTT 3.3, generalised to every prefix
 * length); rows are V_K = V_{K-1}[prefix] . G_K[i_K].  Bags are then summed in
 * CSR order from the unique rows.  Same products in the same order as
 * orc_forward_k, so the result is identical. */
static int cmp_i64(const void *a, const void *b)
{
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

int orc_forward_k_grouped(int32_t T, int32_t K, const int64_t *N, const int32_t *n, const int32_t *d,
                          const int32_t *R, const float *const *cores, const int64_t *indices,
                          const int64_t *offsets, int64_t B, int64_t nnz, double *out)
{
    int rc = check_tables_k(T, K, N, n, d, R);
    if (rc) return rc;
    rc = check_csr_k(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    int64_t maxD;
    const int64_t maxP = maxp_k(T, K, d, R, &maxD);
    int64_t SD = 0;
    for (int t = 0; t < T; ++t) {
        int64_t D = 1;
        for (int k = 0; k < K; ++k) D *= d[K * t + k];
        SD += D;
    }
    memset(out, 0, sizeof(double) * (size_t)(B * SD));
    int64_t col = 0;
    for (int t = 0; t < T; ++t) {
        const int32_t *nt = n + K * t, *dt = d + K * t, *Rt = R + (K + 1) * t;
        const float *const *G = cores + (size_t)K * t;
        int64_t D = 1;
        for (int k = 0; k < K; ++k) D *= dt[k];
        const int64_t l0 = offsets[(int64_t)t * B], l1 = offsets[(int64_t)(t + 1) * B], m = l1 - l0;
        int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
        double *Erows = NULL, *lev = NULL;
        int64_t U = 0;
        if (!rows) return ORC_ERR_NOMEM;
        for (int64_t l = 0; l < m; ++l) rows[l] = indices[l0 + l];
        qsort(rows, (size_t)m, sizeof(int64_t), cmp_i64);
        for (int64_t l = 0; l < m; ++l)
            if (l == 0 || rows[l] != rows[l - 1]) rows[U++] = rows[l];
        Erows = (double *)malloc(sizeof(double) * (size_t)((U > 0 ? U : 1) * D));
        /* one current intermediate per prefix length, recomputed only when
         * the row's prefix of that length changes (rows are sorted, so equal
         * prefixes are consecutive) */
        lev = (double *)malloc(sizeof(double) * (size_t)(K * maxP));
        if (!Erows || !lev) {
            free(rows);
            free(Erows);
            free(lev);
            return ORC_ERR_NOMEM;
        }
        int64_t prevdig[ORC_MAXK];
        for (int k = 0; k < K; ++k) prevdig[k] = -1;
        for (int64_t u = 0; u < U; ++u) {
            int64_t dig[ORC_MAXK];
            decode_k(rows[u], K, nt, dig);
            int same = 1; /* prefix of length k+1 unchanged so far */
            int64_t P = dt[0];
            for (int k = 0; k < K; ++k) {
                same = same && dig[k] == prevdig[k];
                double *Vk = lev + (size_t)k * maxP;
                if (k == 0) {
                    if (!same) {
                        const float *g1 = G[0] + (size_t)dig[0] * dt[0] * Rt[1];
                        for (int64_t e = 0; e < P * Rt[1]; ++e) Vk[e] = (double)g1[e];
                    }
                } else {
                    if (!same) chain_step(lev + (size_t)(k - 1) * maxP, P, Rt[k], G[k], dt[k], Rt[k + 1], dig[k], Vk);
                    P *= dt[k];
                }
            }
            for (int k = 0; k < K; ++k) prevdig[k] = dig[k];
            const double *VK = lev + (size_t)(K - 1) * maxP;
            for (int64_t j = 0; j < D; ++j) Erows[u * D + j] = VK[j];
        }
        for (int64_t b = 0; b < B; ++b) {
            double *acc = out + b * SD + col;
            for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                /* unique id of the row: binary search in the sorted unique rows */
                int64_t lo = 0, hi = U - 1;
                while (lo < hi) {
                    const int64_t mid = (lo + hi) / 2;
                    if (rows[mid] < indices[l]) lo = mid + 1;
                    else hi = mid;
                }
                for (int64_t j = 0; j < D; ++j) acc[j] += Erows[lo * D + j];
            }
        }
        col += D;
        free(rows);
        free(Erows);
        free(lev);
    }
    return ORC_OK;
}

/* Backward of the pooled K-core forward for L = sum(grad_out * out), every
 * index on its own (no reuse), lookups in CSR order.  The chain of one index
 * is kept (V_1 .. V_K), then reversed (FlowTT 3.2: the backward reverses the
 * contraction structure), core K-1 first:
 *   V_{k+1}[p*d_k + j][r] = sum_q V_k[p][q] G_k[i_k][q][j][r]
 *   dG_k[i_k][q][j][r]   += sum_p V_k[p][q] dV_{k+1}[p*d_k + j][r]
 *   dV_k[p][q]            = sum_{j,r} dV_{k+1}[p*d_k + j][r] G_k[i_k][q][j][r]
 * with dV_K = the index's bag row of grad_out and, since V_1 = G_0[i_0],
 * dG_0[i_0] += dV_1.  dG (fp64, shaped like the cores, [T*K]) is overwritten;
 * untouched slices are 0. */
int orc_backward_k(int32_t T, int32_t K, const int64_t *N, const int32_t *n, const int32_t *d, const int32_t *R,
                   const float *const *cores, const int64_t *indices, const int64_t *offsets, int64_t B,
                   int64_t nnz, const float *grad_out, double *const *dG)
{
    int rc = check_tables_k(T, K, N, n, d, R);
    if (rc) return rc;
    rc = check_csr_k(T, N, indices, offsets, B, nnz);
    if (rc) return rc;
    int64_t maxD;
    const int64_t maxP = maxp_k(T, K, d, R, &maxD);
    int64_t SD = 0;
    for (int t = 0; t < T; ++t) {
        int64_t D = 1;
        for (int k = 0; k < K; ++k) D *= d[K * t + k];
        SD += D;
    }
    double *chain = (double *)malloc(sizeof(double) * (size_t)(K * maxP));
    double *dv = (double *)malloc(sizeof(double) * (size_t)(2 * maxP));
    if (!chain || !dv) {
        free(chain);
        free(dv);
        return ORC_ERR_NOMEM;
    }
    int64_t col = 0;
    for (int t = 0; t < T; ++t) {
        const int32_t *nt = n + K * t, *dt = d + K * t, *Rt = R + (K + 1) * t;
        const float *const *G = cores + (size_t)K * t;
        double *const *dGt = dG + (size_t)K * t;
        int64_t P[ORC_MAXK + 1];
        P[0] = 1;
        for (int k = 0; k < K; ++k) P[k + 1] = P[k] * dt[k];
        for (int k = 0; k < K; ++k)
            memset(dGt[k], 0, sizeof(double) * (size_t)nt[k] * Rt[k] * dt[k] * Rt[k + 1]);
        for (int64_t b = 0; b < B; ++b) {
            const float *g = grad_out + (size_t)(b * SD + col);
            for (int64_t l = offsets[(int64_t)t * B + b]; l < offsets[(int64_t)t * B + b + 1]; ++l) {
                int64_t dig[ORC_MAXK];
                decode_k(indices[l], K, nt, dig);
                /* forward chain: chain + (m-1)*maxP holds V_m ([P_m][R_m]) */
                const float *g0 = G[0] + (size_t)dig[0] * dt[0] * Rt[1];
                for (int64_t e = 0; e < P[1] * Rt[1]; ++e) chain[e] = (double)g0[e];
                for (int k = 1; k < K; ++k)
                    chain_step(chain + (size_t)(k - 1) * maxP, P[k], Rt[k], G[k], dt[k], Rt[k + 1], dig[k],
                               chain + (size_t)k * maxP);
                /* reverse: dV_K = g */
                double *dcur = dv, *dnext = dv + maxP;
                for (int64_t e = 0; e < P[K]; ++e) dcur[e] = (double)g[e];
                for (int k = K - 1; k >= 1; --k) {
                    const double *Vk = chain + (size_t)(k - 1) * maxP; /* [P_k][R_k] */
                    const float *gs = G[k] + (size_t)dig[k] * Rt[k] * dt[k] * Rt[k + 1];
                    double *dgs = dGt[k] + (size_t)dig[k] * Rt[k] * dt[k] * Rt[k + 1];
                    const int32_t Rin = Rt[k], dk = dt[k], Rout = Rt[k + 1];
                    for (int32_t q = 0; q < Rin; ++q)
                        for (int32_t j = 0; j < dk; ++j)
                            for (int32_t r = 0; r < Rout; ++r) {
                                double acc = 0.0;
                                for (int64_t p = 0; p < P[k]; ++p)
                                    acc += Vk[p * Rin + q] * dcur[(p * dk + j) * Rout + r];
                                dgs[((size_t)q * dk + j) * Rout + r] += acc;
                            }
                    for (int64_t p = 0; p < P[k]; ++p)
                        for (int32_t q = 0; q < Rin; ++q) {
                            double acc = 0.0;
                            for (int32_t j = 0; j < dk; ++j)
                                for (int32_t r = 0; r < Rout; ++r)
                                    acc += dcur[(p * dk + j) * Rout + r] * (double)gs[((size_t)q * dk + j) * Rout + r];
                            dnext[p * Rin + q] = acc;
                        }
                    double *tmp = dcur;
                    dcur = dnext;
                    dnext = tmp;
                }
                double *dg0 = dGt[0] + (size_t)dig[0] * dt[0] * Rt[1];
                for (int64_t e = 0; e < P[1] * Rt[1]; ++e) dg0[e] += dcur[e];
            }
        }
        col += P[K];
    }
    free(chain);
    free(dv);
    return ORC_OK;
}
