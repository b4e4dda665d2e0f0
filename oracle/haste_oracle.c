/*
 * haste_oracle.c -- plain, slow, fp64 CPU oracle for the group-shared fixed
 * fan-in output layer (head dense classifier + sparse tail) and its
 * sigmoid-BCE training step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only tests/, the smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * Source of the method: gist.science Korean summary of "HASTE: Hardware-Aware
 * Dynamic Sparse Training for Large Output Spaces" (page 1 of the reference
 * text), section "Method", item 1 "Group-Shared Fixed Fan-In Sparsity"
 * (labels in a group share one fan-in index set but keep their own weight
 * vectors; indices are stored once per group), item 2 "Head-Tail
 * Decomposition" (frequent labels use a standard dense classifier).  The
 * pages print no formulas; the definitions below are the plain reading:
 *
 *   tail label t lives in group g = t / G, slot j = t % G            (C1)
 *   z[b][t]  = sum_{f=0}^{F-1} X[b][idx[g][f]] * Wt[t][f]   (f order)
 *   zh[b][h] = sum_{d=0}^{D-1} X[b][d] * Wh[h][d]
 *   loss    += s * (softplus(z) - y*z),  softplus(z) = max(z,0)+log1p(e^-|z|)
 *   dz       = s * (sigmoid(z) - y),     y = 1 iff the label is a positive
 *   dWt[t][f] = sum_b X[b][idx[g][f]] * dz[b][t]
 *   dX[b][d]  = sum_h dzh[b][h]*Wh[h][d]
 *             + sum_{(g,f): idx[g][f]=d} sum_j dz[b][gG+j] * Wt[gG+j][f]
 *
 * Ragged last group (G does not divide L): N_g = ceil(L/G); padded labels
 * t >= L produce no logit, no loss, and their weight gradient is zero.
 * Every function returns, beside each output, the sum of absolute values
 * of the products that formed it (the tolerance scale).
 *
 * All arrays are row-major.  Label-range outputs are in "live label"
 * coordinates: column c of a tail output for groups [g0, g1) is tail label
 * g0*G + c, for c < min(g1*G, L) - g0*G.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t live_end(int64_t L, int G, int64_t g1)
{
    int64_t e = g1 * (int64_t)G;
    return e < L ? e : L;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Storage layout of the tail (Method 1, "memory efficiency": one index set
 * per group).  out = {N_g, stored index count, stored weight rows,
 *                     live labels in the last group}. */
void oracle_layout(int64_t L, int G, int F, int64_t *out)
{
    int64_t ng = (L + G - 1) / G;
    out[0] = ng;
    out[1] = ng * (int64_t)F;
    out[2] = ng * (int64_t)G;
    out[3] = L - (ng - 1) * (int64_t)G;
}

/* Tail logits for rows[0..n_rows) and groups [g0, g1). */
void oracle_tail_logits(int B, int D, int64_t L, int G, int F,
                        const double *X, const int32_t *idx, const double *Wt,
                        const int32_t *rows, int n_rows, int64_t g0, int64_t g1,
                        double *Z, double *Zabs)
{
    (void)B;
    int64_t t0 = g0 * (int64_t)G, t1 = live_end(L, G, g1);
    int64_t ncol = t1 - t0;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        const double *x = X + (int64_t)rows[r] * D;
        for (int64_t t = t0; t < t1; ++t) {
            const int32_t *ix = idx + (t / G) * (int64_t)F;
            const double *w = Wt + t * (int64_t)F;
            double acc = 0.0, aab = 0.0;
            for (int f = 0; f < F; ++f) {
                double p = x[ix[f]] * w[f];
                acc += p;
                aab += fabs(p);
            }
            Z[(int64_t)r * ncol + (t - t0)] = acc;
            if (Zabs) Zabs[(int64_t)r * ncol + (t - t0)] = aab;
        }
    }
}

/* Head logits (Method 2: dense classifier over the frequent labels) for
 * rows[0..n_rows) and head labels [h0, h1). */
void oracle_head_logits(int B, int D, int H, const double *X, const double *Wh,
                        const int32_t *rows, int n_rows, int h0, int h1,
                        double *Z, double *Zabs)
{
    (void)B; (void)H;
    int ncol = h1 - h0;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        const double *x = X + (int64_t)rows[r] * D;
        for (int h = h0; h < h1; ++h) {
            const double *w = Wh + (int64_t)h * D;
            double acc = 0.0, aab = 0.0;
            for (int d = 0; d < D; ++d) {
                double p = x[d] * w[d];
                acc += p;
                aab += fabs(p);
            }
            Z[(int64_t)r * ncol + (h - h0)] = acc;
            if (Zabs) Zabs[(int64_t)r * ncol + (h - h0)] = aab;
        }
    }
}

/* y mask: Y[r][c] = 1 iff global label (label_begin + c) is listed among the
 * positives of row rows[r] (row-CSR: labels[row_ptr[b] .. row_ptr[b+1])). */
void oracle_positive_mask(const int32_t *row_ptr, const int32_t *labels,
                          const int32_t *rows, int n_rows,
                          int64_t label_begin, int64_t n_cols, double *Y)
{
    memset(Y, 0, sizeof(double) * (size_t)n_rows * (size_t)n_cols);
    for (int r = 0; r < n_rows; ++r) {
        int b = rows[r];
        for (int32_t k = row_ptr[b]; k < row_ptr[b + 1]; ++k) {
            int64_t c = (int64_t)labels[k] - label_begin;
            if (c >= 0 && c < n_cols) Y[(int64_t)r * n_cols + c] = 1.0;
        }
    }
}

/* Sigmoid binary cross-entropy on logits, elementwise, scaled by s:
 *   loss_term = s * (max(z,0) + log1p(exp(-|z|)) - y*z)
 *   dz        = s * (sigmoid(z) - y),  sigmoid evaluated without overflow. */
void oracle_bce(int64_t n, const double *z, const double *y, double s,
                double *dz, double *loss_terms)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double zi = z[i], yi = y[i];
        double e = exp(-fabs(zi));
        double sig = zi >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
        if (dz) dz[i] = s * (sig - yi);
        if (loss_terms)
            /* max(z,0) - y*z is exact for y in {0,1}; adding log1p last
             * keeps the small y=1, z>>0 losses accurate */
            loss_terms[i] = s * (((zi > 0.0 ? zi : 0.0) - yi * zi) + log1p(e));
    }
}

/* Tail weight gradient for groups [g0, g1):
 *   dWt[t][f] = sum_b X[b][idx[g][f]] * dZ[b][t]
 * dZ is B x ncol (live labels of the range).  dWt is ncol x F. */
void oracle_tail_dW(int B, int D, int64_t L, int G, int F,
                    const double *X, const int32_t *idx, const double *dZ,
                    int64_t g0, int64_t g1, double *dWt, double *dWabs)
{
    int64_t t0 = g0 * (int64_t)G, t1 = live_end(L, G, g1);
    int64_t ncol = t1 - t0;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < ncol; ++c) {
        int64_t t = t0 + c;
        const int32_t *ix = idx + (t / G) * (int64_t)F;
        for (int f = 0; f < F; ++f) {
            double acc = 0.0, aab = 0.0;
            for (int b = 0; b < B; ++b) {
                double p = X[(int64_t)b * D + ix[f]] * dZ[(int64_t)b * ncol + c];
                acc += p;
                aab += fabs(p);
            }
            dWt[c * F + f] = acc;
            if (dWabs) dWabs[c * F + f] = aab;
        }
    }
}

/* Tail input gradient for n_rows rows, all groups:
 *   dX[r][d] = sum_{(g,f): idx[g][f]=d} sum_j dZ[r][gG+j] * Wt[gG+j][f]
 * dZ is n_rows x L (all live tail labels).  dX, dXabs are n_rows x D and are
 * overwritten. */
void oracle_tail_dX(int D, int64_t L, int G, int F, const int32_t *idx,
                    const double *Wt, const double *dZ, int n_rows,
                    double *dX, double *dXabs)
{
    int64_t ng = (L + G - 1) / G;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        double *out = dX + (int64_t)r * D;
        double *oab = dXabs ? dXabs + (int64_t)r * D : NULL;
        memset(out, 0, sizeof(double) * (size_t)D);
        if (oab) memset(oab, 0, sizeof(double) * (size_t)D);
        const double *dz = dZ + (int64_t)r * L;
        for (int64_t g = 0; g < ng; ++g) {
            const int32_t *ix = idx + g * (int64_t)F;
            int64_t tend = live_end(L, G, g + 1);
            for (int f = 0; f < F; ++f) {
                double acc = 0.0, aab = 0.0;
                for (int64_t t = g * (int64_t)G; t < tend; ++t) {
                    double p = dz[t] * Wt[t * F + f];
                    acc += p;
                    aab += fabs(p);
                }
                out[ix[f]] += acc;
                if (oab) oab[ix[f]] += aab;
            }
        }
    }
}

/* Head weight gradient: dWh[h][d] = sum_b dZh[b][h] * X[b][d]. */
void oracle_head_dW(int B, int D, int H, const double *X, const double *dZh,
                    double *dWh, double *dWabs)
{
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; ++h) {
        for (int d = 0; d < D; ++d) {
            double acc = 0.0, aab = 0.0;
            for (int b = 0; b < B; ++b) {
                double p = dZh[(int64_t)b * H + h] * X[(int64_t)b * D + d];
                acc += p;
                aab += fabs(p);
            }
            dWh[(int64_t)h * D + d] = acc;
            if (dWabs) dWabs[(int64_t)h * D + d] = aab;
        }
    }
}

/* Head input gradient for n_rows rows: dX[r][d] = sum_h dZh[r][h]*Wh[h][d].
 * dZh is n_rows x H.  Overwrites dX, dXabs. */
void oracle_head_dX(int D, int H, const double *Wh, const double *dZh,
                    int n_rows, double *dX, double *dXabs)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        for (int d = 0; d < D; ++d) {
            double acc = 0.0, aab = 0.0;
            for (int h = 0; h < H; ++h) {
                double p = dZh[(int64_t)r * H + h] * Wh[(int64_t)h * D + d];
                acc += p;
                aab += fabs(p);
            }
            dX[(int64_t)r * D + d] = acc;
            if (dXabs) dXabs[(int64_t)r * D + d] = aab;
        }
    }
}

/* Exact top-K per row: order every (value, id) pair by value descending,
 * ties by smaller id first, keep the first K.  ids[c] names column c; when
 * ids is NULL, column c has id id_offset + c.  Plain selection by repeated
 * scans (K is small). */
void oracle_topk(int n_rows, int64_t n_cols, const double *z,
                 const int64_t *ids, int64_t id_offset, int K,
                 double *out_val, int64_t *out_idx)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < n_rows; ++r) {
        const double *row = z + (int64_t)r * n_cols;
        double prev_v = INFINITY;
        int64_t prev_id = -1;
        for (int k = 0; k < K; ++k) {
            double best_v = -INFINITY;
            int64_t best_id = -1;
            for (int64_t c = 0; c < n_cols; ++c) {
                double v = row[c];
                int64_t id = ids ? ids[c] : id_offset + c;
                /* must come strictly after the previous pick in the order */
                int after_prev = (v < prev_v) || (v == prev_v && id > prev_id);
                if (!after_prev) continue;
                if (best_id < 0 || v > best_v || (v == best_v && id < best_id)) {
                    best_v = v;
                    best_id = id;
                }
            }
            out_val[(int64_t)r * K + k] = best_v;
            out_idx[(int64_t)r * K + k] = best_id;
            prev_v = best_v;
            prev_id = best_id;
        }
    }
}

/* Group-major view of the tail positives: the positives whose global label
 * falls in [label_offset, label_offset + L), listed group by group, within a
 * group by row b then slot j.  grp_ptr has N_g + 1 entries; entry e is
 * b * G + j.  Returns the number of entries. */
int64_t oracle_group_positives(int B, const int32_t *row_ptr,
                               const int32_t *labels, int64_t label_offset,
                               int64_t L, int G, int32_t *grp_ptr,
                               int32_t *entries)
{
    int64_t ng = (L + G - 1) / G;
    if (ng <= 0 || B <= 0) {
        grp_ptr[0] = 0;
        return 0;
    }
    memset(grp_ptr, 0, sizeof(int32_t) * (size_t)(ng + 1));
    for (int b = 0; b < B; ++b)
        for (int32_t k = row_ptr[b]; k < row_ptr[b + 1]; ++k) {
            int64_t t = (int64_t)labels[k] - label_offset;
            if (t >= 0 && t < L) grp_ptr[t / G + 1] += 1;
        }
    for (int64_t g = 0; g < ng; ++g) grp_ptr[g + 1] += grp_ptr[g];
    int64_t n = grp_ptr[ng];
    /* Fill each group's slice in (b, j) order by scanning rows in order. */
    int32_t *fill = (int32_t *)calloc((size_t)ng, sizeof(int32_t));
    for (int b = 0; b < B; ++b) {
        /* within a row, emit in ascending slot order per group */
        int32_t k0 = row_ptr[b], k1 = row_ptr[b + 1];
        for (int j = 0; j < G; ++j)
            for (int32_t k = k0; k < k1; ++k) {
                int64_t t = (int64_t)labels[k] - label_offset;
                if (t < 0 || t >= L || (int)(t % G) != j) continue;
                int64_t g = t / G;
                entries[grp_ptr[g] + fill[g]] = b * G + j;
                fill[g] += 1;
            }
    }
    free(fill);
    return n;
}

/* One training step of the tail for groups [g0, g1), streaming group by
 * group so that no B x L array exists: logits, sigmoid-BCE against the
 * positives, weight gradient and input-gradient contribution.
 *   dWt  : ((min(g1*G,L) - g0*G) x F) output, or NULL
 *   dX   : B x D, accumulated (+=), or NULL
 * Returns the summed (scaled) loss of the range. */
double oracle_tail_step(int B, int D, int64_t L, int G, int F,
                        const double *X, const int32_t *idx, const double *Wt,
                        const int32_t *row_ptr, const int32_t *labels,
                        int64_t label_offset, double s, int64_t g0, int64_t g1,
                        double *dWt, double *dX)
{
    int nth = oracle_threads();
    double *loss_th = (double *)calloc((size_t)nth, sizeof(double));
    double *dX_th = NULL;
    if (dX) dX_th = (double *)calloc((size_t)nth * (size_t)B * (size_t)D, sizeof(double));
#pragma omp parallel
    {
        int th = 0;
#ifdef _OPENMP
        th = omp_get_thread_num();
#endif
        double *z = (double *)malloc(sizeof(double) * (size_t)B * (size_t)G);
        double *dz = (double *)malloc(sizeof(double) * (size_t)B * (size_t)G);
        double *myX = dX ? dX_th + (size_t)th * B * D : NULL;
        double myloss = 0.0;
#pragma omp for schedule(static)
        for (int64_t g = g0; g < g1; ++g) {
            const int32_t *ix = idx + g * (int64_t)F;
            int64_t tb = g * (int64_t)G, te = live_end(L, G, g + 1);
            int nlive = (int)(te - tb);
            for (int b = 0; b < B; ++b) {
                const double *x = X + (int64_t)b * D;
                for (int j = 0; j < nlive; ++j) {
                    const double *w = Wt + (tb + j) * F;
                    double acc = 0.0;
                    for (int f = 0; f < F; ++f) acc += x[ix[f]] * w[f];
                    double y = 0.0;
                    for (int32_t k = row_ptr[b]; k < row_ptr[b + 1]; ++k)
                        if ((int64_t)labels[k] - label_offset == tb + j) y = 1.0;
                    double e = exp(-fabs(acc));
                    double sig = acc >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
                    myloss += s * (((acc > 0.0 ? acc : 0.0) - y * acc) + log1p(e));
                    z[b * G + j] = acc;
                    dz[b * G + j] = s * (sig - y);
                }
            }
            if (dWt) {
                for (int j = 0; j < nlive; ++j)
                    for (int f = 0; f < F; ++f) {
                        double acc = 0.0;
                        for (int b = 0; b < B; ++b)
                            acc += X[(int64_t)b * D + ix[f]] * dz[b * G + j];
                        dWt[(tb + j - g0 * (int64_t)G) * F + f] = acc;
                    }
            }
            if (myX) {
                for (int b = 0; b < B; ++b)
                    for (int f = 0; f < F; ++f) {
                        double acc = 0.0;
                        for (int j = 0; j < nlive; ++j)
                            acc += dz[b * G + j] * Wt[(tb + j) * F + f];
                        myX[(int64_t)b * D + ix[f]] += acc;
                    }
            }
        }
        loss_th[th] = myloss;
        free(z);
        free(dz);
    }
    double loss = 0.0;
    for (int t = 0; t < nth; ++t) loss += loss_th[t];
    if (dX) {
        for (int t = 0; t < nth; ++t) {
            const double *src = dX_th + (size_t)t * B * D;
            for (int64_t i = 0; i < (int64_t)B * D; ++i) dX[i] += src[i];
        }
        free(dX_th);
    }
    free(loss_th);
    return loss;
}
