/*
 * CPU oracle for the 3D-RoPE sparse + low-rank hybrid attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition the HIP path is checked against. Only the tests, the smoke
 * check and the bench's CPU-baseline leg load it; the product path never
 * does. It shares no code, header, table or constant with the HIP library.
 *
 * Every routine works on one (batch, head) slice, in fp64, on one thread,
 * with plain loops in the order the method states. Inputs are the exact
 * values the GPU receives, widened to double by the caller.
 *
 * Sources (the pages):
 *  [RoLA]    "RoLA: Rotary-Positioned Low-Rank Linear Attention for Efficient
 *            Diffusion Transformers", arXiv 2609.06712v3 (section summary).
 *  [RoPeSLR] "RoPeSLR: 3D RoPE-driven Sparse-LowRank Attention for Efficient
 *            Diffusion Transformers", arXiv 2605.20659 (abstract, figures,
 *            appendix fragments).
 *
 * Points the pages leave open take the plainest reading:
 *  - tokens are flattened t-major, then h, then w; positions are integer
 *    coordinates from 0 (plus an optional origin offset used by tests);
 *  - the head is split into contiguous t | h | w chunks of adjacent pairs
 *    (2i, 2i+1); pair j of an axis with n pairs turns by p * base^(-2j/(2n));
 *  - block selection scores are the dot product of block means of the
 *    rotated q and k over the valid tokens, scaled by 1/sqrt(D); exact ties
 *    go to the lower block index; indices are stored ascending;
 *  - softmax scale is 1/sqrt(D);
 *  - phi(x) = elu(x) + 1; the normaliser uses the un-rotated features plus
 *    eps after the dot; the combine is additive with a per-head gate;
 *  - with the SiLU feature map (optional; sign-indefinite) the normaliser
 *    is the number of valid tokens instead;
 *  - the token-wise gate (optional) reads the token's raw query row, is a
 *    logistic of one linear form plus a bias, and the low-rank output is
 *    rescaled to the RMS (over the head dims) of the sparse output before
 *    it is added (see orc_token_gate).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Grid coordinates of flattened token l (t-major, then h, then w). */
static void token_coords(long l, int Hg, int Wg, int *t, int *h, int *w)
{
    *t = (int)(l / ((long)Hg * Wg));
    *h = (int)((l / Wg) % Hg);
    *w = (int)(l % Wg);
}

/* Angle of rotary pair j of an axis that owns n pairs, at coordinate p:
 * p * theta_j with theta_j = base^(-2j / d_axis), d_axis = 2n
 * ([RoLA] §3 "3D RoPE", eq. 1: each axis owns its own slice of the head
 * and its own geometric frequency schedule; [RoPeSLR] appendix, per-axis
 * partition of the rotary dimensions). */
static double pair_angle(double base, int n, int j, double p)
{
    double theta = pow(base, -2.0 * (double)j / (2.0 * (double)n));
    return p * theta;
}

/* Rotate pairs [first, first + count) of vector x (in place) by the
 * schedule of an axis with n_axis pairs, at coordinate p. */
static void rotate_pairs(double *x, int first, int count, double base, int n_axis, double p)
{
    for (int j = 0; j < count; ++j) {
        double a = pair_angle(base, n_axis, j, p);
        double c = cos(a), s = sin(a);
        double x0 = x[2 * (first + j)], x1 = x[2 * (first + j) + 1];
        x[2 * (first + j)] = x0 * c - x1 * s;
        x[2 * (first + j) + 1] = x0 * s + x1 * c;
    }
}

/*
 * 3D RoPE of a [L, D] slice ([RoLA] §3 "3D RoPE", eq. 1).
 * pairs[3] = rotary pairs on t, h, w (sum D/2), chunks laid out t | h | w.
 * origin[3] = coordinate offset added to every token (0 for the layer).
 */
void orc_rope3d(int T, int Hg, int Wg, const int origin[3], int D, double base,
                const int pairs[3], const double *x, double *y)
{
    long L = (long)T * Hg * Wg;
    for (long l = 0; l < L; ++l) {
        int c[3];
        token_coords(l, Hg, Wg, &c[0], &c[1], &c[2]);
        double *row = y + l * D;
        memcpy(row, x + l * D, sizeof(double) * D);
        int first = 0;
        for (int a = 0; a < 3; ++a) {
            rotate_pairs(row, first, pairs[a], base, pairs[a], (double)(c[a] + origin[a]));
            first += pairs[a];
        }
    }
}

/*
 * Block mean-pool ([RoLA] Fig. 2: the sparse branch keeps the top-k
 * blocks): block i covers tokens [i*bs, min((i+1)*bs, L)); the mean is over
 * its valid tokens only.
 */
void orc_block_mean(long L, int D, int bs, const double *x, double *out)
{
    long nblk = (L + bs - 1) / bs;
    for (long i = 0; i < nblk; ++i) {
        long lo = i * bs, hi = lo + bs < L ? lo + bs : L;
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (long l = lo; l < hi; ++l) s += x[l * D + d];
            out[i * D + d] = s / (double)(hi - lo);
        }
    }
}

/* Block scores s_ij = <qbar_i, kbar_j> / sqrt(D), [nblk, nblk]. */
void orc_block_scores(long nblk, int D, const double *qbar, const double *kbar, double *s)
{
    double scale = 1.0 / sqrt((double)D);
    for (long i = 0; i < nblk; ++i)
        for (long j = 0; j < nblk; ++j) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += qbar[i * D + d] * kbar[j * D + d];
            s[i * nblk + j] = acc * scale;
        }
}

/* Order used by the selection: larger score first, then lower block index. */
static const double *g_row;
static int by_score_then_index(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    if (g_row[a] > g_row[b]) return -1;
    if (g_row[a] < g_row[b]) return 1;
    return (a > b) - (a < b);
}
static int ascending_int(const void *pa, const void *pb)
{
    int a = *(const int *)pa, b = *(const int *)pb;
    return (a > b) - (a < b);
}

/*
 * Per-query-block top-k ([RoLA] Fig. 2, the top-k spike blocks; §4.1): keep
 * the k key blocks with the largest scores. idx[i, 0..k) ascending;
 * thr[i] = the k-th largest score of row i; next[i] = the (k+1)-th (or
 * -inf when k = nblk), so callers can tell how close the cut is.
 */
void orc_topk_blocks(long nblk, int k, const double *s, int32_t *idx, double *thr, double *next)
{
    int *order = (int *)malloc(sizeof(int) * nblk);
    for (long i = 0; i < nblk; ++i) {
        for (long j = 0; j < nblk; ++j) order[j] = (int)j;
        g_row = s + i * nblk;
        qsort(order, nblk, sizeof(int), by_score_then_index);
        thr[i] = g_row[order[k - 1]];
        next[i] = k < nblk ? g_row[order[k]] : -INFINITY;
        qsort(order, k, sizeof(int), ascending_int);
        for (int m = 0; m < k; ++m) idx[i * k + m] = order[m];
    }
    free(order);
}

/*
 * Block-sparse softmax attention ([RoLA] §4.1: block-sparse attention over
 * the high-energy spikes): for every valid query token of each listed query
 * block i, an exact softmax over the valid key tokens of the kept blocks
 * idx[i, :], scale 1/sqrt(D), then the weighted sum of V.
 * out is [nq, bs, D]; rows past L stay zero. Passing k = nblk with
 * idx[i, :] = 0..nblk-1 gives dense attention.
 */
void orc_block_sparse_attention(long L, int D, int bs, int k, const double *qr, const double *kr,
                                const double *v, const int32_t *idx, int nq,
                                const int32_t *qblocks, double *out)
{
    double scale = 1.0 / sqrt((double)D);
    double *logit = (double *)malloc(sizeof(double) * (size_t)k * bs);
    long *key = (long *)malloc(sizeof(long) * (size_t)k * bs);
    memset(out, 0, sizeof(double) * (size_t)nq * bs * D);
    for (int n = 0; n < nq; ++n) {
        long i = qblocks[n];
        /* gather the valid key tokens of the kept blocks */
        long nk = 0;
        for (int m = 0; m < k; ++m) {
            long j = idx[i * k + m];
            for (long t = j * bs; t < (j + 1) * bs && t < L; ++t) key[nk++] = t;
        }
        for (int r = 0; r < bs; ++r) {
            long lq = i * bs + r;
            if (lq >= L) break;
            double mx = -INFINITY;
            for (long m = 0; m < nk; ++m) {
                double acc = 0.0;
                for (int d = 0; d < D; ++d) acc += qr[lq * D + d] * kr[key[m] * D + d];
                logit[m] = acc * scale;
                if (logit[m] > mx) mx = logit[m];
            }
            double den = 0.0;
            for (long m = 0; m < nk; ++m) {
                logit[m] = exp(logit[m] - mx);
                den += logit[m];
            }
            double *o = out + ((size_t)n * bs + r) * D;
            for (long m = 0; m < nk; ++m) {
                double p = logit[m] / den;
                for (int d = 0; d < D; ++d) o[d] += p * v[key[m] * D + d];
            }
        }
    }
    free(logit);
    free(key);
}

/* phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise. */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)): the activation RoLA's
 * ablation finds best ([RoLA] §5.3, Table 6). */
static double silu(double x) { return x / (1.0 + exp(-x)); }

/*
 * Low-rank features u_l = phi(x_l W [+ E_t[t] + E_h[h] + E_w[w]]) of a
 * [L, D] slice with W [D, r]. The rotary variant ([RoLA] §4.3) feeds the
 * raw, position-free content features (E tables NULL); the absolute-PE
 * variant ([RoPeSLR] abstract: learnable 3D absolute positional embedding
 * injection) adds the per-axis tables before phi.
 *
 * fmap 0: phi = elu + 1; 1: SiLU (per component).
 * fmap 2: positive random features of the exponential kernel (FAVOR+ of
 * Performers, which the [RoPeSLR] appendix uses to linearise the softmax
 * exponential while keeping the branch low-rank): with p = x_l W [+ E] in
 * R^r and r random directions omega_c (rows of omega [r, r], drawn by the
 * caller from N(0, I_r)),
 *     u_c = exp(omega_c . p - |p|^2 / 2) / sqrt(r),
 * so that E_omega[u(p) . u(p')] = exp(p . p'). omega is ignored (may be
 * NULL) for fmap 0 and 1.
 */
void orc_lowrank_features(int T, int Hg, int Wg, int D, int r, const double *x, const double *W,
                          const double *Et, const double *Eh, const double *Ew, int fmap,
                          const double *omega, double *u)
{
    long L = (long)T * Hg * Wg;
    double *p = (double *)malloc(sizeof(double) * (size_t)r);
    for (long l = 0; l < L; ++l) {
        int t, h, w;
        token_coords(l, Hg, Wg, &t, &h, &w);
        for (int c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += x[l * D + d] * W[(long)d * r + c];
            if (Et) acc += Et[(long)t * r + c] + Eh[(long)h * r + c] + Ew[(long)w * r + c];
            p[c] = acc;
        }
        if (fmap == 2) {
            double sq = 0.0;
            for (int c = 0; c < r; ++c) sq += p[c] * p[c];
            for (int c = 0; c < r; ++c) {
                double dot = 0.0;
                for (int j = 0; j < r; ++j) dot += omega[(long)c * r + j] * p[j];
                u[l * r + c] = exp(dot - 0.5 * sq) / sqrt((double)r);
            }
        } else {
            for (int c = 0; c < r; ++c) u[l * r + c] = fmap ? silu(p[c]) : phi(p[c]);
        }
    }
    free(p);
}

/*
 * Rank-truncated rotation rho_pos applied after phi ([RoLA] §4.2-4.3):
 * the r-wide feature is split into t | h | w chunks of lr_pairs[a]
 * adjacent pairs; pair j of axis a reuses the backbone's frequency
 * theta_{a,j} (the axis owns pairs[a] backbone pairs, j < lr_pairs[a]).
 */
void orc_lowrank_rotate(int T, int Hg, int Wg, const int origin[3], int r, double base,
                        const int pairs[3], const int lr_pairs[3], const double *u, double *ur)
{
    long L = (long)T * Hg * Wg;
    for (long l = 0; l < L; ++l) {
        int c[3];
        token_coords(l, Hg, Wg, &c[0], &c[1], &c[2]);
        double *row = ur + l * r;
        memcpy(row, u + l * r, sizeof(double) * r);
        int first = 0;
        for (int a = 0; a < 3; ++a) {
            rotate_pairs(row, first, lr_pairs[a], base, pairs[a], (double)(c[a] + origin[a]));
            first += lr_pairs[a];
        }
    }
}

/*
 * The reusable per-head summary ([RoLA] §4.1 and App. B.1: one
 * query-independent sum at O(L r D)):
 *   S = sum_l fk_l v_l^T   ([r, D], fk = rotated features, or the plain
 *                           features for the absolute-PE variant),
 *   z = sum_l u_l          ([r], un-rotated features).
 */
void orc_lowrank_summary(long L, int D, int r, const double *fk, const double *u,
                         const double *v, double *S, double *z)
{
    memset(S, 0, sizeof(double) * (size_t)r * D);
    memset(z, 0, sizeof(double) * (size_t)r);
    for (long l = 0; l < L; ++l)
        for (int c = 0; c < r; ++c) {
            z[c] += u[l * r + c];
            for (int d = 0; d < D; ++d) S[(long)c * D + d] += fk[l * r + c] * v[l * D + d];
        }
}

/*
 * Per-query readout of the summary ([RoLA] App. A, Algorithm 1; §4.3):
 *   O_lr,l = (fq_l^T S) / (w_l . z + eps)
 * for the listed token rows; fq = rotated query features (plain ones for
 * the absolute-PE variant), w = un-rotated query features. With count > 0
 * (sign-indefinite features such as SiLU, where w . z can vanish) the
 * denominator is count, the number of valid tokens: the readout is then the
 * mean over the tokens.
 */
void orc_lowrank_readout(int D, int r, int nrows, const int64_t *rows, const double *fq,
                         const double *w, const double *S, const double *z, double eps,
                         double count, double *out)
{
    for (int n = 0; n < nrows; ++n) {
        long l = rows[n];
        double den = 0.0;
        for (int c = 0; c < r; ++c) den += w[l * r + c] * z[c];
        den += eps;
        if (count > 0.0) den = count;   /* sign-indefinite features: mean over the tokens */
        for (int d = 0; d < D; ++d) {
            double num = 0.0;
            for (int c = 0; c < r; ++c) num += fq[l * r + c] * S[(long)c * D + d];
            out[(long)n * D + d] = num / den;
        }
    }
}

/*
 * Token-wise gated fusion ([RoLA] §4.4 "Feature Alignment and Gated
 * Fusion"): a scalar gate per token combines the sparse and the low-rank
 * outputs, and the sparse output's RMS is the scale reference of the fusion.
 * For each of the n rows:
 *   g     = 1 / (1 + exp(-(q . wg + bg)))        (q = the raw query row)
 *   rms_s = sqrt(sum_d o_sp[d]^2 / D),  rms_l = sqrt(sum_d o_lr[d]^2 / D)
 *   out   = o_sp + g * rms_s / (rms_l + eps) * o_lr
 * The gate value of every row goes to gate[] when it is not NULL.
 */
void orc_token_gate(long n, int D, const double *q, const double *wg, double bg, const double *o_sp,
                    const double *o_lr, double eps, double *out, double *gate)
{
    for (long i = 0; i < n; ++i) {
        double t = bg;
        for (int d = 0; d < D; ++d) t += q[i * D + d] * wg[d];
        double g = 1.0 / (1.0 + exp(-t));
        double ss = 0.0, sl = 0.0;
        for (int d = 0; d < D; ++d) {
            ss += o_sp[i * D + d] * o_sp[i * D + d];
            sl += o_lr[i * D + d] * o_lr[i * D + d];
        }
        double scale = sqrt(ss / D) / (sqrt(sl / D) + eps);
        for (int d = 0; d < D; ++d) out[i * D + d] = o_sp[i * D + d] + g * scale * o_lr[i * D + d];
        if (gate) gate[i] = g;
    }
}
