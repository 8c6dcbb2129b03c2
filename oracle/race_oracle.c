/*
 * race_oracle.c -- plain fp64 CPU oracle for RACE attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this file
 * or the library built from it: only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Sources (all pages carry the title "RACE Attention: A Strictly Linear-Time
 * Attention for Long-Sequence Training"; tags used below):
 *   [zh]  gist.science/zh/paper/2510.04008, technical summary
 *   [es]  gist.science/es/paper/2510.04008, technical summary
 *   [pt]  gist.science/pt/paper/2510.04008, technical summary
 *   [fr]  gist.science/fr/paper/2510.04008, technical summary
 *   [de]  gist.science/de/paper/2510.04008, technical summary
 *
 * What is computed, step by step, for every (batch, head) slice:
 *   1. rows of Q and K are L2-normalised ([es] §2 kernel with norms,
 *      [fr] §2.A);
 *   2. projected on Gaussian hyperplanes W[L][P][d] ([zh] §2.2);
 *   3. squashed with tanh ([zh] §2.2, [pt] §2);
 *   4. turned into corner logits s_lr = (1/tau) sum_p c_rp z_lp, with
 *      c_rp = +1 when bit p of r is set and -1 otherwise, and
 *   5. a softmax over the R = 2^P hypercube corners of each table gives the
 *      soft assignment phi ([zh] §2.2 soft bucketing, [pt] §2 "tanh then
 *      softmax"; tau = 1/beta is the temperature of [zh] §3);
 *   6. per table and bucket, the key mass A and the value-weighted mass B
 *      are summed ([zh] §2.2 bucket aggregation);
 *   7. each query reads out sum_l phi_l(q)^T B_l / sum_l phi_l(q)^T A_l
 *      ([zh] §2.2 output reconstruction);
 *   8. causal mode keeps running sums A_cum, B_cum that a token updates with
 *      its own key before its query reads them, so query i sees keys j <= i
 *      ([zh] §2.3);
 *   9. the backward pass is the exact derivative of steps 1-8 (the pages
 *      state the method is differentiable end to end, [es] §2 item 3, [fr]
 *      §3 item 3); the chain rule is written out in backward_* below, and
 *      optionally continued to the projection W of step 2 (for learned
 *      hyperplanes; the pages draw W at random and keep it fixed).
 *
 * Parallelism never reorders arithmetic: every running sum is updated in
 * token order and every dot product is summed in index order.  Threads only
 * split independent elements: the columns (or rows) of the running state,
 * and the tokens of a block when hashing.
 *
 * Hard mode (hard != 0) replaces step 5 by the one-hot corner whose bit p is
 * [z_lp >= 0] -- the tau -> 0 limit, used only to pin the oracle against
 * SimHash collision probabilities and angular attention.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ENOMEM 2

#define NORM_EPS 1e-12 /* x_hat = x / max(||x||, NORM_EPS) */
#define BLK 2048       /* tokens hashed together before a sweep */

typedef struct {
    int d, L, P, R, F;
    double tau;
    int hard;
    const double *W; /* [L][P][d] */
} hashp;

static double corner_sign(int r, int p) { return ((r >> p) & 1) ? 1.0 : -1.0; }

/* Steps 1-5 for one row x[d].  Writes x_hat[d], z[L*P], phi[L*R] and ||x||. */
static void hash_row(const hashp *h, const double *x, double *xhat, double *z,
                     double *phi, double *nrm_out)
{
    const int d = h->d, L = h->L, P = h->P, R = h->R;
    double n2 = 0.0;
    for (int t = 0; t < d; ++t) n2 += x[t] * x[t];
    const double nrm = sqrt(n2);
    const double s = nrm > NORM_EPS ? nrm : NORM_EPS;
    for (int t = 0; t < d; ++t) xhat[t] = x[t] / s;

    for (int l = 0; l < L; ++l)
        for (int p = 0; p < P; ++p) {
            const double *w = h->W + ((size_t)l * P + p) * d;
            double u = 0.0;
            for (int t = 0; t < d; ++t) u += w[t] * xhat[t];
            z[l * P + p] = tanh(u);
        }

    for (int l = 0; l < L; ++l) {
        const double *zl = z + (size_t)l * P;
        double *ph = phi + (size_t)l * R;
        if (h->hard) {
            int rstar = 0;
            for (int p = 0; p < P; ++p)
                if (zl[p] >= 0.0) rstar |= 1 << p;
            for (int r = 0; r < R; ++r) ph[r] = (r == rstar) ? 1.0 : 0.0;
            continue;
        }
        double mx = -INFINITY;
        for (int r = 0; r < R; ++r) {
            double sr = 0.0;
            for (int p = 0; p < P; ++p) sr += corner_sign(r, p) * zl[p];
            ph[r] = sr / h->tau;
            if (ph[r] > mx) mx = ph[r];
        }
        double tot = 0.0;
        for (int r = 0; r < R; ++r) {
            ph[r] = exp(ph[r] - mx);
            tot += ph[r];
        }
        for (int r = 0; r < R; ++r) ph[r] /= tot;
    }
    if (nrm_out) *nrm_out = nrm;
}

/* Backward of steps 1-5 for one row: given dL/dphi[L*R], returns dL/dx[d].
 *   ds_lr = phi_lr (dphi_lr - sum_r' phi_lr' dphi_lr')      softmax
 *   dz_lp = (1/tau) sum_r c_rp ds_lr                         corner logits
 *   du_lp = dz_lp (1 - z_lp^2)                               tanh
 *   dxh_t = sum_lp W[l][p][t] du_lp                          projection
 *   dx    = (dxh - (dxh . xh) xh) / ||x||   if ||x|| > eps   normalisation
 *         = dxh / eps                       otherwise                       */
static void hash_row_backward(const hashp *h, const double *x, const double *dphi,
                              double *dx, double *xhat, double *z, double *phi,
                              double *du, double *dxh)
{
    const int d = h->d, L = h->L, P = h->P, R = h->R;
    double nrm;
    hash_row(h, x, xhat, z, phi, &nrm);
    for (int l = 0; l < L; ++l) {
        const double *ph = phi + (size_t)l * R, *dph = dphi + (size_t)l * R;
        double dot = 0.0;
        for (int r = 0; r < R; ++r) dot += ph[r] * dph[r];
        for (int p = 0; p < P; ++p) {
            double dz = 0.0;
            for (int r = 0; r < R; ++r) dz += corner_sign(r, p) * (ph[r] * (dph[r] - dot));
            dz /= h->tau;
            const double zz = z[l * P + p];
            du[l * P + p] = dz * (1.0 - zz * zz);
        }
    }
    for (int t = 0; t < d; ++t) {
        double acc = 0.0;
        for (int lp = 0; lp < L * P; ++lp) acc += h->W[(size_t)lp * d + t] * du[lp];
        dxh[t] = acc;
    }
    if (nrm > NORM_EPS) {
        double proj = 0.0;
        for (int t = 0; t < d; ++t) proj += dxh[t] * xhat[t];
        for (int t = 0; t < d; ++t) dx[t] = (dxh[t] - proj * xhat[t]) / nrm;
    } else {
        for (int t = 0; t < d; ++t) dx[t] = dxh[t] / NORM_EPS;
    }
}

/* ------------------------------------------------------------------------ */
/* Per-block buffers: the soft assignments of a block of tokens, the value  */
/* rows extended by the count column [v | 1], and the ratio gradients D.    */

typedef struct {
    double *phq, *phk; /* [BLK][F] */
    double *v1;        /* [BLK][d+1] */
    double *D;         /* [BLK][d+1] */
    double *out;       /* [BLK][max(F, d+1)] */
} blockbuf;

typedef struct {
    hashp h;
    int d, d1, causal;
    int64_t N;
    const double *q, *k, *v, *g; /* this head's rows */
    const double *o, *m;         /* the oracle's own forward results (backward only) */
} headp;

static int alloc_block(blockbuf *b, int F, int d1)
{
    const int w = F > d1 ? F : d1;
    b->phq = malloc(sizeof(double) * (size_t)BLK * F);
    b->phk = malloc(sizeof(double) * (size_t)BLK * F);
    b->v1 = malloc(sizeof(double) * (size_t)BLK * d1);
    b->D = malloc(sizeof(double) * (size_t)BLK * d1);
    b->out = malloc(sizeof(double) * (size_t)BLK * w);
    return (b->phq && b->phk && b->v1 && b->D && b->out) ? ORC_OK : ORC_ENOMEM;
}

static void free_block(blockbuf *b)
{
    free(b->phq); free(b->phk); free(b->v1); free(b->D); free(b->out);
}

/* Fill the block starting at token b0 (n tokens). */
static void fill_block(const headp *hp, int64_t b0, int n, int need_q, int need_k,
                       int need_D, blockbuf *bb)
{
    const int d = hp->d, d1 = hp->d1, F = hp->h.F, LP = hp->h.L * hp->h.P;
#pragma omp parallel
    {
        double *xh = malloc(sizeof(double) * d);
        double *z = malloc(sizeof(double) * LP);
#pragma omp for schedule(static)
        for (int i = 0; i < n; ++i) {
            const int64_t t = b0 + i;
            if (need_k) hash_row(&hp->h, hp->k + t * d, xh, z, bb->phk + (size_t)i * F, NULL);
            if (need_q) hash_row(&hp->h, hp->q + t * d, xh, z, bb->phq + (size_t)i * F, NULL);
            for (int c = 0; c < d; ++c) bb->v1[(size_t)i * d1 + c] = hp->v[t * d + c];
            bb->v1[(size_t)i * d1 + d] = 1.0;
            if (need_D) {
                /* step 9: n = m o, so d/dn = g/m and d/dm = -(g . o)/m */
                const double mi = hp->m[t];
                double go = 0.0;
                for (int c = 0; c < d; ++c) {
                    bb->D[(size_t)i * d1 + c] = hp->g[t * d + c] / mi;
                    go += hp->g[t * d + c] * hp->o[t * d + c];
                }
                bb->D[(size_t)i * d1 + d] = -go / mi;
            }
        }
        free(xh);
        free(z);
    }
}

static void thread_range(int total, int *lo, int *hi)
{
#ifdef _OPENMP
    const int nt = omp_get_num_threads(), id = omp_get_thread_num();
#else
    const int nt = 1, id = 0;
#endif
    const int base = total / nt, rem = total % nt;
    *lo = id * base + (id < rem ? id : rem);
    *hi = *lo + base + (id < rem ? 1 : 0);
}

/* Column sweep over the tokens of a block, state M[ncol][F] (column-major:
 * column c of the state is M[c*F .. c*F+F)).
 * At each token i, in sweep order (reverse when rev):
 *   upd: M[c][f] += a_i[f] * b_i[c]
 *   rd : out_i[c] = sum_f M[c][f] * h_i[f]        (f in index order)
 * Threads own disjoint column ranges, so each M[c][f] sees tokens in order. */
static void col_sweep(int F, int ncol, int n, int rev, const double *a, const double *b,
                      int bstride, const double *hv, double *M, double *out, int ostride,
                      int upd, int rd)
{
#pragma omp parallel
    {
        int c0, c1;
        thread_range(ncol, &c0, &c1);
        for (int s = 0; s < n && c1 > c0; ++s) {
            const int i = rev ? n - 1 - s : s;
            const double *ai = a + (size_t)i * F, *bi = b + (size_t)i * bstride;
            const double *hi = hv ? hv + (size_t)i * F : NULL;
            for (int c = c0; c < c1; ++c) {
                double *Mc = M + (size_t)c * F;
                if (upd) {
                    const double bc = bi[c];
                    for (int f = 0; f < F; ++f) Mc[f] += ai[f] * bc;
                }
                if (rd) {
                    double acc = 0.0;
                    for (int f = 0; f < F; ++f) acc += Mc[f] * hi[f];
                    out[(size_t)i * ostride + c] = acc;
                }
            }
        }
    }
}

/* Row sweep over the tokens of a block, state M[ncol][F] (column-major).
 *   upd: M[c][f] += a_i[f] * b_i[c]
 *   rd : out_i[f] = sum_c M[c][f] * e_i[c]        (c in index order)
 * Threads own disjoint feature ranges. */
static void row_sweep(int F, int ncol, int n, int rev, const double *a, const double *b,
                      const double *e, double *M, double *out, int upd, int rd)
{
#pragma omp parallel
    {
        int f0, f1;
        thread_range(F, &f0, &f1);
        const int w = f1 - f0;
        double *acc = malloc(sizeof(double) * (w > 0 ? w : 1));
        for (int s = 0; s < n && w > 0; ++s) {
            const int i = rev ? n - 1 - s : s;
            const double *ai = a + (size_t)i * F, *bi = b + (size_t)i * ncol;
            const double *ei = e ? e + (size_t)i * ncol : NULL;
            if (upd)
                for (int c = 0; c < ncol; ++c) {
                    double *Mc = M + (size_t)c * F;
                    for (int f = f0; f < f1; ++f) Mc[f] += ai[f] * bi[c];
                }
            if (rd) {
                for (int f = 0; f < w; ++f) acc[f] = 0.0;
                for (int c = 0; c < ncol; ++c) {
                    const double *Mc = M + (size_t)c * F;
                    for (int f = f0; f < f1; ++f) acc[f - f0] += Mc[f] * ei[c];
                }
                for (int f = f0; f < f1; ++f) out[(size_t)i * F + f] = acc[f - f0];
            }
        }
        free(acc);
    }
}

/* Backward of steps 1-5 for every row of a block.  With dW (may be NULL), also
 * the gradient of the projection u = W x_hat (step 2):
 * dW[lp][t] += sum over the block's rows, in row order, of du_lp xhat_t. */
static int block_hash_backward(const headp *hp, const double *x, int64_t b0, int n,
                               const double *dphi, double *dx, double *dW)
{
    const int d = hp->d, F = hp->h.F, LP = hp->h.L * hp->h.P;
    double *dus = NULL, *xhs = NULL;
    if (dW) {
        dus = malloc(sizeof(double) * (size_t)n * LP);
        xhs = malloc(sizeof(double) * (size_t)n * d);
        if (!dus || !xhs) { free(dus); free(xhs); return ORC_ENOMEM; }
    }
#pragma omp parallel
    {
        double *xh = malloc(sizeof(double) * d), *z = malloc(sizeof(double) * LP);
        double *ph = malloc(sizeof(double) * F), *du = malloc(sizeof(double) * LP);
        double *dxh = malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int i = 0; i < n; ++i) {
            hash_row_backward(&hp->h, x + (b0 + i) * d, dphi + (size_t)i * F,
                              dx + (b0 + i) * d, xh, z, ph, du, dxh);
            if (dus) {
                memcpy(dus + (size_t)i * LP, du, sizeof(double) * LP);
                memcpy(xhs + (size_t)i * d, xh, sizeof(double) * d);
            }
        }
        free(xh); free(z); free(ph); free(du); free(dxh);
    }
    if (dW) {
#pragma omp parallel for schedule(static)
        for (int lp = 0; lp < LP; ++lp)
            for (int i = 0; i < n; ++i) {
                const double g = dus[(size_t)i * LP + lp];
                for (int t = 0; t < d; ++t) dW[(size_t)lp * d + t] += g * xhs[(size_t)i * d + t];
            }
        free(dus);
        free(xhs);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Forward for one head: steps 1-8.                                         */

static int forward_head(const headp *hp, double *o, double *den)
{
    const int d = hp->d, d1 = hp->d1, F = hp->h.F;
    const int64_t N = hp->N;
    blockbuf bb;
    double *M = calloc((size_t)F * d1, sizeof(double)); /* [d1][F]: columns 0..d-1 = B, d = A */
    if (!M || alloc_block(&bb, F, d1) != ORC_OK) { free(M); return ORC_ENOMEM; }

    if (!hp->causal) {
        /* step 6 over all keys, then step 7 for all queries */
        for (int64_t b0 = 0; b0 < N; b0 += BLK) {
            const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
            fill_block(hp, b0, n, 0, 1, 0, &bb);
            col_sweep(F, d1, n, 0, bb.phk, bb.v1, d1, NULL, M, NULL, 0, 1, 0);
        }
    }
    for (int64_t b0 = 0; b0 < N; b0 += BLK) {
        const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
        fill_block(hp, b0, n, 1, hp->causal, 0, &bb);
        /* causal: token i adds its key, then its query reads (step 8) */
        col_sweep(F, d1, n, 0, bb.phk, bb.v1, d1, bb.phq, M, bb.out, d1, hp->causal, 1);
        for (int i = 0; i < n; ++i) {
            const double *nm = bb.out + (size_t)i * d1;
            const double m = nm[d];
            den[b0 + i] = m;
            for (int c = 0; c < d; ++c) o[(b0 + i) * d + c] = (m != 0.0) ? nm[c] / m : 0.0;
        }
    }
    free(M);
    free_block(&bb);
    return ORC_OK;
}

/* Backward for one head: given the oracle's own o and m and dL/do = g.
 * With S_i the state visible to query i (causal: keys j <= i) and
 * G_j the gradient state of key j (causal: queries i >= j):
 *   dphi(q_i) = S_i D_i                     D_i = [g_i/m_i | -(g_i . o_i)/m_i]
 *   G_j       = sum_i phi(q_i) D_i^T
 *   dv_j      = (G_j[:, :d])^T phi(k_j)
 *   dphi(k_j) = G_j [v_j | 1]
 * then the hash backward for dq and dk. */
static int backward_head(const headp *hp, double *dq, double *dk, double *dv, double *dW)
{
    const int d = hp->d, d1 = hp->d1, F = hp->h.F;
    const int64_t N = hp->N;
    const int causal = hp->causal;
    blockbuf bb;
    double *M = calloc((size_t)F * d1, sizeof(double));
    if (!M || alloc_block(&bb, F, d1) != ORC_OK) { free(M); return ORC_ENOMEM; }

    /* query side: state [d1][F] of keys, read with D_i */
    if (!causal)
        for (int64_t b0 = 0; b0 < N; b0 += BLK) {
            const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
            fill_block(hp, b0, n, 0, 1, 0, &bb);
            row_sweep(F, d1, n, 0, bb.phk, bb.v1, NULL, M, NULL, 1, 0);
        }
    for (int64_t b0 = 0; b0 < N; b0 += BLK) {
        const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
        fill_block(hp, b0, n, 0, causal, 1, &bb);
        row_sweep(F, d1, n, 0, bb.phk, bb.v1, bb.D, M, bb.out, causal, 1);
        if (block_hash_backward(hp, hp->q, b0, n, bb.out, dq, dW)) {
            free(M);
            free_block(&bb);
            return ORC_ENOMEM;
        }
    }

    /* key side, dphi(k): state [d1][F] of queries, swept in reverse, read with [v|1] */
    memset(M, 0, sizeof(double) * (size_t)F * d1);
    if (!causal)
        for (int64_t b0 = 0; b0 < N; b0 += BLK) {
            const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
            fill_block(hp, b0, n, 1, 0, 1, &bb);
            row_sweep(F, d1, n, 0, bb.phq, bb.D, NULL, M, NULL, 1, 0);
        }
    for (int64_t e = N; e > 0; e -= BLK) {
        const int64_t b0 = e - BLK > 0 ? e - BLK : 0;
        const int n = (int)(e - b0);
        fill_block(hp, b0, n, causal, 0, causal, &bb);
        row_sweep(F, d1, n, 1, bb.phq, bb.D, bb.v1, M, bb.out, causal, 1);
        if (block_hash_backward(hp, hp->k, b0, n, bb.out, dk, dW)) {
            free(M);
            free_block(&bb);
            return ORC_ENOMEM;
        }
    }

    /* key side, dv: state [d][F] of queries (value columns of D only) */
    memset(M, 0, sizeof(double) * (size_t)F * d1);
    if (!causal)
        for (int64_t b0 = 0; b0 < N; b0 += BLK) {
            const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
            fill_block(hp, b0, n, 1, 0, 1, &bb);
            col_sweep(F, d, n, 0, bb.phq, bb.D, d1, NULL, M, NULL, 0, 1, 0);
        }
    for (int64_t e = N; e > 0; e -= BLK) {
        const int64_t b0 = e - BLK > 0 ? e - BLK : 0;
        const int n = (int)(e - b0);
        fill_block(hp, b0, n, causal, 1, causal, &bb);
        col_sweep(F, d, n, 1, bb.phq, bb.D, d1, bb.phk, M, dv + b0 * d, d, causal, 1);
    }
    free(M);
    free_block(&bb);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Causal streaming over consecutive blocks of one head ([zh] §2.3: the     */
/* running sums A_cum, B_cum carried from token to token).  The state that */
/* one block hands to the next is passed in and out explicitly, so a        */
/* sequence too long to hold at once is processed block by block in the    */
/* same token order as forward_head / backward_head.                        */

/* Forward of one block: M [d1][F] holds the sums of every earlier key on
 * entry (zero for the first block) and of every key up to the block's last
 * on return; each token adds its key before its query reads (step 8). */
static int stream_forward_block(const headp *hp, double *M, double *o, double *den)
{
    const int d = hp->d, d1 = hp->d1, F = hp->h.F;
    blockbuf bb;
    if (alloc_block(&bb, F, d1) != ORC_OK) return ORC_ENOMEM;
    for (int64_t b0 = 0; b0 < hp->N; b0 += BLK) {
        const int n = (int)(hp->N - b0 < BLK ? hp->N - b0 : BLK);
        fill_block(hp, b0, n, 1, 1, 0, &bb);
        col_sweep(F, d1, n, 0, bb.phk, bb.v1, d1, bb.phq, M, bb.out, d1, 1, 1);
        for (int i = 0; i < n; ++i) {
            const double *nm = bb.out + (size_t)i * d1;
            den[b0 + i] = nm[d];
            for (int c = 0; c < d; ++c) o[(b0 + i) * d + c] = nm[c] / nm[d];
        }
    }
    free_block(&bb);
    return ORC_OK;
}

/* Backward of one block, given the block's own o and m from
 * stream_forward_block.  S [d1][F]: sums of the keys before the block (in),
 * through its last key (out).  G [d1][F]: gradient sums sum_i phi(q_i) D_i^T
 * of the queries after the block (in), from its first query on (out).  The
 * three sweeps of backward_head (dq forward with S, dphi(k) and dv in
 * reverse with G) each start from the state handed in. */
static int stream_backward_block(const headp *hp, double *S, double *G, double *dq, double *dk,
                                 double *dv)
{
    const int d = hp->d, d1 = hp->d1, F = hp->h.F;
    const int64_t N = hp->N;
    const size_t sz = sizeof(double) * (size_t)F * d1;
    blockbuf bb;
    double *Gv = malloc(sz);
    if (!Gv || alloc_block(&bb, F, d1) != ORC_OK) { free(Gv); return ORC_ENOMEM; }
    memcpy(Gv, G, sz);
    int err = ORC_OK;
    for (int64_t b0 = 0; b0 < N && !err; b0 += BLK) {
        const int n = (int)(N - b0 < BLK ? N - b0 : BLK);
        fill_block(hp, b0, n, 0, 1, 1, &bb);
        row_sweep(F, d1, n, 0, bb.phk, bb.v1, bb.D, S, bb.out, 1, 1);
        err = block_hash_backward(hp, hp->q, b0, n, bb.out, dq, NULL);
    }
    for (int64_t e = N; e > 0 && !err; e -= BLK) {
        const int64_t b0 = e - BLK > 0 ? e - BLK : 0;
        const int n = (int)(e - b0);
        fill_block(hp, b0, n, 1, 1, 1, &bb);
        row_sweep(F, d1, n, 1, bb.phq, bb.D, bb.v1, G, bb.out, 1, 1);
        err = block_hash_backward(hp, hp->k, b0, n, bb.out, dk, NULL);
        if (!err) col_sweep(F, d, n, 1, bb.phq, bb.D, d1, bb.phk, Gv, dv + b0 * d, d, 1, 1);
    }
    free(Gv);
    free_block(&bb);
    return err;
}

/* ------------------------------------------------------------------------ */
/* Exported entry points.  All tensors are contiguous fp64:                 */
/*   q, k, v, g, o, dq, dk, dv : [BH][N][d]     den : [BH][N]                */
/*   W : [L][P][d], shared by all heads                                     */

static int check_args(int64_t BH, int64_t N, int d, int L, int P, double tau, int hard)
{
    if (BH < 1 || N < 1 || d < 1 || L < 1 || P < 1 || P > 12) return ORC_EINVAL;
    if (!hard && !(tau > 0.0 && isfinite(tau))) return ORC_EINVAL;
    return ORC_OK;
}

static void make_hashp(hashp *h, int d, int L, int P, double tau, int hard, const double *W)
{
    h->d = d; h->L = L; h->P = P; h->R = 1 << P; h->F = L * (1 << P);
    h->tau = tau; h->hard = hard; h->W = W;
}

int race_oracle_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Soft (or hard) assignment of n rows: phi[n][L*R]; optional z[n][L*P]. */
int race_oracle_hash(const double *x, int64_t n, int d, const double *W, int L, int P,
                     double tau, int hard, double *phi, double *z)
{
    if (check_args(1, n, d, L, P, tau, hard)) return ORC_EINVAL;
    hashp h;
    make_hashp(&h, d, L, P, tau, hard, W);
    int err = ORC_OK;
#pragma omp parallel
    {
        double *xh = malloc(sizeof(double) * d), *zz = malloc(sizeof(double) * L * P);
        if (!xh || !zz) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        } else {
#pragma omp for schedule(static)
            for (int64_t i = 0; i < n; ++i) {
                hash_row(&h, x + i * d, xh, zz, phi + i * h.F, NULL);
                if (z) memcpy(z + i * L * P, zz, sizeof(double) * L * P);
            }
        }
        free(xh);
        free(zz);
    }
    return err;
}

int race_oracle_forward(const double *q, const double *k, const double *v, const double *W,
                        int L, int P, double tau, int causal, int hard, int64_t BH, int64_t N,
                        int d, double *o, double *den)
{
    if (check_args(BH, N, d, L, P, tau, hard)) return ORC_EINVAL;
    headp hp;
    memset(&hp, 0, sizeof hp);
    make_hashp(&hp.h, d, L, P, tau, hard, W);
    hp.d = d; hp.d1 = d + 1; hp.causal = causal ? 1 : 0; hp.N = N;
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t off = bh * N * d;
        hp.q = q + off; hp.k = k + off; hp.v = v + off;
        const int err = forward_head(&hp, o + off, den + bh * N);
        if (err) return err;
    }
    return ORC_OK;
}

/* Forward and backward together: the backward uses this call's own forward
 * results, never values supplied from outside.  dW (may be NULL): the
 * gradient of the projection, [L][P][d], summed over every head and over the
 * rows of q and of k. */
int race_oracle_forward_backward_w(const double *q, const double *k, const double *v,
                                   const double *g, const double *W, int L, int P, double tau,
                                   int causal, int64_t BH, int64_t N, int d, double *o,
                                   double *den, double *dq, double *dk, double *dv, double *dW)
{
    if (check_args(BH, N, d, L, P, tau, 0)) return ORC_EINVAL;
    if (dW) memset(dW, 0, sizeof(double) * (size_t)L * P * d);
    headp hp;
    memset(&hp, 0, sizeof hp);
    make_hashp(&hp.h, d, L, P, tau, 0, W);
    hp.d = d; hp.d1 = d + 1; hp.causal = causal ? 1 : 0; hp.N = N;
    for (int64_t bh = 0; bh < BH; ++bh) {
        const int64_t off = bh * N * d;
        hp.q = q + off; hp.k = k + off; hp.v = v + off; hp.g = g + off;
        int err = forward_head(&hp, o + off, den + bh * N);
        if (err) return err;
        hp.o = o + off; hp.m = den + bh * N;
        err = backward_head(&hp, dq + off, dk + off, dv + off, dW);
        if (err) return err;
    }
    return ORC_OK;
}

int race_oracle_forward_backward(const double *q, const double *k, const double *v,
                                 const double *g, const double *W, int L, int P, double tau,
                                 int causal, int64_t BH, int64_t N, int d, double *o,
                                 double *den, double *dq, double *dk, double *dv)
{
    return race_oracle_forward_backward_w(q, k, v, g, W, L, P, tau, causal, BH, N, d, o, den, dq,
                                          dk, dv, NULL);
}

/* Causal forward of one block of a head's rows q, k, v [n][d], continuing a
 * sequence: M [d + 1][L R] holds, column-major (column c is M[c L R ..]),
 * the bucket sums B (columns 0..d-1) and A (column d) of every earlier key on
 * entry and of every key through the block on return. */
int race_oracle_stream_forward(const double *q, const double *k, const double *v,
                               const double *W, int L, int P, double tau, int64_t n, int d,
                               double *M, double *o, double *den)
{
    if (check_args(1, n, d, L, P, tau, 0) || !M) return ORC_EINVAL;
    headp hp;
    memset(&hp, 0, sizeof hp);
    make_hashp(&hp.h, d, L, P, tau, 0, W);
    hp.d = d; hp.d1 = d + 1; hp.causal = 1; hp.N = n;
    hp.q = q; hp.k = k; hp.v = v;
    return stream_forward_block(&hp, M, o, den);
}

/* Causal backward of one block, given its own o and den from
 * race_oracle_stream_forward and g = dL/do [n][d].  S [d + 1][L R]: key
 * sums before the block (in), through it (out).  G [d + 1][L R]: the
 * queries' gradient sums sum_i phi(q_i) D_i^T, D_i = [g_i/m_i | -(g_i .
 * o_i)/m_i], over the queries after the block (in), from the block's first
 * query on (out). */
int race_oracle_stream_backward(const double *q, const double *k, const double *v,
                                const double *g, const double *o, const double *den,
                                const double *W, int L, int P, double tau, int64_t n, int d,
                                double *S, double *G, double *dq, double *dk, double *dv)
{
    if (check_args(1, n, d, L, P, tau, 0) || !S || !G) return ORC_EINVAL;
    headp hp;
    memset(&hp, 0, sizeof hp);
    make_hashp(&hp.h, d, L, P, tau, 0, W);
    hp.d = d; hp.d1 = d + 1; hp.causal = 1; hp.N = n;
    hp.q = q; hp.k = k; hp.v = v; hp.g = g; hp.o = o; hp.m = den;
    return stream_backward_block(&hp, S, G, dq, dk, dv);
}

/* M [ycols][L R] += sum_j phi(x_j) y_j^T over the n rows of x [n][d] and
 * y [n][ycols], in row order (column-major as above).  With y = [v | 1] these
 * are a block's bucket sums B and A ([zh] §2.2); with y = D the gradient sums
 * of race_oracle_stream_backward. */
int race_oracle_block_sums(const double *x, const double *y, int ycols, int64_t n, int d,
                           const double *W, int L, int P, double tau, double *M)
{
    if (check_args(1, n, d, L, P, tau, 0) || ycols < 1 || !M) return ORC_EINVAL;
    hashp h;
    make_hashp(&h, d, L, P, tau, 0, W);
    double *ph = malloc(sizeof(double) * (size_t)BLK * h.F);
    if (!ph) return ORC_ENOMEM;
    for (int64_t b0 = 0; b0 < n; b0 += BLK) {
        const int nb = (int)(n - b0 < BLK ? n - b0 : BLK);
#pragma omp parallel
        {
            double *xh = malloc(sizeof(double) * d), *z = malloc(sizeof(double) * L * P);
#pragma omp for schedule(static)
            for (int i = 0; i < nb; ++i) hash_row(&h, x + (b0 + i) * d, xh, z, ph + (size_t)i * h.F, NULL);
            free(xh);
            free(z);
        }
        col_sweep(h.F, ycols, nb, 0, ph, y + b0 * ycols, ycols, NULL, M, NULL, 0, 1, 0);
    }
    free(ph);
    return ORC_OK;
}
