/*
 * fp64 CPU oracle of FS-B, FreeSolo's balanced tree search (two causal
 * forests, beam search, token-level reranking).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library, with which it shares
 * no code.  Plain loops, full sorts, no caching: every block's forests are
 * built from scratch, so each step can be checked against the page by eye.
 *
 * Page: "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 * Extrapolation" (arXiv 2610.17191).
 *   Sec. 3.4 "Two causal forests"        Eq. 10  admitted sets A^0 = C_i, A^tau
 *   Sec. 3.4 "Beam search"               Eq. 11  node priority U_v
 *   Sec. 3.4 "Token-level reranking"     Eq. 12  reranked score
 *   App. E.1 "Chunks"                    Eq. 18  binary decomposition of M
 *   App. E.1 "Splitting a chunk"         Eq. 19  two power iterations, median split
 *   App. E.1 "Node summaries"            Eq. 20  mu, rho, A, p_min
 *   App. E.1 "Joining chunk roots"       Eq. 21  join nodes, smallest chunk first
 *   App. E.1 "Beam search and reranking"         leaves keep their slots
 * Cell summaries (Eq. 5), availability (Eq. 6) and the readout (Eq. 9, Eq. 17)
 * are those of fsl_oracle.c.
 *
 * Readings where the page leaves a choice open:
 *   - ties go to the smaller cell id everywhere: the farthest cell c* of a
 *     split, equal projections, equal rerank scores; nodes of equal priority
 *     go to the one whose smallest cell id is smaller (the beam's nodes are
 *     disjoint subtrees, so that id names one node);
 *   - projections are sorted ascending and the first ceil(n/2) cells form the
 *     left child;
 *   - u^(t) is normalised to unit length (a zero vector stays zero, and then
 *     every projection is 0 and the split falls back to id order);
 *   - a leaf in the beam keeps its slot; the W^b minus that many remaining
 *     slots take the highest-priority children of the beam's internal nodes;
 *     search ends when every node of the beam is a leaf.
 */
#include "fsl_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- App. E.1 Eq. 18: chunks ------------------------------------------------ */

int32_t oracle_fsb_chunks(int64_t M, int64_t *sizes)
{
    int32_t r = 0;
    for (int k = 62; k >= 0; --k) /* powers of two of M, largest first */
        if ((M >> k) & 1)
            sizes[r++] = (int64_t)1 << k;
    return r;
}

/* ---- forest nodes -------------------------------------------------------------- */

typedef struct {
    int32_t d;
    int64_t n, cap;
    int64_t *count, *cell, *left, *right, *minid;
    double *mu, *rho, *A, *pmin;
} forest;

static void forest_init(forest *F, int32_t d, int64_t cap)
{
    F->d = d;
    F->n = 0;
    F->cap = cap > 0 ? cap : 1;
    F->count = malloc(sizeof(int64_t) * F->cap);
    F->cell = malloc(sizeof(int64_t) * F->cap);
    F->left = malloc(sizeof(int64_t) * F->cap);
    F->right = malloc(sizeof(int64_t) * F->cap);
    F->minid = malloc(sizeof(int64_t) * F->cap);
    F->mu = malloc(sizeof(double) * F->cap * d);
    F->rho = malloc(sizeof(double) * F->cap);
    F->A = malloc(sizeof(double) * F->cap);
    F->pmin = malloc(sizeof(double) * F->cap);
}

static void forest_free(forest *F)
{
    free(F->count); free(F->cell); free(F->left); free(F->right); free(F->minid);
    free(F->mu); free(F->rho); free(F->A); free(F->pmin);
}

static double dist(const double *x, const double *y, int32_t d)
{
    double s = 0.0;
    for (int32_t f = 0; f < d; ++f)
        s += (x[f] - y[f]) * (x[f] - y[f]);
    return sqrt(s);
}

/* Eq. 20 for a node over `cells` (ids into kbar/a) */
static int64_t new_chunk_node(forest *F, const oracle_cfg *cfg, const double *kbar, const double *a,
                              const int64_t *cells, int64_t n)
{
    const int32_t d = F->d;
    const int64_t v = F->n++;
    double *mu = F->mu + v * d;
    for (int32_t f = 0; f < d; ++f) {
        double s = 0.0;
        for (int64_t x = 0; x < n; ++x)
            s += kbar[cells[x] * d + f];
        mu[f] = s / (double)n;
    }
    double rho = 0.0, A = -INFINITY;
    int64_t mn = cells[0];
    for (int64_t x = 0; x < n; ++x) {
        const double r = dist(kbar + cells[x] * d, mu, d);
        if (r > rho)
            rho = r;
        if (a[cells[x]] > A)
            A = a[cells[x]];
        if (cells[x] < mn)
            mn = cells[x];
    }
    F->count[v] = n;
    F->rho[v] = rho;
    F->A[v] = A;
    F->minid[v] = mn;
    F->pmin[v] = ((double)mn + 0.5) * cfg->s; /* min_c p_c: the earliest cell */
    F->cell[v] = n == 1 ? cells[0] : -1;
    F->left[v] = F->right[v] = -1;
    return v;
}

typedef struct {
    double val, mag; /* a projection x_c . u and the size of its terms */
    int64_t id;
} projected;

static int by_projection(const void *x, const void *y) /* ascending, ties to the smaller id */
{
    const projected *p = (const projected *)x, *q = (const projected *)y;
    if (p->val < q->val) return -1;
    if (p->val > q->val) return 1;
    return (p->id < q->id) ? -1 : (p->id > q->id) ? 1 : 0;
}

typedef struct {
    double val;
    int64_t id;
} keyed2;

/* Eq. 19: normalise u to unit length (a zero vector stays zero) */
static void unit(double *u, int32_t d)
{
    double s = 0.0;
    for (int32_t f = 0; f < d; ++f)
        s += u[f] * u[f];
    if (s > 0.0) {
        const double inv = 1.0 / sqrt(s);
        for (int32_t f = 0; f < d; ++f)
            u[f] *= inv;
    }
}

/* App. E.1 "Splitting a chunk": the subtree over cells[0..n), returns its root.
 * min_gap receives the smallest relative gap between the two projections that
 * straddle a median split (near-ties there decide the tree). */
static int64_t build_subtree(forest *F, const oracle_cfg *cfg, const double *kbar, const double *a,
                             const int64_t *cells, int64_t n, double *min_gap)
{
    const int64_t v = new_chunk_node(F, cfg, kbar, a, cells, n);
    if (n == 1)
        return v;
    const int32_t d = F->d;
    const double *mu = F->mu + v * d;
    double *x = malloc(sizeof(double) * n * d); /* centred mean keys x_c = kbar_c - mu_v */
    for (int64_t c = 0; c < n; ++c)
        for (int32_t f = 0; f < d; ++f)
            x[c * d + f] = kbar[cells[c] * d + f] - mu[f];
    /* u^(0) from the farthest cell c*, then two power iterations */
    int64_t star = 0, bestid = 0;
    double best = -1.0;
    for (int64_t c = 0; c < n; ++c) {
        double s = 0.0;
        for (int32_t f = 0; f < d; ++f)
            s += x[c * d + f] * x[c * d + f];
        const double nrm = sqrt(s);
        if (nrm > best || (nrm == best && cells[c] < bestid)) {
            best = nrm;
            bestid = cells[c];
            star = c;
        }
    }
    double *u = malloc(sizeof(double) * d), *w = malloc(sizeof(double) * d);
    for (int32_t f = 0; f < d; ++f)
        u[f] = x[star * d + f];
    unit(u, d);
    for (int t = 0; t < 2; ++t) { /* u^(t+1) proportional to sum_c (x_c . u^(t)) x_c */
        for (int32_t f = 0; f < d; ++f)
            w[f] = 0.0;
        for (int64_t c = 0; c < n; ++c) {
            double p = 0.0;
            for (int32_t f = 0; f < d; ++f)
                p += x[c * d + f] * u[f];
            for (int32_t f = 0; f < d; ++f)
                w[f] += p * x[c * d + f];
        }
        for (int32_t f = 0; f < d; ++f)
            u[f] = w[f];
        unit(u, d);
    }
    /* sort by x_c . u^(2); the first ceil(n/2) go left */
    projected *proj = malloc(sizeof(projected) * n);
    for (int64_t c = 0; c < n; ++c) {
        double p = 0.0, m = 0.0;
        for (int32_t f = 0; f < d; ++f) {
            p += x[c * d + f] * u[f];
            m += fabs(x[c * d + f] * u[f]);
        }
        proj[c].val = p;
        proj[c].mag = m;
        proj[c].id = cells[c];
    }
    qsort(proj, (size_t)n, sizeof(projected), by_projection);
    const int64_t nl = (n + 1) / 2;
    if (min_gap) { /* the two projections that straddle the split, against their term sizes */
        const double m = fmax(proj[nl - 1].mag, proj[nl].mag);
        const double g = m > 0.0 ? fabs(proj[nl].val - proj[nl - 1].val) / m : 0.0;
        if (g < *min_gap)
            *min_gap = g;
    }
    int64_t *order = malloc(sizeof(int64_t) * n);
    for (int64_t c = 0; c < n; ++c)
        order[c] = proj[c].id;
    free(proj); free(w); free(u); free(x);
    const int64_t l = build_subtree(F, cfg, kbar, a, order, nl, min_gap);
    const int64_t r = build_subtree(F, cfg, kbar, a, order + nl, n - nl, min_gap);
    F->left[v] = l;
    F->right[v] = r;
    free(order);
    return v;
}

/* Eq. 21: a join node over nodes a_, b_ */
static int64_t join_nodes(forest *F, int64_t a_, int64_t b_)
{
    const int32_t d = F->d;
    const int64_t v = F->n++;
    const double na = (double)F->count[a_], nb = (double)F->count[b_];
    double *mu = F->mu + v * d;
    for (int32_t f = 0; f < d; ++f)
        mu[f] = (na * F->mu[a_ * d + f] + nb * F->mu[b_ * d + f]) / (na + nb);
    const double ra = F->rho[a_] + dist(F->mu + a_ * d, mu, d);
    const double rb = F->rho[b_] + dist(F->mu + b_ * d, mu, d);
    F->count[v] = F->count[a_] + F->count[b_];
    F->rho[v] = ra > rb ? ra : rb;
    F->A[v] = F->A[a_] > F->A[b_] ? F->A[a_] : F->A[b_];
    F->pmin[v] = F->pmin[a_] < F->pmin[b_] ? F->pmin[a_] : F->pmin[b_];
    F->minid[v] = F->minid[a_] < F->minid[b_] ? F->minid[a_] : F->minid[b_];
    F->cell[v] = -1;
    F->left[v] = a_;
    F->right[v] = b_;
    return v;
}

/* One forest over the admitted cells (ids in arrival order): chunk trees, then
 * the join chain from the smallest chunk upward.  Returns the root, or -1 when
 * M = 0. */
static int64_t build_forest(forest *F, const oracle_cfg *cfg, const double *kbar, const double *a,
                            const int64_t *cells, int64_t M, double *min_gap)
{
    if (M == 0)
        return -1;
    int64_t sizes[64], roots[64];
    const int32_t r = oracle_fsb_chunks(M, sizes);
    int64_t off = 0;
    for (int32_t t = 0; t < r; ++t) {
        roots[t] = build_subtree(F, cfg, kbar, a, cells + off, sizes[t], min_gap);
        off += sizes[t];
    }
    int64_t J = roots[r - 1]; /* J_r is the root of the smallest chunk */
    for (int32_t t = r - 2; t >= 0; --t)
        J = join_nodes(F, roots[t], J);
    return J;
}

int64_t oracle_fsb_forest(const oracle_cfg *cfg, const double *kbar, const double *a, const int64_t *cells,
                          int64_t M, int64_t cap, int64_t *count, int64_t *cell, int64_t *left, int64_t *right,
                          int64_t *minid, double *mu, double *rho, double *A, double *pmin, int64_t *n_nodes,
                          double *min_split_gap)
{
    forest F;
    forest_init(&F, cfg->d, 2 * M + 1);
    double gap = INFINITY;
    const int64_t root = build_forest(&F, cfg, kbar, a, cells, M, &gap);
    if (F.n > cap) {
        forest_free(&F);
        return -2;
    }
    const int32_t d = cfg->d;
    for (int64_t v = 0; v < F.n; ++v) {
        count[v] = F.count[v];
        cell[v] = F.cell[v];
        left[v] = F.left[v];
        right[v] = F.right[v];
        minid[v] = F.minid[v];
        rho[v] = F.rho[v];
        A[v] = F.A[v];
        pmin[v] = F.pmin[v];
        memcpy(mu + v * d, F.mu + v * d, sizeof(double) * d);
    }
    *n_nodes = F.n;
    if (min_split_gap)
        *min_split_gap = gap;
    forest_free(&F);
    return root;
}

/* ---- Eq. 11: node priority ---------------------------------------------------------- */

static double q_norm(const double *q, int32_t d)
{
    double s = 0.0;
    for (int32_t f = 0; f < d; ++f)
        s += q[f] * q[f];
    return sqrt(s);
}

static double node_priority(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const forest *F, int64_t v,
                            const double *q, int64_t i, double *mag)
{
    const int32_t d = F->d;
    double dot = 0.0, m = 0.0;
    for (int32_t f = 0; f < d; ++f) {
        dot += q[f] * F->mu[v * d + f];
        m += fabs(q[f] * F->mu[v * d + f]);
    }
    const double spread = fb->c * q_norm(q, d) * F->rho[v];
    const double g = erf(((double)i - F->pmin[v]) / (2.0 * cfg->sigma)); /* g_h(i - p_v^min) */
    if (mag)
        *mag = (m + spread) / sqrt((double)d) + cfg->lambda * F->A[v] * fabs(g);
    return (dot + spread) / sqrt((double)d) + cfg->lambda * F->A[v] * g;
}

double oracle_fsb_node_priority(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const double *q_i, int64_t i,
                                const double *mu, double rho, double A, double pmin)
{
    forest F;
    F.d = cfg->d;
    F.mu = (double *)mu;
    F.rho = &rho;
    F.A = &A;
    F.pmin = &pmin;
    return node_priority(cfg, fb, &F, 0, q_i, i, NULL);
}

/* ---- App. E.1: beam search ------------------------------------------------------ */

typedef struct {
    double U, mag;
    int64_t node, minid;
} beam_entry;

static int by_priority(const void *x, const void *y) /* U desc, then smaller minimum cell id */
{
    const beam_entry *p = (const beam_entry *)x, *q = (const beam_entry *)y;
    if (p->U > q->U) return -1;
    if (p->U < q->U) return 1;
    return (p->minid < q->minid) ? -1 : (p->minid > q->minid) ? 1 : 0;
}

/* The leaves reached from `root` (at most W^b cells) into out; returns their count.
 * min_gap receives the smallest gap, relative to the larger term size, between the
 * last child kept and the first child dropped at any level. */
static int64_t beam_search(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const forest *F, int64_t root,
                           const double *q, int64_t i, int64_t *out, double *min_gap)
{
    if (root < 0)
        return 0;
    const int64_t W = fb->Wb;
    beam_entry *beam = malloc(sizeof(beam_entry) * (size_t)(W > 0 ? W : 1));
    beam_entry *kids = malloc(sizeof(beam_entry) * (size_t)(2 * (W > 0 ? W : 1)));
    int64_t nb = 0;
    if (W > 0) {
        beam[0].node = root;
        beam[0].minid = F->minid[root];
        beam[0].U = node_priority(cfg, fb, F, root, q, i, &beam[0].mag);
        nb = 1;
    }
    for (;;) {
        int64_t n_leaf = 0, n_kid = 0, n_internal = 0;
        beam_entry *leaves = malloc(sizeof(beam_entry) * (size_t)(nb > 0 ? nb : 1));
        for (int64_t x = 0; x < nb; ++x) {
            const int64_t v = beam[x].node;
            if (F->cell[v] >= 0) {
                leaves[n_leaf++] = beam[x]; /* a leaf keeps its slot */
            } else {
                ++n_internal;
                const int64_t ch[2] = {F->left[v], F->right[v]};
                for (int e = 0; e < 2; ++e) {
                    kids[n_kid].node = ch[e];
                    kids[n_kid].minid = F->minid[ch[e]];
                    kids[n_kid].U = node_priority(cfg, fb, F, ch[e], q, i, &kids[n_kid].mag);
                    ++n_kid;
                }
            }
        }
        if (n_internal == 0) { /* every node of the beam is a leaf */
            for (int64_t x = 0; x < n_leaf; ++x)
                out[x] = F->cell[leaves[x].node];
            free(leaves);
            free(kids);
            free(beam);
            return n_leaf;
        }
        qsort(kids, (size_t)n_kid, sizeof(beam_entry), by_priority);
        int64_t keep = W - n_leaf; /* the remaining slots expand children */
        if (keep > n_kid)
            keep = n_kid;
        if (min_gap && keep < n_kid && keep > 0) {
            const double m = fmax(kids[keep - 1].mag, kids[keep].mag);
            const double g = m > 0.0 ? fabs(kids[keep - 1].U - kids[keep].U) / m : 0.0;
            if (g < *min_gap)
                *min_gap = g;
        }
        nb = 0;
        for (int64_t x = 0; x < n_leaf; ++x)
            beam[nb++] = leaves[x];
        for (int64_t x = 0; x < keep; ++x)
            beam[nb++] = kids[x];
        free(leaves);
    }
}

/* ---- Eq. 12: token-level rerank --------------------------------------------------- */

double oracle_fsb_rerank_score(const oracle_cfg *cfg, const double *q_i, const double *k, double a_c, int64_t i,
                               int64_t c, double *mag)
{
    const int32_t d = cfg->d, s = cfg->s;
    double mx = -INFINITY, mmax = 0.0;
    double *l = malloc(sizeof(double) * s);
    for (int32_t t = 0; t < s; ++t) {
        const int64_t j = c * s + t;
        double dot = 0.0, m = 0.0;
        for (int32_t f = 0; f < d; ++f) {
            dot += q_i[f] * k[j * d + f];
            m += fabs(q_i[f] * k[j * d + f]);
        }
        l[t] = dot / sqrt((double)d);
        if (l[t] > mx)
            mx = l[t];
        if (m / sqrt((double)d) > mmax)
            mmax = m / sqrt((double)d);
    }
    double z = 0.0;
    for (int32_t t = 0; t < s; ++t)
        z += exp(l[t] - mx);
    free(l);
    const double p_c = ((double)c + 0.5) * s;
    const double g = erf(((double)i - p_c) / (2.0 * cfg->sigma));
    if (mag)
        *mag = mmax + cfg->lambda * a_c * fabs(g);
    return mx + log(z) + cfg->lambda * a_c * g; /* log sum_j exp(l_j) + lambda a_c g_h(i - p_c) */
}

/* ---- the whole FS-B branch for one (sequence, head) ---------------------------------- */

int oracle_fsb_head(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const double *q, const double *k,
                    const double *v, const double *g, int64_t i_lo, int64_t i_hi, int32_t *sel, int32_t *cand,
                    int32_t *n_cand, double *gap_beam, double *gap_rerank, double *gap_split, double *out)
{
    if (cfg->N < 0 || cfg->d <= 0 || cfg->s <= 0 || cfg->B <= 0 || cfg->B % cfg->s != 0 || cfg->K < 1 ||
        cfg->sigma <= 0.0 || cfg->lambda < 0.0 || cfg->eps < 0.0 || fb->Wb < 0 || fb->c < 0.0 ||
        i_lo < 0 || i_hi > cfg->N || i_lo > i_hi)
        return -1;
    const int32_t d = cfg->d, K = cfg->K;
    const int64_t Mall = cfg->N / cfg->s;
    const int64_t Wb = fb->Wb;
    double *kbar = malloc(sizeof(double) * (size_t)(Mall > 0 ? Mall : 1) * d);
    double *a = malloc(sizeof(double) * (size_t)(Mall > 0 ? Mall : 1));
    oracle_cell_summaries(cfg, k, kbar, a);
    int64_t *all = malloc(sizeof(int64_t) * (size_t)(Mall > 0 ? Mall : 1));
    int64_t *hi = malloc(sizeof(int64_t) * (size_t)(Mall > 0 ? Mall : 1));
    int64_t *B0 = malloc(sizeof(int64_t) * (size_t)(Wb > 0 ? Wb : 1));
    int64_t *Bt = malloc(sizeof(int64_t) * (size_t)(Wb > 0 ? Wb : 1));
    keyed2 *rank = malloc(sizeof(keyed2) * (size_t)(2 * Wb > 0 ? 2 * Wb : 1));
    double *rmag = malloc(sizeof(double) * (size_t)(2 * Wb > 0 ? 2 * Wb : 1));
    int64_t *T = malloc(sizeof(int64_t) * (size_t)K);
    forest F0, Ft;
    forest_init(&F0, d, 2 * Mall + 1);
    forest_init(&Ft, d, 2 * Mall + 1);
    int64_t cur_block = -1, root0 = -1, roott = -1;
    double split_gap = INFINITY;

    for (int64_t i = i_lo; i < i_hi; ++i) {
        const int64_t blk = i / cfg->B;
        if (blk != cur_block) { /* both forests are fixed within a query block */
            cur_block = blk;
            const int64_t n_avail = oracle_available_count((int64_t)cfg->B * blk, cfg->s);
            int64_t M0 = 0, Mt = 0;
            for (int64_t c = 0; c < n_avail; ++c) { /* Eq. 10, arrival order */
                all[M0++] = c;
                if (a[c] >= fb->tau)
                    hi[Mt++] = c;
            }
            F0.n = Ft.n = 0;
            split_gap = INFINITY;
            root0 = build_forest(&F0, cfg, kbar, a, all, M0, &split_gap);
            roott = build_forest(&Ft, cfg, kbar, a, hi, Mt, &split_gap);
        }
        const double *q_i = q + i * d;
        const int64_t row = i - i_lo;
        double gb = INFINITY;
        const int64_t n0 = beam_search(cfg, fb, &F0, root0, q_i, i, B0, &gb);
        const int64_t nt = beam_search(cfg, fb, &Ft, roott, q_i, i, Bt, &gb);
        /* B_i = B^0 u B^tau, deduplicated */
        int64_t nc = 0;
        for (int64_t x = 0; x < n0 + nt; ++x) {
            const int64_t c = x < n0 ? B0[x] : Bt[x - n0];
            int dup = 0;
            for (int64_t y = 0; y < nc; ++y)
                dup |= rank[y].id == c;
            if (!dup) {
                rank[nc].id = c;
                rank[nc].val = oracle_fsb_rerank_score(cfg, q_i, k, a[c], i, c, &rmag[nc]);
                ++nc;
            }
        }
        if (cand) { /* B_i in ascending id order */
            for (int64_t x = 0; x < 2 * Wb; ++x)
                cand[row * 2 * Wb + x] = -1;
            for (int64_t x = 0; x < nc; ++x) {
                int64_t pos = 0;
                for (int64_t y = 0; y < nc; ++y)
                    pos += rank[y].id < rank[x].id;
                cand[row * 2 * Wb + pos] = (int32_t)rank[x].id;
            }
        }
        if (n_cand)
            n_cand[row] = (int32_t)nc;
        /* sort candidates by (reranked score desc, id asc); keep the magnitudes aligned */
        for (int64_t x = 1; x < nc; ++x) {
            keyed2 kv = rank[x];
            double mv = rmag[x];
            int64_t y = x - 1;
            while (y >= 0 && (rank[y].val < kv.val || (rank[y].val == kv.val && rank[y].id > kv.id))) {
                rank[y + 1] = rank[y];
                rmag[y + 1] = rmag[y];
                --y;
            }
            rank[y + 1] = kv;
            rmag[y + 1] = mv;
        }
        const int64_t nT = nc < K ? nc : K;
        for (int64_t t = 0; t < nT; ++t)
            T[t] = rank[t].id;
        if (sel)
            for (int32_t t = 0; t < K; ++t)
                sel[row * K + t] = t < nT ? (int32_t)T[t] : -1;
        if (gap_beam)
            gap_beam[row] = gb;
        if (gap_rerank) { /* adjacent scores among the K + 1 best decide the ordered selection */
            gap_rerank[row] = INFINITY;
            for (int64_t t = 0; t < K && t + 1 < nc; ++t) {
                const double m = fmax(rmag[t], rmag[t + 1]);
                const double gp = m > 0.0 ? fabs(rank[t].val - rank[t + 1].val) / m : 0.0;
                if (gp < gap_rerank[row])
                    gap_rerank[row] = gp;
            }
        }
        if (gap_split)
            gap_split[row] = split_gap;
        if (out)
            oracle_readout(cfg, q_i, k, v, g, T, nT, out + row * d);
    }
    forest_free(&Ft);
    forest_free(&F0);
    free(T); free(rmag); free(rank); free(Bt); free(B0); free(hi); free(all); free(a); free(kbar);
    return 0;
}
