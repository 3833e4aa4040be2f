/*
 * fp64 CPU oracle of FreeSolo's long-range branch (FS and FS-L).
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU library, with which it shares
 * no code.  Plain loops, plain definitions, no blocking or reordering: each
 * step is written so that it can be checked against the page by eye.
 *
 * Page: "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 * Extrapolation" (arXiv 2610.17191).
 *   Sec. 3.3 "Cells"                 Eq. 5  summaries kbar_c, p_c, a_c
 *   Sec. 3.3 "Query blocks"                 b_i = B floor(i / B)
 *   Sec. 3.3 "Causal availability"   Eq. 6  C_i = {c : (c+1) s <= b_i}
 *   Sec. 3.3 "Cell scoring"          Eq. 7  r_ic
 *   Sec. 3.3 "Query-independent pruning" Eq. 8  A_i = Recent_W u TopP
 *   Sec. 3.3 "Per-query selection"          T_i, S_i
 *   Sec. 3.3 "Token readout"         Eq. 9  softmax readout + RMSNorm
 *   Sec. 2 "Attention"               Eq. 1  softmax readout
 *   App. D.2 "Why sparse readout..." Eq. 17 RMSNorm with epsilon
 *
 * Readings where the page leaves a choice open:
 *   - ties in TopP and top-K are broken by the smaller cell id (the page asks
 *     only for "a common deterministic tie rule", App. C "Bounded cache");
 *   - Recent_W(C) is the min(W, |C|) cells of C with the largest ids;
 *   - only complete cells (N / s of them, rounded down) have summaries;
 *   - RMSNorm adds epsilon to the mean square inside the square root, with a
 *     per-feature gain g (unit gain when g is NULL).
 */
#include "fsl_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- Eq. 5: cell summaries ------------------------------------------------ */

void oracle_cell_summaries(const oracle_cfg *cfg, const double *k, double *kbar, double *a)
{
    const int64_t M = cfg->N / cfg->s; /* complete cells only */
    const int32_t d = cfg->d, s = cfg->s;
    for (int64_t c = 0; c < M; ++c) {
        /* mean key over I_c = {cs, ..., (c+1)s - 1}, summed in index order */
        for (int32_t f = 0; f < d; ++f) {
            double sum = 0.0;
            for (int64_t j = c * s; j < (c + 1) * s; ++j)
                sum += k[j * d + f];
            if (kbar)
                kbar[c * d + f] = sum / s;
        }
        /* largest L2 norm of a key in the cell */
        double best = 0.0;
        for (int64_t j = c * s; j < (c + 1) * s; ++j) {
            double sq = 0.0;
            for (int32_t f = 0; f < d; ++f)
                sq += k[j * d + f] * k[j * d + f];
            const double nrm = sqrt(sq);
            if (j == c * s || nrm > best)
                best = nrm;
        }
        if (a)
            a[c] = best;
    }
}

/* ---- Eq. 6: causal availability ------------------------------------------- */

int64_t oracle_available_count(int64_t b_start, int32_t s)
{
    int64_t n = 0;
    while ((n + 1) * (int64_t)s <= b_start) /* cell n is available iff (n+1)s <= b_i */
        ++n;
    return n;
}

/* ---- ordering helpers: value descending, then id ascending ---------------- */

typedef struct {
    double val;
    int64_t id;
} keyed;

static int by_value_desc_id_asc(const void *x, const void *y)
{
    const keyed *p = (const keyed *)x, *q = (const keyed *)y;
    if (p->val > q->val) return -1;
    if (p->val < q->val) return 1;
    return (p->id < q->id) ? -1 : (p->id > q->id) ? 1 : 0;
}

static double relative_gap(double x, double y)
{
    const double m = fmax(fabs(x), fabs(y));
    return m > 0.0 ? fabs(x - y) / m : 0.0;
}

/* ---- Eq. 8: retained set of one query block -------------------------------- */

int64_t oracle_retained(const oracle_cfg *cfg, int64_t n_avail, const double *a,
                        int32_t *A_out, double *gap_p)
{
    if (gap_p)
        *gap_p = INFINITY;
    if (!cfg->prune) { /* FS: A_i = C_i */
        for (int64_t c = 0; c < n_avail; ++c)
            A_out[c] = (int32_t)c;
        return n_avail;
    }
    char *keep = (char *)calloc((size_t)(n_avail > 0 ? n_avail : 1), 1);
    keyed *order = (keyed *)malloc(sizeof(keyed) * (size_t)(n_avail > 0 ? n_avail : 1));
    /* TopP: the P cells of C with the largest a_c */
    for (int64_t c = 0; c < n_avail; ++c) {
        order[c].val = a[c];
        order[c].id = c;
    }
    qsort(order, (size_t)n_avail, sizeof(keyed), by_value_desc_id_asc);
    const int64_t n_top = n_avail < cfg->P ? n_avail : cfg->P;
    for (int64_t r = 0; r < n_top; ++r)
        keep[order[r].id] = 1;
    if (gap_p && cfg->P > 0 && n_avail > cfg->P)
        *gap_p = relative_gap(order[cfg->P - 1].val, order[cfg->P].val);
    /* Recent_W: the W most recent cells of C */
    const int64_t n_recent = n_avail < cfg->W ? n_avail : cfg->W;
    for (int64_t c = n_avail - n_recent; c < n_avail; ++c)
        keep[c] = 1;
    /* the union, ascending */
    int64_t n = 0;
    for (int64_t c = 0; c < n_avail; ++c)
        if (keep[c])
            A_out[n++] = (int32_t)c;
    free(order);
    free(keep);
    return n;
}

/* ---- Eq. 7: cell score ------------------------------------------------------ */

/* g_h(i - p_c) of the prior */
static double prior_gate(const oracle_cfg *cfg, int64_t i, int64_t c)
{
    const double p_c = ((double)c + 0.5) * cfg->s;        /* cell centre, Eq. 5 */
    return erf(((double)i - p_c) / (2.0 * cfg->sigma));
}

double oracle_cell_score(const oracle_cfg *cfg, const double *q_i, const double *kbar_c,
                         double a_c, int64_t i, int64_t c)
{
    double dot = 0.0;
    for (int32_t f = 0; f < cfg->d; ++f)
        dot += q_i[f] * kbar_c[f];
    const double g = prior_gate(cfg, i, c);
    return dot / sqrt((double)cfg->d) + cfg->lambda * a_c * g;
}

/* The size of the terms r_ic is summed from: sum_f |q_if kbar_cf| / sqrt(d) +
 * lambda a_c |g|.  A floating-point evaluation of Eq. 7 is exact to a few roundings
 * of this size, not of |r_ic| (the content term can cancel), so the near-tie gap of
 * two scores is measured against it. */
double oracle_cell_score_mag(const oracle_cfg *cfg, const double *q_i, const double *kbar_c,
                             double a_c, int64_t i, int64_t c)
{
    double sum = 0.0;
    for (int32_t f = 0; f < cfg->d; ++f)
        sum += fabs(q_i[f] * kbar_c[f]);
    return sum / sqrt((double)cfg->d) + cfg->lambda * a_c * fabs(prior_gate(cfg, i, c));
}

/* ---- Eq. 9 / Eq. 1 / Eq. 17: token readout and RMSNorm --------------------- */

void oracle_readout(const oracle_cfg *cfg, const double *q_i, const double *k, const double *v,
                    const double *g, const int64_t *T, int64_t nT, double *o)
{
    const int32_t d = cfg->d, s = cfg->s;
    if (nT == 0) { /* S_i empty: both u and o are zero */
        for (int32_t f = 0; f < d; ++f)
            o[f] = 0.0;
        return;
    }
    const int64_t nS = nT * s;
    double *logit = (double *)malloc(sizeof(double) * (size_t)nS);
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)nS);
    /* S_i: the tokens of the selected cells */
    int64_t n = 0;
    for (int64_t t = 0; t < nT; ++t)
        for (int64_t j = T[t] * s; j < (T[t] + 1) * s; ++j)
            tok[n++] = j;
    /* l_ij = q_i . k_j / sqrt(d), NoPE */
    double mx = -INFINITY;
    for (int64_t x = 0; x < nS; ++x) {
        double dot = 0.0;
        for (int32_t f = 0; f < d; ++f)
            dot += q_i[f] * k[tok[x] * d + f];
        logit[x] = dot / sqrt((double)d);
        if (logit[x] > mx)
            mx = logit[x];
    }
    /* softmax over S_i jointly, then u = sum p_j v_j */
    double z = 0.0;
    for (int64_t x = 0; x < nS; ++x) {
        logit[x] = exp(logit[x] - mx);
        z += logit[x];
    }
    double ms = 0.0;
    for (int32_t f = 0; f < d; ++f) {
        double u = 0.0;
        for (int64_t x = 0; x < nS; ++x)
            u += logit[x] * v[tok[x] * d + f];
        u /= z;
        o[f] = u;
        ms += u * u;
    }
    /* RMSNorm over the d features */
    ms /= d;
    const double inv = 1.0 / sqrt(ms + cfg->eps);
    for (int32_t f = 0; f < d; ++f)
        o[f] = (g ? g[f] : 1.0) * o[f] * inv;
    free(tok);
    free(logit);
}

/* ---- readout backward (Sec. 3.3 "Training"; App. D.4) ----------------------- */
/*
 * Gradients of the loss through o_i = g (.) u r, r = 1 / sqrt(|u|^2 / d + eps),
 * u = sum_j p_j v_j, p = softmax_j(l_j), l_j = q_i . k_j / sqrt(d) over the tokens
 * j of a fixed selection T (no gradient through the selection), given
 * dout = dL/do_i:
 *   dL/du     = r (g (.) dout) - (r^3 / d) (sum_f g_f dout_f u_f) u
 *   dL/dg    += r dout (.) u
 *   dL/dv_j  += p_j dL/du
 *   dL/dl_j   = p_j (dL/du . v_j - sum_j' p_j' dL/du . v_j')
 *   dL/dq     = sum_j dL/dl_j k_j / sqrt(d),   dL/dk_j += dL/dl_j q_i / sqrt(d).
 *
 * The *_abs outputs (each may be NULL) receive a first-order error scale of the
 * same results: every quantity x carries a size xa, the sum of the absolute
 * values of its own terms where each factor's error is scaled by the size of
 * that factor (for a product a b: aa |b| + |a| ba; for a sum: the sum of the
 * sizes).  The inputs are exact and the softmax weights p_j are taken as known to
 * a relative e (size p_j).  A computation whose products and sums after the
 * softmax round to a relative e then differs from these results by a small
 * multiple of e times the size, also where u, r or the softmax mean cancel.
 */
void oracle_readout_backward(const oracle_cfg *cfg, const double *q_i, const double *k, const double *v,
                             const double *g, const int64_t *T, int64_t nT, const double *dout, double *dq,
                             double *dk, double *dv, double *dg, double *dq_abs, double *dk_abs, double *dv_abs,
                             double *dg_abs)
{
    const int32_t d = cfg->d, s = cfg->s;
    for (int32_t f = 0; f < d; ++f) {
        dq[f] = 0.0;
        if (dq_abs)
            dq_abs[f] = 0.0;
    }
    if (nT == 0) /* o is identically zero: no gradient */
        return;
    const int64_t nS = nT * s;
    const double sd = sqrt((double)d);
    int64_t *tok = malloc(sizeof(int64_t) * nS);
    double *p = malloc(sizeof(double) * nS), *pa = malloc(sizeof(double) * nS);
    double *dl = malloc(sizeof(double) * nS), *dla = malloc(sizeof(double) * nS);
    double *u = malloc(sizeof(double) * d), *ua = malloc(sizeof(double) * d);
    double *du = malloc(sizeof(double) * d), *dua = malloc(sizeof(double) * d);
    int64_t n = 0;
    for (int64_t t = 0; t < nT; ++t)
        for (int32_t x = 0; x < s; ++x)
            tok[n++] = T[t] * s + x;
    /* forward: logits, softmax, u, r */
    double mx = -INFINITY;
    for (int64_t x = 0; x < nS; ++x) {
        double dot = 0.0;
        for (int32_t f = 0; f < d; ++f)
            dot += q_i[f] * k[tok[x] * d + f];
        p[x] = dot / sd;
        if (p[x] > mx)
            mx = p[x];
    }
    double z = 0.0;
    for (int64_t x = 0; x < nS; ++x) {
        p[x] = exp(p[x] - mx);
        z += p[x];
    }
    for (int64_t x = 0; x < nS; ++x) {
        p[x] /= z;
        pa[x] = p[x];
    }
    double ms = 0.0, msa = 0.0;
    for (int32_t f = 0; f < d; ++f) {
        u[f] = 0.0;
        ua[f] = 0.0;
        for (int64_t x = 0; x < nS; ++x) {
            u[f] += p[x] * v[tok[x] * d + f];
            ua[f] += pa[x] * fabs(v[tok[x] * d + f]);
        }
        ms += u[f] * u[f];
        msa += 2.0 * fabs(u[f]) * ua[f];
    }
    const double r = 1.0 / sqrt(ms / d + cfg->eps);
    const double ra = r + r * r * r * (msa / d) / 2.0;
    const double c3 = r * r * r / d, c3a = 3.0 * r * r * ra / d;
    /* RMSNorm backward */
    double sgu = 0.0, sgua = 0.0;
    for (int32_t f = 0; f < d; ++f) {
        const double gf = g ? g[f] : 1.0;
        sgu += gf * dout[f] * u[f];
        sgua += fabs(gf * dout[f]) * ua[f];
    }
    for (int32_t f = 0; f < d; ++f) {
        const double gf = g ? g[f] : 1.0;
        du[f] = r * gf * dout[f] - r * r * r / d * sgu * u[f];
        dua[f] = ra * fabs(gf * dout[f]) + c3a * fabs(sgu * u[f]) + c3 * (sgua * fabs(u[f]) + fabs(sgu) * ua[f]);
        if (dg)
            dg[f] += r * dout[f] * u[f];
        if (dg_abs)
            dg_abs[f] += ra * fabs(dout[f] * u[f]) + r * fabs(dout[f]) * ua[f];
    }
    /* softmax and value backward */
    double delta = 0.0, deltaa = 0.0;
    for (int64_t x = 0; x < nS; ++x) {
        double dp = 0.0, dpa = 0.0;
        for (int32_t f = 0; f < d; ++f) {
            dp += du[f] * v[tok[x] * d + f];
            dpa += dua[f] * fabs(v[tok[x] * d + f]);
        }
        dl[x] = dp; /* dL/dp_j and its size for now */
        dla[x] = dpa;
        delta += p[x] * dp;
        deltaa += pa[x] * fabs(dp) + p[x] * dpa;
        for (int32_t f = 0; f < d; ++f) {
            if (dv)
                dv[tok[x] * d + f] += p[x] * du[f];
            if (dv_abs)
                dv_abs[tok[x] * d + f] += pa[x] * fabs(du[f]) + p[x] * dua[f];
        }
    }
    for (int64_t x = 0; x < nS; ++x) {
        dla[x] = pa[x] * fabs(dl[x] - delta) + p[x] * (dla[x] + deltaa);
        dl[x] = p[x] * (dl[x] - delta);
    }
    /* logits backward */
    for (int64_t x = 0; x < nS; ++x) {
        for (int32_t f = 0; f < d; ++f) {
            dq[f] += dl[x] * k[tok[x] * d + f] / sd;
            if (dq_abs)
                dq_abs[f] += dla[x] * fabs(k[tok[x] * d + f]) / sd;
            if (dk)
                dk[tok[x] * d + f] += dl[x] * q_i[f] / sd;
            if (dk_abs)
                dk_abs[tok[x] * d + f] += dla[x] * fabs(q_i[f]) / sd;
        }
    }
    free(dua); free(du); free(ua); free(u); free(dla); free(dl); free(pa); free(p); free(tok);
}

int oracle_backward_head(const oracle_cfg *cfg, const double *q, const double *k, const double *v, const double *g,
                         const int32_t *sel, const double *dout, int64_t i_lo, int64_t i_hi, double *dq, double *dk,
                         double *dv, double *dg, double *dq_abs, double *dk_abs, double *dv_abs, double *dg_abs)
{
    if (cfg->d <= 0 || cfg->s <= 0 || cfg->K < 1 || i_lo < 0 || i_hi > cfg->N || i_lo > i_hi || cfg->eps < 0.0)
        return -1;
    const int32_t d = cfg->d, K = cfg->K;
    const int64_t M = cfg->N / cfg->s;
    int64_t *T = malloc(sizeof(int64_t) * K);
    for (int64_t i = i_lo; i < i_hi; ++i) {
        const int64_t row = i - i_lo;
        int64_t nT = 0;
        for (int32_t t = 0; t < K; ++t) {
            const int32_t c = sel[row * K + t];
            if (c >= 0) {
                if (c >= M) {
                    free(T);
                    return -1;
                }
                T[nT++] = c;
            }
        }
        oracle_readout_backward(cfg, q + i * d, k, v, g, T, nT, dout + row * d, dq + row * d, dk, dv, dg,
                                dq_abs ? dq_abs + row * d : NULL, dk_abs, dv_abs, dg_abs);
    }
    free(T);
    return 0;
}

/* ---- the whole branch for one (sequence, head) ------------------------------ */

int oracle_head(const oracle_cfg *cfg, const double *q, const double *k, const double *v,
                const double *g, int64_t i_lo, int64_t i_hi, int64_t cap,
                double *kbar, double *a, int32_t *retained, int32_t *n_ret, double *gap_p,
                int32_t *sel, double *gap_k, double *out, double *scores)
{
    if (cfg->N < 0 || cfg->d <= 0 || cfg->s <= 0 || cfg->B <= 0 || cfg->B % cfg->s != 0 ||
        cfg->K < 1 || cfg->P < 0 || cfg->W < 0 || cfg->sigma <= 0.0 || cfg->lambda < 0.0 ||
        cfg->eps < 0.0 || i_lo < 0 || i_hi > cfg->N || i_lo > i_hi)
        return -1;
    const int32_t d = cfg->d, K = cfg->K;
    const int64_t M = cfg->N / cfg->s;
    double *kb = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1) * d);
    double *an = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    oracle_cell_summaries(cfg, k, kb, an);
    if (kbar)
        memcpy(kbar, kb, sizeof(double) * (size_t)M * d);
    if (a)
        memcpy(a, an, sizeof(double) * (size_t)M);

    int32_t *A = (int32_t *)malloc(sizeof(int32_t) * (size_t)(M > 0 ? M : 1));
    keyed *rank = (keyed *)malloc(sizeof(keyed) * (size_t)(M > 0 ? M : 1));
    int64_t *T = (int64_t *)malloc(sizeof(int64_t) * (size_t)K);
    int status = 0;
    int64_t cur_block = -1, nA = 0;

    for (int64_t i = i_lo; i < i_hi; ++i) {
        const int64_t blk = i / cfg->B;
        if (blk != cur_block) { /* the prefix and retained set are fixed within a block */
            cur_block = blk;
            const int64_t b_i = (int64_t)cfg->B * blk;
            const int64_t n_avail = oracle_available_count(b_i, cfg->s);
            double gp;
            nA = oracle_retained(cfg, n_avail, an, A, &gp);
            if (nA > cap) {
                status = -1;
                break;
            }
            if (retained) {
                for (int64_t x = 0; x < cap; ++x)
                    retained[blk * cap + x] = x < nA ? A[x] : -1;
            }
            if (n_ret)
                n_ret[blk] = (int32_t)nA;
            if (gap_p)
                gap_p[blk] = gp;
        }
        const double *q_i = q + i * d;
        const int64_t row = i - i_lo;
        /* Eq. 7 over the retained cells */
        for (int64_t x = 0; x < nA; ++x) {
            rank[x].id = A[x];
            rank[x].val = oracle_cell_score(cfg, q_i, kb + (int64_t)A[x] * d, an[A[x]], i, A[x]);
            if (scores)
                scores[row * cap + x] = rank[x].val;
        }
        if (scores)
            for (int64_t x = nA; x < cap; ++x)
                scores[row * cap + x] = NAN;
        /* T_i: the min(K, |A_i|) best cells */
        qsort(rank, (size_t)nA, sizeof(keyed), by_value_desc_id_asc);
        const int64_t nT = nA < K ? nA : K;
        for (int64_t t = 0; t < nT; ++t)
            T[t] = rank[t].id;
        if (sel)
            for (int32_t t = 0; t < K; ++t)
                sel[row * K + t] = t < nT ? (int32_t)T[t] : -1;
        if (gap_k) { /* adjacent scores among the K + 1 best decide the ordered selection */
            gap_k[row] = INFINITY;
            for (int64_t t = 0; t < K && t + 1 < nA; ++t) { /* |r_t - r_t+1| against their term sizes */
                const double m1 = oracle_cell_score_mag(cfg, q_i, kb + rank[t].id * d, an[rank[t].id], i,
                                                        rank[t].id);
                const double m2 = oracle_cell_score_mag(cfg, q_i, kb + rank[t + 1].id * d, an[rank[t + 1].id], i,
                                                        rank[t + 1].id);
                const double m = fmax(m1, m2);
                const double gp = m > 0.0 ? fabs(rank[t].val - rank[t + 1].val) / m : 0.0;
                if (gp < gap_k[row])
                    gap_k[row] = gp;
            }
        }
        if (out)
            oracle_readout(cfg, q_i, k, v, g, T, nT, out + row * d);
    }
    free(T);
    free(rank);
    free(A);
    free(an);
    free(kb);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Local branch, Sec. 3.2 Eqs. 3-4, and Eq. 2.                              */

/* x turned by R(p): pair (2m, 2m+1) by the angle p * theta_m (Su et al., RoFormer). */
static void rope_rotate(const double *x, int32_t d, double p, double rope_base, double *y)
{
    for (int32_t m = 0; m < d / 2; ++m) {
        const double theta = pow(rope_base, -2.0 * m / d);
        const double c = cos(p * theta), sn = sin(p * theta);
        y[2 * m] = x[2 * m] * c - x[2 * m + 1] * sn;
        y[2 * m + 1] = x[2 * m] * sn + x[2 * m + 1] * c;
    }
}

int oracle_local(int64_t N, int32_t d, int64_t w, double rope_base, const double *q, const double *k,
                 const double *v, double alpha, const double *o_lr, int64_t i_lo, int64_t i_hi, double *out)
{
    if (d <= 0 || (d & 1) || w < 0 || !(rope_base > 0.0) || i_lo < 0 || i_hi > N || i_lo > i_hi)
        return -1;
    /* R(j) k_j for every key the queries can reach, once */
    const int64_t j0 = i_lo - w > 0 ? i_lo - w : 0;
    const int64_t nk = i_hi - j0;
    double *kr = malloc((size_t)(nk > 0 ? nk : 1) * d * sizeof(double));
    double *qr = malloc((size_t)d * sizeof(double));
    double *logit = malloc((size_t)(w + 1) * sizeof(double));
    if (!kr || !qr || !logit) {
        free(kr); free(qr); free(logit);
        return -1;
    }
    for (int64_t j = j0; j < i_hi; ++j)
        rope_rotate(k + j * d, d, (double)j, rope_base, kr + (j - j0) * d);
    for (int64_t i = i_lo; i < i_hi; ++i) {
        rope_rotate(q + i * d, d, (double)i, rope_base, qr);
        const int64_t lo = i - w > 0 ? i - w : 0; /* L_i = [lo, i] */
        double mx = -INFINITY;
        for (int64_t j = lo; j <= i; ++j) {
            double dot = 0.0;
            for (int32_t f = 0; f < d; ++f)
                dot += qr[f] * kr[(j - j0) * d + f];
            logit[j - lo] = dot / sqrt((double)d);
            if (logit[j - lo] > mx)
                mx = logit[j - lo];
        }
        double z = 0.0;
        for (int64_t j = lo; j <= i; ++j) {
            logit[j - lo] = exp(logit[j - lo] - mx);
            z += logit[j - lo];
        }
        double *o = out + (i - i_lo) * d;
        for (int32_t f = 0; f < d; ++f) {
            double u = 0.0;
            for (int64_t j = lo; j <= i; ++j)
                u += logit[j - lo] * v[j * d + f];
            o[f] = u / z + (o_lr ? alpha * o_lr[(i - i_lo) * d + f] : 0.0);
        }
    }
    free(logit);
    free(qr);
    free(kr);
    return 0;
}
