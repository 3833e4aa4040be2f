/*
 * fp64 CPU oracle of FreeSolo's long-range branch (FS and FS-L).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the GPU library.
 *
 * Source: "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 * Extrapolation" (arXiv 2610.17191), Sec. 3.3 (Eqs. 5-9), Sec. 2 (Eq. 1) and
 * App. D.2 (Eq. 17); the local branch of Sec. 3.2 (Eqs. 3-4) and the branch
 * combination of Sec. 3.1 (Eq. 2).  Every array is fp64 and row-major; one call handles one
 * (sequence, head) pair.
 */
#ifndef FSL_ORACLE_H
#define FSL_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t N;      /* tokens in the sequence */
    int32_t d;      /* head dimension */
    int32_t s;      /* cell size (tokens per cell) */
    int32_t B;      /* query-block size, a multiple of s */
    int32_t P;      /* FS-L: cells kept by largest key norm */
    int32_t W;      /* FS-L: most recent cells kept */
    int32_t K;      /* cells selected per query */
    int32_t prune;  /* 1 = FS-L (Eq. 8), 0 = FS (A_i = C_i) */
    double sigma;   /* sigma_h of the erf prior */
    double lambda;  /* lambda_h of the erf prior */
    double eps;     /* RMSNorm epsilon */
} oracle_cfg;

/* Eq. 5: mean key kbar[c] and largest key norm a[c] of every complete cell. */
void oracle_cell_summaries(const oracle_cfg *cfg, const double *k, double *kbar, double *a);

/* Eq. 6: number of cells available to a query whose block starts at b_start. */
int64_t oracle_available_count(int64_t b_start, int32_t s);

/* Eq. 8 (FS-L) or A = C (FS) for one block; ids ascending; returns |A|.
 * gap_p (may be NULL) receives the relative gap between the P-th and (P+1)-th
 * key norms of the block's prefix, or +inf when there is no such boundary. */
int64_t oracle_retained(const oracle_cfg *cfg, int64_t n_avail, const double *a,
                        int32_t *A_out, double *gap_p);

/* Eq. 7: routing score of cell c for query position i. */
double oracle_cell_score(const oracle_cfg *cfg, const double *q_i, const double *kbar_c,
                         double a_c, int64_t i, int64_t c);

/* The size of the terms Eq. 7 sums for (query i, cell c):
 * sum_f |q_if kbar_cf| / sqrt(d) + lambda a_c |erf((i - p_c) / (2 sigma))|.
 * Floating-point scores are exact to a few roundings of this size; near-tie
 * gaps of scores are measured against it. */
double oracle_cell_score_mag(const oracle_cfg *cfg, const double *q_i, const double *kbar_c,
                             double a_c, int64_t i, int64_t c);

/* Eq. 9 with Eq. 17 for one query and a given selection T[0..nT) of cell ids:
 * the joint softmax over the tokens of those cells (NoPE logits q_i . k_j /
 * sqrt(d)), then RMSNorm with gain g (unit gains when g is NULL); o = 0 when
 * nT = 0.  k, v [N, d] hold every token the cells cover; o [d]. */
void oracle_readout(const oracle_cfg *cfg, const double *q_i, const double *k, const double *v,
                    const double *g, const int64_t *T, int64_t nT, double *o);

/*
 * The whole branch for one (sequence, head), for queries i in [i_lo, i_hi).
 *   q, k, v  [N, d];  g [d] or NULL (unit gains)
 *   kbar [N/s, d], a [N/s]                      cell summaries (optional)
 *   retained [NB, cap] (-1 padded), n_ret [NB], gap_p [NB]   per query block
 *       touched by [i_lo, i_hi), indexed by absolute block (optional)
 *   sel [(i_hi-i_lo), K] selected cells (-1 padded), in (score desc, id asc)
 *   gap_k [(i_hi-i_lo)] smallest gap of adjacent scores among the K + 1 best
 *       (the order of the selection and its boundary), each relative to the
 *       larger of the two scores' term sizes (oracle_cell_score_mag), or +inf
 *   out [(i_hi-i_lo), d] long-range output after RMSNorm
 *   scores [(i_hi-i_lo), cap] scores of the retained cells in ascending id
 *       order (optional; NaN padded)
 * cap is the row length of retained/scores: at least |A| of every block.
 * Returns 0, or -1 when cap is too small or an argument is invalid.
 */
int oracle_head(const oracle_cfg *cfg, const double *q, const double *k, const double *v,
                const double *g, int64_t i_lo, int64_t i_hi, int64_t cap,
                double *kbar, double *a, int32_t *retained, int32_t *n_ret, double *gap_p,
                int32_t *sel, double *gap_k, double *out, double *scores);

/*
 * Local branch (Sec. 3.2, Eqs. 3-4) and the branch combination (Sec. 3.1,
 * Eq. 2) for one (sequence, head), queries i in [i_lo, i_hi):
 *   L_i   = {j : 0 <= j <= i, i - j <= w}   (a full window holds w + 1 tokens)
 *   l_ij  = (R(i) q_i) . (R(j) k_j) / sqrt(d), R(p) the RoPE rotation at
 *           position p (Su et al.): feature pair (2m, 2m+1) turned by the angle
 *           p * theta_m, theta_m = rope_base^(-2m/d)
 *   o_sr  = softmax_{j in L_i}(l_ij) V_{L_i}
 *   out_i = o_sr_i + alpha * o_lr_i, or o_sr_i when o_lr is NULL.
 *   q, k, v [N, d];  o_lr, out [(i_hi - i_lo), d].
 * Returns 0, or -1 for invalid arguments (odd d, w < 0, rope_base <= 0).
 */
int oracle_local(int64_t N, int32_t d, int64_t w, double rope_base, const double *q, const double *k,
                 const double *v, double alpha, const double *o_lr, int64_t i_lo, int64_t i_hi, double *out);

/*
 * Readout backward (Sec. 3.3 "Training": gradients flow through the selected
 * tokens only, none through the indices; App. D.4) for one query and a fixed
 * selection T[0..nT): given dout = dL/do_i, writes dq [d] and adds into dk, dv
 * [N, d] (rows of the selected tokens) and dg [d] (may be NULL).  The *_abs
 * arrays (may be NULL) get a first-order error scale of the same results (the
 * sizes of their terms, with every upstream factor's size carried along), the
 * yardstick for comparing a rounded computation with these values.
 * nT = 0 gives dq = 0 and adds nothing.
 */
void oracle_readout_backward(const oracle_cfg *cfg, const double *q_i, const double *k, const double *v,
                             const double *g, const int64_t *T, int64_t nT, const double *dout, double *dq,
                             double *dk, double *dv, double *dg, double *dq_abs, double *dk_abs, double *dv_abs,
                             double *dg_abs);

/* The readout backward of queries i in [i_lo, i_hi) of one (sequence, head) with their
 * selections sel [n, K] (-1 padded) and dout [n, d]: dq [n, d] written; dk, dv [N, d]
 * and dg [d] accumulated (zero them first); *_abs likewise (may be NULL).  Returns 0,
 * or -1 for invalid arguments (a selected cell past the last complete one). */
int oracle_backward_head(const oracle_cfg *cfg, const double *q, const double *k, const double *v, const double *g,
                         const int32_t *sel, const double *dout, int64_t i_lo, int64_t i_hi, double *dq, double *dk,
                         double *dv, double *dg, double *dq_abs, double *dk_abs, double *dv_abs, double *dg_abs);

/* ---- FS-B (Sec. 3.4; App. E.1), in fsb_oracle.c ------------------------- */

typedef struct {
    double tau;  /* the second forest admits cells with a_c >= tau (Eq. 10) */
    int32_t Wb;  /* beam width per forest (the page's W^b = 16) */
    double c;    /* radius weight of Eq. 11 (the page's c = 8) */
} oracle_fsb_cfg;

/* Eq. 18: the binary decomposition of M, largest chunk first; returns r. */
int32_t oracle_fsb_chunks(int64_t M, int64_t *sizes);

/* One forest (App. E.1) over M admitted cells `cells` (ids, arrival order) with
 * mean keys kbar [*, d] and norms a: node arrays of at most cap entries
 * (count = cells below, cell = the cell of a leaf or -1, left/right children
 * or -1, minid = smallest cell id below, mu [n, d], rho, A, pmin = p_v^min).
 * Returns the root (-1 when M = 0, -2 when cap is too small); *n_nodes gets
 * the node count and *min_split_gap the smallest relative gap of the two
 * projections straddling any median split. */
int64_t oracle_fsb_forest(const oracle_cfg *cfg, const double *kbar, const double *a, const int64_t *cells,
                          int64_t M, int64_t cap, int64_t *count, int64_t *cell, int64_t *left, int64_t *right,
                          int64_t *minid, double *mu, double *rho, double *A, double *pmin, int64_t *n_nodes,
                          double *min_split_gap);

/* Eq. 11 for one node summary (mu [d], rho, A, pmin) and query i. */
double oracle_fsb_node_priority(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const double *q_i, int64_t i,
                                const double *mu, double rho, double A, double pmin);

/* Eq. 12 for query i and cell c (k [N, d] holds the cell's tokens); *mag (may be
 * NULL) gets the size of its terms. */
double oracle_fsb_rerank_score(const oracle_cfg *cfg, const double *q_i, const double *k, double a_c, int64_t i,
                               int64_t c, double *mag);

/*
 * FS-B for one (sequence, head), queries i in [i_lo, i_hi): both forests over
 * the block's available cells, a beam of W^b per forest, the union of the
 * leaves reached reranked by Eq. 12, the min(K, |B_i|) best read out (Eq. 9,
 * Eq. 17).  Outputs per query row (each may be NULL):
 *   sel [n, K] (reranked score desc, id asc; -1 padded), cand [n, 2 W^b] the
 *   candidate cells B_i ascending (-1 padded), n_cand [n] = |B_i|,
 *   gap_beam [n] smallest beam-cut gap (relative to the larger term size),
 *   gap_rerank [n] smallest gap of adjacent reranked scores among the K + 1
 *   best (relative to the larger term size),
 *   gap_split [n] smallest median-split gap of the query's block's forests,
 *   out [n, d].
 * Returns 0, or -1 for invalid arguments.
 */
int oracle_fsb_head(const oracle_cfg *cfg, const oracle_fsb_cfg *fb, const double *q, const double *k,
                    const double *v, const double *g, int64_t i_lo, int64_t i_hi, int32_t *sel, int32_t *cand,
                    int32_t *n_cand, double *gap_beam, double *gap_rerank, double *gap_split, double *out);

#ifdef __cplusplus
}
#endif

#endif
