/*
 * fsl.h — C ABI of the MI355X (gfx950) implementation of FreeSolo's long-range
 * sparse-attention branch (FS and FS-L).
 *
 * Page: "FreeSolo: Linear-time Sparse Attention with Zero-Shot Length
 * Extrapolation" (arXiv 2610.17191), Sec. 3.3 ("Cells", "Query blocks",
 * "Causal availability", "Cell scoring", "Query-independent pruning",
 * "Per-query selection", "Token readout", "Inference"), App. C ("Bounded
 * cache", Eq. 15) and App. D.2 (Eq. 17).
 *
 * Conventions shared by every entry point:
 *   - Tensors are contiguous, row-major, on the device: q, k, v, out are
 *     [batch, H, N, d] of the shape's dtype (fp32 or bf16).  Cell summaries
 *     are fp32; ids are int32.  Cell c holds positions c*s .. c*s+s-1; only the
 *     floor(N/s) complete cells have summaries; the query block of position i
 *     is i / B.
 *   - The caller owns every buffer (inputs, outputs, workspace, decode state).
 *     The library never allocates or frees device memory and keeps no mutable
 *     global state.  Outputs are fully overwritten (zero rows, -1 padding).
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is enqueued
 *     on it; no call synchronises.  Decode steps are safe to capture in a HIP
 *     graph (all position-dependent branching happens on the device).
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     a rejected call enqueues nothing and writes nothing.  A launch failure
 *     reported by the runtime gives FS_ERR_HIP.  Faults inside kernels surface
 *     at the caller's next synchronisation, as for any HIP work.
 *   - Ties in key norm (top-P) and in routing score (top-K) are broken in
 *     favour of the smaller cell id.
 */
#ifndef FSL_H
#define FSL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FS_OK = 0,
    FS_ERR_INVALID = 1,      /* NULL required pointer, non-positive size, inconsistent params */
    FS_ERR_UNSUPPORTED = 2,  /* valid per the method, outside what the kernels implement */
    FS_ERR_WORKSPACE = 3,    /* workspace smaller than the matching *_workspace_bytes() */
    FS_ERR_STATE = 4,        /* decode state of the wrong size, or not built by this library */
    FS_ERR_HIP = 5           /* the HIP runtime rejected a launch */
} fs_status;

typedef enum { FS_F32 = 0, FS_BF16 = 1 } fs_dtype;

/* Method parameters (Sec. 3.3; the page's values in App. A are s=32, B=128,
 * P=64, W=8, K=4).  prune = 1 selects FS-L (Eq. 8), prune = 0 selects FS
 * (A_i = C_i).  eps is the RMSNorm epsilon of Eq. 17 (the page uses 1e-8).
 * Kernels support s == 32, B == 128, 1 <= K <= 8, P + W <= 1024; anything
 * else valid gives FS_ERR_UNSUPPORTED. */
typedef struct {
    int32_t s, B, P, W, K, prune;
    float eps;
} fs_params;

/* batch sequences x H heads x N positions x d features (d in {64, 128}).
 * Kernels support N <= 2^22, batch * H <= 65535 and batch * H * ceil(N / 32)
 * <= 2^26 cells; larger shapes give FS_ERR_UNSUPPORTED. */
typedef struct {
    int32_t batch, H;
    int64_t N;
    int32_t d;
    fs_dtype dtype;
} fs_shape;

/* Largest head count accepted (sigma_h and lambda_h travel as launch arguments). */
#define FS_MAX_HEADS 128

const char *fs_status_string(fs_status status);

/*
 * Cell summaries, Eq. 5: for every complete cell c < M = floor(N/s) of every
 * (sequence, head), kbar[c] = (1/s) sum_{j in I_c} k_j and a[c] = max_{j in I_c}
 * ||k_j||_2 (p_c = (c + 1/2) s is implicit).
 *   k           [batch, H, N, d]     shape dtype                    (input)
 *   kbar        [batch, H, M, d]     fp32                           (output)
 *   a           [batch, H, M]        fp32                           (output)
 *   kbar_split  [batch, H, M, 3, d]  bf16 bit patterns, or NULL     (output)
 *               kbar[c] as three bf16 parts hi, mid, lo (hi = bf16(kbar),
 *               mid = bf16(kbar - hi), lo = bf16(kbar - hi - mid)): the operands
 *               fs_score_select feeds to the bf16 matrix cores.  bf16 shapes
 *               only; not written for fp32 shapes.
 *   kbar_norm   [batch, H, M]        fp32, or NULL                  (output)
 *               ||kbar[c]||_2 of the fp32 mean; fs_select_readout uses it to
 *               bound the content term of Eq. 7 (|q . kbar| <= |q| |kbar|).
 * Sums and norms accumulate in fp64 and are rounded once to fp32.
 */
fs_status fs_cell_summaries(const fs_shape *shape, const fs_params *prm, const void *k,
                            float *kbar, float *a, uint16_t *kbar_split, float *kbar_norm,
                            void *stream);

/* Bytes of workspace fs_prune_retained needs (0 on invalid arguments). */
size_t fs_prune_workspace_bytes(const fs_shape *shape, const fs_params *prm);

/*
 * FS-L retained sets, Eqs. 6 and 8: for every query block beta of every
 * (sequence, head), A_beta = Recent_W(C_beta) u TopP_{c in C_beta}(a_c) with
 * C_beta = {c : (c+1) s <= beta B}.  Requires prm->prune == 1.
 *   a           [batch, H, M]            fp32, from fs_cell_summaries (input)
 *   retained    [batch, H, NB, P + W]    int32 cell ids in priority order (a desc, id
 *                                        asc), -1 padded (output)
 *   n_retained  [batch, H, NB]           int32 |A_beta| (output)
 *   workspace   fs_prune_workspace_bytes() bytes of device memory (scratch)
 * NB = ceil(N / B).  Block 0 is always empty.
 */
fs_status fs_prune_retained(const fs_shape *shape, const fs_params *prm, const float *a,
                            int32_t *retained, int32_t *n_retained,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * Routing scores and per-query selection, Eq. 7 and Sec. 3.3 "Per-query
 * selection": r_ic = q_i . kbar_c / sqrt(d) + lambda_h a_c erf((i - p_c) /
 * (2 sigma_h)) over A_i (the retained set of the query's block for FS-L, the
 * whole prefix C_i for FS), and T_i = the min(K, |A_i|) best cells.
 *   q           [batch, H, N, d]        shape dtype (input)
 *   kbar, a     from fs_cell_summaries  (input)
 *   kbar_split  from fs_cell_summaries, or NULL: the scorer then splits kbar
 *               itself (bf16 shapes; ignored for fp32 shapes)
 *   retained, n_retained  from fs_prune_retained (input; NULL when prune == 0)
 *   sigma_h, lambda_h     host [H] fp32 (sigma > 0, lambda >= 0)
 *   sel         [batch, H, N, K] int32, (score desc, id asc), -1 padded (output)
 */
fs_status fs_score_select(const fs_shape *shape, const fs_params *prm, const void *q, const float *kbar,
                          const uint16_t *kbar_split, const float *a, const int32_t *retained,
                          const int32_t *n_retained, const float *sigma_h, const float *lambda_h,
                          int32_t *sel, void *stream);

/*
 * Token readout and RMSNorm, Eq. 9 (softmax over the tokens of the selected
 * cells jointly, NoPE logits q_i . k_j / sqrt(d)) followed by Eq. 17's RMSNorm
 * with gain; rows whose selection is empty are written as zeros.
 *   q, k, v     [batch, H, N, d]  shape dtype (input)
 *   sel         [batch, H, N, K]  int32 from fs_score_select (input)
 *   gain        device [H, d] fp32, or NULL for unit gains
 *   out         [batch, H, N, d]  shape dtype (output)
 */
fs_status fs_readout(const fs_shape *shape, const fs_params *prm, const void *q, const void *k, const void *v,
                     const int32_t *sel, const float *gain, void *out, void *stream);

/* Bytes of workspace fs_readout_backward needs (0 on invalid or unsupported arguments). */
size_t fs_readout_backward_workspace_bytes(const fs_shape *shape, const fs_params *prm);

/*
 * Backward of fs_readout (Sec. 3.3 "Training": gradients reach the shared
 * projections through the selected-token readout; the top-P and top-K indices
 * receive none; App. D.4).  With o_i = g * u_i r_i, u_i = softmax(q_i k_S / sqrt(d)) V_S
 * over the tokens S_i of the cells sel[i] (Eq. 9) and r_i = 1/sqrt(|u_i|^2/d + eps)
 * (Eq. 17), and dout_i = dL/do_i, the selection held fixed:
 *   dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
 *   dv_j = sum_i p_ij du_i,  dgain = sum_i r_i dout_i * u_i,
 * du_i = r_i g*dout_i - (r_i^3/d)(sum_f g_f dout_if u_if) u_i,
 * dS_ij = p_ij (du_i . v_j - du_i . u_i).  The forward is recomputed from the
 * inputs exactly as fs_readout reads them: a row's cells must be distinct, and
 * entries < 0 or not available to the query's block (Eq. 6) are ignored.
 *   q, k, v     [batch, H, N, d]  shape dtype (input)
 *   sel         [batch, H, N, K]  int32 (input), as written by the selection calls
 *   gain        device [H, d] fp32 RMSNorm gains, or NULL for unit gains
 *   dout        [batch, H, N, d]  shape dtype (input)
 *   dq, dk, dv  [batch, H, N, d]  fp32 (output; every element is written, 0 for a
 *               query with no selected cell and for a token no query selected)
 *   dgain       device [H, d] fp32 (output, summed over the batch), or NULL; not
 *               written when gain is NULL
 *   workspace   fs_readout_backward_workspace_bytes() bytes of device memory
 * Deterministic: no floating-point atomics; repeated calls give identical bits.
 * Supported: N <= 65,536 (the per-cell row masks take N^2/(s B) x 16 bytes per
 * (sequence, head)) and batch * H * ceil(N / s) < 2^24.
 */
fs_status fs_readout_backward(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                              const void *v, const int32_t *sel, const float *gain, const void *dout, float *dq,
                              float *dk, float *dv, float *dgain, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Routing and readout in one call: fs_score_select followed by fs_readout
 * (Eq. 7, per-query top-K, Eq. 9 with Eq. 17's RMSNorm), same arguments and
 * results.  For bf16 shapes given kbar_split (and FS, or FS-L with P + W <=
 * 256) it runs as a single kernel in which each 128-query block scores its
 * retained cells, selects, and reads out its selected cells without the
 * selections going through global memory; the outputs are bitwise those of
 * the two separate calls.  Given kbar_norm as well, that kernel passes over a
 * tile of 32 retained cells when an upper bound of every score in it
 * (max lambda_h a_c + max |q_i| max |kbar_c| / sqrt(d), widened for rounding)
 * lies below every query's K-th best score so far: no such cell can be
 * selected, so the results are bitwise unchanged.
 *   q, k, v                [batch, H, N, d]  shape dtype (input)
 *   kbar, kbar_split, kbar_norm, a   from fs_cell_summaries (kbar_split and
 *                          kbar_norm may be NULL)
 *   retained, n_retained   from fs_prune_retained (FS-L; NULL for FS)
 *   sigma_h, lambda_h      host [H] fp32;  gain  device [H, d] fp32 or NULL
 *   out                    [batch, H, N, d] shape dtype (output)
 *   sel                    [batch, H, N, K] int32 (output); may be NULL only
 *                          when the single-kernel form applies
 */
fs_status fs_select_readout(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                            const void *v, const float *kbar, const uint16_t *kbar_split,
                            const float *kbar_norm, const float *a, const int32_t *retained,
                            const int32_t *n_retained, const float *sigma_h, const float *lambda_h,
                            const float *gain, void *out, int32_t *sel, void *stream);

/* Bytes of workspace fs_longrange_prefill needs (0 on invalid arguments). */
size_t fs_prefill_workspace_bytes(const fs_shape *shape, const fs_params *prm);

/*
 * The long-range branch over a whole prompt (Sec. 3.3 "Inference": prompt
 * prefill uses the same causal operator), for every query position i:
 * summaries (Eq. 5), availability (Eq. 6), retention (Eq. 8, FS-L) or the full
 * prefix (FS), scores r_ic (Eq. 7) with g_h(x) = erf(x / (2 sigma_h)), the
 * min(K, |A_i|) best cells T_i, and o_i = RMSNorm(softmax(q_i k_S / sqrt(d)) V_S)
 * over the tokens S_i of T_i (Eq. 9, Eq. 17); o_i = 0 when S_i is empty.
 *   q, k, v     [batch, H, N, d]   shape dtype (input)
 *   sigma_h     host [H] fp32, > 0          lambda_h  host [H] fp32, >= 0
 *   gain        device [H, d] fp32 RMSNorm gains, or NULL for unit gains
 *   out         [batch, H, N, d]   shape dtype, or NULL (output)
 *   sel         [batch, H, N, K]   int32 T_i by (score desc, id asc), -1 padded,
 *               or NULL (output)
 *   state       decode state to fill for continuing at position N (see
 *               fs_decode_state_bytes; requires prune = 1 and v), or NULL;
 *               state_bytes must equal fs_decode_state_bytes() (FS_ERR_STATE)
 *   workspace   fs_prefill_workspace_bytes() bytes of device memory (scratch)
 * At least one of out, sel, state must be non-NULL.  q and v may be NULL when
 * out and sel are both NULL (state-only prefill of a long prefix).
 */
fs_status fs_longrange_prefill(const fs_shape *shape, const fs_params *prm,
                               const void *q, const void *k, const void *v,
                               const float *sigma_h, const float *lambda_h, const float *gain,
                               void *out, int32_t *sel, void *state, size_t state_bytes,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * fs_longrange_prefill without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation).  Same arguments (less the workspace),
 * results and errors as fs_longrange_prefill; the workspace is a fixed
 * device array of fs_noalloc_scratch_bytes() (32 MiB) inside the library,
 * one per GPU, held until the process ends.  Shapes whose
 * fs_prefill_workspace_bytes() exceed it give FS_ERR_WORKSPACE before
 * anything is enqueued (32 MiB covers, e.g., 2 sequences x 16 heads x 16384
 * tokens at d = 128 in bf16; split larger batches into several calls).  The
 * first call on a device looks up that device's copy of the array (no
 * allocation; FS_ERR_HIP if the runtime refuses).  Every call on one GPU uses
 * the same array: calls that overlap on one GPU (different streams, or
 * unordered host threads) race; calls ordered on one stream do not.
 */
size_t fs_noalloc_scratch_bytes(void);
fs_status fs_longrange_prefill_noalloc(const fs_shape *shape, const fs_params *prm,
                                       const void *q, const void *k, const void *v,
                                       const float *sigma_h, const float *lambda_h, const float *gain,
                                       void *out, int32_t *sel, void *state, size_t state_bytes,
                                       void *stream);

/*
 * FS-B, balanced tree search (Sec. 3.4 "Balanced tree search (FS-B)"; App. E.1
 * "Streaming forests").  Wb: beam width per forest (the page's W^b = 16);
 * c: radius weight of the node priority, Eq. 11 (the page's c = 8).
 * Supported: 1 <= Wb <= 16, c >= 0 finite.
 */
typedef struct {
    int32_t Wb;
    float c;
} fs_fsb_params;

/* Bytes of workspace fs_fsb_prefill needs (0 on invalid or unsupported arguments). */
size_t fs_fsb_workspace_bytes(const fs_shape *shape, const fs_params *prm, const fs_fsb_params *fb);

/*
 * FS-B over a whole prompt, for every query position i.  For the query block
 * of i, two causal forests over its available cells C_i (Eq. 6): one over all
 * of them and one over those with a_c >= tau_h (Eq. 10), each a chain of
 * balanced trees over the binary decomposition of its admitted count into
 * aligned chunks (App. E.1, Eqs. 18-21: a chunk is split recursively at the
 * median of its mean keys' projections on the principal direction from two
 * power iterations started at the farthest cell; node summaries mu, rho, A,
 * p_min; join nodes chain the chunk roots, smallest first).  Each forest keeps
 * the Wb highest-priority nodes per level by U_v of Eq. 11 down to the leaves
 * (a leaf in the beam keeps its slot; the other slots take the best children);
 * the leaves of both beams are reranked by Eq. 12 (log-sum-exp of the cell's
 * token logits plus the prior) and the min(K, |B_i|) best form the selection,
 * read out with Eq. 9 and RMSNorm (Eq. 17) as in fs_readout.  Ties go to the
 * smaller cell id (nodes: the smaller smallest cell id below them).
 *   prm          s, B, K, eps as for the other calls (P, W, prune are not used)
 *   q, k, v      [batch, H, N, d] shape dtype (input); v may be NULL when out is
 *   sigma_h, lambda_h   host [H] fp32 as for fs_longrange_prefill
 *   tau_h        host [H] fp32, finite: the second forest's norm threshold (the
 *                page calibrates it as a median cell norm once per checkpoint)
 *   gain         device [H, d] fp32 RMSNorm gains, or NULL for unit gains
 *   out          [batch, H, N, d] shape dtype, or NULL (output)
 *   sel          [batch, H, N, K] int32 (reranked score desc, id asc), -1
 *                padded, or NULL (output)
 *   cand         [batch, H, N, 2 Wb] int32 the candidate cells B_i in ascending
 *                order, -1 padded, or NULL (output)
 *   workspace    fs_fsb_workspace_bytes() bytes of device memory (scratch)
 * Arithmetic: mean keys and norms in fp64 (the trees are built from them in
 * fp64, the second forest admits by the fp64 norm); node priorities and
 * rerank scores in fp32 with exact products on the matrix cores.
 * Supported: at most 4096 cells available to the last block (N <= 131,200 at
 * s = 32, B = 128); larger shapes give FS_ERR_UNSUPPORTED.
 */
fs_status fs_fsb_prefill(const fs_shape *shape, const fs_params *prm, const fs_fsb_params *fb,
                         const void *q, const void *k, const void *v,
                         const float *sigma_h, const float *lambda_h, const float *tau_h, const float *gain,
                         void *out, int32_t *sel, int32_t *cand,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Streaming decode (Sec. 3.3 "Inference"; App. C "Bounded cache", Eq. 15).
 *
 * The decode state is one flat caller-owned device buffer: a 256-byte header
 * (shape, P, W, slot count) followed by one record per (sequence, head).  A
 * record holds P + W + B/s cell slots: the retained set A of the current query
 * block (at most P + W cells, Eq. 8) plus the cells of the block being filled.
 * Each slot keeps the cell's raw keys and values (dtype), its fp32 mean key and
 * norm (Eq. 5), its absolute cell id and whether it is in TopP; the record also
 * keeps the next position, the retained slots in ascending cell-id order and,
 * as a prefetch hint only, the slots the last step read.
 * Memory per (sequence, head) is therefore constant in the context length.
 * Copying the buffer's bytes checkpoints the stream exactly.
 * Supported: FS-L (prune = 1) with P + W + B/s <= 128 slots.
 */

/* Bytes of one decode state for `batch` sequences x H heads (0 on invalid or
 * unsupported arguments, including prune = 0: FS keeps the whole prefix). */
size_t fs_decode_state_bytes(int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                             const fs_params *prm);

/*
 * One decode step of the long-range branch for every (sequence, head), one
 * token each.  With i the record's stored position:
 *   (1) if i is a block start (i % B == 0, i > 0), the B/s cells that just
 *       became eligible are merged into TopP (Eq. 15: TopP(C u D) =
 *       TopP(TopP(C) u D), ties to the smaller id), A = Recent_W u TopP, and
 *       slots whose cell is in neither are freed;
 *   (2) k_new, v_new are appended; when position i completes a cell its
 *       summary (Eq. 5) is formed (fp64 sums, rounded once to fp32);
 *   (3) q is scored against A (Eq. 7, in fp32 as the prefill), its min(K, |A|) best
 *       cells are selected and read out (Eq. 9) with RMSNorm (Eq. 17); the
 *       position advances to i + 1.
 * The output equals the prefill's at position i (same causal operator).
 *   prm              as for the prefill that built the state (K may differ)
 *   state            fs_decode_state_bytes() bytes, filled by
 *                    fs_longrange_prefill (or a byte copy of such a state)   (in/out)
 *   q, k_new, v_new  device [batch, H, d] dtype                             (input)
 *   sigma_h, lambda_h, gain   as for fs_longrange_prefill
 *   out              device [batch, H, d] dtype                             (output)
 *   sel              device [batch, H, K] int32, (score desc, id asc), -1 padded, or NULL
 * Errors: FS_ERR_STATE when state_bytes does not match this shape and prm.  A
 * buffer of the right size whose header was not written by
 * fs_longrange_prefill for this shape is detected on the device: out is set to
 * NaN, sel to -1, and the buffer is left untouched.  One launch per step, no
 * host synchronisation: steps can be captured in a HIP graph.  Steps on the
 * same state must be ordered (same stream or explicit dependencies).
 */
fs_status fs_longrange_decode(const fs_params *prm, int32_t batch, int32_t H, int32_t d,
                              fs_dtype dtype, void *state, size_t state_bytes,
                              const void *q, const void *k_new, const void *v_new,
                              const float *sigma_h, const float *lambda_h, const float *gain,
                              void *out, int32_t *sel, void *stream);

/*
 * An empty decode state, at position 0 (nothing retained, every slot free), for
 * prefilling a prompt entirely through fs_longrange_prefill_chunk.
 *   state   fs_decode_state_bytes() bytes of device memory (FS_ERR_STATE otherwise)
 */
fs_status fs_decode_state_init(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                               void *state, size_t state_bytes, void *stream);

/*
 * Chunked prefill into a decode state (App. C "Bounded cache": the bounded
 * cache is prefilled in fixed-size chunks -- the page uses 2048 tokens -- with
 * the retention update at every block boundary; Sec. 3.3 "Inference").  The n
 * tokens at the state's positions i .. i + n - 1 of every (sequence, head) are
 * processed in one launch, with the same results as n fs_longrange_decode steps
 * (merge at block starts, append and cell summary, Eq. 7 scores over A, top-K,
 * readout with Eq. 17): the same causal operator as the whole-prompt prefill.
 * bf16: the chunk's query blocks are taken in order, each block's queries at
 * once with the whole-prompt prefill's arithmetic, so outputs and selections
 * are bitwise those of fs_longrange_prefill over the whole prompt and the
 * state's cell summaries are bitwise the summary pass's.  fp32: the tokens are
 * taken one by one as decode steps, bitwise n single steps.  Either way the
 * result does not depend on where a prompt is cut into chunks.
 *   state            as for fs_longrange_decode (built by fs_longrange_prefill,
 *                    fs_decode_state_init, or an earlier chunk)            (in/out)
 *   n                tokens per (sequence, head), 1 <= n <= 65536
 *   q, k, v          device [batch, H, n, d] dtype: the chunk's rows          (input)
 *   sigma_h, lambda_h, gain   as for fs_longrange_decode
 *   out              device [batch, H, n, d] dtype                             (output)
 *   sel              device [batch, H, n, K] int32, or NULL                    (output)
 * Errors and the foreign-state check as for fs_longrange_decode (a foreign
 * state gets NaN outputs for every row).
 */
fs_status fs_longrange_prefill_chunk(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                                     void *state, size_t state_bytes, int64_t n,
                                     const void *q, const void *k, const void *v,
                                     const float *sigma_h, const float *lambda_h, const float *gain,
                                     void *out, int32_t *sel, void *stream);

/*
 * Local branch (Sec. 3.2, Eqs. 3-4) and the branch combination (Sec. 3.1,
 * Eq. 2) for every query i of every (sequence, head):
 *   o_sr_i = softmax_{j in L_i}((R(i) q_i) . (R(j) k_j) / sqrt(d)) V_{L_i},
 *   L_i = {j : 0 <= j <= i, i - j <= w} (a full window holds w + 1 tokens),
 *   R(p) turning feature pair (2m, 2m+1) by p * rope_base^(-2m/d) (the RoPE
 *   rotation of Su et al., which the page cites),
 *   out_i = o_sr_i + alpha_h * o_lr_i when o_lr is given, else out_i = o_sr_i.
 *   shape       batch, H, N, d, dtype as for the other calls
 *   w           look-back radius, 0 <= w <= 65535 (the page's w is 512; larger
 *               windows give FS_ERR_UNSUPPORTED)
 *   rope_base   > 1 and finite (RoFormer's 10000 unless the model says otherwise)
 *   q, k, v     device [batch, H, N, d] dtype, unrotated (the same q, k, v as the
 *               long-range branch, which reads them unrotated)          (input)
 *   alpha_h     host [H] fp32, finite; required when o_lr is given, else ignored
 *   o_lr        device [batch, H, N, d] dtype: the long-range output (out of
 *               fs_longrange_prefill), or NULL                          (input)
 *   out         device [batch, H, N, d] dtype; may be the o_lr buffer (each row
 *               is read before it is written)                           (output)
 * Arithmetic: bf16 inputs are rotated in fp32 and kept as bf16 hi + lo parts
 * (logits from three bf16 products with fp32 accumulation); fp32 inputs use
 * fp32 products.  The softmax is exact up to rounding.
 * Errors: FS_ERR_INVALID for a NULL q/k/v/out, w < 0, a bad rope_base, o_lr
 * without alpha_h or a non-finite alpha; FS_ERR_UNSUPPORTED as for the shape.
 */
fs_status fs_local_window(const fs_shape *shape, int64_t w, float rope_base, const void *q, const void *k,
                          const void *v, const float *alpha_h, const void *o_lr, void *out, void *stream);

/*
 * Size in bytes of the local branch's decode state for batch x H heads and
 * look-back radius w (Sec. 3.2; the bounded decode cache of App. C keeps a
 * local ring of the last w tokens).  Layout: a 256-byte header; a table of
 * (cos, sin) of o * theta_m for o = 0 .. w and m < d/2 (fp32 pairs, shared by
 * every head); then per (sequence, head) the next position (int64) and rings of
 * the last w raw keys and the last w raw values of the dtype (token p in slot
 * p mod w; one unused slot when w = 0).  0 for an unsupported or invalid
 * combination (d not 64/128, H > FS_MAX_HEADS, w < 0 or w > 65535,
 * batch * H > 65535).
 */
size_t fs_local_state_bytes(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w);

/*
 * Builds the local decode state for continuing at position pos.
 *   w, rope_base  as for fs_local_window
 *   state         device buffer of exactly fs_local_state_bytes() bytes (FS_ERR_STATE otherwise)
 *   k, v          device [batch, H, n, d] dtype: the n raw (unrotated) keys and
 *                 values at positions pos - n .. pos - 1 (a whole prompt: n = pos;
 *                 its tail is enough: n >= min(pos, w)).  May be NULL when n = 0.
 *   n, pos        0 <= min(pos, w) <= n <= pos
 * Keeps the last min(n, w) tokens.  Errors: FS_ERR_INVALID for a NULL state, a
 * bad rope_base or n, pos out of range.
 */
fs_status fs_local_state_build(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w, float rope_base,
                               void *state, size_t state_bytes, const void *k, const void *v, int64_t n,
                               int64_t pos, void *stream);

/*
 * One decode step of the local branch for the token at each record's next
 * position i (Sec. 3.2, Eqs. 3-4, for the one query i; Sec. 3.1, Eq. 2):
 *   o_sr = softmax_{j in [max(0, i - w), i]}(q_i . R(j - i) k_j / sqrt(d)) V,
 *   out = o_sr + alpha_h * o_lr when o_lr is given, else out = o_sr;
 * then k_new, v_new enter the ring and the position advances.  The result
 * equals row i of fs_local_window over the whole sequence.
 *   q, k_new, v_new  device [batch, H, d] dtype, unrotated              (input)
 *   alpha_h          host [H] fp32, finite; required when o_lr is given
 *   o_lr             device [batch, H, d] dtype (fs_longrange_decode's out), or NULL
 *   out              device [batch, H, d] dtype; may be the o_lr buffer  (output)
 * Arithmetic: fp32.  The query is turned by R(o) for each key's offset o, from
 * the state's fp64-built table and fp32 steps of theta_m (relative error below
 * 1e-6); products, softmax and sums in fp32.
 * Errors: FS_ERR_STATE when state_bytes does not match; a buffer of the right
 * size not built by fs_local_state_build for this shape and w is detected on
 * the device: out is set to NaN and the buffer is left untouched.  One launch
 * per step, no host synchronisation (steps can be captured in a HIP graph);
 * steps on one state must be ordered.
 */
fs_status fs_local_decode(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w, void *state,
                          size_t state_bytes, const void *q, const void *k_new, const void *v_new,
                          const float *alpha_h, const void *o_lr, void *out, void *stream);

/*
 * The whole attention decode step of one token per (sequence, head) in one
 * launch (Sec. 3.1, Eq. 2: out = o_sr + alpha_h * o_lr): the long-range step
 * of fs_longrange_decode (Sec. 3.3 "Inference"; App. C "Bounded cache",
 * Eq. 15) on `state` and the local-branch step of fs_local_decode (Sec. 3.2,
 * Eqs. 3-4) on `local_state`, both at the records' next position.  The result,
 * sel and both final states are bitwise those of fs_longrange_decode (output
 * o_lr) followed by fs_local_decode with that o_lr; the long-range output
 * itself is not stored.  The ring reads of the local step overlap the
 * long-range step's chain of dependent phases, so one call takes far less than
 * the two.
 *   prm, state, state_bytes, sigma_h, lambda_h, gain, sel   as for fs_longrange_decode
 *   w, local_state, local_state_bytes   as for fs_local_decode (the state built by
 *                    fs_local_state_build with this w)                   (in/out)
 *   q, k_new, v_new  device [batch, H, d] dtype, unrotated: the one query, key
 *                    and value both branches read                        (input)
 *   alpha_h          host [H] fp32, finite (required)
 *   out              device [batch, H, d] dtype, not overlapping q, k_new, v_new (output)
 * Errors: those of the two calls (FS_ERR_STATE when either size does not
 * match; batch * H above 65535 is FS_ERR_UNSUPPORTED).  A buffer of the right
 * size with a foreign header is detected on the device, as by the two calls:
 * out is NaN, and that state is left untouched (the other one advances).  One
 * launch, no host synchronisation (capturable in a HIP graph); steps on the
 * same states must be ordered.
 */
fs_status fs_attention_decode(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                              void *state, size_t state_bytes, int64_t w, void *local_state,
                              size_t local_state_bytes, const void *q, const void *k_new, const void *v_new,
                              const float *sigma_h, const float *lambda_h, const float *gain,
                              const float *alpha_h, void *out, int32_t *sel, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FSL_H */
