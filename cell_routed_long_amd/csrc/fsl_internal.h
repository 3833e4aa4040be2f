// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fsl.h"
#include "fsl_device.h"

namespace fsl {

constexpr int kMaxRetainedCap = 1024; // largest P + W accepted by the ABI

// Geometry every kernel shares (derived and validated by the ABI layer).
struct Geometry {
    int32_t bh;        // batch * H
    int32_t H;
    int64_t N;         // positions per sequence
    int32_t d;         // head dimension (64 or 128)
    int32_t bf16;      // 1 = bf16 tensors, 0 = fp32
    int64_t M;         // complete cells per sequence, N / s
    int32_t NB;        // query blocks per sequence, ceil(N / B)
    int32_t s, B, P, W, K, prune;
    int32_t cap;       // row length of the retained lists, P + W
    float eps;
};

// kbar_split (optional): [bh, M, 3, d] bf16 hi/mid/lo parts of kbar.
// kbar_norm (optional): [bh, M] fp32 Euclidean norms of kbar.
// kbar64 [bh, M, d], a64 [bh, M] (optional): the same summaries before the rounding to fp32.
hipError_t launch_cell_summaries(const Geometry &g, const void *k, float *kbar, float *a, uint16_t *kbar_split,
                                 float *kbar_norm, hipStream_t st, double *kbar64 = nullptr, double *a64 = nullptr);

// death[c]: first query block whose TopP no longer holds cell c (INT32_MAX: never leaves).
// ord: [bh, M] scratch (the head's cells in priority order, with their exit blocks).
// emit = 0 computes only the exit blocks (enough to build a decode state).
hipError_t launch_prune(const Geometry &g, const float *a, int32_t *death, int64_t *ord, int32_t *retained,
                        int32_t *n_ret, int emit, hipStream_t st);

// kbar_split (optional, bf16 only): the parts written by launch_cell_summaries.
hipError_t launch_score_topk(const Geometry &g, const HeadConsts &hc, const void *q, const float *kbar,
                             const uint16_t *kbar_split, const float *a, const int32_t *retained,
                             const int32_t *n_ret, int32_t *sel, hipStream_t st);

hipError_t launch_readout(const Geometry &g, const void *q, const void *k, const void *v,
                          const int32_t *sel, const float *gain, void *out, hipStream_t st);

// Readout backward (Sec. 3.3 "Training"): device workspace of one call.
//   du       per query dL/du: [bh, N, d] fp32 (fp32 tensors), or bf16 hi then lo
//            planes of [bh, N, d] each (bf16 tensors)
//   lse, delta [bh, N] fp32: the logits' log2-sum-exp2 (exp2 domain) and du . u
//   masks    [bh, M, NB] 128-bit masks of the rows of each query block that
//            selected each cell (for the cells available to the block)
//   item_start, pstart [bh, M + 1] int32, item_cell [bh, items_max] int32: each
//            cell's query list cut into chunks of at most kChunk queries;
//            multi_cell [bh, multi_max + 1] int32: the count, then the cells of
//            several chunks
//   partial  [bh, p_max, 2, 32, d] fp32 chunk sums of cells with several chunks
//   dg_part  [bh, NB, d], dg2 [H, 32, d] fp32 partial gain gradients
constexpr int64_t kBwdMaxTokens = 65536;            // the masks take N^2 / (s B) x 16 bytes per (sequence, head)
constexpr int kBwdMaxCells = (int)(kBwdMaxTokens / 32);
constexpr int kChunk = 512;                         // queries per chunk of a cell's list
struct BwdBuffers {
    void *du;
    float *lse, *delta;
    void *masks;
    int32_t *item_start, *pstart, *item_cell, *multi_cell;
    float *partial, *dg_part, *dg2;
};
struct BwdSizes {
    int64_t items_max; // chunks per head: M + ceil(N K / kChunk) bounds one per cell plus one per kChunk pairs
    int64_t p_max;     // partial slots per head: a cell of n >= 2 chunks has more than (n - 1) kChunk
                       // pairs and n <= 2 (n - 1), so 2 ceil(N K / kChunk) slots suffice
    int64_t multi_max; // cells of several chunks per head: each has more than kChunk pairs
};
inline BwdSizes bwd_sizes(const Geometry &g)
{
    const int64_t extra = ((int64_t)g.N * g.K + kChunk - 1) / kChunk;
    return BwdSizes{g.M + extra, 2 * extra > 0 ? 2 * extra : 1, extra};
}
hipError_t launch_readout_backward(const Geometry &g, const BwdBuffers &w, const void *q, const void *k,
                                   const void *v, const int32_t *sel, const float *gain, const void *dout, float *dq,
                                   float *dk, float *dv, float *dgain, hipStream_t st);

// Routing and readout of every 128-query block in one launch (bf16 only; the
// retained lists at most kFusedMaxCap long).  sel may be NULL.  With kbar_norm
// (optional) a tile of retained cells is passed over when no cell of it can
// reach any query's top-K (the results do not change).
constexpr int kFusedMaxCap = 256;
hipError_t launch_route_readout(const Geometry &g, const HeadConsts &hc, const void *q, const void *k,
                                const void *v, const uint16_t *kbar_split, const float *kbar_norm, const float *a,
                                const int32_t *retained, const int32_t *n_ret, const float *gain, void *out,
                                int32_t *sel, hipStream_t st);

// Decode state of every (sequence, head) for continuing at position g.N, from
// the prefill's summaries (kbar, a), exit blocks (death) and raw keys/values.
hipError_t launch_state_build(const Geometry &g, const StateLayout &L, const StateHeader &hdr, void *state,
                              const void *k, const void *v, const float *kbar, const float *a,
                              const int32_t *death, hipStream_t st);

// One decode step for bh = batch * H records (n_tok = 0: q, k_new, v_new, out [bh, d],
// sel [bh, K]), or n_tok >= 1 consecutive steps in one launch (rows [bh, n_tok, ...]).
hipError_t launch_decode_step(int32_t bh, int32_t H, int32_t d, int32_t bf16, int32_t K, int32_t P, int32_t W,
                              float eps, const StateLayout &L, const StateHeader &expect, const HeadConsts &hc,
                              void *state, const void *q, const void *k_new, const void *v_new,
                              const float *gain, void *out, int32_t *sel, hipStream_t st, int n_tok = 0);

// Chunked prefill of n tokens into bf16 decode states, one query block at a time
// with the fused prefill's arithmetic (q, k, v, out [bh, n, d]; sel [bh, n, K]).
hipError_t launch_chunk_blocks(int32_t bh, int32_t H, int32_t d, int32_t K, int32_t P, int32_t W, float eps,
                               const StateLayout &L, const StateHeader &expect, const HeadConsts &hc, void *state,
                               const void *q, const void *k, const void *v, const float *gain, void *out,
                               int32_t *sel, int64_t n, hipStream_t st);

// An empty decode state (position 0) for bh records.
hipError_t launch_state_init(int32_t bh, const StateLayout &L, const StateHeader &hdr, void *state, hipStream_t st);

// Local branch (Sec. 3.2, Eqs. 3-4) plus alpha_h * o_lr (Eq. 2) when o_lr is not NULL.
struct LocalConsts {
    float alpha[128]; // alpha_h
    float rope_base;  // RoPE frequencies theta_m = rope_base^(-2m/d)
};
hipError_t launch_local(const Geometry &g, const LocalConsts &lc, int64_t w, const void *q, const void *k,
                        const void *v, const void *o_lr, void *out, hipStream_t st);

// Local-branch decode state: the rotation table and, for every (sequence, head),
// the last min(n, w) of the n tokens given (positions pos - n .. pos - 1).
hipError_t launch_local_state_build(int32_t bh, int32_t d, int32_t bf16, const LocalStateLayout &L,
                                    const LocalStateHeader &hdr, void *state, const void *k, const void *v,
                                    int64_t n, int64_t pos, hipStream_t st);

// One local-branch decode step (plus alpha_h * o_lr when o_lr is not NULL) for bh records.
hipError_t launch_local_decode(int32_t bh, int32_t H, int32_t d, int32_t bf16, const LocalStateLayout &L,
                               const LocalStateHeader &expect, const LocalConsts &lc, void *state, const void *q,
                               const void *k_new, const void *v_new, const void *o_lr, void *out, hipStream_t st);

// The whole attention decode step in one launch: the long-range step on `state`
// and the local step on `lstate` (out = o_sr + alpha_h o_lr), bitwise
// launch_decode_step followed by launch_local_decode with its output as o_lr.
hipError_t launch_attn_decode(int32_t bh, int32_t H, int32_t d, int32_t bf16, int32_t K, int32_t P, int32_t W,
                              float eps, const StateLayout &L, const StateHeader &expect, const HeadConsts &hc,
                              void *state, const LocalStateLayout &LL, const LocalStateHeader &lexpect,
                              const LocalConsts &lc, void *lstate, const void *q, const void *k_new,
                              const void *v_new, const float *gain, void *out, int32_t *sel, hipStream_t st);

// ---- FS-B (Sec. 3.4; App. E.1): two causal forests, beam search, token rerank ----
constexpr int kFsbMaxBeam = 16;          // W^b
constexpr int64_t kFsbMaxCells = 4096;   // admitted cells per forest (N <= 131,072 at s = 32)
constexpr int kFsbMaxLevels = 13;        // chunk sizes 2^0 .. 2^12

// Per-node summary (Eq. 20/21) beside the fp32 mean key: radius, largest norm,
// smallest cell id below (p_min = (minid + 1/2) s) and, for a leaf, its cell (-1 otherwise).
struct FsbNodeMeta {
    float rho, A;
    int32_t minid, cell;
};

// Storage of one forest's chunk trees for one head: every aligned chunk of 2^k
// admitted cells that starts at an even multiple of 2^k (the only ones a binary
// decomposition uses), heap-ordered (node h of a chunk, 1 <= h < 2^(k+1), at h - 1).
struct FsbLayout {
    int64_t Mu;                           // cells the forests can hold: the last block's available cells
    int32_t levels;                       // chunk levels k = 0 .. levels - 1
    int64_t chunk_base[kFsbMaxLevels + 1]; // first chunk of level k, per forest
    int64_t node_base[kFsbMaxLevels + 1];  // first node of level k, per forest
    int64_t chunks, nodes;                 // per forest
};

struct FsbConsts {
    double tau[128]; // the second forest admits cells with a_c >= tau_h (Eq. 10)
    int32_t Wb;      // beam width
    float c;         // radius weight of Eq. 11
};

// Admission of the second forest, chunk trees of both forests, then the search,
// rerank and top-K of every query (sel [bh, N, K]; cand [bh, N, 2 Wb] optional).
hipError_t launch_fsb(const Geometry &g, const FsbLayout &L, const HeadConsts &hc, const FsbConsts &fc,
                      const void *q, const void *k, const double *kbar64, const float *a, const double *a64,
                      int32_t *adm, int32_t *adm_count, float *node_mu, FsbNodeMeta *node_meta, int32_t *sel,
                      int32_t *cand, hipStream_t st);

// Host-side checks of fs_longrange_prefill's arguments (everything but the
// workspace); on FS_OK, *workspace_needed holds the workspace it needs.
fs_status prefill_check(const fs_shape *shape, const fs_params *prm, const void *q, const void *k, const void *v,
                        const float *sigma_h, const float *lambda_h, void *out, int32_t *sel, void *state,
                        size_t state_bytes, size_t *workspace_needed);

} // namespace fsl
