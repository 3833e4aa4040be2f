// C ABI of the long-range branch: argument validation, workspace layout and the
// launch sequence.  Validation happens entirely on the host and before any HIP
// call, so a rejected call touches neither the device nor the runtime.
#include "fsl.h"

#include <climits>
#include <cmath>
#include <cstring>

#include "fsl_internal.h"

#define FSL_EXPORT extern "C" __attribute__((visibility("default")))

namespace fsl {
namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 22; // LDS union bitmap of the readout: N/32 bits <= 16 KB
constexpr int kMaxRetained = kMaxRetainedCap;    // P + W
constexpr int kMaxK = 8;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

fs_status check_params(const fs_params *p)
{
    if (!p)
        return FS_ERR_INVALID;
    if (p->s < 1 || p->B < 1 || p->B % p->s != 0 || p->K < 1 || p->P < 0 || p->W < 0 ||
        (p->prune != 0 && p->prune != 1) || !(p->eps >= 0.0f) || !std::isfinite(p->eps))
        return FS_ERR_INVALID;
    if (p->s != 32 || p->B != 128 || p->K > kMaxK || (int64_t)p->P + p->W > kMaxRetained)
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

// A C caller may store any int in an fs_dtype; reading a value outside the
// enumerators through the C++ enum type is undefined, so validation reads the
// field's bits as an int32 (later reads see a validated value).
static_assert(sizeof(fs_dtype) == sizeof(int32_t), "fs_dtype is int-sized");
bool dtype_valid(const fs_dtype &t)
{
    int32_t v;
    std::memcpy(&v, &t, sizeof v);
    return v == FS_F32 || v == FS_BF16;
}

fs_status check_shape(const fs_shape *sh)
{
    if (!sh)
        return FS_ERR_INVALID;
    if (sh->batch < 1 || sh->H < 1 || sh->N < 1 || sh->d < 1 || !dtype_valid(sh->dtype))
        return FS_ERR_INVALID;
    if ((sh->d != 64 && sh->d != 128) || sh->H > FS_MAX_HEADS || sh->N > kMaxTokens ||
        (int64_t)sh->batch * sh->H > 65535)
        return FS_ERR_UNSUPPORTED;
    // grids: one wave per cell (summaries), one workgroup per 128-query block;
    // at most 2^26 cells keeps every launch below 2^32 work-items
    if ((int64_t)sh->batch * sh->H * ((sh->N + 31) / 32) > ((int64_t)1 << 26))
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

fs_status check_all(const fs_shape *sh, const fs_params *p)
{
    fs_status st = check_shape(sh);
    if (st != FS_OK)
        return st;
    return check_params(p);
}

Geometry geometry(const fs_shape *sh, const fs_params *p)
{
    Geometry g;
    g.bh = sh->batch * sh->H;
    g.H = sh->H;
    g.N = sh->N;
    g.d = sh->d;
    g.bf16 = sh->dtype == FS_BF16;
    g.M = sh->N / p->s;
    g.NB = (int32_t)((sh->N + p->B - 1) / p->B);
    g.s = p->s;
    g.B = p->B;
    g.P = p->P;
    g.W = p->W;
    g.K = p->K;
    g.prune = p->prune;
    g.cap = p->P + p->W > 0 ? p->P + p->W : 1;
    g.eps = p->eps;
    return g;
}

// Workspace of fs_longrange_prefill, carved in this order (256-byte aligned).
struct PrefillLayout {
    size_t kbar, ksplit, knorm, a, death, ord, retained, n_ret, sel, total;
};

PrefillLayout prefill_layout(const Geometry &g)
{
    PrefillLayout L;
    size_t off = 0;
    L.kbar = off;
    off += align_up((size_t)g.bh * g.M * g.d * sizeof(float));
    L.ksplit = off; // bf16 parts of kbar for the scorer (bf16 shapes)
    off += g.bf16 ? align_up((size_t)g.bh * g.M * 3 * g.d * sizeof(uint16_t)) : 0;
    L.knorm = off; // norms of kbar for the fused kernel's tile bound (bf16 shapes)
    off += g.bf16 ? align_up((size_t)g.bh * g.M * sizeof(float)) : 0;
    L.a = off;
    off += align_up((size_t)g.bh * g.M * sizeof(float));
    L.death = off;
    off += g.prune ? align_up((size_t)g.bh * g.M * sizeof(int32_t)) : 0;
    L.ord = off; // cells in priority order with their exit blocks (list building)
    off += g.prune ? align_up((size_t)g.bh * g.M * sizeof(int64_t)) : 0;
    L.retained = off;
    off += g.prune ? align_up((size_t)g.bh * g.NB * g.cap * sizeof(int32_t)) : 0;
    L.n_ret = off;
    off += g.prune ? align_up((size_t)g.bh * g.NB * sizeof(int32_t)) : 0;
    L.sel = off;
    off += align_up((size_t)g.bh * g.N * g.K * sizeof(int32_t));
    L.total = off > 0 ? off : kAlign;
    return L;
}

fs_status check_heads(int H, const float *sigma_h, const float *lambda_h, HeadConsts *hc)
{
    if (!sigma_h || !lambda_h)
        return FS_ERR_INVALID;
    std::memset(hc, 0, sizeof(*hc));
    for (int h = 0; h < H; ++h) {
        if (!(sigma_h[h] > 0.0f) || !std::isfinite(sigma_h[h]) || !(lambda_h[h] >= 0.0f) ||
            !std::isfinite(lambda_h[h]))
            return FS_ERR_INVALID;
        hc->inv_two_sigma[h] = 1.0f / (2.0f * sigma_h[h]);
        hc->lambda[h] = lambda_h[h];
    }
    return FS_OK;
}

inline fs_status hip_status(hipError_t e) { return e == hipSuccess ? FS_OK : FS_ERR_HIP; }

// Streaming decode needs FS-L (a bounded retained set) and at most kMaxSlots
// slots per (sequence, head): P + W retained cells plus B/s pending cells.
fs_status check_decode_params(const fs_params *p)
{
    fs_status st = check_params(p);
    if (st != FS_OK)
        return st;
    if (!p->prune || (int64_t)p->P + p->W + p->B / p->s > kMaxSlots)
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

fs_status check_decode_dims(int32_t batch, int32_t H, int32_t d, const fs_dtype &dtype)
{
    if (batch < 1 || H < 1 || d < 1 || !dtype_valid(dtype))
        return FS_ERR_INVALID;
    if ((d != 64 && d != 128) || H > FS_MAX_HEADS)
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

// Record layout of the decode state (see StateLayout in fsl_device.h).
StateLayout state_layout(int32_t d, fs_dtype dtype, const fs_params *p)
{
    StateLayout L;
    std::memset(&L, 0, sizeof(L));
    const size_t esz = dtype == FS_BF16 ? 2 : 4;
    L.S = p->P + p->W + p->B / p->s;
    size_t off = align_up(sizeof(StateMeta));
    L.off_ridx = (int64_t)off;
    off += align_up((size_t)L.S * sizeof(int32_t));
    L.off_cell = (int64_t)off;
    off += align_up((size_t)L.S * sizeof(int32_t));
    L.off_flags = (int64_t)off;
    off += align_up((size_t)L.S * sizeof(int32_t));
    L.off_a = (int64_t)off;
    off += align_up((size_t)L.S * sizeof(float));
    L.off_kbar = (int64_t)off;
    off += align_up((size_t)L.S * d * sizeof(float));
    L.off_k = (int64_t)off;
    off += align_up((size_t)L.S * p->s * d * esz);
    L.off_v = (int64_t)off;
    off += align_up((size_t)L.S * p->s * d * esz);
    L.rec_bytes = (int64_t)off;
    return L;
}

StateHeader state_header(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, const fs_params *p,
                         const StateLayout &L)
{
    StateHeader h;
    std::memset(&h, 0, sizeof(h));
    h.magic = kStateMagic;
    h.version = kStateVersion;
    h.batch = batch;
    h.H = H;
    h.d = d;
    h.dtype = (int32_t)dtype;
    h.s = p->s;
    h.B = p->B;
    h.P = p->P;
    h.W = p->W;
    h.n_slots = L.S;
    h.rec_bytes = L.rec_bytes;
    return h;
}

size_t state_bytes_of(int32_t batch, int32_t H, const StateLayout &L)
{
    return (size_t)kStateHeaderBytes + (size_t)batch * H * (size_t)L.rec_bytes;
}

// Longest chunk fs_longrange_prefill_chunk takes in one call (the page prefills in chunks of 2048).
constexpr int64_t kMaxChunk = 65536;

// ---- local-branch decode state ----
constexpr int64_t kMaxLocalWindow = 65535; // ring of w tokens, table of w + 1 rows

LocalStateLayout local_layout(int32_t d, fs_dtype dtype, int64_t w)
{
    LocalStateLayout L;
    std::memset(&L, 0, sizeof(L));
    const size_t esz = dtype == FS_BF16 ? 2 : 4;
    L.w = w;
    L.slots = w > 0 ? w : 1;
    L.off_table = kLocalStateHeaderBytes;
    L.off_rec = (int64_t)align_up((size_t)L.off_table + (size_t)(w + 1) * (size_t)(d / 2) * sizeof(float) * 2);
    L.off_k = (int64_t)align_up(sizeof(int64_t));
    L.off_v = (int64_t)align_up((size_t)L.off_k + (size_t)L.slots * d * esz);
    L.rec_bytes = (int64_t)align_up((size_t)L.off_v + (size_t)L.slots * d * esz);
    return L;
}

LocalStateHeader local_header(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w, float rope_base,
                              const LocalStateLayout &L)
{
    LocalStateHeader h;
    std::memset(&h, 0, sizeof(h));
    h.magic = kLocalStateMagic;
    h.version = kLocalStateVersion;
    h.batch = batch;
    h.H = H;
    h.d = d;
    h.dtype = (int32_t)dtype;
    h.w = w;
    h.rec_bytes = L.rec_bytes;
    h.rope_base = rope_base;
    return h;
}

fs_status check_local_dims(int32_t batch, int32_t H, int32_t d, const fs_dtype &dtype, int64_t w)
{
    fs_status st = check_decode_dims(batch, H, d, dtype);
    if (st != FS_OK)
        return st;
    if (w < 0)
        return FS_ERR_INVALID;
    if (w > kMaxLocalWindow || (int64_t)batch * H > 65535)
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

size_t local_state_bytes_of(int32_t batch, int32_t H, const LocalStateLayout &L)
{
    return (size_t)L.off_rec + (size_t)batch * H * (size_t)L.rec_bytes;
}

// alpha_h of Eq. 2: required and finite when o_lr is given, else unused.
fs_status local_alpha(int32_t H, const float *alpha_h, const void *o_lr, LocalConsts *lc)
{
    if (!o_lr)
        return FS_OK;
    if (!alpha_h)
        return FS_ERR_INVALID;
    for (int h = 0; h < H; ++h) {
        if (!std::isfinite(alpha_h[h]))
            return FS_ERR_INVALID;
        lc->alpha[h] = alpha_h[h];
    }
    return FS_OK;
}

// ---- FS-B ----
FsbLayout fsb_layout(const Geometry &g)
{
    FsbLayout L;
    std::memset(&L, 0, sizeof(L));
    const int64_t last = (int64_t)(g.NB - 1) * (g.B / g.s); // cells available to the last block
    L.Mu = g.M < last ? g.M : last;
    int levels = 0;
    while (levels < kFsbMaxLevels && ((int64_t)1 << levels) <= L.Mu)
        ++levels;
    L.levels = levels;
    for (int k = 0; k < levels; ++k) {
        const int64_t chunks = ((L.Mu >> k) + 1) / 2; // chunks of 2^k cells at even multiples of 2^k
        L.chunk_base[k + 1] = L.chunk_base[k] + chunks;
        L.node_base[k + 1] = L.node_base[k] + chunks * ((int64_t(2) << k) - 1);
    }
    L.chunks = L.chunk_base[levels];
    L.nodes = L.node_base[levels];
    return L;
}

struct FsbWorkspace {
    size_t kbar, kbar64, a, a64, adm, cnt, node_mu, node_meta, sel, total;
};

FsbWorkspace fsb_workspace(const Geometry &g, const FsbLayout &L)
{
    FsbWorkspace W;
    size_t off = 0;
    const size_t cells = (size_t)g.bh * (g.M > 0 ? g.M : 1);
    W.kbar = off;
    off += align_up(cells * g.d * sizeof(float));
    W.kbar64 = off;
    off += align_up(cells * g.d * sizeof(double));
    W.a = off;
    off += align_up(cells * sizeof(float));
    W.a64 = off;
    off += align_up(cells * sizeof(double));
    W.adm = off;
    off += align_up(cells * sizeof(int32_t));
    W.cnt = off;
    off += align_up((size_t)g.bh * (g.M + 1) * sizeof(int32_t));
    W.node_mu = off;
    off += align_up((size_t)g.bh * 2 * (L.nodes > 0 ? L.nodes : 1) * g.d * sizeof(float));
    W.node_meta = off;
    off += align_up((size_t)g.bh * 2 * (L.nodes > 0 ? L.nodes : 1) * sizeof(FsbNodeMeta));
    W.sel = off;
    off += align_up((size_t)g.bh * g.N * g.K * sizeof(int32_t));
    W.total = off;
    return W;
}

// Workspace of fs_readout_backward, carved in this order (256-byte aligned).
struct BwdLayout {
    size_t du, lse, delta, masks, item_start, pstart, item_cell, multi_cell, partial, dg_part, dg2, total;
};

BwdLayout bwd_layout(const Geometry &g)
{
    const BwdSizes z = bwd_sizes(g);
    BwdLayout L;
    size_t off = 0;
    L.du = off;
    off += align_up((size_t)g.bh * g.N * g.d * sizeof(float)); // fp32, or two bf16 planes
    L.lse = off;
    off += align_up((size_t)g.bh * g.N * sizeof(float));
    L.delta = off;
    off += align_up((size_t)g.bh * g.N * sizeof(float));
    L.masks = off;
    off += align_up((size_t)g.bh * (g.M > 0 ? g.M : 1) * g.NB * 16);
    L.item_start = off;
    off += align_up((size_t)g.bh * (g.M + 1) * sizeof(int32_t));
    L.pstart = off;
    off += align_up((size_t)g.bh * (g.M + 1) * sizeof(int32_t));
    L.item_cell = off;
    off += align_up((size_t)g.bh * z.items_max * sizeof(int32_t));
    L.multi_cell = off;
    off += align_up((size_t)g.bh * (z.multi_max + 1) * sizeof(int32_t));
    L.partial = off;
    off += align_up((size_t)g.bh * z.p_max * 2 * 32 * g.d * sizeof(float));
    L.dg_part = off;
    off += align_up((size_t)g.bh * g.NB * g.d * sizeof(float));
    L.dg2 = off;
    off += align_up((size_t)g.H * 32 * g.d * sizeof(float));
    L.total = off;
    return L;
}

fs_status check_backward(const fs_shape *shape, const fs_params *prm)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    const Geometry g = geometry(shape, prm);
    // one workgroup per cell on the key side: keep the grid below 2^24 workgroups
    if (g.N > kBwdMaxTokens || (int64_t)g.bh * ((g.N + g.s - 1) / g.s) >= ((int64_t)1 << 24))
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

fs_status check_fsb(const fs_shape *shape, const fs_params *prm, const fs_fsb_params *fb)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    if (!fb)
        return FS_ERR_INVALID;
    if (fb->Wb < 1 || !(fb->c >= 0.0f) || !std::isfinite(fb->c))
        return FS_ERR_INVALID;
    if (fb->Wb > kFsbMaxBeam)
        return FS_ERR_UNSUPPORTED;
    const Geometry g = geometry(shape, prm);
    if (fsb_layout(g).Mu > kFsbMaxCells)
        return FS_ERR_UNSUPPORTED;
    return FS_OK;
}

} // namespace
} // namespace fsl

using namespace fsl;

FSL_EXPORT const char *fs_status_string(fs_status status)
{
    switch (status) {
    case FS_OK: return "ok";
    case FS_ERR_INVALID: return "invalid argument";
    case FS_ERR_UNSUPPORTED: return "unsupported configuration";
    case FS_ERR_WORKSPACE: return "workspace too small";
    case FS_ERR_STATE: return "decode state does not match the parameters";
    case FS_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

FSL_EXPORT fs_status fs_cell_summaries(const fs_shape *shape, const fs_params *prm, const void *k, float *kbar,
                                       float *a, uint16_t *kbar_split, float *kbar_norm, void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    const Geometry g = geometry(shape, prm);
    if (!k || ((!kbar || !a) && g.M > 0)) // no complete cell: nothing to write
        return FS_ERR_INVALID;
    return hip_status(launch_cell_summaries(g, k, kbar, a, g.bf16 ? kbar_split : nullptr, kbar_norm,
                                            static_cast<hipStream_t>(stream)));
}

FSL_EXPORT size_t fs_prune_workspace_bytes(const fs_shape *shape, const fs_params *prm)
{
    if (check_all(shape, prm) != FS_OK)
        return 0;
    const Geometry g = geometry(shape, prm);
    const size_t cells = (size_t)g.bh * (g.M > 0 ? g.M : 1);
    return align_up(cells * sizeof(int32_t)) + align_up(cells * sizeof(int64_t)); // exit blocks, priority order
}

FSL_EXPORT fs_status fs_prune_retained(const fs_shape *shape, const fs_params *prm, const float *a,
                                       int32_t *retained, int32_t *n_retained, void *workspace,
                                       size_t workspace_bytes, void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    if (!prm->prune || !a || !retained || !n_retained || !workspace)
        return FS_ERR_INVALID;
    if (workspace_bytes < fs_prune_workspace_bytes(shape, prm))
        return FS_ERR_WORKSPACE;
    const Geometry g = geometry(shape, prm);
    const size_t cells = (size_t)g.bh * (g.M > 0 ? g.M : 1);
    int32_t *death = static_cast<int32_t *>(workspace);
    int64_t *ord = reinterpret_cast<int64_t *>(static_cast<char *>(workspace) + align_up(cells * sizeof(int32_t)));
    return hip_status(launch_prune(g, a, death, ord, retained, n_retained, 1, static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_score_select(const fs_shape *shape, const fs_params *prm, const void *q, const float *kbar,
                                     const uint16_t *kbar_split, const float *a, const int32_t *retained,
                                     const int32_t *n_retained, const float *sigma_h, const float *lambda_h,
                                     int32_t *sel, void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(shape->H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    const Geometry g = geometry(shape, prm);
    if (!q || !sel || ((!kbar || !a) && g.M > 0) || (g.prune && (!retained || !n_retained)))
        return FS_ERR_INVALID;
    return hip_status(launch_score_topk(g, hc, q, kbar, g.bf16 ? kbar_split : nullptr, a,
                                        g.prune ? retained : nullptr, g.prune ? n_retained : nullptr, sel,
                                        static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_readout(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                                const void *v, const int32_t *sel, const float *gain, void *out, void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    if (!q || !k || !v || !sel || !out)
        return FS_ERR_INVALID;
    const Geometry g = geometry(shape, prm);
    return hip_status(launch_readout(g, q, k, v, sel, gain, out, static_cast<hipStream_t>(stream)));
}

FSL_EXPORT size_t fs_readout_backward_workspace_bytes(const fs_shape *shape, const fs_params *prm)
{
    if (check_backward(shape, prm) != FS_OK)
        return 0;
    return bwd_layout(geometry(shape, prm)).total;
}

FSL_EXPORT fs_status fs_readout_backward(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                                         const void *v, const int32_t *sel, const float *gain, const void *dout,
                                         float *dq, float *dk, float *dv, float *dgain, void *workspace,
                                         size_t workspace_bytes, void *stream)
{
    fs_status st = check_backward(shape, prm);
    if (st != FS_OK)
        return st;
    if (!q || !k || !v || !sel || !dout || !dq || !dk || !dv || !workspace)
        return FS_ERR_INVALID;
    const Geometry g = geometry(shape, prm);
    const BwdLayout L = bwd_layout(g);
    if (workspace_bytes < L.total)
        return FS_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    BwdBuffers w;
    w.du = ws + L.du;
    w.lse = reinterpret_cast<float *>(ws + L.lse);
    w.delta = reinterpret_cast<float *>(ws + L.delta);
    w.masks = ws + L.masks;
    w.item_start = reinterpret_cast<int32_t *>(ws + L.item_start);
    w.pstart = reinterpret_cast<int32_t *>(ws + L.pstart);
    w.item_cell = reinterpret_cast<int32_t *>(ws + L.item_cell);
    w.multi_cell = reinterpret_cast<int32_t *>(ws + L.multi_cell);
    w.partial = reinterpret_cast<float *>(ws + L.partial);
    w.dg_part = reinterpret_cast<float *>(ws + L.dg_part);
    w.dg2 = reinterpret_cast<float *>(ws + L.dg2);
    return hip_status(launch_readout_backward(g, w, q, k, v, sel, gain, dout, dq, dk, dv, gain ? dgain : nullptr,
                                              static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_select_readout(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                                       const void *v, const float *kbar, const uint16_t *kbar_split,
                                       const float *kbar_norm, const float *a, const int32_t *retained,
                                       const int32_t *n_retained, const float *sigma_h,
                                       const float *lambda_h, const float *gain, void *out, int32_t *sel,
                                       void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(shape->H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    const Geometry g = geometry(shape, prm);
    if (!q || !k || !v || !out || ((!kbar || !a) && g.M > 0) || (g.prune && (!retained || !n_retained)))
        return FS_ERR_INVALID;
    const bool fused = g.bf16 && kbar_split && (!g.prune || g.cap <= kFusedMaxCap);
    if (!fused && !sel)
        return FS_ERR_INVALID; // the two-kernel path passes the selections through `sel`
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t *ret = g.prune ? retained : nullptr;
    const int32_t *nr = g.prune ? n_retained : nullptr;
    if (fused)
        return hip_status(launch_route_readout(g, hc, q, k, v, kbar_split, kbar_norm, a, ret, nr, gain, out, sel, s));
    hipError_t e = launch_score_topk(g, hc, q, kbar, g.bf16 ? kbar_split : nullptr, a, ret, nr, sel, s);
    if (e == hipSuccess)
        e = launch_readout(g, q, k, v, sel, gain, out, s);
    return hip_status(e);
}

FSL_EXPORT size_t fs_prefill_workspace_bytes(const fs_shape *shape, const fs_params *prm)
{
    if (check_all(shape, prm) != FS_OK)
        return 0;
    return prefill_layout(geometry(shape, prm)).total;
}

namespace fsl {

fs_status prefill_check(const fs_shape *shape, const fs_params *prm, const void *q, const void *k, const void *v,
                        const float *sigma_h, const float *lambda_h, void *out, int32_t *sel, void *state,
                        size_t state_bytes, size_t *workspace_needed)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(shape->H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!k || (!out && !sel && !state))
        return FS_ERR_INVALID;
    if ((out || sel) && !q)
        return FS_ERR_INVALID;
    if (out && !v)
        return FS_ERR_INVALID;
    if (state) {
        st = check_decode_params(prm);
        if (st != FS_OK)
            return st;
        if (!v)
            return FS_ERR_INVALID;
        if (state_bytes != fs_decode_state_bytes(shape->batch, shape->H, shape->d, shape->dtype, prm))
            return FS_ERR_STATE;
    }
    *workspace_needed = prefill_layout(geometry(shape, prm)).total;
    return FS_OK;
}

} // namespace fsl

FSL_EXPORT fs_status fs_longrange_prefill(const fs_shape *shape, const fs_params *prm, const void *q, const void *k,
                                          const void *v, const float *sigma_h, const float *lambda_h,
                                          const float *gain, void *out, int32_t *sel, void *state,
                                          size_t state_bytes, void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    fs_status st = check_all(shape, prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(shape->H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!k || !workspace || (!out && !sel && !state))
        return FS_ERR_INVALID;
    if ((out || sel) && !q)
        return FS_ERR_INVALID;
    if (out && !v)
        return FS_ERR_INVALID;
    if (state) {
        st = check_decode_params(prm);
        if (st != FS_OK)
            return st;
        if (!v)
            return FS_ERR_INVALID;
        if (state_bytes != fs_decode_state_bytes(shape->batch, shape->H, shape->d, shape->dtype, prm))
            return FS_ERR_STATE;
    }
    const Geometry g = geometry(shape, prm);
    const PrefillLayout L = prefill_layout(g);
    if (workspace_bytes < L.total)
        return FS_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    float *kbar = reinterpret_cast<float *>(ws + L.kbar);
    uint16_t *ksplit = g.bf16 ? reinterpret_cast<uint16_t *>(ws + L.ksplit) : nullptr;
    float *knorm = g.bf16 ? reinterpret_cast<float *>(ws + L.knorm) : nullptr;
    float *a = reinterpret_cast<float *>(ws + L.a);
    int32_t *death = reinterpret_cast<int32_t *>(ws + L.death);
    int64_t *ord = reinterpret_cast<int64_t *>(ws + L.ord);
    int32_t *retained = reinterpret_cast<int32_t *>(ws + L.retained);
    int32_t *n_ret = reinterpret_cast<int32_t *>(ws + L.n_ret);
    int32_t *sel_buf = sel ? sel : reinterpret_cast<int32_t *>(ws + L.sel);
    hipStream_t s = static_cast<hipStream_t>(stream);

    const bool route = out || sel; // state-only calls skip scoring and readout
    const bool fused = out && g.bf16 && (!g.prune || g.cap <= kFusedMaxCap);
    hipError_t e = launch_cell_summaries(g, k, kbar, a, route ? ksplit : nullptr, fused ? knorm : nullptr, s);
    if (e == hipSuccess && g.prune)
        e = launch_prune(g, a, death, ord, retained, n_ret, route ? 1 : 0, s);
    if (e == hipSuccess && fused) {
        e = launch_route_readout(g, hc, q, k, v, ksplit, knorm, a, g.prune ? retained : nullptr,
                                 g.prune ? n_ret : nullptr, gain, out, sel, s);
    } else {
        if (e == hipSuccess && route)
            e = launch_score_topk(g, hc, q, kbar, ksplit, a, g.prune ? retained : nullptr,
                                  g.prune ? n_ret : nullptr, sel_buf, s);
        if (e == hipSuccess && out)
            e = launch_readout(g, q, k, v, sel_buf, gain, out, s);
    }
    if (e == hipSuccess && state) {
        const StateLayout SL = state_layout(g.d, shape->dtype, prm);
        const StateHeader hdr = state_header(shape->batch, shape->H, g.d, shape->dtype, prm, SL);
        e = launch_state_build(g, SL, hdr, state, k, v, kbar, a, death, s);
    }
    return hip_status(e);
}

FSL_EXPORT size_t fs_decode_state_bytes(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, const fs_params *prm)
{
    if (check_decode_dims(batch, H, d, dtype) != FS_OK || check_decode_params(prm) != FS_OK)
        return 0;
    return state_bytes_of(batch, H, state_layout(d, dtype, prm));
}

FSL_EXPORT fs_status fs_longrange_decode(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                                         void *state, size_t state_bytes, const void *q, const void *k_new,
                                         const void *v_new, const float *sigma_h, const float *lambda_h,
                                         const float *gain, void *out, int32_t *sel, void *stream)
{
    fs_status st = check_decode_dims(batch, H, d, dtype);
    if (st != FS_OK)
        return st;
    st = check_decode_params(prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!state || !q || !k_new || !v_new || !out)
        return FS_ERR_INVALID;
    if ((int64_t)batch * H > INT32_MAX)
        return FS_ERR_UNSUPPORTED;
    const StateLayout L = state_layout(d, dtype, prm);
    if (state_bytes != state_bytes_of(batch, H, L))
        return FS_ERR_STATE;
    const StateHeader expect = state_header(batch, H, d, dtype, prm, L);
    return hip_status(launch_decode_step(batch * H, H, d, dtype == FS_BF16 ? 1 : 0, prm->K, prm->P, prm->W, prm->eps,
                                         L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                         static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_decode_state_init(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                                          void *state, size_t state_bytes, void *stream)
{
    fs_status st = check_decode_dims(batch, H, d, dtype);
    if (st != FS_OK)
        return st;
    st = check_decode_params(prm);
    if (st != FS_OK)
        return st;
    if (!state)
        return FS_ERR_INVALID;
    if ((int64_t)batch * H > 65535)
        return FS_ERR_UNSUPPORTED;
    const StateLayout L = state_layout(d, dtype, prm);
    if (state_bytes != state_bytes_of(batch, H, L))
        return FS_ERR_STATE;
    const StateHeader hdr = state_header(batch, H, d, dtype, prm, L);
    return hip_status(launch_state_init(batch * H, L, hdr, state, static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_longrange_prefill_chunk(const fs_params *prm, int32_t batch, int32_t H, int32_t d,
                                                fs_dtype dtype, void *state, size_t state_bytes, int64_t n,
                                                const void *q, const void *k, const void *v, const float *sigma_h,
                                                const float *lambda_h, const float *gain, void *out, int32_t *sel,
                                                void *stream)
{
    fs_status st = check_decode_dims(batch, H, d, dtype);
    if (st != FS_OK)
        return st;
    st = check_decode_params(prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!state || !q || !k || !v || !out || n < 1)
        return FS_ERR_INVALID;
    if (n > kMaxChunk || (int64_t)batch * H > 65535)
        return FS_ERR_UNSUPPORTED;
    const StateLayout L = state_layout(d, dtype, prm);
    if (state_bytes != state_bytes_of(batch, H, L))
        return FS_ERR_STATE;
    const StateHeader expect = state_header(batch, H, d, dtype, prm, L);
    if (dtype == FS_BF16) // block by block, as the whole-prompt prefill
        return hip_status(launch_chunk_blocks(batch * H, H, d, prm->K, prm->P, prm->W, prm->eps, L, expect, hc, state,
                                              q, k, v, gain, out, sel, n, static_cast<hipStream_t>(stream)));
    return hip_status(launch_decode_step(batch * H, H, d, 0, prm->K, prm->P, prm->W, prm->eps, L, expect, hc, state, q,
                                         k, v, gain, out, sel, static_cast<hipStream_t>(stream), (int)n));
}

FSL_EXPORT fs_status fs_local_window(const fs_shape *shape, int64_t w, float rope_base, const void *q, const void *k,
                                     const void *v, const float *alpha_h, const void *o_lr, void *out,
                                     void *stream)
{
    fs_status st = check_shape(shape);
    if (st != FS_OK)
        return st;
    if (!q || !k || !v || !out || w < 0 || !(rope_base > 1.0f) || !std::isfinite(rope_base))
        return FS_ERR_INVALID;
    if (w > kMaxLocalWindow)
        return FS_ERR_UNSUPPORTED;
    LocalConsts lc;
    std::memset(&lc, 0, sizeof(lc));
    lc.rope_base = rope_base;
    st = local_alpha(shape->H, alpha_h, o_lr, &lc);
    if (st != FS_OK)
        return st;
    fs_params p{32, 128, 0, 0, 1, 0, 0.0f}; // only the block size matters here
    const Geometry g = geometry(shape, &p);
    return hip_status(launch_local(g, lc, w, q, k, v, o_lr, out, static_cast<hipStream_t>(stream)));
}


FSL_EXPORT size_t fs_local_state_bytes(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w)
{
    if (check_local_dims(batch, H, d, dtype, w) != FS_OK)
        return 0;
    return local_state_bytes_of(batch, H, local_layout(d, dtype, w));
}

FSL_EXPORT fs_status fs_local_state_build(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w,
                                          float rope_base, void *state, size_t state_bytes, const void *k,
                                          const void *v, int64_t n, int64_t pos, void *stream)
{
    fs_status st = check_local_dims(batch, H, d, dtype, w);
    if (st != FS_OK)
        return st;
    if (!state || !(rope_base > 1.0f) || !std::isfinite(rope_base) || n < 0 || pos < n ||
        n < (pos < w ? pos : w) || (n > 0 && (!k || !v)))
        return FS_ERR_INVALID;
    const LocalStateLayout L = local_layout(d, dtype, w);
    if (state_bytes != local_state_bytes_of(batch, H, L))
        return FS_ERR_STATE;
    const LocalStateHeader hdr = local_header(batch, H, d, dtype, w, rope_base, L);
    return hip_status(launch_local_state_build(batch * H, d, dtype == FS_BF16 ? 1 : 0, L, hdr, state, k, v, n, pos,
                                               static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_local_decode(int32_t batch, int32_t H, int32_t d, fs_dtype dtype, int64_t w, void *state,
                                     size_t state_bytes, const void *q, const void *k_new, const void *v_new,
                                     const float *alpha_h, const void *o_lr, void *out, void *stream)
{
    fs_status st = check_local_dims(batch, H, d, dtype, w);
    if (st != FS_OK)
        return st;
    if (!state || !q || !k_new || !v_new || !out)
        return FS_ERR_INVALID;
    LocalConsts lc;
    std::memset(&lc, 0, sizeof(lc));
    st = local_alpha(H, alpha_h, o_lr, &lc);
    if (st != FS_OK)
        return st;
    const LocalStateLayout L = local_layout(d, dtype, w);
    if (state_bytes != local_state_bytes_of(batch, H, L))
        return FS_ERR_STATE;
    const LocalStateHeader expect = local_header(batch, H, d, dtype, w, 0.0f, L);
    return hip_status(launch_local_decode(batch * H, H, d, dtype == FS_BF16 ? 1 : 0, L, expect, lc, state, q, k_new,
                                          v_new, o_lr, out, static_cast<hipStream_t>(stream)));
}

FSL_EXPORT fs_status fs_attention_decode(const fs_params *prm, int32_t batch, int32_t H, int32_t d, fs_dtype dtype,
                                        void *state, size_t state_bytes, int64_t w, void *local_state,
                                        size_t local_state_bytes, const void *q, const void *k_new, const void *v_new,
                                        const float *sigma_h, const float *lambda_h, const float *gain,
                                        const float *alpha_h, void *out, int32_t *sel, void *stream)
{
    fs_status st = check_local_dims(batch, H, d, dtype, w);
    if (st != FS_OK)
        return st;
    st = check_decode_params(prm);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!state || !local_state || !q || !k_new || !v_new || !out || !alpha_h)
        return FS_ERR_INVALID;
    LocalConsts lc;
    std::memset(&lc, 0, sizeof(lc));
    st = local_alpha(H, alpha_h, out, &lc); // out stands for o_lr: alpha is required
    if (st != FS_OK)
        return st;
    const StateLayout L = state_layout(d, dtype, prm);
    const LocalStateLayout LL = local_layout(d, dtype, w);
    if (state_bytes != state_bytes_of(batch, H, L) || local_state_bytes != local_state_bytes_of(batch, H, LL))
        return FS_ERR_STATE;
    const StateHeader expect = state_header(batch, H, d, dtype, prm, L);
    const LocalStateHeader lexpect = local_header(batch, H, d, dtype, w, 0.0f, LL);
    return hip_status(launch_attn_decode(batch * H, H, d, dtype == FS_BF16 ? 1 : 0, prm->K, prm->P, prm->W, prm->eps,
                                         L, expect, hc, state, LL, lexpect, lc, local_state, q, k_new, v_new, gain,
                                         out, sel, static_cast<hipStream_t>(stream)));
}

FSL_EXPORT size_t fs_fsb_workspace_bytes(const fs_shape *shape, const fs_params *prm, const fs_fsb_params *fb)
{
    if (check_fsb(shape, prm, fb) != FS_OK)
        return 0;
    const Geometry g = geometry(shape, prm);
    return fsb_workspace(g, fsb_layout(g)).total;
}

FSL_EXPORT fs_status fs_fsb_prefill(const fs_shape *shape, const fs_params *prm, const fs_fsb_params *fb,
                                    const void *q, const void *k, const void *v, const float *sigma_h,
                                    const float *lambda_h, const float *tau_h, const float *gain, void *out,
                                    int32_t *sel, int32_t *cand, void *workspace, size_t workspace_bytes,
                                    void *stream)
{
    fs_status st = check_fsb(shape, prm, fb);
    if (st != FS_OK)
        return st;
    HeadConsts hc;
    st = check_heads(shape->H, sigma_h, lambda_h, &hc);
    if (st != FS_OK)
        return st;
    if (!q || !k || !tau_h || !workspace || (!out && !sel && !cand) || (out && !v))
        return FS_ERR_INVALID;
    FsbConsts fc;
    std::memset(&fc, 0, sizeof(fc));
    for (int h = 0; h < shape->H; ++h) {
        if (!std::isfinite(tau_h[h]))
            return FS_ERR_INVALID;
        fc.tau[h] = (double)tau_h[h];
    }
    fc.Wb = fb->Wb;
    fc.c = fb->c;
    const Geometry g = geometry(shape, prm);
    const FsbLayout L = fsb_layout(g);
    const FsbWorkspace W = fsb_workspace(g, L);
    if (workspace_bytes < W.total)
        return FS_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    float *kbar = reinterpret_cast<float *>(ws + W.kbar);
    double *kbar64 = reinterpret_cast<double *>(ws + W.kbar64);
    float *a = reinterpret_cast<float *>(ws + W.a);
    double *a64 = reinterpret_cast<double *>(ws + W.a64);
    int32_t *adm = reinterpret_cast<int32_t *>(ws + W.adm);
    int32_t *cnt = reinterpret_cast<int32_t *>(ws + W.cnt);
    float *node_mu = reinterpret_cast<float *>(ws + W.node_mu);
    FsbNodeMeta *node_meta = reinterpret_cast<FsbNodeMeta *>(ws + W.node_meta);
    int32_t *sel_buf = sel ? sel : reinterpret_cast<int32_t *>(ws + W.sel);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_cell_summaries(g, k, kbar, a, nullptr, nullptr, s, kbar64, a64);
    if (e == hipSuccess)
        e = launch_fsb(g, L, hc, fc, q, k, kbar64, a, a64, adm, cnt, node_mu, node_meta, sel_buf, cand, s);
    if (e == hipSuccess && out)
        e = launch_readout(g, q, k, v, sel_buf, gain, out, s);
    return hip_status(e);
}
