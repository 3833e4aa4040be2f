// Streaming decode of the FS-L long-range branch (FreeSolo, Sec. 3.3
// "Inference"; App. C "Bounded cache", Eq. 15).
//
// Per (sequence, head) the state keeps only the cells FS-L can still read: the
// retained set A of the current query block (at most P + W cells) and the
// B/s cells of the block being filled, each in a fixed-size slot holding its
// raw keys and values, fp32 mean key and norm.  One step, for a token at
// position i, is one launch with one workgroup per (sequence, head):
//   (1) i a block start (i % B == 0, i > 0): the B/s cells that just became
//       eligible (D) are merged into TopP by rank among TopP(C) u D (Eq. 15:
//       TopP(C u D) = TopP(TopP(C) u D)); A = TopP u Recent_W; every slot whose
//       cell is in neither is freed (a discarded cell can never re-enter TopP);
//   (2) the token's key and value are written into its cell's slot (a free
//       slot is taken when a cell starts); when the token completes the cell,
//       its mean key and largest key norm (Eq. 5) are formed in fp64 and
//       rounded once, exactly as the prefill summary kernel does;
//   (3) q is scored against A (Eq. 7, in fp32 with the prefill's arithmetic),
//       its top-K cells are chosen by rank (score desc, id asc), and the
//       readout (Eq. 9) with RMSNorm (Eq. 17) runs over their tokens: each
//       wave gathers one selected cell, keeps its softmax partials (max, sum,
//       weighted values) apart, and the cells are combined in rank order.
// All branching on the position happens on the device, so a step can be
// captured in a HIP graph.  The prefill builds the state directly from its
// exit blocks (state_build_kernel), so no merge chain is replayed.
#include "decode_lr.h"

namespace fsl {
namespace {

// ------------------------------------------------------------------------
// State from a prefill of N tokens: the query block of the last prompt token
// is beta = (N - 1) / B.  Its retained set is A_beta = {c < nav : c leaves
// TopP after beta} u Recent_W, nav = |C_beta|; the cells of block beta itself
// (the last one possibly partial) are pending.  Retained cells take slots
// 0..|A|-1 in ascending id order, pending cells the next ones.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void state_build_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader hdr, const T *__restrict__ k,
                                                               const T *__restrict__ v,
                                                               const float *__restrict__ kbar,
                                                               const float *__restrict__ a,
                                                               const int32_t *__restrict__ death, int64_t N,
                                                               int64_t M, int W)
{
    __shared__ int32_t s_cell[kMaxSlots];
    __shared__ int32_t s_flags[kMaxSlots];
    __shared__ int32_t s_wcnt[kWaves];
    __shared__ int32_t s_count;

    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    if (bh == 0 && t == 0)
        *reinterpret_cast<StateHeader *>(state) = hdr;
    const Record R = record_at(state, L, bh);
    const int32_t *dh = M > 0 ? death + bh * M : nullptr;
    const int64_t beta = (N - 1) / kB;
    const int64_t nav = beta * kCpb < M ? beta * kCpb : M;
    const int64_t recent0 = nav > W ? nav - W : 0;

    for (int x = t; x < kMaxSlots; x += kThreads) {
        s_cell[x] = -1;
        s_flags[x] = 0;
    }
    if (t == 0)
        s_count = 0;
    __syncthreads();
    // non-recent cells still in TopP(C_beta), ascending: block-wide compaction
    for (int64_t base = 0; base < recent0; base += kThreads) {
        const int64_t c = base + t;
        const bool keep = c < recent0 && dh[c] > beta;
        const uint64_t m = __ballot(keep);
        if (lane == 0)
            s_wcnt[wave] = __popcll(m);
        __syncthreads();
        int off = s_count;
        for (int w = 0; w < wave; ++w)
            off += s_wcnt[w];
        const int pos = off + __popcll(m & ((1ull << lane) - 1ull));
        if (keep && pos < L.S) {
            s_cell[pos] = (int32_t)c;
            s_flags[pos] = kFlagTop;
        }
        __syncthreads();
        if (t == 0) {
            int tot = 0;
            for (int w = 0; w < kWaves; ++w)
                tot += s_wcnt[w];
            s_count += tot;
        }
        __syncthreads();
    }
    const int n_old = s_count < L.S ? s_count : L.S;
    const int n_rec = (int)(nav - recent0);
    const int64_t p0 = beta * kCpb, p1 = (N + kS - 1) / kS;
    const int n_pend = (int)(p1 - p0);
    const int n_A = n_old + n_rec;
    // the host sizes S = P + W + B/s, so n_A + n_pend <= S always holds
    for (int x = t; x < n_rec; x += kThreads) {
        const int64_t c = recent0 + x;
        if (n_old + x < L.S) {
            s_cell[n_old + x] = (int32_t)c;
            s_flags[n_old + x] = dh[c] > beta ? kFlagTop : 0;
        }
    }
    for (int x = t; x < n_pend; x += kThreads)
        if (n_A + x < L.S)
            s_cell[n_A + x] = (int32_t)(p0 + x);
    __syncthreads();

    for (int x = t; x < L.S; x += kThreads) {
        const int32_t c = s_cell[x];
        R.cell[x] = c;
        R.flags[x] = s_flags[x];
        R.a[x] = (c >= 0 && c < M) ? a[bh * M + c] : 0.0f;
        R.ridx[x] = x < n_A ? x : -1;
    }
    if (t == 0) {
        R.meta->pos = N;
        R.meta->n_ret = n_A;
        R.meta->cur_slot = (N % kS) != 0 ? n_A + n_pend - 1 : -1;
    }
    if (t < kStateHints)
        R.meta->hint[t] = -1;
    for (int e = t; e < L.S * D; e += kThreads) {
        const int x = e / D, f = e % D;
        const int32_t c = s_cell[x];
        R.kbar[e] = (c >= 0 && c < M) ? kbar[(bh * M + c) * D + f] : 0.0f;
    }
    // raw keys and values of every occupied slot, 16-byte chunks
    constexpr int CPR = D * (int)sizeof(T) / 16;
    T *sk = reinterpret_cast<T *>(R.k);
    T *sv = reinterpret_cast<T *>(R.v);
    for (int e = t; e < L.S * kS * CPR; e += kThreads) {
        const int x = e / (kS * CPR);
        const int rem = e % (kS * CPR);
        const int row = rem / CPR, ch = rem % CPR;
        const int32_t c = s_cell[x];
        if (c < 0)
            continue;
        const int64_t j = (int64_t)c * kS + row;
        if (j >= N)
            continue;
        const int64_t src = (bh * N + j) * D;
        const int64_t dst = ((int64_t)x * kS + row) * D;
        reinterpret_cast<u32x4 *>(sk + dst)[ch] = reinterpret_cast<const u32x4 *>(k + src)[ch];
        reinterpret_cast<u32x4 *>(sv + dst)[ch] = reinterpret_cast<const u32x4 *>(v + src)[ch];
    }
}

template <typename T, int D, bool CHUNK>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader expect, HeadConsts hc,
                                                               const T *__restrict__ q,
                                                               const T *__restrict__ k_new,
                                                               const T *__restrict__ v_new,
                                                               const float *__restrict__ gain,
                                                               T *__restrict__ out, int32_t *__restrict__ sel,
                                                               int H, int K, int P, int W, float eps, int n_tok)
{
    decode_step_body<T, D, CHUNK ? kDecodeChunk : kDecodeStep>(state, L, expect, hc, q, k_new, v_new, gain, out, sel,
                                                               H, K, P, W, eps, n_tok, nullptr, nullptr);
}

template <typename T, int D>
hipError_t build_t(const Geometry &g, const StateLayout &L, const StateHeader &hdr, void *state, const void *k,
                   const void *v, const float *kbar, const float *a, const int32_t *death, hipStream_t st)
{
    hipLaunchKernelGGL((state_build_kernel<T, D>), dim3((unsigned)g.bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, hdr, static_cast<const T *>(k), static_cast<const T *>(v),
                       kbar, a, death, g.N, g.M, g.W);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t step_t(int32_t bh, int32_t H, int32_t K, int32_t P, int32_t W, float eps, const StateLayout &L,
                  const StateHeader &expect, const HeadConsts &hc, void *state, const void *q, const void *k_new,
                  const void *v_new, const float *gain, void *out, int32_t *sel, int n_tok, hipStream_t st)
{
    if (n_tok == 0) // a single decode step
        hipLaunchKernelGGL((decode_step_kernel<T, D, false>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                           static_cast<char *>(state), L, expect, hc, static_cast<const T *>(q),
                           static_cast<const T *>(k_new), static_cast<const T *>(v_new), gain,
                           static_cast<T *>(out), sel, H, K, P, W, eps, 1);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, D, true>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                           static_cast<char *>(state), L, expect, hc, static_cast<const T *>(q),
                           static_cast<const T *>(k_new), static_cast<const T *>(v_new), gain,
                           static_cast<T *>(out), sel, H, K, P, W, eps, n_tok);
    return hipGetLastError();
}

// An empty state at position 0: every slot free, nothing retained.
__global__ void state_init_kernel(char *__restrict__ state, StateLayout L, StateHeader hdr)
{
    const int64_t bh = blockIdx.x;
    if (bh == 0 && threadIdx.x == 0)
        *reinterpret_cast<StateHeader *>(state) = hdr;
    const Record R = record_at(state, L, bh);
    for (int x = threadIdx.x; x < L.S; x += blockDim.x) {
        R.cell[x] = -1;
        R.flags[x] = 0;
        R.ridx[x] = -1;
        R.a[x] = 0.0f;
    }
    if (threadIdx.x == 0) {
        R.meta->pos = 0;
        R.meta->n_ret = 0;
        R.meta->cur_slot = -1;
    }
    if (threadIdx.x < kStateHints)
        R.meta->hint[threadIdx.x] = -1;
}

} // namespace

hipError_t launch_state_build(const Geometry &g, const StateLayout &L, const StateHeader &hdr, void *state,
                              const void *k, const void *v, const float *kbar, const float *a,
                              const int32_t *death, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? build_t<uint16_t, 64>(g, L, hdr, state, k, v, kbar, a, death, st)
                         : build_t<uint16_t, 128>(g, L, hdr, state, k, v, kbar, a, death, st);
    return g.d == 64 ? build_t<float, 64>(g, L, hdr, state, k, v, kbar, a, death, st)
                     : build_t<float, 128>(g, L, hdr, state, k, v, kbar, a, death, st);
}

hipError_t launch_decode_step(int32_t bh, int32_t H, int32_t d, int32_t bf16, int32_t K, int32_t P, int32_t W,
                              float eps, const StateLayout &L, const StateHeader &expect, const HeadConsts &hc,
                              void *state, const void *q, const void *k_new, const void *v_new,
                              const float *gain, void *out, int32_t *sel, hipStream_t st, int n_tok)
{
    if (bf16)
        return d == 64 ? step_t<uint16_t, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out,
                                              sel, n_tok, st)
                       : step_t<uint16_t, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain,
                                               out, sel, n_tok, st);
    return d == 64 ? step_t<float, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                       n_tok, st)
                   : step_t<float, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                        n_tok, st);
}

hipError_t launch_state_init(int32_t bh, const StateLayout &L, const StateHeader &hdr, void *state, hipStream_t st)
{
    hipLaunchKernelGGL(state_init_kernel, dim3((unsigned)bh), dim3(kThreads), 0, st, static_cast<char *>(state), L,
                       hdr);
    return hipGetLastError();
}

} // namespace fsl

