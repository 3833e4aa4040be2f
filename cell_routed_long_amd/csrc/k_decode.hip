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
//   (3) q is scored against A in fp64 (Eq. 7), its top-K cells are chosen by
//       rank (score desc, id asc), and the readout (Eq. 9) with RMSNorm
//       (Eq. 17) runs over their tokens.
// All branching on the position happens on the device, so a step can be
// captured in a HIP graph.  The prefill builds the state directly from its
// exit blocks (state_build_kernel), so no merge chain is replayed.
#include "fsl_internal.h"

#include <climits>

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kS = 32;          // tokens per cell
constexpr int kB = 128;         // tokens per query block
constexpr int kCpb = kB / kS;   // cells per block
constexpr int kKmax = 8;

template <typename T>
__device__ __forceinline__ float elem_to_f32(T x);
template <>
__device__ __forceinline__ float elem_to_f32<uint16_t>(uint16_t x) { return bf16_bits_to_f32(x); }
template <>
__device__ __forceinline__ float elem_to_f32<float>(float x) { return x; }

// n contiguous elements (n * sizeof(T) a multiple of 16 bytes, 16-byte aligned) -> fp32.
template <typename T, int n>
__device__ __forceinline__ void load_row_f32(const T *__restrict__ p, float (&x)[n])
{
    constexpr int EPC = 16 / (int)sizeof(T);
    static_assert(n % EPC == 0, "16-byte chunks");
#pragma unroll
    for (int c = 0; c < n / EPC; ++c) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p + c * EPC);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[c * 8 + 2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
                x[c * 8 + 2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[c * 4 + e] = __uint_as_float(w[e]);
        }
    }
}

struct Record {
    StateMeta *meta;
    int32_t *ret, *cell, *flags;
    float *a, *kbar;
    char *k, *v;
};

__device__ __forceinline__ Record record_at(char *state, const StateLayout &L, int64_t bh)
{
    char *rec = state + kStateHeaderBytes + bh * L.rec_bytes;
    Record R;
    R.meta = reinterpret_cast<StateMeta *>(rec);
    R.ret = reinterpret_cast<int32_t *>(rec + L.off_ret);
    R.cell = reinterpret_cast<int32_t *>(rec + L.off_cell);
    R.flags = reinterpret_cast<int32_t *>(rec + L.off_flags);
    R.a = reinterpret_cast<float *>(rec + L.off_a);
    R.kbar = reinterpret_cast<float *>(rec + L.off_kbar);
    R.k = rec + L.off_k;
    R.v = rec + L.off_v;
    return R;
}

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
        R.ret[x] = x < n_A ? x : -1;
    }
    if (t == 0) {
        R.meta->pos = N;
        R.meta->n_ret = n_A;
        R.meta->cur_slot = (N % kS) != 0 ? n_A + n_pend - 1 : -1;
    }
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

// ------------------------------------------------------------------------
// One decode step.  Thread t owns half (t & 1) of slot t >> 1 while scoring,
// so its 64 (or 32) fp32 mean-key values are loaded at entry, before the
// position is known.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(char *__restrict__ state, StateLayout L,
                                                               StateHeader expect, HeadConsts hc,
                                                               const T *__restrict__ q,
                                                               const T *__restrict__ k_new,
                                                               const T *__restrict__ v_new,
                                                               const float *__restrict__ gain,
                                                               T *__restrict__ out, int32_t *__restrict__ sel,
                                                               int H, int K, int P, int W, float eps)
{
    __shared__ int32_t s_cell[kMaxSlots], s_flags[kMaxSlots], s_ret[kMaxSlots], s_tmp[kMaxSlots];
    __shared__ float s_a[kMaxSlots];
    __shared__ double s_score[kMaxSlots];
    __shared__ float s_q[D];
    __shared__ T s_knew[D];
    __shared__ T s_vnew[D];
    __shared__ int32_t s_sel_slot[kKmax], s_sel_cell[kKmax];
    __shared__ float s_logit[kKmax * kS];
    __shared__ float s_p[kKmax * kS];
    __shared__ float s_upart[kWaves][D];
    __shared__ double s_colsum[kWaves][D];
    __shared__ double s_rowmax[kWaves];
    __shared__ float s_red[kWaves];
    __shared__ int32_t s_int[2];
    __shared__ float s_z;

    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
    T *o_row = out + bh * D;

    const StateHeader *hdr = reinterpret_cast<const StateHeader *>(state);
    const bool valid = hdr->magic == kStateMagic && hdr->version == kStateVersion && hdr->batch == expect.batch &&
                       hdr->H == expect.H && hdr->d == D && hdr->dtype == expect.dtype && hdr->P == P &&
                       hdr->W == W && hdr->n_slots == L.S && hdr->rec_bytes == L.rec_bytes;
    if (!valid) { // not a state of this shape: flag the output, leave the state alone
        if (t < D) {
            if constexpr (sizeof(T) == 2)
                o_row[t] = (T)0x7fc0u; // bf16 quiet NaN
            else
                o_row[t] = __uint_as_float(0x7fc00000u);
        }
        if (sel && t < K)
            sel[bh * K + t] = -1;
        return;
    }
    const Record R = record_at(state, L, bh);
    T *sk = reinterpret_cast<T *>(R.k);
    T *sv = reinterpret_cast<T *>(R.v);

    // ---- entry loads: position, slot tables, token, mean keys ----
    const int64_t i = R.meta->pos;
    int n_ret = R.meta->n_ret;
    n_ret = n_ret < 0 ? 0 : (n_ret > L.S ? L.S : n_ret);
    int cur = R.meta->cur_slot;
    if (t < kMaxSlots) {
        const bool in = t < L.S;
        s_cell[t] = in ? R.cell[t] : -1;
        s_flags[t] = in ? R.flags[t] : 0;
        s_a[t] = in ? R.a[t] : 0.0f;
        s_ret[t] = in ? R.ret[t] : -1;
    }
    if (t < D) {
        s_q[t] = elem_to_f32<T>(q[bh * D + t]);
        s_knew[t] = k_new[bh * D + t];
        s_vnew[t] = v_new[bh * D + t];
    }
    constexpr int FPT = D / 2; // mean-key features per thread
    const int my_slot = t >> 1, my_part = t & 1;
    float kb[FPT];
    if (my_slot < L.S) {
        const float *src = R.kbar + (int64_t)my_slot * D + my_part * FPT;
#pragma unroll
        for (int e = 0; e < FPT; e += 4) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(src + e);
            kb[e] = __uint_as_float(w[0]);
            kb[e + 1] = __uint_as_float(w[1]);
            kb[e + 2] = __uint_as_float(w[2]);
            kb[e + 3] = __uint_as_float(w[3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < FPT; ++e)
            kb[e] = 0.0f;
    }
    __syncthreads();

    const int64_t beta = i / kB;
    const int r = (int)(i % kS);
    const int64_t c_new = i / kS;

    // ---- (1) block boundary: Eq. 15 merge, then A = TopP u Recent_W ----
    if (i % kB == 0 && i > 0) {
        const int64_t d_lo = (beta - 1) * kCpb, d_hi = beta * kCpb;
        const int64_t rec_lo = d_hi > W ? d_hi - W : 0;
        int32_t c = -1;
        float av = 0.0f;
        bool cand = false;
        if (t < L.S) {
            c = s_cell[t];
            av = s_a[t];
            cand = c >= 0 && ((s_flags[t] & kFlagTop) || (c >= d_lo && c < d_hi));
        }
        if (t < kMaxSlots)
            s_tmp[t] = cand ? 1 : 0;
        __syncthreads();
        int rank = 0;
        if (cand)
            for (int u = 0; u < L.S; ++u)
                rank += (s_tmp[u] && ranks_before(s_a[u], s_cell[u], av, c)) ? 1 : 0;
        const bool top = cand && rank < P;
        const bool keep = c >= 0 && (top || (c >= rec_lo && c < d_hi));
        __syncthreads();
        if (t < kMaxSlots) {
            s_flags[t] = top ? kFlagTop : 0;
            s_cell[t] = keep ? c : -1;
            s_tmp[t] = keep ? 1 : 0;
            s_ret[t] = -1;
        }
        __syncthreads();
        if (keep) {
            int pos = 0;
            for (int u = 0; u < L.S; ++u)
                pos += (s_tmp[u] && s_cell[u] < c) ? 1 : 0;
            s_ret[pos] = t;
        }
        n_ret = __syncthreads_count(keep);
        if (t < L.S) {
            R.cell[t] = s_cell[t];
            R.flags[t] = s_flags[t];
            R.ret[t] = s_ret[t];
        }
        if (t == 0)
            R.meta->n_ret = n_ret;
    }

    // ---- (2) append the token; a new cell takes the lowest free slot ----
    if (r == 0) {
        if (wave == 0) {
            int found = -1;
            for (int base = 0; base < L.S; base += kWave) {
                const int x = base + lane;
                const uint64_t m = __ballot(x < L.S && s_cell[x] < 0);
                if (m) {
                    found = base + __ffsll((unsigned long long)m) - 1;
                    break;
                }
            }
            if (lane == 0)
                s_int[0] = found;
        }
        __syncthreads();
        cur = s_int[0];
        if (t == 0 && cur >= 0) {
            s_cell[cur] = (int32_t)c_new;
            R.cell[cur] = (int32_t)c_new;
            R.flags[cur] = 0;
            R.meta->cur_slot = cur;
        }
    }
    const bool can_append = cur >= 0 && cur < L.S; // false only for a corrupted state
    if (can_append && t < D) {
        sk[((int64_t)cur * kS + r) * D + t] = s_knew[t];
        sv[((int64_t)cur * kS + r) * D + t] = s_vnew[t];
    }
    if (r == kS - 1 && can_append) {
        // Eq. 5 for the completed cell: rows 0..s-2 from the slot, row s-1 from this token
        constexpr int FP = D / 8;
        const int row = t >> 3, part = t & 7;
        float x[FP];
        if (row == kS - 1) {
#pragma unroll
            for (int e = 0; e < FP; ++e)
                x[e] = elem_to_f32<T>(s_knew[part * FP + e]);
        } else {
            load_row_f32<T, FP>(sk + ((int64_t)cur * kS + row) * D + part * FP, x);
        }
        double col[FP];
        double sq = 0.0;
#pragma unroll
        for (int e = 0; e < FP; ++e) {
            col[e] = (double)x[e];
            sq += col[e] * col[e];
        }
        sq += shfl_xor_d(sq, 1);
        sq += shfl_xor_d(sq, 2);
        sq += shfl_xor_d(sq, 4);
        double mx = sq;
#pragma unroll
        for (int m = 8; m < kWave; m <<= 1)
            mx = fmax(mx, shfl_xor_d(mx, m));
#pragma unroll
        for (int e = 0; e < FP; ++e) {
#pragma unroll
            for (int m = 8; m < kWave; m <<= 1)
                col[e] += shfl_xor_d(col[e], m);
        }
        if (lane < 8) {
#pragma unroll
            for (int e = 0; e < FP; ++e)
                s_colsum[wave][part * FP + e] = col[e];
        }
        if (lane == 0)
            s_rowmax[wave] = mx;
        __syncthreads();
        if (t < D)
            R.kbar[(int64_t)cur * D + t] =
                (float)(((s_colsum[0][t] + s_colsum[1][t]) + (s_colsum[2][t] + s_colsum[3][t])) * (1.0 / 32.0));
        if (t == 0)
            R.a[cur] = (float)sqrt(fmax(fmax(s_rowmax[0], s_rowmax[1]), fmax(s_rowmax[2], s_rowmax[3])));
    }
    __syncthreads();

    // ---- (3) Eq. 7 over A in fp64, rank-based top-K ----
    if (t < kMaxSlots)
        s_tmp[t] = -1;
    if (t < kKmax) { // every rank below min(K, |A|) is written below; slot 0 keeps reads in bounds regardless
        s_sel_slot[t] = 0;
        s_sel_cell[t] = -1;
    }
    __syncthreads();
    if (t < n_ret && t < L.S) {
        const int u = s_ret[t];
        if (u >= 0 && u < L.S)
            s_tmp[u] = t;
    }
    __syncthreads();
    const bool scored = my_slot < L.S && s_tmp[my_slot] >= 0;
    double dot = 0.0;
    if (scored) {
#pragma unroll
        for (int e = 0; e < FPT; ++e)
            dot = fma((double)s_q[my_part * FPT + e], (double)kb[e], dot);
    }
    dot += shfl_xor_d(dot, 1);
    if (scored && my_part == 0) {
        const int32_t c = s_cell[my_slot];
        const double delta = (double)i - ((double)c + 0.5) * kS;
        const double g = erf(delta / (2.0 * (double)hc.sigma[h]));
        s_score[my_slot] = dot / sqrt((double)D) + (double)hc.lambda[h] * (double)s_a[my_slot] * g;
    }
    __syncthreads();
    if (scored && my_part == 0) {
        const double sc = s_score[my_slot];
        const int32_t c = s_cell[my_slot];
        int rank = 0;
        for (int x = 0; x < n_ret; ++x) {
            const int u = s_ret[x];
            if (u < 0 || u >= L.S)
                continue;
            const double su = s_score[u];
            const int32_t cu = s_cell[u];
            rank += (su > sc || (su == sc && cu < c)) ? 1 : 0;
        }
        if (rank < K) {
            s_sel_slot[rank] = my_slot;
            s_sel_cell[rank] = c;
        }
    }
    const int nT = n_ret < K ? n_ret : K;
    __syncthreads();

    // ---- readout: wave w gathers selections w, w + 4 ----
    constexpr int HALF = D / 2;  // key features per lane (two lanes per token)
    constexpr int FV = D / 64;   // value features per lane
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    float vpre[kS][FV];
    const int j0 = wave;
    if (j0 < nT) {
        const int slot = s_sel_slot[j0];
        const T *vb = sv + (int64_t)slot * kS * D + lane * FV;
#pragma unroll
        for (int row = 0; row < kS; ++row)
#pragma unroll
            for (int e = 0; e < FV; ++e)
                vpre[row][e] = elem_to_f32<T>(vb[(int64_t)row * D + e]);
    }
    for (int j = wave; j < nT; j += kWaves) {
        const int slot = s_sel_slot[j];
        float kr[HALF];
        load_row_f32<T, HALF>(sk + ((int64_t)slot * kS + (lane >> 1)) * D + (lane & 1) * HALF, kr);
        float d0 = 0.0f;
#pragma unroll
        for (int e = 0; e < HALF; ++e)
            d0 = fmaf(s_q[(lane & 1) * HALF + e], kr[e], d0);
        d0 += shfl_xor_f(d0, 1);
        if ((lane & 1) == 0)
            s_logit[j * kS + (lane >> 1)] = d0 * inv_sqrt_d;
    }
    __syncthreads();
    float m = -INFINITY;
    for (int x = lane; x < nT * kS; x += kWave)
        m = fmaxf(m, s_logit[x]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1)
        m = fmaxf(m, shfl_xor_f(m, o));
    for (int x = t; x < nT * kS; x += kThreads)
        s_p[x] = expf(s_logit[x] - m);
    __syncthreads();
    if (wave == 0) {
        float z = 0.0f;
        for (int x = lane; x < nT * kS; x += kWave)
            z += s_p[x];
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1)
            z += shfl_xor_f(z, o);
        if (lane == 0)
            s_z = z;
    }
    float uacc[FV];
#pragma unroll
    for (int e = 0; e < FV; ++e)
        uacc[e] = 0.0f;
    if (j0 < nT) {
#pragma unroll
        for (int row = 0; row < kS; ++row) {
            const float p = s_p[j0 * kS + row];
#pragma unroll
            for (int e = 0; e < FV; ++e)
                uacc[e] = fmaf(p, vpre[row][e], uacc[e]);
        }
    }
    for (int j = wave + kWaves; j < nT; j += kWaves) {
        const int slot = s_sel_slot[j];
        const T *vb = sv + (int64_t)slot * kS * D + lane * FV;
        for (int row = 0; row < kS; ++row) {
            const float p = s_p[j * kS + row];
#pragma unroll
            for (int e = 0; e < FV; ++e)
                uacc[e] = fmaf(p, elem_to_f32<T>(vb[(int64_t)row * D + e]), uacc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < FV; ++e)
        s_upart[wave][lane * FV + e] = uacc[e];
    __syncthreads();

    // ---- normalise, RMSNorm over d (Eq. 17), write ----
    float u = 0.0f;
    if (t < D && nT > 0)
        u = ((s_upart[0][t] + s_upart[1][t]) + (s_upart[2][t] + s_upart[3][t])) / s_z;
    float sq = t < D ? u * u : 0.0f;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1)
        sq += shfl_xor_f(sq, o);
    if (lane == 0)
        s_red[wave] = sq;
    __syncthreads();
    float ms = 0.0f;
#pragma unroll
    for (int w = 0; w < (D + kWave - 1) / kWave; ++w)
        ms += s_red[w];
    const float rs = 1.0f / sqrtf(ms / (float)D + eps);
    if (t < D) {
        const float gv = gain ? gain[(int64_t)h * D + t] : 1.0f;
        const float y = nT > 0 ? gv * u * rs : 0.0f;
        if constexpr (sizeof(T) == 2)
            o_row[t] = (T)f32_to_bf16_bits(y);
        else
            o_row[t] = y;
    }
    if (sel && t < K)
        sel[bh * K + t] = t < nT ? s_sel_cell[t] : -1;
    if (t == 0)
        R.meta->pos = i + 1;
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
                  const void *v_new, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    hipLaunchKernelGGL((decode_step_kernel<T, D>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, expect, hc, static_cast<const T *>(q),
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), gain, static_cast<T *>(out),
                       sel, H, K, P, W, eps);
    return hipGetLastError();
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
                              const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    if (bf16)
        return d == 64 ? step_t<uint16_t, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out,
                                              sel, st)
                       : step_t<uint16_t, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain,
                                               out, sel, st);
    return d == 64 ? step_t<float, 64>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                       st)
                   : step_t<float, 128>(bh, H, K, P, W, eps, L, expect, hc, state, q, k_new, v_new, gain, out, sel,
                                        st);
}

} // namespace fsl
