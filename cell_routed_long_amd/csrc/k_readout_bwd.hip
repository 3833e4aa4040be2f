// Readout backward (FreeSolo, Sec. 3.3 "Training": the top-P and top-K
// indices receive no gradient, the shared projections learn through the
// selected-token readout; App. D.4).  For each query i with selection S_i:
//   o_i = g * u_i r_i,  u_i = sum_{j in S_i} p_ij v_j,  p_i = softmax(q_i k_j / sqrt(d)),
//   r_i = 1 / sqrt(|u_i|^2 / d + eps)                                   (Eq. 9, Eq. 17)
// and, given dout_i = dL/do_i, with the selection held fixed:
//   du_i   = r_i g*dout_i - (r_i^3 / d)(sum_f g_f dout_if u_if) u_i
//   dg    += r_i dout_i * u_i
//   dP_ij  = du_i . v_j,   Delta_i = sum_j p_ij dP_ij = du_i . u_i,   dS_ij = p_ij (dP_ij - Delta_i)
//   dq_i   = sum_j dS_ij k_j / sqrt(d),  dk_j += dS_ij q_i / sqrt(d),  dv_j += p_ij du_i.
//
// No floating-point atomics anywhere: the results are deterministic.
//
// bwd_query_kernel, one workgroup per (sequence, head, 128-query block), four
// waves of 32 queries, over the union of the cells its queries selected (as
// the forward readout):
//   pass A recomputes the forward (logits, online softmax, u), then per query
//   du (as bf16 hi + lo planes for bf16 tensors), Delta and the log-sum-exp of
//   the logits go to a workspace for the key side; each wave sums its queries'
//   gain gradients; and for every cell available to the block a 128-bit mask of
//   the block's rows that selected it is written (cell-major, so the key side
//   reads one cell's masks in a row);
//   pass B gathers each cell again and forms, on the matrix cores,
//     S^T = K Q^T, p = 2^(S^T log2(e)/sqrt(d) - lse), dP^T = V du^T,
//     dS^T = p (dP^T - Delta), dQ^T += K^T dS^T.
//   du never leaves the registers between the passes: the V rows of pass B are
//   stored with their features in the order in which a lane holds du after
//   pass A, so du is the product's B operand as it stands.
//
// The key side balances a very uneven load: under the norm prior most queries
// of a head pick the same few high-norm cells, so one cell can carry thousands
// of queries while most carry none.  bwd_plan_kernel counts each cell's queries
// from the masks and cuts its ascending query list into chunks of at most
// kChunk; bwd_key_kernel runs one wave per chunk and forms, 32 queries at a
// time, with the cell's keys and values kept in registers,
//     S = Q K^T, p = 2^(S log2(e)/sqrt(d) - lse), dP = du V^T, dS = p (dP - Delta),
//     dV += P^T du, dK += dS^T Q;
// a cell of one chunk writes its rows from the wave, the chunks of a larger
// cell write partial sums that bwd_reduce_kernel adds in chunk order.  Every
// row of dk and dv is written (zero where no query selected the token).
//
// bwd_gain_partial_kernel and bwd_gain_kernel sum the per-block gain gradients
// over the batch and blocks in two fixed-order levels.
//
// Precision: q, k, v and dout are exact in bf16; fp32 operands of a product
// (p, du, dS) are split into bf16 hi + lo parts (products with an exact bf16
// operand take two matrix products, p du takes three), so every product keeps
// about 16 mantissa bits before fp32 accumulation.  fp32 tensors use the fp32
// matrix cores.
#include "fsl_internal.h"
#include "readout_math.h"

#include <type_traits>

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kWin = 16; // query blocks whose masks one list window of the key side covers
// Waves per key-side workgroup.  The waves share nothing, and a workgroup holds its LDS until
// its slowest wave ends: with one wave per workgroup a wave with a long chunk never keeps
// the slots of short ones.
constexpr int kKeyWaves = 1;

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Split 8 fp32 values into bf16 hi + lo operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) { split_bf16x8(x, hi, lo); }

// ---- query side --------------------------------------------------------------

template <typename T, int D>
struct QuerySmem;

template <int D>
struct alignas(16) QuerySmem<uint16_t, D> {
    static constexpr int kStrideR = D + 8;  // bf16 elements per row of a 32-row cell tile
    static constexpr int kStrideV = 32 + 8; // bf16 elements per row of a transposed cell tile
    static constexpr int kStrideT = D + 8;  // bf16 elements per row of the 128-row tile
    union {
        struct {
            uint16_t k[32][kStrideR];
            uint16_t vt[D][kStrideV]; // V^T, tokens at vt_pos
        } a;
        struct {
            uint16_t k[32][kStrideR];
            uint16_t vp[32][kStrideR]; // V rows, features at vt_pos within each group of 32
            uint16_t kt[D][kStrideV];  // K^T, tokens at vt_pos
        } b;
        uint16_t tile[128][kStrideT]; // the q tile at entry, the dout tile after pass A
    };
};

template <int D>
struct alignas(16) QuerySmem<float, D> {
    static constexpr int kStride = D + 1;
    float k[32][kStride];
    float v[32][kStride];
};

template <typename T, int D, int KT>
__global__ __launch_bounds__(kThreads, sizeof(T) == 4 && D == 128 ? 1 : 2) void bwd_query_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const int32_t *__restrict__ sel,
    const float *__restrict__ gain, const T *__restrict__ dout, float *__restrict__ dq, void *__restrict__ du_ws,
    float *__restrict__ lse_ws, float *__restrict__ delta_ws, u32x4 *__restrict__ masks,
    float *__restrict__ dg_part, int64_t N, int64_t M, int NB, int H, int cells_per_block, float eps,
    int64_t plane)
{
    __shared__ QuerySmem<T, D> sm;
    __shared__ int32_t sel_s[128][KT];
    __shared__ int32_t ulist[128 * KT];
    __shared__ uint32_t umask[128 * KT][4];
    __shared__ float dg_s[4][D];
    __shared__ int32_t n_u;
    extern __shared__ uint32_t bitmap[]; // ceil(M / 32) words

    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int s = 32;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int beta = (int)(lb % (uint32_t)NB);
    const int64_t head = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(head % H);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t q0 = (int64_t)beta * 128;
    const int64_t qi = q0 + wave * 32 + col;
    const bool q_ok = qi < N;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;
    const int n_words = (int)((n_avail + 31) / 32);

    // ---- the block's selections, their union (ascending ids) ----
    for (int w = threadIdx.x; w < n_words; w += kThreads)
        bitmap[w] = 0u;
    for (int x = threadIdx.x; x < 128 * KT; x += kThreads) {
        const int r = x / KT, j = x % KT;
        int32_t c = -1;
        if (q0 + r < N)
            c = sel[(head * N + q0 + r) * KT + j];
        if (c >= n_avail)
            c = -1; // not a cell of this block's prefix: ignored, as by the forward readout
        sel_s[r][j] = c;
        umask[x][0] = umask[x][1] = umask[x][2] = umask[x][3] = 0u;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < 128 * KT; x += kThreads) {
        const int32_t c = sel_s[x / KT][x % KT];
        if (c >= 0)
            atomicOr(&bitmap[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    if (wave == 0) {
        int total = 0;
        for (int base = 0; base < n_words; base += kWave) {
            const int w = base + lane;
            const uint32_t bits = w < n_words ? bitmap[w] : 0u;
            const int cnt = __popc(bits);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(incl, o, kWave);
                if (lane >= o)
                    incl += y;
            }
            int pos = total + incl - cnt;
            uint32_t b = bits;
            while (b) {
                const int bit = __ffs(b) - 1;
                b &= b - 1u;
                if (pos < 128 * KT)
                    ulist[pos] = w * 32 + bit;
                ++pos;
            }
            total += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            n_u = total < 128 * KT ? total : 128 * KT;
    }
    __syncthreads();
    const int nU = n_u;

    // rows of each union cell: position of the cell in ulist by binary search
    for (int x = threadIdx.x; x < 128 * KT; x += kThreads) {
        const int32_t c = sel_s[x / KT][x % KT];
        if (c < 0)
            continue;
        int lo = 0, hi = nU - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (ulist[mid] < c)
                lo = mid + 1;
            else
                hi = mid;
        }
        const int r = x / KT;
        atomicOr(&umask[lo][r >> 5], 1u << (r & 31));
    }

    int my_sel[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j)
        my_sel[j] = sel_s[wave * 32 + col][j];

    // ---- query fragments ----
    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
    QFrag qf[KC];
    const int rows = (int)(N - q0 < 128 ? N - q0 : 128);
    if constexpr (kBf16) {
        tile_load_bf16<D, kThreads>(&sm.tile[0][0], sm.kStrideT, q + (head * N + q0) * D, rows);
        __syncthreads();
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            qf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.tile[wave * 32 + col][kc * 16 + half * 8]));
    } else {
        const T *qrow = q + (head * N + (q_ok ? qi : 0)) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            qf[kc] = q_ok ? qrow[kc * 2 + half] : 0.0f;
    }

    // cell masks to the key side: [head][cell][block], zero for available cells no row selected
    if constexpr (!kBf16)
        __syncthreads(); // umask complete (the bf16 path synchronised after its tile load)
    {
        u32x4 *mh = masks + head * M * NB + beta;
        for (int x = threadIdx.x; x < nU; x += kThreads)
            mh[(int64_t)ulist[x] * NB] = u32x4{umask[x][0], umask[x][1], umask[x][2], umask[x][3]};
        for (int64_t c = threadIdx.x; c < n_avail; c += kThreads)
            if (!((bitmap[c >> 5] >> (c & 31)) & 1u))
                mh[c * NB] = u32x4{0u, 0u, 0u, 0u};
    }

    // ---- gather roles (bf16): thread (tp, fc) moves tokens 2tp, 2tp+1, features 8fc..8fc+7 ----
    constexpr int CPR = D / 8;
    const int tp = threadIdx.x & 15;
    const int fc = threadIdx.x >> 4;
    const bool gather = fc < CPR;
    u32x4 pk0, pk1, pv0, pv1;
    auto fetch = [&](int cell) {
        if (gather) {
            const T *kc_src = k + (head * N + (int64_t)cell * s + 2 * tp) * D + fc * 8;
            const T *vc_src = v + (head * N + (int64_t)cell * s + 2 * tp) * D + fc * 8;
            pk0 = *reinterpret_cast<const u32x4 *>(kc_src);
            pk1 = *reinterpret_cast<const u32x4 *>(kc_src + D);
            pv0 = *reinterpret_cast<const u32x4 *>(vc_src);
            pv1 = *reinterpret_cast<const u32x4 *>(vc_src + D);
        }
    };
    // the token pair (2tp, 2tp+1) of 8 features, as 8 words of a transposed tile
    auto store_t = [&](uint16_t (*dst)[QuerySmem<uint16_t, D>::kStrideV], const u32x4 &a0, const u32x4 &a1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t x0 = (a0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            const uint32_t x1 = (a1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            *reinterpret_cast<uint32_t *>(&dst[fc * 8 + e][vt_pos(2 * tp)]) = x0 | (x1 << 16);
        }
    };
    // f32: the cell's rows, element by element
    auto load_f32 = [&](int cell) {
        if constexpr (!kBf16) {
            const T *kc_src = k + (head * N + (int64_t)cell * s) * D;
            const T *vc_src = v + (head * N + (int64_t)cell * s) * D;
            for (int e = threadIdx.x; e < 32 * D; e += kThreads) {
                const int row = e / D, f = e % D;
                sm.k[row][f] = kc_src[(int64_t)row * D + f];
                sm.v[row][f] = vc_src[(int64_t)row * D + f];
            }
        }
    };
    auto is_mine = [&](int cell) {
        bool m = false;
#pragma unroll
        for (int j = 0; j < KT; ++j)
            m |= my_sel[j] == cell;
        return m;
    };

    constexpr int DT = D / 32;
    f32x16 acc_o[DT]; // pass A: O^T (unnormalised);  pass B: dQ^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc_o[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // ================= pass A: the forward readout =================
    if constexpr (kBf16) {
        if (nU > 0)
            fetch(ulist[0]);
    }
    for (int x = 0; x < nU; ++x) {
        const int cell = ulist[x];
        __syncthreads();
        if constexpr (kBf16) {
            if (gather) {
                *reinterpret_cast<u32x4 *>(&sm.a.k[2 * tp][fc * 8]) = pk0;
                *reinterpret_cast<u32x4 *>(&sm.a.k[2 * tp + 1][fc * 8]) = pk1;
                store_t(sm.a.vt, pv0, pv1);
            }
        } else {
            load_f32(cell);
        }
        __syncthreads();
        if constexpr (kBf16) {
            if (x + 1 < nU)
                fetch(ulist[x + 1]);
        }
        const bool mine = is_mine(cell);
        if (__ballot(mine) == 0ull)
            continue;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.0f;
        if constexpr (kBf16) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.a.k[col][kc * 16 + half * 8])),
                                qf[kc], acc);
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.k[col][kc * 2 + half], qf[kc], acc);
        }
        float p[16];
        const float alpha = softmax_cell(acc, mine, scale_log2, m_run, l_run, p);
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc_o[dt][r] *= alpha;
        }
        if constexpr (kBf16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bh, bl;
                split_bf16x8(&p[8 * kk], bh, bl);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 av =
                        as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.a.vt[dt * 32 + col][16 * kk + 8 * half]));
                    acc_o[dt] = mfma_bf16(av, bl, acc_o[dt]);
                    acc_o[dt] = mfma_bf16(av, bh, acc_o[dt]);
                }
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc_o[dt] = mfma_f32(sm.v[acc_row(r, half)][dt * 32 + col], p[r], acc_o[dt]);
        }
    }

    // ================= between the passes: du, Delta, lse, gain gradient =================
    // the lane holds features dt*32 + acc_row(r, half) of query col; u = O / l
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float so = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc_o[dt][r] *= inv_l; // now u
            so = fmaf(acc_o[dt][r], acc_o[dt][r], so);
        }
    so += shfl_xor_f(so, 32);
    const float rn = 1.0f / sqrtf(so * (1.0f / (float)D) + eps);
    // dout of the lane's features
    float go[DT][16];
    if constexpr (kBf16) {
        __syncthreads(); // pass A's last LDS reads are done: the tile area takes dout
        tile_load_bf16<D, kThreads>(&sm.tile[0][0], sm.kStrideT, reinterpret_cast<const uint16_t *>(dout) + (head * N + q0) * D,
                                    rows);
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const u32x2 w = *reinterpret_cast<const u32x2 *>(&sm.tile[wave * 32 + col][dt * 32 + 8 * rg + 4 * half]);
                go[dt][4 * rg + 0] = bf16_bits_to_f32(w[0] & 0xffffu);
                go[dt][4 * rg + 1] = bf16_bits_to_f32(w[0] >> 16);
                go[dt][4 * rg + 2] = bf16_bits_to_f32(w[1] & 0xffffu);
                go[dt][4 * rg + 3] = bf16_bits_to_f32(w[1] >> 16);
            }
    } else {
        const T *drow = dout + (head * N + (q_ok ? qi : 0)) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const u32x4 w = q_ok ? *reinterpret_cast<const u32x4 *>(drow + dt * 32 + 8 * rg + 4 * half)
                                     : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    go[dt][4 * rg + e] = __uint_as_float(w[e]);
            }
    }
    const float *gh = gain ? gain + (int64_t)h * D : nullptr;
    // gain gradient r dout * u, summed over the wave's queries (lanes of one half)
    if (gh) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t = rn * go[dt][r] * acc_o[dt][r];
#pragma unroll
                for (int o = 1; o < 32; o <<= 1)
                    t += shfl_xor_f(t, o);
                if (col == 0)
                    dg_s[wave][dt * 32 + acc_row(r, half)] = t;
            }
    }
    // g * dout, and sum_f g_f dout_f u_f
    float sgu = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (gh)
                go[dt][r] *= gh[dt * 32 + acc_row(r, half)];
            sgu = fmaf(go[dt][r], acc_o[dt][r], sgu);
        }
    sgu += shfl_xor_f(sgu, 32);
    const float corr = rn * rn * rn * (1.0f / (float)D) * sgu;
    float delta = 0.0f;
    const bool has = l_run > 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float du = has ? rn * go[dt][r] - corr * acc_o[dt][r] : 0.0f;
            delta = fmaf(du, acc_o[dt][r], delta);
            go[dt][r] = du; // go now holds du
        }
    delta += shfl_xor_f(delta, 32);
    const float lse = has ? m_run + __log2f(l_run) : 0.0f;
    if (q_ok) {
        if constexpr (kBf16) { // bf16 hi and lo planes, the operands the key side multiplies with
            uint16_t *hi = reinterpret_cast<uint16_t *>(du_ws) + (head * N + qi) * D;
            uint16_t *lo = hi + plane;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const float *x = &go[dt][4 * rg];
                    const uint32_t h01 = cvt_pk_bf16(x[0], x[1]), h23 = cvt_pk_bf16(x[2], x[3]);
                    const uint32_t l01 = cvt_pk_bf16(x[0] - __uint_as_float(h01 << 16),
                                                     x[1] - __uint_as_float(h01 & 0xffff0000u));
                    const uint32_t l23 = cvt_pk_bf16(x[2] - __uint_as_float(h23 << 16),
                                                     x[3] - __uint_as_float(h23 & 0xffff0000u));
                    *reinterpret_cast<u32x2 *>(hi + dt * 32 + 8 * rg + 4 * half) = u32x2{h01, h23};
                    *reinterpret_cast<u32x2 *>(lo + dt * 32 + 8 * rg + 4 * half) = u32x2{l01, l23};
                }
        } else {
            float *dst = reinterpret_cast<float *>(du_ws) + (head * N + qi) * D;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    *reinterpret_cast<u32x4 *>(dst + dt * 32 + 8 * rg + 4 * half) =
                        u32x4{__float_as_uint(go[dt][4 * rg]), __float_as_uint(go[dt][4 * rg + 1]),
                              __float_as_uint(go[dt][4 * rg + 2]), __float_as_uint(go[dt][4 * rg + 3])};
        }
        if (half == 0) {
            lse_ws[head * N + qi] = lse;
            delta_ws[head * N + qi] = delta;
        }
    }
    __syncthreads(); // dg_s complete; the tile area is free for pass B
    if (gh)
        for (int f = threadIdx.x; f < D; f += kThreads)
            dg_part[(head * NB + beta) * D + f] = ((dg_s[0][f] + dg_s[1][f]) + dg_s[2][f]) + dg_s[3][f];

    // du as the B operand of dP^T = V du^T: chunk kc = 2 dt + j is the lane's registers 8j..8j+7 of tile dt
    constexpr int KB = kBf16 ? D / 16 : 1;
    bf16x8 duh[KB], dul[KB];
    if constexpr (kBf16) {
#pragma unroll
        for (int kc = 0; kc < KB; ++kc) {
            float t[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                t[e] = go[kc >> 1][8 * (kc & 1) + e];
            split8(t, duh[kc], dul[kc]);
        }
    }

    // ================= pass B: dQ =================
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc_o[dt][r] = 0.0f;
    if constexpr (kBf16) {
        if (nU > 0)
            fetch(ulist[0]);
    }
    for (int x = 0; x < nU; ++x) {
        const int cell = ulist[x];
        __syncthreads();
        if constexpr (kBf16) {
            if (gather) {
                *reinterpret_cast<u32x4 *>(&sm.b.k[2 * tp][fc * 8]) = pk0;
                *reinterpret_cast<u32x4 *>(&sm.b.k[2 * tp + 1][fc * 8]) = pk1;
                store_t(sm.b.kt, pk0, pk1);
                // V rows with features at vt_pos within their group of 32: each half chunk of 4 stays together
                const int g0 = (fc & ~3) * 8;               // first feature of the group of 32
                const int p0 = g0 + vt_pos((fc & 3) * 8);     // features 8fc..8fc+3
                const int p1 = g0 + vt_pos((fc & 3) * 8 + 4); // features 8fc+4..8fc+7
                *reinterpret_cast<u32x2 *>(&sm.b.vp[2 * tp][p0]) = u32x2{pv0[0], pv0[1]};
                *reinterpret_cast<u32x2 *>(&sm.b.vp[2 * tp][p1]) = u32x2{pv0[2], pv0[3]};
                *reinterpret_cast<u32x2 *>(&sm.b.vp[2 * tp + 1][p0]) = u32x2{pv1[0], pv1[1]};
                *reinterpret_cast<u32x2 *>(&sm.b.vp[2 * tp + 1][p1]) = u32x2{pv1[2], pv1[3]};
            }
        } else {
            load_f32(cell);
        }
        __syncthreads();
        if constexpr (kBf16) {
            if (x + 1 < nU)
                fetch(ulist[x + 1]);
        }
        const bool mine = is_mine(cell);
        if (__ballot(mine) == 0ull)
            continue;
        f32x16 acc, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = dp[r] = 0.0f;
        if constexpr (kBf16) {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.b.k[col][kc * 16 + half * 8])),
                                qf[kc], acc);
                const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.b.vp[col][kc * 16 + half * 8]));
                dp = mfma_bf16(av, dul[kc], dp);
                dp = mfma_bf16(av, duh[kc], dp);
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.k[col][kc * 2 + half], qf[kc], acc);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dp = mfma_f32(sm.v[col][dt * 32 + acc_row(r, half)], go[dt][r], dp);
        }
        float ds[16];
        const float lse_eff = mine ? lse : INFINITY; // p = 0 for a cell the query did not select
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(fmaf(acc[r], scale_log2, -lse_eff));
            ds[r] = p * (dp[r] - delta);
        }
        if constexpr (kBf16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bh, bl;
                split_bf16x8(&ds[8 * kk], bh, bl);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 ak =
                        as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.b.kt[dt * 32 + col][16 * kk + 8 * half]));
                    acc_o[dt] = mfma_bf16(ak, bl, acc_o[dt]);
                    acc_o[dt] = mfma_bf16(ak, bh, acc_o[dt]);
                }
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc_o[dt] = mfma_f32(sm.k[acc_row(r, half)][dt * 32 + col], ds[r], acc_o[dt]);
        }
    }
    if (q_ok) {
        const float sc = 1.0f / sqrtf((float)D);
        float *dst = dq + (head * N + qi) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                *reinterpret_cast<u32x4 *>(dst + dt * 32 + 8 * rg + 4 * half) =
                    u32x4{__float_as_uint(acc_o[dt][4 * rg] * sc), __float_as_uint(acc_o[dt][4 * rg + 1] * sc),
                          __float_as_uint(acc_o[dt][4 * rg + 2] * sc), __float_as_uint(acc_o[dt][4 * rg + 3] * sc)};
    }
}

// ---- key side ---------------------------------------------------------------

// One workgroup per (sequence, head): each cell's query count from its masks,
// its chunks of at most kChunk queries (one chunk for a cell no query selected),
// the head's chunk table (chunk -> cell) and, for cells of several chunks, the
// first slot of their partial sums.  item_start[c], pstart[c]: exclusive prefix
// sums over the cells; item_start[M] = the head's chunks.
__global__ __launch_bounds__(256) void bwd_plan_kernel(const u32x4 *__restrict__ masks, int32_t *__restrict__ item_start,
                                                       int32_t *__restrict__ pstart, int32_t *__restrict__ item_cell,
                                                       int32_t *__restrict__ multi_cell, int64_t M, int NB,
                                                       int cells_per_block, int64_t items_max, int64_t multi_max)
{
    __shared__ int32_t n_it[kBwdMaxCells], n_p[kBwdMaxCells];
    __shared__ int32_t wsum[3][4];
    const int64_t head = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int64_t c = threadIdx.x; c < M; c += blockDim.x) {
        const u32x4 *mc = masks + (head * M + c) * NB;
        int cnt = 0;
        for (int bk = (int)(c / cells_per_block) + 1; bk < NB; ++bk) {
            const u32x4 m = mc[bk];
            cnt += __popc(m[0]) + __popc(m[1]) + __popc(m[2]) + __popc(m[3]);
        }
        const int n = cnt > 0 ? (cnt + kChunk - 1) / kChunk : 0; // 0: no query selected the cell
        n_it[c] = n;
        n_p[c] = n > 1 ? n : 0;
    }
    __syncthreads();
    // exclusive scans over the cells: thread t takes cells [t*per, (t+1)*per)
    const int per = (int)((M + 255) / 256);
    const int c0 = threadIdx.x * per;
    int si = 0, sp = 0, sm_ = 0;
    for (int x = 0; x < per; ++x)
        if (c0 + x < M) {
            si += n_it[c0 + x] > 0 ? n_it[c0 + x] : 1; // an unselected cell: one chunk that writes zeros
            sp += n_p[c0 + x];
            sm_ += n_p[c0 + x] > 0;
        }
    int ii = si, ip = sp, im = sm_;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int yi = __shfl_up(ii, o, kWave), yp = __shfl_up(ip, o, kWave), ym = __shfl_up(im, o, kWave);
        if (lane >= o) {
            ii += yi;
            ip += yp;
            im += ym;
        }
    }
    if (lane == kWave - 1) {
        wsum[0][wave] = ii;
        wsum[1][wave] = ip;
        wsum[2][wave] = im;
    }
    __syncthreads();
    int oi = ii - si, op = ip - sp, om = im - sm_;
    for (int w = 0; w < wave; ++w) {
        oi += wsum[0][w];
        op += wsum[1][w];
        om += wsum[2][w];
    }
    int32_t *is = item_start + head * (M + 1), *ps = pstart + head * (M + 1);
    int32_t *ic = item_cell + head * items_max, *mcl = multi_cell + head * (multi_max + 1);
    for (int x = 0; x < per; ++x) {
        const int64_t c = c0 + x;
        if (c >= M)
            break;
        is[c] = oi;
        ps[c] = op;
        if (n_it[c] == 0) // marked: the wave writes the cell's zero rows and nothing else
            ic[oi++] = -1 - (int32_t)c;
        for (int t = 0; t < n_it[c]; ++t)
            ic[oi + t] = (int32_t)c;
        if (n_p[c] > 0)
            mcl[1 + om++] = (int32_t)c;
        oi += n_it[c];
        op += n_p[c];
    }
    if (threadIdx.x == 255) {
        is[M] = oi;
        ps[M] = op;
        mcl[0] = om; // cells of several chunks
    }
}

template <typename T, int D>
struct KeySmem;

// bf16: the tile's q, du hi and du lo rows as pair words, word [m][f] = (row 2m, row 2m + 1) at
// feature f, so an 8-row B operand of one feature is four 4-byte reads
template <int D>
struct alignas(16) KeySmem<uint16_t, D> {
    static constexpr int kStride = D + 4; // words per pair row
    uint32_t pq[kKeyWaves][16][kStride];
    uint32_t ph[kKeyWaves][16][kStride];
    uint32_t pl[kKeyWaves][16][kStride];
};

template <int D>
struct alignas(16) KeySmem<float, D> {
    static constexpr int kStride = D + 1;
    float qr[kKeyWaves][32][kStride];
    float du[kKeyWaves][32][kStride];
};

// One wave per chunk of a cell's query list (kKeyWaves chunks of a head per
// workgroup, each wave on its own): the chunk's queries from the cell's masks,
// 32 at a time; the cell's rows are written once, by the wave itself when the
// cell has one chunk, through the partial sums and bwd_reduce_kernel otherwise.
template <typename T, int D>
__global__ __launch_bounds__(kKeyWaves * kWave, sizeof(T) == 2 && D == 64 ? 2 : 1) void bwd_key_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const void *__restrict__ du_ws,
    const float *__restrict__ lse_ws, const float *__restrict__ delta_ws, const u32x4 *__restrict__ masks,
    const int32_t *__restrict__ item_start, const int32_t *__restrict__ pstart, const int32_t *__restrict__ item_cell,
    float *__restrict__ partial, float *__restrict__ dk, float *__restrict__ dv, int64_t N, int64_t M, int NB,
    int cells_per_block, int64_t items_max, int64_t p_max, int64_t plane)
{
    __shared__ KeySmem<T, D> sm;
    __shared__ uint16_t qlist[kKeyWaves][kChunk]; // the chunk's query positions (N <= 65,536)
    __shared__ __align__(16) float lse_s[kKeyWaves][32];
    __shared__ __align__(16) float delta_s[kKeyWaves][32];

    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int s = 32;
    constexpr int DT = D / 32;
    const int64_t Gq = (items_max + kKeyWaves - 1) / kKeyWaves; // workgroups per head
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t head = (int64_t)(lb / (uint32_t)Gq);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t j = (int64_t)(lb % (uint32_t)Gq) * kKeyWaves + wave;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const int32_t *is = item_start + head * (M + 1);
    if (j >= is[M])
        return;
    const int32_t cj = item_cell[head * items_max + j];
    if (cj < 0) { // a cell no query selected: zero rows
        const int64_t cz = -1 - (int64_t)cj;
        float *dkc = dk + (head * N + cz * 32) * D, *dvc = dv + (head * N + cz * 32) * D;
        for (int e = lane * 4; e < 32 * D; e += kWave * 4) {
            *reinterpret_cast<u32x4 *>(dkc + e) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(dvc + e) = u32x4{0u, 0u, 0u, 0u};
        }
        return;
    }
    const int64_t c = cj;
    const int n_items = is[c + 1] - is[c];
    const int64_t lo_q = (j - is[c]) * (int64_t)kChunk, hi_q = lo_q + kChunk; // the chunk: list entries [lo_q, hi_q)

    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using Frag = typename std::conditional<kBf16, bf16x8, float>::type;
    Frag kf[KC], vf[KC];
    {
        const T *krow = k + (head * N + c * s + col) * D;
        const T *vrow = v + (head * N + c * s + col) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            if constexpr (kBf16) {
                kf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(krow + kc * 16 + half * 8));
                vf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(vrow + kc * 16 + half * 8));
            } else {
                kf[kc] = krow[kc * 2 + half];
                vf[kc] = vrow[kc * 2 + half];
            }
        }
    }
    f32x16 dk_acc[DT], dv_acc[DT]; // [token][feature]: lane col = feature dt*32 + col, rows = tokens
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dk_acc[dt][r] = dv_acc[dt][r] = 0.0f;

    // ---- the chunk's queries, in ascending order, from the cell's masks ----
    const int b0 = (int)(c / cells_per_block) + 1; // first block for which the cell is available
    const u32x4 *mc = masks + (head * M + c) * NB;
    uint16_t *ql = qlist[wave];
    int64_t cum = 0; // list entries before the window
    for (int win = b0; win < NB && cum < hi_q; win += kWin) {
        // lane = (block win + lane/4, mask word lane%4): the list comes out in ascending query order
        const int bk = win + (lane >> 2);
        const uint32_t bits = bk < NB ? mc[bk][lane & 3] : 0u;
        const int cnt = __popc(bits);
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(incl, o, kWave);
            if (lane >= o)
                incl += y;
        }
        const int nw = __shfl(incl, kWave - 1, kWave);
        if (cum + nw > lo_q) {
            int64_t pos = cum + incl - cnt;
            uint32_t b = bits;
            const int base = bk * 128 + (lane & 3) * 32;
            while (b && pos < hi_q) {
                const int bit = __ffs(b) - 1;
                b &= b - 1u;
                if (pos >= lo_q)
                    ql[pos - lo_q] = (uint16_t)(base + bit);
                ++pos;
            }
        }
        cum += nw;
    }
    const int n_q = (int)((cum < hi_q ? cum : hi_q) - lo_q); // queries of this chunk (0 for an unselected cell)
    wave_sync_lds();

    // ---- tiles of 32 queries ----
    const int64_t hN = head * N;
    if constexpr (kBf16) {
        // Lane (col, half) holds query slot col's q, du hi and du lo features kc*16 + half*8 .. +8:
        // the A operands of S = Q K^T and dP = du V^T as loaded.  A padding slot reads a real row
        // (the tile's first); its lse = +inf makes p = 0, so it adds nothing.  The next tile's rows
        // are requested once this tile's products have read the registers.
        const uint16_t *uhi = static_cast<const uint16_t *>(du_ws);
        u32x4 aq[KC], ah[KC], al[KC];
        float n_lse = INFINITY, n_delta = 0.0f;
        auto fetch = [&](int t0) {
            const int slot = t0 + col < n_q ? t0 + col : t0;
            const int64_t r = (hN + ql[slot]) * D + half * 8;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                aq[kc] = *reinterpret_cast<const u32x4 *>(q + r + kc * 16);
                ah[kc] = *reinterpret_cast<const u32x4 *>(uhi + r + kc * 16);
                al[kc] = *reinterpret_cast<const u32x4 *>(uhi + plane + r + kc * 16);
            }
            n_lse = INFINITY;
            n_delta = 0.0f;
            if (lane < 32 && t0 + lane < n_q) {
                n_lse = lse_ws[hN + ql[t0 + lane]];
                n_delta = delta_ws[hN + ql[t0 + lane]];
            }
        };
        // the pair words of this lane's 8 features: adjacent lanes (rows 2m, 2m + 1) swap two words;
        // the even lane then holds features +0..3 of both rows, the odd lane +4..7
        const bool odd = col & 1;
        auto put_pairs = [&](uint32_t (*tile)[KeySmem<uint16_t, D>::kStride], const u32x4 &w, int kc) {
            const uint32_t s0 = odd ? w[0] : w[2], s1 = odd ? w[1] : w[3];
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0xB1, 0xf, 0xf, true);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0xB1, 0xf, 0xf, true);
            const uint32_t o0 = odd ? w[2] : w[0], o1 = odd ? w[3] : w[1]; // own words kept
            const uint32_t lo0 = odd ? r0 : o0, hi0 = odd ? o0 : r0;       // row 2m in the low half
            const uint32_t lo1 = odd ? r1 : o1, hi1 = odd ? o1 : r1;
            const u32x4 pw = u32x4{(lo0 & 0xffffu) | (hi0 << 16), (lo0 >> 16) | (hi0 & 0xffff0000u),
                                   (lo1 & 0xffffu) | (hi1 << 16), (lo1 >> 16) | (hi1 & 0xffff0000u)};
            *reinterpret_cast<u32x4 *>(&tile[col >> 1][kc * 16 + half * 8 + (odd ? 4 : 0)]) = pw;
        };
        auto pairs8 = [&](const uint32_t (*tile)[KeySmem<uint16_t, D>::kStride], int kk, int f) {
            const int m0 = 8 * kk + 2 * half; // rows acc_row(8kk + e, half): pairs m0, m0+1, m0+4, m0+5
            return as_bf16x8(u32x4{tile[m0][f], tile[m0 + 1][f], tile[m0 + 4][f], tile[m0 + 5][f]});
        };
        if (n_q > 0)
            fetch(0);
        for (int t0 = 0; t0 < n_q; t0 += 32) {
            if (lane < 32) {
                lse_s[wave][lane] = n_lse;
                delta_s[wave][lane] = n_delta;
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                put_pairs(sm.pq[wave], aq[kc], kc);
                put_pairs(sm.ph[wave], ah[kc], kc);
                put_pairs(sm.pl[wave], al[kc], kc);
            }
            // ---- S = Q K^T and dP = du V^T: [query][token], lane col = token ----
            f32x16 sacc, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sacc[r] = dp[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                sacc = mfma_bf16(as_bf16x8(aq[kc]), kf[kc], sacc);
                dp = mfma_bf16(as_bf16x8(al[kc]), vf[kc], dp);
                dp = mfma_bf16(as_bf16x8(ah[kc]), vf[kc], dp);
            }
            if (t0 + 32 < n_q)
                fetch(t0 + 32);
            wave_sync_lds(); // pair tiles, lse and Delta visible to the whole wave
            float p[16], ds[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) { // rows 8g + 4 half + 0..3: one 16-byte read each
                const float4 l4 = *reinterpret_cast<const float4 *>(&lse_s[wave][8 * g + 4 * half]);
                const float4 d4 = *reinterpret_cast<const float4 *>(&delta_s[wave][8 * g + 4 * half]);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g + e;
                    p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lv[e]));
                    ds[r] = p[r] * (dp[r] - dv4[e]);
                }
            }
            // ---- dV += P^T du and dK += dS^T Q: [token][feature], contraction over the tile's queries ----
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 ph, pl, sh, sl;
                split_bf16x8(&p[8 * kk], ph, pl);
                split_bf16x8(&ds[8 * kk], sh, sl);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int f = dt * 32 + col;
                    const bf16x8 uhb = pairs8(sm.ph[wave], kk, f), ulb = pairs8(sm.pl[wave], kk, f);
                    const bf16x8 qb = pairs8(sm.pq[wave], kk, f);
                    dv_acc[dt] = mfma_bf16(pl, uhb, dv_acc[dt]);
                    dv_acc[dt] = mfma_bf16(ph, ulb, dv_acc[dt]);
                    dv_acc[dt] = mfma_bf16(ph, uhb, dv_acc[dt]);
                    dk_acc[dt] = mfma_bf16(sl, qb, dk_acc[dt]);
                    dk_acc[dt] = mfma_bf16(sh, qb, dk_acc[dt]);
                }
            }
            wave_sync_lds(); // the pair tiles are read: the next tile may overwrite them
        }
    } else {
        // fp32: rows staged in LDS, fetched when needed
        constexpr int CQ = D / 4; // 16-byte chunks per row
        constexpr int PER = 32 * CQ / kWave;
        for (int t0 = 0; t0 < n_q; t0 += 32) {
            const int nt = n_q - t0 < 32 ? n_q - t0 : 32;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int ch = lane + kWave * u, row = ch / CQ, c4 = (ch % CQ) * 4;
                u32x4 wq = u32x4{0u, 0u, 0u, 0u}, wu = wq;
                if (row < nt) {
                    const int64_t at = (hN + ql[t0 + row]) * D + c4;
                    wq = *reinterpret_cast<const u32x4 *>(q + at);
                    wu = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(du_ws) + at);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.qr[wave][row][c4 + e] = __uint_as_float(wq[e]);
                    sm.du[wave][row][c4 + e] = __uint_as_float(wu[e]);
                }
            }
            if (lane < 32) {
                const bool ok = lane < nt;
                lse_s[wave][lane] = ok ? lse_ws[hN + ql[t0 + lane]] : INFINITY; // p = 0 for padding rows
                delta_s[wave][lane] = ok ? delta_ws[hN + ql[t0 + lane]] : 0.0f;
            }
            wave_sync_lds();
            f32x16 sacc, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sacc[r] = dp[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                sacc = mfma_f32(sm.qr[wave][col][kc * 2 + half], kf[kc], sacc);
                dp = mfma_f32(sm.du[wave][col][kc * 2 + half], vf[kc], dp);
            }
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qs = acc_row(r, half);
                p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lse_s[wave][qs]));
                ds[r] = p[r] * (dp[r] - delta_s[wave][qs]);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qs = acc_row(r, half);
                    dv_acc[dt] = mfma_f32(p[r], sm.du[wave][qs][dt * 32 + col], dv_acc[dt]);
                    dk_acc[dt] = mfma_f32(ds[r], sm.qr[wave][qs][dt * 32 + col], dk_acc[dt]);
                }
            wave_sync_lds(); // the staged rows are read: the next tile may overwrite them
        }
    }

    // ---- out: lane (col, half) holds features dt*32 + col of tokens acc_row(r, half) ----
    const float sc = 1.0f / sqrtf((float)D);
    float *dkc, *dvc;
    if (n_items == 1) {
        dkc = dk + (head * N + c * s) * D;
        dvc = dv + (head * N + c * s) * D;
    } else { // partial sums of this chunk, added by bwd_reduce_kernel
        dkc = partial + ((head * p_max + pstart[head * (M + 1) + c] + (j - is[c])) * 2) * (32 * D);
        dvc = dkc + 32 * D;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t at = (int64_t)acc_row(r, half) * D + dt * 32 + col;
            dkc[at] = dk_acc[dt][r] * sc;
            dvc[at] = dv_acc[dt][r];
        }
}

// Workgroup m of a head adds, in chunk order, the partial sums of the head's m-th
// cell of several chunks; workgroup multi_max writes zeros for the tokens of the
// incomplete last cell.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float *__restrict__ partial,
                                                         const int32_t *__restrict__ item_start,
                                                         const int32_t *__restrict__ pstart,
                                                         const int32_t *__restrict__ multi_cell, float *__restrict__ dk,
                                                         float *__restrict__ dv, int64_t N, int64_t M, int D,
                                                         int64_t p_max, int64_t multi_max)
{
    constexpr int s = 32;
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int64_t m = (int64_t)(lb % (uint32_t)(multi_max + 1));
    const int64_t head = (int64_t)(lb / (uint32_t)(multi_max + 1));
    if (m == multi_max) {
        const int64_t r0 = M * s; // the incomplete last cell: its tokens are never read
        for (int64_t e = threadIdx.x; e < (N - r0) * D; e += blockDim.x) {
            dk[(head * N + r0) * D + e] = 0.0f;
            dv[(head * N + r0) * D + e] = 0.0f;
        }
        return;
    }
    if (M == 0)
        return; // no complete cell: the plan did not run
    const int32_t *mcl = multi_cell + head * (multi_max + 1);
    if (m >= mcl[0])
        return;
    const int64_t c = mcl[1 + m];
    const int32_t *is = item_start + head * (M + 1);
    const int n = is[c + 1] - is[c];
    const float *p0 = partial + (head * p_max + pstart[head * (M + 1) + c]) * 2 * (32 * D);
    float *dkc = dk + (head * N + c * s) * D, *dvc = dv + (head * N + c * s) * D;
    // thread: four consecutive floats of dk and of dv; the chunks' loads four at a time, added in chunk order
    const int64_t stride = 2 * 32 * D;
    for (int e = threadIdx.x * 4; e < 32 * D; e += blockDim.x * 4) {
        float4 tk = make_float4(0.0f, 0.0f, 0.0f, 0.0f), tv = tk;
        for (int x0 = 0; x0 < n; x0 += 4) {
            float4 a[4], b[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (x0 + u < n) {
                    a[u] = *reinterpret_cast<const float4 *>(p0 + (x0 + u) * stride + e);
                    b[u] = *reinterpret_cast<const float4 *>(p0 + (x0 + u) * stride + 32 * D + e);
                }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (x0 + u < n) {
                    tk.x += a[u].x; tk.y += a[u].y; tk.z += a[u].z; tk.w += a[u].w;
                    tv.x += b[u].x; tv.y += b[u].y; tv.z += b[u].z; tv.w += b[u].w;
                }
        }
        *reinterpret_cast<float4 *>(dkc + e) = tk;
        *reinterpret_cast<float4 *>(dvc + e) = tv;
    }
}

// dgain[h, f] = sum over sequences b and blocks of dg_part[b*H + h][block][f], in two
// levels: kGainGroups workgroups per head sum consecutive rows, then the groups in order
constexpr int kGainGroups = 32;
__global__ __launch_bounds__(256) void bwd_gain_partial_kernel(const float *__restrict__ dg_part,
                                                               float *__restrict__ dg2, int batch, int H, int NB, int D)
{
    __shared__ float part[256];
    const int h = blockIdx.x / kGainGroups, grp = blockIdx.x % kGainGroups;
    const int slices = 256 / D; // 4 (D = 64) or 2 (D = 128)
    const int f = threadIdx.x % D, sl = threadIdx.x / D;
    const int rows = batch * NB;
    const int r0 = (int)((int64_t)rows * grp / kGainGroups), r1 = (int)((int64_t)rows * (grp + 1) / kGainGroups);
    float t = 0.0f;
    for (int x = r0 + sl; x < r1; x += slices) {
        const int b = x / NB, beta = x % NB;
        t += dg_part[(((int64_t)b * H + h) * NB + beta) * D + f];
    }
    part[threadIdx.x] = t;
    __syncthreads();
    if (sl == 0) {
        float y = part[f];
        for (int j = 1; j < slices; ++j)
            y += part[j * D + f];
        dg2[((int64_t)h * kGainGroups + grp) * D + f] = y;
    }
}

__global__ __launch_bounds__(128) void bwd_gain_kernel(const float *__restrict__ dg2, float *__restrict__ dgain, int D)
{
    const int h = blockIdx.x;
    for (int f = threadIdx.x; f < D; f += blockDim.x) {
        float y = 0.0f;
        for (int g = 0; g < kGainGroups; ++g)
            y += dg2[((int64_t)h * kGainGroups + g) * D + f];
        dgain[(int64_t)h * D + f] = y;
    }
}

template <typename T, int D, int KT>
hipError_t launch_query(const Geometry &g, const BwdBuffers &w, const void *q, const void *k, const void *v,
                        const int32_t *sel, const float *gain, const void *dout, float *dq, hipStream_t st)
{
    dim3 grid((unsigned)((int64_t)g.NB * g.bh));
    const size_t words = (size_t)((g.M + 31) / 32);
    const size_t dyn = (words > 0 ? words : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((bwd_query_kernel<T, D, KT>), grid, dim3(kThreads), dyn, st, static_cast<const T *>(q),
                       static_cast<const T *>(k), static_cast<const T *>(v), sel, gain, static_cast<const T *>(dout),
                       dq, w.du, w.lse, w.delta, reinterpret_cast<u32x4 *>(w.masks), w.dg_part, g.N, g.M, g.NB, g.H,
                       g.B / g.s, g.eps, (int64_t)g.bh * g.N * g.d);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const Geometry &g, const BwdBuffers &w, const void *q, const void *k, const void *v,
                        const int32_t *sel, const float *gain, const void *dout, float *dq, float *dk, float *dv,
                        float *dgain, hipStream_t st)
{
    hipError_t e;
    switch (g.K) {
    case 1: e = launch_query<T, D, 1>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 2: e = launch_query<T, D, 2>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 3: e = launch_query<T, D, 3>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 4: e = launch_query<T, D, 4>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 5: e = launch_query<T, D, 5>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 6: e = launch_query<T, D, 6>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    case 7: e = launch_query<T, D, 7>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    default: e = launch_query<T, D, 8>(g, w, q, k, v, sel, gain, dout, dq, st); break;
    }
    if (e != hipSuccess)
        return e;
    const BwdSizes z = bwd_sizes(g);
    const u32x4 *masks = reinterpret_cast<const u32x4 *>(w.masks);
    if (g.M > 0) {
        hipLaunchKernelGGL(bwd_plan_kernel, dim3((unsigned)g.bh), dim3(256), 0, st, masks, w.item_start, w.pstart,
                           w.item_cell, w.multi_cell, g.M, g.NB, g.B / g.s, z.items_max, z.multi_max);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        hipLaunchKernelGGL((bwd_key_kernel<T, D>), dim3((unsigned)(((z.items_max + kKeyWaves - 1) / kKeyWaves) * g.bh)),
                           dim3(kKeyWaves * kWave), 0,
                           st, static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), w.du,
                           w.lse, w.delta, masks, w.item_start, w.pstart, w.item_cell, w.partial, dk, dv, g.N, g.M,
                           g.NB, g.B / g.s, z.items_max, z.p_max, (int64_t)g.bh * g.N * g.d);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((z.multi_max + 1) * g.bh)), dim3(256), 0, st, w.partial,
                       w.item_start, w.pstart, w.multi_cell, dk, dv, g.N, g.M, g.d, z.p_max, z.multi_max);
    if ((e = hipGetLastError()) != hipSuccess || !gain || !dgain)
        return e;
    hipLaunchKernelGGL(bwd_gain_partial_kernel, dim3((unsigned)(g.H * kGainGroups)), dim3(256), 0, st, w.dg_part, w.dg2,
                       g.bh / g.H, g.H, g.NB, g.d);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(bwd_gain_kernel, dim3((unsigned)g.H), dim3(128), 0, st, w.dg2, dgain, g.d);
    return hipGetLastError();
}

} // namespace

hipError_t launch_readout_backward(const Geometry &g, const BwdBuffers &w, const void *q, const void *k,
                                   const void *v, const int32_t *sel, const float *gain, const void *dout, float *dq,
                                   float *dk, float *dv, float *dgain, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_typed<uint16_t, 64>(g, w, q, k, v, sel, gain, dout, dq, dk, dv, dgain, st)
                         : launch_typed<uint16_t, 128>(g, w, q, k, v, sel, gain, dout, dq, dk, dv, dgain, st);
    return g.d == 64 ? launch_typed<float, 64>(g, w, q, k, v, sel, gain, dout, dq, dk, dv, dgain, st)
                     : launch_typed<float, 128>(g, w, q, k, v, sel, gain, dout, dq, dk, dv, dgain, st);
}

} // namespace fsl
