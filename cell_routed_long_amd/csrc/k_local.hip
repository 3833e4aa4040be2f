// Local branch (FreeSolo, Sec. 3.2, Eqs. 3-4) with the branch combination of
// Sec. 3.1 (Eq. 2):
//   o_sr_i = softmax_{j in L_i}((R(i) q_i) . (R(j) k_j) / sqrt(d)) V_{L_i},
//   L_i = {j : 0 <= j <= i, i - j <= w},   out_i = o_sr_i + alpha_h o_lr_i,
// R(p) turning feature pair (2m, 2m+1) by p * theta_m, theta_m = base^(-2m/d)
// (RoFormer's rotation, which the page cites).
//
// One workgroup (4 waves, 32 queries each) per (sequence, head, 128-query
// block).  The block's window is walked in 32-token tiles: each tile's keys
// are rotated while they are staged in LDS and every wave applies the tile to
// its queries on the matrix cores,
//   S^T[32 tokens x 32 queries] = K_tile . Q^T,   O^T[d x 32] += V_tile^T . P^T,
// with an online softmax in which tokens outside a query's window get p = 0.
// Only offsets matter (Eq. 3: R(i)^T R(j) = R(j - i)), so positions are taken
// relative to the block start: every angle is below (w + 160) * theta_0, and
// cos/sin of (32 a + b) theta_m come from two small tables (per tile: 32 a,
// stepped from the first tile by 32 theta_m; per workgroup: b < 32), built in
// fp64, by the angle-addition formulas.
//
// Precision (bf16): the rotated q and k are split into bf16 hi + lo parts and
// the logits take three products (lo.hi and hi.lo in one accumulator, hi.hi in
// another, added at the end), so they keep ~16 mantissa bits; the probabilities are split
// likewise for P.V.  With q and k rounded to bf16 after the rotation the
// outputs of high-norm keys drift by up to 0.08 from the exact ones, and with
// bf16 probabilities by up to 0.02.  fp32 tensors use the fp32 matrix cores
// on the rotated values directly.
#include "fsl_internal.h"
#include "readout_math.h"

#include <type_traits>

namespace fsl {
namespace {

constexpr int kThreads = 256;


template <typename T, int D>
struct LocalSmem;

template <int D>
struct alignas(16) LocalSmem<uint16_t, D> {
    static constexpr int kStrideK = D + 8; // bf16 elements per K row
    static constexpr int kStrideV = 32 + 8;
    static constexpr int kStrideT = D + 8;
    union {
        struct {
            uint16_t k[2][32][kStrideK]; // rotated keys: hi and lo parts
            uint16_t vt[D][kStrideV];
        };
        uint16_t tile[128][kStrideT]; // rotated queries (hi, then lo) at entry; the output tile at exit
    };
};

template <int D>
struct alignas(16) LocalSmem<float, D> {
    static constexpr int kStride = D + 1;
    float k[32][kStride];
    float v[32][kStride];
};

__device__ __forceinline__ float2 sincos_pair(double ang)
{
    double sn, cs;
    sincos(ang, &sn, &cs);
    return make_float2((float)cs, (float)sn);
}

// (cos, sin) of (A + B) from those of A and B
__device__ __forceinline__ float2 cs_add(float2 a, float2 b)
{
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.y, b.x, a.x * b.y));
}

// (x, y) turned by the angle whose (cos, sin) is cs
__device__ __forceinline__ float2 rotate(float x, float y, float2 cs)
{
    return make_float2(fmaf(x, cs.x, -y * cs.y), fmaf(x, cs.y, y * cs.x));
}

// LONG: windows of many tiles.  A running fp32 sum over n tiles can lose about
// n * 2^-24 of its value (every tile's contribution is rounded into a total that
// may already hold the window's largest terms); over the ~2,050 tiles of the
// largest window that is 1e-4.  The long form therefore sums each run of kRun
// tiles separately and adds the run into a second total, which bounds the loss by
// about (kRun + n / kRun) * 2^-24.  The second set of accumulators costs registers,
// so that form runs one workgroup per CU.
constexpr int kRun = 16;
constexpr int64_t kLongWindow = 1024; // windows at least this long take the long form

template <typename T, int D, bool LONG>
__global__ __launch_bounds__(kThreads, LONG ? 1 : 2) void local_window_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                                const T *__restrict__ v,
                                                                const T *__restrict__ o_lr, T *__restrict__ out,
                                                                LocalConsts lc, int64_t N, int NB, int H,
                                                                int64_t w)
{
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int NP = D / 2; // feature pairs
    __shared__ LocalSmem<T, D> sm;
    __shared__ double s_theta[NP];
    // s_row and s_base keep pair m = 4 j + e at tab_ix(m) = e (NP / 4) + j: a lane rotates
    // the pairs 4 j .. 4 j + 3 of a 16-byte chunk, so for each e the 16 lanes of a row
    // read consecutive entries (distinct banks) instead of entries 4 apart
    __shared__ float2 s_row[32][NP];  // (cos, sin) of b theta_m, b < 32
    __shared__ float2 s_base[2][NP];  // (cos, sin) of a tile's offset times theta_m (double-buffered)
    auto tab_ix = [](int m) { return (m & 3) * (NP / 4) + (m >> 2); };
    __shared__ float2 s_step[NP];     // (cos, sin) of 32 theta_m: one tile further
    __shared__ float2 s_qbase[4][NP]; // (cos, sin) of 32 a theta_m for the block's 128 query rows

    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int beta = (int)(lb % (uint32_t)NB);
    const int64_t head = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(head % H);
    const int t = threadIdx.x;
    const int wave = t / kWave;
    const int lane = t & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t q0 = (int64_t)beta * 128;
    const int64_t qi = q0 + wave * 32 + col;
    const bool q_ok = qi < N;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D); // logits in the exp2 domain

    // the window's tiles: token starts t_lo, t_lo + 32, ... below min(N, q0 + 128)
    const int64_t lo_tok = q0 - w > 0 ? q0 - w : 0;
    const int64_t t_lo = lo_tok & ~(int64_t)31;
    const int64_t t_end = N < q0 + 128 ? N : q0 + 128;
    const int n_tiles = (int)((t_end - t_lo + 31) / 32);

    // ---- rotation tables ----
    if (t < NP)
        s_theta[t] = pow((double)lc.rope_base, -2.0 * (double)t / (double)D);
    __syncthreads();
    for (int e = t; e < 32 * NP; e += kThreads)
        s_row[e / NP][tab_ix(e % NP)] = sincos_pair((double)(e / NP) * s_theta[e % NP]);
    for (int e = t; e < 4 * NP; e += kThreads)
        s_qbase[e / NP][e % NP] = sincos_pair((double)(32 * (e / NP)) * s_theta[e % NP]);
    // tile x starts 32 x tokens after tile 0: its angles are the previous tile's turned by
    // 32 theta_m (one fp32 angle addition, about 6e-8 relative each).  A short window has
    // at most 37 tiles; the long form takes the angles afresh from fp64 every kRun tiles,
    // so the stepped angles never carry more than kRun additions however long the window.
    if (t < NP) {
        s_base[0][tab_ix(t)] = sincos_pair((double)(t_lo - q0) * s_theta[t]);
        s_step[t] = sincos_pair(32.0 * s_theta[t]);
    }
    auto tile_base = [&](int x, int buf) { // tile x, from tile x - 1 whose angles are in buf ^ 1
        if (t < NP) {
            if (LONG && x % kRun == 0)
                s_base[buf][tab_ix(t)] = sincos_pair((double)(t_lo - q0 + 32 * (int64_t)x) * s_theta[t]);
            else
                s_base[buf][tab_ix(t)] = cs_add(s_base[buf ^ 1][tab_ix(t)], s_step[t]);
        }
    };
    __syncthreads();

    // ---- rotated query fragments ----
    constexpr int KC = kBf16 ? D / 16 : D / 2;
    using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
    QFrag qf[KC], qf_lo[kBf16 ? KC : 1];
    const int rows = (int)(N - q0 < 128 ? N - q0 : 128);
    if constexpr (kBf16) {
        constexpr int CPR = D / 8;                     // 16-byte chunks per row
        constexpr int QCH = 128 * CPR / kThreads;      // chunks per thread
        u32x4 qh[QCH], ql[QCH];
        const uint16_t *qsrc = reinterpret_cast<const uint16_t *>(q) + (head * N + q0) * D;
#pragma unroll
        for (int u = 0; u < QCH; ++u) {
            const int c = t + u * kThreads, r = c / CPR, f8 = (c % CPR) * 8;
            const u32x4 x = r < rows ? *reinterpret_cast<const u32x4 *>(qsrc + (int64_t)r * D + f8) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = f8 / 2 + e;
                const float2 cs = cs_add(s_qbase[r >> 5][m], s_row[r & 31][tab_ix(m)]);
                const uint32_t xe = x[e];
                const float2 y = rotate(bf16_bits_to_f32(xe & 0xffffu), bf16_bits_to_f32(xe >> 16), cs);
                const uint32_t hp = cvt_pk_bf16(y.x, y.y);
                qh[u][e] = hp;
                ql[u][e] = cvt_pk_bf16(y.x - __uint_as_float(hp << 16), y.y - __uint_as_float(hp & 0xffff0000u));
            }
        }
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int u = 0; u < QCH; ++u) {
                const int c = t + u * kThreads;
                *reinterpret_cast<u32x4 *>(&sm.tile[c / CPR][(c % CPR) * 8]) = pass == 0 ? qh[u] : ql[u];
            }
            __syncthreads();
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 f = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.tile[wave * 32 + col][kc * 16 + half * 8]));
                if (pass == 0)
                    qf[kc] = f;
                else
                    qf_lo[kc] = f;
            }
            __syncthreads();
        }
    } else {
        const T *qrow = q + (head * N + (q_ok ? qi : 0)) * D;
        const int r = wave * 32 + col;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) { // this lane keeps element 2 kc + half of the rotated pair kc
            const float2 cs = cs_add(s_qbase[r >> 5][kc], s_row[r & 31][tab_ix(kc)]);
            const float2 y = q_ok ? rotate(qrow[2 * kc], qrow[2 * kc + 1], cs) : make_float2(0.0f, 0.0f);
            qf[kc] = half ? y.y : y.x;
        }
    }

    // ---- tile staging roles (bf16): K in 16-byte chunks, V^T by (token pair, 8-feature chunk) ----
    constexpr int CPR = D / 8;
    constexpr int KCH = (32 * CPR) / kThreads; // K chunks per thread: 1 or 2
    const int tp = t & 15;
    const int fc = t >> 4; // V roles exist for fc < CPR
    u32x4 pk[KCH > 0 ? KCH : 1], pv0, pv1;
    auto fetch = [&](int x) { // rows past N read row N - 1; their logits are masked
        const int64_t ts = t_lo + 32 * (int64_t)x;
        const T *kc_src = k + head * N * D;
        const T *vc_src = v + head * N * D;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int ch = t + u * kThreads;
            const int64_t j = ts + ch / CPR < N ? ts + ch / CPR : N - 1;
            pk[u] = *reinterpret_cast<const u32x4 *>(kc_src + j * D + (ch % CPR) * 8);
        }
        if (fc < CPR) {
            const int64_t j0 = ts + 2 * tp < N ? ts + 2 * tp : N - 1, j1 = ts + 2 * tp + 1 < N ? ts + 2 * tp + 1 : N - 1;
            pv0 = *reinterpret_cast<const u32x4 *>(vc_src + j0 * D + fc * 8);
            pv1 = *reinterpret_cast<const u32x4 *>(vc_src + j1 * D + fc * 8);
        }
    };
    if constexpr (kBf16)
        fetch(0);

    constexpr int DT = D / 32; // feature tiles of the output
    f32x16 o_acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o_acc[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f; // m_run in the exp2 domain
    f32x16 o_tot[LONG ? DT : 1];            // LONG: the completed runs of kRun tiles
    float l_tot = 0.0f;
    if constexpr (LONG) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o_tot[dt][r] = 0.0f;
    }
    const int64_t my_lo = qi - w; // the query's window is [my_lo, qi]

    for (int x = 0; x < n_tiles; ++x) {
        const int64_t ts = t_lo + 32 * (int64_t)x;
        const int buf = x & 1;
        __syncthreads();
        // ---- the tile's rotated keys and its values into LDS ----
        if constexpr (kBf16) {
#pragma unroll
            for (int u = 0; u < KCH; ++u) {
                const int ch = t + u * kThreads, row = ch / CPR, f8 = (ch % CPR) * 8;
                u32x4 kh, kl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = f8 / 2 + e;
                    const float2 cs = cs_add(s_base[buf][tab_ix(m)], s_row[row][tab_ix(m)]);
                    const uint32_t xe = pk[u][e];
                    const float2 y = rotate(bf16_bits_to_f32(xe & 0xffffu), bf16_bits_to_f32(xe >> 16), cs);
                    const uint32_t hp = cvt_pk_bf16(y.x, y.y);
                    kh[e] = hp;
                    kl[e] = cvt_pk_bf16(y.x - __uint_as_float(hp << 16), y.y - __uint_as_float(hp & 0xffff0000u));
                }
                *reinterpret_cast<u32x4 *>(&sm.k[0][row][f8]) = kh;
                *reinterpret_cast<u32x4 *>(&sm.k[1][row][f8]) = kl;
            }
            if (fc < CPR) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a0 = (pv0[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t a1 = (pv1[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t *>(&sm.vt[fc * 8 + e][vt_pos(2 * tp)]) = a0 | (a1 << 16);
                }
            }
        } else {
            const T *kc_src = k + head * N * D;
            const T *vc_src = v + head * N * D;
            for (int e = t; e < 32 * NP; e += kThreads) {
                const int row = e / NP, m = e % NP;
                const int64_t j = ts + row < N ? ts + row : N - 1;
                const float2 y = rotate(kc_src[j * D + 2 * m], kc_src[j * D + 2 * m + 1],
                                        cs_add(s_base[buf][tab_ix(m)], s_row[row][tab_ix(m)]));
                sm.k[row][2 * m] = y.x;
                sm.k[row][2 * m + 1] = y.y;
                sm.v[row][2 * m] = vc_src[j * D + 2 * m];
                sm.v[row][2 * m + 1] = vc_src[j * D + 2 * m + 1];
            }
        }
        if (x + 1 < n_tiles)
            tile_base(x + 1, buf ^ 1); // read at the next tile's staging, after the barrier below
        __syncthreads();
        if constexpr (kBf16) {
            if (x + 1 < n_tiles)
                fetch(x + 1); // overlaps the matrix work below
        }

        if constexpr (LONG) {
            if (x % kRun == 0 && x > 0) { // close the run of tiles x - kRun .. x - 1
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        o_tot[dt][r] += o_acc[dt][r];
                        o_acc[dt][r] = 0.0f;
                    }
                l_tot += l_run;
                l_run = 0.0f;
            }
        }

        // does the tile meet the query's window?
        const bool mine = q_ok && ts <= qi && ts + 31 >= my_lo;
        if (__ballot(mine) == 0ull)
            continue; // no query of this wave reads the tile

        // ---- logits S^T[32 tokens x 32 queries], tokens outside the window masked ----
        f32x16 acc;
        if constexpr (kBf16) {
            f32x16 acc_s; // the small products (lo.hi, hi.lo); acc takes hi.hi: two interleaved chains
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[r] = 0.0f;
                acc_s[r] = 0.0f;
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const bf16x8 kl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.k[1][col][kc * 16 + half * 8]));
                const bf16x8 kh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.k[0][col][kc * 16 + half * 8]));
                acc_s = mfma_bf16(kl, qf[kc], acc_s);
                acc = mfma_bf16(kh, qf[kc], acc);
                acc_s = mfma_bf16(kh, qf_lo[kc], acc_s);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] += acc_s[r];
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                acc = mfma_f32(sm.k[col][kc * 2 + half], qf[kc], acc);
        }
        // the tile's rows inside this query's window, tile-relative: lo_r <= row <= hi_r
        // (j >= qi - w, j <= qi, j < N); most tiles lie wholly inside every window
        const int64_t lo64 = my_lo - ts, hi64 = (qi < N - 1 ? qi : N - 1) - ts;
        const int lo_r = lo64 < 0 ? 0 : (lo64 > 32 ? 32 : (int)lo64);
        const int hi_r = hi64 > 31 ? 31 : (hi64 < -1 ? -1 : (int)hi64);
        if (__ballot(lo_r > 0 || hi_r < 31) != 0ull) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row(r, half);
                if (row < lo_r || row > hi_r)
                    acc[r] = -INFINITY;
            }
        }

        // ---- online softmax (exp2 domain) ----
        float p[16];
        const float alpha = softmax_cell(acc, mine, scale_log2, m_run, l_run, p);
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o_acc[dt][r] *= alpha;
            if constexpr (LONG) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        o_tot[dt][r] *= alpha;
                l_tot *= alpha;
            }
        }

        // ---- O^T[d x 32 queries] += V^T . P^T ----
        if constexpr (kBf16) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bh, bl;
                split_bf16x8(&p[8 * kk], bh, bl);
                bf16x8 av[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    av[dt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.vt[dt * 32 + col][16 * kk + 8 * half]));
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o_acc[dt] = mfma_bf16(av[dt], bl, o_acc[dt]);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o_acc[dt] = mfma_bf16(av[dt], bh, o_acc[dt]);
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o_acc[dt] = mfma_f32(sm.v[acc_row(r, half)][dt * 32 + col], p[r], o_acc[dt]);
        }
    }

    if constexpr (LONG) { // the last, partial run
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                o_acc[dt][r] += o_tot[dt][r];
        l_run += l_tot;
    }

    // ---- o_sr = O / l, plus alpha_h o_lr (Eq. 2), written out ----
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f; // every valid query holds its own token
    const float alpha_h = lc.alpha[h];
    if constexpr (kBf16) {
        uint16_t *dst = reinterpret_cast<uint16_t *>(out) + (head * N + q0) * D;
        __syncthreads(); // the last tile's LDS reads are done: the tile area takes the output
        if (o_lr) {
            tile_load_bf16<D, kThreads>(&sm.tile[0][0], sm.kStrideT,
                                        reinterpret_cast<const uint16_t *>(o_lr) + (head * N + q0) * D, rows);
            __syncthreads();
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = dt * 32 + 8 * rg + 4 * half;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = o_acc[dt][4 * rg + e] * inv_l;
                uint32_t *cell = reinterpret_cast<uint32_t *>(&sm.tile[wave * 32 + col][d0]);
                if (o_lr) {
                    const uint32_t w0 = cell[0], w1 = cell[1];
                    y[0] = fmaf(alpha_h, bf16_bits_to_f32(w0 & 0xffffu), y[0]);
                    y[1] = fmaf(alpha_h, bf16_bits_to_f32(w0 >> 16), y[1]);
                    y[2] = fmaf(alpha_h, bf16_bits_to_f32(w1 & 0xffffu), y[2]);
                    y[3] = fmaf(alpha_h, bf16_bits_to_f32(w1 >> 16), y[3]);
                }
                *reinterpret_cast<u32x2 *>(cell) = u32x2{cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3])};
            }
        __syncthreads();
        tile_store_bf16<D, kThreads>(dst, &sm.tile[0][0], sm.kStrideT, rows);
    } else if (q_ok) {
        T *dst = out + (head * N + qi) * D;
        const T *src = o_lr ? o_lr + (head * N + qi) * D : nullptr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = dt * 32 + 8 * rg + 4 * half;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = o_acc[dt][4 * rg + e] * inv_l;
                if (src) {
                    const u32x4 s4 = *reinterpret_cast<const u32x4 *>(src + d0);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = fmaf(alpha_h, __uint_as_float(s4[e]), y[e]);
                }
                *reinterpret_cast<u32x4 *>(dst + d0) =
                    u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
            }
    }
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const LocalConsts &lc, int64_t w, const void *q, const void *k, const void *v,
                    const void *o_lr, void *out, hipStream_t st)
{
    dim3 grid((unsigned)((int64_t)g.NB * g.bh)); // one linear range, renumbered per XCD in the kernel
    if (w >= kLongWindow)
        hipLaunchKernelGGL((local_window_kernel<T, D, true>), grid, dim3(kThreads), 0, st, static_cast<const T *>(q),
                           static_cast<const T *>(k), static_cast<const T *>(v), static_cast<const T *>(o_lr),
                           static_cast<T *>(out), lc, g.N, g.NB, g.H, w);
    else
        hipLaunchKernelGGL((local_window_kernel<T, D, false>), grid, dim3(kThreads), 0, st,
                           static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v),
                           static_cast<const T *>(o_lr), static_cast<T *>(out), lc, g.N, g.NB, g.H, w);
    return hipGetLastError();
}

} // namespace

hipError_t launch_local(const Geometry &g, const LocalConsts &lc, int64_t w, const void *q, const void *k,
                        const void *v, const void *o_lr, void *out, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, lc, w, q, k, v, o_lr, out, st)
                         : launch_t<uint16_t, 128>(g, lc, w, q, k, v, o_lr, out, st);
    return g.d == 64 ? launch_t<float, 64>(g, lc, w, q, k, v, o_lr, out, st)
                     : launch_t<float, 128>(g, lc, w, q, k, v, o_lr, out, st);
}

} // namespace fsl
