// Routing and readout of one 128-query block in a single launch (FreeSolo,
// Sec. 3.3 "Cell scoring" Eq. 7, "Per-query selection", "Token readout" Eq. 9,
// App. D.2 Eq. 17), for bf16 tensors.
//
// The separate scorer and readout kernels each wait on a chain of dependent
// memory round trips per block (count -> retained list -> mean keys; stored
// selections -> union -> cells) with little work in flight, and both read the
// block's queries.  Here one workgroup does both steps for its block:
//   entry     the query fragments (kept in registers for both matrix products),
//             |A_beta| and the retained list are requested together;
//   routing   the retained mean keys (bf16 hi/mid/lo parts from the summary
//             pass) are staged 32 cells at a time, the next tile in flight
//             while the matrix cores score the current one (once the first
//             tile's keys show that the tile bound will not pass over it);
//             each lane keeps its query's top-K in registers, exactly as
//             fs_score_select does;
//   union     the selections go to LDS (and, if asked, to global memory) and
//             the block's distinct selected cells are listed in id order;
//   readout   each listed cell's keys and values are gathered once into LDS
//             (both row-major; the P.V operand comes from transposing LDS
//             reads) and applied to every query of the block on the matrix
//             cores with the running softmax, exactly as fs_readout does; the
//             next cell is in flight while the current one is on the matrix
//             cores;
//   epilogue  RMSNorm, then the block's output tile goes out through LDS with
//             coalesced 16-byte stores.
// The arithmetic is the same as the two separate kernels, so the results are
// bitwise those of fs_score_select followed by fs_readout.
#include "fsl_internal.h"
#include "readout_math.h"

#include <cfloat>
#include <climits>
#include <type_traits>

namespace fsl {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;


template <int D>
struct alignas(16) FusedSmem {
    static constexpr int kStride = D + 8;   // bf16 elements per row (16-byte pad against bank conflicts)
    static constexpr int kStrideVR = D + 16; // bf16 elements per V row (transposed reads of 4 rows hit distinct banks)
    union {
        uint16_t kb[3][32][kStride]; // routing: one tile of mean-key parts
        struct {                     // readout: one cell
            uint16_t k[32][kStride];
            uint16_t v[32][kStrideVR];
        };
        uint16_t tile[128][kStride]; // epilogue: the block's output tile
    };
    float prior[32];
    float pc[32];
    int32_t id[32];
};

// Three workgroups per CU (168 VGPRs) hide more of each block's memory latency; at
// d = 128 the compiler then spills a few lane constants, and more of them for K > 4,
// where two workgroups per CU are kept.
template <int D, int KT>
constexpr int kFusedBlocksPerCU = (D <= 64 || KT <= 4) ? 3 : 2;

template <int D, int KT>
__global__ __launch_bounds__(kThreads, (kFusedBlocksPerCU<D, KT>)) void route_readout_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ kbar_split, const float *__restrict__ kbar_norm, const float *__restrict__ a,
    const int32_t *__restrict__ retained,
    const int32_t *__restrict__ n_ret, const float *__restrict__ gain, uint16_t *__restrict__ out,
    int32_t *__restrict__ sel, int64_t N, int64_t M, int NB, int cap, int prune, int H, int s,
    int cells_per_block, float eps, HeadConsts hc)
{
    __shared__ FusedSmem<D> sm;
    __shared__ int32_t s_A[kFusedMaxCap];
    __shared__ int32_t sel_s[128][KT];
    __shared__ int32_t ulist[128 * KT];
    __shared__ int32_t n_u;
    extern __shared__ uint32_t bitmap[]; // ceil(M / 32) words

    constexpr int PER = D / 8;  // mean-key elements staged per thread and tile
    constexpr int SCH = PER / 8; // 16-byte chunks per part and thread
    constexpr int KC = D / 16;  // k-steps of the bf16 matrix products
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    // a head's blocks from the last: without pruning (FS) a later block scores more cells,
    // so the longest start first and the kernel ends on short ones
    const int beta = NB - 1 - (int)(lb % (uint32_t)NB);
    const int64_t head = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(head % H);
    const int t = threadIdx.x;
    const int wave = t / kWave;
    const int lane = t & (kWave - 1);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int64_t q0 = (int64_t)beta * 128;
    const int64_t qi = q0 + wave * 32 + col; // this lane's query position
    const bool q_ok = qi < N;
    const float qpos = (float)qi; // exact: N <= 2^22
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D); // readout logits in the exp2 domain
    const float inv2s = hc.inv_two_sigma[h];
    const float lam = hc.lambda[h];

    int64_t n_avail = (int64_t)beta * cells_per_block;
    if (n_avail > M)
        n_avail = M;

    // ---- entry: |A|, the retained list and the query fragments, all at once ----
    const int nA = prune ? n_ret[head * NB + beta] : (int)n_avail;
    const int32_t my_ret = prune && t < cap ? retained[(head * NB + beta) * (int64_t)cap + t] : 0;
    bf16x8 qf[KC];
    {
        // lanes past N load row N-1 and are masked where their results would count
        // (routing keys, the tile bound, selections); nothing here waits for the
        // loads, so the retained list and first mean-key tile are requested with them
        const uint16_t *qrow = q + (head * N + (q_ok ? qi : N - 1)) * D;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            qf[kc] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qrow + kc * 16 + half * 8));
    }
    if (prune && t < cap)
        s_A[t] = my_ret;
    __syncthreads();

    // ---- routing (Eq. 7) with the running top-K of this lane's query ----
    const int srow = t >> 3, spart = t & 7; // staging role: row of the tile, feature part
    u32x4 pre3[3 * SCH];
    int pre_id;
    float pre_a;
    // the tile bound needs every retained cell's prior and mean-key norm: one
    // load each per block, kept in registers until the first tile is scored
    constexpr int kBoundTiles = 256; // the tile bound covers retained lists of up to 8192 cells
    const bool bound = kbar_norm != nullptr && nA > 32 && nA <= kBoundTiles * 32;
    __shared__ float s_tpr[kBoundTiles], s_tkn[kBoundTiles], s_qn[kThreads / kWave];
    __shared__ uint32_t s_tau[2][kThreads / kWave];
    if (bound) { // the largest |q_i| of this wave, for the tile bound (read after a later barrier);
        // computed before any later load is issued, so it waits for the query fragments only
        float ss = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4 w = __builtin_bit_cast(u32x4, qf[kc]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // the element goes through a named copy: hipcc miscompiles a bit cast
                // of a vector element taken in place (it reads element 0)
                const uint32_t we = w[e];
                const bf16x2 x = __builtin_bit_cast(bf16x2, we);
                ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
            }
        }
        ss += shfl_xor_f(ss, 32); // the partner lane holds the other half of the features
        // + 2^-100: covers subnormal elements, should the dot product flush them
        const float qn = q_ok ? sqrtf(ss) * (1.0f + 0x1p-10f) + 0x1p-100f : 0.0f;
        const bool badq = __ballot(!(qn <= FLT_MAX)) != 0ull;
        const float qm = wave_max_f(qn);
        if (lane == 0)
            s_qn[wave] = badq ? INFINITY : qm;
    }
    float b_pr = 0.0f, b_kn = 0.0f;
    if (bound && t < nA) { // lambda is applied where the values are first used, so nothing waits here
        const int64_t id = head * M + (prune ? s_A[t] : t);
        b_pr = a[id];
        b_kn = kbar_norm[id];
    }
    const uint16_t *kbs_h = kbar_split + head * M * 3 * D; // this head's mean-key parts
    int pre_t0 = -1;                                       // the tile whose parts pre3 holds
    auto prefetch = [&](int t0) {
        pre_t0 = t0;
        const int x = t0 + srow;
        pre_id = x < nA ? (prune ? s_A[x] : x) : -1;
        // no branch around the loads: a value merged from two paths would make the wave
        // wait for the loads right here.  Padding rows read cell 0, and their scores never
        // count (their id stays -1).
        const int cid = pre_id >= 0 ? pre_id : 0;
        // < 3 d M elements: the offset fits 32 bits
        const uint16_t *src = kbs_h + (uint32_t)(cid * 3 * D + spart * PER);
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
            for (int u = 0; u < SCH; ++u)
                pre3[part * SCH + u] = *reinterpret_cast<const u32x4 *>(src + part * D + u * 8);
        pre_a = a[head * M + cid];
    };
    if (nA > 0)
        prefetch(0);

    uint64_t kl[KT]; // this lane's best keys so far
#pragma unroll
    for (int j = 0; j < KT; ++j)
        kl[j] = 0;
    // Tile bound (with kbar_norm): every score in a tile is at most
    //   max_c (lambda a_c) + max_i |q_i| max_c |kbar_c| / sqrt(d)
    // (Cauchy-Schwarz on the content term; 0 < g <= 1 for every available cell,
    // whose centre lies at least s/2 before the block), widened for rounding.
    // When it falls below every query's K-th best key so far, no cell of the
    // tile can enter any top-K, and the tile is passed over: the selections are
    // those of scoring every cell.  The first tile is always scored.
    // per 32-cell tile of the retained list: the largest lambda a_c and the largest |kbar_c|
    // (NaN or infinite values make the tile's maximum infinite, so it is never passed over)
    auto tile_max = [&](int x, float pr, float kn) { // thread's cell x of the list; all threads call it
        pr = pr <= FLT_MAX ? pr : INFINITY;
        kn = kn <= FLT_MAX ? kn : INFINITY;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            pr = fmaxf(pr, shfl_xor_f(pr, o));
            kn = fmaxf(kn, shfl_xor_f(kn, o));
        }
        if ((lane & 31) == 0) {
            s_tpr[x >> 5] = pr;
            s_tkn[x >> 5] = kn;
        }
    };
    int iter = 0;
    for (int t0 = 0; t0 < nA; t0 += 32, ++iter) {
        const int par = iter & 1; // tau slots alternate, so no wave overwrites one still being read
        if (bound && t0 > 0) {
            const uint32_t tau = wave_min_u32(q_ok ? (uint32_t)(kl[KT - 1] >> 32) : 0xffffffffu);
            if (lane == 0)
                s_tau[par][wave] = tau;
        }
        __syncthreads();
        // bound of a tile against the block's smallest K-th best key (tau);
        // tau only grows, so a tile found below it now stays below it later
        uint32_t tau = 0;
        float qn = 0.0f;
        auto tile_below = [&](int tb) {
            const float pm = s_tpr[tb >> 5], km = s_tkn[tb >> 5];
            const float ub = (pm + qn * km * inv_sqrt_d * (1.0f + 0x1p-10f)) * (1.0f + 0x1p-10f);
            // ub >= 0: its ranking key's high word is its bits with the sign bit set
            return ub <= FLT_MAX && (__float_as_uint(ub) | 0x80000000u) < tau;
        };
        if (bound && t0 > 0) {
            qn = s_qn[0];
            tau = s_tau[par][0];
#pragma unroll
            for (int w = 1; w < kThreads / kWave; ++w) {
                qn = fmaxf(qn, s_qn[w]);
                tau = min(tau, s_tau[par][w]);
            }
            // tau stays fixed until a tile is scored: pass over every tile below it at once
            // (the test is uniform over the block, so every wave leaves or stays together)
            while (t0 < nA && tile_below(t0))
                t0 += 32;
            if (t0 >= nA)
                break;
            if (pre_t0 != t0)
                prefetch(t0); // the tile held in registers was passed over
        }
        if (spart == 0) {
            sm.id[srow] = pre_id >= 0 ? 0x7fffffff - pre_id : -1;   // low half of the ranking key
            sm.prior[srow] = pre_id >= 0 ? lam * pre_a : 0.0f;
            sm.pc[srow] = pre_id >= 0 ? (float)pre_id * s + 0.5f * s : 0.0f;
        }
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
            for (int u = 0; u < SCH; ++u)
                *reinterpret_cast<u32x4 *>(&sm.kb[part][srow][spart * PER + u * 8]) = pre3[part * SCH + u];
        if (bound && t0 == 0) { // loaded before the tile, so here already; read after a later barrier
            tile_max(t, t < nA ? lam * b_pr : 0.0f, t < nA ? b_kn : 0.0f);
            for (int x0 = kThreads; x0 < nA; x0 += kThreads) { // lists past 256 cells (FS)
                const int x = x0 + t;
                float pr = 0.0f, kn = 0.0f;
                if (x < nA) {
                    const int64_t id = head * M + (prune ? s_A[x] : x);
                    pr = lam * a[id];
                    kn = kbar_norm[id];
                }
                tile_max(x, pr, kn);
            }
        }
        __syncthreads();
        // the next tile, in flight under the matrix work below, unless the bound passes over
        // it; with the bound on, the first tile's keys decide (without them it seldom fails)
        if (t0 + 32 < nA && !(bound && (t0 == 0 || tile_below(t0 + 32))))
            prefetch(t0 + 32);

        f32x16 acc;
        // three independent accumulators (lo, mid, hi parts) keep the matrix cores busy;
        // the parts are added smallest first
        f32x16 acc3[3];
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc3[sp][r] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
            for (int sp = 2; sp >= 0; --sp) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.kb[sp][col][kc * 16 + half * 8]);
                acc3[sp] = mfma_bf16(as_bf16x8(w), qf[kc], acc3[sp]);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = (acc3[2][r] + acc3[1][r]) + acc3[0][r];
        // this lane's 16 rows come in 4 runs of 4 consecutive rows; their keys are made and
        // taken in two halves of 8 rows (fewer registers live at once; the top-K does not
        // depend on the order in which distinct keys enter it)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float prv[8], pcv[8];
            int idv[8]; // low key halves; -1 on padding rows
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2) {
                const int r0 = 8 * (2 * hh + g2) + 4 * half;
                const u32x4 vp = *reinterpret_cast<const u32x4 *>(&sm.prior[r0]);
                const u32x4 vc = *reinterpret_cast<const u32x4 *>(&sm.pc[r0]);
                const u32x4 vi = *reinterpret_cast<const u32x4 *>(&sm.id[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    prv[4 * g2 + e] = __uint_as_float(vp[e]);
                    pcv[4 * g2 + e] = __uint_as_float(vc[e]);
                    idv[4 * g2 + e] = (int)vi[e];
                }
            }
            // erf only below 4 (from there on it rounds to 1 in fp32, and fmaf(prior,
            // 1, content) == prior + content); a wave takes the long path only if
            // one of its queries is that close to one of these cells
            float pcmax = pcv[0];
#pragma unroll
            for (int r = 1; r < 8; ++r)
                pcmax = fmaxf(pcmax, pcv[r]);
            const bool need_erf = __ballot(q_ok && (qpos - pcmax) * inv2s < 4.0f) != 0ull;
            uint64_t key[8];
            if (need_erf) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    float g = 1.0f;
                    const float x = (qpos - pcv[r]) * inv2s; // (i - p_c) / (2 sigma_h), i - p_c exact
                    if (x < 4.0f)
                        g = erff(x);
                    const float score = fmaf(prv[r], g, acc[8 * hh + r] * inv_sqrt_d);
                    key[r] = (q_ok && idv[r] >= 0) ? rank_key(score, (uint32_t)idv[r]) : 0;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float score = fmaf(prv[r], 1.0f, acc[8 * hh + r] * inv_sqrt_d);
                    key[r] = (q_ok && idv[r] >= 0) ? rank_key(score, (uint32_t)idv[r]) : 0;
                }
            }
            take_tile_keys<KT, 8>(kl, key, t0 == 0 && hh == 0);
        }
    }
    // merge with the partner lane (same query, other 16 rows of every tile)
    {
        uint64_t pk[KT]; // the partner's list as it was, before either lane inserts
#pragma unroll
        for (int j = 0; j < KT; ++j)
            pk[j] = ((uint64_t)(uint32_t)shfl_xor_i((int)(kl[j] >> 32), 32) << 32) |
                    (uint32_t)shfl_xor_i((int)(uint32_t)kl[j], 32);
#pragma unroll
        for (int j = 0; j < KT; ++j)
            insert_key<KT>(kl, pk[j]);
    }

    // ---- selections to LDS (and global), then their union in id order ----
    const int n_words = (int)((n_avail + 31) / 32);
    for (int w = t; w < n_words; w += kThreads)
        bitmap[w] = 0u;
    int my_sel[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j)
        my_sel[j] = (q_ok && kl[j]) ? 0x7fffffff - (int32_t)(uint32_t)kl[j] : -1;
    if (half == 0) {
#pragma unroll
        for (int j = 0; j < KT; ++j)
            sel_s[wave * 32 + col][j] = my_sel[j];
        if (sel && q_ok) {
            int32_t *dst = sel + (head * N + qi) * KT;
#pragma unroll
            for (int j = 0; j < KT; ++j)
                dst[j] = my_sel[j];
        }
    }
    __syncthreads();
    for (int x = t; x < 128 * KT; x += kThreads) {
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

    // ---- readout (Eq. 9): one gathered cell at a time, next one in flight ----
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int KCH = (32 * CPR) / kThreads; // K chunks per thread: 1 or 2
    u32x4 pk[KCH], pv[KCH];
    const uint16_t *k_h = k + head * N * D, *v_h = v + head * N * D; // this head's keys and values
    auto fetch = [&](int cell) {
        // element offsets within the head: N d <= 2^29, so 32 bits hold them
        const uint32_t base = (uint32_t)cell * (uint32_t)(s * D);
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int ch = t + u * kThreads;
            const uint32_t off = base + (uint32_t)((ch / CPR) * D + (ch % CPR) * 8);
            pk[u] = *reinterpret_cast<const u32x4 *>(k_h + off);
            pv[u] = *reinterpret_cast<const u32x4 *>(v_h + off);
        }
    };
    if (nU > 0)
        fetch(ulist[0]);

    constexpr int DT = D / 32; // feature tiles of the output
    f32x16 o_acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            o_acc[dt][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f; // m_run in the exp2 domain

    for (int x = 0; x < nU; ++x) {
        const int cell = ulist[x];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int ch = t + u * kThreads;
            *reinterpret_cast<u32x4 *>(&sm.k[ch / CPR][(ch % CPR) * 8]) = pk[u];
            *reinterpret_cast<u32x4 *>(&sm.v[ch / CPR][(ch % CPR) * 8]) = pv[u];
        }
        __syncthreads();
        if (x + 1 < nU)
            fetch(ulist[x + 1]);

        bool mine = false;
#pragma unroll
        for (int j = 0; j < KT; ++j)
            mine |= my_sel[j] == cell;
        if (__ballot(mine) == 0ull)
            continue; // no query of this wave reads the cell

        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[r] = 0.0f;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(&sm.k[col][kc * 16 + half * 8]);
            acc = mfma_bf16(as_bf16x8(w), qf[kc], acc);
        }
        float p[16];
        const float alpha = softmax_cell(acc, mine, scale_log2, m_run, l_run, p);
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o_acc[dt][r] *= alpha;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 bh, bl;
            split_bf16x8(&p[8 * kk], bh, bl);
            // A = V^T rows: lane (col, half) needs V[t][dt * 32 + col] for the tokens t of its
            // probabilities (16 kk + 4 half + 0..3, then + 8); two transposed 4-row reads
            // from row-major V give them (lane j of a 16-lane group names row j / 4, and
            // features 4 (j % 4) .. +3 of the group's 16)
            const int r0 = 16 * kk + 4 * half + ((lane & 15) >> 2);
            const int c0 = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            // two feature tiles at a time (fewer registers live): lo parts of both, then hi
            // parts, so no product waits on the one just before it
            constexpr int DP = DT < 2 ? DT : 2;
#pragma unroll
            for (int d0 = 0; d0 < DT; d0 += DP) {
                bf16x8 av[DP];
#pragma unroll
                for (int j = 0; j < DP; ++j) {
                    const int dt = d0 + j;
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)&sm.v[r0][dt * 32 + c0]);
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)&sm.v[r0 + 8][dt * 32 + c0]);
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    av[j] = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
                }
#pragma unroll
                for (int j = 0; j < DP; ++j)
                    o_acc[d0 + j] = mfma_bf16(av[j], bl, o_acc[d0 + j]);
#pragma unroll
                for (int j = 0; j < DP; ++j)
                    o_acc[d0 + j] = mfma_bf16(av[j], bh, o_acc[d0 + j]);
            }
        }
    }

    // ---- normalise, RMSNorm over d (Eq. 17), write through LDS ----
    const float c = rms_factor<DT>(o_acc, l_run, eps); // y = c * o, times the gain
    __syncthreads(); // the last cell's LDS reads are done: the tile area takes the output
    // one straight-line copy with the gain vector and one without (the test is uniform)
    auto emit = [&](auto with_gain) {
        const float *gh = gain + (int64_t)h * D;
        u32x4 gv[DT][4]; // this lane's 4-feature runs of the gain vector, loaded together
        if constexpr (decltype(with_gain)::value) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    gv[dt][rg] = *reinterpret_cast<const u32x4 *>(gh + dt * 32 + 8 * rg + 4 * half);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int d0 = dt * 32 + 8 * rg + 4 * half;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[e] = o_acc[dt][4 * rg + e] * c;
                    if constexpr (decltype(with_gain)::value)
                        y[e] = l_run > 0.0f ? y[e] * __uint_as_float(gv[dt][rg][e]) : 0.0f;
                }
                *reinterpret_cast<u32x2 *>(&sm.tile[wave * 32 + col][d0]) =
                    u32x2{cvt_pk_bf16(y[0], y[1]), cvt_pk_bf16(y[2], y[3])};
            }
    };
    if (gain)
        emit(std::true_type{});
    else
        emit(std::false_type{});
    __syncthreads();
    tile_store_bf16<D, kThreads>(out + (head * N + q0) * D, &sm.tile[0][0], sm.kStride,
                                 (int)(N - q0 < 128 ? N - q0 : 128));
}

template <int D, int KT>
hipError_t launch_k(const Geometry &g, const HeadConsts &hc, const void *q, const void *k, const void *v,
                    const uint16_t *kbar_split, const float *kbar_norm, const float *a, const int32_t *retained,
                    const int32_t *n_ret, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    dim3 grid((unsigned)((int64_t)g.NB * g.bh)); // one linear range, renumbered per XCD in the kernel
    const size_t words = (size_t)((g.M + 31) / 32);
    const size_t dyn = (words > 0 ? words : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((route_readout_kernel<D, KT>), grid, dim3(kThreads), dyn, st,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), kbar_split, kbar_norm, a, retained, n_ret, gain,
                       static_cast<uint16_t *>(out), sel, g.N, g.M, g.NB, g.cap, g.prune, g.H, g.s, g.B / g.s, g.eps,
                       hc);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Geometry &g, const HeadConsts &hc, const void *q, const void *k, const void *v,
                    const uint16_t *ks, const float *kn, const float *a, const int32_t *retained,
                    const int32_t *n_ret, const float *gain, void *out, int32_t *sel, hipStream_t st)
{
    switch (g.K) {
    case 1: return launch_k<D, 1>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 2: return launch_k<D, 2>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 3: return launch_k<D, 3>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 4: return launch_k<D, 4>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 5: return launch_k<D, 5>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 6: return launch_k<D, 6>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    case 7: return launch_k<D, 7>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    default: return launch_k<D, 8>(g, hc, q, k, v, ks, kn, a, retained, n_ret, gain, out, sel, st);
    }
}

} // namespace

hipError_t launch_route_readout(const Geometry &g, const HeadConsts &hc, const void *q, const void *k,
                                const void *v, const uint16_t *kbar_split, const float *kbar_norm, const float *a,
                                const int32_t *retained, const int32_t *n_ret, const float *gain, void *out,
                                int32_t *sel, hipStream_t st)
{
    return g.d == 64 ? launch_d<64>(g, hc, q, k, v, kbar_split, kbar_norm, a, retained, n_ret, gain, out, sel, st)
                     : launch_d<128>(g, hc, q, k, v, kbar_split, kbar_norm, a, retained, n_ret, gain, out, sel, st);
}

} // namespace fsl
