// FS-B, FreeSolo's balanced tree search (Sec. 3.4 "Balanced tree search
// (FS-B)"; App. E.1 "Streaming forests"): for every query block, two causal
// forests over the available cells (all of them, Eq. 10's A^0, and those with
// a_c >= tau_h, A^tau), a beam of W^b nodes per forest ranked by Eq. 11 down to
// the leaves, and the union of the leaves reranked with the token keys (Eq. 12);
// the K best cells are the selection, read out by the readout kernel.
//
// Three kernels:
//   * fsb_admit_kernel: per head, the second forest's admitted cells in arrival
//     order and their running count (a_c in fp64, so the admission equals an
//     fp64 evaluation exactly).
//   * fsb_build_kernel: the aligned chunks of 2^k admitted cells that start at
//     an even multiple of 2^k (the only chunks a binary decomposition of the
//     admitted count uses, App. E.1 "Chunks"), for both forests of every head:
//     a workgroup per chunk of more than sixteen cells, a wave per smaller one.
//     A chunk never changes once complete, so its tree is built once and
//     serves every block whose forest holds it.  Per node: fp64 mean, farthest
//     cell, two power iterations (Eq. 19), then the node's cells are sorted by
//     their projection in LDS (bitonic) and halved; node summaries (Eq. 20) are
//     written heap-ordered, mean keys as fp32.  A wave takes a node where a
//     level has at least as many nodes as waves; above that every wave takes a
//     slice of a node.  The chunks are taken largest first (the longest chains
//     start at once).
//   * fsb_search_kernel: one workgroup per (sequence, head, 128-query block).
//     It forms the block's join nodes (Eq. 21) from its chunks' roots and runs
//     the 128 beams level-synchronously: each level every query's internal
//     beam nodes are marked in an LDS bitmap over the block's forest nodes and
//     their children collected into one list, scored for all 128 queries
//     32 nodes at a time on the matrix cores (the q . mu term of Eq. 11: bf16
//     queries against each fp32 mean's bf16 hi + mid + lo parts, fp32 queries
//     on the fp32 products), and each query keeps its leaves plus its best
//     W^b - #leaves children (a bitonic sort and merge over the query's lane
//     pair); a level where every query keeps all its children skips the
//     priorities.  The level's node list is dynamic LDS sized by the forest, so
//     a bf16 search fits two workgroups on a CU at moderate lengths.
//     The union of the leaves reached is then reranked cell by cell: a cell's
//     32 token keys are staged once and the logits of all 128 queries come
//     from the matrix cores; each query that has the cell as a candidate takes
//     the log-sum-exp (Eq. 12) and keeps its top K.
//
// Ties follow the oracle's readings: the smaller cell id (nodes: the smaller
// smallest cell id below, which names one node among disjoint subtrees).
#include "fsl_internal.h"

#include <type_traits>

#include <climits>

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ double wave_sum_d(double x)
{
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
        x += shfl_xor_d(x, m); // x + y == y + x: every lane ends with the same sum
    return x;
}

// ---------------------------------------------------------------- admission

__global__ __launch_bounds__(kThreads) void fsb_admit_kernel(const double *__restrict__ a64, int32_t *__restrict__ adm,
                                                          int32_t *__restrict__ cnt, int64_t M, int H, FsbConsts fc)
{
    const int64_t bh = blockIdx.x;
    const double tau = fc.tau[bh % H];
    const double *ah = a64 + bh * M;
    int32_t *admh = adm + bh * M;
    int32_t *cnth = cnt + bh * (M + 1);
    __shared__ int32_t s_wave[kWaves];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    if (threadIdx.x == 0)
        cnth[0] = 0;
    int32_t base = 0;
    for (int64_t c0 = 0; c0 < M; c0 += kThreads) {
        const int64_t c = c0 + threadIdx.x;
        const bool in = c < M && ah[c] >= tau; // Eq. 10: a_c >= tau_h, in fp64
        const uint64_t bal = __ballot(in);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0)
            s_wave[wave] = __popcll(bal);
        __syncthreads();
        int32_t off = base, tot = 0;
        for (int w = 0; w < kWaves; ++w) {
            off += w < wave ? s_wave[w] : 0;
            tot += s_wave[w];
        }
        if (in)
            admh[off + before] = (int32_t)c;
        if (c < M)
            cnth[c + 1] = off + before + (in ? 1 : 0);
        base += tot;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- construction

constexpr int kBuildThreads = 512;
constexpr int kBuildWaves = kBuildThreads / kWave;
constexpr int kWaveChunkK = 4; // chunks of at most 2^4 cells: one wave each, kBuildWaves to a workgroup

// workgroups for the chunks of 2^k cells (ck per forest, over `groups` forests)
__host__ __device__ inline int64_t build_span(int64_t ck, int64_t groups, int k)
{
    return k > kWaveChunkK ? ck * groups : (ck * groups + kBuildWaves - 1) / kBuildWaves;
}

template <int D>
__global__ __launch_bounds__(kBuildThreads, 6) void fsb_build_kernel(const double *__restrict__ kbar64,
                                                               const float *__restrict__ a,
                                                               const int32_t *__restrict__ adm,
                                                               const int32_t *__restrict__ cnt,
                                                               float *__restrict__ node_mu,
                                                               FsbNodeMeta *__restrict__ node_meta, int64_t M,
                                                               FsbLayout L, int64_t groups)
{
    constexpr int FPL = D / kWave; // features per lane
    constexpr int NW = kBuildWaves;
    __shared__ int32_t perm[kFsbMaxCells];
    __shared__ double key[kFsbMaxCells];

    // the largest chunks first: a chunk's build is a chain that grows with its size (the
    // 2^k-cell root alone takes 2^k cells through every pass), so the longest chains start
    // at once and the many small chunks fill the CUs around them.  A chunk of at most
    // 2^kWaveChunkK cells is built by one wave alone (its team), kBuildWaves of them to a
    // workgroup; a larger one by the whole workgroup.  `groups`: (sequence, head, forest)
    // triples.
    int64_t w = blockIdx.x;
    int k = L.levels - 1;
    int64_t ck = L.chunk_base[k + 1] - L.chunk_base[k]; // chunks of 2^k cells per forest
    while (k > 0 && w >= build_span(ck, groups, k)) {
        w -= build_span(ck, groups, k);
        --k;
        ck = L.chunk_base[k + 1] - L.chunk_base[k];
    }
    const bool wm = k <= kWaveChunkK; // one wave per chunk
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave); // uniform: node and slice values stay scalar
    const int64_t cw = wm ? w * NW + wave : w; // the chunk among the ck * groups of this size
    if (cw >= ck * groups)
        return; // a spare wave of the last workgroup of small chunks
    const int64_t grp = cw / ck, jj = cw - grp * ck;
    const int64_t bh = grp / 2;
    const int f = (int)(grp - bh * 2);
    const int64_t n = (int64_t)1 << k, start = 2 * jj * n;
    const int64_t Mf = f == 0 ? L.Mu : cnt[bh * (M + 1) + L.Mu];
    if (start + n > Mf)
        return; // not a complete chunk of this forest: never read
    const int team_waves = wm ? 1 : NW, team_wave = wm ? 0 : wave;
    int32_t *const perm_t = wm ? perm + wave * (1 << kWaveChunkK) : perm; // the team's cells
    double *const key_t = wm ? key + wave * (1 << kWaveChunkK) : key;
    auto team_sync = [&]() {
        if (wm)
            wave_lds_sync();
        else
            __syncthreads();
    };
    for (int64_t p = wm ? lane : t; p < n; p += wm ? kWave : kBuildThreads)
        perm_t[p] = f == 0 ? (int32_t)(start + p) : adm[bh * M + start + p];
    team_sync();
    const int64_t out0 = (bh * 2 + f) * L.nodes + L.node_base[k] + jj * (2 * n - 1);
    const double *kb = kbar64 + bh * M * D;
    const float *ah = a + bh * M;

    // Levels with fewer nodes than waves (and at least kCoopCells cells a node) take
    // every wave: wpn waves share a node, each walking a contiguous slice of its cells;
    // their sums meet in LDS (added in slice order) and the node's sort steps on
    // workgroup barriers.  Other levels take one wave per node.
    constexpr int kCoopCells = 16;
    constexpr int kBatch = 4; // cells per memory round trip in the node passes
    __shared__ double s_best[NW];
    __shared__ int32_t s_bestc[NW], s_mn[NW];
    __shared__ float s_A[NW];
    // the slices' partial sums (one D-vector per wave) use the first NW * D entries of
    // key: the level's projections are written only after the last partial is read
    static_assert(NW * D <= kFsbMaxCells, "the partial sums fit in the key area");
    double(*const s_part)[D] = reinterpret_cast<double(*)[D]>(key);

    for (int l = 0; l <= k; ++l) {
        const int64_t nv = n >> l, nodes = (int64_t)1 << l;
        // waves per node; coop only when the team is the whole workgroup
        const int wpn = (nodes < team_waves && nv >= kCoopCells) ? team_waves / (int)nodes : 1;
        const bool coop = wpn > 1; // then nodes * wpn == NW: every wave takes one node, once
        auto node_sync = [&]() {
            if (coop)
                __syncthreads();
            else
                wave_lds_sync();
        };
        for (int64_t s = team_wave / wpn; s < nodes; s += team_waves / wpn) {
            const int sp = team_wave % wpn;                     // this wave's slice of the node
            const int64_t xb = sp * (nv / wpn), xe = xb + nv / wpn; // its cells (all of them if wpn = 1)
            int32_t *cells = perm_t + s * nv;
            double *keys = key_t + s * nv;
            const int64_t node = out0 + nodes + s - 1; // heap index nodes + s
            float *mu_out = node_mu + node * D;
            if (nv == 1) { // a leaf: the cell itself
                const int32_t c = cells[0];
#pragma unroll
                for (int e = 0; e < FPL; ++e)
                    mu_out[lane + kWave * e] = (float)kb[(int64_t)c * D + lane + kWave * e];
                if (lane == 0)
                    node_meta[node] = FsbNodeMeta{0.0f, ah[c], c, c};
                continue;
            }
            // the node's passes, with its slice resident in registers or streamed in batches
            auto node_passes = [&](auto mode) {
                // Every pass below walks the wave's cells in order, kBatch at a time: the
                // batch's ids, then all of its rows (and norms) requested together, then the
                // arithmetic in cell order (each sum keeps its order of additions), so a pass
                // waits for memory once per batch instead of once per cell.  A slice of at
                // most kBatch cells (every node of the two lowest levels, small chunks) is
                // fetched once and every pass runs on the registers.  Slices are powers of two.
                const int64_t nb_full = xb + (xe - xb) / kBatch * kBatch;
                constexpr bool resident = decltype(mode)::value;
                double rows[kBatch][FPL];
                int32_t ids[kBatch];
                float an[kBatch];
                auto fetch = [&](int64_t x0, int cnt) {
#pragma unroll
                    for (int j = 0; j < kBatch; ++j)
                        ids[j] = j < cnt ? cells[x0 + j] : cells[x0];
#pragma unroll
                    for (int j = 0; j < kBatch; ++j) {
#pragma unroll
                        for (int e = 0; e < FPL; ++e)
                            rows[j][e] = kb[(int64_t)ids[j] * D + lane + kWave * e];
                        an[j] = ah[ids[j]];
                    }
                };
                if constexpr (resident)
                    fetch(xb, (int)(xe - xb));
                // apply body(x, j) to cells x = xb .. xe - 1 in order, the rows in rows[j]
                auto walk = [&](auto &&body) {
                    if constexpr (resident) {
#pragma unroll
                        for (int j = 0; j < kBatch; ++j)
                            if (j < xe - xb)
                                body(xb + j, j);
                        return;
                    }
                    for (int64_t x0 = xb; x0 < nb_full; x0 += kBatch) {
                        fetch(x0, kBatch);
#pragma unroll
                        for (int j = 0; j < kBatch; ++j)
                            body(x0 + j, j);
                    }
                    for (int64_t x0 = nb_full; x0 < xe; x0 += kBatch) {
                        const int cnt = (int)(xe - x0 < kBatch ? xe - x0 : kBatch);
                        fetch(x0, cnt);
#pragma unroll
                        for (int j = 0; j < kBatch; ++j)
                            if (j < cnt)
                                body(x0 + j, j);
                    }
                };
                // a D-vector summed over the node's slices, in slice order (every wave of the
                // node gets the same sum); then the barrier that frees s_part
                auto slices_sum = [&](double (&v)[FPL]) {
                    if (!coop)
                        return;
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        s_part[wave][lane + kWave * e] = v[e];
                    __syncthreads();
#pragma unroll
                    for (int e = 0; e < FPL; ++e) {
                        double sum = 0.0;
                        for (int j = 0; j < wpn; ++j)
                            sum += s_part[s * wpn + j][lane + kWave * e];
                        v[e] = sum;
                    }
                    __syncthreads();
                };

                // mean of the cells' mean keys, summed in the node's cell order (one wave) or
                // in slice order of the slices' sums (several)
                double mu[FPL];
#pragma unroll
                for (int e = 0; e < FPL; ++e)
                    mu[e] = 0.0;
                walk([&](int64_t, int j) {
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        mu[e] += rows[j][e];
                });
                slices_sum(mu);
#pragma unroll
                for (int e = 0; e < FPL; ++e)
                    mu[e] = mu[e] / (double)nv;
                // distances from the mean: the farthest cell (smaller id on ties) starts the
                // power iteration and gives the radius; the largest norm and the earliest cell
                double best = -1.0;
                int32_t bestc = INT_MAX, mn = INT_MAX;
                float A = -INFINITY;
                walk([&](int64_t, int j) {
                    const int32_t c = ids[j];
                    double sq = 0.0;
#pragma unroll
                    for (int e = 0; e < FPL; ++e) {
                        const double xv = rows[j][e] - mu[e];
                        sq += xv * xv;
                    }
                    const double nrm = sqrt(wave_sum_d(sq));
                    if (nrm > best || (nrm == best && c < bestc)) {
                        best = nrm;
                        bestc = c;
                    }
                    mn = min(mn, c);
                    A = fmaxf(A, an[j]);
                });
                if (coop) { // the slices' results, combined by the same rules (order-free)
                    if (lane == 0) {
                        s_best[wave] = best;
                        s_bestc[wave] = bestc;
                        s_A[wave] = A;
                        s_mn[wave] = mn;
                    }
                    __syncthreads();
                    best = -1.0;
                    bestc = INT_MAX;
                    mn = INT_MAX;
                    A = -INFINITY;
                    for (int j = 0; j < wpn; ++j) {
                        const int w2 = (int)s * wpn + j;
                        const double nb = s_best[w2];
                        const int32_t cb = s_bestc[w2];
                        if (nb > best || (nb == best && cb < bestc)) {
                            best = nb;
                            bestc = cb;
                        }
                        A = fmaxf(A, s_A[w2]);
                        mn = min(mn, s_mn[w2]);
                    }
                }
                double u[FPL];
                auto normalise = [&]() {
                    double sq = 0.0;
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        sq += u[e] * u[e];
                    sq = wave_sum_d(sq);
                    if (sq > 0.0) {
                        const double inv = 1.0 / sqrt(sq);
#pragma unroll
                        for (int e = 0; e < FPL; ++e)
                            u[e] *= inv;
                    }
                };
                if (resident && !coop) { // the farthest cell's row is one of the registers
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        u[e] = 0.0;
#pragma unroll
                    for (int j = 0; j < kBatch; ++j)
                        if (j < xe - xb && ids[j] == bestc)
#pragma unroll
                            for (int e = 0; e < FPL; ++e)
                                u[e] = rows[j][e] - mu[e];
                } else {
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        u[e] = kb[(int64_t)bestc * D + lane + kWave * e] - mu[e];
                }
                normalise();
                for (int it = 0; it < 2; ++it) { // u <- sum_c (x_c . u) x_c, normalised (Eq. 19)
                    double wv[FPL];
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        wv[e] = 0.0;
                    walk([&](int64_t, int j) {
                        double xv[FPL], p = 0.0;
#pragma unroll
                        for (int e = 0; e < FPL; ++e) {
                            xv[e] = rows[j][e] - mu[e];
                            p += xv[e] * u[e];
                        }
                        p = wave_sum_d(p);
#pragma unroll
                        for (int e = 0; e < FPL; ++e)
                            wv[e] += p * xv[e];
                    });
                    slices_sum(wv);
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        u[e] = wv[e];
                    normalise();
                }
                walk([&](int64_t x, int j) { // projections on u^(2)
                    double p = 0.0;
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        p += (rows[j][e] - mu[e]) * u[e];
                    p = wave_sum_d(p);
                    if (lane == 0)
                        keys[x] = p;
                });
                if (sp == 0) {
#pragma unroll
                    for (int e = 0; e < FPL; ++e)
                        mu_out[lane + kWave * e] = (float)mu[e];
                    if (lane == 0)
                        node_meta[node] = FsbNodeMeta{(float)best, A, mn, -1};
                }
                node_sync();
                // sort the node's cells by (projection asc, id asc); the first half goes left
                for (int64_t size = 2; size <= nv; size <<= 1) {
                    for (int64_t stride = size >> 1; stride > 0; stride >>= 1) {
                        for (int64_t p = sp * kWave + lane; p < nv / 2; p += wpn * kWave) {
                            const int64_t i1 = 2 * p - (p & (stride - 1)), i2 = i1 + stride;
                            const bool asc = (i1 & size) == 0;
                            const double k1 = keys[i1], k2 = keys[i2];
                            const int32_t c1 = cells[i1], c2 = cells[i2];
                            const bool gt = k1 > k2 || (k1 == k2 && c1 > c2);
                            if (gt == asc) {
                                keys[i1] = k2;
                                keys[i2] = k1;
                                cells[i1] = c2;
                                cells[i2] = c1;
                            }
                        }
                        node_sync();
                    }
                }
            };
            if (xe - xb <= kBatch)
                node_passes(std::true_type{});
            else
                node_passes(std::false_type{});
        }
        team_sync();
    }
}

// ---------------------------------------------------------------- search

// Compare-exchange of two 64-bit keys: afterwards hi >= lo.
__device__ __forceinline__ void cx_desc(uint64_t &hi, uint64_t &lo)
{
    const uint64_t a = hi, b = lo;
    const bool sw = a < b;
    hi = sw ? b : a;
    lo = sw ? a : b;
}

// Bitonic sort of N keys into descending order (N a power of two; every index a
// compile-time constant after unrolling, so the keys stay in registers).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&x)[N])
{
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & k) == 0)
                        cx_desc(x[i], x[l]); // this run descending
                    else
                        cx_desc(x[l], x[i]); // this run ascending
                }
            }
}

// The N largest of two descending lists a and b, descending, into a: the
// elementwise larger of a and b reversed is a bitonic sequence that holds them,
// and a bitonic merge orders it.
template <int N>
__device__ __forceinline__ void merge_top_desc(uint64_t (&a)[N], const uint64_t (&b)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i)
        a[i] = a[i] > b[N - 1 - i] ? a[i] : b[N - 1 - i];
#pragma unroll
    for (int j = N >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int l = i ^ j;
            if (l > i)
                cx_desc(a[i], a[l]);
        }
}

constexpr int kMaxChunksPerForest = kFsbMaxLevels; // popcount of an admitted count below 2^13
constexpr int kMaxKids = 2 * kFsbMaxBeam;
constexpr uint32_t kJoinRef = 0x40000000u;

// Dynamic LDS of the search: bm and wb of fsb_search_words(Mu) words each, then the
// node list of up to 32 words' worth of entries per word; a forest of Mu cells has
// fewer than 2 Mu nodes (chunk trees and join nodes), and the candidate union at
// most Mu cells.
__host__ __device__ inline int fsb_search_words(int64_t Mu) { return (int)((2 * Mu + 63) / 32); }
inline size_t fsb_search_lds(int64_t Mu)
{
    const int nw = fsb_search_words(Mu);
    return (size_t)nw * 2 * sizeof(uint32_t) + (size_t)nw * 32 * sizeof(uint16_t);
}

template <typename T, int D>
struct SearchSmem {
    // bf16 queries read a node mean 8 features at a time (16-byte aligned rows; 4 words
    // of pad put 16 consecutive rows on distinct banks); fp32 ones one feature per lane
    static constexpr int kMuStride = sizeof(T) == 2 ? D + 4 : D + 1;
    // Per-query rows: the lanes of a wave each take their own query's row at the same
    // index, so rows are an odd number of words long (one word of pad) and the lanes'
    // words fall on distinct banks.
    int32_t beam[128][kFsbMaxBeam + 1]; // node refs of each query's beam
    int32_t nb[128];
    int32_t nk[128], nleaf[128];
    int32_t kpar[128][kFsbMaxBeam + 1]; // the beam's internal nodes, whose children 2 j, 2 j + 1 are ranked
    float ku[128][kMaxKids + 1];        // the children's priority (Eq. 11)
    uint16_t kmin[128][kMaxKids + 2];   // their smallest cell id
    uint16_t cand[128][kMaxKids + 2];   // candidate cells (forest 0, then the second forest)
    int32_t ncand[128];
    int32_t nlist;
    int32_t need_sel; // some query of the level has more children than free beam slots
    union {
        float mu[32][kMuStride];  // a tile of node means
        float ut[kWaves][32][33]; // then the tile's priorities: [wave][node row][query column]
        uint16_t kt16[32][D + 8];
        float kt32[32][D + 1];
    };
    float trho[32], tA[32];
    int32_t tmin[32];
    alignas(16) float jmu[kMaxChunksPerForest][D];
    FsbNodeMeta jmeta[kMaxChunksPerForest];
    int32_t jcount[kMaxChunksPerForest];
    double red[2][kThreads / kWave];
    // the block's forest: chunk t has 2^ck[t] cells, its nodes from node index cbase[t],
    // forest-local index lbase[t] .. lbase[t+1] - 1; join node t at lbase[r] + t
    int32_t ck[kMaxChunksPerForest];
    int64_t cbase[kMaxChunksPerForest];
    int32_t lbase[kMaxChunksPerForest + 1];
    int32_t r;
};

// bf16 queries: two workgroups per CU (at most 256 VGPRs, 80 KB of LDS at 16k tokens)
template <typename T>
constexpr int kSearchWavesPerSimd = sizeof(T) == 2 ? 2 : 1;

template <typename T, int D>
__global__ __launch_bounds__(kThreads, kSearchWavesPerSimd<T>) void fsb_search_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                              const float *__restrict__ a,
                                                              const int32_t *__restrict__ cnt,
                                                              const float *__restrict__ node_mu,
                                                              const FsbNodeMeta *__restrict__ node_meta,
                                                              int32_t *__restrict__ sel, int32_t *__restrict__ cand,
                                                              HeadConsts hc, FsbConsts fc, FsbLayout L, int64_t N,
                                                              int64_t M, int NB, int H, int K)
{
    constexpr bool kBf16 = sizeof(T) == 2;
    __shared__ SearchSmem<T, D> sm;
    // sized by the launch for this forest size (fsb_search_lds): bm and wb of nw words, then list
    extern __shared__ uint32_t dyn[];
    const int nw = fsb_search_words(L.Mu);
    uint32_t *const bm = dyn;                                  // the level's node set, or the candidates' cells
    int32_t *const wb = reinterpret_cast<int32_t *>(dyn + nw); // prefix counts of bm
    uint16_t *const list = reinterpret_cast<uint16_t *>(dyn + 2 * nw); // the level's nodes, or the candidates' cells
    const uint32_t lb = xcd_logical_block(blockIdx.x, gridDim.x);
    // a head's blocks from the last: later blocks search larger forests, so the longest start
    // first and the kernel ends on short ones
    const int beta = NB - 1 - (int)(lb % (uint32_t)NB);
    const int64_t bh = (int64_t)(lb / (uint32_t)NB);
    const int h = (int)(bh % H);
    const int t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1), half = lane >> 5, col = lane & 31;
    const int qs = wave * 32 + col; // this lane's query slot in the block
    const int64_t i = (int64_t)beta * 128 + qs;
    const bool q_ok = i < N;
    const float lam = hc.lambda[h], its = hc.inv_two_sigma[h];
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int Wb = fc.Wb;
    const int64_t n_avail = ((int64_t)beta * 128 / 32) < L.Mu ? ((int64_t)beta * 128 / 32) : L.Mu;

    // ---- the query as the B operand of the products: bf16, features 16 kc + 8 half .. + 7
    // (32x32x16); fp32, feature 2 kc + half (32x32x2) ----
    const T *qrow = q + (bh * N + (q_ok ? i : 0)) * D;
    constexpr int KB = kBf16 ? D / 16 : 1;
    constexpr int KF = kBf16 ? 1 : D / 2;
    bf16x8 qb[KB];
    float qf[KF];
    float qsq = 0.0f;
    if constexpr (kBf16) {
#pragma unroll
        for (int kc = 0; kc < KB; ++kc) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(qrow) + kc * 16 + half * 8);
            qb[kc] = as_bf16x8(w);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t we = w[e];
                const float x0 = bf16_bits_to_f32(we & 0xffffu), x1 = bf16_bits_to_f32(we >> 16);
                qsq = fmaf(x1, x1, fmaf(x0, x0, qsq));
            }
        }
    } else {
#pragma unroll
        for (int kc = 0; kc < KF; ++kc) {
            qf[kc] = qrow[2 * kc + half];
            qsq = fmaf(qf[kc], qf[kc], qsq);
        }
    }
    qsq += shfl_xor_f(qsq, 32);
    const float qnorm = sqrtf(qsq);

    if (t < 128)
        sm.ncand[t] = 0;

    for (int f = 0; f < 2; ++f) {
        const int64_t Mf = f == 0 ? n_avail : cnt[bh * (M + 1) + n_avail];
        if (Mf == 0)
            continue; // an empty forest adds no candidates (a block-uniform branch)
        // ---- the forest's chunks (Eq. 18) and join nodes (Eq. 21) ----
        if (t == 0) {
            int r = 0, lbase = 0;
            int64_t off = 0;
            for (int kk = kFsbMaxLevels - 1; kk >= 0; --kk) {
                if (!((Mf >> kk) & 1))
                    continue;
                const int64_t jj = (off >> kk) / 2; // the chunk starts at an even multiple of 2^kk
                sm.ck[r] = kk;
                sm.cbase[r] = (bh * 2 + f) * L.nodes + L.node_base[kk] + jj * ((2 << kk) - 1);
                sm.lbase[r] = lbase;
                lbase += (2 << kk) - 1;
                off += (int64_t)1 << kk;
                ++r;
            }
            sm.lbase[r] = lbase;
            sm.r = r;
        }
        __syncthreads();
        const int r = sm.r;
        // join nodes from the smallest chunk up: J_t over root(G_t) and J_(t+1) (or root(G_(r-1)))
        for (int jt = r - 2; jt >= 0; --jt) {
            const int64_t ra = sm.cbase[jt];
            const FsbNodeMeta ma = node_meta[ra];
            const double na = (double)((int64_t)1 << sm.ck[jt]);
            const float *mb_mu;
            FsbNodeMeta mb;
            double nbn;
            if (jt == r - 2) {
                mb_mu = node_mu + sm.cbase[r - 1] * D;
                mb = node_meta[sm.cbase[r - 1]];
                nbn = (double)((int64_t)1 << sm.ck[r - 1]);
            } else {
                mb_mu = sm.jmu[jt + 1];
                mb = sm.jmeta[jt + 1];
                nbn = (double)sm.jcount[jt + 1];
            }
            double da = 0.0, db = 0.0;
            if (t < D) {
                const double xa = node_mu[ra * D + t], xb = mb_mu[t];
                const double m = (na * xa + nbn * xb) / (na + nbn);
                sm.jmu[jt][t] = (float)m;
                da = (xa - m) * (xa - m);
                db = (xb - m) * (xb - m);
            }
            da = wave_sum_d(da);
            db = wave_sum_d(db);
            if (lane == 0) {
                sm.red[0][wave] = da;
                sm.red[1][wave] = db;
            }
            __syncthreads();
            if (t == 0) {
                double sa = 0.0, sb = 0.0;
                for (int w = 0; w < kWaves; ++w) {
                    sa += sm.red[0][w];
                    sb += sm.red[1][w];
                }
                const float rho = fmaxf(ma.rho + (float)sqrt(sa), mb.rho + (float)sqrt(sb));
                sm.jmeta[jt] = FsbNodeMeta{rho, fmaxf(ma.A, mb.A), min(ma.minid, mb.minid), -1};
                sm.jcount[jt] = (int32_t)(na + nbn);
            }
            __syncthreads();
        }
        const int lj = sm.lbase[r];
        // node refs: chunk node (t, heap h) = t << 16 | h; join node t = kJoinRef | t
        auto is_leaf = [&](int32_t ref) {
            return !(ref & kJoinRef) && (ref & 0xffff) >= (1 << sm.ck[ref >> 16]);
        };
        auto local_of = [&](int32_t ref) {
            return (ref & kJoinRef) ? lj + (ref & 0xffff) : sm.lbase[ref >> 16] + (ref & 0xffff) - 1;
        };
        // the node of local id lp (the inverse of local_of)
        auto ref_of = [&](int lp) -> int32_t {
            if (lp >= lj)
                return (int32_t)(kJoinRef | (lp - lj));
            int ct = 0; // chunk bases ascend: count those at or below lp
#pragma unroll
            for (int c = 1; c < kMaxChunksPerForest; ++c)
                ct += (c < r && lp >= sm.lbase[c]) ? 1 : 0;
            return (int32_t)((ct << 16) | (lp - sm.lbase[ct] + 1));
        };
        // child c (0 or 1) of internal node ref
        auto child_of = [&](int32_t ref, int c) -> int32_t {
            if (ref & kJoinRef) {
                const int jt = ref & 0xffff;
                if (c == 0)
                    return (jt << 16) | 1;
                return jt + 1 <= r - 2 ? (int32_t)(kJoinRef | (jt + 1)) : (int32_t)(((r - 1) << 16) | 1);
            }
            return ref + (ref & 0xffff) + c; // heap 2h, 2h + 1
        };
        const int32_t root = r == 1 ? (int32_t)((0 << 16) | 1) : (int32_t)(kJoinRef | 0);
        if (t < 128) {
            sm.beam[t][0] = root;
            sm.nb[t] = (int64_t)beta * 128 + t < N ? 1 : 0;
        }
        const int nwords = (sm.lbase[r] + r - 1 + 31) / 32;

        // ---- beam search, level by level ----
        for (;;) {
            for (int x = t; x < nwords; x += kThreads)
                bm[x] = 0u;
            if (t == 0)
                sm.need_sel = 0;
            __syncthreads();
            int nk = 0;
            { // expand this query's internal nodes, the pair's lanes taking half the beam each
              // (entries 8 half .. 8 half + 7; the parents in beam order, the second lane's after
              // the first's); leaves keep their slots.  Slots past nb hold stale refs, never used.
                constexpr int kHalfBeam = kFsbMaxBeam / 2;
                const int nbq = sm.nb[qs];
                int32_t refs[kHalfBeam];
#pragma unroll
                for (int e = 0; e < kHalfBeam; ++e)
                    refs[e] = sm.beam[qs][kHalfBeam * half + e];
                bool internal[kHalfBeam];
                int ni = 0, nl = 0;
#pragma unroll
                for (int e = 0; e < kHalfBeam; ++e) {
                    const bool here = kHalfBeam * half + e < nbq;
                    const bool leaf = here && is_leaf(refs[e]);
                    internal[e] = here && !leaf;
                    ni += internal[e] ? 1 : 0;
                    nl += leaf ? 1 : 0;
                }
                const int ni_other = __shfl_xor(ni, 32, kWave), nl_other = __shfl_xor(nl, 32, kWave);
                int pos = half ? ni_other : 0;
#pragma unroll
                for (int e = 0; e < kHalfBeam; ++e) {
                    if (internal[e]) { // the node is marked; the list takes both its children
                        sm.kpar[qs][pos++] = refs[e];
                        const int lp = local_of(refs[e]);
                        atomicOr(&bm[lp >> 5], 1u << (lp & 31));
                    }
                }
                nk = 2 * (ni + ni_other);
                const int nleaf = nl + nl_other;
                if (half == 0) {
                    sm.nk[qs] = nk;
                    sm.nleaf[qs] = nleaf;
                    if (nk > Wb - nleaf)
                        sm.need_sel = 1;
                }
            }
            if (!__syncthreads_or(nk > 0))
                break; // every beam holds only leaves
            if (sm.need_sel == 0) {
                // every query keeps all its children (the beams are not full yet): no
                // priorities are needed.  The beam takes its leaves, then the children in
                // the parents' order; the kept set is the one a ranking would keep, and no
                // later step depends on the order of a beam's nodes.
                if (half == 0 && nk > 0) {
                    const int nbq = sm.nb[qs];
                    int32_t refs[kFsbMaxBeam], par[kFsbMaxBeam];
#pragma unroll
                    for (int e = 0; e < kFsbMaxBeam; ++e) {
                        refs[e] = sm.beam[qs][e];
                        par[e] = sm.kpar[qs][e];
                    }
                    int nb2 = 0;
#pragma unroll
                    for (int e = 0; e < kFsbMaxBeam; ++e)
                        if (e < nbq && is_leaf(refs[e]))
                            sm.beam[qs][nb2++] = refs[e];
#pragma unroll
                    for (int j = 0; j < kFsbMaxBeam; ++j)
                        if (2 * j < nk) {
                            sm.beam[qs][nb2++] = child_of(par[j], 0);
                            sm.beam[qs][nb2++] = child_of(par[j], 1);
                        }
                    sm.nb[qs] = nb2;
                }
                __syncthreads();
                continue;
            }
            // the level's node list, two entries (children 0 and 1) per marked node: prefix
            // counts of marked nodes over the bitmap words, one word per lane of wave 0 (64
            // words a round, the total carried).  Children of different nodes are different
            // nodes, so the list never holds more entries than the forest has nodes.
            if (wave == 0) {
                int32_t carry = 0;
                for (int x0 = 0; x0 < nwords; x0 += kWave) {
                    const int x = x0 + lane;
                    const int32_t c = x < nwords ? __popc(bm[x]) : 0;
                    int32_t incl = c;
#pragma unroll
                    for (int off = 1; off < kWave; off <<= 1) {
                        const int32_t y = __shfl_up(incl, off, kWave);
                        if (lane >= off)
                            incl += y;
                    }
                    if (x < nwords)
                        wb[x] = carry + incl - c;
                    carry += __shfl(incl, kWave - 1, kWave);
                }
                if (lane == 0)
                    sm.nlist = 2 * carry;
            }
            __syncthreads();
            for (int lp = t; lp < nwords * 32; lp += kThreads) { // one local id per thread
                const uint32_t word = bm[lp >> 5];
                if ((word >> (lp & 31)) & 1u) {
                    const int32_t pos = 2 * (wb[lp >> 5] + __popc(word & ((1u << (lp & 31)) - 1u)));
                    const int32_t pref = ref_of(lp);
                    list[pos] = (uint16_t)local_of(child_of(pref, 0));
                    list[pos + 1] = (uint16_t)local_of(child_of(pref, 1));
                }
            }
            __syncthreads();
            const int Z = sm.nlist;
            // ---- priorities (Eq. 11) of the level's nodes, 32 at a time, for all 128 queries ----
            for (int t0 = 0; t0 < Z; t0 += 32) {
                { // stage the tile's means and summaries
                    const int row = t / 8, part = t % 8;
                    constexpr int FP = D / 8; // features per thread
                    const int u = t0 + row;
                    const float *src = nullptr;
                    FsbNodeMeta meta{0.0f, 0.0f, 0, -1};
                    if (u < Z) {
                        const int l = list[u];
                        if (l >= lj) {
                            src = sm.jmu[l - lj];
                            meta = sm.jmeta[l - lj];
                        } else {
                            int ct = 0;
                            while (ct + 1 < r && l >= sm.lbase[ct + 1])
                                ++ct;
                            const int64_t gi = sm.cbase[ct] + (l - sm.lbase[ct]);
                            src = node_mu + gi * D;
                            meta = node_meta[gi];
                        }
                    }
                    // 16-byte loads (node and join means are rows of D floats, 16-byte aligned)
#pragma unroll
                    for (int e = 0; e < FP; e += 4) {
                        const float4 v4 = src ? *reinterpret_cast<const float4 *>(src + part * FP + e)
                                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        sm.mu[row][part * FP + e] = v4.x;
                        sm.mu[row][part * FP + e + 1] = v4.y;
                        sm.mu[row][part * FP + e + 2] = v4.z;
                        sm.mu[row][part * FP + e + 3] = v4.w;
                    }
                    if (part == 0) {
                        sm.trho[row] = meta.rho;
                        sm.tA[row] = meta.A;
                        sm.tmin[row] = meta.minid;
                    }
                }
                __syncthreads();
                f32x16 acc;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr)
                    acc[rr] = 0.0f;
                if constexpr (kBf16) {
                    // q . mu with mu as bf16 hi + mid + lo parts (exactly the fp32 mean) and the
                    // products added in one fp32 accumulator, smallest part first in each step
#pragma unroll
                    for (int kc = 0; kc < KB; ++kc) {
                        const float *mrow = &sm.mu[col][kc * 16 + half * 8]; // node row col
                        const u32x4 m0 = *reinterpret_cast<const u32x4 *>(mrow);
                        const u32x4 m1 = *reinterpret_cast<const u32x4 *>(mrow + 4);
                        u32x4 ph, pm, pl;
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const float x0 = __uint_as_float(w < 2 ? m0[2 * w] : m1[2 * w - 4]);
                            const float x1 = __uint_as_float(w < 2 ? m0[2 * w + 1] : m1[2 * w - 3]);
                            const uint32_t hp = cvt_pk_bf16(x0, x1);
                            const float r0 = x0 - __uint_as_float(hp << 16), r1 = x1 - __uint_as_float(hp & 0xffff0000u);
                            const uint32_t mp = cvt_pk_bf16(r0, r1);
                            ph[w] = hp;
                            pm[w] = mp;
                            pl[w] = cvt_pk_bf16(r0 - __uint_as_float(mp << 16), r1 - __uint_as_float(mp & 0xffff0000u));
                        }
                        acc = mfma_bf16(as_bf16x8(pl), qb[kc], acc);
                        acc = mfma_bf16(as_bf16x8(pm), qb[kc], acc);
                        acc = mfma_bf16(as_bf16x8(ph), qb[kc], acc);
                    }
                } else {
#pragma unroll
                    for (int kc = 0; kc < KF; ++kc)
                        acc = mfma_f32(sm.mu[col][2 * kc + half], qf[kc], acc); // node row col, query column col
                }
                __syncthreads(); // every wave has read the means: the area takes the priorities
                // erf only below 4 (from there on it rounds to 1 in fp32); a wave takes it
                // only if one of its queries is that close to a node's earliest cell
                float pm[16], pmax = -INFINITY;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    pm[rr] = ((float)sm.tmin[acc_row(rr, half)] + 0.5f) * 32.0f;
                    pmax = fmaxf(pmax, pm[rr]);
                }
                const bool need_erf = __ballot(((float)i - pmax) * its < 4.0f) != 0ull;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int row = acc_row(rr, half);
                    float g = 1.0f;
                    if (need_erf) {
                        const float x = ((float)i - pm[rr]) * its;
                        if (x < 4.0f)
                            g = erff(x);
                    }
                    sm.ut[wave][row][col] =
                        fmaf(fmaf(fc.c * qnorm, sm.trho[row], acc[rr]), inv_sqrt_d, lam * sm.tA[row] * g);
                }
                wave_lds_sync();
                for (int e = half; e < sm.nk[qs]; e += 2) {
                    // the child's position in the level's node list: after both children of
                    // every node marked before its parent
                    const int lp = local_of(sm.kpar[qs][e >> 1]);
                    const int u = 2 * (wb[lp >> 5] + __popc(bm[lp >> 5] & ((1u << (lp & 31)) - 1u))) + (e & 1) - t0;
                    if (u >= 0 && u < 32) {
                        sm.ku[qs][e] = sm.ut[wave][u][col];
                        sm.kmin[qs][e] = (uint16_t)sm.tmin[u];
                    }
                }
                __syncthreads();
            }
            // ---- each query keeps its leaves and its best Wb - #leaves children ----
            {
                // this lane's children (every other one) sorted, then the best kFsbMaxBeam of
                // its list and the partner lane's (which ranked the others); the keys are
                // distinct, so this is the order any exact top-kFsbMaxBeam selection gives
                static_assert(kMaxKids == 2 * kFsbMaxBeam, "each lane of the pair ranks half the children");
                uint64_t top[kFsbMaxBeam];
                const int nkq = sm.nk[qs];
#pragma unroll
                for (int j = 0; j < kFsbMaxBeam; ++j) {
                    const int e = 2 * j + half;
                    top[j] = e < nkq ? rank_key(sm.ku[qs][e], ((0xffffu - sm.kmin[qs][e]) << 16) | (uint32_t)e) : 0ull;
                }
                sort_desc<kFsbMaxBeam>(top);
                uint64_t other[kFsbMaxBeam];
#pragma unroll
                for (int j = 0; j < kFsbMaxBeam; ++j) {
                    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)top[j], 32, kWave);
                    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(top[j] >> 32), 32, kWave);
                    other[j] = ((uint64_t)hi << 32) | lo;
                }
                merge_top_desc<kFsbMaxBeam>(top, other);
                if (nkq > 0) {
                    // both lanes of the pair hold the same top list; each takes half of the
                    // old beam (its leaves, at an offset from the partner's count) and half of
                    // the kept children, which are a prefix of the list (zero keys sort last).
                    // The old beam and the parents are read before any write.
                    constexpr int kHalfBeam = kFsbMaxBeam / 2;
                    const int nbq = sm.nb[qs];
                    int32_t refs[kHalfBeam], par[kHalfBeam];
#pragma unroll
                    for (int e = 0; e < kHalfBeam; ++e) {
                        refs[e] = sm.beam[qs][kHalfBeam * half + e];
                        // in bounds for every key
                        par[e] = sm.kpar[qs][(int)(top[kHalfBeam * half + e] & 0xffffu) >> 1];
                    }
                    bool leaf[kHalfBeam];
                    int nl = 0;
#pragma unroll
                    for (int e = 0; e < kHalfBeam; ++e) {
                        leaf[e] = kHalfBeam * half + e < nbq && is_leaf(refs[e]);
                        nl += leaf[e] ? 1 : 0;
                    }
                    const int nl_other = __shfl_xor(nl, 32, kWave);
                    const int NL = nl + nl_other; // the beam's leaves (sm.nleaf)
                    int pos = half ? nl_other : 0;
#pragma unroll
                    for (int e = 0; e < kHalfBeam; ++e)
                        if (leaf[e])
                            sm.beam[qs][pos++] = refs[e];
                    const int keep = Wb - NL;
                    int nkept = 0;
#pragma unroll
                    for (int e = 0; e < kFsbMaxBeam; ++e)
                        nkept += (e < keep && top[e] != 0ull) ? 1 : 0;
#pragma unroll
                    for (int e = 0; e < kHalfBeam; ++e) {
                        const int ee = kHalfBeam * half + e;
                        if (ee < nkept)
                            sm.beam[qs][NL + ee] = child_of(par[e], (int)(top[ee] & 1u));
                    }
                    if (half == 0)
                        sm.nb[qs] = NL + nkept;
                }
            }
            __syncthreads();
        }
        // ---- the leaves reached join the query's candidates (deduplicated) ----
        if (half == 0) {
            // every beam node is a leaf now: all their cells are requested at once,
            // then taken in beam order
            const int nbq = sm.nb[qs];
            int32_t leaf_cell[kFsbMaxBeam];
#pragma unroll
            for (int e = 0; e < kFsbMaxBeam; ++e) {
                leaf_cell[e] = -1;
                if (e < nbq) {
                    const int32_t ref = sm.beam[qs][e];
                    leaf_cell[e] = node_meta[sm.cbase[ref >> 16] + (ref & 0xffff) - 1].cell;
                }
            }
            // one forest's leaves are distinct cells: a leaf can repeat only a candidate
            // of the forest before, at most kFsbMaxBeam of them, compared in registers
            int nc = sm.ncand[qs];
            const int nc0 = nc;
            int32_t prev[kFsbMaxBeam];
#pragma unroll
            for (int x = 0; x < kFsbMaxBeam; ++x)
                prev[x] = x < nc0 ? (int32_t)sm.cand[qs][x] : -1;
#pragma unroll
            for (int e = 0; e < kFsbMaxBeam; ++e) {
                if (e < nbq) {
                    const int32_t cell = leaf_cell[e];
                    bool dup = false;
#pragma unroll
                    for (int x = 0; x < kFsbMaxBeam; ++x)
                        dup |= prev[x] == cell;
                    if (!dup)
                        sm.cand[qs][nc++] = (uint16_t)cell; // cell ids < kFsbMaxCells
                }
            }
            sm.ncand[qs] = nc;
        }
        __syncthreads();
    }

    // ---- candidates in ascending id order; their union over the block ----
    const int mwords = (int)((n_avail + 31) / 32);
    for (int x = t; x < mwords; x += kThreads)
        bm[x] = 0u;
    __syncthreads();
    if (half == 0) {
        // the query's candidates (distinct ids) in ascending order: each one's rank is
        // the number of smaller ones, counted in registers
        const int nc = sm.ncand[qs];
        int32_t cv[kMaxKids];
#pragma unroll
        for (int x = 0; x < kMaxKids; ++x)
            cv[x] = x < nc ? (int32_t)sm.cand[qs][x] : INT_MAX;
#pragma unroll
        for (int x = 0; x < kMaxKids; ++x) {
            if (x < nc) {
                int rank = 0;
#pragma unroll
                for (int y = 0; y < kMaxKids; ++y)
                    rank += cv[y] < cv[x] ? 1 : 0;
                sm.cand[qs][rank] = (uint16_t)cv[x];
                atomicOr(&bm[cv[x] >> 5], 1u << (cv[x] & 31));
            }
        }
    }
    __syncthreads();
    if (wave == 0) { // prefix counts over the words, one word per lane (as for a level)
        int32_t carry = 0;
        for (int x0 = 0; x0 < mwords; x0 += kWave) {
            const int x = x0 + lane;
            const int32_t c = x < mwords ? __popc(bm[x]) : 0;
            int32_t incl = c;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int32_t y = __shfl_up(incl, off, kWave);
                if (lane >= off)
                    incl += y;
            }
            if (x < mwords)
                wb[x] = carry + incl - c;
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (lane == 0)
            sm.nlist = carry;
    }
    __syncthreads();
    for (int c = t; c < mwords * 32; c += kThreads) { // one cell id per thread
        const uint32_t word = bm[c >> 5];
        if ((word >> (c & 31)) & 1u)
            list[wb[c >> 5] + __popc(word & ((1u << (c & 31)) - 1u))] = (uint16_t)c;
    }
    __syncthreads();

    // ---- rerank (Eq. 12): one candidate cell at a time, all queries on the matrix cores ----
    uint64_t topk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        topk[e] = 0ull;
    const int nc = sm.ncand[qs];
    const int Zc = sm.nlist;
    const T *kh = k + bh * N * D;
    // bf16: a cell's 32 token keys, 16 bytes per thread, the next cell's in flight while the
    // current one is on the matrix cores
    constexpr int KR = kBf16 ? (32 * D / 8 + kThreads - 1) / kThreads : 1;
    u32x4 pre[KR];
    auto fetch_keys = [&](int32_t c) {
        const uint16_t *src = reinterpret_cast<const uint16_t *>(kh) + (int64_t)c * 32 * D;
#pragma unroll
        for (int r = 0; r < KR; ++r) {
            const int x = t + r * kThreads;
            if (x < 32 * D / 8)
                pre[r] = *reinterpret_cast<const u32x4 *>(src + (int64_t)(x / (D / 8)) * D + (x % (D / 8)) * 8);
        }
    };
    if (kBf16 && Zc > 0)
        fetch_keys(list[0]);
    int cp = 0; // this lane's place in its candidates (both lists ascend)
    for (int u = 0; u < Zc; ++u) {
        const int32_t c = list[u];
        if constexpr (kBf16) {
#pragma unroll
            for (int r = 0; r < KR; ++r) {
                const int x = t + r * kThreads;
                if (x < 32 * D / 8)
                    *reinterpret_cast<u32x4 *>(&sm.kt16[x / (D / 8)][(x % (D / 8)) * 8]) = pre[r];
            }
        } else {
            const float *src = reinterpret_cast<const float *>(kh) + (int64_t)c * 32 * D;
            for (int x = t; x < 32 * D; x += kThreads)
                sm.kt32[x / D][x % D] = src[x];
        }
        __syncthreads();
        if (kBf16 && u + 1 < Zc)
            fetch_keys(list[u + 1]);
        f32x16 acc;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            acc[rr] = 0.0f;
        if constexpr (kBf16) {
#pragma unroll
            for (int kc = 0; kc < KB; ++kc)
                acc = mfma_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(&sm.kt16[col][kc * 16 + half * 8])), qb[kc],
                                acc);
        } else {
#pragma unroll
            for (int kc = 0; kc < D / 2; ++kc)
                acc = mfma_f32(sm.kt32[col][2 * kc + half], qf[kc], acc);
        }
        // is c one of this query's candidates? (sorted, at most 2 Wb; the cells come ascending)
        while (cp < nc && (int32_t)sm.cand[qs][cp] < c)
            ++cp;
        const bool mine = cp < nc && (int32_t)sm.cand[qs][cp] == c;
        float m = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            m = fmaxf(m, acc[rr] * inv_sqrt_d);
        m = fmaxf(m, shfl_xor_f(m, 32));
        float z = 0.0f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            z += expf(acc[rr] * inv_sqrt_d - m);
        z += shfl_xor_f(z, 32);
        if (mine) {
            const float g = erff(((float)i - ((float)c + 0.5f) * 32.0f) * its);
            const float score = m + logf(z) + lam * a[bh * M + c] * g;
            insert_key<8>(topk, rank_key(score, 0x7fffffffu - (uint32_t)c));
        }
        __syncthreads();
    }
    if (half == 0 && q_ok) {
        int32_t *dst = sel + (bh * N + i) * K;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < K)
                dst[e] = topk[e] ? (int32_t)(0x7fffffffu - (uint32_t)topk[e]) : -1;
        if (cand) {
            int32_t *cd = cand + (bh * N + i) * 2 * Wb;
            for (int x = 0; x < 2 * Wb; ++x)
                cd[x] = x < nc ? (int32_t)sm.cand[qs][x] : -1;
        }
    }
}

template <typename T, int D>
hipError_t launch_t(const Geometry &g, const FsbLayout &L, const HeadConsts &hc, const FsbConsts &fc, const void *q,
                    const void *k, const double *kbar64, const float *a, const double *a64, int32_t *adm,
                    int32_t *adm_count, float *node_mu, FsbNodeMeta *node_meta, int32_t *sel, int32_t *cand,
                    hipStream_t st)
{
    hipLaunchKernelGGL(fsb_admit_kernel, dim3((unsigned)g.bh), dim3(kThreads), 0, st, a64, adm, adm_count, g.M, g.H,
                       fc);
    if (L.Mu > 0) {
        const int64_t groups = (int64_t)g.bh * 2; // (sequence, head, forest) triples
        int64_t blocks = 0;
        for (int k = 0; k < L.levels; ++k)
            blocks += build_span(L.chunk_base[k + 1] - L.chunk_base[k], groups, k);
        hipLaunchKernelGGL((fsb_build_kernel<D>), dim3((unsigned)blocks), dim3(kBuildThreads), 0, st, kbar64, a,
                           adm, adm_count, node_mu, node_meta, g.M, L, groups);
    }
    hipLaunchKernelGGL((fsb_search_kernel<T, D>), dim3((unsigned)((int64_t)g.bh * g.NB)), dim3(kThreads),
                       fsb_search_lds(L.Mu), st,
                       static_cast<const T *>(q), static_cast<const T *>(k), a, adm_count, node_mu, node_meta, sel,
                       cand, hc, fc, L, g.N, g.M, g.NB, g.H, g.K);
    return hipGetLastError();
}

} // namespace

hipError_t launch_fsb(const Geometry &g, const FsbLayout &L, const HeadConsts &hc, const FsbConsts &fc,
                      const void *q, const void *k, const double *kbar64, const float *a, const double *a64,
                      int32_t *adm, int32_t *adm_count, float *node_mu, FsbNodeMeta *node_meta, int32_t *sel,
                      int32_t *cand, hipStream_t st)
{
    if (g.bf16)
        return g.d == 64 ? launch_t<uint16_t, 64>(g, L, hc, fc, q, k, kbar64, a, a64, adm, adm_count, node_mu,
                                                  node_meta, sel, cand, st)
                         : launch_t<uint16_t, 128>(g, L, hc, fc, q, k, kbar64, a, a64, adm, adm_count, node_mu,
                                                   node_meta, sel, cand, st);
    return g.d == 64 ? launch_t<float, 64>(g, L, hc, fc, q, k, kbar64, a, a64, adm, adm_count, node_mu, node_meta,
                                           sel, cand, st)
                     : launch_t<float, 128>(g, L, hc, fc, q, k, kbar64, a, a64, adm, adm_count, node_mu, node_meta,
                                            sel, cand, st);
}

} // namespace fsl
