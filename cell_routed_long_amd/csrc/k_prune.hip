// FS-L retained sets (FreeSolo, Sec. 3.3 "Query-independent pruning", Eq. 8, over
// the causal prefix of Eq. 6): A_beta = Recent_W(C_beta) u TopP(a_c), C_beta the
// cells ending at or before the block start beta*B.
//
// Instead of replaying the incremental top-P merge block after block (one long
// serial chain per head), the prefill computes for every cell the block at
// which it leaves TopP.  A cell c belongs to TopP(C_beta) iff fewer than P cells
// of C_beta outrank it by (a desc, id asc).  The outranking cells of C_beta only
// grow with beta, so if e is the P-th outranking cell in id order, c is in
// TopP(C_beta) exactly for the blocks that contain c and satisfy
// beta < death(c) = e / (B/s) + 1 (the first block in which e is available).
// This gives the same sets as the page's Eq. 15 merge (App. C "Bounded cache")
// with every block independent:
//   prune_death_kernel: one wave per cell scans the head's norms 64 ids at a
//       time; the ballot of "id x outranks c" counts outranking cells, and the
//       P-th one is located inside the 64-id window where the count reaches P;
//   prune_emit_kernel:  one wave per (head, block) collects the non-recent cells
//       still alive plus the W most recent cells and writes them in priority
//       order (a desc, id asc), so that the scorer meets the cells with the
//       largest prior terms first.
#include "fsl_internal.h"

#include <climits>

namespace fsl {
namespace {

constexpr int kDeathThreads = 256;
constexpr int kDeathCells = kDeathThreads / kWave; // cells per workgroup, one per wave

__global__ __launch_bounds__(kDeathThreads) void prune_death_kernel(const float *__restrict__ a,
                                                                    int32_t *__restrict__ death, int64_t M,
                                                                    int P, int cells_per_block)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t head = blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kDeathCells + (threadIdx.x / kWave);
    if (c >= M)
        return; // whole wave
    const float *ah = a + head * M;
    const float ac = ah[c];
    int64_t e = -1; // id of the P-th cell outranking c, in id order
    if (P > 0) {
        int count = 0;
        for (int64_t base = 0; base < M; base += kWave) {
            const int64_t x = base + lane;
            const float ax = x < M ? ah[x] : 0.0f;
            const bool o = x < M && (ax > ac || (ax == ac && x < c)); // x ranks before c
            const uint64_t m = __ballot(o);
            const int n = __popcll(m);
            if (count + n >= P) {
                const int before = __popcll(m & ((1ull << lane) - 1ull));
                const uint64_t hit = __ballot(o && before == P - count - 1);
                e = base + __ffsll((unsigned long long)hit) - 1;
                break;
            }
            count += n;
        }
    }
    if (lane == 0) {
        int32_t dth;
        if (P == 0)
            dth = 0; // never in TopP
        else if (e < 0)
            dth = INT32_MAX;
        else
            dth = (int32_t)(e / cells_per_block + 1);
        death[head * M + c] = dth;
    }
}

__global__ __launch_bounds__(kWave) void prune_emit_kernel(const int32_t *__restrict__ death,
                                                           const float *__restrict__ a,
                                                           int32_t *__restrict__ retained,
                                                           int32_t *__restrict__ n_ret, int64_t M, int NB,
                                                           int cap, int W, int cells_per_block)
{
    __shared__ __attribute__((aligned(16))) int32_t s_id[kMaxRetainedCap + 4];
    __shared__ __attribute__((aligned(16))) float s_a[kMaxRetainedCap + 4];
    const int beta = blockIdx.x;
    const int64_t head = blockIdx.y;
    const int lane = threadIdx.x;
    int64_t n_avail = (int64_t)beta * cells_per_block; // |C_beta|, Eq. 6
    if (n_avail > M)
        n_avail = M;
    const int64_t recent0 = n_avail > W ? n_avail - W : 0;
    const int32_t *dh = death + head * M;
    const float *ah = a + head * M;
    int32_t *dst = retained + (head * NB + beta) * (int64_t)cap;
    int count = 0;
    // non-recent cells still in TopP: exit blocks and norms, 8 windows of 64 per round trip
    constexpr int kWin = 8;
    for (int64_t base = 0; base < recent0; base += kWin * kWave) {
        int32_t dv[kWin];
        float av[kWin];
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
            const int64_t c = base + u * kWave + lane;
            dv[u] = c < recent0 ? dh[c] : 0;
            av[u] = c < recent0 ? ah[c] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kWin; ++u) {
            const int64_t c = base + u * kWave + lane;
            const bool keep = c < recent0 && dv[u] > beta;
            const uint64_t mask = __ballot(keep);
            const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
            if (keep && pos < cap) {
                s_id[pos] = (int32_t)c;
                s_a[pos] = av[u];
            }
            count += __popcll(mask);
        }
    }
    if (count > cap - (int)(n_avail - recent0)) // only reachable with non-finite norms
        count = cap - (int)(n_avail - recent0);
    // the W most recent cells
    for (int64_t c = recent0 + lane; c < n_avail; c += kWave) {
        s_id[count + (c - recent0)] = (int32_t)c;
        s_a[count + (c - recent0)] = ah[c];
    }
    count += (int)(n_avail - recent0);
    const int n4 = (count + 3) & ~3;
    for (int x = count + lane; x < n4; x += kWave) { // padding ranks last
        s_a[x] = -INFINITY;
        s_id[x] = INT32_MAX;
    }
    __syncthreads();
    // priority order (a desc, id asc): each cell's rank is the number of cells before it
    for (int x = lane; x < count; x += kWave) {
        const float ax = s_a[x];
        const int32_t cx = s_id[x];
        int rank = 0;
        for (int y = 0; y < n4; y += 4) {
            const u32x4 va = *reinterpret_cast<const u32x4 *>(&s_a[y]);
            const u32x4 vi = *reinterpret_cast<const u32x4 *>(&s_id[y]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rank += ranks_before(__uint_as_float(va[e]), (int)vi[e], ax, cx) ? 1 : 0;
        }
        dst[rank] = cx;
    }
    for (int x = count + lane; x < cap; x += kWave)
        dst[x] = -1;
    if (lane == 0)
        n_ret[head * NB + beta] = count;
}

// For list building, two passes that need no per-block sort:
//   prune_rank_kernel: four lanes per cell compare its key (norm_key) with
//       every key of the head, staged in LDS, 64 keys per round (16 per lane):
//       the number of larger keys is the cell's rank in priority order (a
//       desc, id asc), and the P-th larger key in id order is its exit
//       block's cell e (a prefix sum over the four lanes' counts tells which
//       lane's 16 keys hold it).  The cell is written as (exit block, id) at
//       its rank, so `ord` lists the head's cells in priority order;
//   prune_list_kernel: the order is staged in LDS once per 16 blocks of a head,
//       and one wave per block keeps, in that order, the cells of C_beta still
//       in TopP (exit block > beta) or among the W most recent, which is A_beta
//       already in priority order.
constexpr int kRankMaxCells = 4096; // keys of one head in LDS (32 KB)
constexpr int kRankThreads = 256;   // 64 cells per workgroup, four lanes each

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x)
{
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, true);
}

__global__ __launch_bounds__(kRankThreads) void prune_rank_kernel(const float *__restrict__ a,
                                                                  int32_t *__restrict__ death,
                                                                  int64_t *__restrict__ ord, int64_t M, int P,
                                                                  int cells_per_block)
{
    __shared__ __attribute__((aligned(16))) uint64_t s_key[kRankMaxCells];
    const int64_t head = blockIdx.y;
    const int t = threadIdx.x;
    const int m = (int)M; // <= kRankMaxCells (host check)
    const int m64 = (m + 63) & ~63;
    const float *ah = a + head * M;
    for (int x = t; x < m64; x += kRankThreads)
        s_key[x] = x < m ? norm_key(ah[x], x) : 0; // 0 is below every key
    __syncthreads();
    const int c = blockIdx.x * (kRankThreads / 4) + t / 4;
    const int sub = t & 3; // this lane's 16 keys of every 64
    const uint64_t kc = s_key[c < m ? c : 0];
    int count = 0, e = -1; // larger keys in the rounds so far; the P-th of them in id order
    for (int base = 0; base < m64; base += 64) {
        uint64_t k[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(&s_key[base + 16 * sub + 2 * j]);
            k[2 * j] = ((uint64_t)w[1] << 32) | w[0];
            k[2 * j + 1] = ((uint64_t)w[3] << 32) | w[2];
        }
        int n = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            n += k[j] > kc ? 1 : 0;
        // counts of the quad's four lanes (quad_perm broadcasts of lanes 0..3)
        const int n0 = dpp_i<0x00>(n), n1 = dpp_i<0x55>(n), n2 = dpp_i<0xAA>(n), n3 = dpp_i<0xFF>(n);
        const int before = count + (sub > 0 ? n0 : 0) + (sub > 1 ? n1 : 0) + (sub > 2 ? n2 : 0);
        int e_here = -1;
        if (before < P && before + n >= P) { // the P-th larger key is one of these 16
            int need = P - before;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (k[j] > kc && need > 0 && --need == 0)
                    e_here = base + 16 * sub + j;
        }
        e_here = max(e_here, dpp_i<0xB1>(e_here)); // quad_perm [1,0,3,2]
        e_here = max(e_here, dpp_i<0x4E>(e_here)); // quad_perm [2,3,0,1]
        e = max(e, e_here);
        count += (n0 + n1) + (n2 + n3);
    }
    if (c >= m || sub != 0)
        return;
    const int32_t dth = P == 0 ? 0 : (e < 0 ? INT32_MAX : (int32_t)(e / cells_per_block + 1));
    death[head * M + c] = dth;
    ord[head * M + count] = ((int64_t)dth << 32) | (uint32_t)c; // keys are distinct: ranks are a permutation
}

constexpr int kListThreads = 1024; // 16 blocks of one head per workgroup, one wave each
constexpr int kListBlocks = kListThreads / kWave;

__global__ __launch_bounds__(kListThreads) void prune_list_kernel(const int64_t *__restrict__ ord,
                                                                  int32_t *__restrict__ retained,
                                                                  int32_t *__restrict__ n_ret, int64_t M, int NB,
                                                                  int cap, int W, int cells_per_block)
{
    __shared__ int64_t s_ord[kRankMaxCells]; // the head's cells in priority order, read once
    const int64_t head = blockIdx.y;
    const int t = threadIdx.x, lane = t & (kWave - 1);
    const int m = (int)M; // <= kRankMaxCells (host check)
    const int64_t *oh = ord + head * M;
    for (int x = t; x < m; x += kListThreads)
        s_ord[x] = oh[x];
    __syncthreads();
    const int beta = blockIdx.x * kListBlocks + t / kWave;
    if (beta >= NB)
        return; // whole wave
    const int n_avail = (int64_t)beta * cells_per_block < M ? beta * cells_per_block : m; // |C_beta|, Eq. 6
    const int recent0 = n_avail > W ? n_avail - W : 0;
    int32_t *dst = retained + (head * NB + beta) * (int64_t)cap;
    int count = 0;
    for (int base = 0; base < m; base += kWave) {
        const int j = base + lane;
        const int64_t ov = j < m ? s_ord[j] : -1;
        const int32_t c = (int32_t)(uint32_t)ov;
        const int32_t d = (int32_t)(ov >> 32);
        const bool keep = c >= 0 && (c < recent0 ? d > beta : c < n_avail);
        const uint64_t mask = __ballot(keep);
        const int pos = count + __popcll(mask & ((1ull << lane) - 1ull));
        if (keep && pos < cap) // at most P non-recent cells stay in TopP(C_beta): pos < P + W
            dst[pos] = c;
        count += __popcll(mask);
    }
    if (count > cap)
        count = cap;
    for (int x = count + lane; x < cap; x += kWave)
        dst[x] = -1;
    if (lane == 0)
        n_ret[head * NB + beta] = count;
}

} // namespace

hipError_t launch_prune(const Geometry &g, const float *a, int32_t *death, int64_t *ord, int32_t *retained,
                        int32_t *n_ret, int emit, hipStream_t st)
{
    const int cpb = g.B / g.s;
    if (emit && g.M > 0 && g.M <= kRankMaxCells) {
        dim3 grid((unsigned)((g.M + kRankThreads / 4 - 1) / (kRankThreads / 4)), (unsigned)g.bh);
        hipLaunchKernelGGL(prune_rank_kernel, grid, dim3(kRankThreads), 0, st, a, death, ord, g.M, g.P, cpb);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        dim3 grid2((unsigned)((g.NB + kListBlocks - 1) / kListBlocks), (unsigned)g.bh);
        hipLaunchKernelGGL(prune_list_kernel, grid2, dim3(kListThreads), 0, st, ord, retained, n_ret, g.M, g.NB,
                           g.cap, g.W, cpb);
        return hipGetLastError();
    }
    if (g.M > 0) {
        dim3 grid((unsigned)((g.M + kDeathCells - 1) / kDeathCells), (unsigned)g.bh);
        hipLaunchKernelGGL(prune_death_kernel, grid, dim3(kDeathThreads), 0, st, a, death, g.M, g.P, cpb);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if (!emit)
        return hipSuccess;
    dim3 grid2((unsigned)g.NB, (unsigned)g.bh);
    hipLaunchKernelGGL(prune_emit_kernel, grid2, dim3(kWave), 0, st, death, a, retained, n_ret, g.M, g.NB, g.cap, g.W,
                       cpb);
    return hipGetLastError();
}

} // namespace fsl
