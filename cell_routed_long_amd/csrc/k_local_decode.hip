// Streaming decode of the local branch (FreeSolo, Sec. 3.2, Eqs. 3-4; the
// window moves one token per step) with the branch combination of Eq. 2.
//
// A step for the token at position i reads the window [max(0, i - w), i]: the
// step's own k_new, v_new (offset o = 0) and the ring's tokens i - o for
// 0 < o < min(i + 1, w + 1).  Logits take the relative form of Eq. 3,
// q_i . R(-o) k_{i-o}, with R(-o) turning feature pair m by -o theta_m; the
// cos/sin of o theta_m come from a table built once per state in fp64, so the
// ring holds raw keys and no angle grows with the position.
//
// One workgroup per (sequence, head).  Sixteen lanes share a row (a token):
// each holds d/16 features of its key, value and table entries, so a row is
// one coalesced read per array.  Every group of 16 lanes runs its own online
// softmax over its rows; the groups meet in LDS at the end.  Row loads of
// kUnroll passes are issued before any of them is used.  Finally the new token
// goes into slot i mod (w + 1), whose old token i - w - 1 is outside this and
// every later window.
#include "fsl_internal.h"

namespace fsl {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;
constexpr int kGroups = kThreads / kLanesPerRow; // rows per pass of the workgroup
constexpr int kUnroll = 4;                        // passes whose loads are in flight together

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_bits_to_f32(x); }
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return (uint16_t)f32_to_bf16_bits(x); }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// NDW consecutive dwords (NDW = 2, 4 or 8; 8-byte aligned, 16-byte for NDW >= 4).
template <int NDW>
__device__ __forceinline__ void load_dwords(const char *p, uint32_t (&r)[NDW])
{
    if constexpr (NDW == 2) {
        const u32x2 a = *reinterpret_cast<const u32x2 *>(p);
        r[0] = a.x;
        r[1] = a.y;
    } else {
#pragma unroll
        for (int c = 0; c < NDW / 4; ++c) {
            const u32x4 a = reinterpret_cast<const u32x4 *>(p)[c];
            r[4 * c] = a.x;
            r[4 * c + 1] = a.y;
            r[4 * c + 2] = a.z;
            r[4 * c + 3] = a.w;
        }
    }
}

// Feature e of a lane's features held as raw dwords.
template <typename T, int NDW>
__device__ __forceinline__ float feature(const uint32_t (&r)[NDW], int e)
{
    if constexpr (sizeof(T) == 2)
        return bf16_bits_to_f32((e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xffffu));
    else
        return __uint_as_float(r[e]);
}

// ---- rotation table: (cos, sin) of o * theta_m, theta_m = base^(-2m/d) ----
__global__ __launch_bounds__(256) void local_table_kernel(float2 *__restrict__ table, int64_t R, int NP, int d,
                                                          float rope_base)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= R * NP)
        return;
    const int m = (int)(e % NP);
    const double theta = pow((double)rope_base, -2.0 * (double)m / (double)d);
    double sn, cs;
    sincos((double)(e / NP) * theta, &sn, &cs);
    table[e] = make_float2((float)cs, (float)sn);
}

// ---- records from the n tokens before position pos (the window keeps the last min(n, w)) ----
template <typename T, int D>
__global__ __launch_bounds__(256) void local_state_build_kernel(char *__restrict__ state, LocalStateLayout L,
                                                                LocalStateHeader hdr, const T *__restrict__ k,
                                                                const T *__restrict__ v, int64_t n, int64_t pos)
{
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x;
    if (bh == 0 && t == 0)
        *reinterpret_cast<LocalStateHeader *>(state) = hdr;
    char *rec = state + L.off_rec + bh * L.rec_bytes;
    if (t == 0)
        *reinterpret_cast<int64_t *>(rec) = pos;
    constexpr int CPR = D * (int)sizeof(T) / 16; // 16-byte chunks per row
    const int64_t keep = n < L.R - 1 ? n : L.R - 1;
    for (int64_t e = t; e < keep * CPR; e += 256) {
        const int64_t r = n - keep + e / CPR; // row of the given tokens; its position is pos - n + r
        const int ch = (int)(e % CPR);
        const int64_t slot = (pos - n + r) % L.R;
        reinterpret_cast<u32x4 *>(rec + L.off_k + slot * D * (int64_t)sizeof(T))[ch] =
            reinterpret_cast<const u32x4 *>(k + (bh * n + r) * D)[ch];
        reinterpret_cast<u32x4 *>(rec + L.off_v + slot * D * (int64_t)sizeof(T))[ch] =
            reinterpret_cast<const u32x4 *>(v + (bh * n + r) * D)[ch];
    }
}

// ---- one step ----
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void local_decode_kernel(char *__restrict__ state, LocalStateLayout L,
                                                                LocalStateHeader expect, LocalConsts lc,
                                                                const T *__restrict__ q,
                                                                const T *__restrict__ k_new,
                                                                const T *__restrict__ v_new,
                                                                const T *__restrict__ o_lr, T *__restrict__ out,
                                                                int H)
{
    constexpr int FPL = D / kLanesPerRow;        // features per lane
    constexpr int NDW = FPL * (int)sizeof(T) / 4; // dwords of a lane's key (or value) features
    constexpr int NP = D / 2;
    static_assert(FPL % 2 == 0, "whole feature pairs per lane");

    __shared__ float s_knew[D], s_vnew[D];
    __shared__ float s_m[kGroups], s_l[kGroups];
    __shared__ float s_acc[kGroups][D + 1];

    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % H);
    const int t = threadIdx.x;
    const int grp = t / kLanesPerRow, part = t % kLanesPerRow;
    char *rec = state + L.off_rec + bh * L.rec_bytes; // in bounds: the host checked the buffer size
    const LocalStateHeader hv = *reinterpret_cast<const LocalStateHeader *>(state);
    const int64_t i = *reinterpret_cast<const int64_t *>(rec);
    const int bad = (int)(hv.magic != kLocalStateMagic) | (int)(hv.version != kLocalStateVersion) |
                    (int)(hv.batch != expect.batch) | (int)(hv.H != expect.H) | (int)(hv.d != D) |
                    (int)(hv.dtype != expect.dtype) | (int)(hv.w != expect.w) |
                    (int)(hv.rec_bytes != expect.rec_bytes) | (int)(i < 0);
    T *o_row = out + bh * D;
    if (bad) { // not a state of this shape: flag the output, leave the state alone
        if (t < D) {
            if constexpr (sizeof(T) == 2)
                o_row[t] = (T)0x7fc0u; // bf16 quiet NaN
            else
                o_row[t] = __uint_as_float(0x7fc00000u);
        }
        return;
    }
    const int64_t R = L.R;
    const int64_t nwin = i + 1 < R ? i + 1 : R; // offsets 0 .. nwin - 1
    const int64_t slot0 = i % R;
    if (t < D) {
        s_knew[t] = to_f32<T>(k_new[bh * D + t]);
        s_vnew[t] = to_f32<T>(v_new[bh * D + t]);
    }
    float qf[FPL];
#pragma unroll
    for (int e = 0; e < FPL; ++e)
        qf[e] = to_f32<T>(q[bh * D + part * FPL + e]);
    __syncthreads();

    const char *kring = rec + L.off_k + part * FPL * (int64_t)sizeof(T);
    const char *vring = rec + L.off_v + part * FPL * (int64_t)sizeof(T);
    const char *tab = state + L.off_table + part * (FPL / 2) * (int64_t)sizeof(float2);
    const float scale = 1.4426950408889634f / sqrtf((float)D); // log2(e) / sqrt(d): exp2 domain
    float m = -INFINITY, l = 0.0f, acc[FPL];
#pragma unroll
    for (int e = 0; e < FPL; ++e)
        acc[e] = 0.0f;

    for (int64_t base = 0; base < nwin; base += kGroups * kUnroll) {
        uint32_t kr[kUnroll][NDW], vr[kUnroll][NDW], cr[kUnroll][FPL];
        int64_t orow[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t o = base + u * kGroups + grp;
            orow[u] = o;
            const int64_t oc = o < nwin ? o : 0; // rows past the window read offset 0 (in bounds, unused)
            int64_t slot = slot0 - oc;
            slot += slot < 0 ? R : 0;
            load_dwords<NDW>(kring + slot * D * (int64_t)sizeof(T), kr[u]);
            load_dwords<NDW>(vring + slot * D * (int64_t)sizeof(T), vr[u]);
            load_dwords<FPL>(tab + oc * NP * (int64_t)sizeof(float2), cr[u]);
        }
        float x[kUnroll];
        float mx = m;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool fresh = orow[u] == 0; // the step's own token, not yet in the ring
            float dot = 0.0f;
#pragma unroll
            for (int p = 0; p < FPL / 2; ++p) {
                const float c = __uint_as_float(cr[u][2 * p]), sn = __uint_as_float(cr[u][2 * p + 1]);
                const float k0 = fresh ? s_knew[part * FPL + 2 * p] : feature<T, NDW>(kr[u], 2 * p);
                const float k1 = fresh ? s_knew[part * FPL + 2 * p + 1] : feature<T, NDW>(kr[u], 2 * p + 1);
                // q . R(-o) k with R(-o)(k0, k1) = (k0 c + k1 s, -k0 s + k1 c)
                dot = fmaf(qf[2 * p], fmaf(k0, c, k1 * sn), dot);
                dot = fmaf(qf[2 * p + 1], fmaf(-k0, sn, k1 * c), dot);
            }
#pragma unroll
            for (int msk = 1; msk < kLanesPerRow; msk <<= 1)
                dot += __shfl_xor(dot, msk, kWave);
            x[u] = orow[u] < nwin ? dot * scale : -INFINITY;
            mx = fmaxf(mx, x[u]);
        }
        if (mx > m) { // the group's running maximum grows: rescale what it holds
            const float f = exp2f(m - mx);
            l *= f;
#pragma unroll
            for (int e = 0; e < FPL; ++e)
                acc[e] *= f;
            m = mx;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const bool fresh = orow[u] == 0;
            const float p = orow[u] < nwin ? exp2f(x[u] - m) : 0.0f;
            l += p;
#pragma unroll
            for (int e = 0; e < FPL; ++e) {
                const float vv = fresh ? s_vnew[part * FPL + e] : feature<T, NDW>(vr[u], e);
                acc[e] = fmaf(p, vv, acc[e]);
            }
        }
    }

    // the groups' partial softmaxes meet (a group without rows has m = -inf and weight 0)
#pragma unroll
    for (int e = 0; e < FPL; ++e)
        s_acc[grp][part * FPL + e] = acc[e];
    if (part == 0) {
        s_m[grp] = m;
        s_l[grp] = l;
    }
    __syncthreads();
    if (t < D) {
        float M = s_m[0]; // group 0 holds offset 0, so M is finite
#pragma unroll
        for (int g = 1; g < kGroups; ++g)
            M = fmaxf(M, s_m[g]);
        float z = 0.0f, u = 0.0f;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const float f = exp2f(s_m[g] - M);
            z = fmaf(s_l[g], f, z);
            u = fmaf(s_acc[g][t], f, u);
        }
        u /= z;
        const float y = o_lr ? fmaf(lc.alpha[h], to_f32<T>(o_lr[bh * D + t]), u) : u;
        o_row[t] = from_f32<T>(y);
        reinterpret_cast<T *>(rec + L.off_k)[slot0 * D + t] = k_new[bh * D + t];
        reinterpret_cast<T *>(rec + L.off_v)[slot0 * D + t] = v_new[bh * D + t];
    }
    if (t == 0)
        *reinterpret_cast<int64_t *>(rec) = i + 1;
}

template <typename T, int D>
hipError_t build_t(int32_t bh, const LocalStateLayout &L, const LocalStateHeader &hdr, void *state, const void *k,
                   const void *v, int64_t n, int64_t pos, hipStream_t st)
{
    hipLaunchKernelGGL((local_state_build_kernel<T, D>), dim3((unsigned)bh), dim3(256), 0, st,
                       static_cast<char *>(state), L, hdr, static_cast<const T *>(k), static_cast<const T *>(v), n,
                       pos);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t step_t(int32_t bh, int32_t H, const LocalStateLayout &L, const LocalStateHeader &expect,
                  const LocalConsts &lc, void *state, const void *q, const void *k_new, const void *v_new,
                  const void *o_lr, void *out, hipStream_t st)
{
    hipLaunchKernelGGL((local_decode_kernel<T, D>), dim3((unsigned)bh), dim3(kThreads), 0, st,
                       static_cast<char *>(state), L, expect, lc, static_cast<const T *>(q),
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), static_cast<const T *>(o_lr),
                       static_cast<T *>(out), H);
    return hipGetLastError();
}

} // namespace

hipError_t launch_local_state_build(int32_t bh, int32_t d, int32_t bf16, const LocalStateLayout &L,
                                    const LocalStateHeader &hdr, void *state, const void *k, const void *v,
                                    int64_t n, int64_t pos, hipStream_t st)
{
    const int NP = d / 2;
    const int64_t entries = L.R * NP;
    hipLaunchKernelGGL(local_table_kernel, dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<float2 *>(static_cast<char *>(state) + L.off_table), L.R, NP, d,
                       hdr.rope_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (bf16)
        return d == 64 ? build_t<uint16_t, 64>(bh, L, hdr, state, k, v, n, pos, st)
                       : build_t<uint16_t, 128>(bh, L, hdr, state, k, v, n, pos, st);
    return d == 64 ? build_t<float, 64>(bh, L, hdr, state, k, v, n, pos, st)
                   : build_t<float, 128>(bh, L, hdr, state, k, v, n, pos, st);
}

hipError_t launch_local_decode(int32_t bh, int32_t H, int32_t d, int32_t bf16, const LocalStateLayout &L,
                               const LocalStateHeader &expect, const LocalConsts &lc, void *state, const void *q,
                               const void *k_new, const void *v_new, const void *o_lr, void *out, hipStream_t st)
{
    if (bf16)
        return d == 64 ? step_t<uint16_t, 64>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st)
                       : step_t<uint16_t, 128>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st);
    return d == 64 ? step_t<float, 64>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st)
                   : step_t<float, 128>(bh, H, L, expect, lc, state, q, k_new, v_new, o_lr, out, st);
}

} // namespace fsl
