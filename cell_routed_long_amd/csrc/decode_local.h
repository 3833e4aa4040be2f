// One decode step of the local branch (FreeSolo, Sec. 3.2, Eqs. 3-4; the
// window moves one token per step) with the branch combination of Eq. 2, as
// device functions shared by the local decode kernel and the fused attention
// decode kernel.
//
// A step for the token at position i reads the window [max(0, i - w), i]: the
// step's own k_new, v_new (offset o = 0) and the ring's w slots, which hold
// the tokens i - w .. i - 1 (offsets w .. 1; those before position 0 are
// masked).  Logits take the relative form of Eq. 3, q_i . R(-o) k_{i-o} =
// (R(o) q_i) . k_{i-o}, with R(o) turning feature pair m by o theta_m; the ring
// holds raw keys, so no angle grows with the position.
//
// A step has 32 groups of 16 lanes (512 threads).  Sixteen lanes share a row
// (a ring slot) and hold d/16 of its features, so a row is one coalesced read
// per array; a group owns kRows consecutive slots per pass, and a pass of the
// 32 groups covers 32 kRows slots (the whole w = 512 ring for bf16, every load
// of it in flight together).  The loads go by slot, so they do not wait for
// the position; the offsets follow once it arrives.  Along a group's slots the
// offset falls by one per slot, with one jump from 1 to w where the ring wraps:
// the group turns the query once with the (cos, sin) table entry of its first
// offset (built in fp64 with the state), then by -theta_m per slot, and takes
// R(w) q at the wrap.  Every group runs an online softmax over its rows; the
// groups meet in LDS, where 512 / d adjacent lanes finish each feature.  The
// new token then replaces the oldest one, in slot i mod w, after every read of
// the ring.  The groups' results, and so the step's, do not depend on which
// waves run which groups.
#pragma once

#include "fsl_internal.h"

namespace fsl {
namespace {
namespace ldec {

constexpr int kThreads = 512;                    // threads of one step
constexpr int kLanesPerRow = 16;
constexpr int kGroups = kThreads / kLanesPerRow; // 32 groups of 16 lanes

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

// Sum over the 16 lanes of a DPP row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_f<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);  // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x); // row_half_mirror
    x += dpp_f<0x140>(x); // row_mirror
    return x;
}

template <typename T, int D>
struct Shape {
    static constexpr int FPL = D / kLanesPerRow;         // features per lane
    static constexpr int NPL = FPL / 2;                  // feature pairs per lane
    static constexpr int NDW = FPL * (int)sizeof(T) / 4; // dwords of a lane's key (or value) features
    static constexpr int NP = D / 2;
    static constexpr int kRows = 32 / (int)sizeof(T);    // slots per group and pass (16 bf16, 8 fp32)
    static constexpr int kPass = kGroups * kRows;        // slots per pass
    static constexpr int TPF = kThreads / D;             // lanes per feature in the final combination: 4 or 8
    static constexpr int GPT = kGroups / TPF;            // groups each of them combines
    static_assert(FPL % 2 == 0, "whole feature pairs per lane");
};

// The groups' softmax partials (a group without rows has m = -inf and weight 0)
// and the logit of offset 0, the step's own token (exp2 domain).
template <int D>
struct Smem {
    float m[kGroups], l[kGroups];
    float acc[kGroups][D + 1];
    float x0;
};

// What a thread loads at the start of its part of a step: the header, the
// position, its lane's features of q and k_new, the (cos, sin) of theta_m and
// of w theta_m for its feature pairs, and the new key and value of the feature
// te it finishes in the combination.  Nothing here waits for memory.  (The new
// token's value enters only in the combination, through vn_t, so no value row
// stays live across a group's ring loop.)
template <typename T, int D>
struct Entry {
    LocalStateHeader hv;
    int64_t i;
    char *rec;
    const char *tab;
    uint32_t qr[Shape<T, D>::NDW], kr0[Shape<T, D>::NDW];
    uint32_t stp[Shape<T, D>::FPL], cw[Shape<T, D>::FPL];
    T kn_t, vn_t;
};

template <typename T, int D>
__device__ __forceinline__ Entry<T, D> step_entry(char *__restrict__ state, const LocalStateLayout &L,
                                                  const T *__restrict__ q, const T *__restrict__ k_new,
                                                  const T *__restrict__ v_new, int64_t bh, int part, int te)
{
    using S = Shape<T, D>;
    Entry<T, D> e;
    const int64_t w = L.w;
    e.rec = state + L.off_rec + bh * L.rec_bytes; // in bounds: the host checked the buffer size
    e.tab = state + L.off_table + part * S::NPL * (int64_t)sizeof(float2);
    const int64_t lane_off = part * S::FPL * (int64_t)sizeof(T);
    // nothing branches on the header: every address here lies inside the buffer
    // whatever the header holds, and a foreign header only changes what is written
    e.hv = *reinterpret_cast<const LocalStateHeader *>(state);
    e.i = *reinterpret_cast<const int64_t *>(e.rec);
    load_dwords<S::NDW>(reinterpret_cast<const char *>(q + bh * D) + lane_off, e.qr);
    load_dwords<S::NDW>(reinterpret_cast<const char *>(k_new + bh * D) + lane_off, e.kr0);
    load_dwords<S::FPL>(e.tab + (w > 0 ? 1 : 0) * S::NP * (int64_t)sizeof(float2), e.stp); // (cos, sin) of theta_m
    load_dwords<S::FPL>(e.tab + w * S::NP * (int64_t)sizeof(float2), e.cw);                // of w theta_m
    e.kn_t = k_new[bh * D + te];
    e.vn_t = v_new[bh * D + te];
    return e;
}

// Group grp's rows (part: this lane's place in the group), written to sm.
template <typename T, int D>
__device__ __forceinline__ void step_group(const Entry<T, D> &e, const LocalStateLayout &L, int grp, int part,
                                           Smem<D> &sm)
{
    using S = Shape<T, D>;
    constexpr int FPL = S::FPL, NPL = S::NPL, NDW = S::NDW, NP = S::NP, kRows = S::kRows, kPass = S::kPass;
    const int64_t w = L.w;
    const int64_t lane_off = part * FPL * (int64_t)sizeof(T);
    const char *kring = e.rec + L.off_k + lane_off;
    const char *vring = e.rec + L.off_v + lane_off;
    // log2(e) / sqrt(d): the softmax works in the exp2 domain with the hardware exp2 (one
    // instruction; results below 2^-126 flush to 0, far below any weight that counts next
    // to the largest, which is 1)
    const float scale = 1.4426950408889634f / sqrtf((float)D);

    // slot of token i - 1 (offset 1); slots of offsets above min(i, w) hold no token yet.
    // Slots and offsets fit in 32 bits: w <= 65535.
    const int wi = (int)w;
    const int64_t i_nn = e.i > 0 ? e.i : 0;
    const int last = (int)((i_nn + w - 1) % L.slots);
    const int n_valid = (int)(i_nn < w ? i_nn : w);
    // offset of slot s: last - s + 1, or that plus w past the wrap (always in 1 .. w)
    auto offset_of = [&](int sl) { return sl <= last ? last - sl + 1 : last - sl + 1 + wi; };
    constexpr int kHalf = kRows / 2; // rows per softmax update

    // A group adds up to w / 32 rows one after another; a running fp32 sum of n terms
    // can lose about n * 2^-24 of its value, 1e-4 at the largest window.  Each run of
    // kRunPasses passes is therefore summed on its own and then added into a second
    // total (acc_t, l_t): the loss stays near (rows per run + runs) * 2^-24.  Windows
    // of up to kRunPasses passes never close a run.
    constexpr int kRunPasses = 8;
    float m = -INFINITY, l = 0.0f, acc[FPL], l_t = 0.0f, acc_t[FPL];
#pragma unroll
    for (int x = 0; x < FPL; ++x) {
        acc[x] = 0.0f;
        acc_t[x] = 0.0f;
    }

    for (int base = 0; base < wi; base += kPass) {
        // the pass's rows and the angle of the group's first offset are requested
        // before anything waits for memory
        const int s0 = base + grp * kRows; // the group's first slot in this pass
        uint32_t kr[kRows][NDW], vr[kRows][NDW], c0[FPL];
        // (loads complete in issue order: the angle goes between the two halves, so
        // the first half's rows can be used while the second half arrives)
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
            if (u == kRows / 2)
                load_dwords<FPL>(e.tab + (int64_t)offset_of(s0 < wi ? s0 : 0) * NP * (int64_t)sizeof(float2), c0);
            const int sc = s0 + u < wi ? s0 + u : 0; // slots past the ring read slot 0 (in bounds, unused)
            load_dwords<NDW>(kring + (int64_t)sc * D * (int64_t)sizeof(T), kr[u]);
            load_dwords<NDW>(vring + (int64_t)sc * D * (int64_t)sizeof(T), vr[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // q and the angle w theta_m are loop-invariant; these empty asm statements
        // keep their use (and the wait for them) here, behind the pass's loads,
        // instead of hoisted in front of the loop
        uint32_t qv[NDW], cwv[FPL];
#pragma unroll
        for (int x = 0; x < NDW; ++x) {
            qv[x] = e.qr[x];
            asm volatile("" : "+v"(qv[x]));
        }
#pragma unroll
        for (int x = 0; x < FPL; ++x) {
            cwv[x] = e.cw[x];
            asm volatile("" : "+v"(cwv[x]));
        }

        // R(o0) q for the first offset; R(w) q, taken where the slots wrap from offset 1 to w
        float qx[NPL], qy[NPL], wx[NPL], wy[NPL];
#pragma unroll
        for (int p = 0; p < NPL; ++p) {
            const float q0 = feature<T, NDW>(qv, 2 * p), q1 = feature<T, NDW>(qv, 2 * p + 1);
            const float c = __uint_as_float(c0[2 * p]), sn = __uint_as_float(c0[2 * p + 1]);
            qx[p] = fmaf(q0, c, -q1 * sn);
            qy[p] = fmaf(q0, sn, q1 * c);
            const float cwc = __uint_as_float(cwv[2 * p]), cws = __uint_as_float(cwv[2 * p + 1]);
            wx[p] = fmaf(q0, cwc, -q1 * cws);
            wy[p] = fmaf(q0, cws, q1 * cwc);
        }
#pragma unroll
        for (int hh = 0; hh < kRows; hh += kHalf) {
            float x[kHalf];
            float mx = m;
#pragma unroll
            for (int uu = 0; uu < kHalf; ++uu) {
                const int u = hh + uu;
                const int s = s0 + u;
                if (u > 0) { // offset of slot s: one less than slot s - 1's, or w at the wrap
                    const bool wrap = s == last + 1;
#pragma unroll
                    for (int p = 0; p < NPL; ++p) {
                        const float c = __uint_as_float(e.stp[2 * p]), sn = __uint_as_float(e.stp[2 * p + 1]);
                        const float nx = fmaf(qx[p], c, qy[p] * sn); // R(-1)
                        const float ny = fmaf(-qx[p], sn, qy[p] * c);
                        qx[p] = wrap ? wx[p] : nx;
                        qy[p] = wrap ? wy[p] : ny;
                    }
                }
                float dot = 0.0f;
#pragma unroll
                for (int p = 0; p < NPL; ++p) {
                    dot = fmaf(qx[p], feature<T, NDW>(kr[u], 2 * p), dot);
                    dot = fmaf(qy[p], feature<T, NDW>(kr[u], 2 * p + 1), dot);
                }
                dot = row16_sum(dot);
                x[uu] = (s < wi && offset_of(s) <= n_valid) ? dot * scale : -INFINITY;
                mx = fmaxf(mx, x[uu]);
            }
            if (mx > m) { // the group's running maximum grows: rescale what it holds
                const float f = __builtin_amdgcn_exp2f(m - mx);
                l *= f;
                l_t *= f;
#pragma unroll
                for (int y = 0; y < FPL; ++y) {
                    acc[y] *= f;
                    acc_t[y] *= f;
                }
                m = mx;
            }
#pragma unroll
            for (int uu = 0; uu < kHalf; ++uu) {
                const float p = x[uu] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x[uu] - m);
                l += p;
#pragma unroll
                for (int y = 0; y < FPL; ++y)
                    acc[y] = fmaf(p, feature<T, NDW>(vr[hh + uu], y), acc[y]);
            }
        }
        if ((base / kPass) % kRunPasses == kRunPasses - 1) { // close the run
#pragma unroll
            for (int y = 0; y < FPL; ++y) {
                acc_t[y] += acc[y];
                acc[y] = 0.0f;
            }
            l_t += l;
            l = 0.0f;
        }
    }
#pragma unroll
    for (int y = 0; y < FPL; ++y)
        acc[y] += acc_t[y];
    l += l_t;

    // offset 0, the step's own token: group 0 leaves its logit for the combination
    if (grp == 0) {
        float dot = 0.0f;
#pragma unroll
        for (int y = 0; y < FPL; ++y)
            dot = fmaf(feature<T, NDW>(e.qr, y), feature<T, NDW>(e.kr0, y), dot);
        dot = row16_sum(dot);
        if (part == 0)
            sm.x0 = dot * scale;
    }

#pragma unroll
    for (int y = 0; y < FPL; ++y)
        sm.acc[grp][part * FPL + y] = acc[y];
    if (part == 0) {
        sm.m[grp] = m;
        sm.l[grp] = l;
    }
}

// After every group's partials are in sm: thread c of the step's 512 (TPF
// adjacent lanes per feature te = c / TPF, each combining GPT groups, then
// added up by DPP) finishes feature te, the step's own token joining as one
// more term (logit sm.x0, value v_new[te]): out = o_sr + alpha * olr when
// combine is set, else o_sr; then the new token enters the ring and the
// position advances.  A header that does not match `expect` gives NaN and leaves the
// record alone.
template <typename T, int D>
__device__ __forceinline__ void step_finish(const Entry<T, D> &e, const LocalStateLayout &L,
                                            const LocalStateHeader &expect, const Smem<D> &sm, int c, bool combine,
                                            float alpha, float olr, T *__restrict__ out, int64_t bh)
{
    using S = Shape<T, D>;
    constexpr int TPF = S::TPF, GPT = S::GPT;
    const int te = c / TPF, sub = c % TPF;
    const float x0 = sm.x0;
    float M = x0; // offset 0 is always in the window, so M is finite
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
        M = fmaxf(M, sm.m[g]);
    float z = 0.0f, u = 0.0f;
#pragma unroll
    for (int gg = 0; gg < GPT; ++gg) {
        const int g = sub * GPT + gg;
        const float fw = __builtin_amdgcn_exp2f(sm.m[g] - M);
        z = fmaf(sm.l[g], fw, z);
        u = fmaf(sm.acc[g][te], fw, u);
    }
    z += dpp_f<0xB1>(z); // quad_perm [1,0,3,2]
    u += dpp_f<0xB1>(u);
    z += dpp_f<0x4E>(z); // quad_perm [2,3,0,1]
    u += dpp_f<0x4E>(u);
    if constexpr (TPF == 8) {
        z += dpp_f<0x141>(z); // row_half_mirror: the two quads of each 8-lane half
        u += dpp_f<0x141>(u);
    }
    const float p0 = __builtin_amdgcn_exp2f(x0 - M);
    z += p0;
    u = fmaf(p0, to_f32<T>(e.vn_t), u);

    const LocalStateHeader &hv = e.hv;
    const int64_t w = L.w, i = e.i;
    const bool bad = hv.magic != kLocalStateMagic || hv.version != kLocalStateVersion || hv.batch != expect.batch ||
                     hv.H != expect.H || hv.d != D || hv.dtype != expect.dtype || hv.w != expect.w ||
                     hv.rec_bytes != expect.rec_bytes || i < 0;
    T *o_row = out + bh * D;
    if (sub == 0) {
        u /= z;
        const float y = combine ? fmaf(alpha, olr, u) : u;
        if (bad) { // not a state of this shape: flag the output, leave the state alone
            if constexpr (sizeof(T) == 2)
                o_row[te] = (T)0x7fc0u; // bf16 quiet NaN
            else
                o_row[te] = __uint_as_float(0x7fc00000u);
        } else {
            o_row[te] = from_f32<T>(y);
            if (w > 0) { // the new token replaces token i - w, read above for the last time
                const int64_t slot = i % w;
                reinterpret_cast<T *>(e.rec + L.off_k)[slot * D + te] = e.kn_t;
                reinterpret_cast<T *>(e.rec + L.off_v)[slot * D + te] = e.vn_t;
            }
        }
    }
    if (c == 0 && !bad)
        *reinterpret_cast<int64_t *>(e.rec) = i + 1;
}

} // namespace ldec
} // namespace
} // namespace fsl
