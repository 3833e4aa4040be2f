// Per-lane arithmetic of the block-union readout (FreeSolo, Sec. 3.3 "Token
// readout", Eq. 9; App. D.2 Eq. 17), shared by the readout kernel and the
// fused routing+readout kernel so that the two give bitwise equal outputs.
//
// Layout: a wave owns 32 queries; the 32 x 32 logits tile of one gathered cell
// (tokens x queries) sits in a 32x32 MFMA accumulator, so lane (col, half)
// holds 16 logits of query col, and the partner lane (half ^ 1) the other 16.
#pragma once

#include "fsl_device.h"

namespace fsl {

// V^T rows keep a 32-token cell or tile in the order 0-3, 8-11, 4-7, 12-15,
// 16-19, 24-27, 20-23, 28-31: then the 8 tokens a lane feeds to one P.V product
// (16 kk + 4 half + 0..3 and 16 kk + 8 + 4 half + 0..3, the order of its
// probabilities in the logits accumulator) are 16 contiguous bytes.
__device__ __forceinline__ int vt_pos(int tok) { return tok ^ (((tok >> 2) ^ (tok >> 3)) & 1) * 12; }

constexpr float kLazy = 16.0f; // the running max moves only when it grows by more than 2^16

// One cell of the online softmax, exp2 domain: p = 2^(l * scale_log2 - m) for
// this lane's 16 logits, with the running max m and sum l of the query.  The
// max moves only when a logit exceeds it by more than kLazy, so p <= 2^kLazy
// and rescaling is rare; the first cell always sets it (o and l are still 0,
// so alpha = 1 there).  A query that did not select the cell takes m = +inf:
// its p are exactly 0 and m, l do not change.  Returns the factor alpha that
// the query's output accumulators must be multiplied by before adding P V.
__device__ __forceinline__ float softmax_cell(const f32x16 &acc, bool mine, float scale_log2, float &m_run,
                                              float &l_run, float (&p)[16])
{
    float amax = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r)
        amax = fmaxf(amax, acc[r]);
    const float tmax = fmaxf(amax, shfl_xor_f(amax, 32)) * scale_log2; // scale > 0: max commutes
    float alpha = 1.0f;
    if (mine && tmax > m_run + kLazy) {
        alpha = m_run == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - tmax);
        m_run = tmax;
    }
    const float m_eff = mine ? m_run : INFINITY;
    float psum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], scale_log2, -m_eff));
        psum += p[r];
    }
    psum += shfl_xor_f(psum, 32);
    l_run = l_run * alpha + psum;
    return alpha;
}

// Eight probabilities as bf16 hi + lo parts (hi = bf16(x), lo = bf16(x - hi),
// nearest-even), the B operands of the two P.V matrix products.
__device__ __forceinline__ void split_bf16x8(const float *x, bf16x8 &hi, bf16x8 &lo)
{
    u32x4 h, l;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t hp = cvt_pk_bf16(x[2 * w], x[2 * w + 1]);
        h[w] = hp;
        l[w] = cvt_pk_bf16(x[2 * w] - __uint_as_float(hp << 16), x[2 * w + 1] - __uint_as_float(hp & 0xffff0000u));
    }
    hi = as_bf16x8(h);
    lo = as_bf16x8(l);
}

// RMSNorm (Eq. 17) of the query's normalised output u = o / l: the factor c
// with y = c * o (before the gain), c = (1 / l) / sqrt(sum(o^2) / l^2 / d + eps).
// The lane holds half of the query's d accumulators, its partner the rest.
// c = 0 for a query with no selected cell (l = 0, o = 0).
template <int DT>
__device__ __forceinline__ float rms_factor(const f32x16 (&o)[DT], float l_run, float eps)
{
    float so = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            so = fmaf(o[dt][r], o[dt][r], so);
    so += shfl_xor_f(so, 32);
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const float ms = so * inv_l * inv_l * (1.0f / (float)(DT * 32));
    return inv_l / sqrtf(ms + eps);
}

} // namespace fsl
