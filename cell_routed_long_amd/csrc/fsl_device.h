// Device helpers shared by the gfx950 kernels of the long-range branch.
//
// MFMA conventions used throughout (CDNA3/CDNA4 32x32 tiles, wave64):
//   v_mfma_f32_32x32x16_bf16 : A[32 x 16], B[16 x 32] -> C[32 x 32] fp32
//   v_mfma_f32_32x32x2_f32   : A[32 x 2],  B[2 x 32]  -> C[32 x 32] fp32
// Lane l supplies row (l % 32) of A and column (l % 32) of B; its k values are
// the contiguous group (l / 32) of the instruction's k range.  Accumulator
// register r of lane l holds C[8 (r / 4) + 4 (l / 32) + (r % 4)][l % 32].
// The kernels put the query index on the C column, so each lane owns one
// query and 16 of the 32 rows (cells or tokens); its partner lane l ^ 32 owns
// the other 16 rows of the same query.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsl {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (within the 32-row tile) held by accumulator register r of a lane in half `half`.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// (value desc, id asc): does (v1, i1) rank before (v2, i2)?
__device__ __forceinline__ bool ranks_before(float v1, int i1, float v2, int i2)
{
    return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Insert (v, id) into the sorted list tv/ti of the first K (<= KMAX) entries.
// Every index is a compile-time constant after unrolling, so the list stays in
// registers for any run-time K.
template <int KMAX>
__device__ __forceinline__ void topk_insert(float (&tv)[KMAX], int (&ti)[KMAX], int K, float v, int id)
{
    float thr_v = tv[0];
    int thr_i = ti[0];
#pragma unroll
    for (int j = 1; j < KMAX; ++j)
        if (j == K - 1) {
            thr_v = tv[j];
            thr_i = ti[j];
        }
    if (!ranks_before(v, id, thr_v, thr_i))
        return;
#pragma unroll
    for (int j = KMAX - 1; j >= 0; --j) {
        if (j >= K)
            continue;
        const bool above_prev = (j > 0) && ranks_before(v, id, tv[j > 0 ? j - 1 : 0], ti[j > 0 ? j - 1 : 0]);
        if (above_prev) {
            tv[j] = tv[j - 1];
            ti[j] = ti[j - 1];
        } else if (ranks_before(v, id, tv[j], ti[j])) {
            tv[j] = v;
            ti[j] = id;
        }
    }
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int x, int m) { return __shfl_xor(x, m, kWave); }
__device__ __forceinline__ double shfl_xor_d(double x, int m) { return __shfl_xor(x, m, kWave); }

// ---- wave-wide reductions on the DPP network (no LDS round trip) ----------
// Call with all 64 lanes active.  Within each row of 16 lanes the butterfly
// pairs lanes i^1, i^2 (quad permutes), then mirrors within 8 and 16 lanes;
// the four row results are combined through v_readlane, so every lane gets the
// same value in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ int readlane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ double readlane_d(double x, int l)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ float wave_sum_f(float x)
{
    x += dpp_f<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);  // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x); // row_half_mirror
    x += dpp_f<0x140>(x); // row_mirror
    return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}
__device__ __forceinline__ float wave_max_f(float x)
{
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x)
{
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, true));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, true));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xf, 0xf, true));
    x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xf, 0xf, true));
    const uint32_t a0 = (uint32_t)readlane_i((int)x, 0), a1 = (uint32_t)readlane_i((int)x, 16);
    const uint32_t a2 = (uint32_t)readlane_i((int)x, 32), a3 = (uint32_t)readlane_i((int)x, 48);
    return min(min(a0, a1), min(a2, a3));
}

// ---- XCD-aware block order ---------------------------------------------------
// The dispatcher deals workgroups round-robin over the 8 XCDs (each with its own
// L2).  Renumbering the linear workgroup id so that XCD x receives the x-th
// contiguous run of logical blocks keeps the blocks of one head (which share
// its mean keys and its most-selected cells) on one L2.
constexpr int kXcds = 8;
// 32-bit arithmetic: the host keeps every grid below 2^24 workgroups.
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t w, uint32_t total)
{
    const uint32_t per = (total + kXcds - 1) / kXcds; // blocks on the fuller XCDs
    const uint32_t full = total - (per - 1) * kXcds;  // XCDs that receive `per` blocks
    const uint32_t xcd = w % kXcds, idx = w / kXcds;
    return xcd < full ? xcd * per + idx : full * per + (xcd - full) * (per - 1) + idx;
}

// Round x0, x1 to bf16 (nearest even, hardware conversion) and pack them.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float x0, float x1)
{
    const bf16x2 v = {(__bf16)x0, (__bf16)x1};
    return __builtin_bit_cast(uint32_t, v);
}

// The ranking (score desc, id asc) as one order-preserving 64-bit key: the
// score's bits made monotone above 0x7fffffff - id.  A larger key ranks
// first; 0 marks an empty entry (every real key is larger).
__device__ __forceinline__ uint64_t rank_key(float score, uint32_t low)
{
    uint32_t u = __float_as_uint(score + 0.0f); // -0 -> +0: equal scores must tie
    u ^= (uint32_t)((int32_t)u >> 31) | 0x80000000u;
    return ((uint64_t)u << 32) | low;
}

// TopP's order (norm desc, id asc) as one 64-bit key: the fp32 norm's bits made
// monotone above 0x7fffffff - cell.  For norms (never -0 or NaN) it is exactly
// that order; a larger key ranks first and every key is nonzero.
__device__ __forceinline__ uint64_t norm_key(float a, int32_t cell)
{
    uint32_t u = __float_as_uint(a);
    u = (u >> 31) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - cell);
}

// Insert key into the descending list kl of KT keys (a select network: a key
// below the last entry moves nothing).
template <int KT>
__device__ __forceinline__ void insert_key(uint64_t (&kl)[KT], uint64_t key)
{
#pragma unroll
    for (int j = KT - 1; j > 0; --j)
        kl[j] = key > kl[j - 1] ? kl[j - 1] : (key > kl[j] ? key : kl[j]);
    kl[0] = key > kl[0] ? key : kl[0];
}


// Enter one scored tile's NK keys of this lane into its descending top-KT list.
// On the first tile the list is empty and its first KT keys go in without a
// test.  The rest are first tested as a group against the K-th best (on the
// high words, which can only let too many through): the retained cells come
// in priority order, so after the first tile a key seldom enters, and a wave
// skips the select network unless one of its lanes keeps one of these keys.
// The keys are consumed.
template <int KT, int NK = 16>
__device__ __forceinline__ void take_tile_keys(uint64_t (&kl)[KT], uint64_t (&key)[NK], bool first)
{
    if (first) {
#pragma unroll
        for (int r = 0; r < KT && r < NK; ++r) {
            insert_key<KT>(kl, key[r]);
            key[r] = 0; // now in the list: must not enter twice
        }
    }
    const uint32_t kth = (uint32_t)(kl[KT - 1] >> 32);
    bool any = false;
#pragma unroll
    for (int r = 0; r < NK; ++r)
        any |= (uint32_t)(key[r] >> 32) >= kth;
    if (__ballot(any) == 0ull)
        return;
#pragma unroll
    for (int r = 0; r < NK; ++r)
        if (__ballot(key[r] > kl[KT - 1]))
            insert_key<KT>(kl, key[r]);
}

// ---- coalesced tile transfers through LDS (bf16, 128 rows) -------------------
// A workgroup's 128 query rows are one contiguous span of global memory, while
// the matrix-core layouts give each lane one row.  Moving a tile through LDS
// with 16-byte accesses by consecutive threads makes every wave instruction
// touch 4 whole rows instead of 32 partial ones.  Rows at or past `rows` are
// zero-filled on load and skipped on store.  stride: LDS row pitch in elements.
template <int D, int NT, int ROWS = 128>
__device__ __forceinline__ void tile_load_bf16(uint16_t *lds, int stride, const uint16_t *__restrict__ g, int rows)
{
    constexpr int CPR = D / 8; // 16-byte chunks per row
    for (int c = threadIdx.x; c < ROWS * CPR; c += NT) {
        const int r = c / CPR, c8 = (c % CPR) * 8;
        const u32x4 w = r < rows ? *reinterpret_cast<const u32x4 *>(g + (int64_t)r * D + c8) : u32x4{0, 0, 0, 0};
        *reinterpret_cast<u32x4 *>(lds + r * stride + c8) = w;
    }
}
template <int D, int NT, int ROWS = 128>
__device__ __forceinline__ void tile_store_bf16(uint16_t *__restrict__ g, const uint16_t *lds, int stride, int rows)
{
    constexpr int CPR = D / 8;
    for (int c = threadIdx.x; c < ROWS * CPR; c += NT) {
        const int r = c / CPR, c8 = (c % CPR) * 8;
        if (r < rows)
            *reinterpret_cast<u32x4 *>(g + (int64_t)r * D + c8) = *reinterpret_cast<const u32x4 *>(lds + r * stride + c8);
    }
}

// Per-head routing constants, passed by value with every launch.
struct HeadConsts {
    float inv_two_sigma[128]; // 1 / (2 sigma_h)
    float lambda[128];        // lambda_h
};

} // namespace fsl

namespace fsl {

// ---- streaming decode state (one flat caller-owned buffer) ----------------
// Layout: a StateHeader padded to kStateHeaderBytes, then one record per
// (sequence, head), each rec_bytes long.  A record holds n_slots cell slots
// (P + W retained + B/s cells of the block being filled); a slot carries the
// cell's raw keys and values, its fp32 mean key and norm, its absolute cell id
// (-1 = free), whether the cell is in TopP, and its position in the retained
// set A listed in ascending cell-id order (-1 = not in A).
constexpr uint32_t kStateMagic = 0x31534C46u; // "FLS1"
constexpr uint32_t kStateVersion = 2;
constexpr int64_t kStateHeaderBytes = 256;
constexpr int32_t kFlagTop = 1; // the slot's cell belongs to TopP of the current prefix
constexpr int kMaxSlots = 128;  // P + W + B/s supported by the decode kernels

struct StateHeader {
    uint32_t magic, version;
    int32_t batch, H, d, dtype, s, B, P, W, n_slots, pad;
    int64_t rec_bytes;
};

constexpr int kStateHints = 4; // one per wave of the decode step kernel

struct StateMeta {
    int64_t pos;               // next position to be processed
    int32_t n_ret;             // |A| of the current block
    int32_t cur_slot;          // slot of the cell receiving tokens, -1 if none yet
    int32_t hint[kStateHints]; // per wave of the step kernel: the slot it read first at the previous step
                               // (-1: none); only a prefetch hint, results never depend on it
};

struct StateLayout {
    int32_t S;         // slots per record
    int32_t pad;
    int64_t rec_bytes; // bytes per (sequence, head) record
    int64_t off_ridx, off_cell, off_flags, off_a, off_kbar, off_k, off_v; // offsets inside a record
};


// ---- streaming state of the local branch (one flat caller-owned buffer) ---
// Layout: a LocalStateHeader padded to kLocalStateHeaderBytes; the rotation
// table, (w + 1) x d/2 float2 (cos, sin) of o * theta_m for offsets o = 0 .. w,
// shared by every record; then one record per (sequence, head), rec_bytes long:
// the next position (int64, padded to 256 bytes), then a ring of the last w raw
// keys and one of the last w raw values (token p in slot p mod w; one unused
// slot when w = 0), each slots x d of the input dtype.
constexpr uint32_t kLocalStateMagic = 0x314C4C46u; // "FLL1"
constexpr uint32_t kLocalStateVersion = 2;
constexpr int64_t kLocalStateHeaderBytes = 256;

struct LocalStateHeader {
    uint32_t magic, version;
    int32_t batch, H, d, dtype;
    int64_t w, rec_bytes;
    float rope_base;
    int32_t pad;
};

struct LocalStateLayout {
    int64_t w;         // look-back radius: the table has w + 1 rows
    int64_t slots;     // ring slots, max(w, 1)
    int64_t off_table; // from the start of the buffer
    int64_t off_rec;   // first record, from the start of the buffer
    int64_t rec_bytes; // bytes per (sequence, head) record
    int64_t off_k, off_v; // inside a record
};

} // namespace fsl
