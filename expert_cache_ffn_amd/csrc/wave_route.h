// Wave-level routing helpers shared by the routing kernels and the one-token
// decode GEMV that derives its own routing: DPP reductions and the top-k of one
// token's logits by one wave (order: logit descending, ties to the lower expert
// id, NaN as -inf; gates: softmax over the selected logits, or the full softmax
// at the selected experts).
#pragma once

#include <climits>

#include "device_common.h"

namespace ecf {

// ---------------------------------------------------------------------------------
// Wave-wide reductions without LDS round trips: four DPP steps inside each row of
// 16 lanes (xor 1, xor 2, mirror within 8, mirror within 16: afterwards every lane
// of a row holds the same row result, each pair having combined the same two
// operands), then the four row results read into scalar registers and combined in
// row order.  The result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t x)
{
    return ((uint64_t)dpp32<CTRL>((uint32_t)(x >> 32)) << 32) | dpp32<CTRL>((uint32_t)x);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, dpp32<kDppXor1>(x));
    x = max(x, dpp32<kDppXor2>(x));
    x = max(x, dpp32<kDppHalfMirror>(x));
    x = max(x, dpp32<kDppMirror>(x));
    const uint32_t r0 = __builtin_amdgcn_readlane((int)x, 0), r1 = __builtin_amdgcn_readlane((int)x, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)x, 32), r3 = __builtin_amdgcn_readlane((int)x, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ float wave_sum_f32(float x)
{
    x += __uint_as_float(dpp32<kDppXor1>(__float_as_uint(x)));
    x += __uint_as_float(dpp32<kDppXor2>(__float_as_uint(x)));
    x += __uint_as_float(dpp32<kDppHalfMirror>(__float_as_uint(x)));
    x += __uint_as_float(dpp32<kDppMirror>(__float_as_uint(x)));
    const float r0 = __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(x), 0));
    const float r1 = __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(x), 16));
    const float r2 = __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(x), 32));
    const float r3 = __uint_as_float(__builtin_amdgcn_readlane((int)__float_as_uint(x), 48));
    return (r0 + r1) + (r2 + r3);
}

// Selection key of (logit v, expert e): the fp32 bits mapped to an unsigned
// order-preserving code (sign folded), then the complement of e, so a larger
// key is a larger logit, or an equal logit with a lower expert id.  -0 counts as
// +0 (the two compare equal), NaN as -inf.  Key 0 = not selectable.
__device__ __forceinline__ uint64_t sel_key(float v, int e)
{
    if (v != v)
        v = -INFINITY;
    uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ float key_value(uint64_t key)
{
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// ---------------------------------------------------------------------------------
// Top-k of one token's logits by one wave.  MAXS = logits held per lane.  Each of
// the k rounds takes the wave maximum of the lanes' best remaining keys; the
// winner is wave-uniform and its owner lane retires it.  The maximum is taken
// on the 32-bit logit code first; when one lane holds that code (equal logits
// in several lanes are rare) its key is the winner, otherwise the largest low
// word (complemented expert id) among those lanes decides.
template <int MAXS>
__device__ __forceinline__ void topk_wave(const float *__restrict__ lg, int E, int k, int renorm,
                                          int lane, int32_t *idx_out, float *gate_out, int *sidx)
{
    uint64_t key[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
        const int e = lane + 64 * s;
        key[s] = e < E ? sel_key(lg[e], e) : 0ull;
    }
    float my_v = 0.f, m0 = 0.f, rsum = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t b = 0;
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
            b = umax64(b, key[s]);
        const uint32_t bh = (uint32_t)(b >> 32), bl = (uint32_t)b;
        const uint32_t mh = wave_max_u32(bh);
        const uint64_t tied = __ballot(bh == mh);
        const uint32_t ml = __popcll(tied) == 1 ? (uint32_t)__builtin_amdgcn_readlane((int)bl, __ffsll((long long)tied) - 1)
                                                 : wave_max_u32(bh == mh ? bl : 0u);
        const uint64_t w = ((uint64_t)mh << 32) | ml;
        const int we = (int)~(uint32_t)w;
        const float wv = key_value(w);
        if ((we & 63) == lane) {
#pragma unroll
            for (int s = 0; s < MAXS; ++s)
                if (s == (we >> 6))
                    key[s] = 0ull;
        }
        if (j == 0)
            m0 = wv;
        rsum += expf(wv - m0);  // the selected experts' softmax terms, j ascending
        if (lane == j) {
            my_v = wv;
            my_e = we;
        }
    }
    const float ex = lane < k ? expf(my_v - m0) : 0.f;
    float denom;
    if (renorm) {
        denom = rsum;
    } else {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < MAXS; ++q) {
            const int e = lane + 64 * q;
            if (e < E) {
                float v = lg[e];
                if (v != v)
                    v = -INFINITY;
                s += expf(v - m0);
            }
        }
        denom = wave_sum_f32(s);
    }
    if (lane < k) {
        idx_out[lane] = my_e;
        gate_out[lane] = ex / denom;
        if (sidx)
            sidx[lane] = my_e;
    }
}

}  // namespace ecf
