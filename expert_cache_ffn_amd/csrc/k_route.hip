// Routing kernels: router logits (fp64-accumulated GEMV), wave-level top-k with
// softmax gates, and the stable counting-sort permutation of routed rows.
//
// The router activates k of the E experts per token (FreeToken paper
// explainer, section "MoE opens one door and closes another"); the softmax
// gating and the sort are the standard definitions, with these readings:
//  * logits are exact products summed in fp64 and rounded once to fp32, the
//    precision the top-k decision is taken in;
//  * top-k order is logit descending, ties to the lower expert id; NaN logits
//    rank as -inf;
//  * gates are the softmax over the k selected logits (renorm = 1) or the
//    full softmax probabilities at the selected experts (renorm = 0);
//  * the permutation lists the rows f = t*k + j of expert 0, then 1, ...,
//    each group in ascending f (a stable sort by expert).
#include <climits>

#include "device_common.h"
#include "ecf_internal.h"
#include "wave_route.h"

namespace ecf {

__device__ __forceinline__ double wave_sum_f64(double x)
{
    const auto step = [](double v, uint64_t o) { return v + __longlong_as_double((long long)o); };
    x = step(x, dpp64<kDppXor1>((uint64_t)__double_as_longlong(x)));
    x = step(x, dpp64<kDppXor2>((uint64_t)__double_as_longlong(x)));
    x = step(x, dpp64<kDppHalfMirror>((uint64_t)__double_as_longlong(x)));
    x = step(x, dpp64<kDppMirror>((uint64_t)__double_as_longlong(x)));
    double r[4];
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint64_t b = (uint64_t)__double_as_longlong(x);
        const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 16 * row);
        const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, 16 * row);
        r[row] = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
    return (r[0] + r[1]) + (r[2] + r[3]);
}

// ---------------------------------------------------------------------------------
// Router GEMV.  Block = one expert x TT tokens; its 4 waves interleave over d in
// 16-byte vectors.  grid = (E, ceil(T / TT)).
template <bool BF16, int TT>
__global__ __launch_bounds__(256) void k_router_logits(const void *__restrict__ x,
                                                       const void *__restrict__ wr, int T, int d,
                                                       int E, float *__restrict__ logits)
{
    __shared__ double red[4][TT];
    const int e = blockIdx.x, t0 = blockIdx.y * TT;
    const int nt = min(TT, T - t0);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int V = BF16 ? 8 : 4;
    double acc[TT];
#pragma unroll
    for (int q = 0; q < TT; ++q)
        acc[q] = 0.0;
    for (int c = threadIdx.x * V; c < d; c += 256 * V) {
        float wv[V], xv[V];
        if (BF16) {
            uint4 u = *reinterpret_cast<const uint4 *>((const uint16_t *)wr + (size_t)e * d + c);
            uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wv[2 * i] = bf_lo(p[i]);
                wv[2 * i + 1] = bf_hi(p[i]);
            }
        } else {
            float4 u = *reinterpret_cast<const float4 *>((const float *)wr + (size_t)e * d + c);
            wv[0] = u.x, wv[1] = u.y, wv[2] = u.z, wv[3] = u.w;
        }
#pragma unroll
        for (int q = 0; q < TT; ++q) {
            if (q < nt) {
                if (BF16) {
                    uint4 u = *reinterpret_cast<const uint4 *>((const uint16_t *)x + (size_t)(t0 + q) * d + c);
                    uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xv[2 * i] = bf_lo(p[i]);
                        xv[2 * i + 1] = bf_hi(p[i]);
                    }
                } else {
                    float4 u = *reinterpret_cast<const float4 *>((const float *)x + (size_t)(t0 + q) * d + c);
                    xv[0] = u.x, xv[1] = u.y, xv[2] = u.z, xv[3] = u.w;
                }
#pragma unroll
                for (int i = 0; i < V; ++i)
                    acc[q] = fma((double)xv[i], (double)wv[i], acc[q]);  // product exact in fp64
            }
        }
    }
#pragma unroll
    for (int q = 0; q < TT; ++q) {
        const double v = wave_sum_f64(acc[q]);
        if (lane == 0)
            red[w][q] = v;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int q = threadIdx.x;
        double s = (red[0][q] + red[1][q]) + (red[2][q] + red[3][q]);
        logits[(size_t)(t0 + q) * E + e] = (float)s;
    }
}

template <int MAXS>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E, int k,
                                              int renorm, int32_t *__restrict__ idx,
                                              float *__restrict__ gate)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T)
        return;
    topk_wave<MAXS>(logits + (size_t)t * E, E, k, renorm, threadIdx.x & 63, idx + (size_t)t * k,
                    gate + (size_t)t * k, nullptr);
}

// ---------------------------------------------------------------------------------
// Scans and peer matching.

// Exclusive scan of v over the block (blockDim multiple of 64, <= 1024).
// sh: >= 17 ints of LDS.  *total receives the block sum.
// Inclusive scan over the wave by DPP: row_shr 1, 2, 4, 8 inside each row of 16
// lanes, then lane 15 of rows 0 and 2 into rows 1 and 3 (row_bcast:15), then
// lane 31 into rows 2 and 3 (row_bcast:31).  Lanes a step does not write (no
// source lane, or a row outside its row mask) take `old` = 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += dpp_or0<0x111, 0xF>(x);
    x += dpp_or0<0x112, 0xF>(x);
    x += dpp_or0<0x114, 0xF>(x);
    x += dpp_or0<0x118, 0xF>(x);
    x += dpp_or0<0x142, 0xA>(x);
    x += dpp_or0<0x143, 0xC>(x);
    return x;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_or0_64(uint64_t x)
{
    return ((uint64_t)dpp_or0<CTRL, ROWS>((uint32_t)(x >> 32)) << 32) | dpp_or0<CTRL, ROWS>((uint32_t)x);
}
__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t x)
{
    x += dpp_or0_64<0x111, 0xF>(x);
    x += dpp_or0_64<0x112, 0xF>(x);
    x += dpp_or0_64<0x114, 0xF>(x);
    x += dpp_or0_64<0x118, 0xF>(x);
    x += dpp_or0_64<0x142, 0xA>(x);
    x += dpp_or0_64<0x143, 0xC>(x);
    return x;
}

__device__ int block_excl_scan(int v, int *sh, int *total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int x = (int)wave_incl_scan((uint32_t)v);
    if (lane == 63)
        sh[w] = x;
    __syncthreads();
    if (w == 0) {  // the (at most 16) wave totals, scanned by wave 0
        const int t = lane < nw ? sh[lane] : 0;
        const int inc = (int)wave_incl_scan((uint32_t)t);
        if (lane < nw)
            sh[lane] = inc - t;
        if (lane == 15)
            sh[16] = inc;
    }
    __syncthreads();
    const int res = sh[w] + x - v;
    *total = sh[16];
    __syncthreads();
    return res;
}

// block_excl_scan for 64-bit values (sums of packed bit fields).
__device__ unsigned long long block_excl_scan64(unsigned long long v, unsigned long long *sh,
                                                unsigned long long *total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const unsigned long long x = wave_incl_scan64(v);
    if (lane == 63)
        sh[w] = x;
    __syncthreads();
    if (w == 0) {  // the (at most 16) wave totals, scanned by wave 0
        const unsigned long long t = lane < nw ? sh[lane] : 0ull;
        const unsigned long long inc = wave_incl_scan64(t);
        if (lane < nw)
            sh[lane] = inc - t;
        if (lane == 15)
            sh[16] = inc;
    }
    __syncthreads();
    const unsigned long long res = sh[w] + x - v;
    *total = sh[16];
    __syncthreads();
    return res;
}

// Lanes of the wave whose key equals this lane's key (valid lanes only).
__device__ __forceinline__ uint64_t match_peers(int key, bool valid, int nbits)
{
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

// Rank the rows [beg, end) in order, one 64-row chunk at a time, against the
// running per-expert bases in LDS (base[e] = next free position of expert e).
__device__ __forceinline__ void stable_scatter_wave(const int *__restrict__ keys_lds,
                                                    const int32_t *__restrict__ keys_g, int beg,
                                                    int end, int *base, int nbits, int lane,
                                                    int32_t *__restrict__ perm,
                                                    int32_t *__restrict__ pos)
{
    for (int c0 = beg; c0 < end; c0 += 64) {
        const int f = c0 + lane;
        const bool valid = f < end;
        const int key = valid ? (keys_lds ? keys_lds[f] : keys_g[f]) : 0;
        const uint64_t peers = match_peers(key, valid, nbits);
        if (valid) {
            const int rank = __popcll(peers & lanemask_lt(lane));
            const int b = base[key];
            const int p = b + rank;
            perm[p] = f;
            pos[f] = p;
            if (lane == __ffsll((unsigned long long)peers) - 1)
                base[key] = b + __popcll(peers);
        }
    }
}

__device__ __forceinline__ int key_bits(int E)
{
    int b = 0;
    while ((1 << b) < E)
        ++b;
    return b;
}

// ---------------------------------------------------------------------------------
// Single-block routing for small R (decode): top-k, counts, scan, active list,
// prefill tile list and the stable scatter, in one launch.
template <int MAXS>
__global__ __launch_bounds__(1024) void k_route_small(
    const float *__restrict__ logits, int T, int E, int k, int renorm, int MT,
    int32_t *__restrict__ idx, float *__restrict__ gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
    int32_t *__restrict__ active, int32_t *__restrict__ n_active, int32_t *__restrict__ tiles,
    int32_t *__restrict__ n_tiles)
{
    extern __shared__ int smem[];
    const int R = T * k;
    int *sidx = smem;
    int *hist = smem + R;
    __shared__ unsigned long long sc[17];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int t = wv; t < T; t += 16)
        topk_wave<MAXS>(logits + (size_t)t * E, E, k, renorm, lane, idx + (size_t)t * k,
                        gate + (size_t)t * k, sidx + t * k);
    for (int e = tid; e < E; e += 1024)
        hist[e] = 0;
    __syncthreads();
    for (int f = tid; f < R; f += 1024)
        atomicAdd(&hist[sidx[f]], 1);
    __syncthreads();
    // one scan of three packed fields: rows (bits 0..20), active experts
    // (21..41) and prefill tiles (42..62); each is at most R + E < 2^21
    const int c = tid < E ? hist[tid] : 0;
    const int nte = (c + MT - 1) / MT;
    constexpr unsigned long long M21 = (1ull << 21) - 1;
    unsigned long long tot;
    const unsigned long long run = block_excl_scan64(
        (unsigned long long)c | ((unsigned long long)(c > 0) << 21) | ((unsigned long long)nte << 42), sc, &tot);
    const int off = (int)(run & M21), aoff = (int)((run >> 21) & M21), toff = (int)(run >> 42);
    if (tid < E) {
        counts[tid] = c;
        offsets[tid] = off;
        if (c > 0)
            active[aoff] = tid;
        for (int m = 0; m < nte; ++m) {
            tiles[2 * (toff + m)] = tid;
            tiles[2 * (toff + m) + 1] = m * MT;
        }
        hist[tid] = off;  // scatter base; only this thread read hist[tid] since the last barrier
    }
    if (tid == 0) {
        offsets[E] = (int)(tot & M21);
        *n_active = (int)((tot >> 21) & M21);
        *n_tiles = (int)(tot >> 42);
    }
    __syncthreads();
    if (wv == 0)
        stable_scatter_wave(sidx, nullptr, 0, R, hist, key_bits(E), lane, perm, pos);
}

// ---------------------------------------------------------------------------------
// Multi-block counting sort for large R: per-segment counts, one scan block,
// per-segment stable scatter.  Segment s = rows [s*kSortSeg, (s+1)*kSortSeg).

__global__ __launch_bounds__(256) void k_sort_count(const int32_t *__restrict__ idx, int R, int E,
                                                    int32_t *__restrict__ seg_counts)
{
    extern __shared__ int hist[];
    for (int e = threadIdx.x; e < E; e += 256)
        hist[e] = 0;
    __syncthreads();
    const int beg = blockIdx.x * kSortSeg, end = min(R, beg + kSortSeg);
    for (int f = beg + threadIdx.x; f < end; f += 256)
        atomicAdd(&hist[idx[f]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        seg_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block.  Expert e's segments are split over P = min(16, 1024 / E) threads
// (thread t: expert t % E, part t / E, a contiguous run of segments each), so
// the per-segment loads are spread out and batched instead of walked by one
// thread; the parts' sums meet in LDS, then each part writes its bases.
__global__ __launch_bounds__(1024) void k_sort_scan(
    const int32_t *__restrict__ seg_counts, int S, int E, int MT, int32_t *__restrict__ seg_base,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active, int32_t *__restrict__ tiles, int32_t *__restrict__ n_tiles)
{
    __shared__ int sc[17];
    __shared__ int part[1024];  // part[p * E + e]: rows of expert e in part p's segments
    __shared__ int eoff[1024];  // first sorted row of expert e
    const int P = min(16, max(1, 1024 / E));
    const int t = threadIdx.x, e = t % E, p = t / E;
    const bool on = p < P;
    const int s0 = on ? (int)((int64_t)S * p / P) : 0, s1 = on ? (int)((int64_t)S * (p + 1) / P) : 0;
    int c = 0;
#pragma unroll 8
    for (int s = s0; s < s1; ++s)
        c += seg_counts[(size_t)s * E + e];
    if (on)
        part[t] = c;
    __syncthreads();
    int pre = 0, ce = 0;  // rows of e in parts before p; all rows of e
    if (on)
        for (int q = 0; q < P; ++q) {
            const int v = part[q * E + e];
            pre += q < p ? v : 0;
            ce += v;
        }
    // the expert-level scans run over the part-0 threads, which are threads 0..E-1
    const bool lead = on && p == 0;
    const int cl = lead ? ce : 0;
    int tot, na, ntt;
    const int off = block_excl_scan(cl, sc, &tot);
    const int aoff = block_excl_scan(cl > 0 ? 1 : 0, sc, &na);
    const int nte = (cl + MT - 1) / MT;
    const int toff = block_excl_scan(nte, sc, &ntt);
    if (lead) {
        counts[e] = cl;
        offsets[e] = off;
        eoff[e] = off;
        if (cl > 0)
            active[aoff] = e;
        for (int m = 0; m < nte; ++m) {
            tiles[2 * (toff + m)] = e;
            tiles[2 * (toff + m) + 1] = m * MT;
        }
    }
    if (t == 0) {
        offsets[E] = tot;
        *n_active = na;
        *n_tiles = ntt;
    }
    __syncthreads();
    if (on) {
        int run = eoff[e] + pre;
#pragma unroll 8
        for (int s = s0; s < s1; ++s) {
            const int v = seg_counts[(size_t)s * E + e];
            seg_base[(size_t)s * E + e] = run;
            run += v;
        }
    }
}

// Each of the 4 waves owns a contiguous quarter of the segment; its bases are
// the segment base plus the counts of the quarters before it.
__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t *__restrict__ idx, int R, int E,
                                                      const int32_t *__restrict__ seg_base,
                                                      int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ pos)
{
    extern __shared__ int hw[];  // [4][E]
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int beg = blockIdx.x * kSortSeg, end = min(R, beg + kSortSeg);
    constexpr int Q = kSortSeg / 4;
    const int qb = min(end, beg + w * Q), qe = min(end, beg + (w + 1) * Q);
    for (int i = threadIdx.x; i < 4 * E; i += 256)
        hw[i] = 0;
    __syncthreads();
    for (int f = qb + lane; f < qe; f += 64)
        atomicAdd(&hw[w * E + idx[f]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        int run = seg_base[(size_t)blockIdx.x * E + e];
        for (int q = 0; q < 4; ++q) {
            const int t = hw[q * E + e];
            hw[q * E + e] = run;
            run += t;
        }
    }
    __syncthreads();
    stable_scatter_wave(nullptr, idx, qb, qe, hw + w * E, key_bits(E), lane, perm, pos);
}

// ---------------------------------------------------------------------------------
// Launchers.

int launch_router_logits(const ecf_shape &s, const void *x, const void *wr, int T, float *logits,
                         hipStream_t st)
{
    if (T <= 0)
        return ECF_OK;
    ProfScope p("router_logits", st);
    // Tokens per block: 2 for decode-sized batches (more, shorter blocks: the
    // kernel is latency-bound there; measured against 1, 4, 8 and 16 at 1, 4 and
    // 16 tokens), 8 above 32 tokens, where each block re-reading the expert's
    // router row for only 2 tokens would multiply the cache traffic.
#define ECF_ROUTER(TTV)                                                                            \
    {                                                                                              \
        dim3 grid(s.n_experts, (T + (TTV) - 1) / (TTV));                                           \
        if (s.a_dtype == ECF_BF16)                                                                 \
            hipLaunchKernelGGL((k_router_logits<true, TTV>), grid, dim3(256), 0, st, x, wr, T,     \
                               s.hidden, s.n_experts, logits);                                     \
        else                                                                                       \
            hipLaunchKernelGGL((k_router_logits<false, TTV>), grid, dim3(256), 0, st, x, wr, T,    \
                               s.hidden, s.n_experts, logits);                                     \
    }
    if (T <= 32)
        ECF_ROUTER(2)
    else
        ECF_ROUTER(8)
#undef ECF_ROUTER
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_route(const ecf_shape &s, const float *logits, int T, const RouteOut &o, hipStream_t st)
{
    const int E = s.n_experts, k = s.top_k, R = T * k;
    const int maxs = (E + 63) / 64;
    if (R <= kSmallRouteRows) {
        ProfScope p("route_small", st);
        const size_t sh = sizeof(int) * (size_t)(R + E);
#define ECF_ROUTE_SMALL(MS)                                                                       \
    hipLaunchKernelGGL((k_route_small<MS>), dim3(1), dim3(1024), sh, st, logits, T, E, k,         \
                       s.renorm_topk, prefill_mt(s), o.idx, o.gate, o.counts, o.offsets, o.perm,      \
                       o.pos, o.active, o.n_active, o.tiles, o.n_tiles)
        if (maxs <= 1)
            ECF_ROUTE_SMALL(1);
        else if (maxs <= 2)
            ECF_ROUTE_SMALL(2);
        else if (maxs <= 4)
            ECF_ROUTE_SMALL(4);
        else if (maxs <= 8)
            ECF_ROUTE_SMALL(8);
        else
            ECF_ROUTE_SMALL(16);
#undef ECF_ROUTE_SMALL
        ECF_HIP_CHECK(hipGetLastError());
        return ECF_OK;
    }
    {
        ProfScope p("topk", st);
        dim3 grid((T + 3) / 4);
#define ECF_TOPK(MS)                                                                              \
    hipLaunchKernelGGL((k_topk<MS>), grid, dim3(256), 0, st, logits, T, E, k, s.renorm_topk, o.idx, \
                       o.gate)
        if (maxs <= 1)
            ECF_TOPK(1);
        else if (maxs <= 2)
            ECF_TOPK(2);
        else if (maxs <= 4)
            ECF_TOPK(4);
        else if (maxs <= 8)
            ECF_TOPK(8);
        else
            ECF_TOPK(16);
#undef ECF_TOPK
        ECF_HIP_CHECK(hipGetLastError());
    }
    const int S = (R + kSortSeg - 1) / kSortSeg;
    {
        ProfScope p("sort_count", st);
        hipLaunchKernelGGL(k_sort_count, dim3(S), dim3(256), sizeof(int) * E, st, o.idx, R, E,
                           o.seg_counts);
        ECF_HIP_CHECK(hipGetLastError());
    }
    {
        ProfScope p("sort_scan", st);
        hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(1024), 0, st, o.seg_counts, S, E, prefill_mt(s),
                           o.seg_base, o.counts, o.offsets, o.active, o.n_active, o.tiles,
                           o.n_tiles);
        ECF_HIP_CHECK(hipGetLastError());
    }
    {
        ProfScope p("sort_scatter", st);
        hipLaunchKernelGGL(k_sort_scatter, dim3(S), dim3(256), sizeof(int) * 4 * E, st, o.idx, R, E,
                           o.seg_base, o.perm, o.pos);
        ECF_HIP_CHECK(hipGetLastError());
    }
    return ECF_OK;
}

}  // namespace ecf
