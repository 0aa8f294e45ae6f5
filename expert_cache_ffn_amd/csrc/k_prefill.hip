// Prefill-path expert kernels: grouped GEMMs over the expert-sorted rows on
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16), bf16 or MXFP4 weights.
//
// In prefill thousands of tokens reach nearly every expert of a layer
// (FreeToken paper explainer, section "Wall 1: prefill" -- sparsity vanishes),
// so each expert is a small dense GEMM: its rows are contiguous in the
// counting-sort order and tiled BM = 128 rows at a time (the tile list comes
// from the routing kernels).
//
//   GEMM1: [a | b] = X_perm . [W_gate ; W_up]^T, h = silu(a) * b -> H (bf16)
//          A rows are gathered from x through perm; the gate and up rows of the
//          same intermediate index sit in one tile so SwiGLU runs in registers.
//   GEMM2: Y = H . W_down^T (fp32), combined per token by k_combine.
//
// Tiles go through LDS, double-buffered: global -> registers for tile k+1
// while the MFMAs consume tile k.  bf16 rows of BK = 64 elements (eight 16-B
// chunks) are stored with chunk c of row r at slot c ^ (r & 7), so the 32
// rows an MFMA operand read touches fall in different bank groups.
// MXFP4 weights stay 4-bit in LDS (a quarter of the bf16 bytes) and are
// expanded to bf16 in registers with v_cvt_scalef32_pk_bf16_fp4, which applies
// the E8M0 block scale exactly; the products then run on bf16 MFMA.
#include "device_common.h"
#include "ecf_internal.h"

namespace ecf {

namespace {
constexpr int BM = kPrefillMT;  // 128 rows per tile
constexpr int BK = 64;          // reduction elements per stage
constexpr int MXROW = 3;        // MXFP4 LDS row stride in 16-B units (32 B nibbles + pad)

__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

__device__ __forceinline__ float e8m0_f(uint32_t s)
{
    return __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
}

__device__ __forceinline__ bf16x8_t frag_bf16(const uint4 *tile, int row, int kc)
{
    return __builtin_bit_cast(bf16x8_t, tile[swz(row, kc)]);
}

// 8 MXFP4 elements (one dword of nibbles) -> bf16x8, scaled.
__device__ __forceinline__ bf16x8_t frag_mx(const uint4 *tile, const uint8_t *sc, int row, int kc)
{
    const uint32_t w = reinterpret_cast<const uint32_t *>(tile)[row * MXROW * 4 + kc];
    const float s = e8m0_f(sc[row * 2 + (kc >> 2)]);
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
    bf16x8_t r;
    r[0] = p0[0], r[1] = p0[1], r[2] = p1[0], r[3] = p1[1];
    r[4] = p2[0], r[5] = p2[1], r[6] = p3[0], r[7] = p3[1];
    return r;
}

// One 128-row weight tile of the current stage: bf16 (4 chunks per thread) or
// MXFP4 (1 chunk of nibbles per thread, scale pairs by threads < 128).
template <bool MX>
struct BTile {
    uint4 r[MX ? 1 : 4];
    uint32_t s;
};

// rowp[q]: start of weight row for loader slot q (bf16: rows (tid>>3)+32q; MX: row tid>>1).
template <bool MX>
__device__ __forceinline__ void load_b(BTile<MX> &bt, const char *const *rowp, const uint8_t *srow,
                                       int K, int kt, int tid)
{
    if (MX) {
        bt.r[0] = *reinterpret_cast<const uint4 *>(rowp[0] + (size_t)kt * 32 + (tid & 1) * 16);
        if (tid < 128)
            bt.s = *reinterpret_cast<const uint16_t *>(srow + (size_t)kt * 2);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bt.r[q] = *reinterpret_cast<const uint4 *>(rowp[q] + (size_t)kt * BK * 2 + (tid & 7) * 16);
    }
}

template <bool MX>
__device__ __forceinline__ void store_b(const BTile<MX> &bt, uint4 *tile, uint8_t *sc, int tid)
{
    if (MX) {
        tile[(tid >> 1) * MXROW + (tid & 1)] = bt.r[0];
        if (tid < 128)
            *reinterpret_cast<uint16_t *>(sc + tid * 2) = (uint16_t)bt.s;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            tile[swz((tid >> 3) + 32 * q, tid & 7)] = bt.r[q];
    }
}

__device__ __forceinline__ void load_a(uint4 ra[4], const uint16_t *const *arow, int kt)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        ra[q] = *reinterpret_cast<const uint4 *>(arow[q] + (size_t)kt * BK);
}

__device__ __forceinline__ void store_a(const uint4 ra[4], uint4 *tile, int tid)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        tile[swz((tid >> 3) + 32 * q, tid & 7)] = ra[q];
}

// Per-thread start of weight row `row` of a [rows][K] matrix in the blob section.
template <bool MX>
__device__ __forceinline__ const char *wrow_ptr(const char *sec, int row, int K)
{
    return sec + (size_t)row * (MX ? K / 2 : K * 2);
}
}  // namespace

// GEMM1 + SwiGLU.  grid = (I / 64, max tiles); block = 4 waves in 2 x 2, each
// wave 64 rows x 32 intermediate columns of both gate and up.
template <bool MX>
__global__ __launch_bounds__(256) void k_gemm1_swiglu(
    const uint64_t *__restrict__ ptrs, size_t off_g, size_t off_u, size_t off_sg, size_t off_su,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const uint16_t *__restrict__ x, int d, int I, int k, int E, int R, uint16_t *__restrict__ H)
{
    constexpr int BN = 64;
    __shared__ uint4 As[2][BM * 8];
    __shared__ uint4 Bs[2][2 * BN * (MX ? MXROW : 8)];
    __shared__ uint8_t Sc[2][MX ? 2 * BN * 2 : 1];
    if ((int)blockIdx.y >= *n_tiles)
        return;
    const int e = tiles[2 * blockIdx.y], m0 = tiles[2 * blockIdx.y + 1];
    if ((unsigned)e >= (unsigned)E)  // routing metadata is produced on the device; never index past it
        return;
    const uint64_t blob = ptrs[e];
    const int rb = offsets[e] + m0;
    const int mrows = min(BM, offsets[e + 1] - rb);
    if (!blob || m0 < 0 || rb < 0 || mrows <= 0 || rb + mrows > R)
        return;
    const int i0 = blockIdx.x * BN;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;

    const uint16_t *arow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = min((tid >> 3) + 32 * q, mrows - 1);
        const size_t t = (size_t)(perm[rb + row] / k);
        arow[q] = x + t * d + (tid & 7) * 8;
    }
    const char *bsec_g = (const char *)blob + off_g, *bsec_u = (const char *)blob + off_u;
    const char *brow[4];
    const uint8_t *srow = nullptr;
    if (MX) {
        const int row = tid >> 1;  // 0..127: < 64 gate, else up
        brow[0] = wrow_ptr<true>(row < BN ? bsec_g : bsec_u, i0 + (row & (BN - 1)), d);
        if (tid < 128)
            srow = (const uint8_t *)blob + (tid < BN ? off_sg : off_su) + (size_t)(i0 + (tid & (BN - 1))) * (d / 32);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = (tid >> 3) + 32 * q;
            brow[q] = wrow_ptr<false>(row < BN ? bsec_g : bsec_u, i0 + (row & (BN - 1)), d);
        }
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[a][b][j] = 0.f;

    const int nk = d / BK;
    uint4 ra[4];
    BTile<MX> bt;
    load_a(ra, arow, 0);
    load_b<MX>(bt, brow, srow, d, 0, tid);
    store_a(ra, As[0], tid);
    store_b<MX>(bt, Bs[0], Sc[0], tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_a(ra, arow, kt + 1);
            load_b<MX>(bt, brow, srow, d, kt + 1, tid);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kc = ks * 2 + (l >> 5);
            bf16x8_t af[2], bf[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                af[ms] = frag_bf16(As[cur], wm * 64 + ms * 32 + (l & 31), kc);
#pragma unroll
            for (int gu = 0; gu < 2; ++gu) {
                const int n = gu * BN + wn * 32 + (l & 31);
                bf[gu] = MX ? frag_mx(Bs[cur], Sc[cur], n, kc) : frag_bf16(Bs[cur], n, kc);
            }
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int gu = 0; gu < 2; ++gu)
                    acc[ms][gu] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf[gu], acc[ms][gu], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_a(ra, As[cur ^ 1], tid);
            store_b<MX>(bt, Bs[cur ^ 1], Sc[cur ^ 1], tid);
        }
        __syncthreads();
    }
    // epilogue: lane holds rows (j/4)*8 + (l/32)*4 + j%4 of column l%32
    const int col = i0 + wn * 32 + (l & 31);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = wm * 64 + ms * 32 + (j >> 2) * 8 + (l >> 5) * 4 + (j & 3);
            if (m < mrows)
                H[(size_t)(rb + m) * I + col] = f_to_bf(silu_mul(acc[ms][0][j], acc[ms][1][j]));
        }
}

// GEMM2: Y[r][o] = H[r] . W_down[o].  grid = (d / 128, max tiles); 4 waves in
// 2 x 2, each 64 rows x 64 outputs.
template <bool MX>
__global__ __launch_bounds__(256) void k_gemm2_down(
    const uint64_t *__restrict__ ptrs, size_t off_d, size_t off_sd, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles, const int32_t *__restrict__ offsets,
    const uint16_t *__restrict__ H, int d, int I, int E, int R, float *__restrict__ Y)
{
    constexpr int BN = 128;
    __shared__ uint4 As[2][BM * 8];
    __shared__ uint4 Bs[2][BN * (MX ? MXROW : 8)];
    __shared__ uint8_t Sc[2][MX ? BN * 2 : 1];
    if ((int)blockIdx.y >= *n_tiles)
        return;
    const int e = tiles[2 * blockIdx.y], m0 = tiles[2 * blockIdx.y + 1];
    if ((unsigned)e >= (unsigned)E)  // routing metadata is produced on the device; never index past it
        return;
    const uint64_t blob = ptrs[e];
    const int rb = offsets[e] + m0;
    const int mrows = min(BM, offsets[e + 1] - rb);
    if (!blob || m0 < 0 || rb < 0 || mrows <= 0 || rb + mrows > R)
        return;
    const int o0 = blockIdx.x * BN;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;

    const uint16_t *arow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = min((tid >> 3) + 32 * q, mrows - 1);
        arow[q] = H + (size_t)(rb + row) * I + (tid & 7) * 8;
    }
    const char *bsec = (const char *)blob + off_d;
    const char *brow[4];
    const uint8_t *srow = nullptr;
    if (MX) {
        brow[0] = wrow_ptr<true>(bsec, o0 + (tid >> 1), I);
        if (tid < 128)
            srow = (const uint8_t *)blob + off_sd + (size_t)(o0 + tid) * (I / 32);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            brow[q] = wrow_ptr<false>(bsec, o0 + (tid >> 3) + 32 * q, I);
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[a][b][j] = 0.f;

    const int nk = I / BK;
    uint4 ra[4];
    BTile<MX> bt;
    load_a(ra, arow, 0);
    load_b<MX>(bt, brow, srow, I, 0, tid);
    store_a(ra, As[0], tid);
    store_b<MX>(bt, Bs[0], Sc[0], tid);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            load_a(ra, arow, kt + 1);
            load_b<MX>(bt, brow, srow, I, kt + 1, tid);
        }
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int kc = ks * 2 + (l >> 5);
            bf16x8_t af[2], bf[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
                af[ms] = frag_bf16(As[cur], wm * 64 + ms * 32 + (l & 31), kc);
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const int n = wn * 64 + ns * 32 + (l & 31);
                bf[ns] = MX ? frag_mx(Bs[cur], Sc[cur], n, kc) : frag_bf16(Bs[cur], n, kc);
            }
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
                    acc[ms][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bf[ns], acc[ms][ns], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_a(ra, As[cur ^ 1], tid);
            store_b<MX>(bt, Bs[cur ^ 1], Sc[cur ^ 1], tid);
        }
        __syncthreads();
    }
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int col = o0 + wn * 64 + ns * 32 + (l & 31);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int m = wm * 64 + ms * 32 + (j >> 2) * 8 + (l >> 5) * 4 + (j & 3);
                if (m < mrows)
                    Y[(size_t)(rb + m) * d + col] = acc[ms][ns][j];
            }
        }
}

// ---------------------------------------------------------------------------------

int launch_prefill_gemm1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, uint16_t *H, hipStream_t st)
{
    dim3 grid(s.inter / 64, max_tiles(s, T));
    ProfScope p("prefill_gemm1", st);
    if (s.w_dtype == ECF_MXFP4)
        hipLaunchKernelGGL((k_gemm1_swiglu<true>), grid, dim3(256), 0, st, ex.ptrs, ex.lay.off[0],
                           ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.tiles, o.n_tiles, o.offsets,
                           o.perm, (const uint16_t *)x, s.hidden, s.inter, s.top_k, s.n_experts, T * s.top_k, H);
    else
        hipLaunchKernelGGL((k_gemm1_swiglu<false>), grid, dim3(256), 0, st, ex.ptrs, ex.lay.off[0],
                           ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.tiles, o.n_tiles, o.offsets,
                           o.perm, (const uint16_t *)x, s.hidden, s.inter, s.top_k, s.n_experts, T * s.top_k, H);
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_prefill_gemm2(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const uint16_t *H,
                         int T, float *Y, hipStream_t st)
{
    dim3 grid(s.hidden / 128, max_tiles(s, T));
    ProfScope p("prefill_gemm2", st);
    if (s.w_dtype == ECF_MXFP4)
        hipLaunchKernelGGL((k_gemm2_down<true>), grid, dim3(256), 0, st, ex.ptrs, ex.lay.off[2],
                           ex.lay.off[5], o.tiles, o.n_tiles, o.offsets, H, s.hidden, s.inter, s.n_experts, T * s.top_k, Y);
    else
        hipLaunchKernelGGL((k_gemm2_down<false>), grid, dim3(256), 0, st, ex.ptrs, ex.lay.off[2],
                           ex.lay.off[5], o.tiles, o.n_tiles, o.offsets, H, s.hidden, s.inter, s.n_experts, T * s.top_k, Y);
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
