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
//          A rows are gathered from x through perm; one block owns 128
//          intermediate columns of both gate and up, so SwiGLU runs in
//          registers on matching accumulator fragments.
//   GEMM2: Y = H . W_down^T (fp32), combined per token by k_combine.
//
// Block = 4 waves (2 x 2), tile 128 rows x 256 weight rows, BK = 64; each wave
// owns 64 rows x 128 weight rows (2 x 4 MFMA 32x32 fragments, accumulators in
// AGPRs).  Software pipeline of depth 2 through registers: the global loads
// of k-tile kt+2 are issued before the MFMAs of k-tile kt, and stored to the
// free LDS buffer after them, so two k-tiles of MFMA work cover each load's
// latency.  (Direct global->LDS loads were measured against: the compiler
// cannot tell which in-flight LDS DMA a later LDS read depends on and drains
// them all, which serialises the pipeline.)
//
// bf16 rows of 64 elements (eight 16-B chunks) sit in LDS with chunk c of row r
// at slot c ^ (r & 7), so the 32 rows one MFMA operand read touches spread over
// the banks.  MXFP4 weights stay 4-bit in LDS (a quarter of the bf16 bytes) and
// are expanded in registers by v_cvt_scalef32_pk_bf16_fp4, which applies the
// E8M0 block scale exactly; products run on bf16 MFMA.
//
// Blocks are issued round-robin over the 8 XCDs (block b runs on XCD b % 8),
// each with its own L2.  The 1-D block index is remapped so each XCD walks a
// contiguous range of (tile, N-tile) work items, N-tile fastest: the blocks
// sharing one expert tile's A rows run on the same XCD at about the same time.
#include "device_common.h"
#include "ecf_internal.h"

namespace ecf {

namespace {
constexpr int BM = kPrefillMT;  // 128 rows per tile
constexpr int BN = 256;         // weight rows per block
constexpr int BK = 64;          // reduction elements per stage

__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// MXFP4 LDS tile: row = 32 bytes (two 16-B halves), halves swapped on odd
// groups of 8 rows to spread the banks.
__device__ __forceinline__ int mx_slot(int row, int half) { return row * 2 + (half ^ ((row >> 3) & 1)); }

__device__ __forceinline__ float e8m0_f(uint32_t s)
{
    return __uint_as_float(s == 0 ? 0x00400000u : (s << 23));
}

// 16-byte load through a global-address-space pointer (the blob addresses come
// from a device table, so they would otherwise be generic/flat pointers).
typedef const __attribute__((address_space(1))) u32x4_t *gptr16;
typedef const __attribute__((address_space(1))) uint16_t *gptr2;
__device__ __forceinline__ u32x4_t ldg16(const void *p) { return *(gptr16)(uintptr_t)p; }
__device__ __forceinline__ uint32_t ldg2(const void *p) { return *(gptr2)(uintptr_t)p; }

__device__ __forceinline__ bf16x8_t frag_bf16(const u32x4_t *tile, int row, int kc)
{
    return __builtin_bit_cast(bf16x8_t, tile[swz(row, kc)]);
}

// 8 MXFP4 elements of row `row`, k-chunk kc (0..7) -> bf16x8 scaled by the block scale.
__device__ __forceinline__ bf16x8_t frag_mx(const u32x4_t *tile, const uint8_t *sc, int row, int kc)
{
    const uint32_t *t32 = reinterpret_cast<const uint32_t *>(tile);
    const uint32_t w = t32[mx_slot(row, kc >> 2) * 4 + (kc & 3)];
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

// One stage of global data held in registers between load and LDS store.
template <bool MX>
struct Stage {
    u32x4_t a[4];             // A: rows (tid>>3) + 32q, chunk tid&7
    u32x4_t b[MX ? 2 : 8];    // B bf16: rows (tid>>3) + 32q; MX: rows (tid>>1) + 128q, half tid&1
    uint32_t s;               // MX: the two scale bytes of row tid
};

template <bool MX>
struct Ptrs {
    const char *a[4];
    const char *b[MX ? 2 : 8];
    const uint8_t *s;
};

template <bool MX>
__device__ __forceinline__ void gload(Stage<MX> &st, const Ptrs<MX> &p, int kt)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        st.a[q] = ldg16(p.a[q] + (size_t)kt * BK * 2);
    if (MX) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            st.b[q] = ldg16(p.b[q] + (size_t)kt * BK / 2);
        st.s = ldg2(p.s + (size_t)kt * 2);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            st.b[q] = ldg16(p.b[q] + (size_t)kt * BK * 2);
    }
}

template <bool MX>
__device__ __forceinline__ void sstore(const Stage<MX> &st, u32x4_t *As, u32x4_t *Bs, uint8_t *Sc, int tid)
{
#pragma unroll
    for (int q = 0; q < 4; ++q)
        As[swz((tid >> 3) + 32 * q, tid & 7)] = st.a[q];
    if (MX) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
            Bs[mx_slot((tid >> 1) + 128 * q, tid & 1)] = st.b[q];
        *reinterpret_cast<uint16_t *>(Sc + tid * 2) = (uint16_t)st.s;
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            Bs[swz((tid >> 3) + 32 * q, tid & 7)] = st.b[q];
    }
}

// Map the 1-D block index to a work item so that each XCD gets a contiguous
// run of items (see the file header).  Returns -1 past the real work.
__device__ __forceinline__ int xcd_item(int b, int total)
{
    if (b >= total)
        return -1;
    const int x = b & 7, i = b >> 3, q = total >> 3, r = total & 7;
    return x * q + min(x, r) + i;
}
}  // namespace

// MODE 1: GEMM1 + SwiGLU (A = x rows through perm, K = d, out H bf16 [R][I]).
// MODE 2: GEMM2          (A = H rows,           K = I, out Y fp32 [R][d]).
// grid = max tiles * NT blocks (1-D), NT = N / 128 (MODE 1) or d / 256 (MODE 2).
template <int MODE, bool MX>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm(
    const uint64_t *__restrict__ ptrs, size_t off_w0, size_t off_w1, size_t off_s0, size_t off_s1,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, const uint16_t *__restrict__ A,
    int K, int N, int lda, int k, int E, int R, int NT, void *__restrict__ out)
{
    __shared__ u32x4_t As[2][BM * 8];
    __shared__ u32x4_t Bs[2][MX ? BN * 2 : BN * 8];
    __shared__ uint8_t Sc[2][MX ? BN * 2 : 4];

    const int item = xcd_item(blockIdx.x, *n_tiles * NT);
    if (item < 0)
        return;
    const int ti = item / NT, nt = item - ti * NT;
    const int e = tiles[2 * ti], m0 = tiles[2 * ti + 1];
    if ((unsigned)e >= (unsigned)E)  // routing metadata is produced on the device; never index past it
        return;
    const uint64_t blob = ptrs[e];
    const int rb = offsets[e] + m0;
    const int mrows = min(BM, offsets[e + 1] - rb);
    if (!blob || m0 < 0 || rb < 0 || mrows <= 0 || rb + mrows > R)
        return;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
    // MODE 1: this block's intermediate columns [n0, n0 + 128); MODE 2: outputs [n0, n0 + 256)
    const int n0 = nt * (MODE == 1 ? BN / 2 : BN);

    Ptrs<MX> p;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = min((tid >> 3) + 32 * q, mrows - 1);
        const size_t arow = MODE == 1 ? (size_t)(perm[rb + row] / k) : (size_t)(rb + row);
        p.a[q] = (const char *)(A + arow * lda + (tid & 7) * 8);
    }
    // weight row r of the block's B tile (0..255) -> matrix row in the blob
    auto brow = [&](int r, size_t &sec_off, size_t &sc_off) {
        if (MODE == 1) {
            sec_off = r < BN / 2 ? off_w0 : off_w1;
            sc_off = r < BN / 2 ? off_s0 : off_s1;
            return n0 + (r & (BN / 2 - 1));
        }
        sec_off = off_w0;
        sc_off = off_s0;
        return n0 + r;
    };
    if (MX) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            size_t so, sco;
            const int r = brow((tid >> 1) + 128 * q, so, sco);
            p.b[q] = (const char *)blob + so + (size_t)r * (K / 2) + (tid & 1) * 16;
        }
        size_t so, sco;
        const int r = brow(tid, so, sco);
        p.s = (const uint8_t *)blob + sco + (size_t)r * (K / 32);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            size_t so, sco;
            const int r = brow((tid >> 3) + 32 * q, so, sco);
            p.b[q] = (const char *)blob + so + (size_t)r * K * 2 + (tid & 7) * 16;
        }
        p.s = nullptr;
    }
    // B-tile rows of this wave's 4 column blocks
    int bbase[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
        bbase[cb] = MODE == 1 ? (cb >> 1) * (BN / 2) + wn * 64 + (cb & 1) * 32 : wn * 128 + cb * 32;
    // MFMA row blocks of this wave that hold real rows
    const int nms = max(0, min(2, (mrows - wm * 64 + 31) / 32));

    f32x16_t acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[a][b][j] = 0.f;

    const int nk = K / BK;
    Stage<MX> s0, s1;
    gload<MX>(s0, p, 0);
    if (nk > 1)
        gload<MX>(s1, p, 1);
    sstore<MX>(s0, As[0], Bs[0], Sc[0], tid);
    __syncthreads();
    // NXT holds k-tile kt+1 (loaded one iteration ago); FRE is free and receives
    // k-tile kt+2.  Two copies of the body alternate the roles so both stages
    // stay in named registers.
#define ECF_GEMM_BODY(KT, NXT, FRE)                                                                  \
    {                                                                                               \
        const int cur = (KT) & 1;                                                                   \
        if ((KT) + 2 < nk)                                                                          \
            gload<MX>(FRE, p, (KT) + 2);                                                            \
        if (nms > 0) {                                                                              \
            _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks)                                  \
            {                                                                                       \
                const int kc = ks * 2 + (l >> 5);                                                   \
                bf16x8_t af[2], bfr[4];                                                             \
                _Pragma("unroll") for (int ms = 0; ms < 2; ++ms) if (ms < nms) af[ms] =            \
                    frag_bf16(As[cur], wm * 64 + ms * 32 + (l & 31), kc);                           \
                _Pragma("unroll") for (int cb = 0; cb < 4; ++cb)                                    \
                {                                                                                   \
                    const int n = bbase[cb] + (l & 31);                                             \
                    bfr[cb] = MX ? frag_mx(Bs[cur], Sc[cur], n, kc) : frag_bf16(Bs[cur], n, kc);     \
                }                                                                                   \
                _Pragma("unroll") for (int ms = 0; ms < 2; ++ms) if (ms < nms)                      \
                    _Pragma("unroll") for (int cb = 0; cb < 4; ++cb) acc[ms][cb] =                  \
                        __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[cb], acc[ms][cb], 0, 0, 0); \
            }                                                                                       \
        }                                                                                           \
        if ((KT) + 1 < nk)                                                                          \
            sstore<MX>(NXT, As[cur ^ 1], Bs[cur ^ 1], Sc[cur ^ 1], tid);                            \
        __syncthreads();                                                                            \
    }
    for (int kt = 0; kt < nk; kt += 2) {
        ECF_GEMM_BODY(kt, s1, s0)
        if (kt + 1 < nk)
            ECF_GEMM_BODY(kt + 1, s0, s1)
    }
#undef ECF_GEMM_BODY

    // epilogue: a lane holds rows (j/4)*8 + (l/32)*4 + j%4 of column l%32 of each fragment
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
        if (ms >= nms)
            continue;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int m = wm * 64 + ms * 32 + (j >> 2) * 8 + (l >> 5) * 4 + (j & 3);
            if (m >= mrows)
                continue;
            if (MODE == 1) {
                uint16_t *H = (uint16_t *)out + (size_t)(rb + m) * N + n0 + wn * 64 + (l & 31);
                H[0] = f_to_bf(silu_mul(acc[ms][0][j], acc[ms][2][j]));
                H[32] = f_to_bf(silu_mul(acc[ms][1][j], acc[ms][3][j]));
            } else {
                float *Y = (float *)out + (size_t)(rb + m) * N + n0 + wn * 128 + (l & 31);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    Y[cb * 32] = acc[ms][cb][j];
            }
        }
    }
}

// ---------------------------------------------------------------------------------

int launch_prefill_gemm1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, uint16_t *H, hipStream_t st)
{
    const int NT = s.inter / (BN / 2);
    const int nblk = max_tiles(s, T) * NT;
    ProfScope p("prefill_gemm1", st);
#define ECF_G1(MXV)                                                                                  \
    hipLaunchKernelGGL((k_grouped_gemm<1, MXV>), dim3(nblk), dim3(256), 0, st, ex.ptrs, ex.lay.off[0], \
                       ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.tiles, o.n_tiles, o.offsets, o.perm, \
                       (const uint16_t *)x, s.hidden, s.inter, s.hidden, s.top_k, s.n_experts, T * s.top_k,  \
                       NT, (void *)H)
    if (s.w_dtype == ECF_MXFP4)
        ECF_G1(true);
    else
        ECF_G1(false);
#undef ECF_G1
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_prefill_gemm2(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const uint16_t *H,
                         int T, float *Y, hipStream_t st)
{
    const int NT = s.hidden / BN;
    const int nblk = max_tiles(s, T) * NT;
    ProfScope p("prefill_gemm2", st);
#define ECF_G2(MXV)                                                                                  \
    hipLaunchKernelGGL((k_grouped_gemm<2, MXV>), dim3(nblk), dim3(256), 0, st, ex.ptrs, ex.lay.off[2], \
                       ex.lay.off[2], ex.lay.off[5], ex.lay.off[5], o.tiles, o.n_tiles, o.offsets, o.perm, H, \
                       s.inter, s.hidden, s.inter, s.top_k, s.n_experts, T * s.top_k, NT, (void *)Y)
    if (s.w_dtype == ECF_MXFP4)
        ECF_G2(true);
    else
        ECF_G2(false);
#undef ECF_G2
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
