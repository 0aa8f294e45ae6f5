// Prefill-path expert kernels: grouped GEMMs over the expert-sorted rows on
// gfx950 MFMA (v_mfma_f32_32x32x16_bf16), bf16 or MXFP4 weights.
//
// In prefill thousands of tokens reach nearly every expert of a layer
// (FreeToken paper explainer, section "Wall 1: prefill" -- sparsity vanishes),
// so each expert is a small dense GEMM: its rows are contiguous in the
// counting-sort order and tiled BM rows at a time (128 for bf16 weights, 320
// for MXFP4; the tile list comes from the routing kernels).
//
//   GEMM1: [a | b] = X_perm . [W_gate ; W_up]^T, h = silu(a) * b -> H (bf16)
//          A rows are gathered from x through perm; one block owns 128
//          intermediate columns of both gate and up, so SwiGLU runs in
//          registers on matching accumulator fragments.
//   GEMM2: Y = H . W_down^T (fp32), combined per token by k_combine.
//
// Block = NW waves as WM x (NW / WM), tile BM rows x BNT weight rows, BK = 64
// (bf16: 8 waves on 128 x 256, each 64 x 64; MXFP4: 8 waves on 320 x 256, each
// 160 rows x 64 weight rows, i.e. up to 5 x 2 MFMA 32x32 fragments).  Software pipeline of depth 2 through
// registers: in program order the loads of k-tile kt+2 come before the MFMAs
// of k-tile kt and the LDS stores of k-tile kt+1 after them (the compiler's
// schedule of that order measured faster than pinning it with scheduling
// barriers).  Operands arrive by raw buffer loads: one 32-bit offset register
// per row, the k-tile's column in a scalar offset.  (Direct global->LDS loads
// were measured against: the compiler cannot tell which in-flight LDS DMA a
// later LDS read depends on and drains them all, which serialises the
// pipeline.)
//
// bf16 rows of 64 elements (eight 16-B chunks) sit in LDS XOR-swizzled (see
// swz), so the 32 rows one MFMA operand read touches spread over the banks.
// MXFP4 weights stay 4-bit in LDS (a quarter of the bf16 bytes) and are
// expanded in registers by v_cvt_scalef32_pk_bf16_fp4, which applies the E8M0
// block scale exactly; products run on bf16 MFMA.
//
// Blocks are issued round-robin over the 8 XCDs (block b runs on XCD b % 8),
// each with its own L2.  The 1-D block index is remapped so each XCD walks a
// contiguous range of (tile, N-tile) work items, N-tile fastest: the blocks
// sharing one expert tile's A rows run on the same XCD at about the same time.
#include "device_common.h"
#include "ecf_internal.h"

namespace ecf {

namespace {
constexpr int BK = 64;  // reduction elements per stage

// bf16 tile rows of eight 16-B chunks; chunk c of row r sits at c ^ (r & 7) ^ bit 3
// of r.  A 16-B-per-lane read of one chunk over rows r0..r0+15 then touches 16
// distinct 16-B bank groups mod 256 B (and any 8 aligned rows 8 distinct groups
// mod 128 B), so it is conflict-free whether the LDS serves 8 or 16 lanes of a
// 128-bit access per cycle.
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7) ^ ((row >> 3) & 1)); }

// MXFP4 LDS tile: row = 32 bytes (two 16-B halves); the halves swap with bit 2
// xor bit 3 of the row, so one half over 16 consecutive rows (or 8 aligned
// rows) covers distinct bank groups.
__device__ __forceinline__ int mx_slot(int row, int half) { return row * 2 + (half ^ (((row >> 2) ^ (row >> 3)) & 1)); }

// E8M0 scale byte -> 2^(s - 127) (s = 0: the subnormal 2^-127; 0xFF: NaN, as OCP
// MX v1.0 defines it).
__device__ __forceinline__ float e8m0_f(uint32_t s)
{
    return __uint_as_float(s == 0 ? 0x00400000u : s == 255 ? 0x7FC00000u : (s << 23));
}

__device__ __forceinline__ bf16x8_t frag_bf16(const u32x4_t *tile, int row, int kc)
{
    return __builtin_bit_cast(bf16x8_t, tile[swz(row, kc)]);
}

// 8 MXFP4 elements (one dword of nibbles, element 2i in the low nibble of byte
// i) -> bf16x8, each multiplied by the block scale s (exact: s is a power of 2).
__device__ __forceinline__ bf16x8_t cvt_mx8(uint32_t w, float s)
{
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
// BNT = weight rows per block tile; NBL = 16-B B chunks per thread and stage.
// A stage covers KS sub-tiles of BK = 64 reduction elements each.
template <bool MX, int BM, int BNT, int KS, int NTH>
struct Stage {
    static constexpr int NAL = BM * 8 / NTH;                // 16-B A chunks per thread and sub-tile
    static constexpr int NBL = (MX ? BNT * 2 : BNT * 8) / NTH;  // 16-B B chunks per thread and sub-tile
    static_assert(NAL >= 1 && NBL >= 1, "tile too small for the block");
    u32x4_t a[NAL * KS];      // A: rows (tid>>3) + (NTH/8)q, chunk tid&7, per sub-tile
    u32x4_t b[NBL * KS];      // B bf16: rows (tid>>3) + (NTH/8)q; MX: rows (tid>>1) + (NTH/2)q, half tid&1
    uint32_t s;               // MX: the 2*KS scale bytes of row tid (tid < BNT)
};

// Operand loads are raw buffer loads: a block-uniform resource (base and byte
// size, in scalar registers), this thread's 32-bit row offset, and the k-tile's
// column offset as the uniform soffset -- one VGPR per row and no per-k-tile
// address arithmetic in vector registers.  A load at or past the size returns 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // 0x00020000: word 3 of a raw-buffer resource on gfx9 parts (32-bit data format)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

template <bool MX, int BM, int BNT, int NTH>
struct Ptrs {
    uint32_t a[Stage<MX, BM, BNT, 1, NTH>::NAL];  // A rows, this thread's 16-B chunk (bytes from A's base)
    uint32_t b[Stage<MX, BM, BNT, 1, NTH>::NBL];  // B rows within the blob, this thread's 16-B chunk
    uint32_t s;                                   // MX: this thread's scale row within the blob
};

// BAUX: cache policy of the weight loads (2 = non-temporal, 0 = default).
template <int BAUX, bool MX, int BM, int BNT, int KS, int NTH>
__device__ __forceinline__ void gload(Stage<MX, BM, BNT, KS, NTH> &st, const Ptrs<MX, BM, BNT, NTH> &p, rsrc_t ra,
                                      rsrc_t rb, int kt, int tid)
{
    constexpr int NAL = Stage<MX, BM, BNT, KS, NTH>::NAL, NBL = Stage<MX, BM, BNT, KS, NTH>::NBL;
#pragma unroll
    for (int sub = 0; sub < KS; ++sub) {
        const int col = (kt * KS + sub) * BK;  // first reduction element of the sub-tile
#pragma unroll
        for (int q = 0; q < NAL; ++q)
            st.a[sub * NAL + q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, p.a[q], col * 2, 0));
#pragma unroll
        for (int q = 0; q < NBL; ++q)
            st.b[sub * NBL + q] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, p.b[q], MX ? col / 2 : col * 2, BAUX));
    }
    // every thread loads (threads past BNT re-read row 0's scales), so the number
    // of loads in flight is the same on every path and the compiler's load
    // counters can wait for exactly the older stage
    if (MX)
        st.s = KS == 2 ? __builtin_amdgcn_raw_buffer_load_b32(rb, p.s, kt * 4, 0)
                       : (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, p.s, kt * 2, 0);
}

// Registers -> LDS.  Sub-tile `sub` of A sits at As + sub * BM * 8 and of B at
// Bs + sub * (B tile size).  MX scales are widened to fp32 here, once per row
// and stage, and stored group-major: Scf[group * (BNT + 32) + row] (the pad
// puts the two lane halves' reads on different banks).
template <bool MX, int BM, int BNT, int KS, int NTH>
__device__ __forceinline__ void sstore(const Stage<MX, BM, BNT, KS, NTH> &st, u32x4_t *As, u32x4_t *Bs, float *Scf,
                                       int tid)
{
    constexpr int NAL = Stage<MX, BM, BNT, KS, NTH>::NAL, NBL = Stage<MX, BM, BNT, KS, NTH>::NBL;
    constexpr int BT = MX ? BNT * 2 : BNT * 8;  // 16-B slots of one B sub-tile
#pragma unroll
    for (int sub = 0; sub < KS; ++sub) {
#pragma unroll
        for (int q = 0; q < NAL; ++q)
            As[sub * BM * 8 + swz((tid >> 3) + (NTH / 8) * q, tid & 7)] = st.a[sub * NAL + q];
#pragma unroll
        for (int q = 0; q < NBL; ++q) {
            if (MX)
                Bs[sub * BT + mx_slot((tid >> 1) + (NTH / 2) * q, tid & 1)] = st.b[sub * NBL + q];
            else
                Bs[sub * BT + swz((tid >> 3) + (NTH / 8) * q, tid & 7)] = st.b[sub * NBL + q];
        }
    }
    if (MX && (BNT >= NTH || tid < BNT)) {
        // The empty asm keeps the widening here, after the stage's other stores:
        // left free, the compiler hoists it next to the load, and waiting for
        // that load there waits for every load issued before it.
        uint32_t sc = st.s;
        asm volatile("" : "+v"(sc));
#pragma unroll
        for (int gi = 0; gi < 2 * KS; ++gi)
            Scf[gi * (BNT + 32) + tid] = e8m0_f((sc >> (8 * gi)) & 0xffu);
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

template <int V>
struct IC {
    static constexpr int value = V;
};
}  // namespace

// MODE 1: GEMM1 + SwiGLU (A = x rows through perm, K = d, out H bf16 [R][I]).
// MODE 2: GEMM2          (A = H rows,           K = I, out Y fp32 [R][d]).
// BNT weight rows per block (MODE 1: BNT/2 gate + BNT/2 up rows), MINB blocks
// per CU asked of the register allocator.
// grid = max tiles * NT blocks (1-D), NT = I / (BNT/2) (MODE 1) or d / BNT (MODE 2).
//
// Reduction order inside a 64-wide k-tile: at MFMA step ks (0..3), lanes 0-31
// feed k-chunk ks and lanes 32-63 feed k-chunk 4 + ks (8 elements each), for A
// and B alike, so every chunk is used once.  Lane half g then reads the 32
// MXFP4 elements 32g..32g+31 -- 16 bytes, exactly one E8M0 scale group -- with
// a single LDS read per k-tile.
template <int MODE, bool MX, int BM, int BNT, int MINB, int KS, int WM, int NW>
__global__ __launch_bounds__(64 * NW, MINB) void k_grouped_gemm(
    const uint64_t *__restrict__ ptrs, size_t off_w0, size_t off_w1, size_t off_s0, size_t off_s1,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, const uint16_t *__restrict__ A,
    int K, int N, int lda, int k, int E, int R, int NT, uint32_t blob_bytes, void *__restrict__ out)
{
    constexpr int NTH = 64 * NW, WN = NW / WM, WROWS = BM / WM, NMSMAX = WROWS / 32;
    constexpr int NCB = BNT / (32 * WN);  // 32-column MFMA blocks per wave
    static_assert(NW % WM == 0 && NCB >= (MODE == 1 ? 2 : 1) && NMSMAX >= 1, "wave layout");
    constexpr int BT = MX ? BNT * 2 : BNT * 8;  // 16-B slots of one B sub-tile
    // bf16 gate/up weights are streamed with non-temporal loads (each k-tile
    // takes whole 128-B lines of a row; 800 -> 756 us for the 4096-token layer).
    // MXFP4 k-tiles take 32 B of a line whose rest the next three k-tiles use,
    // and the bf16 down GEMM got slower with them: default policy there.
    constexpr int BAUX = (!MX && MODE == 1) ? 2 : 0;
    __shared__ u32x4_t As[2][KS * BM * 8];
    __shared__ u32x4_t Bs[2][KS * BT];
    __shared__ float Scf[2][MX ? 2 * KS * (BNT + 32) : 4];

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
    // NW waves, WM of them along M (4 waves as 2 x 2: 64 rows per wave; WM = 1
    // halves the per-MFMA B-fragment work at the cost of A reads)
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6, wm = w / WN, wn = w % WN, g = l >> 5;
    // MODE 1: this block's intermediate columns [n0, n0 + BNT/2); MODE 2: outputs [n0, n0 + BNT)
    const int n0 = nt * (MODE == 1 ? BNT / 2 : BNT);

    Ptrs<MX, BM, BNT, NTH> p;
#pragma unroll
    for (int q = 0; q < Stage<MX, BM, BNT, 1, NTH>::NAL; ++q) {
        const int row = min((tid >> 3) + (NTH / 8) * q, mrows - 1);
        const size_t arow = MODE == 1 ? (size_t)(perm[rb + row] / k) : (size_t)row;  // from abase
        p.a[q] = (uint32_t)(arow * lda * 2 + (tid & 7) * 16);
    }
    // A: all of x (MODE 1; under 4 GiB, checked by the launcher) or the rows from
    // the tile's first on (MODE 2); B: the blob
    const size_t abytes = MODE == 1 ? (size_t)(R / k) * lda * 2 : (size_t)(R - rb) * lda * 2;
    const rsrc_t ra = make_rsrc(A + (MODE == 1 ? 0 : (size_t)rb * lda), (uint32_t)min(abytes, (size_t)0xFFFFFFFFu));
    const rsrc_t rbs = make_rsrc((const void *)blob, blob_bytes);
    // weight row r of the block's B tile -> (section, scale section, matrix row)
    auto brow = [&](int r, size_t &sec_off, size_t &sc_off) {
        if (MODE == 1) {
            sec_off = r < BNT / 2 ? off_w0 : off_w1;
            sc_off = r < BNT / 2 ? off_s0 : off_s1;
            return n0 + (r & (BNT / 2 - 1));
        }
        sec_off = off_w0;
        sc_off = off_s0;
        return n0 + r;
    };
    if (MX) {
#pragma unroll
        for (int q = 0; q < Stage<MX, BM, BNT, 1, NTH>::NBL; ++q) {
            size_t so, sco;
            const int r = brow((tid >> 1) + (NTH / 2) * q, so, sco);
            p.b[q] = (uint32_t)(so + (size_t)r * (K / 2) + (tid & 1) * 16);
        }
        size_t so, sco;
        const int r = brow(tid < BNT ? tid : 0, so, sco);
        p.s = (uint32_t)(sco + (size_t)r * (K / 32));
    } else {
#pragma unroll
        for (int q = 0; q < Stage<MX, BM, BNT, 1, NTH>::NBL; ++q) {
            size_t so, sco;
            const int r = brow((tid >> 3) + (NTH / 8) * q, so, sco);
            p.b[q] = (uint32_t)(so + (size_t)r * K * 2 + (tid & 7) * 16);
        }
        p.s = 0;
    }
    // B-tile rows (lane's row within each of this wave's column blocks)
    int brw[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
        brw[cb] = (l & 31) + (MODE == 1 ? (cb < NCB / 2 ? wn * (BNT / 2 / WN) + cb * 32
                                                       : BNT / 2 + wn * (BNT / 2 / WN) + (cb - NCB / 2) * 32)
                                        : wn * (BNT / WN) + cb * 32);
    const int nk = K / (BK * KS);

    // The pipelined main loop and epilogue, instantiated per number of MFMA
    // row blocks (0, 1, 2) this wave owns, so the loop body has no branches.
    auto run = [&](auto nms_c) __attribute__((always_inline)) {
        constexpr int NMS = decltype(nms_c)::value;
        f32x16_t acc[NMSMAX][NCB];
#pragma unroll
        for (int a = 0; a < NMSMAX; ++a)
#pragma unroll
            for (int b = 0; b < NCB; ++b)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    acc[a][b][j] = 0.f;
        Stage<MX, BM, BNT, KS, NTH> s0, s1;
        gload<BAUX>(s0, p, ra, rbs, 0, tid);
        gload<BAUX>(s1, p, ra, rbs, 1, tid);
        sstore(s0, As[0], Bs[0], Scf[0], tid);
        __syncthreads();
        // NXT holds k-tile kt+1 (loaded one iteration ago); FRE is free and
        // receives k-tile kt+2.  Two copies of the body alternate the roles so
        // both stages stay in named registers.  Loads and stores are issued on
        // every iteration (nk is even and >= 2; past the end the last k-tile is
        // re-read into a buffer nobody reads): branch-free, the compiler's
        // load counters wait only for the older stage, which keeps two k-tiles
        // of loads in flight.
#define ECF_GEMM_BODY(KT, NXT, FRE)                                                                  \
    {                                                                                               \
        const int cur = (KT) & 1;                                                                   \
        gload<BAUX>(FRE, p, ra, rbs, min((KT) + 2, nk - 1), tid);                                   \
        if (NMS > 0) {                                                                              \
            _Pragma("unroll") for (int sub = 0; sub < KS; ++sub)                                    \
            {                                                                                       \
                const u32x4_t *Asb = As[cur] + sub * BM * 8, *Bsb = Bs[cur] + sub * BT;             \
                float bsc[NCB];                                                                     \
                if (MX) {                                                                           \
                    _Pragma("unroll") for (int cb = 0; cb < NCB; ++cb)                              \
                        bsc[cb] = Scf[cur][(sub * 2 + g) * (BNT + 32) + brw[cb]];                   \
                }                                                                                   \
                _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks)                              \
                {                                                                                   \
                    const int kc = 4 * g + ks;                                                      \
                    bf16x8_t af[NMSMAX], bfr[NCB];                                                  \
                    _Pragma("unroll") for (int ms = 0; ms < NMS; ++ms) af[ms] =                    \
                        frag_bf16(Asb, wm * WROWS + ms * 32 + (l & 31), kc);                        \
                    _Pragma("unroll") for (int cb = 0; cb < NCB; ++cb) bfr[cb] =                    \
                        MX ? cvt_mx8(reinterpret_cast<const uint32_t *>(Bsb)[mx_slot(brw[cb], g) * 4 + ks], \
                                     bsc[cb])                                                       \
                           : frag_bf16(Bsb, brw[cb], kc);                                           \
                    _Pragma("unroll") for (int ms = 0; ms < NMS; ++ms)                              \
                        _Pragma("unroll") for (int cb = 0; cb < NCB; ++cb) acc[ms][cb] =            \
                            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[cb], acc[ms][cb], 0, 0, 0); \
                }                                                                                   \
            }                                                                                       \
        }                                                                                           \
        sstore(NXT, As[cur ^ 1], Bs[cur ^ 1], Scf[cur ^ 1], tid);                                   \
        __syncthreads();                                                                            \
    }
        for (int kt = 0; kt < nk; kt += 2) {
            ECF_GEMM_BODY(kt, s1, s0)
            ECF_GEMM_BODY(kt + 1, s0, s1)
        }
#undef ECF_GEMM_BODY
        // epilogue: a lane holds rows (j/4)*8 + (l/32)*4 + j%4 of column l%32 of each fragment
#pragma unroll
        for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int m = wm * WROWS + ms * 32 + (j >> 2) * 8 + (l >> 5) * 4 + (j & 3);
                if (m >= mrows)
                    continue;
                if (MODE == 1) {
                    uint16_t *H = (uint16_t *)out + (size_t)(rb + m) * N + n0 + wn * (BNT / 2 / WN) + (l & 31);
#pragma unroll
                    for (int cb = 0; cb < NCB / 2; ++cb)
                        H[cb * 32] = f_to_bf(silu_mul(acc[ms][cb][j], acc[ms][cb + NCB / 2][j]));
                } else {
                    // Y is read once, by the combine: non-temporal stores (bf16
                    // down GEMM 491 -> 445 us; MXFP4 unchanged)
                    float *Y = (float *)out + (size_t)(rb + m) * N + n0 + wn * (BNT / WN) + (l & 31);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        __builtin_nontemporal_store(acc[ms][cb][j], Y + cb * 32);
                }
            }
        }
    };
    // MFMA row blocks of this wave that hold real rows (uniform over the wave)
    // (with WM = 1 a block of 65..96 rows runs 4 row blocks: one wasted, one fewer instance)
    const int nms = __builtin_amdgcn_readfirstlane(max(0, min(NMSMAX, (mrows - wm * WROWS + 31) / 32)));
    static_assert(NMSMAX <= 5, "row-block instances below cover up to 5");
    if constexpr (NMSMAX >= 5) {
        if (nms >= 5) {
            run(IC<NMSMAX>{});
            return;
        }
    }
    if constexpr (NMSMAX >= 4) {
        if (nms == 4) {
            run(IC<4>{});
            return;
        }
    }
    if constexpr (NMSMAX >= 3) {
        if (nms == 3) {
            run(IC<3>{});
            return;
        }
    }
    if (nms == 2)
        run(IC<2>{});
    else if (nms == 1)
        run(IC<1>{});
    else
        run(IC<0>{});
}

// ---------------------------------------------------------------------------------

// Tile choice per weight format, measured on MI355X (bf16: 4096-token layer,
// d 4096, I 1024, top-6; MXFP4: 8192-token layer, I 2048, top-8).  bf16 (HBM-
// bound): 128 x 256 tiles, 8 waves as 2 x 4 (64 x 64 each), one block per CU --
// half the A re-reads of 128 x 128 tiles with 4 waves (layer 1.48 -> 1.41 ms).
// MXFP4: 320 x
// 256 tiles, 8 waves as 2 x 4 (160 rows x 64 weight rows each), one block per
// CU -- each expanded B fragment feeds up to five MFMAs, and an expert with up
// to 320 rows streams its weights through one tile: with ~256 +- 16 rows per
// expert, 256-row tiles left a tail tile (a whole weight pass for a few dozen
// rows) on half the experts; 320-row tiles took the layer from 3.94 to 3.64 ms
// (256-row tiles with 8 waves were 5% faster than 4 waves on 128 x 256).  Two-sub-tile
// stages, a 1 x 4 wave layout, three blocks per CU, expanding MXFP4 to bf16 once
// at the LDS store, 4 waves on 256 x 256 and 8 waves on 128 x 256 were each
// slower or spilled registers.
#ifndef ECF_BF16_BNT
#define ECF_BF16_BNT 256
#define ECF_BF16_MINB 1
#define ECF_BF16_KS 1
#define ECF_BF16_WM 2
#endif
#ifndef ECF_BF16_NW
#define ECF_BF16_NW 8
#endif
#ifndef ECF_MX_BNT
#define ECF_MX_BNT 256
#define ECF_MX_MINB 1
#define ECF_MX_KS 1
#define ECF_MX_WM 2
#endif
#ifndef ECF_MX_NW
#define ECF_MX_NW 8
#endif


int launch_prefill_gemm1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, uint16_t *H, hipStream_t st)
{
    const bool mx = s.w_dtype == ECF_MXFP4;
    const int bnt = mx ? ECF_MX_BNT : ECF_BF16_BNT;
    const int NT = s.inter / (bnt / 2);
    // the kernel addresses x rows and blob rows with 32-bit byte offsets
    if ((size_t)T * s.hidden * 2 > 0xFFFFFFFFull || ex.lay.bytes > 0xFFFFFFFFull)
        return set_error(ECF_EUNSUPPORTED, "prefill path: x (%d x %d bf16) and one expert blob (%zu B) must each "
                         "be under 4 GiB", T, s.hidden, ex.lay.bytes);
    const int nblk = max_tiles(s, T) * NT;
    ProfScope p("prefill_gemm1", st);
#define ECF_G1(MXV, BNV, MBV, KSV, WMV, NWV)                                                               \
    hipLaunchKernelGGL((k_grouped_gemm<1, MXV, (MXV) ? ECF_MX_BM : kPrefillMT, BNV, MBV, KSV, WMV, NWV>), dim3(nblk), \
                       dim3(64 * (NWV)), 0, st, ex.ptrs,                                                     \
                       ex.lay.off[0], ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.tiles, o.n_tiles,         \
                       o.offsets, o.perm, (const uint16_t *)x, s.hidden, s.inter, s.hidden, s.top_k,         \
                       s.n_experts, T * s.top_k, NT, (uint32_t)ex.lay.bytes, (void *)H)
    // K = d; the main loop takes an even number of stages of KS sub-tiles: d % (128 * KS) == 0
    // (d is a multiple of 256)
    if (mx)
        ECF_G1(true, ECF_MX_BNT, ECF_MX_MINB, ECF_MX_KS, ECF_MX_WM, ECF_MX_NW);
    else
        ECF_G1(false, ECF_BF16_BNT, ECF_BF16_MINB, ECF_BF16_KS, ECF_BF16_WM, ECF_BF16_NW);
#undef ECF_G1
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_prefill_gemm2(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const uint16_t *H,
                         int T, float *Y, hipStream_t st)
{
    const bool mx = s.w_dtype == ECF_MXFP4;
    const int bnt = mx ? ECF_MX_BNT : ECF_BF16_BNT;
    const int NT = s.hidden / bnt;
    if (ex.lay.bytes > 0xFFFFFFFFull)  // blob rows are addressed with 32-bit byte offsets
        return set_error(ECF_EUNSUPPORTED, "prefill path: one expert blob (%zu B) must be under 4 GiB", ex.lay.bytes);
    const int nblk = max_tiles(s, T) * NT;
    ProfScope p("prefill_gemm2", st);
#define ECF_G2(MXV, BNV, MBV, KSV, WMV, NWV)                                                               \
    hipLaunchKernelGGL((k_grouped_gemm<2, MXV, (MXV) ? ECF_MX_BM : kPrefillMT, BNV, MBV, KSV, WMV, NWV>), dim3(nblk), \
                       dim3(64 * (NWV)), 0, st, ex.ptrs,                                                     \
                       ex.lay.off[2], ex.lay.off[2], ex.lay.off[5], ex.lay.off[5], o.tiles, o.n_tiles,         \
                       o.offsets, o.perm, H, s.inter, s.hidden, s.inter, s.top_k, s.n_experts, T * s.top_k,  \
                       NT, (uint32_t)ex.lay.bytes, (void *)Y)
    // K = I; the main loop takes an even number of stages: two-sub-tile stages
    // only when I % 256 == 0 (I % 128 == 0 holds on this path)
    if (mx) {
        if (s.inter % (128 * ECF_MX_KS) == 0)
            ECF_G2(true, ECF_MX_BNT, ECF_MX_MINB, ECF_MX_KS, ECF_MX_WM, ECF_MX_NW);
        else
            ECF_G2(true, ECF_MX_BNT, ECF_MX_MINB, 1, ECF_MX_WM, ECF_MX_NW);
    } else {
        if (s.inter % (128 * ECF_BF16_KS) == 0)
            ECF_G2(false, ECF_BF16_BNT, ECF_BF16_MINB, ECF_BF16_KS, ECF_BF16_WM, ECF_BF16_NW);
        else
            ECF_G2(false, ECF_BF16_BNT, ECF_BF16_MINB, 1, ECF_BF16_WM, ECF_BF16_NW);
    }
#undef ECF_G2
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
