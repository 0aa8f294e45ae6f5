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
// 160 rows x 64 weight rows, i.e. up to 5 x 2 MFMA 32x32 fragments).
//
// Operand tiles go from global memory straight into LDS (buffer_load ... lds,
// 16 bytes per lane, gfx950), three stages deep: while the MFMAs of k-tile kt
// run, the loads of k-tile kt+2 are in flight and those of kt+1 land.  Each
// stage is its own LDS array, so the compiler's wait before an LDS read covers
// only the loads into that stage; the end of a k-tile waits for this wave's
// loads of k-tile kt+1 and then meets the other waves (stage_barrier).  No
// operand passes through registers on its way to LDS.  Against a depth-2
// pipeline through registers on one GPU: MXFP4 GEMM1 2145 -> 2038 us, GEMM2
// 1129 -> 1077 us, bf16 GEMM1 752 -> 745 us.  Loads use raw buffer resources:
// one 32-bit offset register per row, the k-tile's column in a scalar offset.
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
// 128-bit access per cycle.  (A layout with 8-row blocks stored chunk-major,
// which needs one LDS address register per stage instead of one per chunk,
// measured slower: its global->LDS loads put consecutive lanes on different
// rows, so the loads coalesce worse; bf16 GEMM1 743 -> 837 us.)
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

// Operand loads are raw buffer loads: a block-uniform resource (base and byte
// size, in scalar registers), this thread's 32-bit row offset, and the k-tile's
// column offset as the uniform soffset -- one VGPR per row and no per-k-tile
// address arithmetic in vector registers.  A lane whose offset lies at or past
// the size reads zeros and touches no memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // 0x00020000: word 3 of a raw-buffer resource on gfx9 parts (32-bit data format)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a raw buffer straight into LDS: lane l's bytes land at
// lds + 16 l (the LDS base is wave-uniform; it goes to M0).  AUX is the cache
// policy.  The 16-byte form is gfx950's; hipcc's host pass cannot check it
// against a gfx950 target, so the body exists in the device pass only (the
// host pass needs no more than the kernel's signature).
template <int AUX>
__device__ __forceinline__ void lds_load16(rsrc_t r, u32x4_t *lds, uint32_t voff, uint32_t soff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, AUX);
#endif
}

// Per-thread global offsets of one k-tile's A and B chunks (the k-tile's column
// goes in the load's soffset).  The tiles travel from global memory straight
// into LDS (buffer_load ... lds, 16 bytes per lane): load q of wave w fills
// the 64 16-B slots [q*NTH + 64w, +64) of the tile, lane l the slot
// q*NTH + 64w + l, so each lane's offset names the global chunk that the
// swizzle puts in that slot.
template <bool MX, int BM, int BNT, int NTH>
struct Ptrs {
    static constexpr int NAL = BM * 8 / NTH;                    // A loads per thread and k-tile
    static constexpr int NBL = (MX ? BNT * 2 : BNT * 8) / NTH;  // B loads per thread and k-tile
    static_assert(NAL >= 1 && NBL >= 1 && BM * 8 % NTH == 0 && (MX ? BNT * 2 : BNT * 8) % NTH == 0,
                  "tile too small for the block");
    uint32_t a[NAL];  // A: tile row (tid>>3) + (NTH/8)q, chunk (tid&7) ^ swizzle(row)
    uint32_t b[NBL];  // B bf16: as A; MX: row (tid>>1) + (NTH/2)q, half (tid&1) ^ swizzle(row)
    uint32_t s;       // MX: this thread's scale row within the blob
};

// The end of a k-tile: wait until at most N of this wave's memory loads are
// outstanding (the N issued for the k-tile two ahead, so the next k-tile's
// have landed in LDS) and its LDS operations are done, then meet the other
// waves.  One asm statement with a memory clobber, so the compiler moves no
// load or LDS access across the wait or the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
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

// run(IC<n>) for n = min(nms, N): one instance of the main loop per number of
// MFMA row blocks, so the loop body has no branches on it
template <int N, typename F>
__device__ __forceinline__ void dispatch_rows(int nms, F &run)
{
    if constexpr (N == 0) {
        run(IC<0>{});
    } else {
        if (nms >= N)
            run(IC<N>{});
        else
            dispatch_rows<N - 1>(nms, run);
    }
}
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
template <int MODE, bool MX, int BM, int BNT, int MINB, int WM, int NW>
__global__ __launch_bounds__(64 * NW, MINB) void k_grouped_gemm(
    const uint64_t *__restrict__ ptrs, size_t off_w0, size_t off_w1, size_t off_s0, size_t off_s1,
    const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm, const uint16_t *__restrict__ A,
    int K, int N, int lda, int k, int E, int R, int NT, uint32_t blob_bytes, void *__restrict__ out)
{
    constexpr int NTH = 64 * NW, WN = NW / WM, WROWS = BM / WM, NMSMAX = WROWS / 32;
    constexpr int NCB = BNT / (32 * WN);  // 32-column MFMA blocks per wave
    static_assert(NW % WM == 0 && NCB >= (MODE == 1 ? 2 : 1) && NMSMAX >= 1, "wave layout");
    constexpr int BT = MX ? BNT * 2 : BNT * 8;  // 16-B slots of one B tile
    using P = Ptrs<MX, BM, BNT, NTH>;
    // loads issued per thread and k-tile: A and B chunks, and (MXFP4) the scale word
    constexpr int NLD = P::NAL + P::NBL + (MX ? 1 : 0);
    // Three LDS stages, each its own array: the compiler then sees which stage
    // an in-flight global->LDS load writes, and an LDS read of one stage does
    // not wait for the loads into another.
    __shared__ u32x4_t A0[BM * 8], A1[BM * 8], A2[BM * 8];
    __shared__ u32x4_t B0[BT], B1[BT], B2[BT];
    __shared__ float Scf[2][MX ? 2 * (BNT + 32) : 4];

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

    // A: all of x (MODE 1; under 4 GiB, checked by the launcher) or the rows from
    // the tile's first on (MODE 2); B: the blob
    const size_t abytes = MODE == 1 ? (size_t)(R / k) * lda * 2 : (size_t)(R - rb) * lda * 2;
    // Tile rows past the expert's last row load nothing: their offset lies past
    // the A resource's size, so the buffer load returns zeros without a memory
    // access (the range check takes the per-lane offset).  A resource of 2 GiB
    // or more cannot place such an offset; its pad rows re-read the last row.
    const bool a_oob = abytes < 0x80000000ull;
    // both resources under 2 GiB: an offset of 2^31 reads nothing from either
    const bool nil_ok = a_oob && blob_bytes < 0x80000000u;
    // load q of wave w fills tile rows 8 (q * NW + w) .. +7, lane l the slot of
    // row (tid >> 3) + (NTH / 8) q at position l & 7: the chunk swz puts there
    auto achunk = [](int r, int c) { return c ^ (r & 7) ^ ((r >> 3) & 1); };
    P p;
#pragma unroll
    for (int q = 0; q < P::NAL; ++q) {
        const int r = (tid >> 3) + (NTH / 8) * q, row = min(r, mrows - 1);
        const size_t arow = MODE == 1 ? (size_t)(perm[rb + row] / k) : (size_t)row;  // from abase
        p.a[q] = r < mrows || !a_oob ? (uint32_t)(arow * lda * 2 + achunk(r, tid & 7) * 16) : 0x80000000u;
    }
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
        for (int q = 0; q < P::NBL; ++q) {
            size_t so, sco;
            const int br = (tid >> 1) + (NTH / 2) * q;
            const int r = brow(br, so, sco);
            const int half = (tid & 1) ^ (((br >> 2) ^ (br >> 3)) & 1);  // mx_slot inverted
            p.b[q] = (uint32_t)(so + (size_t)r * (K / 2) + half * 16);
        }
        size_t so, sco;
        const int r = brow(tid < BNT ? tid : 0, so, sco);
        p.s = (uint32_t)(sco + (size_t)r * (K / 32));
    } else {
#pragma unroll
        for (int q = 0; q < P::NBL; ++q) {
            size_t so, sco;
            const int br = (tid >> 3) + (NTH / 8) * q;
            const int r = brow(br, so, sco);
            p.b[q] = (uint32_t)(so + (size_t)r * K * 2 + achunk(br, tid & 7) * 16);
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
    const int nk = K / BK;
    // Epilogue: wave w's staging buffer of 32 rows, carved from the stage arrays
    // (free by then) without crossing one.  MODE 2: kYst fp32 per row (rows 4
    // apart land 32 banks apart); MODE 1: kHst bf16 per row (80 B: rows 4
    // apart land 16 banks apart, a half-wave writes 16 banks).
    constexpr int kYst = 72, kHst = 40;
    constexpr int kYslots = MODE == 2 ? 32 * kYst / 4 : 32 * kHst / 8;  // 16-B slots per buffer
    constexpr int nA = BM * 8 / kYslots, nB = BT / kYslots;  // buffers per A / B stage array
    static_assert(3 * nA + 3 * nB >= NW, "LDS for the staged output");
    auto ybuf_of_wave = [&](int wv) -> float * {
        constexpr int dA = nA > 0 ? nA : 1, dB = nB > 0 ? nB : 1;
        u32x4_t *p;
        if (wv < 3 * nA) {
            p = (wv / dA == 0 ? A0 : wv / dA == 1 ? A1 : A2) + (wv % dA) * kYslots;
        } else {
            const int v = wv - 3 * nA;
            p = (v / dB == 0 ? B0 : v / dB == 1 ? B1 : B2) + (v % dB) * kYslots;
        }
        return reinterpret_cast<float *>(p);
    };

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
        // MXFP4 scale words travel through registers two k-tiles ahead and are
        // widened into Scf for the next k-tile at the end of each k-tile.
        auto sload = [&](int kt, bool real) -> uint32_t {
            (void)real;  // MXFP4 reloads the last k-tile's scales too (see dma_tile)
            return MX ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rbs, p.s, kt * 2, 0) : 0u;
        };
        auto sput = [&](uint32_t sc, float *dst) __attribute__((always_inline)) {
            if (MX && (BNT >= NTH || tid < BNT)) {
                // The empty asm keeps the widening here, after the k-tile's
                // MFMAs: left free, the compiler hoists it next to the load, and
                // waiting for that load there waits for every load issued before it.
                asm volatile("" : "+v"(sc));
#pragma unroll
                for (int gi = 0; gi < 2; ++gi)
                    dst[gi * (BNT + 32) + tid] = e8m0_f((sc >> (8 * gi)) & 0xffu);
            }
        };
        // k-tile kt of A and B into LDS stage (Ad, Bd).  bf16 gate/up weights are
        // streamed with non-temporal loads (each k-tile takes whole 128-B lines
        // of a row; 800 -> 756 us for the 4096-token layer).  MXFP4 k-tiles take
        // 32 B of a line whose rest the next three k-tiles use, and the bf16 down
        // GEMM got slower with them: default policy there.
        // real = false: a k-tile past the end, loaded only so that every k-tile
        // issues the same loads.  bf16: with resources under 2 GiB its offsets
        // lie past them, so the loads read nothing (zeros into a stage nobody
        // reads; bf16 GEMM1 +1.6% in an interleaved A/B).  MXFP4 reloads the last
        // k-tile (reading nothing was 1.4% slower there).
        auto dma_tile = [&](u32x4_t *Ad, u32x4_t *Bd, int kt, bool real) __attribute__((always_inline)) {
            const int col = kt * BK;
            const bool nil = !MX && !real && nil_ok;
#pragma unroll
            for (int q = 0; q < P::NAL; ++q)
                lds_load16<0>(ra, Ad + q * NTH + 64 * w, nil ? 0x80000000u : p.a[q], col * 2);
#pragma unroll
            for (int q = 0; q < P::NBL; ++q)
                lds_load16<(!MX && MODE == 1) ? 2 : 0>(rbs, Bd + q * NTH + 64 * w, nil ? 0x80000000u : p.b[q],
                                                       MX ? col / 2 : col * 2);
        };
        dma_tile(A0, B0, 0, true);
        const uint32_t sc0 = sload(0, true);
        dma_tile(A1, B1, min(1, nk - 1), nk > 1);
        uint32_t sc_next = sload(min(1, nk - 1), nk > 1);
        sput(sc0, Scf[0]);
        stage_barrier<NLD>();
        // One k-tile: the loads of k-tile kt+2 go out first (into the stage
        // k-tile kt-1 used), then the MFMAs of k-tile kt, then the wait for
        // k-tile kt+1.  Past the end a k-tile's loads go to a stage nobody reads
        // (reading nothing, see dma_tile), so every k-tile issues the same NLD loads.
        auto body = [&](int kt, const u32x4_t *Ac, const u32x4_t *Bc, u32x4_t *An, u32x4_t *Bn)
                        __attribute__((always_inline)) {
            const int cur = kt & 1;
            dma_tile(An, Bn, min(kt + 2, nk - 1), kt + 2 < nk);
            const uint32_t sc_new = sload(min(kt + 2, nk - 1), kt + 2 < nk);
            // issue them here, two k-tiles ahead of their use (the scheduler
            // would otherwise sink them below the MFMAs)
            asm volatile("" ::: "memory");
            if (NMS > 0) {
                float bsc[NCB];
                if (MX) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        bsc[cb] = Scf[cur][g * (BNT + 32) + brw[cb]];
                }
#pragma unroll
                for (int ks = 0; ks < BK / 16; ++ks) {
                    const int kc = 4 * g + ks;
                    bf16x8_t af[NMSMAX], bfr[NCB];
#pragma unroll
                    for (int ms = 0; ms < NMS; ++ms)
                        af[ms] = frag_bf16(Ac, wm * WROWS + ms * 32 + (l & 31), kc);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        bfr[cb] = MX ? cvt_mx8(reinterpret_cast<const uint32_t *>(Bc)[mx_slot(brw[cb], g) * 4 + ks], bsc[cb])
                                     : frag_bf16(Bc, brw[cb], kc);
#pragma unroll
                    for (int ms = 0; ms < NMS; ++ms)
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            acc[ms][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ms], bfr[cb], acc[ms][cb], 0, 0, 0);
                }
            }
            // MXFP4: the compiler's MFMA/LDS interleaving strategy for small
            // GEMM loops.  It reads each k-tile's first A fragments of all row
            // blocks at once and then keeps five reads in flight, each about
            // eight MFMAs ahead of its use (two, two MFMAs ahead, without it):
            // GEMM1 2014 -> 1949 us, GEMM2 1080 -> 1056 us in an interleaved A/B
            // on one GPU.  bf16 was about 0.7% slower with it.
            if constexpr (MX)
                __builtin_amdgcn_iglp_opt(0);
            sput(sc_next, Scf[cur ^ 1]);
            sc_next = sc_new;
            stage_barrier<NLD>();
        };
        // stage of k-tile kt = kt % 3; each call names its arrays statically
        int kt = 0;
        for (; kt + 3 <= nk; kt += 3) {
            body(kt, A0, B0, A2, B2);
            body(kt + 1, A1, B1, A0, B0);
            body(kt + 2, A2, B2, A1, B1);
        }
        if (kt < nk)
            body(kt, A0, B0, A2, B2);
        if (kt + 1 < nk)
            body(kt + 1, A1, B1, A0, B0);
        // the last loads (of k-tiles nobody reads) land before the wave moves on
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (MODE == 2) {
            // Y goes out through LDS: each wave puts one 32 x 64 fp32 block (a row
            // block of its two column fragments) in its own padded LDS buffer, then
            // reads it back by rows, 16 bytes per lane, so a store writes 256
            // contiguous bytes of each of 4 rows instead of 128 bytes of 2 (a
            // quarter of the store instructions; MXFP4 layer 3.32 -> 3.29 ms in
            // an interleaved A/B on one GPU, bf16 unchanged).  Every wave's last loads have
            // landed and every LDS read of the k-loop is done only once all waves
            // get here.
            __syncthreads();
            static_assert(NCB == 2, "staged Y: two 32-column fragments per wave");
            float *eb = ybuf_of_wave(w);
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        eb[((j >> 2) * 8 + (l >> 5) * 4 + (j & 3)) * kYst + cb * 32 + (l & 31)] = acc[ms][cb][j];
                // a wave's LDS accesses complete in order: no wait between the
                // writes and the reads, only no reordering by the compiler
                asm volatile("" ::: "memory");
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = i * 4 + (l >> 4), c4 = (l & 15) * 4;
                    const int m = wm * WROWS + ms * 32 + r;
                    const f32x4v v = *reinterpret_cast<const f32x4v *>(eb + r * kYst + c4);
                    if (m < mrows)
                        // Y is read once, by the combine: non-temporal stores
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<f32x4v *>((float *)out + (size_t)(rb + m) * N + n0 + wn * (BNT / WN) + c4));
                }
                asm volatile("" ::: "memory");
            }
            return;
        } else {
            // H (bf16, after SwiGLU) goes out the same way: a wave's 32 x 32 block
            // per row block, written to LDS 2 bytes per lane and read back by rows,
            // 16 bytes per lane (2 stores per row block instead of 16; GEMM1
            // +2.5% MXFP4, +1% bf16 in an interleaved A/B on one GPU)
            __syncthreads();
            static_assert(NCB == 2, "staged H: one gate and one up fragment per wave");
            uint16_t *hb = reinterpret_cast<uint16_t *>(ybuf_of_wave(w));
#pragma unroll
            for (int ms = 0; ms < NMS; ++ms) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    hb[((j >> 2) * 8 + (l >> 5) * 4 + (j & 3)) * kHst + (l & 31)] =
                        f_to_bf(silu_mul(acc[ms][0][j], acc[ms][1][j]));
                asm volatile("" ::: "memory");
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = i * 16 + (l >> 2), c8 = (l & 3) * 8;
                    const int m = wm * WROWS + ms * 32 + r;
                    const uint4 v = *reinterpret_cast<const uint4 *>(hb + r * kHst + c8);
                    if (m < mrows)
                        *reinterpret_cast<uint4 *>((uint16_t *)out + (size_t)(rb + m) * N + n0 + wn * (BNT / 2 / WN) + c8) = v;
                }
                asm volatile("" ::: "memory");
            }
            return;
        }
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
    dispatch_rows<NMSMAX>(nms, run);
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
// slower or spilled registers.  With the global->LDS pipeline: 4 waves of
// 320 x 64 each (one wave per SIMD, 512 registers) spilled; pinning each A
// fragment's LDS read two row blocks ahead of its MFMAs with scheduling
// groups made MXFP4 GEMM1 slower (2060 -> 2235 us).
#ifndef ECF_BF16_BNT
#define ECF_BF16_BNT 256
#define ECF_BF16_MINB 1
#define ECF_BF16_WM 2
#endif
#ifndef ECF_BF16_NW
#define ECF_BF16_NW 8
#endif
#ifndef ECF_MX_BNT
#define ECF_MX_BNT 256
#define ECF_MX_MINB 1
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
#define ECF_G1(MXV, BNV, MBV, WMV, NWV)                                                                     \
    hipLaunchKernelGGL((k_grouped_gemm<1, MXV, (MXV) ? ECF_MX_BM : kPrefillMT, BNV, MBV, WMV, NWV>), dim3(nblk), \
                       dim3(64 * (NWV)), 0, st, ex.ptrs,                                                     \
                       ex.lay.off[0], ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.tiles, o.n_tiles,         \
                       o.offsets, o.perm, (const uint16_t *)x, s.hidden, s.inter, s.hidden, s.top_k,         \
                       s.n_experts, T * s.top_k, NT, (uint32_t)ex.lay.bytes, (void *)H)
    // K = d, a multiple of the 64-element k-tile
    if (mx)
        ECF_G1(true, ECF_MX_BNT, ECF_MX_MINB, ECF_MX_WM, ECF_MX_NW);
    else
        ECF_G1(false, ECF_BF16_BNT, ECF_BF16_MINB, ECF_BF16_WM, ECF_BF16_NW);
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
#define ECF_G2(MXV, BNV, MBV, WMV, NWV)                                                                     \
    hipLaunchKernelGGL((k_grouped_gemm<2, MXV, (MXV) ? ECF_MX_BM : kPrefillMT, BNV, MBV, WMV, NWV>), dim3(nblk), \
                       dim3(64 * (NWV)), 0, st, ex.ptrs,                                                     \
                       ex.lay.off[2], ex.lay.off[2], ex.lay.off[5], ex.lay.off[5], o.tiles, o.n_tiles,         \
                       o.offsets, o.perm, H, s.inter, s.hidden, s.inter, s.top_k, s.n_experts, T * s.top_k,  \
                       NT, (uint32_t)ex.lay.bytes, (void *)Y)
    // K = I, a multiple of the 64-element k-tile on this path
    if (mx)
        ECF_G2(true, ECF_MX_BNT, ECF_MX_MINB, ECF_MX_WM, ECF_MX_NW);
    else
        ECF_G2(false, ECF_BF16_BNT, ECF_BF16_MINB, ECF_BF16_WM, ECF_BF16_NW);
#undef ECF_G2
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
