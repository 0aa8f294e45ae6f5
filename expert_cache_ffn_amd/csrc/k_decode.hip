// Decode-path expert kernels: weight-streaming GEMVs for the few rows each
// expert receives when T is small, and the fixed-order gate-weighted combine.
//
// Each block streams a band of one expert's weight rows exactly once from HBM
// and applies it to all (up to kDecodeNT per pass) routed rows of that expert.
// Lanes work in groups of 8: a group reads 8 x 16 B = 128 contiguous bytes of
// one weight row per step (one full cache line), so a wave touches 8 lines per
// load instruction.  Activations of the block's rows are staged once in LDS:
// bf16 activations with bf16 or MXFP4 weights as bf16 (they meet the weights
// in bf16-pair dot products), fp32 activations and the down projection's h as
// fp32.  The intermediate h stays fp32 on this path.
//
// Expert FFN (SwiGLU, the standard definition; the pages do not fix the expert
// form): h = silu(W_gate . v) * (W_up . v), y = W_down . h.  GPU tensor cores
// run the experts that are resident (FreeToken paper explainer, section
// "Design: two-tier expert memory"; news.ainew.jp article on FreeToken, the
// paragraph on the q* co-scheduling policy).
#include <type_traits>

#include "device_common.h"
#include "ecf_internal.h"
#include "wave_route.h"

namespace ecf {

// E8M0 scale byte -> 2^(s - 127) (s = 0: the subnormal 2^-127; 0xFF: NaN, as OCP
// MX v1.0 defines it, so the whole block's products become NaN).
__device__ __forceinline__ float e8m0_scale(uint32_t s)
{
    return __uint_as_float(s == 0 ? 0x00400000u : s == 255 ? 0x7FC00000u : (s << 23));
}

// Weight formats of the GEMV path.
enum { WF_F32 = 0, WF_BF16 = 1, WF_MX = 2 };

// Staged activation rows in LDS are padded by 4 floats after every 32, so the
// 8 lanes of a group, which read 16-byte pieces 32 (MXFP4), 8 (bf16) or 4 (fp32)
// floats apart, hit distinct banks.  A 16-byte piece never crosses a pad.
__device__ __forceinline__ int xpad(int c) { return c + ((c >> 5) << 2); }
__host__ __device__ constexpr int xpad_len(int n) { return n + (n >> 3); }

// Stage one activation row of n elements (a multiple of 8; src 16-byte aligned)
// as padded fp32 in LDS, 16 bytes per thread and load.
template <bool SRC_BF16>
__device__ __forceinline__ void stage_row(float *__restrict__ dst, const void *__restrict__ src, int n, int tid)
{
    if (SRC_BF16) {
        for (int c = tid * 8; c < n; c += 2048) {
            const uint4 v = *reinterpret_cast<const uint4 *>((const uint16_t *)src + c);
            *reinterpret_cast<float4 *>(dst + xpad(c)) = make_float4(bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y));
            *reinterpret_cast<float4 *>(dst + xpad(c + 4)) =
                make_float4(bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w));
        }
    } else {
        for (int c = tid * 4; c < n; c += 1024)
            *reinterpret_cast<float4 *>(dst + xpad(c)) = *reinterpret_cast<const float4 *>((const float *)src + c);
    }
}

// bf16 activation rows staged as bf16 (exact copies) for the dot2 path: padded
// by 8 elements (16 bytes) after every 32, so the 16-byte pieces the 8 lanes
// of a group read (64 bytes apart for MXFP4, 16 for bf16 weights) hit
// distinct banks.
__device__ __forceinline__ int xpadh(int c) { return c + ((c >> 5) << 3); }
__host__ __device__ constexpr int xpadh_len(int n) { return n + (n >> 2); }

__device__ __forceinline__ void stage_row_bf16(uint16_t *__restrict__ dst, const uint16_t *__restrict__ src, int n,
                                               int tid)
{
    for (int c = tid * 8; c < n; c += 2048)
        *reinterpret_cast<uint4 *>(dst + xpadh(c)) = *reinterpret_cast<const uint4 *>(src + c);
}

// a.lo * b.lo + a.hi * b.hi + c over bf16 pairs (products exact), fp32 sum.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// The loops below take the number of staged rows either at run time (NTC = 0:
// nt) or as a template argument (NTC = 1..kDecodeNT), and FULL = true when the
// row segment is a whole number of load batches (no piece can pass its end):
// with both fixed the unrolled loops carry no per-piece branches.  The MXFP4
// gate/up GEMV runs that way (one token, I 1024: 12.3 -> 10.2 us); the other
// GEMVs keep the run-time form, which the extra registers of the fixed one
// made slower (bf16 down 100.7 -> 102.1 us, MXFP4 down 39.1 -> 40.5 us at 16
// tokens; bf16 gate/up unchanged).

// Activation offsets below are already padded: cp = xpad(c) or xpadh(c) of the
// piece's first element c.  A piece (8 elements from c % 8 == 0, or 4) never
// crosses a pad, so element c + i sits at cp + i.  For MXFP4 each batch starts
// at a multiple of 32 (a 16-byte load holds 32 elements, and segments start at
// multiples of 32), and xpad(c0 + off) = xpad(c0) + xpad(off) for c0 % 32 == 0:
// the offsets are then one base per batch plus constants.

// part[q][i] += w-pair i . x-pair i for the 4 bf16 pairs at padded offset cp.
template <int NTC>
__device__ __forceinline__ void dot2_rows(const uint32_t (&w)[4], const uint16_t *__restrict__ xh, int ldp, int cp,
                                          int nt, float (&part)[kDecodeNT][4])
{
#pragma unroll
    for (int q = 0; q < kDecodeNT; ++q) {
        if (q < (NTC ? NTC : nt)) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xh + q * ldp + cp);
            part[q][0] = dot2(w[0], xv.x, part[q][0]);
            part[q][1] = dot2(w[1], xv.y, part[q][1]);
            part[q][2] = dot2(w[2], xv.z, part[q][2]);
            part[q][3] = dot2(w[3], xv.w, part[q][3]);
        }
    }
}

// part[q][i % 4] += w[i] * xs[q][c + i] over the nt staged rows (cp = xpad(c)).
template <int N, int NTC>
__device__ __forceinline__ void fma_rows(const float (&w)[N], const float *__restrict__ xs, int ld, int cp, int nt,
                                         float (&part)[kDecodeNT][4])
{
#pragma unroll
    for (int q = 0; q < kDecodeNT; ++q) {
        if (q < (NTC ? NTC : nt)) {
            const float *xp = xs + q * xpad_len(ld);
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                const float4 xv = *reinterpret_cast<const float4 *>(xp + cp + i);
                part[q][0] = fmaf(w[i], xv.x, part[q][0]);
                part[q][1] = fmaf(w[i + 1], xv.y, part[q][1]);
                part[q][2] = fmaf(w[i + 2], xv.z, part[q][2]);
                part[q][3] = fmaf(w[i + 3], xv.w, part[q][3]);
            }
        }
    }
}

// One lane's share of a weight row segment [kbeg, kend), held in registers: a
// 16-byte load holds V weights (f32 4, bf16 8, MXFP4 32 = one E8M0 scale
// group, whose scale byte srow[c / 32] is loaded beside it); a group of 8
// lanes covers 8*V elements per load and UNR loads.  MXFP4 elements are
// expanded to fp32 by v_cvt_scalef32_pk_f32_fp4 (element 2i in the low nibble
// of byte i; the power-of-two scale is applied exactly).
// a 16-byte MXFP4 load feeds 4x the arithmetic of a bf16 one, so it takes
// twice the loads in flight
template <int WF>
constexpr int kRowUnr = WF == WF_MX ? 8 : 4;

template <int WF, int UNR_ = kRowUnr<WF>>
struct RowRegs {
    static constexpr int V = WF == WF_MX ? 32 : WF == WF_BF16 ? 8 : 4;
    static constexpr int UNR = UNR_;
    static constexpr int SPAN = 8 * V * UNR;  // elements one group covers per batch
    uint4 wv[UNR];
    uint32_t sb[UNR];

    template <bool FULL>
    __device__ __forceinline__ void load(const void *__restrict__ wrow, const uint8_t *__restrict__ srow, int c0,
                                         int kend)
    {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * 8 * V;
            if (FULL || c < kend) {
                const size_t byte = WF == WF_MX ? (size_t)c / 2 : (size_t)c * (WF == WF_BF16 ? 2 : 4);
                wv[u] = ld_nt16((const char *)wrow + byte);
                if (WF == WF_MX)
                    sb[u] = srow[c / 32];
            }
        }
    }

    template <int NTC, bool FULL>
    __device__ __forceinline__ void apply(const float *__restrict__ xs, int ld, int c0, int kend, int nt,
                                          float (&part)[kDecodeNT][4]) const
    {
        const int xb = xpad(c0);  // MXFP4: c0 % 32 == 0
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * 8 * V;
            if (!FULL && c >= kend)
                break;
            const uint32_t p[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            if (WF == WF_MX) {
                const float sc = e8m0_scale(sb[u]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {  // 8 elements per dword
                    const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[i], sc, 0);
                    const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[i], sc, 1);
                    const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[i], sc, 2);
                    const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[i], sc, 3);
                    const float wf[8] = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
                    fma_rows<8, NTC>(wf, xs, ld, xb + xpad(u * 8 * V + 8 * i), nt, part);
                }
            } else if (WF == WF_BF16) {
                float wf[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wf[2 * i] = bf_lo(p[i]);
                    wf[2 * i + 1] = bf_hi(p[i]);
                }
                fma_rows<8, NTC>(wf, xs, ld, xpad(c), nt, part);
            } else {
                float wf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    wf[i] = __uint_as_float(p[i]);
                fma_rows<4, NTC>(wf, xs, ld, xpad(c), nt, part);
            }
        }
    }

    // Same sums against bf16-staged activations with bf16-pair dot products
    // (bf16 or MXFP4 weights; MXFP4 expands to bf16 pairs, exactly).
    template <int NTC, bool FULL>
    __device__ __forceinline__ void apply2(const uint16_t *__restrict__ xh, int ldp, int c0, int kend, int nt,
                                           float (&part)[kDecodeNT][4]) const
    {
        const int xb = xpadh(c0);  // MXFP4: c0 % 32 == 0
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * 8 * V;
            if (!FULL && c >= kend)
                break;
            const uint32_t p[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
            if (WF == WF_MX) {
                const float sc = e8m0_scale(sb[u]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {  // 8 elements per dword
                    const uint32_t w[4] = {
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[i], sc, 0)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[i], sc, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[i], sc, 2)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[i], sc, 3))};
                    dot2_rows<NTC>(w, xh, ldp, xb + xpadh(u * 8 * V + 8 * i), nt, part);
                }
            } else {
                dot2_rows<NTC>(p, xh, ldp, xpadh(c), nt, part);
            }
        }
    }
};

// Dot products of one weight row segment [kbeg, kend) against nt staged rows;
// the segment streams through registers one batch of UNR loads at a time.
// Each row keeps 4 independent partial sums (element i of every 4 goes to
// sum i), so the FMA chains are a quarter as long.
template <int WF, int NTC, bool FULL>
__device__ __forceinline__ void row_dots(const void *__restrict__ wrow, const uint8_t *__restrict__ srow,
                                         const float *__restrict__ xs, int ld, int kbeg, int kend, int sub, int nt,
                                         float acc[kDecodeNT])
{
    RowRegs<WF> rr;
    float part[kDecodeNT][4] = {};
    for (int c = kbeg + sub * RowRegs<WF>::V; c < kend; c += RowRegs<WF>::SPAN) {
        rr.template load<FULL>(wrow, srow, c, kend);
        rr.template apply<NTC, FULL>(xs, ld, c, kend, nt, part);
    }
#pragma unroll
    for (int q = 0; q < kDecodeNT; ++q)
        acc[q] += (part[q][0] + part[q][1]) + (part[q][2] + part[q][3]);
}

// The activation piece each 4 (fp32) or 8 (bf16-pair) weights meet is the same
// for every row of a group, so the multi-row forms below read it from LDS once
// and apply it to all RPG rows.  Each row's partial sums see exactly the
// sequence of operations of the one-row form.
// Weights of 16-B piece u of a row as fp32, 8 at a time (MXFP4: dword pc).
template <int WF, int UNR>
__device__ __forceinline__ void piece_f32(const RowRegs<WF, UNR> &rr, int u, int pc, float (&wf)[8])
{
    const uint32_t p[4] = {rr.wv[u].x, rr.wv[u].y, rr.wv[u].z, rr.wv[u].w};
    if (WF == WF_MX) {
        const float sc = e8m0_scale(rr.sb[u]);
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[pc], sc, 0);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[pc], sc, 1);
        const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[pc], sc, 2);
        const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p[pc], sc, 3);
        wf[0] = v0[0], wf[1] = v0[1], wf[2] = v1[0], wf[3] = v1[1];
        wf[4] = v2[0], wf[5] = v2[1], wf[6] = v3[0], wf[7] = v3[1];
    } else if (WF == WF_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wf[2 * i] = bf_lo(p[i]);
            wf[2 * i + 1] = bf_hi(p[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            wf[i] = __uint_as_float(p[i]);
    }
}

// apply() of RPG rows at once against fp32-staged activations.
template <int WF, int RPG, int UNR, int NTC, bool FULL>
__device__ __forceinline__ void apply_rows(const RowRegs<WF, UNR> (&rr)[RPG], const float *__restrict__ xs, int ld,
                                           int c0, int kend, int nt, float (&part)[RPG][kDecodeNT][4])
{
    const int xb = xpad(c0);  // MXFP4: c0 % 32 == 0
    constexpr int V = RowRegs<WF, UNR>::V;
    constexpr int NP = WF == WF_MX ? 4 : 1;                       // pieces per 16-B load
    constexpr int NE = WF == WF_MX ? 8 : (WF == WF_BF16 ? 8 : 4);  // weights per piece
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * 8 * V;
        if (!FULL && c >= kend)
            break;
#pragma unroll
        for (int pc = 0; pc < NP; ++pc) {
            float wf[RPG][8];
#pragma unroll
            for (int r = 0; r < RPG; ++r)
                piece_f32(rr[r], u, pc, wf[r]);
#pragma unroll
            for (int q = 0; q < kDecodeNT; ++q) {
                if (q < (NTC ? NTC : nt)) {
                    const float *xp = xs + q * xpad_len(ld);
#pragma unroll
                    for (int i = 0; i < NE; i += 4) {
                        const float4 xv = *reinterpret_cast<const float4 *>(
                            xp + (WF == WF_MX ? xb + xpad(u * 8 * V + 8 * pc) : xpad(c + 8 * pc)) + i);
#pragma unroll
                        for (int r = 0; r < RPG; ++r) {
                            part[r][q][0] = fmaf(wf[r][i], xv.x, part[r][q][0]);
                            part[r][q][1] = fmaf(wf[r][i + 1], xv.y, part[r][q][1]);
                            part[r][q][2] = fmaf(wf[r][i + 2], xv.z, part[r][q][2]);
                            part[r][q][3] = fmaf(wf[r][i + 3], xv.w, part[r][q][3]);
                        }
                    }
                }
            }
        }
    }
}

// apply2() of RPG rows at once against bf16-staged activations.
template <int WF, int RPG, int UNR, int NTC, bool FULL>
__device__ __forceinline__ void apply2_rows(const RowRegs<WF, UNR> (&rr)[RPG], const uint16_t *__restrict__ xh,
                                            int ldp, int c0, int kend, int nt, float (&part)[RPG][kDecodeNT][4])
{
    const int xb = xpadh(c0);  // MXFP4: c0 % 32 == 0
    constexpr int V = RowRegs<WF, UNR>::V;
    constexpr int NP = WF == WF_MX ? 4 : 1;  // pieces of 8 elements per 16-B load
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int c = c0 + u * 8 * V;
        if (!FULL && c >= kend)
            break;
#pragma unroll
        for (int pc = 0; pc < NP; ++pc) {
            uint32_t w[RPG][4];
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                const uint32_t p[4] = {rr[r].wv[u].x, rr[r].wv[u].y, rr[r].wv[u].z, rr[r].wv[u].w};
                if (WF == WF_MX) {
                    const float sc = e8m0_scale(rr[r].sb[u]);
                    w[r][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[pc], sc, 0));
                    w[r][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[pc], sc, 1));
                    w[r][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[pc], sc, 2));
                    w[r][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(p[pc], sc, 3));
                } else {
                    w[r][0] = p[0], w[r][1] = p[1], w[r][2] = p[2], w[r][3] = p[3];
                }
            }
#pragma unroll
            for (int q = 0; q < kDecodeNT; ++q) {
                if (q < (NTC ? NTC : nt)) {
                    const uint4 xv = *reinterpret_cast<const uint4 *>(
                        xh + q * ldp + (WF == WF_MX ? xb + xpadh(u * 8 * V + 8 * pc) : xpadh(c + 8 * pc)));
#pragma unroll
                    for (int r = 0; r < RPG; ++r) {
                        part[r][q][0] = dot2(w[r][0], xv.x, part[r][q][0]);
                        part[r][q][1] = dot2(w[r][1], xv.y, part[r][q][1]);
                        part[r][q][2] = dot2(w[r][2], xv.z, part[r][q][2]);
                        part[r][q][3] = dot2(w[r][3], xv.w, part[r][q][3]);
                    }
                }
            }
        }
    }
}

// row_dots over RPG rows at once: each batch's loads for every row are issued
// before any of them is used (RPG times the loads in flight), then the rows
// meet the staged activations together, each piece read from LDS once for all
// RPG rows (MXFP4 down at 16 tokens 50 -> 41 us, its LDS reads a quarter).
template <int WF, int RPG, int NTC, bool FULL>
__device__ __forceinline__ void row_dots_multi(const char *const (&wrow)[RPG], const uint8_t *const (&srow)[RPG],
                                               const float *__restrict__ xs, int ld, int kbeg, int kend, int sub,
                                               int nt, float (&acc)[RPG][kDecodeNT])
{
    // the loads in flight per lane stay those of one row in row_dots
    using Regs = RowRegs<WF, (kRowUnr<WF> / RPG > 0 ? kRowUnr<WF> / RPG : 1)>;
    Regs rr[RPG];
    float part[RPG][kDecodeNT][4] = {};
    for (int c = kbeg + sub * Regs::V; c < kend; c += Regs::SPAN) {
#pragma unroll
        for (int r = 0; r < RPG; ++r)
            rr[r].template load<FULL>(wrow[r], srow[r], c, kend);
        apply_rows<WF, RPG, Regs::UNR, NTC, FULL>(rr, xs, ld, c, kend, nt, part);
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r)
#pragma unroll
        for (int q = 0; q < kDecodeNT; ++q)
            acc[r][q] += (part[r][q][0] + part[r][q][1]) + (part[r][q][2] + part[r][q][3]);
}

// row_dots2 over RPG rows at once (as row_dots_multi).
template <int WF, int RPG, int NTC, bool FULL>
__device__ __forceinline__ void row_dots2_multi(const char *const (&wrow)[RPG], const uint8_t *const (&srow)[RPG],
                                                const uint16_t *__restrict__ xh, int ldp, int kbeg, int kend,
                                                int sub, int nt, float (&acc)[RPG][kDecodeNT])
{
    using Regs = RowRegs<WF, (kRowUnr<WF> / RPG > 0 ? kRowUnr<WF> / RPG : 1)>;
    Regs rr[RPG];
    float part[RPG][kDecodeNT][4] = {};
    for (int c = kbeg + sub * Regs::V; c < kend; c += Regs::SPAN) {
#pragma unroll
        for (int r = 0; r < RPG; ++r)
            rr[r].template load<FULL>(wrow[r], srow[r], c, kend);
        apply2_rows<WF, RPG, Regs::UNR, NTC, FULL>(rr, xh, ldp, c, kend, nt, part);
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r)
#pragma unroll
        for (int q = 0; q < kDecodeNT; ++q)
            acc[r][q] += (part[r][q][0] + part[r][q][1]) + (part[r][q][2] + part[r][q][3]);
}

// row_dots against bf16-staged activations (bf16 or MXFP4 weights).
template <int WF, int NTC, bool FULL>
__device__ __forceinline__ void row_dots2(const void *__restrict__ wrow, const uint8_t *__restrict__ srow,
                                          const uint16_t *__restrict__ xh, int ldp, int kbeg, int kend, int sub,
                                          int nt, float acc[kDecodeNT])
{
    RowRegs<WF> rr;
    float part[kDecodeNT][4] = {};
    for (int c = kbeg + sub * RowRegs<WF>::V; c < kend; c += RowRegs<WF>::SPAN) {
        rr.template load<FULL>(wrow, srow, c, kend);
        rr.template apply2<NTC, FULL>(xh, ldp, c, kend, nt, part);
    }
#pragma unroll
    for (int q = 0; q < kDecodeNT; ++q)
        acc[q] += (part[q][0] + part[q][1]) + (part[q][2] + part[q][3]);
}

// f(integral_constant<int, nt>, bool_constant<full>) for nt in 1..kDecodeNT
template <typename F>
__device__ __forceinline__ void dispatch_rows_full(int nt, bool full, F &f)
{
    static_assert(kDecodeNT == 2, "one instance per row count");
    if (nt >= 2) {
        if (full)
            f(std::integral_constant<int, 2>{}, std::true_type{});
        else
            f(std::integral_constant<int, 2>{}, std::false_type{});
    } else {
        if (full)
            f(std::integral_constant<int, 1>{}, std::true_type{});
        else
            f(std::integral_constant<int, 1>{}, std::false_type{});
    }
}

// gate/up + SwiGLU.  Block = IB intermediate rows (gate and up) of one active
// expert, split into KP parts along d.  grid = (I / IB, max active experts).
// bf16 activations with bf16 or MXFP4 weights stay bf16 in LDS and meet the
// weights in bf16-pair dot products (half the LDS reads and FMA instructions of
// the fp32 form; every product is exact either way).
// The 16-row MXFP4 form asks for four waves per SIMD (at most 128 registers):
// left free it took 131 and ran three (16 tokens: 69.9 against 65.4 us).
template <int WF, bool ABF, int IB, int KP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WF == WF_MX && IB >= 16 ? 4 : 1))) void k_decode_gateup(
    const uint64_t *__restrict__ ptrs, size_t off_gate, size_t off_up, size_t off_sgate, size_t off_sup,
    const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const void *__restrict__ x, int d, int I, int k, int E, int R, int ntp, float *__restrict__ H)
{
    // 32 groups of 8 lanes over the block's 2*IB rows (gate, then up) x KP parts;
    // with RPG = 2 a group takes gate row i and up row i together
    static_assert((2 * IB * KP) % 32 == 0 && 2 * IB * KP / 32 <= 2, "32 groups of 8 lanes per block");
    constexpr int RPG = 2 * IB * KP / 32, OG = 2 * IB / RPG;
    constexpr bool DOT2 = ABF && WF != WF_F32;
    static_assert(RPG == 1 || DOT2, "two rows per group only on the bf16-pair path");
    // elements a group covers per batch of loads (as row_dots2_multi / row_dots2 / row_dots take them)
    constexpr int kSpan = RPG > 1 ? RowRegs<WF, (kRowUnr<WF> / RPG > 0 ? kRowUnr<WF> / RPG : 1)>::SPAN : RowRegs<WF>::SPAN;
    // [min(kDecodeNT, T)][xpadh_len(d)] bf16 (DOT2) or [..][xpad_len(d)] fp32; an expert has at most T rows
    extern __shared__ float xs[];
    uint16_t *xh = reinterpret_cast<uint16_t *>(xs);
    __shared__ float red[KP][2 * IB][kDecodeNT];
    if ((int)blockIdx.y >= *n_active)
        return;
    const int e = active[blockIdx.y];
    if ((unsigned)e >= (unsigned)E)  // routing metadata is produced on the device; never index past it
        return;
    const uint64_t blob = ptrs[e];
    const int r0 = offsets[e], ne = offsets[e + 1] - r0;
    if (!blob || r0 < 0 || ne <= 0 || r0 + ne > R)
        return;
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 7;
    const int g = tid >> 3;  // group 0..31
    const int rho = g % OG, kap = g / OG;
    const int i0 = blockIdx.x * IB;
    const char *wrow[RPG];
    const uint8_t *srow[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {  // block rows rho, rho + OG: row < IB is gate, else up
        const int br = rho + r * OG;
        const size_t sec = br < IB ? off_gate : off_up;
        const size_t ssec = br < IB ? off_sgate : off_sup;
        const int irow = i0 + (br % IB);
        wrow[r] = (const char *)blob + sec +
                  (WF == WF_MX ? (size_t)irow * d / 2 : (size_t)irow * d * (WF == WF_BF16 ? 2 : 4));
        srow[r] = (const uint8_t *)blob + ssec + (size_t)irow * (d / 32);
    }
    const int Lk = d / KP, kbeg = kap * Lk, kend = kbeg + Lk;
    for (int tp = 0; tp < ne; tp += ntp) {
        const int nt = min(ntp, ne - tp);
        for (int q = 0; q < nt; ++q) {
            const size_t t = (size_t)(perm[r0 + tp + q] / k);
            if (DOT2)
                stage_row_bf16(xh + q * xpadh_len(d), (const uint16_t *)x + t * d, d, tid);
            else
                stage_row<ABF>(xs + q * xpad_len(d), ABF ? (const void *)((const uint16_t *)x + t * d)
                                                         : (const void *)((const float *)x + t * d), d, tid);
        }
        __syncthreads();
        {
            float acc[RPG][kDecodeNT] = {};
            auto dots = [&](auto ntc, auto fullc) __attribute__((always_inline)) {
                constexpr int NTC = decltype(ntc)::value;
                constexpr bool FULL = decltype(fullc)::value;
                if (RPG > 1)
                    row_dots2_multi<WF, RPG, NTC, FULL>(wrow, srow, xh, xpadh_len(d), kbeg, kend, sub, nt, acc);
                else if (DOT2)
                    row_dots2<WF, NTC, FULL>(wrow[0], srow[0], xh, xpadh_len(d), kbeg, kend, sub, nt, acc[0]);
                else
                    row_dots<WF, NTC, FULL>(wrow[0], srow[0], xs, d, kbeg, kend, sub, nt, acc[0]);
            };
            if (WF == WF_MX)
                dispatch_rows_full(nt, Lk % kSpan == 0, dots);
            else
                dots(std::integral_constant<int, 0>{}, std::false_type{});
#pragma unroll
            for (int r = 0; r < RPG; ++r)
#pragma unroll
                for (int q = 0; q < kDecodeNT; ++q) {
                    acc[r][q] += __shfl_xor(acc[r][q], 1, 64);
                    acc[r][q] += __shfl_xor(acc[r][q], 2, 64);
                    acc[r][q] += __shfl_xor(acc[r][q], 4, 64);
                }
            if (sub == 0)
#pragma unroll
                for (int r = 0; r < RPG; ++r)
#pragma unroll
                    for (int q = 0; q < kDecodeNT; ++q)
                        red[kap][rho + r * OG][q] = acc[r][q];
            __syncthreads();
            for (int t2 = tid; t2 < IB * nt; t2 += 256) {
                const int il = t2 % IB, q = t2 / IB;
                float a = 0.f, b = 0.f;
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    a += red[p][il][q];
                    b += red[p][IB + il][q];
                }
                H[(size_t)(r0 + tp + q) * I + i0 + il] = silu_mul(a, b);
            }
            __syncthreads();
        }
    }
}

// gate/up + SwiGLU at one token, every expert resident, with the routing done
// in the kernel itself: no routing kernel (and no launch) sits between the
// router GEMV and this one.  Every block takes the token's top-k from the
// logits by one wave (the routing kernels' top-k, so the same experts, order
// and gates) while its other waves stage x.  At one token the routed rows are
// the k selected experts in ascending id: row r is the r-th smallest selected
// expert, and its slot f = j is the position of that expert in the top-k list.
// The blocks are persistent: item = r * (I / IB) + column block, strided by the
// grid, each computed as one block of k_decode_gateup computes its rows.
// Block 0 also writes the routing tables the down projection and the combine
// read, with the values the routing kernel gives them at one token.
template <int WF, int IB, int KP, int MAXS>
__global__ __launch_bounds__(256) void k_decode_gateup_route1(
    const float *__restrict__ logits, int E, int k, int renorm, const uint64_t *__restrict__ ptrs,
    size_t off_gate, size_t off_up, size_t off_sgate, size_t off_sup, const uint16_t *__restrict__ x, int d,
    int I, int32_t *__restrict__ idx, float *__restrict__ gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ pos,
    int32_t *__restrict__ active, int32_t *__restrict__ n_active, int32_t *__restrict__ tiles,
    int32_t *__restrict__ n_tiles, float *__restrict__ H)
{
    static_assert(WF != WF_F32, "bf16-pair path only");
    static_assert((2 * IB * KP) % 32 == 0 && 2 * IB * KP / 32 <= 2, "32 groups of 8 lanes per block");
    constexpr int RPG = 2 * IB * KP / 32, OG = 2 * IB / RPG;
    constexpr int kSpan = RPG > 1 ? RowRegs<WF, (kRowUnr<WF> / RPG > 0 ? kRowUnr<WF> / RPG : 1)>::SPAN
                                  : RowRegs<WF>::SPAN;
    extern __shared__ float xs[];  // [xpadh_len(d)] bf16
    uint16_t *xh = reinterpret_cast<uint16_t *>(xs);
    __shared__ float red[KP][2 * IB][kDecodeNT];
    __shared__ int32_t sid[32];  // top-k experts, j order (k <= 32)
    __shared__ float sg[32];
    __shared__ int sexp[32];     // selected experts in ascending id: the row order
    __shared__ int srank[32];    // row of slot j
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        topk_wave<MAXS>(logits, E, k, renorm, lane, sid, sg, nullptr);
    } else {
        for (int c = (tid - 64) * 8; c < d; c += 192 * 8)
            *reinterpret_cast<uint4 *>(xh + xpadh(c)) = *reinterpret_cast<const uint4 *>(x + c);
    }
    __syncthreads();
    if (tid < k) {
        const int e = sid[tid];
        int r = 0;
        for (int j = 0; j < k; ++j)
            r += sid[j] < e;
        srank[tid] = r;
        sexp[r] = e;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        if (tid < k) {
            const int r = srank[tid];
            idx[tid] = sid[tid];
            gate[tid] = sg[tid];
            pos[tid] = r;
            perm[r] = tid;
            active[r] = sexp[r];
            tiles[2 * r] = sexp[r];
            tiles[2 * r + 1] = 0;
        }
        for (int e = tid; e < E; e += 256) {
            int c = 0, below = 0;
            for (int j = 0; j < k; ++j) {
                c += sid[j] == e;
                below += sid[j] < e;
            }
            counts[e] = c;
            offsets[e] = below;
        }
        if (tid == 0) {
            offsets[E] = k;
            *n_active = k;
            *n_tiles = k;
        }
    }
    const int g = tid >> 3, sub = lane & 7;
    const int rho = g % OG, kap = g / OG;
    const int Lk = d / KP, kbeg = kap * Lk, kend = kbeg + Lk;
    const bool full = Lk % kSpan == 0;
    const int nb = I / IB, items = k * nb;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int r = it / nb, i0 = (it - r * nb) * IB;
        const int e = sexp[r];
        if ((unsigned)e >= (unsigned)E)
            continue;
        const uint64_t blob = ptrs[e];
        if (!blob)
            continue;
        const char *wrow[RPG];
        const uint8_t *srow[RPG];
#pragma unroll
        for (int q = 0; q < RPG; ++q) {  // block rows rho, rho + OG: row < IB is gate, else up
            const int br = rho + q * OG;
            const size_t sec = br < IB ? off_gate : off_up;
            const size_t ssec = br < IB ? off_sgate : off_sup;
            const int irow = i0 + (br % IB);
            wrow[q] = (const char *)blob + sec + (WF == WF_MX ? (size_t)irow * d / 2 : (size_t)irow * d * 2);
            srow[q] = (const uint8_t *)blob + ssec + (size_t)irow * (d / 32);
        }
        float acc[RPG][kDecodeNT] = {};
        auto dots = [&](auto fullc) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(fullc)::value;
            if (RPG > 1)
                row_dots2_multi<WF, RPG, 1, FULL>(wrow, srow, xh, xpadh_len(d), kbeg, kend, sub, 1, acc);
            else
                row_dots2<WF, 1, FULL>(wrow[0], srow[0], xh, xpadh_len(d), kbeg, kend, sub, 1, acc[0]);
        };
        if (full)
            dots(std::true_type{});
        else
            dots(std::false_type{});
#pragma unroll
        for (int q = 0; q < RPG; ++q) {
            acc[q][0] += __shfl_xor(acc[q][0], 1, 64);
            acc[q][0] += __shfl_xor(acc[q][0], 2, 64);
            acc[q][0] += __shfl_xor(acc[q][0], 4, 64);
        }
        if (sub == 0)
#pragma unroll
            for (int q = 0; q < RPG; ++q)
                red[kap][rho + q * OG][0] = acc[q][0];
        __syncthreads();
        if (tid < IB) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                a += red[p][tid][0];
                b += red[p][IB + tid][0];
            }
            H[(size_t)r * I + i0 + tid] = silu_mul(a, b);
        }
        __syncthreads();
    }
}

// down projection: Y[r][o] = W_down[e][o] . h[r].  Block = OB output rows of
// one active expert, KP parts along I.  grid = (d / OB, max active experts).
template <int WF, int OB, int KP>
__global__ __launch_bounds__(256) void k_decode_down(
    const uint64_t *__restrict__ ptrs, size_t off_down, size_t off_sdown, const int32_t *__restrict__ active,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const float *__restrict__ H, int d, int I, int E, int R, int ntp, float *__restrict__ Y)
{
    // 32 groups of 8 lanes; KP groups share a row; each group takes RPG rows
    static_assert((OB * KP) % 32 == 0, "32 groups of 8 lanes per block");
    constexpr int RPG = OB * KP / 32, OG = OB / RPG;
    extern __shared__ float hs[];  // [min(kDecodeNT, T)][xpad_len(I)]
    __shared__ float red[KP][OB][kDecodeNT];
    if ((int)blockIdx.y >= *n_active)
        return;
    const int e = active[blockIdx.y];
    if ((unsigned)e >= (unsigned)E)
        return;
    const uint64_t blob = ptrs[e];
    const int r0 = offsets[e], ne = offsets[e + 1] - r0;
    if (!blob || r0 < 0 || ne <= 0 || r0 + ne > R)
        return;
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 7;
    const int g = tid >> 3;
    const int rho = g % OG, kap = g / OG;
    const int o0 = blockIdx.x * OB;
    const char *wrow[RPG];
    const uint8_t *srow[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {  // this group's rows rho, rho + OG, ...
        const size_t orow = (size_t)(o0 + rho + r * OG);
        wrow[r] = (const char *)blob + off_down +
                  (WF == WF_MX ? orow * I / 2 : orow * I * (WF == WF_BF16 ? 2 : 4));
        srow[r] = (const uint8_t *)blob + off_sdown + orow * (I / 32);
    }
    const int Lk = I / KP, kbeg = kap * Lk, kend = kbeg + Lk;
    for (int tp = 0; tp < ne; tp += ntp) {
        const int nt = min(ntp, ne - tp);
        for (int q = 0; q < nt; ++q)
            for (int c = tid * 4; c < I; c += 1024)  // I is a multiple of 64: whole float4s
                *reinterpret_cast<float4 *>(hs + q * xpad_len(I) + xpad(c)) =
                    *reinterpret_cast<const float4 *>(H + (size_t)(r0 + tp + q) * I + c);
        __syncthreads();
        {
            float acc[RPG][kDecodeNT] = {};
            auto dots = [&](auto ntc, auto fullc) __attribute__((always_inline)) {
                constexpr int NTC = decltype(ntc)::value;
                constexpr bool FULL = decltype(fullc)::value;
                if (RPG == 1)
                    row_dots<WF, NTC, FULL>(wrow[0], srow[0], hs, I, kbeg, kend, sub, nt, acc[0]);
                else
                    row_dots_multi<WF, RPG, NTC, FULL>(wrow, srow, hs, I, kbeg, kend, sub, nt, acc);
            };
            dots(std::integral_constant<int, 0>{}, std::false_type{});
#pragma unroll
            for (int r = 0; r < RPG; ++r)
#pragma unroll
                for (int q = 0; q < kDecodeNT; ++q) {
                    acc[r][q] += __shfl_xor(acc[r][q], 1, 64);
                    acc[r][q] += __shfl_xor(acc[r][q], 2, 64);
                    acc[r][q] += __shfl_xor(acc[r][q], 4, 64);
                }
            if (sub == 0)
#pragma unroll
                for (int r = 0; r < RPG; ++r)
#pragma unroll
                    for (int q = 0; q < kDecodeNT; ++q)
                        red[kap][rho + r * OG][q] = acc[r][q];
            __syncthreads();
            for (int i = tid; i < OB * nt; i += 256) {
                const int ol = i % OB, q = i / OB;
                float sum = 0.f;
#pragma unroll
                for (int p = 0; p < KP; ++p)
                    sum += red[p][ol][q];
                Y[(size_t)(r0 + tp + q) * d + o0 + ol] = sum;
            }
            __syncthreads();
        }
    }
}

// Down projection and combine of one token: T = 1, so each of the R = k <= 8
// routed rows has its own expert and row j is the token's j-th expert.  Block =
// OB output rows of every routed expert, split into KP = 32 / OB parts along I;
// grid = d / OB.  Each lane issues its first batch of loads for all k rows
// before it stages h, so the weight stream starts as soon as the experts are
// known.  out[o] = residual[o] + sum over j ascending of gate[j] *
// (W_down[e_j][o] . h_j): k_combine's fixed-order sum, with no Y in memory.
template <int WF, int OB, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_decode_down_combine1(
    const uint64_t *__restrict__ ptrs, size_t off_down, size_t off_sdown, const int32_t *__restrict__ idx,
    const float *__restrict__ gate, const int32_t *__restrict__ pos, const float *__restrict__ H, int d, int I,
    int k, int E, const float *residual, float *out, void *out_act)
{
    constexpr int KP = 32 / OB;
    constexpr int V = WF == WF_MX ? 32 : 8;  // elements per 16-byte load
    constexpr int UB = WF == WF_MX ? 1 : 2;  // loads per row in one batch
    extern __shared__ float hs[];            // [k][xpad_len(I)] fp32
    __shared__ float red[KP][OB][8];
    __shared__ uint64_t sblob[8];
    __shared__ float sg[8];
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 7, g = tid >> 3;
    const int o0 = blockIdx.x * OB;
    if (tid < k) {
        const int e = idx[tid], p = pos[tid];
        const bool ok = (unsigned)e < (unsigned)E && (unsigned)p < (unsigned)k;
        sblob[tid] = ok ? ptrs[e] : 0ull;
        sg[tid] = gate[tid];
    }
    __syncthreads();
    const int ol = g % OB, part = g / OB;
    const int Lk = I / KP, kb = part * Lk, ke = kb + Lk;
    const size_t orow = (size_t)(o0 + ol);
    const char *row[8];
    const uint8_t *srow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t b = j < k ? sblob[j] : 0ull;
        row[j] = b ? (const char *)b + off_down + (WF == WF_MX ? orow * I / 2 : orow * I * 2) : nullptr;
        srow[j] = b ? (const uint8_t *)b + off_sdown + orow * (I / 32) : nullptr;
    }
    uint4 wv[8][UB];
    uint32_t sb[8][UB];
    auto load = [&](int c0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (row[j]) {
#pragma unroll
                for (int u = 0; u < UB; ++u) {
                    const int c = c0 + u * 8 * V;
                    if (c < ke) {
                        wv[j][u] = ld_nt16(row[j] + (WF == WF_MX ? (size_t)c / 2 : (size_t)c * 2));
                        if (WF == WF_MX)
                            sb[j][u] = srow[j][c / 32];
                    }
                }
            }
        }
    };
    int c0 = kb + sub * V;
    if (c0 < ke)
        load(c0);
    for (int j = 0; j < k; ++j) {
        const int p = min(max(pos[j], 0), k - 1);
        for (int c = tid * 4; c < I; c += 1024)  // I is a multiple of 64: whole float4s
            *reinterpret_cast<float4 *>(hs + j * xpad_len(I) + xpad(c)) =
                *reinterpret_cast<const float4 *>(H + (size_t)p * I + c);
    }
    __syncthreads();
    float pj[8][4] = {};
    for (; c0 < ke; c0 += 8 * V * UB) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (row[j]) {
                const float *hj = hs + j * xpad_len(I);
#pragma unroll
                for (int u = 0; u < UB; ++u) {
                    const int c = c0 + u * 8 * V;
                    if (c >= ke)
                        break;
                    const uint32_t pw[4] = {wv[j][u].x, wv[j][u].y, wv[j][u].z, wv[j][u].w};
#pragma unroll
                    for (int i = 0; i < (WF == WF_MX ? 4 : 1); ++i) {
                        float wf[8];
                        if (WF == WF_MX) {
                            const float sc = e8m0_scale(sb[j][u]);
                            const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[i], sc, 0);
                            const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[i], sc, 1);
                            const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[i], sc, 2);
                            const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(pw[i], sc, 3);
                            wf[0] = v0[0], wf[1] = v0[1], wf[2] = v1[0], wf[3] = v1[1];
                            wf[4] = v2[0], wf[5] = v2[1], wf[6] = v3[0], wf[7] = v3[1];
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                wf[2 * q] = bf_lo(pw[q]);
                                wf[2 * q + 1] = bf_hi(pw[q]);
                            }
                        }
                        const int ce = c + 8 * i;
                        const float4 h0 = *reinterpret_cast<const float4 *>(hj + xpad(ce));
                        const float4 h1 = *reinterpret_cast<const float4 *>(hj + xpad(ce + 4));
                        pj[j][0] = fmaf(wf[0], h0.x, pj[j][0]);
                        pj[j][1] = fmaf(wf[1], h0.y, pj[j][1]);
                        pj[j][2] = fmaf(wf[2], h0.z, pj[j][2]);
                        pj[j][3] = fmaf(wf[3], h0.w, pj[j][3]);
                        pj[j][0] = fmaf(wf[4], h1.x, pj[j][0]);
                        pj[j][1] = fmaf(wf[5], h1.y, pj[j][1]);
                        pj[j][2] = fmaf(wf[6], h1.z, pj[j][2]);
                        pj[j][3] = fmaf(wf[7], h1.w, pj[j][3]);
                    }
                }
            }
        }
        if (c0 + 8 * V * UB < ke)
            load(c0 + 8 * V * UB);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float a = (pj[j][0] + pj[j][1]) + (pj[j][2] + pj[j][3]);
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        if (sub == 0)
            red[part][ol][j] = a;
    }
    __syncthreads();
    if (tid < OB) {
        const size_t o = (size_t)o0 + tid;
        float s = 0.f;
        for (int j = 0; j < k; ++j) {
            if (!sblob[j])
                continue;
            float y = 0.f;
#pragma unroll
            for (int p = 0; p < KP; ++p)
                y += red[p][tid][j];
            s = fmaf(sg[j], y, s);
        }
        if (residual)
            s = residual[o] + s;
        out[o] = s;
        if (out_act) {
            if (OUT_BF16)
                ((uint16_t *)out_act)[o] = f_to_bf(s);
            else
                ((float *)out_act)[o] = s;
        }
    }
}

// out[t][c] = residual[t][c] + (sum over j ascending of gate[t][j] * Y[pos[t*k+j]][c]
//             for GPU-evaluated experts) + host_part[t][c].
// The partial sums of host-evaluated experts arrive in host_part (techfeed
// summary of "Meet FreeToken", section "Bandwidth-adaptive execution (q*
// policy)": GPU and CPU partial sums are added at the end).
// NT_Y: Y is read with non-temporal loads.  A prefill Y (hundreds of MB) is
// read once and never again (combine 95 -> 88 us bf16, 255 -> 223 us MXFP4);
// a decode Y (a few MB) was just written and sits in the caches, where plain
// loads are faster (16 tokens: 4.3 against 5.3 us).
template <bool OUT_BF16, bool NT_Y>
__global__ __launch_bounds__(256) void k_combine(
    const int32_t *__restrict__ idx, const float *__restrict__ gate, const int32_t *__restrict__ pos,
    const uint64_t *__restrict__ ptrs, const float *__restrict__ Y, int k, int d,
    int E, int R, const float *residual, const float *__restrict__ host_part, float *out, void *out_act)
{
    // The token's k (row, gate) pairs are read once into LDS (-1: expert not
    // evaluated here), so the k row loads below do not wait on each other.
    __shared__ int srow[32];
    __shared__ float sg[32];
    const int t = blockIdx.y;
    if ((int)threadIdx.x < k) {
        const int f = t * k + threadIdx.x;
        const int e = idx[f], p = pos[f];
        const bool ok = (unsigned)e < (unsigned)E && (unsigned)p < (unsigned)R && ptrs[e];
        srow[threadIdx.x] = ok ? p : -1;
        sg[threadIdx.x] = gate[f];
    }
    __syncthreads();
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d)
        return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // Eight rows at a time: all eight loads are issued before the first is
    // used (a skipped row -- not evaluated here, or past k -- loads row 0 and
    // is then left out by a select, so no load sits behind a branch), then the
    // rows are added in ascending j.  (With a branch per row the compiler
    // waited for each row's load before issuing the next: decode at one token
    // 49.9-51.6 -> 48.6 us, at four 113 -> 111 us.)
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 y[8];
        int p[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            p[u] = j0 + u < k ? srow[j0 + u] : -1;
            const size_t at = (size_t)(p[u] < 0 ? 0 : p[u]) * d + c;
            if (NT_Y) {
                const uint4 yu = ld_nt16(Y + at);
                y[u] = make_float4(__uint_as_float(yu.x), __uint_as_float(yu.y), __uint_as_float(yu.z),
                                   __uint_as_float(yu.w));
            } else {
                y[u] = *reinterpret_cast<const float4 *>(Y + at);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool use = p[u] >= 0;
            const float g = use ? sg[j0 + u] : 0.f;
            s.x = use ? fmaf(g, y[u].x, s.x) : s.x;
            s.y = use ? fmaf(g, y[u].y, s.y) : s.y;
            s.z = use ? fmaf(g, y[u].z, s.z) : s.z;
            s.w = use ? fmaf(g, y[u].w, s.w) : s.w;
        }
    }
    const size_t o = (size_t)t * d + c;
    if (host_part) {
        const float4 h = *reinterpret_cast<const float4 *>(host_part + o);
        s.x += h.x, s.y += h.y, s.z += h.z, s.w += h.w;
    }
    if (residual) {
        const float4 r = *reinterpret_cast<const float4 *>(residual + o);
        s.x = r.x + s.x, s.y = r.y + s.y, s.z = r.z + s.z, s.w = r.w + s.w;
    }
    *reinterpret_cast<float4 *>(out + o) = s;
    if (out_act) {
        if (OUT_BF16) {
            uint16_t *a = (uint16_t *)out_act + o;
            const uint32_t lo = (uint32_t)f_to_bf(s.x) | ((uint32_t)f_to_bf(s.y) << 16);
            const uint32_t hi = (uint32_t)f_to_bf(s.z) | ((uint32_t)f_to_bf(s.w) << 16);
            *reinterpret_cast<uint2 *>(a) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<float4 *>((float *)out_act + o) = s;
        }
    }
}

// ---------------------------------------------------------------------------------

int launch_decode_gateup(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const void *x,
                         int T, float *H, hipStream_t st)
{
    const int R = T * s.top_k;
    const int maxa = std::min(s.n_experts, R);
    constexpr int KP = 2;
    const int ntp = std::min(kDecodeNT, T);  // an expert has at most T rows
    const bool dot2 = s.a_dtype == ECF_BF16 && s.w_dtype != ECF_F32;
    const size_t sh = dot2 ? sizeof(uint16_t) * ntp * xpadh_len(s.hidden) : sizeof(float) * ntp * xpad_len(s.hidden);
    ProfScope p("decode_gateup", st);
    const bool abf = s.a_dtype == ECF_BF16;
#define ECF_GU(WFV, AB, IBV, KPV)                                                                   \
    hipLaunchKernelGGL((k_decode_gateup<WFV, AB, IBV, KPV>), dim3(s.inter / (IBV), maxa), dim3(256), sh, st, \
                       ex.ptrs, ex.lay.off[0], ex.lay.off[1], ex.lay.off[3], ex.lay.off[4], o.active,   \
                       o.n_active, o.offsets, o.perm, x, s.hidden, s.inter, s.top_k, s.n_experts, R,  \
                       ntp, H)
    // MXFP4 (bf16 activations, checked with the shape): with 64 or more routed
    // rows, 16-row blocks whose groups load gate row i and up row i together
    // (d 4096, I 1024, 16 tokens: 74.0 -> 71.3 us); at one token (6 rows) the
    // 8-row blocks are faster (14.0 against 15.0 us).
    // bf16: 2-row blocks (gate row i and up row i) with each row split over 8
    // groups (1 KB each), so every expert spreads over 8x more blocks than
    // 8-row blocks in 2 parts: d 4096, I 1024, gate/up 223 -> 197 us at 16
    // tokens, 71 -> 60 us at 4, 24 -> 21 us at 1 (MXFP4 got slower split this
    // way: its rows are a quarter as long and its arithmetic per byte 4x).
    if (s.w_dtype == ECF_MXFP4 && R >= 64)
        ECF_GU(WF_MX, true, 16, KP);
    else if (s.w_dtype == ECF_MXFP4)
        ECF_GU(WF_MX, true, 8, KP);
    else if (s.w_dtype == ECF_BF16)
        ECF_GU(WF_BF16, true, 2, 8);
    else if (abf)
        ECF_GU(WF_F32, true, 8, KP);
    else
        ECF_GU(WF_F32, false, 8, KP);
#undef ECF_GU
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

bool gateup_route1_ok(const ecf_shape &s, int T)
{
    return T == 1 && s.a_dtype == ECF_BF16 && (s.w_dtype == ECF_BF16 || s.w_dtype == ECF_MXFP4);
}

int launch_decode_gateup_route1(const ecf_shape &s, const ExpertTables &ex, const float *logits, const void *x,
                                const RouteOut &o, float *H, hipStream_t st)
{
    const bool mx = s.w_dtype == ECF_MXFP4;
    const int IBV = mx ? 8 : 2;
    const int items = s.top_k * (s.inter / IBV);
    // Persistent blocks, at most 4 per CU: d 4096, I 1024, top-6 (3,072 bf16 /
    // 768 MXFP4 items), one-token layer 47.5 -> 44.3 us bf16, 34.8 -> 30.7 us
    // MXFP4 against the routing kernel + k_decode_gateup (512 blocks: 45.5 /
    // 33.0; one block per item: 46.8 / 31.1).
    const int grid = std::max(1, std::min(items, 1024));
    const size_t sh = sizeof(uint16_t) * xpadh_len(s.hidden);
    const int maxs = (s.n_experts + 63) / 64;
    ProfScope p("decode_gateup", st);
#define ECF_GR(WFV, IB, KPV, MS)                                                                          \
    hipLaunchKernelGGL((k_decode_gateup_route1<WFV, IB, KPV, MS>), dim3(grid), dim3(256), sh, st, logits,  \
                       s.n_experts, s.top_k, s.renorm_topk, ex.ptrs, ex.lay.off[0], ex.lay.off[1],         \
                       ex.lay.off[3], ex.lay.off[4], (const uint16_t *)x, s.hidden, s.inter, o.idx, o.gate, \
                       o.counts, o.offsets, o.perm, o.pos, o.active, o.n_active, o.tiles, o.n_tiles, H)
#define ECF_GR_MS(WFV, IB, KPV)        \
    if (maxs <= 1)                     \
        ECF_GR(WFV, IB, KPV, 1);       \
    else if (maxs <= 2)                \
        ECF_GR(WFV, IB, KPV, 2);       \
    else if (maxs <= 4)                \
        ECF_GR(WFV, IB, KPV, 4);       \
    else if (maxs <= 8)                \
        ECF_GR(WFV, IB, KPV, 8);       \
    else                               \
        ECF_GR(WFV, IB, KPV, 16)
    if (mx) {
        ECF_GR_MS(WF_MX, 8, 2);
    } else {
        ECF_GR_MS(WF_BF16, 2, 8);
    }
#undef ECF_GR_MS
#undef ECF_GR
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_decode_down(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *H,
                       int T, float *Y, hipStream_t st)
{
    const int R = T * s.top_k;
    const int maxa = std::min(s.n_experts, R);
    constexpr int KP = 1;
    const int ntp = std::min(kDecodeNT, T);
    const size_t sh = sizeof(float) * ntp * xpad_len(s.inter);
    ProfScope p("decode_down", st);
#define ECF_DN(WFV, OBV, KPV)                                                                       \
    hipLaunchKernelGGL((k_decode_down<WFV, OBV, KPV>), dim3(s.hidden / (OBV), maxa), dim3(256), sh, st, \
                       ex.ptrs, ex.lay.off[2], ex.lay.off[5], o.active, o.n_active, o.offsets, H,     \
                       s.hidden, s.inter, s.n_experts, R, ntp, Y)
    // MXFP4 rows are a quarter of a bf16 row, so a 32-row block reads only 17 KB
    // after its fixed chain of latencies (routing tables, h staging, barrier);
    // with 64 or more routed rows 128-row blocks (each group's 4 rows loaded
    // together) still fill the GPU: d 4096, I 1024, 16 tokens 53.6 -> 50.0 us.
    // Below that (e.g. 6 rows at one token) there are too few of them.
    // bf16: 16-row blocks, each row split over 4 groups (512 B each), each group
    // two rows: down 107 -> 103 us at 16 tokens, 35 -> 34 us at 4.
    if (s.w_dtype == ECF_MXFP4 && R >= 64)
        ECF_DN(WF_MX, 128, KP);
    else if (s.w_dtype == ECF_MXFP4)
        ECF_DN(WF_MX, 32, KP);
    else if (s.w_dtype == ECF_BF16)
        ECF_DN(WF_BF16, 16, 4);
    else
        ECF_DN(WF_F32, 32, KP);
#undef ECF_DN
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

// Output rows per block of the fused one-token down + combine: 8, so each of
// the 4 parts along I is a whole number of 32-element scale groups when
// I % 128 == 0.  MXFP4 only: at d 4096, I 1024, top-6 it takes 9.7 us against
// 9.8 + 4.0 us for the down kernel and the combine; for bf16 weights (4x the
// bytes per row) the fused form took 18.4 us against 11.6 + 4.0 us.
constexpr int kDcOb = 8;

bool down_combine1_ok(const ecf_shape &s, int T)
{
    return T == 1 && s.top_k <= 8 && s.a_dtype == ECF_BF16 && s.w_dtype == ECF_MXFP4 &&
           s.inter % (32 * (32 / kDcOb)) == 0;
}

int launch_decode_down_combine1(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *H,
                                const float *residual, float *out, void *out_act, hipStream_t st)
{
    if (!down_combine1_ok(s, 1))
        return set_error(ECF_EUNSUPPORTED, "fused down + combine: one token, k <= 8, MXFP4 weights, I %% 128 == 0");
    const size_t sh = sizeof(float) * s.top_k * xpad_len(s.inter);
    ProfScope p("decode_down_combine", st);
#define ECF_DC(WFV, OB)                                                                                  \
    hipLaunchKernelGGL((k_decode_down_combine1<WFV, OB, true>), dim3(s.hidden / (OB)), dim3(256), sh, st,  \
                       ex.ptrs, ex.lay.off[2], ex.lay.off[5], o.idx, o.gate, o.pos, H, s.hidden, s.inter, \
                       s.top_k, s.n_experts, residual, out, out_act)
    ECF_DC(WF_MX, kDcOb);
#undef ECF_DC
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_combine(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *Y, int T,
                   const float *residual, const float *host_part, float *out, void *out_act,
                   hipStream_t st)
{
    dim3 grid((s.hidden / 4 + 255) / 256, T);
    ProfScope p("combine", st);
    const bool nt = (size_t)T * s.top_k * s.hidden * 4 > ((size_t)32 << 20);  // Y above 32 MB
#define ECF_CB(OBF, NTV)                                                                            \
    hipLaunchKernelGGL((k_combine<OBF, NTV>), grid, dim3(256), 0, st, o.idx, o.gate, o.pos, ex.ptrs, Y, \
                       s.top_k, s.hidden, s.n_experts, T * s.top_k, residual, host_part, out, out_act)
    if (s.a_dtype == ECF_BF16 && nt)
        ECF_CB(true, true);
    else if (s.a_dtype == ECF_BF16)
        ECF_CB(true, false);
    else if (nt)
        ECF_CB(false, true);
    else
        ECF_CB(false, false);
#undef ECF_CB
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
