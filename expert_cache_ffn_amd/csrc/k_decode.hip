// Decode-path expert kernels: weight-streaming GEMVs for the few rows each
// expert receives when T is small, and the fixed-order gate-weighted combine.
//
// Each block streams a band of one expert's weight rows exactly once from HBM
// and applies it to all (up to kDecodeNT per pass) routed rows of that expert.
// Lanes work in groups of 8: a group reads 8 x 16 B = 128 contiguous bytes of
// one weight row per step (one full cache line), so a wave touches 8 lines per
// load instruction.  Activations of the block's rows are staged once in LDS as
// fp32.  The intermediate h stays fp32 on this path.
//
// Expert FFN (SwiGLU, the standard definition; the pages do not fix the expert
// form): h = silu(W_gate . v) * (W_up . v), y = W_down . h.  GPU tensor cores
// run the experts that are resident (FreeToken paper explainer, section
// "Design: two-tier expert memory"; news.ainew.jp article on FreeToken, the
// paragraph on the q* co-scheduling policy).
#include "device_common.h"
#include "ecf_internal.h"

namespace ecf {

// Dot products of one weight row segment [kbeg, kend) against nt staged rows.
// V weights per 16-byte load; group of 8 lanes covers 8*V elements per step.
template <bool WBF>
__device__ __forceinline__ void row_dots(const void *__restrict__ wrow, const float *__restrict__ xs,
                                         int ld, int kbeg, int kend, int sub, int nt,
                                         float acc[kDecodeNT])
{
    constexpr int V = WBF ? 8 : 4;
    constexpr int UNR = 4;
    for (int c0 = kbeg + sub * V; c0 < kend; c0 += 8 * V * UNR) {
        uint4 wv[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * 8 * V;
            if (c < kend)
                wv[u] = ld_nt16((const char *)wrow + (size_t)c * (WBF ? 2 : 4));
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int c = c0 + u * 8 * V;
            if (c >= kend)
                break;
            float wf[V];
            if (WBF) {
                const uint32_t p[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wf[2 * i] = bf_lo(p[i]);
                    wf[2 * i + 1] = bf_hi(p[i]);
                }
            } else {
                wf[0] = __uint_as_float(wv[u].x);
                wf[1] = __uint_as_float(wv[u].y);
                wf[2] = __uint_as_float(wv[u].z);
                wf[3] = __uint_as_float(wv[u].w);
            }
#pragma unroll
            for (int q = 0; q < kDecodeNT; ++q) {
                if (q < nt) {
                    const float *xp = xs + q * ld + c;
                    float s = acc[q];
#pragma unroll
                    for (int i = 0; i < V; i += 4) {
                        const float4 xv = *reinterpret_cast<const float4 *>(xp + i);
                        s = fmaf(wf[i], xv.x, s);
                        s = fmaf(wf[i + 1], xv.y, s);
                        s = fmaf(wf[i + 2], xv.z, s);
                        s = fmaf(wf[i + 3], xv.w, s);
                    }
                    acc[q] = s;
                }
            }
        }
    }
}

__device__ __forceinline__ float load_act(const void *x, bool abf, size_t i)
{
    return abf ? bf_to_f(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// gate/up + SwiGLU.  Block = IB intermediate rows (gate and up) of one active
// expert, split into KP parts along d.  grid = (I / IB, max active experts).
template <bool WBF, bool ABF, int IB, int KP>
__global__ __launch_bounds__(256) void k_decode_gateup(
    const uint64_t *__restrict__ ptrs, size_t off_gate, size_t off_up,
    const int32_t *__restrict__ active, const int32_t *__restrict__ n_active,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ perm,
    const void *__restrict__ x, int d, int I, int k, int E, int R, int ntp, float *__restrict__ H)
{
    static_assert(2 * IB * KP == 32, "32 groups of 8 lanes per block");
    extern __shared__ float xs[];  // [min(kDecodeNT, T)][d]; an expert has at most T rows
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
    const int i0 = blockIdx.x * IB;
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 7;
    const int g = tid >> 3;  // group 0..31
    const int rho = g % (2 * IB), kap = g / (2 * IB);
    const size_t sec = rho < IB ? off_gate : off_up;
    const int irow = i0 + (rho % IB);
    const char *wrow = (const char *)blob + sec + (size_t)irow * d * (WBF ? 2 : 4);
    const int Lk = d / KP, kbeg = kap * Lk, kend = kbeg + Lk;
    for (int tp = 0; tp < ne; tp += ntp) {
        const int nt = min(ntp, ne - tp);
        for (int q = 0; q < nt; ++q) {
            const size_t t = (size_t)(perm[r0 + tp + q] / k);
            for (int c = tid; c < d; c += 256)
                xs[q * d + c] = load_act(x, ABF, t * d + c);
        }
        __syncthreads();
        float acc[kDecodeNT] = {};
        row_dots<WBF>(wrow, xs, d, kbeg, kend, sub, nt, acc);
#pragma unroll
        for (int q = 0; q < kDecodeNT; ++q) {
            acc[q] += __shfl_xor(acc[q], 1, 64);
            acc[q] += __shfl_xor(acc[q], 2, 64);
            acc[q] += __shfl_xor(acc[q], 4, 64);
        }
        if (sub == 0)
#pragma unroll
            for (int q = 0; q < kDecodeNT; ++q)
                red[kap][rho][q] = acc[q];
        __syncthreads();
        if (tid < IB * nt) {
            const int il = tid % IB, q = tid / IB;
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

// down projection: Y[r][o] = W_down[e][o] . h[r].  Block = OB output rows of
// one active expert, KP parts along I.  grid = (d / OB, max active experts).
template <bool WBF, int OB, int KP>
__global__ __launch_bounds__(256) void k_decode_down(
    const uint64_t *__restrict__ ptrs, size_t off_down, const int32_t *__restrict__ active,
    const int32_t *__restrict__ n_active, const int32_t *__restrict__ offsets,
    const float *__restrict__ H, int d, int I, int E, int R, int ntp, float *__restrict__ Y)
{
    static_assert(OB * KP == 32, "32 groups of 8 lanes per block");
    extern __shared__ float hs[];  // [min(kDecodeNT, T)][I]
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
    const int o0 = blockIdx.x * OB;
    const int tid = threadIdx.x, lane = tid & 63, sub = lane & 7;
    const int g = tid >> 3;
    const int rho = g % OB, kap = g / OB;
    const char *wrow = (const char *)blob + off_down + (size_t)(o0 + rho) * I * (WBF ? 2 : 4);
    const int Lk = I / KP, kbeg = kap * Lk, kend = kbeg + Lk;
    for (int tp = 0; tp < ne; tp += ntp) {
        const int nt = min(ntp, ne - tp);
        for (int q = 0; q < nt; ++q)
            for (int c = tid; c < I; c += 256)
                hs[q * I + c] = H[(size_t)(r0 + tp + q) * I + c];
        __syncthreads();
        float acc[kDecodeNT] = {};
        row_dots<WBF>(wrow, hs, I, kbeg, kend, sub, nt, acc);
#pragma unroll
        for (int q = 0; q < kDecodeNT; ++q) {
            acc[q] += __shfl_xor(acc[q], 1, 64);
            acc[q] += __shfl_xor(acc[q], 2, 64);
            acc[q] += __shfl_xor(acc[q], 4, 64);
        }
        if (sub == 0)
#pragma unroll
            for (int q = 0; q < kDecodeNT; ++q)
                red[kap][rho][q] = acc[q];
        __syncthreads();
        if (tid < OB * nt) {
            const int ol = tid % OB, q = tid / OB;
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < KP; ++p)
                s += red[p][ol][q];
            Y[(size_t)(r0 + tp + q) * d + o0 + ol] = s;
        }
        __syncthreads();
    }
}

// out[t][c] = residual[t][c] + (sum over j ascending of gate[t][j] * Y[pos[t*k+j]][c]
//             for GPU-evaluated experts) + host_part[t][c].
// The partial sums of host-evaluated experts arrive in host_part (techfeed
// summary of "Meet FreeToken", section "Bandwidth-adaptive execution (q*
// policy)": GPU and CPU partial sums are added at the end).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_combine(
    const int32_t *__restrict__ idx, const float *__restrict__ gate, const int32_t *__restrict__ pos,
    const uint64_t *__restrict__ ptrs, const float *__restrict__ Y, int k, int d,
    int E, int R, const float *residual, const float *__restrict__ host_part, float *out, void *out_act)
{
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d)
        return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const int f = t * k + j;
        const int e = idx[f], p = pos[f];
        if ((unsigned)e >= (unsigned)E || (unsigned)p >= (unsigned)R || !ptrs[e])
            continue;
        const float g = gate[f];
        const float4 y = *reinterpret_cast<const float4 *>(Y + (size_t)p * d + c);
        s.x = fmaf(g, y.x, s.x);
        s.y = fmaf(g, y.y, s.y);
        s.z = fmaf(g, y.z, s.z);
        s.w = fmaf(g, y.w, s.w);
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
    constexpr int IB = 8, KP = 2;
    dim3 grid(s.inter / IB, maxa);
    const int ntp = std::min(kDecodeNT, T);  // an expert has at most T rows
    const size_t sh = sizeof(float) * ntp * s.hidden;
    ProfScope p("decode_gateup", st);
    const bool wbf = s.w_dtype == ECF_BF16, abf = s.a_dtype == ECF_BF16;
#define ECF_GU(WB, AB)                                                                              \
    hipLaunchKernelGGL((k_decode_gateup<WB, AB, IB, KP>), grid, dim3(256), sh, st, ex.ptrs,          \
                       ex.lay.off[0], ex.lay.off[1], o.active, o.n_active, o.offsets, o.perm, x,      \
                       s.hidden, s.inter, s.top_k, s.n_experts, R, ntp, H)
    if (wbf && abf)
        ECF_GU(true, true);
    else if (wbf)
        ECF_GU(true, false);
    else if (abf)
        ECF_GU(false, true);
    else
        ECF_GU(false, false);
#undef ECF_GU
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_decode_down(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *H,
                       int T, float *Y, hipStream_t st)
{
    const int R = T * s.top_k;
    const int maxa = std::min(s.n_experts, R);
    constexpr int OB = 32, KP = 1;
    dim3 grid(s.hidden / OB, maxa);
    const int ntp = std::min(kDecodeNT, T);
    const size_t sh = sizeof(float) * ntp * s.inter;
    ProfScope p("decode_down", st);
    if (s.w_dtype == ECF_BF16)
        hipLaunchKernelGGL((k_decode_down<true, OB, KP>), grid, dim3(256), sh, st, ex.ptrs, ex.lay.off[2],
                           o.active, o.n_active, o.offsets, H, s.hidden, s.inter, s.n_experts, R, ntp, Y);
    else
        hipLaunchKernelGGL((k_decode_down<false, OB, KP>), grid, dim3(256), sh, st, ex.ptrs,
                           ex.lay.off[2], o.active, o.n_active, o.offsets, H, s.hidden, s.inter, s.n_experts,
                           R, ntp, Y);
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

int launch_combine(const ecf_shape &s, const ExpertTables &ex, const RouteOut &o, const float *Y, int T,
                   const float *residual, const float *host_part, float *out, void *out_act,
                   hipStream_t st)
{
    dim3 grid((s.hidden / 4 + 255) / 256, T);
    ProfScope p("combine", st);
    if (s.a_dtype == ECF_BF16)
        hipLaunchKernelGGL((k_combine<true>), grid, dim3(256), 0, st, o.idx, o.gate, o.pos, ex.ptrs, Y,
                           s.top_k, s.hidden, s.n_experts, T * s.top_k, residual, host_part, out, out_act);
    else
        hipLaunchKernelGGL((k_combine<false>), grid, dim3(256), 0, st, o.idx, o.gate, o.pos, ex.ptrs, Y,
                           s.top_k, s.hidden, s.n_experts, T * s.top_k, residual, host_part, out, out_act);
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

}  // namespace ecf
