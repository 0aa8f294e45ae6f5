// Measurement kernel: a plain streaming read of a device buffer, the yardstick
// for the HBM bandwidth the layer's kernels reach.  Each block reads one
// contiguous chunk of the buffer front to back, 16 bytes per lane and load
// (non-temporal), eight loads in flight; two blocks per CU.  On MI355X this
// reads 7.0-7.1 TB/s, against 5.9-6.0 TB/s for a grid-stride sweep (every
// block stepping through the whole buffer together) and 6.1-6.9 TB/s with 1, 3
// or 4 blocks per CU.  The XOR of every 32-bit word goes to one sink word (so
// no load is dead code and the result can be checked), one atomic per block.
#include <algorithm>

#include "device_common.h"
#include "ecf_internal.h"

namespace ecf {
namespace {

__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ src, size_t n16,
                                                     uint32_t *__restrict__ sink)
{
    constexpr int UNR = 8;
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per, end = beg + per < n16 ? beg + per : n16;
    uint32_t x = 0;
    size_t i = beg + threadIdx.x;
    for (; i + (UNR - 1) * 256 < end; i += UNR * 256) {
        uint4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            v[u] = ld_nt16(src + i + u * 256);
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
        const uint4 v = ld_nt16(src + i);
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        x ^= __shfl_xor(x, off, 64);
    // one atomic per block: the sink word is a single address, and the atomics
    // of every wave of the grid arriving together at the end cost ~17 us
    __shared__ uint32_t wx[4];
    if ((threadIdx.x & 63) == 0)
        wx[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicXor(sink, (wx[0] ^ wx[1]) ^ (wx[2] ^ wx[3]));
}

// Measurement kernel: the bf16 MFMA rate this GPU sustains, the yardstick for
// the prefill GEMMs' MFMA fraction.  Each wave runs `iters` rounds of eight
// independent v_mfma_f32_32x32x16_bf16 on operands held in registers: four
// distinct pseudo-random A and B fragments, so the operands change from one
// MFMA to the next as they do in a GEMM (with constant operands the part runs
// at a higher clock than under a real GEMM).  No memory traffic in the loop;
// the accumulators reach the sink only if their sum is a value it cannot be,
// so nothing is dead code.
__global__ __launch_bounds__(256) void k_mfma_rate(int iters, uint32_t seed, float *__restrict__ sink)
{
    bf16x8_t a[4], b[4];
    uint32_t h = 0x9E3779B9u * (threadIdx.x + 1 + 256 * blockIdx.x) + seed;
    auto next = [&h]() {  // xorshift32
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return (float)(h & 0xFFFFu) * (1.f / 65536.f) - 0.5f;
    };
    for (int q = 0; q < 4; ++q)
        for (int i = 0; i < 8; ++i) {
            a[q][i] = (__bf16)next();
            b[q][i] = (__bf16)next();
        }
    f32x16_t acc[8];
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 16; ++i)
            acc[j][i] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j + 1) & 3], acc[j], 0, 0, 0);
    }
    float r = 0.f;
    for (int j = 0; j < 8; ++j)
        for (int i = 0; i < 16; ++i)
            r += acc[j][i];
    if (r == 1.0e30f)
        *sink = r;
}

}  // namespace
}  // namespace ecf

using namespace ecf;

extern "C" int ecf_stream_read(const void *d_buf, size_t bytes, uint32_t *d_sink, void *stream)
{
    if (!d_buf || !d_sink || bytes % 16 || (uintptr_t)d_buf % 16)
        return set_error(ECF_EINVAL, "ecf_stream_read: need a 16-byte aligned buffer of a multiple of 16 bytes");
    if (bytes == 0)
        return ECF_OK;
    int dev = 0, cus = 0;
    ECF_HIP_CHECK(hipGetDevice(&dev));
    ECF_HIP_CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const size_t n16 = bytes / 16;
    const size_t want = (n16 + 256 * 8 - 1) / (256 * 8);  // blocks with a full unrolled pass each
    const int grid = (int)std::max<size_t>(1, std::min<size_t>(want, (size_t)cus * 2));
    hipStream_t st = (hipStream_t)stream;
    hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, st, (const uint4 *)d_buf, n16, d_sink);
    ECF_HIP_CHECK(hipGetLastError());
    return ECF_OK;
}

extern "C" int ecf_mfma_rate(int32_t iters, int32_t blocks_per_cu, float *d_sink, void *stream, double *flop)
{
    if (iters <= 0 || blocks_per_cu <= 0 || blocks_per_cu > 8 || !d_sink || !flop)
        return set_error(ECF_EINVAL, "ecf_mfma_rate: need iters > 0, 1 <= blocks_per_cu <= 8, a sink and flop");
    int dev = 0, cus = 0;
    ECF_HIP_CHECK(hipGetDevice(&dev));
    ECF_HIP_CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    const int grid = cus * blocks_per_cu;
    hipLaunchKernelGGL(k_mfma_rate, dim3(grid), dim3(256), 0, (hipStream_t)stream, (int)iters, 0x5EEDu, d_sink);
    ECF_HIP_CHECK(hipGetLastError());
    *flop = (double)grid * 4 * iters * 8 * (2.0 * 32 * 32 * 16);
    return ECF_OK;
}
