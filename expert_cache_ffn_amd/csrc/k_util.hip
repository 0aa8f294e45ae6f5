// Measurement kernel: a plain streaming read of a device buffer, the yardstick
// for the HBM bandwidth the layer's kernels reach.  Each block reads one
// contiguous chunk of the buffer front to back, 16 bytes per lane and load
// (non-temporal), eight loads in flight; two blocks per CU.  On MI355X this
// reads 7.0-7.1 TB/s, against 5.9-6.0 TB/s for a grid-stride sweep (every
// block stepping through the whole buffer together) and 6.1-6.9 TB/s with 1, 3
// or 4 blocks per CU.  The XOR of every 32-bit word goes to one sink word (so
// no load is dead code and the result can be checked).
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
    if ((threadIdx.x & 63) == 0)
        atomicXor(sink, x);
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
