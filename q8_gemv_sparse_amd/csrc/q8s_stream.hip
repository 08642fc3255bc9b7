// q8s_stream.hip -- a plain streaming read of device memory: the ceiling the
// weight streams are measured against.
//
// Every kernel of the path is bound by the bytes of its weight rows, so each
// is reported as a fraction of the HBM peak and of what the simplest possible
// reader reaches on the same device: 16-byte non-temporal loads, each
// workgroup on a contiguous span with its lanes on consecutive chunks, eight
// loads in flight a lane, every byte read once, reduced (xor of 32-bit
// words) to one word per workgroup so the loads cannot be dropped.  It
// computes nothing of the method.
#include "q8s.h"
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

namespace {

constexpr int SR_THREADS = 256;
constexpr int SR_U = 8;  // loads in flight a lane

// Workgroup b reads the contiguous span [b*per, (b+1)*per) of 16-byte
// chunks, its lanes on consecutive chunks: on MI355X this measured 7.0 TB/s
// over 2 GiB, against 5.9 TB/s when the whole grid strides over the buffer
// together (each workgroup's reads then stay within its own DRAM pages).
__global__ void __launch_bounds__(SR_THREADS) k_stream_read(const i32x4 *__restrict__ p, int64_t n16,
                                                            uint32_t *__restrict__ out)
{
    __shared__ uint32_t part[SR_THREADS / WAVE];
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t end = min(b0 + per, n16);
    constexpr int64_t stride = SR_THREADS;
    int64_t i = b0 + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (SR_U - 1) * stride < end; i += SR_U * stride) {
        i32x4 v[SR_U];
#pragma unroll
        for (int u = 0; u < SR_U; u++)
            v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < SR_U; u++)
            acc ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    }
    for (; i < end; i += stride) {
        const i32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    for (int off = 32; off >= 1; off >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & (WAVE - 1)) == 0)
        part[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
        for (int w = 0; w < SR_THREADS / WAVE; w++)
            r ^= part[w];
        out[blockIdx.x] = r;
    }
}

} // namespace

hipError_t stream_read_launch(const void *buf, int64_t bytes, uint32_t *out, hipStream_t st)
{
    hipLaunchKernelGGL(k_stream_read, dim3(Q8S_STREAM_WGS), dim3(SR_THREADS), 0, st,
                       reinterpret_cast<const i32x4 *>(buf), bytes / 16, out);
    return hipGetLastError();
}

} // namespace q8s
