// q8s_norm.hip -- the residual add + RMSNorm row kernel with a Q8_0
// epilogue, and the standalone Q8_0 activation quantiser.
//
// add_rmsnorm_q8 follows codegen_cuda/forward_shim.rs (module doc: a sum and
// the RMS norm of it as one row kernel writing the sum; a weighted norm scales
// and never shifts, fn kernel_refusal; under one-word int8 numerics the
// activation is quantised in its producer's epilogue).
//
// One workgroup of 256 threads per row; a thread owns 8 consecutive values of
// every 2048-value segment, so four neighbouring threads own one Q8_0 block
// and the block's absolute maximum needs two DPP steps.  The mean square is
// summed in double and the normalised value formed in double, then rounded to
// float32 once: that float32 value decides the int8 codes.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

constexpr int NORM_THREADS = 256;
constexpr int NORM_SEG = NORM_THREADS * 8;

// Quantise 8 consecutive values held by one thread of a 4-thread block group;
// writes the 8 codes and (first thread of the group) the block scale.
Q8S_DEV void quant8_store(const float (&v)[8], int8_t *q, float *scale, bool leader)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp_f<DPP_XOR1>(amax));
    amax = fmaxf(amax, dpp_f<DPP_XOR2>(amax));
    const float d = q8_scale(amax);
    const float id = q8_inv(d);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo |= (uint32_t)(q8_code(v[i], id) & 0xFF) << (8 * i);
        hi |= (uint32_t)(q8_code(v[4 + i], id) & 0xFF) << (8 * i);
    }
    *reinterpret_cast<uint2 *>(q) = make_uint2(lo, hi);
    if (leader)
        *scale = d;
}

// SEGS > 0: the row has at most SEGS 2048-value segments, and each thread keeps
// its sums and weights in registers between the two passes.  SEGS == 0: any
// length; the second pass re-forms the sums from h and r (the same float32
// adds, bit for bit).
template <int SEGS>
__global__ void __launch_bounds__(NORM_THREADS) k_add_rmsnorm_q8(const float *__restrict__ h, const float *__restrict__ r,
                                                                 const float *__restrict__ w, int d, float eps,
                                                                 float *__restrict__ sum, float *__restrict__ y,
                                                                 int8_t *__restrict__ yq, float *__restrict__ ys)
{
    constexpr int NS = SEGS > 0 ? SEGS : 1;
    __shared__ double wsum[NORM_THREADS / WAVE];
    const int64_t row = blockIdx.x;
    const float *hr = h + row * d;
    const float *rr = r + row * d;
    const int t8 = threadIdx.x * 8;

    f32x4 sv[NS][2], wv[NS][2];
    double ss = 0.0;
    if (SEGS > 0) {
#pragma unroll
        for (int g = 0; g < NS; g++) {
            const int base = t8 + g * NORM_SEG;
            if (base < d) {
                const f32x4 a0 = ldf4(hr + base), a1 = ldf4(hr + base + 4);
                const f32x4 b0 = ldf4(rr + base), b1 = ldf4(rr + base + 4);
                wv[g][0] = ldf4(w + base);
                wv[g][1] = ldf4(w + base + 4);
                sv[g][0] = a0 + b0;
                sv[g][1] = a1 + b1;
            }
        }
#pragma unroll
        for (int g = 0; g < NS; g++) {
            const int base = t8 + g * NORM_SEG;
            if (base < d) {
                *reinterpret_cast<f32x4 *>(sum + row * d + base) = sv[g][0];
                *reinterpret_cast<f32x4 *>(sum + row * d + base + 4) = sv[g][1];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    ss += (double)sv[g][0][i] * (double)sv[g][0][i] + (double)sv[g][1][i] * (double)sv[g][1][i];
            }
        }
    } else {
        for (int base = t8; base < d; base += NORM_SEG) {
            const f32x4 s0 = ldf4(hr + base) + ldf4(rr + base), s1 = ldf4(hr + base + 4) + ldf4(rr + base + 4);
            *reinterpret_cast<f32x4 *>(sum + row * d + base) = s0;
            *reinterpret_cast<f32x4 *>(sum + row * d + base + 4) = s1;
#pragma unroll
            for (int i = 0; i < 4; i++)
                ss += (double)s0[i] * (double)s0[i] + (double)s1[i] * (double)s1[i];
        }
    }
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0)
        wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < NORM_THREADS / WAVE; i++)
        tot += wsum[i];
    const double inv = 1.0 / sqrt(tot / (double)d + (double)eps);

    for (int g = 0; SEGS > 0 ? g < NS : true; g++) {
        const int base = t8 + g * NORM_SEG;
        if (base >= d)
            break;
        f32x4 s0, s1, w0, w1;
        if (SEGS > 0) {
            s0 = sv[g][0];
            s1 = sv[g][1];
            w0 = wv[g][0];
            w1 = wv[g][1];
        } else {
            s0 = ldf4(hr + base) + ldf4(rr + base);
            s1 = ldf4(hr + base + 4) + ldf4(rr + base + 4);
            w0 = ldf4(w + base);
            w1 = ldf4(w + base + 4);
        }
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[i] = (float)(((double)s0[i] * inv) * (double)w0[i]);
            v[4 + i] = (float)(((double)s1[i] * inv) * (double)w1[i]);
        }
        if (y) {
            *reinterpret_cast<f32x4 *>(y + row * d + base) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4 *>(y + row * d + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
        if (yq)
            quant8_store(v, yq + row * d + base, ys + row * (d / QB) + base / QB, (threadIdx.x & 3) == 0);
    }
}

// q8_quantize_rows: the same epilogue on a given f32 row set.  Threads own 8
// values; the grid covers rows x 2048-value segments.
__global__ void __launch_bounds__(NORM_THREADS) k_quantize_rows(const float *__restrict__ x, int64_t n,
                                                                int8_t *__restrict__ xq, float *__restrict__ xs)
{
    const int64_t row = blockIdx.y;
    const int64_t base = (int64_t)blockIdx.x * NORM_SEG + threadIdx.x * 8;
    if (base >= n)
        return;  // whole 4-thread groups leave together: n is a multiple of 32
    const float *p = x + row * n + base;
    const f32x4 a0 = ldf4(p), a1 = ldf4(p + 4);
    const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    quant8_store(v, xq + row * n + base, xs + row * (n / QB) + base / QB, (threadIdx.x & 3) == 0);
}

hipError_t quantize_launch(const float *x, int64_t rows, int64_t n, int8_t *xq, float *xs, hipStream_t st)
{
    dim3 grid((unsigned)((n + NORM_SEG - 1) / NORM_SEG), (unsigned)rows);
    hipLaunchKernelGGL(k_quantize_rows, grid, dim3(NORM_THREADS), 0, st, x, n, xq, xs);
    return hipGetLastError();
}

hipError_t add_rmsnorm_launch(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              float *sum, float *y, int8_t *yq, float *ys, hipStream_t st)
{
    const int segs = (int)((d + NORM_SEG - 1) / NORM_SEG);
    const dim3 grid((unsigned)rows), block(NORM_THREADS);
    if (segs <= 1)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<1>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys);
    else if (segs <= 2)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<2>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys);
    else if (segs <= 4)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<4>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys);
    else
        hipLaunchKernelGGL((k_add_rmsnorm_q8<0>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys);
    return hipGetLastError();
}

} // namespace q8s
