// q8s_route.hip -- the mixture's router and top-K.
//
// What it computes is fn emit_moe_forward's route (codegen_cuda::qwen_emit
// module page): logits of an f32 router, softmax over every expert, the K
// largest kept and their weights renormalised to sum 1 (forward_shim.rs fn
// kernel_refusal refuses biased, grouped or un-renormalised routers).  The
// logits live in scratch, as arena.rs fn scratch's `rl`.
//
// Two launches:
//   k_logits  one workgroup per (expert, tile of rows); its four waves split d
//             in quarters, so the whole router streams from HBM across ~E
//             workgroups.  Products and sums are in double, so near-equal
//             logits are ranked as the double-precision definition ranks them.
//   k_topk    one workgroup per row: the K best by (logit descending, index
//             ascending) -- for E <= 256 a coarse count over order-preserving
//             32-bit keys picks the candidates and an exact double-precision
//             rank orders them (topk_select), beyond that K selection rounds
//             of a workgroup arg-max -- then the kept weights.
// Handing the logits over at the kernel boundary costs one short launch; doing
// it inside one launch needs a device-scope release by every workgroup, which
// measured several times slower on this chip.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

constexpr int RT_THREADS = 256;
constexpr int RT_WAVES = RT_THREADS / WAVE;

size_t route_scratch_bytes(int64_t rows, int64_t E) { return align256((size_t)rows * E * sizeof(double)); }

template <int RT>
__global__ void __launch_bounds__(RT_THREADS) k_logits(const float *__restrict__ x, const float *__restrict__ Wr,
                                                       int rows, int d, int E, double *__restrict__ logits)
{
    __shared__ double part[RT_WAVES][RT];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int r0 = blockIdx.y * RT;
    const int q = d / RT_WAVES;  // a wave's quarter of d (d is a multiple of 32)
    const float *wr = Wr + (int64_t)e * d + wid * q;

    double acc[RT];
#pragma unroll
    for (int r = 0; r < RT; r++)
        acc[r] = 0.0;
    constexpr int UN = 4;
    for (int t0 = lane * 4; t0 < q; t0 += WAVE * 4 * UN) {
        f32x4 a[UN];
#pragma unroll
        for (int u = 0; u < UN; u++) {
            const int t = t0 + u * WAVE * 4;
            a[u] = t < q ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wr + t)) : f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int r = 0; r < RT; r++) {
            const float *xr = x + (int64_t)min(r0 + r, rows - 1) * d + wid * q;
#pragma unroll
            for (int u = 0; u < UN; u++) {
                const int t = t0 + u * WAVE * 4;
                if (t < q) {
                    const f32x4 b = ldf4(xr + t);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[r] += (double)a[u][i] * (double)b[i];
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RT; r++) {
        const double v = wave_sum_f64(acc[r]);
        if (lane == 0)
            part[wid][r] = v;
    }
    __syncthreads();
    if (threadIdx.x < RT && r0 + (int)threadIdx.x < rows) {
        const int r = threadIdx.x;
        logits[(int64_t)(r0 + r) * E + e] = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
    }
}

// The logits over Q8_0 router rows (lane_link.rs fn prim, Moe arm: a router
// of quantized checkpoint rows): the same grid, a thread taking one 16-byte
// chunk (half a block) of the row a pass, so a block's halves sit in
// neighbouring lanes.
//   ACT 0: l = sum_t (q*s) * x[t]                       in double
//   ACT 1: l = sum_b (ws*xs) * isum_b, the block's exact int32 dot joined
//          from the two lanes' halves, added by the even lane
template <int ACT, int RT>
__global__ void __launch_bounds__(RT_THREADS)
    k_logits_q8(const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xs,
                const int8_t *__restrict__ Wrq, const float *__restrict__ Wrs, int rows, int d, int E,
                double *__restrict__ logits)
{
    __shared__ double part[RT_WAVES][RT];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int e = blockIdx.x;
    const int r0 = blockIdx.y * RT;
    const int nch = d >> 4, nb = d >> 5;
    const int8_t *wq = Wrq + (int64_t)e * d;
    const float *ws = Wrs + (int64_t)e * nb;

    double acc[RT];
#pragma unroll
    for (int r = 0; r < RT; r++)
        acc[r] = 0.0;
    // nch is even, so both lanes of a block's pair run the same passes
    for (int c = threadIdx.x; c < nch; c += RT_THREADS) {
        const i32x4 wv = ld_stream16(wq + c * 16);
        const float s = __builtin_nontemporal_load(ws + (c >> 1));
#pragma unroll
        for (int r = 0; r < RT; r++) {
            const int64_t xr = min(r0 + r, rows - 1);
            if (ACT == 0) {
                const float *xp = x + xr * d + c * 16;
#pragma unroll
                for (int v4 = 0; v4 < 4; v4++) {
                    const f32x4 b = ldf4(xp + v4 * 4);
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int q = (int)(int8_t)((wv[v4] >> (8 * i)) & 0xFF);
                        acc[r] += ((double)q * (double)s) * (double)b[i];
                    }
                }
            } else {
                int is = chunk_dot_i8(wv, ld16(xq + xr * d + c * 16));
                is += dpp_i<DPP_XOR1>(is);
                if ((lane & 1) == 0)
                    acc[r] += ((double)s * (double)xs[xr * nb + (c >> 1)]) * (double)is;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RT; r++) {
        const double v = wave_sum_f64(acc[r]);
        if (lane == 0)
            part[wid][r] = v;
    }
    __syncthreads();
    if (threadIdx.x < RT && r0 + (int)threadIdx.x < rows) {
        const int r = threadIdx.x;
        logits[(int64_t)(r0 + r) * E + e] = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
    }
}

__global__ void __launch_bounds__(RT_THREADS) k_topk(const double *__restrict__ logits, int E, int k,
                                                     int32_t *__restrict__ idx, float *__restrict__ wts)
{
    extern __shared__ double Lbig[];  // [E], for rows of more than TOPK_LDS_E logits
    __shared__ TopkLds t;
    __shared__ double bl[RT_WAVES];
    __shared__ int be[RT_WAVES];
    const int64_t row = blockIdx.x;
    const double *lr = logits + row * E;

    if (E <= TOPK_LDS_E) {
        topk_load(t, lr, E);
        __syncthreads();
        topk_select(t, E, k);
        __syncthreads();
    } else {
        for (int i = threadIdx.x; i < E; i += RT_THREADS)
            Lbig[i] = lr[i];
        __syncthreads();
        // K rounds of a workgroup arg-max; a chosen logit is retired to -inf
        // by the thread that scans it (real logits are finite and k <= E)
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        for (int jj = 0; jj < k; jj++) {
            double b = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = threadIdx.x; i < E; i += RT_THREADS)
                if (route_better(Lbig[i], i, b, bi)) {
                    b = Lbig[i];
                    bi = i;
                }
            for (int o = 32; o >= 1; o >>= 1) {
                const double b2 = __shfl_xor(b, o);
                const int i2 = __shfl_xor(bi, o);
                if (route_better(b2, i2, b, bi)) {
                    b = b2;
                    bi = i2;
                }
            }
            if (lane == 0) {
                bl[wid] = b;
                be[wid] = bi;
            }
            __syncthreads();
            double wb = bl[0];
            int wi = be[0];
            for (int w = 1; w < RT_WAVES; w++)
                if (route_better(bl[w], be[w], wb, wi)) {
                    wb = bl[w];
                    wi = be[w];
                }
            if (threadIdx.x == 0) {
                t.ch[jj] = wi;
                t.kl[jj] = wb;
            }
            if ((int)threadIdx.x == (wi % RT_THREADS))
                Lbig[wi] = -INFINITY;
            __syncthreads();
        }
    }
    if (threadIdx.x < WAVE)
        route_finish(t.kl, t.ch, k, idx + row * k, wts + row * k);
}

namespace {

hipError_t topk_go(const double *logits, int64_t rows, int64_t E, int64_t k, int32_t *idx, float *wts, hipStream_t st)
{
    const size_t big = E > TOPK_LDS_E ? (size_t)E * sizeof(double) : 0;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)rows), dim3(RT_THREADS), big, st, logits, (int)E, (int)k, idx, wts);
    return hipGetLastError();
}

} // namespace

hipError_t route_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                        float *wts, void *scratch, hipStream_t st)
{
    double *logits = reinterpret_cast<double *>(scratch);
    if (rows == 1)
        hipLaunchKernelGGL((k_logits<1>), dim3((unsigned)E, 1), dim3(RT_THREADS), 0, st, x, Wr, (int)rows, (int)d,
                           (int)E, logits);
    else
        hipLaunchKernelGGL((k_logits<4>), dim3((unsigned)E, (unsigned)((rows + 3) / 4)), dim3(RT_THREADS), 0, st, x,
                           Wr, (int)rows, (int)d, (int)E, logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    return topk_go(logits, rows, E, k, idx, wts, st);
}

hipError_t route_q8_launch(const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq, const float *Wrs,
                           int64_t rows, int64_t d, int64_t E, int64_t k, int act, int32_t *idx, float *wts,
                           void *scratch, hipStream_t st)
{
    double *logits = reinterpret_cast<double *>(scratch);
    const dim3 block(RT_THREADS);
    const dim3 g1((unsigned)E, (unsigned)rows), g4((unsigned)E, (unsigned)((rows + 3) / 4));
    if (act == 0 && rows == 1)
        hipLaunchKernelGGL((k_logits_q8<0, 1>), g1, block, 0, st, x, xq, xs, Wrq, Wrs, (int)rows, (int)d, (int)E,
                           logits);
    else if (act == 0)
        hipLaunchKernelGGL((k_logits_q8<0, 4>), g4, block, 0, st, x, xq, xs, Wrq, Wrs, (int)rows, (int)d, (int)E,
                           logits);
    else if (rows == 1)
        hipLaunchKernelGGL((k_logits_q8<1, 1>), g1, block, 0, st, x, xq, xs, Wrq, Wrs, (int)rows, (int)d, (int)E,
                           logits);
    else
        hipLaunchKernelGGL((k_logits_q8<1, 4>), g4, block, 0, st, x, xq, xs, Wrq, Wrs, (int)rows, (int)d, (int)E,
                           logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    return topk_go(logits, rows, E, k, idx, wts, st);
}

} // namespace q8s
