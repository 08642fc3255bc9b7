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
//             ascending) -- for E <= 256 each thread ranks one logit against
//             all E at once, beyond that K selection rounds of a workgroup
//             arg-max -- then the kept weights.
// Handing the logits over at the kernel boundary costs one short launch; doing
// it inside one launch needs a device-scope release by every workgroup, which
// measured several times slower on this chip.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

constexpr int RT_THREADS = 256;
constexpr int RT_WAVES = RT_THREADS / WAVE;
constexpr int TOPK_RANK_MAX_E = 256;

size_t route_scratch_bytes(int64_t rows, int64_t E) { return align256((size_t)rows * E * sizeof(double)); }

// (l, e) ranks before (l', e') when l > l', or l == l' and e < e'.
Q8S_DEV bool better(double l, int e, double l2, int e2) { return l > l2 || (l == l2 && e < e2); }

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

// The kept weights: softmax over all E, then renormalised over the kept K,
//   w_j = p_j / sum_i p_i,  p_e = exp(l_e - m) / sum_all exp(l - m),
// where the all-expert denominator cancels; with m the largest logit (the
// rank-0 choice) this is w_j = exp(l_j - m) / sum_i exp(l_i - m), formed in
// double from the K kept logits only, one lane per kept slot of wave 0.
Q8S_DEV void finish_row(const double *kl, const int *ch, int k, int32_t *idx_row, float *wts_row)
{
    const int j = threadIdx.x;
    const double p = j < k ? exp(kl[j] - kl[0]) : 0.0;
    const double kept = wave_sum_f64(p);
    if (j < k) {
        idx_row[j] = ch[j];
        wts_row[j] = (float)(p / kept);
    }
}

__global__ void __launch_bounds__(RT_THREADS) k_topk(const double *__restrict__ logits, int E, int k,
                                                     int32_t *__restrict__ idx, float *__restrict__ wts)
{
    extern __shared__ double L[];  // [E]
    __shared__ int ch[Q8S_MAX_K_DEV];
    __shared__ double kl[Q8S_MAX_K_DEV];
    __shared__ double bl[RT_WAVES];
    __shared__ int be[RT_WAVES];
    const int64_t row = blockIdx.x;
    const double *lr = logits + row * E;
    for (int i = threadIdx.x; i < E; i += RT_THREADS)
        L[i] = lr[i];
    __syncthreads();

    if (E <= TOPK_RANK_MAX_E) {
        // rank of each logit among all E: S = 256/E (a power of two) threads
        // per logit each count the better ones in a share of the E, and sum;
        // the K of rank < K are the kept set, in rank order
        int S = 1;
        while (S * 2 * E <= RT_THREADS && S < WAVE)
            S *= 2;
        const int i = threadIdx.x / S, part = threadIdx.x % S;
        int rank = 0;
        double li = 0.0;
        if (i < E) {
            li = L[i];
            const int j0 = part * E / S, j1 = (part + 1) * E / S;
            int j = j0;
            for (; j + 8 <= j1; j += 8) {
                double v[8];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    v[u] = L[j + u];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    rank += better(v[u], j + u, li, i) ? 1 : 0;
            }
            for (; j < j1; j++)
                rank += better(L[j], j, li, i) ? 1 : 0;
        }
        for (int o = 1; o < S; o <<= 1)
            rank += __shfl_xor(rank, o);
        if (i < E && part == 0 && rank < k) {
            ch[rank] = i;
            kl[rank] = li;
        }
        __syncthreads();
    } else {
        // K rounds of a workgroup arg-max; a chosen logit is retired to -inf
        // by the thread that scans it (real logits are finite and k <= E)
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        for (int jj = 0; jj < k; jj++) {
            double b = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = threadIdx.x; i < E; i += RT_THREADS)
                if (better(L[i], i, b, bi)) {
                    b = L[i];
                    bi = i;
                }
            for (int o = 32; o >= 1; o >>= 1) {
                const double b2 = __shfl_xor(b, o);
                const int i2 = __shfl_xor(bi, o);
                if (better(b2, i2, b, bi)) {
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
                if (better(bl[w], be[w], wb, wi)) {
                    wb = bl[w];
                    wi = be[w];
                }
            if (threadIdx.x == 0) {
                ch[jj] = wi;
                kl[jj] = wb;
            }
            if ((int)threadIdx.x == (wi % RT_THREADS))
                L[wi] = -INFINITY;
            __syncthreads();
        }
    }
    if (threadIdx.x < WAVE)
        finish_row(kl, ch, k, idx + row * k, wts + row * k);
}

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
    hipLaunchKernelGGL(k_topk, dim3((unsigned)rows), dim3(RT_THREADS), (size_t)E * sizeof(double), st, logits, (int)E,
                       (int)k, idx, wts);
    return hipGetLastError();
}

} // namespace q8s
