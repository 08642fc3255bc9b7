// q8s_route.hip -- the mixture's router and top-K in one launch.
//
// What it computes is fn emit_moe_forward's route (codegen_cuda::qwen_emit
// module page): logits of an f32 router, softmax over every expert, the K
// largest kept and their weights renormalised to sum 1 (forward_shim.rs fn
// kernel_refusal refuses biased, grouped or un-renormalised routers).  The
// scratch is arena.rs fn scratch's: logits (`rl`) and an arrival count (`rc`)
// that the last block to arrive resets.
//
// Each wave forms one expert's logit for RT activation rows (the router row is
// loaded once for all of them) with double-precision sums, so near-equal
// logits are ranked as the double-precision definition ranks them.  The
// workgroup that arrives last for a tile of rows reads the tile's logits back
// and runs softmax and the K selection rounds for each of its rows.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_WAVES = ROUTE_THREADS / WAVE;

// Scratch layout: arrival counters first, in a region sized for the most row
// tiles any call can have, then the logits.  Every call finds its counters at
// the same place whatever its row count, so one zero-filled buffer serves
// calls of any size up to the one it was sized for.
constexpr size_t ROUTE_COUNTER_BYTES = (size_t)(65535 + 3) / 4 * sizeof(int);

size_t route_scratch_bytes(int64_t rows, int64_t E)
{
    return align256(ROUTE_COUNTER_BYTES) + align256((size_t)rows * E * sizeof(double));
}

struct Cand {
    double l;
    int e;
};

// (l, e) ranks before (l', e') when l > l', or l == l' and e < e'.
Q8S_DEV bool better(double l, int e, double l2, int e2) { return l > l2 || (l == l2 && e < e2); }

template <int RT>
__global__ void __launch_bounds__(ROUTE_THREADS) k_route(const float *__restrict__ x, const float *__restrict__ Wr,
                                                         int rows, int d, int E, int k, double *__restrict__ logits,
                                                         int *__restrict__ counters, int32_t *__restrict__ idx,
                                                         float *__restrict__ wts)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int e = blockIdx.x * ROUTE_WAVES + wid;
    const int r0 = blockIdx.y * RT;
    const int nr = min(RT, rows - r0);

    if (e < E) {
        double acc[RT];
#pragma unroll
        for (int r = 0; r < RT; r++)
            acc[r] = 0.0;
        const float *wr = Wr + (int64_t)e * d;
        for (int t = lane * 4; t < d; t += WAVE * 4) {
            const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wr + t));
#pragma unroll
            for (int r = 0; r < RT; r++) {
                const f32x4 b = ldf4(x + (int64_t)min(r0 + r, rows - 1) * d + t);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[r] += (double)a[i] * (double)b[i];
            }
        }
#pragma unroll
        for (int r = 0; r < RT; r++) {
            const double v = wave_sum_f64(acc[r]);
            if (lane == 0 && r < nr)
                logits[(int64_t)(r0 + r) * E + e] = v;
        }
    }

    // Arrival: the last workgroup of this row tile finishes the route.
    __shared__ int is_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = (atomicAdd(&counters[blockIdx.y], 1) == (int)gridDim.x - 1);
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();

    __shared__ Cand wbest[ROUTE_WAVES];
    __shared__ double wred[ROUTE_WAVES];
    __shared__ int chosen[Q8S_MAX_K_DEV];
    __shared__ double bcast;
    for (int r = 0; r < nr; r++) {
        const double *l = logits + (int64_t)(r0 + r) * E;
        // maximum logit
        double mx = -INFINITY;
        for (int i = threadIdx.x; i < E; i += ROUTE_THREADS)
            mx = fmax(mx, l[i]);
        for (int o = 32; o >= 1; o >>= 1)
            mx = fmax(mx, __shfl_xor(mx, o));
        if (lane == 0)
            wred[wid] = mx;
        __syncthreads();
        if (threadIdx.x == 0) {
            double m2 = wred[0];
            for (int i = 1; i < ROUTE_WAVES; i++)
                m2 = fmax(m2, wred[i]);
            bcast = m2;
        }
        __syncthreads();
        mx = bcast;
        // softmax denominator over all E
        double z = 0.0;
        for (int i = threadIdx.x; i < E; i += ROUTE_THREADS)
            z += exp(l[i] - mx);
        z = wave_sum_f64(z);
        __syncthreads();
        if (lane == 0)
            wred[wid] = z;
        __syncthreads();
        if (threadIdx.x == 0) {
            double zz = 0.0;
            for (int i = 0; i < ROUTE_WAVES; i++)
                zz += wred[i];
            bcast = zz;
        }
        __syncthreads();
        const double zsum = bcast;
        // K selection rounds: best (logit, index) not yet chosen
        for (int j = 0; j < k; j++) {
            Cand c{-INFINITY, 0x7fffffff};
            for (int i = threadIdx.x; i < E; i += ROUTE_THREADS) {
                bool taken = false;
                for (int q = 0; q < j; q++)
                    taken |= (chosen[q] == i);
                const double li = l[i];
                if (!taken && better(li, i, c.l, c.e))
                    c = Cand{li, i};
            }
            for (int o = 32; o >= 1; o >>= 1) {
                const double l2 = __shfl_xor(c.l, o);
                const int e2 = __shfl_xor(c.e, o);
                if (better(l2, e2, c.l, c.e))
                    c = Cand{l2, e2};
            }
            if (lane == 0)
                wbest[wid] = c;
            __syncthreads();
            if (threadIdx.x == 0) {
                Cand b = wbest[0];
                for (int i = 1; i < ROUTE_WAVES; i++)
                    if (better(wbest[i].l, wbest[i].e, b.l, b.e))
                        b = wbest[i];
                chosen[j] = b.e;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            double p[Q8S_MAX_K_DEV];
            double kept = 0.0;
            for (int j = 0; j < k; j++) {
                p[j] = exp(l[chosen[j]] - mx) / zsum;
                kept += p[j];
            }
            for (int j = 0; j < k; j++) {
                idx[(int64_t)(r0 + r) * k + j] = chosen[j];
                wts[(int64_t)(r0 + r) * k + j] = (float)(p[j] / kept);
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0)
        counters[blockIdx.y] = 0;
}

hipError_t route_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                        float *wts, void *scratch, hipStream_t st)
{
    int *counters = reinterpret_cast<int *>(scratch);
    double *logits = reinterpret_cast<double *>(reinterpret_cast<char *>(scratch) + align256(ROUTE_COUNTER_BYTES));
    const unsigned gx = (unsigned)((E + ROUTE_WAVES - 1) / ROUTE_WAVES);
    if (rows == 1) {
        hipLaunchKernelGGL((k_route<1>), dim3(gx, 1), dim3(ROUTE_THREADS), 0, st, x, Wr, (int)rows, (int)d, (int)E,
                           (int)k, logits, counters, idx, wts);
    } else {
        hipLaunchKernelGGL((k_route<4>), dim3(gx, (unsigned)((rows + 3) / 4)), dim3(ROUTE_THREADS), 0, st, x, Wr,
                           (int)rows, (int)d, (int)E, (int)k, logits, counters, idx, wts);
    }
    return hipGetLastError();
}

} // namespace q8s
