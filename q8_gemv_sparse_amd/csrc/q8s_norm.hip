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
#include "q8s_norm_row.h"

namespace q8s {

// SEGS > 0: the row has at most SEGS 2048-value segments (NormShare).
// SEGS == 0: any length; the second pass re-forms the sums from h and r (the
// same float32 adds, bit for bit).
template <int SEGS>
__global__ void __launch_bounds__(NORM_THREADS) k_add_rmsnorm_q8(const float *__restrict__ h, const float *__restrict__ r,
                                                                 const float *__restrict__ w, int d, float eps,
                                                                 float *__restrict__ sum, float *__restrict__ y,
                                                                 int8_t *__restrict__ yq, float *__restrict__ ys,
                                                                 int8_t *__restrict__ yl)
{
    constexpr int NS = SEGS > 0 ? SEGS : 1;
    __shared__ double wsum[NORM_THREADS / WAVE];
    const int64_t row = blockIdx.x;
    const float *hr = h + row * d;
    const float *rr = r + row * d;
    const int t8 = threadIdx.x * 8;

    NormShare<NS> n;
    double ss = 0.0;
    if (SEGS > 0) {
        norm_load<NS>(n, hr, rr, w, d, t8);
#pragma unroll
        for (int g = 0; g < NS; g++) {
            const int base = t8 + g * NORM_SEG;
            if (base < d) {
                *reinterpret_cast<f32x4 *>(sum + row * d + base) = n.sv[g][0];
                *reinterpret_cast<f32x4 *>(sum + row * d + base + 4) = n.sv[g][1];
            }
        }
        ss = norm_squares<NS>(n, d, t8);
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
    const double inv = norm_inv(ss, d, eps, wsum);

    for (int g = 0; SEGS > 0 ? g < NS : true; g++) {
        const int base = t8 + g * NORM_SEG;
        if (base >= d)
            break;
        float v[8];
        if (SEGS > 0) {
            norm_values(n.sv[g][0], n.sv[g][1], n.wv[g][0], n.wv[g][1], inv, v);
        } else {
            norm_values(ldf4(hr + base) + ldf4(rr + base), ldf4(hr + base + 4) + ldf4(rr + base + 4), ldf4(w + base),
                        ldf4(w + base + 4), inv, v);
        }
        if (y) {
            *reinterpret_cast<f32x4 *>(y + row * d + base) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4 *>(y + row * d + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
        if (yq) {
            // with yl: the two-word form (words and scales those of the one-word form)
            if (yl)
                quant8x2_store(v, yq + row * d + base, yl + row * d + base, ys + row * (d / QB) + base / QB,
                               (threadIdx.x & 3) == 0);
            else
                quant8_store(v, yq + row * d + base, ys + row * (d / QB) + base / QB, (threadIdx.x & 3) == 0);
        }
    }
}

// The mixture block's first launch: the add + norm of the row, exactly as
// k_add_rmsnorm_q8 forms it (the same shares, sums and roundings), and one
// router logit per workgroup (fn emit_moe_forward's router over the normed
// row), in double.  The router is RF:
//   0  float32 rows Wr:           l = sum_t Wr[e][t] * y[t]
//   1  Q8_0 rows Wrq/Wrs (lane_link.rs fn prim, Moe arm: quantized checkpoint
//      rows) against the float32 normed row:  l = sum_t (q*s) * y[t]
//   2  Q8_0 rows against the normed row's Q8_0 form (the one-word int8
//      numerics, where every reader of the norm is a Q8_0 projection):
//      l = sum_b (ws*ys) * isum_b, each block's isum exact in int32
// Every workgroup of a row forms the whole normed row -- it re-reads h, r and
// w, 24 bytes a value, mostly from cache -- so no workgroup waits for another;
// the workgroup of expert 0 also writes the sum and the activation the gate-up
// launch reads (float32 x and/or its Q8_0 form, whichever is given).
template <int SEGS, int RF>
__global__ void __launch_bounds__(NORM_THREADS)
    k_norm_logits(const float *__restrict__ h, const float *__restrict__ r, const float *__restrict__ w, int d,
                  float eps, const float *__restrict__ Wr, const int8_t *__restrict__ Wrq,
                  const float *__restrict__ Wrs, int E, float *__restrict__ sum, float *__restrict__ x,
                  int8_t *__restrict__ xq, float *__restrict__ xs, double *__restrict__ logits,
                  int8_t *__restrict__ xl)
{
    __shared__ double wsum[NORM_THREADS / WAVE];
    __shared__ double lsum[NORM_THREADS / WAVE];
    const int e = blockIdx.x;
    const int64_t row = blockIdx.y;
    const bool writer = e == 0;
    const int t8 = threadIdx.x * 8;
    const int nb = d / QB;

    // h, r and w first, then the router row: waits on the vector-memory
    // counter are in issue order, so the norm can start once its (cached)
    // inputs land while the router row is still streaming in
    NormShare<SEGS> n;
    f32x4 rr4[SEGS][2];
    norm_load_raw<SEGS>(n, rr4, h + row * d, r + row * d, w, d, t8);
    f32x4 rv[SEGS][2];
    uint2 rq[SEGS];
    float rs[SEGS];
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        const int base = min(t8 + g * NORM_SEG, d - 8);  // no branch: see norm_load_raw
        if (RF == 0) {
            const float *wr = Wr + (int64_t)e * d + base;
            rv[g][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wr));
            rv[g][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wr + 4));
        } else {
            const uint64_t q = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(Wrq + (int64_t)e * d + base));
            rq[g] = make_uint2((uint32_t)q, (uint32_t)(q >> 32));
            rs[g] = __builtin_nontemporal_load(Wrs + (int64_t)e * nb + base / QB);
        }
    }
    norm_add<SEGS>(n, rr4, d, t8);
    if (writer) {
#pragma unroll
        for (int g = 0; g < SEGS; g++) {
            const int base = t8 + g * NORM_SEG;
            if (base < d) {
                *reinterpret_cast<f32x4 *>(sum + row * d + base) = n.sv[g][0];
                *reinterpret_cast<f32x4 *>(sum + row * d + base + 4) = n.sv[g][1];
            }
        }
    }
    const double inv = norm_inv(norm_squares<SEGS>(n, d, t8), d, eps, wsum);

    double lg = 0.0;
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        const int base = t8 + g * NORM_SEG;
        if (base < d) {
            float v[8];
            norm_values(n.sv[g][0], n.sv[g][1], n.wv[g][0], n.wv[g][1], inv, v);
            if (RF == 0) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    lg += (double)rv[g][0][i] * (double)v[i];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    lg += (double)rv[g][1][i] * (double)v[4 + i];
            } else if (RF == 1) {
                const double s = (double)rs[g];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const int q = (int)(int8_t)(((i < 4 ? rq[g].x : rq[g].y) >> (8 * (i & 3))) & 0xFF);
                    lg += ((double)q * s) * (double)v[i];
                }
            }
            if (writer && x) {
                *reinterpret_cast<f32x4 *>(x + row * d + base) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(x + row * d + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
            if (RF == 2 || (writer && xq)) {
                float ys;
                const uint2 c = quant8(v, ys);
                const bool leader = (threadIdx.x & 3) == 0;
                // two words (xl given): the low words, written and dotted
                const uint2 lw = xl ? low8(v, c, ys) : make_uint2(0u, 0u);
                if (writer && xq) {
                    *reinterpret_cast<uint2 *>(xq + row * d + base) = c;
                    if (xl)
                        *reinterpret_cast<uint2 *>(xl + row * d + base) = lw;
                    if (leader)
                        xs[row * nb + base / QB] = ys;
                }
                if (RF == 2) {
                    // the block's exact dots: this thread's 8 products, then
                    // the four threads of the block (integer adds); the low
                    // words' dot is weighed 1/128 (zero in one word)
                    int is = __builtin_amdgcn_sdot4((int)c.x, (int)rq[g].x, 0, false);
                    is = __builtin_amdgcn_sdot4((int)c.y, (int)rq[g].y, is, false);
                    is += dpp_i<DPP_XOR1>(is);
                    is += dpp_i<DPP_XOR2>(is);
                    int il = __builtin_amdgcn_sdot4((int)lw.x, (int)rq[g].x, 0, false);
                    il = __builtin_amdgcn_sdot4((int)lw.y, (int)rq[g].y, il, false);
                    il += dpp_i<DPP_XOR1>(il);
                    il += dpp_i<DPP_XOR2>(il);
                    if (leader)
                        lg += ((double)rs[g] * (double)ys) * ((double)is + (double)il / 128.0);
                }
            }
        }
    }
    lg = wave_sum_f64(lg);
    if ((threadIdx.x & 63) == 0)
        lsum[threadIdx.x >> 6] = lg;
    __syncthreads();
    if (threadIdx.x == 0)
        logits[row * E + e] = ((lsum[0] + lsum[1]) + lsum[2]) + lsum[3];
}

// q8_quantize_rows: the same epilogue on a given f32 row set.  Threads own 8
// values of the rows taken as one array (n is a multiple of 32, so a block
// never straddles two rows and block b of the array is block b of xs), so
// every thread of every workgroup has work whatever n is: 512 hidden rows of
// 768 values are 192 full workgroups, not 512 of which 62 % sat idle.
__global__ void __launch_bounds__(NORM_THREADS) k_quantize_rows(const float *__restrict__ x, int64_t total,
                                                                int8_t *__restrict__ xq, float *__restrict__ xs)
{
    const int64_t base = ((int64_t)blockIdx.x * NORM_THREADS + threadIdx.x) * 8;
    if (base >= total)
        return;  // whole 4-thread groups leave together: total is a multiple of 32
    const f32x4 a0 = ldf4(x + base), a1 = ldf4(x + base + 4);
    const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    quant8_store(v, xq + base, xs + base / QB, (threadIdx.x & 3) == 0);
}

// q8_quantize_rows_x2: the two-word form, the same grid (words and scales
// equal k_quantize_rows', plus the low words).
__global__ void __launch_bounds__(NORM_THREADS) k_quantize_rows_x2(const float *__restrict__ x, int64_t total,
                                                                   int8_t *__restrict__ xq, int8_t *__restrict__ xl,
                                                                   float *__restrict__ xs)
{
    const int64_t base = ((int64_t)blockIdx.x * NORM_THREADS + threadIdx.x) * 8;
    if (base >= total)
        return;  // whole 4-thread groups leave together: total is a multiple of 32
    const f32x4 a0 = ldf4(x + base), a1 = ldf4(x + base + 4);
    const float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    quant8x2_store(v, xq + base, xl + base, xs + base / QB, (threadIdx.x & 3) == 0);
}

hipError_t quantize_launch(const float *x, int64_t rows, int64_t n, int8_t *xq, float *xs, hipStream_t st)
{
    const int64_t total = rows * n;
    const dim3 grid((unsigned)((total + 8 * NORM_THREADS - 1) / (8 * NORM_THREADS)));
    hipLaunchKernelGGL(k_quantize_rows, grid, dim3(NORM_THREADS), 0, st, x, total, xq, xs);
    return hipGetLastError();
}

hipError_t quantize_x2_launch(const float *x, int64_t rows, int64_t n, int8_t *xq, int8_t *xl, float *xs,
                              hipStream_t st)
{
    const int64_t total = rows * n;
    const dim3 grid((unsigned)((total + 8 * NORM_THREADS - 1) / (8 * NORM_THREADS)));
    hipLaunchKernelGGL(k_quantize_rows_x2, grid, dim3(NORM_THREADS), 0, st, x, total, xq, xl, xs);
    return hipGetLastError();
}

hipError_t add_rmsnorm_launch(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              float *sum, float *y, int8_t *yq, float *ys, hipStream_t st, int8_t *yl)
{
    const int segs = (int)((d + NORM_SEG - 1) / NORM_SEG);
    const dim3 grid((unsigned)rows), block(NORM_THREADS);
    if (segs <= 1)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<1>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys, yl);
    else if (segs <= 2)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<2>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys, yl);
    else if (segs <= 4)
        hipLaunchKernelGGL((k_add_rmsnorm_q8<4>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys, yl);
    else
        hipLaunchKernelGGL((k_add_rmsnorm_q8<0>), grid, block, 0, st, h, r, w, (int)d, eps, sum, y, yq, ys, yl);
    return hipGetLastError();
}

bool norm_logits_supported(int64_t d) { return d <= NORM_LOGITS_MAX_D; }

namespace {

template <int RF>
void norm_logits_go(int segs, dim3 grid, hipStream_t st, const float *h, const float *r, const float *w, int d,
                    float eps, const RouterRows &rt, int E, float *sum, float *x, int8_t *xq, float *xs,
                    double *logits, int8_t *xl)
{
    const dim3 block(NORM_THREADS);
    if (segs <= 1)
        hipLaunchKernelGGL((k_norm_logits<1, RF>), grid, block, 0, st, h, r, w, d, eps, rt.Wr, rt.Wrq, rt.Wrs, E, sum,
                           x, xq, xs, logits, xl);
    else if (segs <= 2)
        hipLaunchKernelGGL((k_norm_logits<2, RF>), grid, block, 0, st, h, r, w, d, eps, rt.Wr, rt.Wrq, rt.Wrs, E, sum,
                           x, xq, xs, logits, xl);
    else
        hipLaunchKernelGGL((k_norm_logits<4, RF>), grid, block, 0, st, h, r, w, d, eps, rt.Wr, rt.Wrq, rt.Wrs, E, sum,
                           x, xq, xs, logits, xl);
}

} // namespace

hipError_t norm_logits_launch(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              const RouterRows &rt, int64_t E, float *sum, float *x, int8_t *xq, float *xs,
                              double *logits, hipStream_t st, int8_t *xl)
{
    const int segs = (int)((d + NORM_SEG - 1) / NORM_SEG);
    const dim3 grid((unsigned)E, (unsigned)rows);
    if (!rt.Wrq)
        norm_logits_go<0>(segs, grid, st, h, r, w, (int)d, eps, rt, (int)E, sum, x, xq, xs, logits, xl);
    else if (rt.act == 0)
        norm_logits_go<1>(segs, grid, st, h, r, w, (int)d, eps, rt, (int)E, sum, x, xq, xs, logits, xl);
    else
        norm_logits_go<2>(segs, grid, st, h, r, w, (int)d, eps, rt, (int)E, sum, x, xq, xs, logits, xl);
    return hipGetLastError();
}

} // namespace q8s
