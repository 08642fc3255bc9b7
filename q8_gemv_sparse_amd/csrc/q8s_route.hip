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
//             From 16 rows up, k_logits_tile: one workgroup per 4 experts x 4
//             rows, reading each row from cache once for several products.
//   k_topk    one workgroup per row: the K best by (logit descending, index
//             ascending) -- for E <= 256 every logit's exact rank in one pass
//             over order-preserving 64-bit codes (topk_select), beyond that K
//             selection rounds of a workgroup arg-max -- then the kept weights.
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

// The 16 sums v[0..15] of a wave, reduced across its 64 lanes together: each
// exchange halves the values a lane keeps (xor 32, xor 16, then the 16- and
// 8-lane mirrors, whose partners differ in lane bits 3 and 2), and two more
// exchanges (xor 2, xor 1) add the rest, so lane l ends with the whole wave's
// sum of v[(l >> 2) & 15], as do lanes l ^ 1, l ^ 2 and l ^ 3.  Every index is
// summed by the same tree of additions.
Q8S_DEV double wave_sum16_d(const double (&v)[16], int lane)
{
    double w8[8], w4[4], w2[2];
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
#pragma unroll
    for (int i = 0; i < 8; i++)
        w8[i] = (b5 ? v[i + 8] : v[i]) + __shfl_xor(b5 ? v[i] : v[i + 8], 32);
#pragma unroll
    for (int i = 0; i < 4; i++)
        w4[i] = (b4 ? w8[i + 4] : w8[i]) + __shfl_xor(b4 ? w8[i] : w8[i + 4], 16);
#pragma unroll
    for (int i = 0; i < 2; i++)
        w2[i] = (b3 ? w4[i + 2] : w4[i]) + dpp_d<DPP_MIRROR>(b3 ? w4[i] : w4[i + 2]);
    double w = (b2 ? w2[1] : w2[0]) + dpp_d<DPP_HALF_MIRROR>(b2 ? w2[0] : w2[1]);
    w += dpp_d<DPP_XOR2>(w);
    return w + dpp_d<DPP_XOR1>(w);
}

// Many rows (a chunk): one workgroup per tile of LG_E experts x LG_R rows, so
// each router row and activation row it reads from cache serves 4 dot
// products.  A thread takes 8 consecutive values of d per 2048 and keeps the
// 16 products' running sums (double); the sums meet through wave_sum16_d and
// LDS, waves added in order.  (Tiles of 4 experts x 8 rows, 32 sums a thread,
// gave half the workgroups, one a CU with one wave a SIMD, and took the chunk's
// router + dense projection call 0.6 us longer: 12.9 against 12.3 us at 64
// rows, the logits the same to the bit.)
constexpr int LG_E = 4, LG_R = 4;
constexpr int64_t LG_MIN_ROWS = 16;

__global__ void __launch_bounds__(RT_THREADS) k_logits_tile(const float *__restrict__ x, const float *__restrict__ Wr,
                                                            int rows, int d, int E, double *__restrict__ logits)
{
    __shared__ double part[RT_WAVES][LG_E * LG_R];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int e0 = blockIdx.x * LG_E, r0 = blockIdx.y * LG_R;
    double acc[LG_E * LG_R];  // [e][r]
#pragma unroll
    for (int i = 0; i < LG_E * LG_R; i++)
        acc[i] = 0.0;
    // d is a multiple of 32, so a thread's 8 values lie inside the row
    for (int k = threadIdx.x * 8; k < d; k += RT_THREADS * 8) {
        f32x4 w[LG_E][2], xv[LG_R][2];
#pragma unroll
        for (int e = 0; e < LG_E; e++) {
            const float *wp = Wr + (int64_t)min(e0 + e, E - 1) * d + k;
            w[e][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wp));
            w[e][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(wp + 4));
        }
#pragma unroll
        for (int r = 0; r < LG_R; r++) {
            const float *xp = x + (int64_t)min(r0 + r, rows - 1) * d + k;
            xv[r][0] = ldf4(xp);
            xv[r][1] = ldf4(xp + 4);
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int e = 0; e < LG_E; e++) {
                const double we = (double)w[e][i >> 2][i & 3];
#pragma unroll
                for (int r = 0; r < LG_R; r++)
                    acc[e * LG_R + r] += we * (double)xv[r][i >> 2][i & 3];
            }
    }
    const double v = wave_sum16_d(acc, lane);
    if ((lane & 3) == 0)
        part[wid][(lane >> 2) & 15] = v;
    __syncthreads();
    if (threadIdx.x < LG_E * LG_R) {
        const int e = threadIdx.x / LG_R, r = threadIdx.x % LG_R;
        if (e0 + e < E && r0 + r < rows)
            logits[(int64_t)(r0 + r) * E + e0 + e] =
                ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
    }
}

// The logits over Q8_0 router rows (lane_link.rs fn prim, Moe arm: a router
// of quantized checkpoint rows): the same grid, a thread taking one 16-byte
// chunk (half a block) of the row a pass, so a block's halves sit in
// neighbouring lanes.
//   ACT 0: l = sum_t (q*s) * x[t]                       in double
//   ACT 1: l = sum_b (ws*xs) * isum_b, the block's exact int32 dot joined
//          from the two lanes' halves, added by the even lane
//   ACT 2: l = sum_b (ws*xs) * (isum_b + isum_lo_b / 128), the two-word
//          activation's two exact dots a block (words xq, low words xl)
template <int ACT, int RT>
__global__ void __launch_bounds__(RT_THREADS)
    k_logits_q8(const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xs,
                const int8_t *__restrict__ Wrq, const float *__restrict__ Wrs, int rows, int d, int E,
                double *__restrict__ logits, const int8_t *__restrict__ xl)
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
            } else if (ACT == 1) {
                int is = chunk_dot_i8(wv, ld16(xq + xr * d + c * 16));
                is += dpp_i<DPP_XOR1>(is);
                if ((lane & 1) == 0)
                    acc[r] += ((double)s * (double)xs[xr * nb + (c >> 1)]) * (double)is;
            } else {
                int is = chunk_dot_i8(wv, ld16(xq + xr * d + c * 16));
                int il = chunk_dot_i8(wv, ld16(xl + xr * d + c * 16));
                is += dpp_i<DPP_XOR1>(is);
                il += dpp_i<DPP_XOR1>(il);
                if ((lane & 1) == 0)
                    acc[r] += ((double)s * (double)xs[xr * nb + (c >> 1)]) * ((double)is + (double)il / 128.0);
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

// The logit a route_code came from (route_code maps -0 to +0, which no use
// of the kept logits tells apart).
Q8S_DEV double route_decode(uint64_t c)
{
    const uint64_t b = (c >> 63) ? (c & 0x7fffffffffffffffull) : ~c;
    return __longlong_as_double((long long)b);
}

// (code c, index i) ranks before (c2, i2): the greater code, ties to the
// lower index; i2 == INT_MAX stands for no candidate yet.
Q8S_DEV bool code_better(uint64_t c, int i, uint64_t c2, int i2)
{
    return i2 == 0x7fffffff || c > c2 || (c == c2 && i < i2);
}

__global__ void __launch_bounds__(RT_THREADS) k_topk(const double *__restrict__ logits, int E, int k,
                                                     int32_t *__restrict__ idx, float *__restrict__ wts)
{
    extern __shared__ uint64_t Cbig[];  // [E] codes, for rows of more than TOPK_LDS_E logits
    __shared__ TopkLds t;
    __shared__ uint64_t bl[RT_WAVES];
    __shared__ int be[RT_WAVES];
    __shared__ uint32_t retired[Q8S_MAX_E_DEV / 32];
    const int64_t row = blockIdx.x;
    const double *lr = logits + row * E;

    if (E <= TOPK_LDS_E) {
        topk_load(t, lr, E);
        __syncthreads();
        topk_select(t, E, k);
        __syncthreads();
    } else {
        // K rounds of a workgroup arg-max over the logits' order-preserving
        // codes (route_code: NaNs rank above +inf or below -inf by their sign
        // bit, as in the one-pass rank), ties to the lower index; a chosen
        // expert is retired by a flag of its own, so every round picks a new
        // one whatever the logits hold (k <= E)
        for (int i = threadIdx.x; i < E; i += RT_THREADS)
            Cbig[i] = route_code(lr[i]);
        for (int i = threadIdx.x; i < (E + 31) / 32; i += RT_THREADS)
            retired[i] = 0u;
        __syncthreads();
        const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
        for (int jj = 0; jj < k; jj++) {
            uint64_t b = 0;
            int bi = 0x7fffffff;
            for (int i = threadIdx.x; i < E; i += RT_THREADS)
                if (!((retired[i >> 5] >> (i & 31)) & 1u) && code_better(Cbig[i], i, b, bi)) {
                    b = Cbig[i];
                    bi = i;
                }
            for (int o = 32; o >= 1; o >>= 1) {
                const uint64_t b2 = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(b >> 32), o) << 32) |
                                    (uint32_t)__shfl_xor((int)(uint32_t)b, o);
                const int i2 = __shfl_xor(bi, o);
                if (i2 != 0x7fffffff && code_better(b2, i2, b, bi)) {
                    b = b2;
                    bi = i2;
                }
            }
            if (lane == 0) {
                bl[wid] = b;
                be[wid] = bi;
            }
            __syncthreads();
            uint64_t wb = bl[0];
            int wi = be[0];
            for (int w = 1; w < RT_WAVES; w++)
                if (be[w] != 0x7fffffff && code_better(bl[w], be[w], wb, wi)) {
                    wb = bl[w];
                    wi = be[w];
                }
            if (threadIdx.x == 0) {
                t.ch[jj] = wi;
                t.kl[jj] = route_decode(wb);
                retired[wi >> 5] |= 1u << (wi & 31);
            }
            __syncthreads();
        }
    }
    if (threadIdx.x < WAVE)
        route_finish(t.kl, t.ch, k, idx + row * k, wts + row * k);
}

namespace {

hipError_t topk_go(const double *logits, int64_t rows, int64_t E, int64_t k, int32_t *idx, float *wts, hipStream_t st)
{
    const size_t big = E > TOPK_LDS_E ? (size_t)E * sizeof(uint64_t) : 0;
    hipLaunchKernelGGL(k_topk, dim3((unsigned)rows), dim3(RT_THREADS), big, st, logits, (int)E, (int)k, idx, wts);
    return hipGetLastError();
}

} // namespace

hipError_t logits_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, double *logits,
                         hipStream_t st)
{
    static_assert(LG_E * LG_R == 16 && RT_WAVES == 4, "k_logits_tile reduces 16 sums over four waves");
    if (rows == 1)
        hipLaunchKernelGGL((k_logits<1>), dim3((unsigned)E, 1), dim3(RT_THREADS), 0, st, x, Wr, (int)rows, (int)d,
                           (int)E, logits);
    else if (rows >= LG_MIN_ROWS)
        hipLaunchKernelGGL(k_logits_tile, dim3((unsigned)((E + LG_E - 1) / LG_E), (unsigned)((rows + LG_R - 1) / LG_R)),
                           dim3(RT_THREADS), 0, st, x, Wr, (int)rows, (int)d, (int)E, logits);
    else
        hipLaunchKernelGGL((k_logits<4>), dim3((unsigned)E, (unsigned)((rows + 3) / 4)), dim3(RT_THREADS), 0, st, x,
                           Wr, (int)rows, (int)d, (int)E, logits);
    return hipGetLastError();
}

hipError_t route_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                        float *wts, void *scratch, hipStream_t st)
{
    double *logits = reinterpret_cast<double *>(scratch);
    hipError_t err = logits_launch(x, Wr, rows, d, E, logits, st);
    if (err != hipSuccess)
        return err;
    return topk_go(logits, rows, E, k, idx, wts, st);
}

hipError_t route_q8_launch(const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq, const float *Wrs,
                           int64_t rows, int64_t d, int64_t E, int64_t k, int act, int32_t *idx, float *wts,
                           void *scratch, hipStream_t st, const int8_t *xl)
{
    double *logits = reinterpret_cast<double *>(scratch);
    const dim3 block(RT_THREADS);
    const dim3 g1((unsigned)E, (unsigned)rows), g4((unsigned)E, (unsigned)((rows + 3) / 4));
    auto go = [&](auto kernel, dim3 grid) {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, x, xq, xs, Wrq, Wrs, (int)rows, (int)d, (int)E, logits, xl);
    };
    if (act == 0)
        rows == 1 ? go(k_logits_q8<0, 1>, g1) : go(k_logits_q8<0, 4>, g4);
    else if (act == 1)
        rows == 1 ? go(k_logits_q8<1, 1>, g1) : go(k_logits_q8<1, 4>, g4);
    else
        rows == 1 ? go(k_logits_q8<2, 1>, g1) : go(k_logits_q8<2, 4>, g4);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    return topk_go(logits, rows, E, k, idx, wts, st);
}

} // namespace q8s
