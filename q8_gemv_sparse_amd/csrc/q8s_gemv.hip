// q8s_gemv.hip -- Q8_0 matrix x activation rows on gfx950.
//
// Three kernels:
//   k_norm_gemv   batch 1 with the residual add + RMSNorm fused in: every
//                 workgroup forms the normed row itself, then streams its
//                 rows against it (no launch waits for a norm launch).
//   k_gemv_rows   the streaming GEMV for batch 1 and small m: weights stream
//                 from HBM once, every activation row a wave serves sits in
//                 its registers.  f32 activations (dequantise in kernel) or
//                 one-word int8 activations (v_dot4_i32_i8, exact int32 block
//                 sums).  Rows longer than one wave's slice are cut along k
//                 across the waves of a workgroup and joined through LDS in a
//                 fixed order.
//   k_gemm_i8     int8 activations with many rows: v_mfma_i32_16x16x32_i8,
//                 whose k of 32 is one Q8_0 block, so every MFMA result is an
//                 exact int32 block sum that is scaled by its weight and
//                 activation scales in registers (the register-dequant GEMM of
//                 fn emit_marlin_q8_gemm, codegen_cuda::qwen_emit module page).
#include "q8s_device.h"
#include "q8s_internal.h"
#include "q8s_norm_row.h"

namespace q8s {

// ---------------------------------------------------------------------------
// streaming GEMV
//
// Lanes form groups of LPR; a group owns one weight row at a time and each
// lane of it C 16-byte chunks of that row (chunk c*LPR + lane).  A wave step
// covers G = 64/LPR rows, U steps are loaded before any is consumed (so each
// lane has U*C 16-byte loads in flight).  MR activation rows ride along, so
// every weight row is read once for all of them.
//
// SPLIT = false: waves are independent and grid-stride over row blocks.
// SPLIT = true : a workgroup of up to 8 waves shares each row block; the ks
//                chunk slices of the row are dealt to the waves (wave w takes
//                slices w, w + 8, ...); partials meet in LDS and are summed in
//                slice order.

template <int ACT, int LPR, int C, int MR, int U, bool SPLIT>
__global__ void __launch_bounds__(SPLIT ? 512 : 256) k_gemv_rows(const int8_t *__restrict__ Wq, const float *__restrict__ Ws,
                                                    int n_out, int n_in, const float *__restrict__ x,
                                                    const int8_t *__restrict__ xq, const float *__restrict__ xs, int m,
                                                    float *__restrict__ y)
{
    constexpr int G = WAVE / LPR;
    constexpr int RB = G * U;
    const int lane = threadIdx.x & 63, lig = lane % LPR, grp = lane / LPR;
    const int wid = threadIdx.x >> 6;
    const int nch = n_in >> 4, nb = n_in >> 5;
    const int nw = blockDim.x >> 6;
    const int ks = SPLIT ? (nch + LPR * C - 1) / (LPR * C) : 1;
    const int r0 = blockIdx.y * MR;

    // The slice a wave starts on (SPLIT waves loop over slices s, s + nw, ...).
    int s = SPLIT ? wid : 0;
    int ch0 = s * LPR * C;
    int sl = min(LPR * C, nch - ch0);
    XSlice<ACT, C> xv[MR];
    auto load_xs = [&]() {
#pragma unroll
        for (int r = 0; r < MR; r++) {
            const int rr = min(r0 + r, m - 1);
            load_x<LPR, C>(xv[r], ACT == 0 ? x + (int64_t)rr * n_in : nullptr,
                           ACT == 1 ? xq + (int64_t)rr * n_in : nullptr, ACT == 1 ? xs + (int64_t)rr * nb : nullptr,
                           ch0, sl, lig);
        }
    };
    if (!SPLIT || s < ks)
        load_xs();

    __shared__ float part[16][MR][RB];
    const int nrb = (n_out + RB - 1) / RB;
    int64_t rb, step;
    if (SPLIT) {
        rb = blockIdx.x;
        step = gridDim.x;
    } else {
        rb = (int64_t)blockIdx.x * (blockDim.x >> 6) + wid;
        step = (int64_t)gridDim.x * (blockDim.x >> 6);
    }
    for (; rb < nrb; rb += step) {
        for (int sv = SPLIT ? wid : 0; sv < ks; sv += SPLIT ? nw : 1) {
            if (SPLIT && sv != s) {
                s = sv;
                ch0 = s * LPR * C;
                sl = min(LPR * C, nch - ch0);
                load_xs();
            }
            RowSlice<C> w[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int o = min((int)(rb * RB) + u * G + grp, n_out - 1);
                load_row<LPR, C>(w[u], Wq + (int64_t)o * n_in, Ws + (int64_t)o * nb, ch0, sl, lig);
            }
            float acc[MR][U];
#pragma unroll
            for (int r = 0; r < MR; r++)
#pragma unroll
                for (int u = 0; u < U; u++)
                    acc[r][u] = group_sum<LPR>(row_dot(w[u], xv[r], lig));
            if (lig == 0) {
#pragma unroll
                for (int u = 0; u < U; u++) {
                    const int o = (int)(rb * RB) + u * G + grp;
#pragma unroll
                    for (int r = 0; r < MR; r++) {
                        if (SPLIT)
                            part[s][r][u * G + grp] = acc[r][u];
                        else if (o < n_out && r0 + r < m)
                            y[(int64_t)(r0 + r) * n_out + o] = acc[r][u];
                    }
                }
            }
        }
        if (SPLIT) {
            __syncthreads();
            for (int t = threadIdx.x; t < MR * RB; t += blockDim.x) {
                const int r = t / RB, i = t % RB;
                const int o = (int)(rb * RB) + i;
                float v = 0.0f;
                for (int q = 0; q < ks; q++)
                    v += part[q][r][i];
                if (o < n_out && r0 + r < m)
                    y[(int64_t)(r0 + r) * n_out + o] = v;
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// add + norm fused into the batch-1 GEMV
//
// Every 256-thread workgroup requests the row's h, r and w and then its weight
// rows (which do not depend on the norm, so their latency overlaps it), forms
// the row's add + norm exactly as add_rmsnorm_q8 does (q8s_norm_row.h) into
// LDS -- float32, or
// its Q8_0 form in int8 numerics -- and each wave then forms its U row groups'
// dots against the LDS row.  The price of no norm launch is the row's h, r
// and w re-read by every workgroup (12 bytes a value, mostly from cache).  The
// workgroup of row block 0 also writes the sum and the normed row.  The row
// fits one wave's slice (n_in <= 4096) and at most two 2048-value segments.
template <int ACT, int LPR, int C, int SEGS, int U>
__global__ void __launch_bounds__(NORM_THREADS)
    k_norm_gemv(const float *__restrict__ h, const float *__restrict__ r, const float *__restrict__ w, int d,
                float eps, const int8_t *__restrict__ Wq, const float *__restrict__ Ws, int n_out,
                float *__restrict__ sum, float *__restrict__ y, int8_t *__restrict__ yq, float *__restrict__ ys,
                float *__restrict__ out)
{
    constexpr int G = WAVE / LPR;
    constexpr int RB = G * U;
    constexpr int NX = NORM_SEG * SEGS;
    __shared__ double wsum[NORM_THREADS / WAVE];
    __shared__ __align__(16) float xf[ACT == 0 ? NX : 4];
    __shared__ __align__(16) int8_t xqs[ACT == 1 ? NX : 16];
    __shared__ __align__(16) float xss[ACT == 1 ? NX / QB : 4];
    const int lane = threadIdx.x & 63, lig = lane % LPR, grp = lane / LPR;
    const int wid = threadIdx.x >> 6;
    const int nch = d >> 4, nb = d >> 5;
    const bool writer = blockIdx.x == 0;
    const int64_t rb = (int64_t)blockIdx.x * (NORM_THREADS / WAVE) + wid;
    const bool rows = rb * RB < n_out;

    // h, r and w first, then the weight rows: waits on the vector-memory
    // counter are in issue order, so the norm can start once its (cached)
    // inputs land while the weight rows are still streaming in
    const int t8 = threadIdx.x * 8;
    NormShare<SEGS> n;
    f32x4 rr4[SEGS][2];
    norm_load_raw<SEGS>(n, rr4, h, r, w, d, t8);
    RowSlice<C> wr[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int o = min((int)(rb * RB) + u * G + grp, n_out - 1);
        load_row_flat<LPR, C>(wr[u], Wq + (int64_t)o * d, Ws + (int64_t)o * nb, 0, nch, lig);
    }
    norm_add<SEGS>(n, rr4, d, t8);
    if (writer) {
#pragma unroll
        for (int g = 0; g < SEGS; g++) {
            const int base = t8 + g * NORM_SEG;
            if (base < d) {
                *reinterpret_cast<f32x4 *>(sum + base) = n.sv[g][0];
                *reinterpret_cast<f32x4 *>(sum + base + 4) = n.sv[g][1];
            }
        }
    }
    const double inv = norm_inv(norm_squares<SEGS>(n, d, t8), d, eps, wsum);
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        const int base = t8 + g * NORM_SEG;
        if (base < d) {
            float v[8];
            norm_values(n.sv[g][0], n.sv[g][1], n.wv[g][0], n.wv[g][1], inv, v);
            if (ACT == 0) {
                *reinterpret_cast<f32x4 *>(xf + base) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(xf + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
            } else {
                quant8_store(v, xqs + base, xss + base / QB, (threadIdx.x & 3) == 0);
            }
            if (writer && y) {
                *reinterpret_cast<f32x4 *>(y + base) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(y + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
            if (writer && yq)
                quant8_store(v, yq + base, ys + base / QB, (threadIdx.x & 3) == 0);
        }
    }
    __syncthreads();
    if (!rows)
        return;
    XSlice<ACT, C> xv;
    load_x<LPR, C>(xv, xf, xqs, xss, 0, nch, lig);
#pragma unroll
    for (int u = 0; u < U; u++) {
        const float a = group_sum<LPR>(row_dot(wr[u], xv, lig));
        const int o = (int)(rb * RB) + u * G + grp;
        if (lig == 0 && o < n_out)
            out[o] = a;
    }
}

// ---------------------------------------------------------------------------
// int8 MFMA GEMM (m >= GEMM_MIN_ROWS)
//
// Workgroup tile: 16 outputs x 64 rows (four 16-row MFMA tiles); its eight
// waves take interleaved Q8_0 blocks of k (wave w: blocks w, w + 8, ...).  Per
// block and row tile one v_mfma_i32_16x16x32_i8 yields the 16x16 exact int32
// block sums; each lane then adds isum * (ws[o][b] * xs[r][b]) for the four
// (r, o) it holds.  The waves' float partials are summed in wave order
// through LDS.
//
// Latency is the whole cost at these sizes (9.4 MB of weights), so:
//   * every activation scale of the tile goes to LDS once, up front (one
//     barrier, not one per pass of k);
//   * a wave requests all its weight fragments and scales before its first
//     MFMA, in straight-line code (GEMM_WB blocks a wave at most);
//   * activation fragments (from cache) are requested a batch of GEMM_AB
//     blocks ahead of the MFMAs that use them.
//
// Operand layout of v_mfma_i32_16x16x32_i8 (lane l, j = l%16, g = l/16):
//   A (16x32, rows x k):    A[j][8g .. 8g+7]
//   B (32x16, k x outputs): B[8g .. 8g+7][j]
//   D (16x16):              D[4g + i][j], i < 4
// Both operands are read as 8 contiguous bytes of a row: the weight row
// o0 + j and the activation row (tile row j).

constexpr int GEMM_TN = 16;
constexpr int GEMM_TM = 64;
constexpr int GEMM_PB = 64;            // Q8_0 blocks of k per pass
constexpr int GEMM_NW = 8;             // waves (measured 15.5 vs 16.3 us with 4 for the 64-row chunk's projection)
constexpr int GEMM_WQ = GEMM_PB / GEMM_NW;  // blocks of a pass one wave takes
constexpr int GEMM_AB = 4;             // activation blocks requested ahead

__global__ void __launch_bounds__(GEMM_NW * 64) k_gemm_i8(const int8_t *__restrict__ Wq, const float *__restrict__ Ws, int n_out,
                                                 int n_in, const int8_t *__restrict__ xq, const float *__restrict__ xs,
                                                 int m, float *__restrict__ y)
{
    typedef int v4i __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) float xsT[GEMM_PB][GEMM_TM];  // activation scales, block-major
    __shared__ float red[GEMM_NW][GEMM_TM][GEMM_TN + 1];

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int nb = n_in >> 5;
    const int o0 = blockIdx.x * GEMM_TN;
    const int rt0 = blockIdx.y * GEMM_TM;
    const int o = min(o0 + j, n_out - 1);
    const int8_t *wrow = Wq + (int64_t)o * n_in + 8 * g;
    const float *wsrow = Ws + (int64_t)o * nb;
    const int8_t *arow[4];
#pragma unroll
    for (int t = 0; t < 4; t++)
        arow[t] = xq + (int64_t)min(rt0 + 16 * t + j, m - 1) * n_in + 8 * g;

    float acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[t][i] = 0.0f;

    for (int p0 = 0; p0 < nb; p0 += GEMM_PB) {
        // the wave's weight fragments and scales of this pass (blocks
        // p0 + wid + NW q), all requested at once in straight-line code; a block
        // past the row re-reads the row's last block and is not used
        long bfrag[GEMM_WQ];
        float wsc[GEMM_WQ];
#pragma unroll
        for (int q = 0; q < GEMM_WQ; q++) {
            const int b = min(p0 + wid + GEMM_NW * q, nb - 1);
            bfrag[q] = __builtin_nontemporal_load(reinterpret_cast<const long *>(wrow + (int64_t)b * QB));
            wsc[q] = ld_stream_f32(wsrow + b);
        }
        auto load_a = [&](long (&a)[GEMM_AB][4], int q0) {
#pragma unroll
            for (int u = 0; u < GEMM_AB; u++) {
                const int b = min(p0 + wid + GEMM_NW * (q0 + u), nb - 1);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    a[u][t] = *reinterpret_cast<const long *>(arow[t] + (int64_t)b * QB);
            }
        };
        long afrag[2][GEMM_AB][4];
        load_a(afrag[0], 0);
        if (p0 > 0)
            __syncthreads();  // the previous pass is done with xsT
        for (int e = threadIdx.x; e < GEMM_PB * GEMM_TM; e += blockDim.x) {
            const int r = e / GEMM_PB, bb = e % GEMM_PB;
            xsT[bb][r] = xs[(int64_t)min(rt0 + r, m - 1) * nb + min(p0 + bb, nb - 1)];
        }
        __syncthreads();
#pragma unroll
        for (int q0 = 0; q0 < GEMM_WQ; q0 += GEMM_AB) {
            const int cur = (q0 / GEMM_AB) & 1;
            if (q0 + GEMM_AB < GEMM_WQ)
                load_a(afrag[cur ^ 1], q0 + GEMM_AB);
#pragma unroll
            for (int u = 0; u < GEMM_AB; u++) {
                const int q = q0 + u;
                const int bb = wid + GEMM_NW * q;  // block within the pass
                if (p0 + bb < nb) {
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        v4i isum = __builtin_amdgcn_mfma_i32_16x16x32_i8(afrag[cur][u][t], bfrag[q],
                                                                         v4i{0, 0, 0, 0}, 0, 0, 0);
                        const f32x4 sx = *reinterpret_cast<const f32x4 *>(&xsT[bb][16 * t + 4 * g]);
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[t][i] = __builtin_fmaf((float)isum[i], wsc[q] * sx[i], acc[t][i]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            red[wid][16 * t + 4 * g + i][j] = acc[t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < GEMM_TM * GEMM_TN; e += blockDim.x) {
        const int r = e / GEMM_TN, c = e % GEMM_TN;
        float v = red[0][r][c];
#pragma unroll
        for (int w = 1; w < GEMM_NW; w++)
            v += red[w][r][c];
        if (rt0 + r < m && o0 + c < n_out)
            y[(int64_t)(rt0 + r) * n_out + o0 + c] = v;
    }
}

// ---------------------------------------------------------------------------
// host dispatch

namespace {

struct Shape {
    int lpr, c, ks;
};

template <int ACT, int LPR, int C, int MR, bool SPLIT>
hipError_t launch_rows(const GemvArgs &a, int ks, hipStream_t st)
{
    // one or two rows' loads in flight per lane group: at these sizes many
    // waves with few loads each beat fewer waves with more (measured)
    constexpr int U = (C == 1) ? 2 : 1;
    constexpr int RB = (WAVE / LPR) * U;
    const int64_t nrb = (a.n_out + RB - 1) / RB;
    dim3 grid, block;
    if (SPLIT) {
        block = dim3(64 * std::min(ks, 8));
        grid = dim3((unsigned)std::min<int64_t>(nrb, 16384), (unsigned)((a.m + MR - 1) / MR));
    } else {
        block = dim3(256);
        grid = dim3((unsigned)std::min<int64_t>((nrb + 3) / 4, 16384), (unsigned)((a.m + MR - 1) / MR));
    }
    hipLaunchKernelGGL((k_gemv_rows<ACT, LPR, C, MR, U, SPLIT>), grid, block, 0, st, a.Wq, a.Ws, (int)a.n_out,
                       (int)a.n_in, a.x, a.xq, a.xs, (int)a.m, a.y);
    return hipGetLastError();
}

// Activation rows per pass: as many as keep the activation slices in a
// modest register budget (f32 slices are 16 floats a chunk, int8 ones 5
// words).
template <int ACT, int C, bool SPLIT>
constexpr int mr_max()
{
    return ACT == 1 ? 4 : (SPLIT ? 1 : (C <= 2 ? 4 : 2));
}

template <int ACT, int LPR, int C, bool SPLIT>
hipError_t launch_mr(const GemvArgs &a, int ks, hipStream_t st)
{
    constexpr int MRX = mr_max<ACT, C, SPLIT>();
    if (a.m == 1)
        return launch_rows<ACT, LPR, C, 1, SPLIT>(a, ks, st);
    return launch_rows<ACT, LPR, C, MRX, SPLIT>(a, ks, st);
}

template <int ACT>
hipError_t launch_act(const GemvArgs &a, const SliceShape &sh, hipStream_t st)
{
    if (sh.ks > 1)
        return launch_mr<ACT, 64, 4, true>(a, sh.ks, st);
    switch (sh.lpr * 8 + sh.c) {
    case 16 * 8 + 1:
        return launch_mr<ACT, 16, 1, false>(a, 1, st);
    case 16 * 8 + 3:
        return launch_mr<ACT, 16, 3, false>(a, 1, st);
    case 64 * 8 + 1:
        return launch_mr<ACT, 64, 1, false>(a, 1, st);
    case 64 * 8 + 2:
        return launch_mr<ACT, 64, 2, false>(a, 1, st);
    default:
        return launch_mr<ACT, 64, 4, false>(a, 1, st);
    }
}

} // namespace

hipError_t gemv_launch(const GemvArgs &a, hipStream_t st)
{
    if (a.act == 1 && a.m >= GEMM_MIN_ROWS) {
        dim3 grid((unsigned)((a.n_out + GEMM_TN - 1) / GEMM_TN), (unsigned)((a.m + GEMM_TM - 1) / GEMM_TM));
        hipLaunchKernelGGL(k_gemm_i8, grid, dim3(GEMM_NW * 64), 0, st, a.Wq, a.Ws, (int)a.n_out, (int)a.n_in, a.xq, a.xs,
                           (int)a.m, a.y);
        return hipGetLastError();
    }
    const SliceShape sh = slice_shape(a.n_in);
    return a.act == 0 ? launch_act<0>(a, sh, st) : launch_act<1>(a, sh, st);
}

bool norm_gemv_supported(int64_t rows, int64_t d)
{
    return rows == 1 && d <= 2 * 2048 && slice_shape(d).ks == 1;
}

namespace {

template <int ACT, int LPR, int C, int SEGS>
hipError_t norm_gemv_go(const NormGemvArgs &a, hipStream_t st)
{
    // eight (or six) 16-byte loads a lane in flight: U row groups of C chunks
    constexpr int U = C <= 2 ? 4 : 2;
    constexpr int RB = (WAVE / LPR) * U;
    const int64_t nrb = (a.n_out + RB - 1) / RB;
    const dim3 grid((unsigned)((nrb + NORM_THREADS / WAVE - 1) / (NORM_THREADS / WAVE)));
    hipLaunchKernelGGL((k_norm_gemv<ACT, LPR, C, SEGS, U>), grid, dim3(NORM_THREADS), 0, st, a.h, a.r, a.w, (int)a.d,
                       a.eps, a.Wq, a.Ws, (int)a.n_out, a.sum, a.y, a.yq, a.ys, a.out);
    return hipGetLastError();
}

// a row of at most 2048 values is one segment; rows in (2048, 4096] take lane
// groups of 64 with 4 chunks and two segments
template <int ACT>
hipError_t norm_gemv_shape(const NormGemvArgs &a, hipStream_t st)
{
    const SliceShape sh = slice_shape(a.d);
    switch (sh.lpr * 8 + sh.c) {
    case 16 * 8 + 1:
        return norm_gemv_go<ACT, 16, 1, 1>(a, st);
    case 16 * 8 + 3:
        return norm_gemv_go<ACT, 16, 3, 1>(a, st);
    case 64 * 8 + 1:
        return norm_gemv_go<ACT, 64, 1, 1>(a, st);
    case 64 * 8 + 2:
        return norm_gemv_go<ACT, 64, 2, 1>(a, st);
    default:
        return norm_gemv_go<ACT, 64, 4, 2>(a, st);
    }
}

} // namespace

hipError_t norm_gemv_launch(const NormGemvArgs &a, hipStream_t st)
{
    return a.act == 0 ? norm_gemv_shape<0>(a, st) : norm_gemv_shape<1>(a, st);
}

} // namespace q8s
