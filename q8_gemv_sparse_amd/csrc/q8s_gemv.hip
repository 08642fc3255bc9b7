// q8s_gemv.hip -- Q8_0 matrix x activation rows on gfx950.
//
// Three kernels:
//   k_norm_gemv   batch 1 with the residual add + RMSNorm fused in: every
//                 workgroup forms the normed row itself, then streams its
//                 rows against it (no launch waits for a norm launch).
//   k_gemv_rows   the streaming GEMV for batch 1 and small m: weights stream
//                 from HBM once, every activation row a wave serves sits in
//                 its registers.  f32 activations (dequantise in kernel),
//                 one-word int8 activations (v_dot4_i32_i8, exact int32 block
//                 sums) or two-word ones (two exact block dots a block, the
//                 low word's weighed 1/128).  Rows longer than one wave's slice are cut along k
//                 across the waves of a workgroup and joined through LDS in a
//                 fixed order.
//   k_gemm_i8     int8 activations (one or two words) with many rows: v_mfma_i32_16x16x32_i8,
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
                                                    float *__restrict__ y, const int8_t *__restrict__ xl)
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
            if constexpr (ACT == 2)
                load_x2<LPR, C>(xv[r], xq + (int64_t)rr * n_in, xl + (int64_t)rr * n_in, xs + (int64_t)rr * nb, ch0,
                                sl, lig);
            else
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
                float *__restrict__ out, int8_t *__restrict__ yl)
{
    constexpr int G = WAVE / LPR;
    constexpr int RB = G * U;
    constexpr int NX = NORM_SEG * SEGS;
    __shared__ double wsum[NORM_THREADS / WAVE];
    __shared__ __align__(16) float xf[ACT == 0 ? NX : 4];
    __shared__ __align__(16) int8_t xqs[ACT >= 1 ? NX : 16];
    __shared__ __align__(16) int8_t xls[ACT == 2 ? NX : 16];
    __shared__ __align__(16) float xss[ACT >= 1 ? NX / QB : 4];
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
            const bool lead = (threadIdx.x & 3) == 0;
            if (ACT == 0) {
                *reinterpret_cast<f32x4 *>(xf + base) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(xf + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
            } else if (ACT == 1) {
                quant8_store(v, xqs + base, xss + base / QB, lead);
            } else {
                quant8x2_store(v, xqs + base, xls + base, xss + base / QB, lead);
            }
            if (writer && y) {
                *reinterpret_cast<f32x4 *>(y + base) = f32x4{v[0], v[1], v[2], v[3]};
                *reinterpret_cast<f32x4 *>(y + base + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
            if (writer && yq) {
                if (ACT == 2)
                    quant8x2_store(v, yq + base, yl + base, ys + base / QB, lead);
                else
                    quant8_store(v, yq + base, ys + base / QB, lead);
            }
        }
    }
    __syncthreads();
    if (!rows)
        return;
    XSlice<ACT, C> xv;
    if constexpr (ACT == 2)
        load_x2<LPR, C>(xv, xqs, xls, xss, 0, nch, lig);
    else
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
// Workgroup tile: 16 outputs x 16*MT activation rows (MT = 1 or 2 MFMA row
// tiles), eight waves.  k is walked in passes of GemmPass::KB Q8_0 blocks
// (1 KiB of every row; 512 bytes for 32-row tiles in two words).  A pass's operands -- the 16 weight rows, the tile's
// activation rows and both sets of scales -- are read from global memory with
// coalesced 16-byte loads into registers, stored to LDS, and the MFMA
// fragments are read back from LDS.  Two passes are in flight: while a pass is
// contracted, the next one but one is already requested (register double
// buffer), so at the usual n_in of 2048 in one word every global load of the
// workgroup is issued before its first MFMA.
//
// Wave w takes blocks w, w + 8, w + 16, w + 24 of a pass (w, w + 8 at 16
// blocks a pass: the same blocks in the same order over k), for every row tile:
// per block it reads the weight fragment once, and per row tile one
// v_mfma_i32_16x16x32_i8 yields the 16x16 exact int32 block sums, to which
// each lane adds isum * (ws[o][b] * xs[r][b]) for the four (r, o) it holds.
// The eight waves' partials of an output meet in LDS and are summed in wave
// order.
//
// Operand layout of v_mfma_i32_16x16x32_i8 (lane l, j = l%16, g = l/16):
//   A (16x32, rows x k):    A[j][8g .. 8g+7]
//   B (32x16, k x outputs): B[8g .. 8g+7][j]
//   D (16x16):              D[4g + i][j], i < 4
// Both fragments are 8 contiguous bytes of an LDS row: activation row j of
// the tile and weight row j (rows swizzled, gemm_swizzle).

constexpr int GEMM_TN = 16;                    // outputs of a tile
// Q8_0 blocks of k per pass: 32 (1 KiB of a row), 16 for 32-row tiles in two
// words, so the staged words and low words of the 32 rows (32 KiB) leave
// room for two workgroups a CU (at 32 a pass they took 107 KiB of LDS: one a
// CU, and a 64-row chunk's 512 workgroups ran in two rounds)
template <int MT, bool X2>
struct GemmPass {
    static constexpr int KB = (X2 && MT == 2) ? 16 : 32;
    static constexpr int ROW = KB * QB;          // LDS bytes per staged row
    static constexpr int CH = KB * QB / 16;      // 16-byte chunks of a staged row
};
constexpr int GEMM_NW = 8;                     // waves

// LDS rows are stored swizzled in 8-byte units: unit u of row r sits at unit
// u ^ gemm_swizzle(r % 16).  A wave's fragment reads of one block (8 bytes of
// 16 rows, at the same unit) then fall on distinct banks both when 16 lanes
// share 32 banks and when 32 lanes share 64 -- without padding, so the
// staging writes (16-byte units, a permutation of a row) stay whole.
Q8S_DEV int gemm_swizzle(int r) { return 2 * (r & 15) + ((r >> 3) & 1); }

// Stores the row's 16-byte chunk k (units 2k, 2k + 1) at its swizzled place:
// chunk k ^ (s >> 1), its two halves exchanged when s is odd.
Q8S_DEV void put_swizzled(int8_t *row, int r, int k, i32x4 v)
{
    const int sw = gemm_swizzle(r);
    if (sw & 1)
        v = i32x4{v[2], v[3], v[0], v[1]};
    *reinterpret_cast<i32x4 *>(row + 16 * (k ^ (sw >> 1))) = v;
}

// X2: two-word activations, their low words staged beside the words.
template <int MT, bool X2>
struct GemmLds {
    static constexpr int TM = 16 * MT;
    using P = GemmPass<MT, X2>;
    int8_t w[GEMM_TN][P::ROW];
    int8_t a[TM][P::ROW];
    int8_t l[X2 ? TM : 1][P::ROW];
    float ws[P::KB][GEMM_TN + 1];
    float xs[P::KB][TM + 4];
    union {
        float part[GEMM_NW][TM][GEMM_TN + 4];  // row pitch 20: a wave's 64 writes hit 64 banks
        TopkLds tk;                            // the top-K rider's rows, done before the first pass
    };
};

// A pass's global loads of one thread.
template <int MT, bool X2>
struct GemmStage {
    using P = GemmPass<MT, X2>;
    static constexpr int WL = GEMM_TN * P::CH / (GEMM_NW * WAVE);       // weight chunks
    static constexpr int AL = 16 * MT * P::CH / (GEMM_NW * WAVE);       // activation chunks
    static constexpr int XL = 16 * MT * P::KB / (GEMM_NW * WAVE);       // activation scales
    static_assert(WL >= 1 && AL >= 1 && XL >= 1, "every thread stages whole chunks");
    i32x4 w[WL];
    i32x4 a[AL];
    i32x4 l[X2 ? AL : 1];
    float ws;
    float xs[XL];
};

// X2 (two-word activations, the low words xl): a block's two exact int32
// sums, one MFMA each against the same weight fragment, joined as
// 128 * isum + isum_lo (below 2^27 in magnitude) and scaled by ws * xs / 128.
//
// TK: the launch also carries the top-K of `tk.rows` rows of router logits
// (E <= TOPK_LDS_E), as k_topk computes it, so the top-K needs no launch of
// its own.  Workgroup w ranks row w after its first two passes' loads are
// issued, so the ranking runs while they are in flight (its logit requested
// before them, so its wait does not wait for them), and keeps the kept
// choices in LDS; their weights (a double exp each) are formed after the
// contraction, when its registers are free.  Rows past the workgroups (a
// grid smaller than the rows) are ranked at the end.
template <int MT, bool X2, bool TK>
__global__ void __launch_bounds__(GEMM_NW * WAVE)
    k_gemm_i8(const int8_t *__restrict__ Wq, const float *__restrict__ Ws, int n_out, int n_in,
              const int8_t *__restrict__ xq, const float *__restrict__ xs, int m, float *__restrict__ y,
              const int8_t *__restrict__ xl, TopkRider tk)
{
    typedef int v4i __attribute__((ext_vector_type(4)));
    using L = GemmLds<MT, X2>;
    using S = GemmStage<MT, X2>;
    constexpr int TM = L::TM;
    constexpr int GEMM_KB = GemmPass<MT, X2>::KB, GEMM_CH = GemmPass<MT, X2>::CH;
    static_assert(sizeof(TopkLds) <= sizeof(float) * GEMM_NW * TM * (GEMM_TN + 4), "the rider fits the partials");
    static_assert(GEMM_NW * WAVE >= TOPK_LDS_E, "one thread a logit");
    __shared__ __attribute__((aligned(16))) L sm;
    __shared__ TopkKept kept;  // (TK) row w's choices, from the ranking to the weights

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int nb = n_in >> 5, np = (nb + GEMM_KB - 1) / GEMM_KB;
    const int o0 = blockIdx.x * GEMM_TN, r0 = blockIdx.y * TM;

    // Global reads of pass p: chunk c of a staged row is bytes 16c .. 16c+15
    // of the pass's 1 KiB; rows past the matrix and chunks past the row are
    // clamped to the last ones (their products are never used).
    auto issue = [&](S &st, int p) {
        const int64_t bmax = (int64_t)n_in - 16;
        const int64_t k0 = (int64_t)p * GEMM_KB * QB;
#pragma unroll
        for (int i = 0; i < S::WL; i++) {
            const int c = tid + i * GEMM_NW * WAVE;
            const int64_t o = min(o0 + c / GEMM_CH, n_out - 1);
            st.w[i] = ld_stream16(Wq + o * n_in + min(k0 + (c % GEMM_CH) * 16, bmax));
        }
#pragma unroll
        for (int i = 0; i < S::AL; i++) {
            const int c = tid + i * GEMM_NW * WAVE;
            const int64_t r = min(r0 + c / GEMM_CH, m - 1);
            st.a[i] = ld16(xq + r * n_in + min(k0 + (c % GEMM_CH) * 16, bmax));
            if constexpr (X2)
                st.l[i] = ld16(xl + r * n_in + min(k0 + (c % GEMM_CH) * 16, bmax));
        }
        {
            // the tile's GEMM_TN x GEMM_KB scales, one a thread (threads past
            // them, at 16 blocks a pass, reload the last row's)
            const int64_t o = min(o0 + min(tid / GEMM_KB, GEMM_TN - 1), n_out - 1);
            st.ws = ld_stream_f32(Ws + o * nb + min(p * GEMM_KB + tid % GEMM_KB, nb - 1));
        }
#pragma unroll
        for (int i = 0; i < S::XL; i++) {
            const int e = tid + i * GEMM_NW * WAVE;
            const int64_t r = min(r0 + e / GEMM_KB, m - 1);
            st.xs[i] = xs[r * nb + min(p * GEMM_KB + e % GEMM_KB, nb - 1)];
        }
    };
    auto stage = [&](const S &st, int p) {
#pragma unroll
        for (int i = 0; i < S::WL; i++) {
            const int c = tid + i * GEMM_NW * WAVE;
            put_swizzled(&sm.w[c / GEMM_CH][0], c / GEMM_CH, c % GEMM_CH, st.w[i]);
        }
#pragma unroll
        for (int i = 0; i < S::AL; i++) {
            const int c = tid + i * GEMM_NW * WAVE;
            put_swizzled(&sm.a[c / GEMM_CH][0], c / GEMM_CH, c % GEMM_CH, st.a[i]);
            if constexpr (X2)
                put_swizzled(&sm.l[c / GEMM_CH][0], c / GEMM_CH, c % GEMM_CH, st.l[i]);
        }
        // a block past the row gets weight scale 0, so it adds exactly 0
        if (tid < GEMM_KB * GEMM_TN)
            sm.ws[tid % GEMM_KB][tid / GEMM_KB] = p * GEMM_KB + tid % GEMM_KB < nb ? st.ws : 0.0f;
#pragma unroll
        for (int i = 0; i < S::XL; i++) {
            const int e = tid + i * GEMM_NW * WAVE;
            sm.xs[e % GEMM_KB][e / GEMM_KB] = st.xs[i];
        }
    };

    // Branch-free: blocks past the row carry weight scale 0.
    float acc[MT][4];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[t][i] = 0.0f;
    auto contract = [&]() {
        const int sj = gemm_swizzle(j);  // row 16t + j has the same swizzle as row j
#pragma unroll
        for (int q = 0; q < GEMM_KB / GEMM_NW; q++) {
            const int b = wid + GEMM_NW * q;
            const int off = 8 * ((4 * b + g) ^ sj);  // the fragment's 8 bytes in the row
            const long bf = *reinterpret_cast<const long *>(&sm.w[j][off]);
            const float sw = sm.ws[b][j];
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const long af = *reinterpret_cast<const long *>(&sm.a[16 * t + j][off]);
                v4i isum = __builtin_amdgcn_mfma_i32_16x16x32_i8(af, bf, v4i{0, 0, 0, 0}, 0, 0, 0);
                const f32x4 sx = *reinterpret_cast<const f32x4 *>(&sm.xs[b][16 * t + 4 * g]);
                if constexpr (X2) {
                    const long lf = *reinterpret_cast<const long *>(&sm.l[16 * t + j][off]);
                    const v4i ilo = __builtin_amdgcn_mfma_i32_16x16x32_i8(lf, bf, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[t][i] = __builtin_fmaf((float)(isum[i] * 128 + ilo[i]), (sw * sx[i]) * 0.0078125f,
                                                   acc[t][i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[t][i] = __builtin_fmaf((float)isum[i], sw * sx[i], acc[t][i]);
                }
            }
            // one block's fragments live at a time (hoisting every block's
            // LDS reads above the first MFMA costs registers the staging needs)
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto pass = [&](S &st, int p) {
        if (p > 0)
            __syncthreads();  // every wave is done with the previous pass's LDS
        stage(st, p);
        __syncthreads();
        if (p + 2 < np)
            issue(st, p + 2);
        contract();
    };

    const int wg = blockIdx.x + gridDim.x * blockIdx.y, nwg = gridDim.x * gridDim.y;
    double lv = 0.0;
    if constexpr (TK)  // a relaxed atomic load: kept in place, ahead of the passes' loads
        lv = __hip_atomic_load(tk.logits + (int64_t)min(wg, tk.rows - 1) * tk.E + min(tid, tk.E - 1),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    S st0, st1;
    issue(st0, 0);
    if constexpr (TK)
        issue(st1, min(1, np - 1));  // unconditional, so the logit's wait is exact (np = 1 reloads pass 0)
    else if (np > 1)
        issue(st1, 1);
    if constexpr (TK) {
        if (wg < tk.rows) {
            topk_put(sm.tk, lv, tk.E);
            __syncthreads();
            topk_select(sm.tk, tk.E, tk.k);
            __syncthreads();
            if (tid < tk.k) {
                kept.kl[tid] = sm.tk.kl[tid];
                kept.ch[tid] = sm.tk.ch[tid];
            }
            // the first pass's barriers order these before the partials' writes
        }
    }
    for (int p = 0; p < np; p += 2) {
        pass(st0, p);
        if (p + 1 < np)
            pass(st1, p + 1);
    }

    // the waves' partials, summed in wave order
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            sm.part[wid][16 * t + 4 * g + i][j] = acc[t][i];
    __syncthreads();
    for (int e = tid; e < TM * GEMM_TN; e += GEMM_NW * WAVE) {
        const int r = e / GEMM_TN, c = e % GEMM_TN;
        float v = sm.part[0][r][c];
#pragma unroll
        for (int w = 1; w < GEMM_NW; w++)
            v += sm.part[w][r][c];
        if (r0 + r < m && o0 + c < n_out)
            y[(int64_t)(r0 + r) * n_out + o0 + c] = v;
    }
    if constexpr (TK) {
        // the kept choices were written by wave 0's own lanes
        if (wg < tk.rows && tid < WAVE)
            route_finish(kept.kl, kept.ch, tk.k, tk.idx + (int64_t)wg * tk.k, tk.wts + (int64_t)wg * tk.k);
        for (int row = wg + nwg; row < tk.rows; row += nwg) {
            __syncthreads();  // the partials (or the previous row) are read
            topk_load(sm.tk, tk.logits + (int64_t)row * tk.E, tk.E);
            __syncthreads();
            topk_select(sm.tk, tk.E, tk.k);
            __syncthreads();
            if (tid < WAVE)
                route_finish(sm.tk.kl, sm.tk.ch, tk.k, tk.idx + (int64_t)row * tk.k, tk.wts + (int64_t)row * tk.k);
        }
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
                       (int)a.n_in, a.x, a.xq, a.xs, (int)a.m, a.y, a.xl);
    return hipGetLastError();
}

// Activation rows per pass: as many as keep the activation slices in a
// modest register budget (f32 slices are 16 floats a chunk, int8 ones 5
// words).
template <int ACT, int C, bool SPLIT>
constexpr int mr_max()
{
    return ACT >= 1 ? 4 : (SPLIT ? 1 : (C <= 2 ? 4 : 2));
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

namespace {

// The matrix-core path: row tiles of 16 rows for m <= 16, else of 32 (64-row
// tiles would spill registers; two 32-row tiles of the same weights run on
// one XCD, blockIdx.y apart by a multiple of 8 workgroups when n_out is a
// multiple of 128, so the second read of the weights can hit its L2).
template <bool TK>
hipError_t gemm_go(const GemvArgs &a, const TopkRider &tk, hipStream_t st)
{
    const int mt = a.m <= 16 ? 1 : 2;
    const dim3 grid((unsigned)((a.n_out + GEMM_TN - 1) / GEMM_TN), (unsigned)((a.m + 16 * mt - 1) / (16 * mt)));
    const dim3 block(GEMM_NW * WAVE);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, a.Wq, a.Ws, (int)a.n_out, (int)a.n_in, a.xq, a.xs, (int)a.m,
                           a.y, a.xl, tk);
    };
    if (a.act == 2)
        mt == 1 ? go(k_gemm_i8<1, true, TK>) : go(k_gemm_i8<2, true, TK>);
    else
        mt == 1 ? go(k_gemm_i8<1, false, TK>) : go(k_gemm_i8<2, false, TK>);
    return hipGetLastError();
}

} // namespace

hipError_t gemv_launch(const GemvArgs &a, hipStream_t st)
{
    if (a.act >= 1 && a.m >= GEMM_MIN_ROWS)
        return gemm_go<false>(a, TopkRider{}, st);
    const SliceShape sh = slice_shape(a.n_in);
    if (a.act == 2)
        return launch_act<2>(a, sh, st);
    return a.act == 0 ? launch_act<0>(a, sh, st) : launch_act<1>(a, sh, st);
}

bool gemv_topk_fused(int64_t m, int64_t E, int act) { return act >= 1 && m >= GEMM_MIN_ROWS && E <= TOPK_LDS_E; }

hipError_t gemv_topk_launch(const GemvArgs &a, const double *logits, int64_t rows, int64_t E, int64_t k, int32_t *idx,
                            float *wts, hipStream_t st)
{
    return gemm_go<true>(a, TopkRider{logits, (int)rows, (int)E, (int)k, idx, wts}, st);
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
                       a.eps, a.Wq, a.Ws, (int)a.n_out, a.sum, a.y, a.yq, a.ys, a.out, a.yl);
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
    if (a.act == 2)
        return norm_gemv_shape<2>(a, st);
    return a.act == 0 ? norm_gemv_shape<0>(a, st) : norm_gemv_shape<1>(a, st);
}

} // namespace q8s
