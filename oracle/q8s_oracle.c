/*
 * q8s_oracle.c -- the CPU oracle for the Q8_0 GEMV / sparse-MoE hot path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT.  Only the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the HIP library under
 * q8_gemv_sparse_amd/csrc, and that library never calls it.
 *
 * Every function here is a plain, slow, obviously-correct statement of what the
 * path computes: loops in index order, double precision for every
 * floating-point sum, no blocking, no fusion, no reordering.  Build it with
 * floating-point contraction off and no fast-math (oracle/build.py does), so
 * that the few float32 steps (the residual sum and the activation quantiser)
 * are single IEEE float32 operations.
 *
 * Sources (the pages this follows), cited by page and item:
 *   [Q8Ref]      codegen_cuda::qwen_emit module page, struct Q8Ref:
 *                W[o][t] = quants[o*in + t] * scales[o*nb + t/32].
 *   [MoeWeights] same page, struct MoeWeights: router [E,d], gate/up
 *                [E*dff, d], down [E*d, dff], expert e's rows start at e*dff
 *                (gate/up) or e*d (down).
 *   [emit_moe]   same page, fn emit_moe_forward: router GEMV, top-K route
 *                (softmax, keep K, renormalise), each kept expert's SwiGLU with
 *                an expert-indexed weight base, weighted combine; f32
 *                activations times int8 weights with f64 sums.
 *   [Q8MatKind]  same page, enum Q8MatKind, and codegen_cuda/lane/mod.rs
 *                module doc (CudaKnobs `activations`): f32 activations with
 *                f64 sums, or llama.cpp's one int8 word per activation.
 *   [numerics]   codegen_cuda/forward_shim.rs, impl Shim for ForwardShim,
 *                fn numerics / fn fits: 32-bit integer accumulators.
 *   [add_norm]   codegen_cuda/forward_shim.rs module doc: a sum and the RMS
 *                norm of it as one row kernel writing the sum; a weighted RMS
 *                norm scales and never shifts (fn kernel_refusal).
 *   [epilogue]   codegen_cuda/forward_shim.rs module doc: under the one-word
 *                int8 numerics the activation a Q8_0 projection reads is
 *                quantised in its producer's epilogue.
 *   [variants]   codegen_cuda/lane_link.rs, fn prim (Moe arm: the router as
 *                quantized checkpoint rows or as float values) and fn
 *                class_launch (SharedExpertFusion arm: a shared expert's gated
 *                pair and down product carried by the mixture's launch);
 *                arena.rs fn scratch (Moe arm: K*dff + sdff hidden values).
 *   [scratch]    codegen_cuda/lane/arena.rs, fn scratch / fn array_bytes: a
 *                quantised activation is int8 words plus one f32 scale a
 *                32-value block; the decode mixture keeps its hidden row
 *                quantised (hq/hs) in one-word int8 mode.
 *   [two_word]   codegen_cuda/lane/mod.rs module doc (CudaKnobs
 *                `activations`: a two-word ~14-bit int8 activation) and
 *                arena.rs fn scratch / fn quant_parts / fn array_bytes: under
 *                two words a quantised activation is its words, its low words
 *                and one f32 scale a block; fn moe_dp4a_kernels' two-pass
 *                (logit-exact) trio.
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the project's design notes):
 *   - the activation quantiser is llama.cpp's Q8_0 reference quantiser with an
 *     f32 scale: d = amax/127, id = 1/d (0 when d = 0), q = round-half-away(v*id)
 *     clamped to [-127, 127], every step in float32;
 *   - RMSNorm: y = (s / sqrt(mean(s^2) + eps)) * w, eps inside the root;
 *   - routing ranks by logit, ties to the lower expert index; softmax over all
 *     E experts, then the kept weights renormalised to sum 1;
 *   - a shared expert is added to the mixture's weighted sum with weight 1 (no
 *     gate of its own; the pages decompose a router/shared-gate merge), after
 *     it; a Q8_0 router under one-word int8 numerics reads the quantised row;
 *   - the two-word activation's low word is the rest of v*id after the word,
 *     in 128ths of a step, rounded half away from zero: v ~= d*(q + lo/128);
 *   - SiLU(z) = z / (1 + exp(-z)); the hidden row h = SiLU(g) * u is held as a
 *     float32 tensor between the gate-up and the down projection (and, in int8
 *     mode, quantised per 32-value block of each expert's row).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define QBLOCK 32

/* ---------------------------------------------------------------------------
 * G -- Q8_0 GEMV with f32 activations [Q8Ref], [emit_moe], [Q8MatKind]:
 *   y[r][o] = sum_t (Wq[o*n_in + t] * Ws[o*nb + t/32]) * x[r*n_in + t]
 * every product and the sum in double, t in index order.
 */
void oracle_gemv_f32(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in,
                     const float *x, int64_t m, double *y)
{
    int64_t nb = n_in / QBLOCK;
    for (int64_t r = 0; r < m; r++) {
        for (int64_t o = 0; o < n_out; o++) {
            double acc = 0.0;
            for (int64_t t = 0; t < n_in; t++) {
                double w = (double)Wq[o * n_in + t] * (double)Ws[o * nb + t / QBLOCK];
                acc += w * (double)x[r * n_in + t];
            }
            y[r * n_out + o] = acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Q -- the Q8_0 activation quantiser [Q8MatKind] (llama.cpp's one int8 word),
 * [scratch] (f32 scale per 32 values).  Each 32-value block of each row:
 *   amax = max |v|;  d = amax / 127;  id = d ? 1/d : 0;
 *   q = clamp(round_half_away_from_zero(v * id), -127, 127)
 * all in float32.  roundf rounds halfway cases away from zero.
 */
void oracle_quantize(const float *v, int64_t rows, int64_t n, int8_t *q, float *d)
{
    int64_t nb = n / QBLOCK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *blk = v + r * n + b * QBLOCK;
            float amax = 0.0f;
            for (int t = 0; t < QBLOCK; t++) {
                float a = fabsf(blk[t]);
                if (a > amax)
                    amax = a;
            }
            float dsc = amax / 127.0f;
            float id = (dsc != 0.0f) ? 1.0f / dsc : 0.0f;
            for (int t = 0; t < QBLOCK; t++) {
                float p = blk[t] * id;
                float rq = roundf(p);
                if (rq > 127.0f)
                    rq = 127.0f;
                if (rq < -127.0f)
                    rq = -127.0f;
                q[r * n + b * QBLOCK + t] = (int8_t)rq;
            }
            d[r * nb + b] = dsc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * The exact int32 block dots of the one-word int8 mode [numerics]:
 *   isum[r][o][b] = sum_{t in block b} Wq[o][t] * xq[r][t]
 * |isum| <= 32 * 127 * 127 = 516128, so int32 holds it exactly.
 */
void oracle_block_dots(const int8_t *Wq, int64_t n_out, int64_t n_in, const int8_t *xq,
                       int64_t m, int32_t *isum)
{
    int64_t nb = n_in / QBLOCK;
    for (int64_t r = 0; r < m; r++)
        for (int64_t o = 0; o < n_out; o++)
            for (int64_t b = 0; b < nb; b++) {
                int32_t s = 0;
                for (int t = 0; t < QBLOCK; t++)
                    s += (int32_t)Wq[o * n_in + b * QBLOCK + t] * (int32_t)xq[r * n_in + b * QBLOCK + t];
                isum[(r * n_out + o) * nb + b] = s;
            }
}

/* ---------------------------------------------------------------------------
 * I -- Q8_0 GEMV with one-word int8 activations [Q8MatKind], [numerics]:
 *   y[r][o] = sum_b (Ws[o][b] * xs[r][b]) * isum[r][o][b]
 * the block dots exact in int32, the scaling and the sum over blocks in double.
 */
void oracle_gemv_i8(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in,
                    const int8_t *xq, const float *xs, int64_t m, double *y)
{
    int64_t nb = n_in / QBLOCK;
    for (int64_t r = 0; r < m; r++) {
        for (int64_t o = 0; o < n_out; o++) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                int32_t s = 0;
                for (int t = 0; t < QBLOCK; t++)
                    s += (int32_t)Wq[o * n_in + b * QBLOCK + t] * (int32_t)xq[r * n_in + b * QBLOCK + t];
                acc += ((double)Ws[o * nb + b] * (double)xs[r * nb + b]) * (double)s;
            }
            y[r * n_out + o] = acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * Q2 -- the two-word (~14-bit) int8 activation [two_word]: per 32-value block
 * its words, its low words and one f32 scale.  The words are Q's codes (same
 * d, same id); the low word holds the rest of v*id in 128ths of one step:
 *   p  = v * id                       (float32, as in Q)
 *   q  = Q's code of v
 *   lo = clamp(round_half_away_from_zero((p - q) * 128), -127, 127)
 * so v ~= d * (q + lo/128).  |p - q| <= 1/2, so |lo| <= 64 and the clamp never
 * binds; p - q is exact (Sterbenz) and the factor 128 a power of two, so lo is
 * the nearest 128th of p - q.  The factor is a reading: the pages print the
 * two words and the one scale, not the low word's weight.
 */
void oracle_quantize_x2(const float *v, int64_t rows, int64_t n, int8_t *q, int8_t *lo, float *d)
{
    int64_t nb = n / QBLOCK;
    oracle_quantize(v, rows, n, q, d);
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            float dsc = d[r * nb + b];
            float id = (dsc != 0.0f) ? 1.0f / dsc : 0.0f;
            for (int t = 0; t < QBLOCK; t++) {
                int64_t i = r * n + b * QBLOCK + t;
                float p = v[i] * id;
                float rest = (p - (float)q[i]) * 128.0f;
                float rl = roundf(rest);
                if (rl > 127.0f)
                    rl = 127.0f;
                if (rl < -127.0f)
                    rl = -127.0f;
                lo[i] = (int8_t)rl;
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * I2 -- Q8_0 GEMV with two-word int8 activations [two_word]: two exact int32
 * block dots a block, one against the words and one against the low words,
 *   y[r][o] = sum_b (Ws[o][b] * xs[r][b]) * (isum_hi[b] + isum_lo[b] / 128)
 * the block dots exact in int32, the scaling and the sum over blocks in
 * double (isum_hi + isum_lo/128 is exact in double).
 */
void oracle_gemv_i8x2(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in, const int8_t *xq,
                      const int8_t *xl, const float *xs, int64_t m, double *y)
{
    int64_t nb = n_in / QBLOCK;
    for (int64_t r = 0; r < m; r++) {
        for (int64_t o = 0; o < n_out; o++) {
            double acc = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                int32_t sh = 0, sl = 0;
                for (int t = 0; t < QBLOCK; t++) {
                    int32_t w = (int32_t)Wq[o * n_in + b * QBLOCK + t];
                    sh += w * (int32_t)xq[r * n_in + b * QBLOCK + t];
                    sl += w * (int32_t)xl[r * n_in + b * QBLOCK + t];
                }
                double blk = (double)sh + (double)sl / 128.0;
                acc += ((double)Ws[o * nb + b] * (double)xs[r * nb + b]) * blk;
            }
            y[r * n_out + o] = acc;
        }
    }
}

/* ---------------------------------------------------------------------------
 * N -- residual add + weighted RMSNorm [add_norm]:
 *   sum = h + r                     (one float32 add per element, written)
 *   ms  = (1/d) sum_i sum_i^2       (double, index order)
 *   y   = (sum / sqrt(ms + eps)) * w  computed as (sum * inv) * w in double,
 *         inv = 1 / sqrt(ms + eps)
 * y is returned in double; the path stores it as float32 (and/or its Q8_0 form,
 * [epilogue]), which the caller derives by rounding and oracle_quantize.
 */
void oracle_add_rmsnorm(const float *h, const float *r, const float *w, int64_t rows, int64_t d,
                        float eps, float *sum, double *y)
{
    for (int64_t i = 0; i < rows; i++) {
        double ss = 0.0;
        for (int64_t t = 0; t < d; t++) {
            float s = h[i * d + t] + r[i * d + t];
            sum[i * d + t] = s;
            ss += (double)s * (double)s;
        }
        double ms = ss / (double)d;
        double inv = 1.0 / sqrt(ms + (double)eps);
        for (int64_t t = 0; t < d; t++)
            y[i * d + t] = ((double)sum[i * d + t] * inv) * (double)w[t];
    }
}

/* The softmax, top-K and renormalisation of one row's logits l[E]. */
static void route_row(const double *l, int64_t E, int64_t k, int32_t *idx, double *wts)
{
    double *p = (double *)malloc((size_t)E * sizeof(double));
    char *taken = (char *)calloc((size_t)E, 1);
    double mx = l[0];
    for (int64_t e = 1; e < E; e++)
        if (l[e] > mx)
            mx = l[e];
    double z = 0.0;
    for (int64_t e = 0; e < E; e++) {
        p[e] = exp(l[e] - mx);
        z += p[e];
    }
    for (int64_t e = 0; e < E; e++)
        p[e] = p[e] / z;
    double kept = 0.0;
    for (int64_t j = 0; j < k; j++) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; e++) {
            if (taken[e])
                continue;
            if (best < 0 || l[e] > l[best])
                best = e; /* strict '>' keeps the lower index on a tie */
        }
        taken[best] = 1;
        idx[j] = (int32_t)best;
        kept += p[best];
    }
    for (int64_t j = 0; j < k; j++)
        wts[j] = p[idx[j]] / kept;
    free(p);
    free(taken);
}

/* ---------------------------------------------------------------------------
 * R -- the top-K softmax router [emit_moe] (softmax, keep K, renormalise),
 * forward_shim.rs fn kernel_refusal (no router bias; renormalising; a softmax
 * over every expert, not grouped):
 *   l[e] = sum_t Wr[e][t] * x[t]      (double)
 *   p    = softmax over all E         (double, max subtracted)
 *   idx  = the K experts of largest l, ties to the lower index, in rank order
 *   w[j] = p[idx[j]] / sum_{i<K} p[idx[i]]
 * logits may be NULL.
 */
void oracle_route(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k,
                  int32_t *idx, double *wts, double *logits)
{
    double *l = (double *)malloc((size_t)E * sizeof(double));
    for (int64_t i = 0; i < rows; i++) {
        for (int64_t e = 0; e < E; e++) {
            double acc = 0.0;
            for (int64_t t = 0; t < d; t++)
                acc += (double)Wr[e * d + t] * (double)x[i * d + t];
            l[e] = acc;
            if (logits)
                logits[i * E + e] = acc;
        }
        route_row(l, E, k, idx + i * k, wts + i * k);
    }
    free(l);
}

/* ---------------------------------------------------------------------------
 * R8 -- the router over quantized checkpoint rows (lane_link.rs fn prim, Moe
 * arm: a mixture's router is either quantized rows or float values).  The
 * router rows Wrq/Wrs are a Q8_0 matrix [Q8Ref] of E rows, so the logits are
 * that matrix's GEMV: G over f32 x (act 0), I over the one-word int8
 * activation xq/xs (act 1), or I2 over the two-word one xq/xl/xs (act 2) -- a
 * norm whose readers are all Q8_0 projections is read in its quantised form
 * only under those numerics (lane_link.rs, fn only_projections: a router of
 * float values keeps it f32).  Then the softmax, top-K and renormalisation of
 * R.  logits may be NULL; xl is read under act 2 only.
 */
void oracle_route_q8x(int act, const float *x, const int8_t *xq, const int8_t *xl, const float *xs,
                      const int8_t *Wrq, const float *Wrs, int64_t rows, int64_t d, int64_t E, int64_t k,
                      int32_t *idx, double *wts, double *logits)
{
    double *l = (double *)malloc((size_t)(rows * E) * sizeof(double));
    if (act == 2)
        oracle_gemv_i8x2(Wrq, Wrs, E, d, xq, xl, xs, rows, l);
    else if (act)
        oracle_gemv_i8(Wrq, Wrs, E, d, xq, xs, rows, l);
    else
        oracle_gemv_f32(Wrq, Wrs, E, d, x, rows, l);
    for (int64_t i = 0; i < rows; i++)
        route_row(l + i * E, E, k, idx + i * k, wts + i * k);
    if (logits)
        memcpy(logits, l, (size_t)(rows * E) * sizeof(double));
    free(l);
}

/* R8 in f32 or one-word numerics (act 0 or 1). */
void oracle_route_q8(int act, const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq,
                     const float *Wrs, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx, double *wts,
                     double *logits)
{
    oracle_route_q8x(act, x, xq, NULL, xs, Wrq, Wrs, rows, d, E, k, idx, wts, logits);
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_moe_shared(int act, const float *x, const float *Wr, const int8_t *Wrq, const float *Wrs,
                      const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus, const int8_t *Wdq,
                      const float *Wds, const int8_t *Sgq, const float *Sgs, const int8_t *Suq, const float *Sus,
                      const int8_t *Sdq, const float *Sds, int64_t sdff, int64_t rows, int64_t d, int64_t dff,
                      int64_t E, int64_t k, int32_t *idx, double *wts, float *h, double *y);

/* One expert's SwiGLU FFN on one row, for M and MS: gate/up rows gq/gs, uq/us
 * [n, d], down rows dq/ds [d, n]:
 *   g = Wg . x, u = Wu . x                    (G, or I on Q(x), or I2 on Q2(x))
 *   hj[o] = float32( SiLU(g[o]) * u[o] )      (a float32 tensor)
 *   dn[o'] = Wd[o'] . hj                      (G, or I on Q(hj), or I2 on Q2(hj))
 * act 1 reads the row's Q8_0 form xq/xs, act 2 its two-word form xq/xl/xs. */
static void expert_ffn(int act, const float *xr, const int8_t *xq, const int8_t *xl, const float *xs,
                       const int8_t *gq, const float *gs, const int8_t *uq, const float *us, const int8_t *dq,
                       const float *ds, int64_t d, int64_t n, float *hj, double *dn)
{
    double *g = (double *)malloc((size_t)n * sizeof(double));
    double *u = (double *)malloc((size_t)n * sizeof(double));
    if (act == 0) {
        oracle_gemv_f32(gq, gs, n, d, xr, 1, g);
        oracle_gemv_f32(uq, us, n, d, xr, 1, u);
    } else if (act == 1) {
        oracle_gemv_i8(gq, gs, n, d, xq, xs, 1, g);
        oracle_gemv_i8(uq, us, n, d, xq, xs, 1, u);
    } else {
        oracle_gemv_i8x2(gq, gs, n, d, xq, xl, xs, 1, g);
        oracle_gemv_i8x2(uq, us, n, d, xq, xl, xs, 1, u);
    }
    for (int64_t o = 0; o < n; o++)
        hj[o] = (float)(silu(g[o]) * u[o]);
    if (act == 0) {
        oracle_gemv_f32(dq, ds, d, n, hj, 1, dn);
    } else {
        int8_t *hq = (int8_t *)malloc((size_t)n);
        int8_t *hl = (int8_t *)malloc((size_t)n);
        float *hs = (float *)malloc((size_t)(n / QBLOCK) * sizeof(float));
        if (act == 1) {
            oracle_quantize(hj, 1, n, hq, hs);
            oracle_gemv_i8(dq, ds, d, n, hq, hs, 1, dn);
        } else {
            oracle_quantize_x2(hj, 1, n, hq, hl, hs);
            oracle_gemv_i8x2(dq, ds, d, n, hq, hl, hs, 1, dn);
        }
        free(hq);
        free(hl);
        free(hs);
    }
    free(g);
    free(u);
}

/* ---------------------------------------------------------------------------
 * M -- the sparse MoE FFN block [emit_moe], [MoeWeights], each row apart:
 *   route x (always from the float32 x, [epilogue]: an f32 router reads x);
 *   for each kept expert j (e = idx[j]): h[j], dn[j] = expert_ffn of expert e
 *   y[o'] = sum_{j<K} w[j] * dn[j][o']                  (double, j order)
 * act = 0: f32 activations; act = 1: one-word int8 activations, where x is
 * quantised once per row and each expert's hidden row per 32-value block
 * ([scratch]: hq/hs over K*dff); act = 2: the same in two words ([two_word]:
 * Q2 and I2 in place of Q and I).
 * Outputs: idx [rows*k], wts [rows*k] (double), h [rows*k*dff] (float32),
 * y [rows*d] (double).  Returns 0, or -1 for an unknown mode.
 */
int oracle_moe(int act, const float *x, const float *Wr, const int8_t *Wgq, const float *Wgs,
               const int8_t *Wuq, const float *Wus, const int8_t *Wdq, const float *Wds,
               int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
               int32_t *idx, double *wts, float *h, double *y)
{
    return oracle_moe_shared(act, x, Wr, NULL, NULL, Wgq, Wgs, Wuq, Wus, Wdq, Wds, NULL, NULL, NULL, NULL, NULL,
                             NULL, 0, rows, d, dff, E, k, idx, wts, h, y);
}

/* ---------------------------------------------------------------------------
 * MS -- M with the variants linked into the same mixture launch (lane_link.rs
 * fn prim, Moe arm; fn class_launch, SharedExpertFusion arm; arena.rs
 * fn scratch, Moe arm, whose hidden scratch holds K*dff + sdff values a row):
 *   - the router as Q8_0 rows (Wrq/Wrs, Wr NULL): logits as R8, which under
 *     act 1 reads the row's Q8_0 form; or float32 rows Wr as M;
 *   - a shared expert (sdff > 0): an always-on SwiGLU expert of its own width
 *     sdff -- gate/up Sg/Su [sdff, d], down Sd [d, sdff] -- whose down row is
 *     added, unweighted, to the mixture's sum:
 *       y[o'] = (sum_{j<K} w[j] * dn[j][o']) + dn_s[o']
 *     its hidden row h_s (float32; Q8_0 per block under act 1) after the K
 *     routed ones.
 * h is [rows, K*dff + sdff].  Returns 0, or -1 for an unknown mode.
 */
int oracle_moe_shared(int act, const float *x, const float *Wr, const int8_t *Wrq, const float *Wrs,
                      const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus, const int8_t *Wdq,
                      const float *Wds, const int8_t *Sgq, const float *Sgs, const int8_t *Suq, const float *Sus,
                      const int8_t *Sdq, const float *Sds, int64_t sdff, int64_t rows, int64_t d, int64_t dff,
                      int64_t E, int64_t k, int32_t *idx, double *wts, float *h, double *y)
{
    if (act < 0 || act > 2)
        return -1;
    const int64_t nbd = d / QBLOCK, nbf = dff / QBLOCK, hw = k * dff + sdff;
    int8_t *xq = (int8_t *)malloc((size_t)(rows * d));
    int8_t *xl = (int8_t *)malloc((size_t)(rows * d));
    float *xs = (float *)malloc((size_t)(rows * nbd) * sizeof(float));
    double *dn = (double *)malloc((size_t)d * sizeof(double));

    if (act == 1)
        oracle_quantize(x, rows, d, xq, xs);
    else if (act == 2)
        oracle_quantize_x2(x, rows, d, xq, xl, xs);
    if (Wrq)
        oracle_route_q8x(act, x, xq, xl, xs, Wrq, Wrs, rows, d, E, k, idx, wts, NULL);
    else
        oracle_route(x, Wr, rows, d, E, k, idx, wts, NULL);
    for (int64_t i = 0; i < rows; i++) {
        const float *xr = x + i * d;
        double *yr = y + i * d;
        for (int64_t o = 0; o < d; o++)
            yr[o] = 0.0;
        for (int64_t j = 0; j < k; j++) {
            int64_t e = idx[i * k + j];
            expert_ffn(act, xr, xq + i * d, xl + i * d, xs + i * nbd, Wgq + e * dff * d, Wgs + e * dff * nbd, Wuq + e * dff * d,
                       Wus + e * dff * nbd, Wdq + e * d * dff, Wds + e * d * nbf, d, dff, h + i * hw + j * dff, dn);
            double wj = wts[i * k + j];
            for (int64_t o = 0; o < d; o++)
                yr[o] += wj * dn[o];
        }
        if (sdff > 0) {
            expert_ffn(act, xr, xq + i * d, xl + i * d, xs + i * nbd, Sgq, Sgs, Suq, Sus, Sdq, Sds, d, sdff,
                       h + i * hw + k * dff, dn);
            for (int64_t o = 0; o < d; o++)
                yr[o] += dn[o];
        }
    }
    free(xq);
    free(xl);
    free(xs);
    free(dn);
    return 0;
}
