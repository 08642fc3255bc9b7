/*
 * q8s.h -- C ABI of the Q8_0 GEMV / sparse mixture-of-experts library for
 * MI355X (gfx950).  libq8s.so exports exactly the functions declared here.
 *
 * Sources, cited by page and item (the text of each page is the authority on
 * what an operation computes):
 *   - codegen_cuda::qwen_emit module page: struct Q8Ref (Q8_0 rows: int8 quants
 *     row-major plus one f32 scale per 32 inputs, W[o][t] = q[o*in+t] *
 *     s[o*nb + t/32]); struct MoeWeights (stacked experts, router [E,d],
 *     gate/up [E*dff,d], down [E*d,dff], expert e's rows from e*dff or e*d);
 *     fn emit_moe_forward (router GEMV, softmax top-K, renormalise, SwiGLU per
 *     kept expert with an expert-indexed weight base, weighted combine);
 *     enum Q8MatKind and fn moe_dp4a_kernels (router + top-K, then quantise,
 *     gate-up-SwiGLU, down-combine).
 *   - codegen_cuda/forward_shim.rs: module doc (sum + RMS norm as one row
 *     kernel writing the sum; the Q8_0 activation quantised in its producer's
 *     epilogue; every stage reads and writes whole buffers); fn kernel_refusal
 *     (no bias on an RMSNorm or a mixture; renormalised softmax routing over
 *     every expert); fn numerics (32-bit integer accumulators).
 *   - codegen_cuda/lane_link.rs: fn prim, Moe arm (refuses more than 32 kept
 *     experts or more than 8192 experts); Matmul arm (weight rows are the
 *     outputs).
 *   - codegen_cuda/lane/arena.rs: fn scratch (router logits, choices,
 *     weights, an arrival counter left zero by the launch that uses it,
 *     per-choice results of a chunk's mixture) and const ALIGN.
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device addresses (e.g. torch.cuda
 *     tensors' data_ptr()).  The caller allocates and owns every buffer --
 *     inputs, outputs and scratch; the library allocates nothing and keeps
 *     no device state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no call synchronises the host.
 *   - Layouts are row-major and dense.  A Q8_0 matrix [n_out, n_in] is a
 *     pair: quants int8 [n_out, n_in] and scales f32 [n_out, n_in/32].  A
 *     Q8_0 activation row set [rows, n] is int8 [rows, n] + f32 [rows, n/32].
 *   - Every reduced dimension (n_in, d, dff, n) is a positive multiple of 32.
 *     Every pointer is 16-byte aligned.  Outputs never overlap inputs or each
 *     other (whole buffers).  Sizes are 64-bit.
 *   - Validation happens on the host, before any HIP call: a refused call
 *     returns a negative Q8S_E* code, enqueues nothing and leaves a message
 *     naming the violated rule in q8s_last_error() (thread-local).  A launch
 *     failure returns Q8S_ELAUNCH with the HIP error string.
 *   - `act` picks the activation numerics (enum Q8MatKind): Q8S_ACT_F32 reads
 *     f32 activations; Q8S_ACT_INT8 reads one-word Q8_0 activations and forms
 *     exact int32 dots per 32-value block.  The two-word activation (act 2)
 *     has entry points of its own (the *_x2 calls) and is taken by the
 *     whole-block calls (moe_ffn_block, moe_ffn_block_ex, moe_ffn_stack,
 *     moe_ffn_block_noalloc); every other call refuses act 2.
 *   - Expert choices (idx) are read on the device.  An index outside [0, E)
 *     is never dereferenced: that choice contributes zero.
 */
#ifndef Q8S_H
#define Q8S_H

#include <stddef.h>
#include <stdint.h>

/* Entry points keep default visibility; the library hides everything else. */
#if defined(__GNUC__) || defined(__clang__)
#define Q8S_API __attribute__((visibility("default")))
#else
#define Q8S_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define Q8S_OK 0
#define Q8S_EINVAL (-1)       /* null pointer, bad shape, overlapping buffers */
#define Q8S_EUNSUPPORTED (-2) /* outside the kernels' limits or an unknown mode */
#define Q8S_EALIGN (-3)       /* a pointer not 16-byte aligned */
#define Q8S_ESCRATCH (-4)     /* scratch missing or smaller than q8s_scratch_bytes */
#define Q8S_ELAUNCH (-5)      /* the HIP launch failed */

#define Q8S_ACT_F32 0  /* f32 activations (dequantise in kernel) */
#define Q8S_ACT_INT8 1 /* one-word Q8_0 int8 activations */
#define Q8S_ACT_X2 2   /* two-word int8 activations (the *_x2 calls and the whole-block calls) */

/* Ids of the calls that take scratch, for q8s_scratch_bytes. */
#define Q8S_FN_ROUTE 1
#define Q8S_FN_DOWN 2
#define Q8S_FN_BLOCK 3
#define Q8S_FN_STACK 4

#define Q8S_MAX_K 32
#define Q8S_MAX_E 8192

/* The static scratch of moe_ffn_block_noalloc, bytes per GPU (32 MiB). */
#define Q8S_NOALLOC_SCRATCH_BYTES (32ll << 20)

/*
 * q8_gemv -- Q8_0 matrix times activation rows (struct Q8Ref; fn prim,
 * Matmul arm: weight rows are outputs).
 *   y[r][o] = sum_t Wq[o][t] * Ws[o][t/32] * x[r][t]      (act = F32)
 *   y[r][o] = sum_b Ws[o][b] * xs[r][b] * isum(r,o,b),     (act = INT8)
 *             isum(r,o,b) = sum_{t in b} Wq[o][t]*xq[r][t] exact in int32
 * Wq: device int8 [n_out, n_in]; Ws: device f32 [n_out, n_in/32].
 * x: device f32 [m, n_in] (F32; NULL otherwise).  xq/xs: device int8
 * [m, n_in] / f32 [m, n_in/32] (INT8; NULL otherwise).  y: device f32
 * [m, n_out], written whole.  m >= 1.  Each weight row is read from HBM once
 * per call for m <= 4 (register path) and for any m in INT8 mode (matrix-core
 * path for m >= 5).  Limits: n_in <= 65536.
 */
Q8S_API int q8_gemv(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in,
            const float *x, const int8_t *xq, const float *xs, int64_t m,
            float *y, int act, void *stream);

/*
 * q8_quantize_rows -- the Q8_0 activation quantiser ("quantize" of the
 * quantise/gate-up/down trio, fn moe_dp4a_kernels; llama.cpp's one int8 word,
 * enum Q8MatKind), per 32-value block, all in float32:
 *   amax = max|v|; d = amax/127; id = d ? 1/d : 0;
 *   q = clamp(round-half-away-from-zero(v*id), -127, 127)
 * x: device f32 [rows, n]; xq: device int8 [rows, n]; xs: device f32
 * [rows, n/32].
 */
Q8S_API int q8_quantize_rows(const float *x, int64_t rows, int64_t n, int8_t *xq, float *xs, void *stream);

/*
 * q8_quantize_rows_x2 -- the two-word (~14-bit) int8 activation (the lane's
 * default numerics, codegen_cuda/lane/mod.rs module doc, CudaKnobs
 * `activations`; arena.rs fn quant_parts: a quantised array's words, its low
 * words, one f32 scale a block).  Per 32-value block, in float32:
 *   d, id and the words q exactly as q8_quantize_rows;
 *   lo = clamp(round-half-away((v*id - q) * 128), -127, 127)
 * so v ~= d * (q + lo/128).  The low word's weight of 1/128 of a step is a
 * reading: the pages print the two words and the one scale, not that weight.
 * x: device f32 [rows, n]; xq, xl: device int8 [rows, n]; xs: device f32
 * [rows, n/32].  Limits as q8_quantize_rows.
 */
Q8S_API int q8_quantize_rows_x2(const float *x, int64_t rows, int64_t n, int8_t *xq, int8_t *xl, float *xs,
                                void *stream);

/*
 * q8_gemv_x2 -- the Q8_0 GEMV with two-word int8 activations (fn
 * moe_dp4a_kernels' two-pass, logit-exact numerics): two exact int32 block
 * dots a block, one against the words and one against the low words,
 *   y[r][o] = sum_b Ws[o][b] * xs[r][b] * (isum_hi[b] + isum_lo[b] / 128)
 * Wq/Ws as q8_gemv; xq/xl/xs as q8_quantize_rows_x2 writes them, m rows;
 * y: device f32 [m, n_out].  Below five rows the vector units form the two
 * dots; from five rows on, the matrix cores (v_mfma_i32_16x16x32_i8 twice a
 * block, words and low words against the same weight fragment), each exact
 * int32.  Limits as q8_gemv.
 */
Q8S_API int q8_gemv_x2(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in, const int8_t *xq,
                       const int8_t *xl, const float *xs, int64_t m, float *y, void *stream);

/*
 * add_rmsnorm_q8 -- residual add + weighted RMSNorm as one row kernel that
 * writes the sum (forward_shim.rs module doc, add_norm), quantising its
 * output to Q8_0 in its epilogue:
 *   sum = h + r                                       (float32 add, written)
 *   y   = (sum / sqrt(mean(sum^2) + eps)) * w          (double inside the row,
 *                                                      rounded to float32)
 *   yq, ys = Q8_0(y) by the q8_quantize_rows rule
 * h, r: device f32 [rows, d]; w: device f32 [d]; sum: device f32 [rows, d]
 * (required); y: device f32 [rows, d] or NULL; yq/ys: device int8 [rows, d]
 * and f32 [rows, d/32], both or neither.  At least one of y, yq is given.
 * eps >= 0.  Limits: d <= 65536.
 */
Q8S_API int add_rmsnorm_q8(const float *h, const float *r, const float *w, int64_t rows, int64_t d,
                   float eps, float *sum, float *y, int8_t *yq, float *ys, void *stream);

/*
 * add_rmsnorm_q8_x2 -- add_rmsnorm_q8 with the normed rows' two-word form
 * (the lane's default activations, codegen_cuda/lane/mod.rs module doc;
 * arena.rs fn quant_parts) written in the same epilogue:
 *   sum, y          exactly as add_rmsnorm_q8
 *   yq, yl, ys      exactly as q8_quantize_rows_x2(y) writes them (yq and ys
 *                   equal add_rmsnorm_q8's one-word form)
 * One launch where add_rmsnorm_q8 followed by q8_quantize_rows_x2 is two.
 * h, r, w, sum as add_rmsnorm_q8; y: device f32 [rows, d] or NULL; yq, yl:
 * device int8 [rows, d]; ys: device f32 [rows, d/32] (all three required).
 * eps >= 0.  Limits as add_rmsnorm_q8.
 */
Q8S_API int add_rmsnorm_q8_x2(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              float *sum, float *y, int8_t *yq, int8_t *yl, float *ys, void *stream);

/*
 * moe_route_topk -- the mixture's router and top-K (fn emit_moe_forward:
 * softmax, keep K, renormalise; fn kernel_refusal: no bias, a softmax over
 * every expert):
 *   l[r][e] = sum_t Wr[e][t] * x[r][t]   (double sums)
 *   p = softmax_e(l[r]);  idx[r] = the K largest l, ties to the lower index,
 *   in rank order;  wts[r][j] = p[idx[r][j]] / sum_{i<K} p[idx[r][i]]
 * x: device f32 [rows, d] (the router reads f32 x in both numerics);
 * Wr: device f32 [E, d]; idx: device int32 [rows, k]; wts: device f32
 * [rows, k].  1 <= k <= min(32, E), E <= 8192.
 * scratch: device, >= q8s_scratch_bytes(Q8S_FN_ROUTE, ...) bytes, 256-byte
 * aligned: the rows' double-precision logits (arena.rs fn scratch, `rl`);
 * no initial contents are needed.  Two kernels run, logits then top-K.
 * Non-finite logits have a defined rank at every E: a NaN ranks above every
 * number when its sign bit is clear and below every number when it is set,
 * ties to the lower index; a kept NaN makes every kept weight NaN.  The
 * choices are always K distinct experts.
 */
Q8S_API int moe_route_topk(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k,
                   int32_t *idx, float *wts, void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_route_topk_gemv -- moe_route_topk of a chunk's rows and a dense Q8_0
 * projection of the same rows in one call (a prefill chunk runs each
 * projection of the step over the block of rows, codegen_cuda/lane/mod.rs
 * module doc; the router and a projection that reads the same normed rows,
 * such as a shared expert's gate and up or a dense layer beside the mixture,
 * are independent of each other):
 *   idx, wts      exactly as moe_route_topk(x, Wr, ...) writes them
 *   y = D . x     exactly as q8_gemv(Dq, Ds, n_out, d, xq, xs, act = INT8)
 *                 (act 1) or q8_gemv_x2(Dq, Ds, n_out, d, xq, xl, xs) (act 2)
 *                 writes it, each element bit for bit
 * The top-K runs inside the projection's launch: its workgroups rank the
 * rows' logits while their first weight tiles are in flight, so the call is
 * two launches (logits, then projection + top-K) where the two calls are
 * three.  This holds from 5 rows up with E <= 256; otherwise the call runs
 * the two calls' launches in turn, with the same results.
 * x: device f32 [rows, d] (the router's input); Wr: device f32 [E, d];
 * idx/wts: device int32/f32 [rows, k]; Dq: device int8 [n_out, d]; Ds:
 * device f32 [n_out, d/32]; xq/xs: device int8 [rows, d] and f32
 * [rows, d/32], x's Q8_0 form (add_rmsnorm_q8's epilogue, q8_quantize_rows
 * or q8_quantize_rows_x2); xl: device int8 [rows, d], the low words, for
 * act 2 and NULL for act 1; y: device f32 [rows, n_out].  act: 1 or 2 (the
 * f32 mode is refused with Q8S_EUNSUPPORTED).  scratch as moe_route_topk.
 * Limits: those of moe_route_topk and q8_gemv; every output is disjoint
 * from every input.
 */
Q8S_API int moe_route_topk_gemv(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k,
                                int32_t *idx, float *wts, const int8_t *Dq, const float *Ds, int64_t n_out,
                                const int8_t *xq, const int8_t *xl, const float *xs, float *y, int act,
                                void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_gate_up -- each kept expert's gate and up projections with SiLU gating
 * (fn emit_moe_forward; struct MoeWeights stacked rows, expert base taken from
 * idx on the device):
 *   for every row r, slot j (e = idx[r][j]), output o < dff:
 *     g = Wg[e*dff + o] . x[r],  u = Wu[e*dff + o] . x[r]
 *     h[r][j][o] = SiLU(g) * u,   SiLU(z) = z / (1 + exp(-z))
 *   INT8: the dots read x's Q8_0 form (xq/xs, written by add_rmsnorm_q8's
 *   epilogue or q8_quantize_rows), and the hidden row is also written in its
 *   Q8_0 form, each 32-value block of each (r, j) row quantised by the
 *   q8_quantize_rows rule from the float32 h (arena.rs fn scratch: hq/hs).
 * x: device f32 [rows, d] (F32) or NULL; xq/xs: device Q8_0 [rows, d] (INT8)
 * or NULL.  Wgq/Wuq: device int8 [E*dff, d]; Wgs/Wus: device f32
 * [E*dff, d/32].  idx: device int32 [rows, k].  h: device f32
 * [rows, k, dff] (required for F32, and for INT8 with rows > 1, where the
 * grouped chunk kernels stage the float32 hidden rows in it before a quantise
 * pass forms hq/hs; optional for INT8 with one row).  hq/hs: device int8
 * [rows, k, dff] and f32 [rows, k, dff/32] (INT8 only; required, except that
 * a chunk of rows in the grouped kernels may pass both NULL to write only the
 * float32 rows and quantise them itself with q8_quantize_rows).  A choice
 * whose expert index is invalid gets zeros.
 * This replaces the plainer form
 *   moe_gate_up(x, xq, xs, Wgq, Wgs, Wuq, Wus, idx, rows, d, dff, E, k, h,
 *               act, scratch, scratch_bytes, stream)
 * in two ways: it also returns the hidden rows' Q8_0 form (hq, hs), which the
 * int8 down projection reads (arena.rs fn scratch keeps hq/hs beside h); and
 * it takes no scratch, because each (expert, tile) workgroup of a chunk
 * gathers its own choices on the device, so no grouping state passes between
 * calls.
 */
Q8S_API int moe_gate_up(const float *x, const int8_t *xq, const float *xs,
                const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                const int32_t *idx, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                float *h, int8_t *hq, float *hs, int act, void *stream);

/*
 * moe_down_combine -- each kept expert's down projection, weighted and
 * summed in slot order (fn emit_moe_forward):
 *   y[r][o] = sum_{j<K} wts[r][j] * (Wd[e*d + o] . h[r][j]),  e = idx[r][j]
 * F32 reads h: device f32 [rows, k, dff].  INT8 reads the hidden row's Q8_0
 * form hq/hs (device int8 [rows, k, dff], f32 [rows, k, dff/32], as
 * moe_gate_up writes it) and forms exact int32 block dots.  Wdq: device int8
 * [E*d, dff]; Wds: device f32 [E*d, dff/32]; idx/wts: device [rows, k];
 * y: device f32 [rows, d].  scratch: device, >= q8s_scratch_bytes(Q8S_FN_DOWN,
 * ...) bytes, 256-byte aligned (zero bytes when rows == 1, where NULL is
 * accepted): per-choice results of a chunk, combined per row in slot order.
 * This replaces the plainer form
 *   moe_down_combine(h, Wdq, Wds, idx, wts, rows, d, dff, E, k, y, act,
 *                    scratch, scratch_bytes, stream)
 * by also taking hq/hs, the hidden rows' Q8_0 form from moe_gate_up: in INT8
 * the down projection reads those, not h (h may then be NULL).  The scratch
 * carries only this call's per-choice results, never state from the gate-up.
 */
Q8S_API int moe_down_combine(const float *h, const int8_t *hq, const float *hs,
                     const int8_t *Wdq, const float *Wds, const int32_t *idx, const float *wts,
                     int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                     float *y, int act, void *scratch, size_t scratch_bytes, void *stream);

/*
 * add_rmsnorm_gemv -- add_rmsnorm_q8 feeding a Q8_0 projection, as one call
 * (forward_shim.rs module doc: the sum and the norm as one row kernel, the
 * Q8_0 activation quantised in its producer's epilogue; struct Q8Ref):
 *   sum, y (and/or yq, ys) exactly as add_rmsnorm_q8 writes them;
 *   out[r] = Q8_0(Wq, Ws) . y[r]          (act = F32, as q8_gemv)
 *   out[r] = Q8_0(Wq, Ws) . Q8_0(y[r])    (act = INT8, as q8_gemv)
 * For one row of d <= 4096 it is one launch: every workgroup forms the normed
 * row itself (re-reading h, r and w, mostly from cache) while its weight rows
 * stream in.  Otherwise it runs add_rmsnorm_q8 then q8_gemv.
 * h, r: device f32 [rows, d]; w: device f32 [d]; Wq: device int8
 * [n_out, d]; Ws: device f32 [n_out, d/32]; sum: device f32 [rows, d]; y:
 * device f32 [rows, d], required for F32, optional for INT8; yq/ys: device
 * int8 [rows, d] and f32 [rows, d/32], both or neither, required for INT8;
 * out: device f32 [rows, n_out].  eps >= 0.  Limits as add_rmsnorm_q8 and
 * q8_gemv.
 */
Q8S_API int add_rmsnorm_gemv(const float *h, const float *r, const float *w, float eps,
                     const int8_t *Wq, const float *Ws, int64_t rows, int64_t d, int64_t n_out,
                     float *sum, float *y, int8_t *yq, float *ys, float *out, int act, void *stream);

/*
 * add_rmsnorm_gemv_x2 -- add_rmsnorm_gemv in two-word int8 numerics: sum and
 * y exactly as add_rmsnorm_q8 writes them, (yq, yl, ys) the two-word form of
 * y as q8_quantize_rows_x2 writes it, and
 *   out[r] = Q8_0(Wq, Ws) . X2(y[r])         (as q8_gemv_x2)
 * For one row of d <= 4096 it is one launch: every workgroup forms the normed
 * row's two-word form in LDS while its weight rows stream in.  Otherwise it
 * runs add_rmsnorm_q8, q8_quantize_rows_x2 and q8_gemv_x2.  Every output is
 * required: sum, y: device f32 [rows, d]; yq, yl: device int8 [rows, d]; ys:
 * device f32 [rows, d/32]; out: device f32 [rows, n_out].  Other arguments
 * and limits as add_rmsnorm_gemv.
 */
Q8S_API int add_rmsnorm_gemv_x2(const float *h, const float *r, const float *w, float eps, const int8_t *Wq,
                                const float *Ws, int64_t rows, int64_t d, int64_t n_out, float *sum, float *y,
                                int8_t *yq, int8_t *yl, float *ys, float *out, void *stream);

/*
 * moe_topk_gate_up_x2 -- moe_topk_gate_up in two-word numerics (the
 * mixture's second launch under act 2 of moe_ffn_block): each row's top-K
 * taken from its logits inside every gate-up workgroup, the gate/up dots over
 * the row's two-word form (xq, xl, xs, as q8_quantize_rows_x2 writes it), and
 * each hidden block written in two words (hq, hl, hs; rows of k*dff values).
 * idx/wts: device [rows, k], written.  E <= 256.  Limits as moe_gate_up.
 */
Q8S_API int moe_topk_gate_up_x2(const double *logits, const int8_t *xq, const int8_t *xl, const float *xs,
                                const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                                int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int32_t *idx,
                                float *wts, int8_t *hq, int8_t *hl, float *hs, void *stream);

/*
 * add_rmsnorm_router -- add_rmsnorm_q8 with the mixture's router fused in
 * (forward_shim.rs module doc: the norm as one row kernel writing the sum;
 * fn emit_moe_forward: the router over the normed row):
 *   sum, x (and/or xq, xs) exactly as add_rmsnorm_q8 writes them;
 *   logits[r][e] = sum_t Wr[e][t] * x[r][t]   (double sums)
 * One workgroup per (expert, row) forms the whole normed row itself, so no
 * launch waits for a norm launch.  h, r: device f32 [rows, d]; w: device f32
 * [d]; Wr: device f32 [E, d]; sum: device f32 [rows, d]; x: device f32
 * [rows, d] or NULL; xq/xs: device int8 [rows, d] and f32 [rows, d/32], both
 * or neither; at least one of x, xq.  logits: device double [rows, E] (16-byte
 * aligned).  Limits: d <= 8192 (Q8S_EUNSUPPORTED beyond), E <= 8192.
 */
Q8S_API int add_rmsnorm_router(const float *h, const float *r, const float *w, float eps,
                       const float *Wr, int64_t rows, int64_t d, int64_t E, float *sum,
                       float *x, int8_t *xq, float *xs, double *logits, void *stream);

/*
 * moe_topk_gate_up -- moe_gate_up that takes each row's top-K from the
 * router logits itself (fn emit_moe_forward: softmax, keep K, renormalise):
 *   idx[r], wts[r] = the K largest logits[r] (ties to the lower index, in rank
 *                    order) and their renormalised softmax weights, exactly
 *                    as moe_route_topk forms them from the same logits;
 *   h (and hq/hs)  = as moe_gate_up with those choices.
 * Every gate-up workgroup ranks the row's E logits in LDS, so the choices
 * need no launch of their own.  logits: device double [rows, E] (as
 * add_rmsnorm_router writes them).  Other arguments as moe_gate_up; idx:
 * device int32 [rows, k] and wts: device f32 [rows, k] are outputs here.
 * Rows run one by one (a chunk of rows in INT8 mode reads each expert once
 * per row here; moe_gate_up groups them).  Limits: E <= 256
 * (Q8S_EUNSUPPORTED beyond), k <= min(32, E).  A NaN logit ranks above every
 * number when its sign bit is clear and below every number when it is set;
 * a kept NaN makes every kept weight NaN (the renormalisation sums them).
 * The choices are K distinct experts whatever the logits hold.
 */
Q8S_API int moe_topk_gate_up(const double *logits, const float *x, const int8_t *xq, const float *xs,
                     const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                     int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                     int32_t *idx, float *wts, float *h, int8_t *hq, float *hs, int act, void *stream);

/*
 * moe_ffn_block -- the whole mixture block of one layer as one call: the
 * residual add + RMSNorm row kernel feeding the mixture (forward_shim.rs
 * module doc), then fn emit_moe_forward's router, top-K, gate-up + SiLU and
 * down-combine (the mixture linked as one launch unit: lane_link.rs fn prim,
 * Moe arm).  It computes, for each row r,
 *   sum[r] = h[r] + r[r];  x = RMSNorm(sum[r]) * w       (as add_rmsnorm_q8)
 *   idx[r], wts[r] = top-K of the router over x          (as moe_route_topk)
 *   out[r] = sum_j wts[r][j] * down_e(SiLU(gate_e x) * up_e x), e = idx[r][j]
 *                                                        (as moe_gate_up then
 *                                                         moe_down_combine)
 * with the same numerics as that sequence of calls in mode `act` (INT8: x and
 * each hidden row in Q8_0 form, exact int32 block dots; the router always
 * reads f32 x).  h, r: device f32 [rows, d]; w: device f32 [d]; Wr: device
 * f32 [E, d]; gate/up/down: as moe_gate_up and moe_down_combine.  Outputs:
 * sum (the residual stream, f32 [rows, d]), idx (int32 [rows, k]), wts (f32
 * [rows, k]), out (f32 [rows, d], the mixture's output).  scratch: device,
 * >= q8s_scratch_bytes(Q8S_FN_BLOCK, ...) bytes, 256-byte aligned, no initial
 * contents needed; it holds the logits, the normed row and its Q8_0 form and
 * the hidden rows between the launches.  Decode rows run three launches
 * (add_rmsnorm_router, moe_topk_gate_up, moe_down_combine); a chunk of rows
 * in INT8 mode, E > 256 or d > 8192 run add_rmsnorm_q8, moe_route_topk,
 * moe_gate_up and moe_down_combine.  eps >= 0; limits as moe_route_topk and
 * moe_gate_up.
 * act = 2 runs the block in two-word numerics (fn moe_dp4a_kernels'
 * two-pass, logit-exact trio): x and each hidden block in two words (as
 * q8_quantize_rows_x2), two exact int32 dots a block (as q8_gemv_x2), the
 * router still reading f32 x.  A chunk of rows (rows > 1, d <= 2048,
 * dff <= 4096) runs the grouped kernels in two words, each chosen expert's
 * weights read once (as moe_gate_up_x2 then moe_down_combine_x2); other
 * rows take the three-launch form (E <= 256, d <= 8192, each row's weights
 * read for that row); anything else is Q8S_EUNSUPPORTED.  moe_ffn_block_ex
 * takes act 2 the same way, its Q8_0 router reading the row's two words (two
 * exact dots a block) and its shared expert in two words.  The other mixture
 * calls refuse act 2.
 */
Q8S_API int moe_ffn_block(const float *h, const float *r, const float *w, float eps, const float *Wr,
                  const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                  const int8_t *Wdq, const float *Wds, int64_t rows, int64_t d, int64_t dff,
                  int64_t E, int64_t k, float *sum, int32_t *idx, float *wts, float *out, int act,
                  void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_route_topk_q8 -- moe_route_topk over a router held as Q8_0 rows
 * (lane_link.rs fn prim, Moe arm: the router as quantized checkpoint rows;
 * struct Q8Ref's layout):
 *   F32:  l[r][e] = sum_t (Wrq[e][t] * Wrs[e][t/32]) * x[r][t]   (double)
 *   INT8: l[r][e] = sum_b (Wrs[e][b] * xs[r][b]) * isum_b, each isum_b the
 *         exact int32 dot of a 32-value block of Wrq[e] and xq[r], scaled and
 *         summed in double (the one-word int8 numerics, where a norm whose
 *         readers are all Q8_0 projections is read in its Q8_0 form only:
 *         lane_link.rs fn only_projections)
 *   then the softmax, top-K and weights exactly as moe_route_topk.
 * x: device f32 [rows, d] (F32) or NULL; xq/xs: device int8 [rows, d] and
 * f32 [rows, d/32] (INT8) or NULL.  Wrq: device int8 [E, d]; Wrs: device f32
 * [E, d/32].  idx, wts, scratch (q8s_scratch_bytes(Q8S_FN_ROUTE, ...)) and
 * limits as moe_route_topk.
 */
Q8S_API int moe_route_topk_q8(const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq,
                      const float *Wrs, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                      float *wts, int act, void *scratch, size_t scratch_bytes, void *stream);

/*
 * add_rmsnorm_router_q8 -- add_rmsnorm_router over Q8_0 router rows:
 *   sum, x (and/or xq, xs) exactly as add_rmsnorm_q8 writes them;
 *   logits[r] as moe_route_topk_q8 forms them, from the normed row (F32) or
 *   from its Q8_0 form (INT8: each workgroup quantises the normed row by the
 *   q8_quantize_rows rule itself, whether or not xq is requested).
 * Wrq: device int8 [E, d]; Wrs: device f32 [E, d/32]; other arguments and
 * limits as add_rmsnorm_router.
 */
Q8S_API int add_rmsnorm_router_q8(const float *h, const float *r, const float *w, float eps,
                          const int8_t *Wrq, const float *Wrs, int64_t rows, int64_t d, int64_t E,
                          float *sum, float *x, int8_t *xq, float *xs, double *logits, int act,
                          void *stream);

/*
 * moe_gate_up_x2, moe_down_combine_x2 -- moe_gate_up and moe_down_combine in
 * two-word numerics (fn moe_dp4a_kernels' two-pass, logit-exact trio; arena.rs
 * fn quant_parts: words, low words, one scale a block): the activation is
 * xq/xl/xs (as q8_quantize_rows_x2 writes it), each block's value two exact
 * int32 dots joined as 128 * isum + isum_lo and scaled by ws * xs / 128 (as
 * q8_gemv_x2), the hidden rows quantised in two words (hq/hl/hs, device int8
 * [rows, k, dff] twice and f32 [rows, k, dff/32]).  A chunk of rows (rows > 1,
 * d <= 2048, dff <= 4096) runs the grouped kernels, each chosen expert's
 * weights read once: moe_gate_up_x2 then requires h (device f32
 * [rows, k, dff], the float32 hidden rows it stages) and may leave out
 * hq/hl/hs; moe_down_combine_x2 needs scratch of
 * q8s_scratch_bytes(Q8S_FN_DOWN, ..., Q8S_ACT_X2).  Other arguments, limits
 * and refusals as moe_gate_up / moe_down_combine in INT8 mode.
 */
Q8S_API int moe_gate_up_x2(const int8_t *xq, const int8_t *xl, const float *xs, const int8_t *Wgq, const float *Wgs,
                           const int8_t *Wuq, const float *Wus, const int32_t *idx, int64_t rows, int64_t d,
                           int64_t dff, int64_t E, int64_t k, float *h, int8_t *hq, int8_t *hl, float *hs,
                           void *stream);
Q8S_API int moe_down_combine_x2(const int8_t *hq, const int8_t *hl, const float *hs, const int8_t *Wdq,
                                const float *Wds, const int32_t *idx, const float *wts, int64_t rows, int64_t d,
                                int64_t dff, int64_t E, int64_t k, float *y, void *scratch, size_t scratch_bytes,
                                void *stream);

/*
 * moe_ffn_stack -- `layers` mixture blocks in a row, each layer with weights
 * of its own, as one call (forward_shim.rs module doc: the sum and the RMS
 * norm of it as one row kernel; the whole forward captured as one graph):
 *   s_0 = h + r
 *   for l = 0 .. layers-1:  x_l = RMSNorm(s_l) * w[l]   (as moe_ffn_block)
 *                           m_l = mixture_l(x_l)        (router Wr[l], experts
 *                                                        Wgq[l] .. Wds[l])
 *                           s_{l+1} = s_l + m_l         (a float32 add)
 *   out = s_layers (the residual stream after the last layer)
 * The residual add of layer l is deferred into layer l + 1's add + norm row
 * kernel (it reads m_l and s_l and forms their sum), and the last layer's is
 * folded into its down-combine epilogue: each layer is moe_ffn_block's
 * launches, nothing in between, so out equals the chain of moe_ffn_block
 * calls (h = m_{l-1}, r = s_{l-1}) followed by one float32 add, bit for bit.
 * h, r: device f32 [rows, d]; w, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds: HOST
 * arrays of `layers` device pointers, each as moe_ffn_block's argument of
 * that name.  Outputs: out (device f32 [rows, d]); idx (device int32
 * [layers, rows, k]) and wts (device f32 [layers, rows, k]), each layer's
 * choices.  scratch: device, >= q8s_scratch_bytes(Q8S_FN_STACK, ...) bytes,
 * 256-byte aligned, no initial contents needed.  1 <= layers <= 1024; other
 * limits and numerics (act 0, 1 or 2) as moe_ffn_block.
 */
Q8S_API int moe_ffn_stack(const float *h, const float *r, int64_t layers, const float *const *w,
                          const float *const *Wr, const int8_t *const *Wgq, const float *const *Wgs,
                          const int8_t *const *Wuq, const float *const *Wus, const int8_t *const *Wdq,
                          const float *const *Wds, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                          float eps, float *out, int32_t *idx, float *wts, int act, void *scratch,
                          size_t scratch_bytes, void *stream);

/*
 * moe_ffn_block_noalloc -- moe_ffn_block without a scratch argument and
 * without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments (less scratch), outputs, numerics, kernels and
 * limits as moe_ffn_block; the scratch those kernels use is a fixed array of
 * Q8S_NOALLOC_SCRATCH_BYTES in device memory that the library holds on each
 * GPU it runs on until the process ends.  Sizes whose
 * q8s_scratch_bytes(Q8S_FN_BLOCK, ...) exceed it are refused with
 * Q8S_EUNSUPPORTED before any HIP call.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress), so make one call
 * outside any graph capture first.  The array needs no initial contents and
 * keeps the last call's; every call on one GPU shares it, so calls that
 * overlap on one GPU (on different streams, or from several threads) race:
 * order them on one stream.  It calls no device allocation of any kind
 * (hipMalloc, hipFree or an allocating library routine).
 */
Q8S_API int moe_ffn_block_noalloc(const float *h, const float *r, const float *w, float eps, const float *Wr,
                                  const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                                  const int8_t *Wdq, const float *Wds, int64_t rows, int64_t d, int64_t dff,
                                  int64_t E, int64_t k, float *sum, int32_t *idx, float *wts, float *out, int act,
                                  void *stream);

/*
 * moe_ffn_block_ex -- moe_ffn_block with the variants linked into the
 * mixture's launch (lane_link.rs fn prim, Moe arm; fn class_launch,
 * SharedExpertFusion arm; arena.rs fn scratch, Moe arm):
 *   - the router: float32 rows Wr (Wrq, Wrs NULL), or Q8_0 rows Wrq/Wrs (Wr
 *     NULL), read as moe_route_topk_q8 reads them in mode act (INT8: the
 *     normed row's Q8_0 form);
 *   - a shared expert when sdff > 0: an always-on SwiGLU expert of width
 *     sdff -- Sgq/Suq device int8 [sdff, d], Sgs/Sus device f32
 *     [sdff, d/32], Sdq device int8 [d, sdff], Sds device f32 [d, sdff/32] --
 *     whose output is added, unweighted, after the routed sum:
 *       out[r] = (sum_j wts[r][j] * down_e(...)) + Sd . (SiLU(Sg x) * (Su x))
 *     its hidden row in the routed experts' numerics.  sdff == 0 (the six
 *     pointers NULL): no shared expert.
 * scratch: >= q8s_block_scratch_bytes(rows, d, dff, sdff, E, k, act) bytes.
 * Other arguments, outputs and limits as moe_ffn_block; sdff a multiple of
 * 32, at most 65536, and the down-combine holds at most 512 (slot, slice)
 * partials (Q8S_EUNSUPPORTED beyond).  Decode rows run three launches, the
 * shared expert's tiles inside the gate-up launch and its slices inside the
 * down-combine; a chunk of rows in INT8 mode runs it after the grouped
 * kernels as a gate-up and a down-combine that adds into out.
 */
Q8S_API int moe_ffn_block_ex(const float *h, const float *r, const float *w, float eps, const float *Wr,
                     const int8_t *Wrq, const float *Wrs, const int8_t *Wgq, const float *Wgs,
                     const int8_t *Wuq, const float *Wus, const int8_t *Wdq, const float *Wds,
                     const int8_t *Sgq, const float *Sgs, const int8_t *Suq, const float *Sus,
                     const int8_t *Sdq, const float *Sds, int64_t sdff, int64_t rows, int64_t d,
                     int64_t dff, int64_t E, int64_t k, float *sum, int32_t *idx, float *wts, float *out,
                     int act, void *scratch, size_t scratch_bytes, void *stream);

/*
 * moe_topk_gate_up_ex -- moe_topk_gate_up with a shared expert (lane_link.rs
 * fn class_launch, SharedExpertFusion arm): the same launch also forms the
 * shared expert's hidden row
 *   h[r][k*dff + o] = SiLU(Sg[o] . x[r]) * (Su[o] . x[r]),   o < sdff
 * after the K routed ones, so h (and hq/hs) hold k*dff + sdff values a row.
 * Sgq/Suq: device int8 [sdff, d]; Sgs/Sus: device f32 [sdff, d/32]; sdff a
 * multiple of 32, or 0 with the four pointers NULL (then exactly
 * moe_topk_gate_up).  Other arguments and limits as moe_topk_gate_up; rows
 * run one by one.
 */
Q8S_API int moe_topk_gate_up_ex(const double *logits, const float *x, const int8_t *xq, const float *xs,
                        const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                        const int8_t *Sgq, const float *Sgs, const int8_t *Suq, const float *Sus,
                        int64_t sdff, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                        int32_t *idx, float *wts, float *h, int8_t *hq, float *hs, int act, void *stream);

/*
 * moe_down_combine_ex -- moe_down_combine with a shared expert's down row
 * added, unweighted, after the routed sum (as moe_ffn_block_ex):
 *   y[r][o] = (sum_{j<K} wts[r][j] * (Wd[e*d + o] . h[r][j])) + Sd[o] . h[r][K]
 * h (or hq/hs) as moe_topk_gate_up_ex writes it: k*dff + sdff values a row.
 * Sdq: device int8 [d, sdff]; Sds: device f32 [d, sdff/32]; sdff 0 with both
 * NULL: no shared expert.  Rows run one by one (no scratch); other arguments
 * and limits as moe_down_combine.
 */
Q8S_API int moe_down_combine_ex(const float *h, const int8_t *hq, const float *hs,
                        const int8_t *Wdq, const float *Wds, const int8_t *Sdq, const float *Sds,
                        int64_t sdff, const int32_t *idx, const float *wts, int64_t rows, int64_t d,
                        int64_t dff, int64_t E, int64_t k, float *y, int act, void *stream);

/* Bytes of scratch moe_ffn_block_ex needs for these sizes (0 for invalid). */
Q8S_API size_t q8s_block_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t sdff, int64_t E, int64_t k,
                               int act);

/*
 * q8s_scratch_bytes -- bytes of scratch the call `fn` (Q8S_FN_ROUTE,
 * Q8S_FN_DOWN or Q8S_FN_BLOCK) needs for these sizes; 0 for a call that needs
 * none, or for an unknown fn.
 */
Q8S_API size_t q8s_scratch_bytes(int fn, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act);

/*
 * q8s_moe_path -- which kernels the mixture's expert stages run for these
 * sizes (lane/mod.rs module doc: decode rows one by one, prefill chunks
 * grouped by expert; lane_link.rs fn class_launch: a chunk's mixture over its
 * rows sorted by expert).  It covers moe_gate_up, moe_down_combine (and their
 * _x2 forms), moe_ffn_block and moe_ffn_stack, whose routed stages follow
 * the same rule:
 *   Q8S_PATH_ROWS          the decode kernels, row by row (one row, float32
 *                          activations, or rows past the grouped kernels'
 *                          limits: d > 2048 or dff > 4096);
 *   Q8S_PATH_GROUPED       choices grouped by expert, each expert's weights
 *                          read once a chunk, on the vector units (v_dot4);
 *   Q8S_PATH_GROUPED_MFMA  the same grouping on the matrix cores, from 8
 *                          choices an expert on average (rows*k >= 8*E), with
 *                          d and dff multiples of 256 and 16 staged rows of
 *                          max(d, dff) values (two words: twice the bytes)
 *                          within 64 KiB.
 * Host logic only (no device call).  Returns Q8S_EINVAL for non-positive
 * sizes, k > E or an unknown act.
 */
#define Q8S_PATH_ROWS 0
#define Q8S_PATH_GROUPED 1
#define Q8S_PATH_GROUPED_MFMA 2
Q8S_API int q8s_moe_path(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act);

/* The message of this thread's last refused or failed call ("" if none). */
Q8S_API const char *q8s_last_error(void);

/* The library's version string. */
Q8S_API const char *q8s_version(void);

/*
 * q8s_stream_read -- the read ceiling the weight streams are measured
 * against.  Every kernel above is bound by the bytes of its weight rows, so a
 * caller timing them can state each one's bandwidth as a fraction of what the
 * plainest reader reaches on the same device.  This call reads `bytes` of
 * device memory at `buf` once, in 16-byte non-temporal loads spread over
 * Q8S_STREAM_WGS workgroups (each a contiguous span, its lanes on
 * consecutive chunks, eight loads in flight a lane), and reduces them (xor of 32-bit words) to one word
 * per workgroup in `out`, so no load can be dropped.  It computes nothing of
 * the method.
 * buf: device, 16-byte aligned, `bytes` a positive multiple of 16; out:
 * device uint32 [Q8S_STREAM_WGS], owned by the caller, disjoint from buf.
 */
#define Q8S_STREAM_WGS 2048
Q8S_API int q8s_stream_read(const void *buf, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8S_H */
