// q8s_internal.h -- launch-side declarations shared by the library's
// translation units (host code; the C ABI lives in q8s_abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace q8s {

// Most experts kept per row, and most experts (lane_link.rs fn prim, Moe arm).
constexpr int Q8S_MAX_K_DEV = 32;
constexpr int Q8S_MAX_E_DEV = 8192;

// Most experts whose top-K a gate-up workgroup takes itself (one logit per
// thread at least), and the longest row the fused norm + router launch holds
// in registers (four 2048-value segments).
constexpr int ROUTE_FUSED_MAX_E = 256;
constexpr int64_t NORM_LOGITS_MAX_D = 8192;

// Rows from which int8-activation projections go to the MFMA GEMM (below it
// the register GEMV serves up to four rows a pass).
constexpr int64_t GEMM_MIN_ROWS = 5;

// How a row of n_in values is cut for the streaming kernels: lane groups of
// `lpr` lanes holding `c` 16-byte chunks each; `ks` slices (waves) when one
// wave's share (lpr*c chunks) does not cover the row.
struct SliceShape {
    int lpr, c, ks;
};

inline SliceShape slice_shape(int64_t n_in)
{
    const int64_t nch = n_in / 16;
    if (nch <= 16)
        return {16, 1, 1};
    if (nch <= 48)
        return {16, 3, 1};
    if (nch <= 64)
        return {64, 1, 1};
    if (nch <= 128)
        return {64, 2, 1};
    if (nch <= 256)
        return {64, 4, 1};
    return {64, 4, (int)((nch + 255) / 256)};
}

// Longest reduced dimension the streaming kernels take (16 slices of 4096).
constexpr int64_t MAX_NIN = 65536;

struct GemvArgs {
    const int8_t *Wq;
    const float *Ws;
    int64_t n_out, n_in;
    const float *x;
    const int8_t *xq;
    const float *xs;
    int64_t m;
    float *y;
    int act;             // 0 f32, 1 one-word int8, 2 two-word int8
    const int8_t *xl;    // two words: the low words
};
hipError_t gemv_launch(const GemvArgs &a, hipStream_t st);
// The matrix-core GEMM of `a` (act 1 or 2, m >= GEMM_MIN_ROWS) carrying the
// top-K of `rows` rows of E logits (E <= 256): idx/wts as route_launch
// writes them, in the same launch.  gemv_topk_fused says when it applies.
bool gemv_topk_fused(int64_t m, int64_t E, int act);
hipError_t gemv_topk_launch(const GemvArgs &a, const double *logits, int64_t rows, int64_t E, int64_t k, int32_t *idx,
                            float *wts, hipStream_t st);

// add + norm fused into the batch-1 GEMV (one row, d <= 4096)
struct NormGemvArgs {
    const float *h, *r, *w;
    float eps;
    const int8_t *Wq;
    const float *Ws;
    int64_t d, n_out;
    float *sum, *y;
    int8_t *yq;
    float *ys, *out;
    int act;             // 0 f32, 1 one-word int8, 2 two-word int8
    int8_t *yl;          // two words: the normed row's low words
};
bool norm_gemv_supported(int64_t rows, int64_t d);
hipError_t norm_gemv_launch(const NormGemvArgs &a, hipStream_t st);

hipError_t quantize_launch(const float *x, int64_t rows, int64_t n, int8_t *xq, float *xs, hipStream_t st);
hipError_t quantize_x2_launch(const float *x, int64_t rows, int64_t n, int8_t *xq, int8_t *xl, float *xs,
                              hipStream_t st);
hipError_t stream_read_launch(const void *buf, int64_t bytes, uint32_t *out, hipStream_t st);
// with yl (and yq, ys): the normed rows' two-word form in the epilogue
hipError_t add_rmsnorm_launch(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              float *sum, float *y, int8_t *yq, float *ys, hipStream_t st, int8_t *yl = nullptr);
// The router's rows: float32 Wr [E, d], or Q8_0 Wrq [E, d] + Wrs [E, d/32]
// (Wrq non-null); a Q8_0 router reads float32 activations (act 0) or their
// one-word int8 form (act 1).
struct RouterRows {
    const float *Wr;
    const int8_t *Wrq;
    const float *Wrs;
    int act;
};

// add + norm of each row fused with the router's logits (grid E x rows); the
// normed activation goes to x and/or xq/xs (whichever is non-null), logits to
// `logits`
bool norm_logits_supported(int64_t d);
hipError_t norm_logits_launch(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps,
                              const RouterRows &rt, int64_t E, float *sum, float *x, int8_t *xq, float *xs,
                              double *logits, hipStream_t st, int8_t *xl = nullptr);

// router scratch: f64 logits [rows, E]
size_t route_scratch_bytes(int64_t rows, int64_t E);
// the first of route_launch's two launches: the f64 logits [rows, E]
hipError_t logits_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, double *logits,
                         hipStream_t st);
hipError_t route_launch(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                        float *wts, void *scratch, hipStream_t st);
// the router over Q8_0 rows: float32 x (act 0), its Q8_0 form xq/xs (act 1),
// or its two-word form xq/xl/xs (act 2)
hipError_t route_q8_launch(const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq, const float *Wrs,
                           int64_t rows, int64_t d, int64_t E, int64_t k, int act, int32_t *idx, float *wts,
                           void *scratch, hipStream_t st, const int8_t *xl = nullptr);

struct MoeArgs {
    const float *x;
    const int8_t *xq;
    const float *xs;
    const int8_t *Wgq;
    const float *Wgs;
    const int8_t *Wuq;
    const float *Wus;
    const int8_t *Wdq;
    const float *Wds;
    const int32_t *idx;
    const float *wts;
    int64_t rows, d, dff, E, k;
    float *h;
    int8_t *hq;
    float *hs;
    float *y;
    int act;
    void *scratch;
    // the fused route + gate-up launch: logits in, choices and weights out
    const double *logits;
    int32_t *idx_w;
    float *wts_w;
    // a shared expert (sdff > 0): gate/up [sdff, d], down [d, sdff], its
    // hidden row after the K routed ones (rows of k*dff + sdff values)
    const int8_t *Sgq;
    const float *Sgs;
    const int8_t *Suq;
    const float *Sus;
    const int8_t *Sdq;
    const float *Sds;
    int64_t sdff;
    // the down-combine adds its result to y instead of writing it
    bool acc_out;
    // two-word numerics (act 2): the low words of x and of the hidden rows
    const int8_t *xl;
    int8_t *hl;
    // the residual stream the down-combine adds to its output (null: none)
    const float *resid;
};
hipError_t gate_up_launch(const MoeArgs &a, hipStream_t st);
// gate-up that takes each row's top-K from `logits` itself (E <= ROUTE_FUSED_MAX_E)
hipError_t route_gate_up_launch(const MoeArgs &a, hipStream_t st);
size_t down_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t k, int act);
hipError_t down_launch(const MoeArgs &a, hipStream_t st);
// whether a shared expert of sdff fits the down-combine's (slot, slice)
// partials next to k slots of dff
bool shared_fits(int64_t dff, int64_t sdff, int64_t k);
// the shared expert alone, per row (gate-up, then a down-combine that adds
// into y): a chunk's grouped kernels carry no shared expert
hipError_t shared_launch(const MoeArgs &a, hipStream_t st);
// the down-combine row by row (the decode kernel for any rows: no grouping)
hipError_t row_down_launch(const MoeArgs &a, hipStream_t st);

// a chunk's mixture (rows > 1, int8 activations): choices grouped by expert,
// for d <= 2048 and dff <= 4096 (one slice of a wave each)
bool chunk_supported(int64_t d, int64_t dff);
// whether such a chunk's grouped gate-up and down run on the matrix cores
// (k_grouped_mfma) rather than the vector units
bool chunk_wide_sizes(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act);
hipError_t chunk_gate_up_launch(const MoeArgs &a, hipStream_t st);
size_t chunk_down_scratch_bytes(int64_t rows, int64_t d, int64_t k);
hipError_t chunk_down_launch(const MoeArgs &a, hipStream_t st);

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Compute units of the current device (read once per device, then cached);
// launch shapes that depend on how many workgroups the chip holds at once
// compare against it.
int device_cus();

// the whole mixture block: add + norm, router + top-K, gate-up, down-combine
struct BlockArgs {
    const float *h, *r, *w;
    float eps;
    RouterRows rt;
    const int8_t *Wgq;
    const float *Wgs;
    const int8_t *Wuq;
    const float *Wus;
    const int8_t *Wdq;
    const float *Wds;
    int64_t rows, d, dff, E, k;
    float *sum;
    int32_t *idx;
    float *wts;
    float *out;
    int act;
    void *scratch;
    // the shared expert (sdff 0: none)
    const int8_t *Sgq;
    const float *Sgs;
    const int8_t *Suq;
    const float *Sus;
    const int8_t *Sdq;
    const float *Sds;
    int64_t sdff;
    // the residual stream added to the mixture's output (null: none)
    const float *resid;
};
size_t block_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t sdff, int64_t E, int64_t k, int act);

// L mixture blocks in a row (a stack of layers), each layer's weights its
// own: the per-layer pointers are host arrays of L device pointers
struct StackArgs {
    const float *h, *r;
    int64_t layers;
    const float *const *w;
    const float *const *Wr;
    const int8_t *const *Wgq;
    const float *const *Wgs;
    const int8_t *const *Wuq;
    const float *const *Wus;
    const int8_t *const *Wdq;
    const float *const *Wds;
    int64_t rows, d, dff, E, k;
    float eps;
    float *out;
    int32_t *idx;
    float *wts;
    int act;
    void *scratch;
};
size_t stack_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act);
hipError_t stack_launch(const StackArgs &s, hipStream_t st);
bool block_fused(int64_t rows, int64_t d, int64_t dff, int64_t E, int act);
// a chunk of rows in int8 numerics (one or two words) runs the grouped kernels
bool block_chunk(int64_t rows, int64_t d, int64_t dff, int act);
hipError_t block_launch(const BlockArgs &b, hipStream_t st);

} // namespace q8s
