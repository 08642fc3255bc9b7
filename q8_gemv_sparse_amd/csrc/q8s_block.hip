// q8s_block.hip -- the whole mixture block as one call: residual add + norm,
// router + top-K, gate-up, down-combine (fn emit_moe_forward on the
// codegen_cuda::qwen_emit module page, fed by forward_shim.rs's add + norm row
// kernel; lane_link.rs fn prim, Moe arm, links the mixture as one launch
// unit).
//
// For decode rows (and any rows in float32 numerics) it runs three dependent
// launches instead of five:
//   k_norm_logits    add + norm of the row inside every router workgroup, one
//                    logit each (no norm launch);
//   k_route_gate_up  every gate-up workgroup ranks the row's logits itself
//                    (no top-K launch);
//   k_down           down-combine, as moe_down_combine runs it.
// Each removed launch is a dependent launch's fixed latency saved; the work
// repeated instead (the norm per router workgroup, the ranking per gate-up
// workgroup) reads a few KB from cache.  A chunk of rows in int8 numerics runs
// the grouped kernels (add_rmsnorm_q8, moe_route_topk, then the chunk gate-up
// and down), as do rows too long or experts too many for the fused launches.
//
// The router is float32 or Q8_0 rows (lane_link.rs fn prim, Moe arm); a
// shared expert rides in the gate-up and down-combine launches (fn
// class_launch, SharedExpertFusion arm), except under a chunk's grouped
// kernels, after which it runs as its own gate-up and an adding down-combine.
//
// Scratch, 256-byte aligned pieces in this order: the logits (double
// [rows, E]), the normed row x (f32 [rows, d]), its Q8_0 form (int8
// [rows, d] + f32 [rows, d/32]), the hidden rows (f32 [rows, k*dff + sdff]
// in f32 numerics; their Q8_0 form in int8), then for a chunk the f32 hidden
// rows [rows, k, dff] the grouped kernels stage and the shared expert's own
// hidden rows [rows, sdff], then moe_down_combine's scratch.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {

namespace {

struct BlockScratch {
    double *logits;
    float *x;
    int8_t *xq;
    float *xs;
    float *h;
    int8_t *hq;
    float *hs;
    int8_t *xl;  // two words: the low words of the normed row and of the hidden rows
    int8_t *hl;
    float *sh;  // a chunk's shared hidden rows (f32, or their Q8_0 form below)
    int8_t *shq;
    float *shs;
    int8_t *shl;  // two words: their low words
    void *down;
    size_t bytes;
};

bool chunk_mode(int64_t rows, int64_t d, int64_t dff, int act) { return act >= 1 && rows > 1 && chunk_supported(d, dff); }

BlockScratch carve(char *base, int64_t rows, int64_t d, int64_t dff, int64_t sdff, int64_t E, int64_t k, int act)
{
    BlockScratch s{};
    size_t off = 0;
    auto take = [&](size_t n) {
        char *p = base ? base + off : nullptr;
        off += align256(n);
        return p;
    };
    const bool chunk = chunk_mode(rows, d, dff, act);
    // hidden values a row: the routed ones and, outside a chunk, the shared
    const size_t nh = (size_t)rows * (size_t)(k * dff + (chunk ? 0 : sdff));
    s.logits = reinterpret_cast<double *>(take((size_t)(rows * E) * sizeof(double)));
    s.x = reinterpret_cast<float *>(take((size_t)(rows * d) * 4));
    if (act >= 1) {  // one or two int8 words
        s.xq = reinterpret_cast<int8_t *>(take((size_t)(rows * d)));
        s.xs = reinterpret_cast<float *>(take((size_t)(rows * d / QB) * 4));
        s.hq = reinterpret_cast<int8_t *>(take(nh));
        s.hs = reinterpret_cast<float *>(take(nh / QB * 4));
        if (act == 2) {
            s.xl = reinterpret_cast<int8_t *>(take((size_t)(rows * d)));
            s.hl = reinterpret_cast<int8_t *>(take(nh));
        }
        if (chunk)  // the chunk kernels stage the float32 hidden rows
            s.h = reinterpret_cast<float *>(take(nh * 4));
    } else {
        s.h = reinterpret_cast<float *>(take(nh * 4));
    }
    if (chunk && sdff > 0) {
        const size_t ns = (size_t)(rows * sdff);
        s.shq = reinterpret_cast<int8_t *>(take(ns));
        s.shs = reinterpret_cast<float *>(take(ns / QB * 4));
        if (act == 2)
            s.shl = reinterpret_cast<int8_t *>(take(ns));
    }
    const size_t dn = down_scratch_bytes(rows, d, dff, k, act);
    s.down = dn ? take(dn) : nullptr;
    s.bytes = off;
    return s;
}

} // namespace

size_t block_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t sdff, int64_t E, int64_t k, int act)
{
    return carve(nullptr, rows, d, dff, sdff, E, k, act).bytes;
}

bool block_chunk(int64_t rows, int64_t d, int64_t dff, int act) { return chunk_mode(rows, d, dff, act); }

bool block_fused(int64_t rows, int64_t d, int64_t dff, int64_t E, int act)
{
    return E <= ROUTE_FUSED_MAX_E && norm_logits_supported(d) && !chunk_mode(rows, d, dff, act);
}

hipError_t block_launch(const BlockArgs &b, hipStream_t st)
{
    const BlockScratch s = carve(static_cast<char *>(b.scratch), b.rows, b.d, b.dff, b.sdff, b.E, b.k, b.act);
    const bool chunk = chunk_mode(b.rows, b.d, b.dff, b.act);
    MoeArgs a{};
    a.x = b.act == 0 ? s.x : nullptr;
    a.xq = s.xq;
    a.xs = s.xs;
    a.Wgq = b.Wgq;
    a.Wgs = b.Wgs;
    a.Wuq = b.Wuq;
    a.Wus = b.Wus;
    a.Wdq = b.Wdq;
    a.Wds = b.Wds;
    a.idx = b.idx;
    a.wts = b.wts;
    a.rows = b.rows;
    a.d = b.d;
    a.dff = b.dff;
    a.E = b.E;
    a.k = b.k;
    a.h = s.h;
    a.hq = s.hq;
    a.hs = s.hs;
    a.xl = s.xl;
    a.hl = s.hl;
    a.y = b.out;
    a.act = b.act;
    a.scratch = s.down;
    a.resid = b.resid;
    if (!chunk) {
        a.Sgq = b.Sgq;
        a.Sgs = b.Sgs;
        a.Suq = b.Suq;
        a.Sus = b.Sus;
        a.Sdq = b.Sdq;
        a.Sds = b.Sds;
        a.sdff = b.sdff;
    }
    // the router reads the normed row's Q8_0 form only for Q8_0 rows in int8
    // numerics (a float router reads float32)
    RouterRows rt = b.rt;
    rt.act = b.act;
    hipError_t err;
    if (block_fused(b.rows, b.d, b.dff, b.E, b.act)) {
        err = norm_logits_launch(b.h, b.r, b.w, b.rows, b.d, b.eps, rt, b.E, b.sum,
                                 b.act == 0 ? s.x : nullptr, s.xq, s.xs, s.logits, st, s.xl);
        if (err != hipSuccess)
            return err;
        a.logits = s.logits;
        a.idx_w = b.idx;
        a.wts_w = b.wts;
        err = route_gate_up_launch(a, st);
    } else {
        // two words: the normed row's words, low words and scales in the same
        // epilogue (the same words and scales as the one-word epilogue's)
        err = add_rmsnorm_launch(b.h, b.r, b.w, b.rows, b.d, b.eps, b.sum, s.x, s.xq, s.xs, st,
                                 b.act == 2 ? s.xl : nullptr);
        if (err != hipSuccess)
            return err;
        if (rt.Wrq)
            err = route_q8_launch(s.x, s.xq, s.xs, rt.Wrq, rt.Wrs, b.rows, b.d, b.E, b.k, rt.act, b.idx, b.wts,
                                  s.logits, st, s.xl);
        else
            err = route_launch(s.x, rt.Wr, b.rows, b.d, b.E, b.k, b.idx, b.wts, s.logits, st);
        if (err != hipSuccess)
            return err;
        err = gate_up_launch(a, st);
    }
    if (err != hipSuccess)
        return err;
    err = down_launch(a, st);
    if (err != hipSuccess || !chunk || b.sdff == 0)
        return err;
    MoeArgs sa = a;
    sa.Sgq = b.Sgq;
    sa.Sgs = b.Sgs;
    sa.Suq = b.Suq;
    sa.Sus = b.Sus;
    sa.Sdq = b.Sdq;
    sa.Sds = b.Sds;
    sa.sdff = b.sdff;
    sa.h = nullptr;
    sa.hq = s.shq;
    sa.hs = s.shs;
    sa.hl = s.shl;
    return shared_launch(sa, st);
}

// A stack of L layers (forward_shim.rs module doc: the sum and the RMS norm
// of it as one row kernel; the whole forward one graph of launches):
//   s_0 = h + r;  for each layer l:  x_l = RMSNorm(s_l) * w_l,
//   m_l = mixture_l(x_l),  s_{l+1} = s_l + m_l;   out = s_L.
// Each layer is one block call.  The residual add s_l + m_l of layer l is
// deferred into layer l + 1's first launch, whose add + norm row kernel reads
// m_l as h and s_l as r and writes their sum; the last layer's add is folded
// into its down-combine epilogue, which writes s_L itself.  Nothing runs
// between the layers' launches.  Scratch: the block's, then the running sums
// s_l (two, alternating) and the mixture output m_l.
size_t stack_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act)
{
    return block_scratch_bytes(rows, d, dff, 0, E, k, act) + 3 * align256((size_t)(rows * d) * 4);
}

hipError_t stack_launch(const StackArgs &a, hipStream_t st)
{
    char *base = static_cast<char *>(a.scratch);
    const size_t bs = block_scratch_bytes(a.rows, a.d, a.dff, 0, a.E, a.k, a.act);
    const size_t vb = align256((size_t)(a.rows * a.d) * 4);
    float *S[2] = {reinterpret_cast<float *>(base + bs), reinterpret_cast<float *>(base + bs + vb)};
    float *M = reinterpret_cast<float *>(base + bs + 2 * vb);
    const int64_t nk = a.rows * a.k;
    for (int64_t l = 0; l < a.layers; l++) {
        const bool last = l == a.layers - 1;
        BlockArgs b{};
        b.h = l == 0 ? a.h : M;
        b.r = l == 0 ? a.r : S[(l - 1) & 1];
        b.w = a.w[l];
        b.eps = a.eps;
        b.rt = RouterRows{a.Wr[l], nullptr, nullptr, 0};
        b.Wgq = a.Wgq[l];
        b.Wgs = a.Wgs[l];
        b.Wuq = a.Wuq[l];
        b.Wus = a.Wus[l];
        b.Wdq = a.Wdq[l];
        b.Wds = a.Wds[l];
        b.rows = a.rows;
        b.d = a.d;
        b.dff = a.dff;
        b.E = a.E;
        b.k = a.k;
        b.sum = S[l & 1];
        b.idx = a.idx + l * nk;
        b.wts = a.wts + l * nk;
        b.out = last ? a.out : M;
        b.resid = last ? S[l & 1] : nullptr;
        b.act = a.act;
        b.scratch = a.scratch;
        const hipError_t err = block_launch(b, st);
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

} // namespace q8s
