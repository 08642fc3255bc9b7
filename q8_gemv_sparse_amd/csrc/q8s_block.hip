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
// Scratch, 256-byte aligned pieces in this order: the logits (double
// [rows, E]), the normed row x (f32 [rows, d]), its Q8_0 form (int8
// [rows, d] + f32 [rows, d/32]), the hidden rows (f32 [rows, k, dff] in f32
// numerics; their Q8_0 form in int8, plus the f32 rows when rows > 1), then
// moe_down_combine's scratch.
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
    void *down;
    size_t bytes;
};

BlockScratch carve(char *base, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act)
{
    BlockScratch s{};
    size_t off = 0;
    auto take = [&](size_t n) {
        char *p = base ? base + off : nullptr;
        off += align256(n);
        return p;
    };
    const size_t nh = (size_t)(rows * k * dff);
    s.logits = reinterpret_cast<double *>(take((size_t)(rows * E) * sizeof(double)));
    s.x = reinterpret_cast<float *>(take((size_t)(rows * d) * 4));
    if (act == 1) {
        s.xq = reinterpret_cast<int8_t *>(take((size_t)(rows * d)));
        s.xs = reinterpret_cast<float *>(take((size_t)(rows * d / QB) * 4));
        s.hq = reinterpret_cast<int8_t *>(take(nh));
        s.hs = reinterpret_cast<float *>(take(nh / QB * 4));
        if (rows > 1)  // the chunk kernels stage the float32 hidden rows
            s.h = reinterpret_cast<float *>(take(nh * 4));
    } else {
        s.h = reinterpret_cast<float *>(take(nh * 4));
    }
    const size_t dn = down_scratch_bytes(rows, d, dff, k, act);
    s.down = dn ? take(dn) : nullptr;
    s.bytes = off;
    return s;
}

} // namespace

size_t block_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act)
{
    return carve(nullptr, rows, d, dff, E, k, act).bytes;
}

bool block_fused(int64_t rows, int64_t d, int64_t dff, int64_t E, int act)
{
    return E <= ROUTE_FUSED_MAX_E && norm_logits_supported(d) && !(act == 1 && rows > 1 && chunk_supported(d, dff));
}

hipError_t block_launch(const BlockArgs &b, hipStream_t st)
{
    const BlockScratch s = carve(static_cast<char *>(b.scratch), b.rows, b.d, b.dff, b.E, b.k, b.act);
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
    a.y = b.out;
    a.act = b.act;
    a.scratch = s.down;
    hipError_t err;
    if (block_fused(b.rows, b.d, b.dff, b.E, b.act)) {
        err = norm_logits_launch(b.h, b.r, b.w, b.rows, b.d, b.eps, b.Wr, b.E, b.sum, b.act == 0 ? s.x : nullptr, s.xq,
                                 s.xs, s.logits, st);
        if (err != hipSuccess)
            return err;
        a.logits = s.logits;
        a.idx_w = b.idx;
        a.wts_w = b.wts;
        err = route_gate_up_launch(a, st);
    } else {
        err = add_rmsnorm_launch(b.h, b.r, b.w, b.rows, b.d, b.eps, b.sum, s.x, s.xq, s.xs, st);
        if (err != hipSuccess)
            return err;
        err = route_launch(s.x, b.Wr, b.rows, b.d, b.E, b.k, b.idx, b.wts, s.logits, st);
        if (err != hipSuccess)
            return err;
        err = gate_up_launch(a, st);
    }
    if (err != hipSuccess)
        return err;
    return down_launch(a, st);
}

} // namespace q8s
