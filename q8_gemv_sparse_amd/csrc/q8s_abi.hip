// q8s_abi.hip -- the C ABI declared in include/q8s.h.
//
// Each entry point checks its arguments on the host before any HIP call --
// null pointers, shapes, alignment, limits, overlapping buffers, scratch size
// -- and refuses by naming the rule it breaks, in the style of the refusals
// of codegen_cuda/forward_shim.rs (fn kernel_refusal) and lane_link.rs (fn
// prim).  Accepted calls enqueue their kernels on the caller's stream and
// return without synchronising.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/q8s.h"
#include "q8s_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

// Clears a stale error left by an earlier, unrelated HIP call, so a launch
// failure is reported as this call's own.
void clear_stale() { (void)hipGetLastError(); }

int launched(hipError_t e, const char *fn)
{
    if (e != hipSuccess)
        return fail(Q8S_ELAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_err.clear();
    return Q8S_OK;
}

struct Span {
    const void *p;
    size_t bytes;
    const char *name;
};

// A buffer list check: present, 16-byte aligned.  Returns 0 or an error code.
int check_ptrs(const char *fn, const std::vector<Span> &v)
{
    for (const Span &s : v) {
        if (!s.p)
            return fail(Q8S_EINVAL, "%s: `%s` is null", fn, s.name);
        if (reinterpret_cast<uintptr_t>(s.p) % 16 != 0)
            return fail(Q8S_EALIGN, "%s: `%s` is not 16-byte aligned", fn, s.name);
    }
    return 0;
}

bool overlap(const Span &a, const Span &b)
{
    const char *pa = static_cast<const char *>(a.p), *pb = static_cast<const char *>(b.p);
    return pa < pb + b.bytes && pb < pa + a.bytes;
}

// Outputs may overlap neither an input nor another output: every stage reads
// and writes whole buffers (forward_shim.rs module doc).
int check_disjoint(const char *fn, const std::vector<Span> &ins, const std::vector<Span> &outs)
{
    for (size_t i = 0; i < outs.size(); i++) {
        for (const Span &in : ins)
            if (overlap(outs[i], in))
                return fail(Q8S_EINVAL, "%s: output `%s` overlaps input `%s` -- a stage writes whole buffers of its own",
                            fn, outs[i].name, in.name);
        for (size_t j = i + 1; j < outs.size(); j++)
            if (overlap(outs[i], outs[j]))
                return fail(Q8S_EINVAL, "%s: outputs `%s` and `%s` overlap", fn, outs[i].name, outs[j].name);
    }
    return 0;
}

int check_dim32(const char *fn, const char *name, int64_t n)
{
    if (n <= 0 || n % 32 != 0)
        return fail(Q8S_EINVAL, "%s: `%s` = %lld is not a positive multiple of 32 (whole Q8_0 blocks)", fn, name,
                    (long long)n);
    if (n > q8s::MAX_NIN)
        return fail(Q8S_EUNSUPPORTED, "%s: `%s` = %lld exceeds the kernels' longest row of %lld values", fn, name,
                    (long long)n, (long long)q8s::MAX_NIN);
    return 0;
}

int check_count(const char *fn, const char *name, int64_t n, int64_t hi)
{
    if (n <= 0)
        return fail(Q8S_EINVAL, "%s: `%s` = %lld must be at least 1", fn, name, (long long)n);
    if (n > hi)
        return fail(Q8S_EUNSUPPORTED, "%s: `%s` = %lld exceeds %lld", fn, name, (long long)n, (long long)hi);
    return 0;
}

int check_act(const char *fn, int act)
{
    if (act == Q8S_ACT_F32 || act == Q8S_ACT_INT8)
        return 0;
    if (act == 2)
        return fail(Q8S_EUNSUPPORTED,
                    "%s: act = 2 (two-word int8 activations) is served by q8_quantize_rows_x2, q8_gemv_x2, "
                    "add_rmsnorm_gemv_x2, moe_gate_up_x2, moe_topk_gate_up_x2, moe_down_combine_x2, moe_route_topk_gemv, "
                    "moe_ffn_block and moe_ffn_stack", fn);
    return fail(Q8S_EUNSUPPORTED, "%s: unknown activation mode act = %d", fn, act);
}

int check_moe_shape(const char *fn, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k)
{
    int rc;
    if ((rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "d", d)) ||
        (rc = check_dim32(fn, "dff", dff)))
        return rc;
    if (E <= 0)
        return fail(Q8S_EINVAL, "%s: `E` = %lld must be at least 1", fn, (long long)E);
    if (k <= 0 || k > E)
        return fail(Q8S_EINVAL, "%s: k = %lld kept experts of E = %lld: 1 <= k <= E", fn, (long long)k, (long long)E);
    if (k > Q8S_MAX_K || E > Q8S_MAX_E)
        return fail(Q8S_EUNSUPPORTED, "%s: more than %d experts kept, or more than %d experts (k = %lld, E = %lld)", fn,
                    Q8S_MAX_K, Q8S_MAX_E, (long long)k, (long long)E);
    if (E * dff > INT32_MAX || E * d > INT32_MAX)
        return fail(Q8S_EUNSUPPORTED, "%s: E*dff or E*d past 2^31 rows", fn);
    return 0;
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

} // namespace

extern "C" {

const char *q8s_last_error(void) { return g_err.c_str(); }

const char *q8s_version(void) { return "q8s 0.1 gfx950"; }

int q8s_stream_read(const void *buf, int64_t bytes, uint32_t *out, void *stream)
{
    const char *fn = "q8s_stream_read";
    if (bytes <= 0 || bytes % 16 != 0)
        return fail(Q8S_EINVAL, "%s: `bytes` = %lld is not a positive multiple of 16 (whole 16-byte loads)", fn,
                    (long long)bytes);
    std::vector<Span> ins = {{buf, (size_t)bytes, "buf"}};
    std::vector<Span> outs = {{out, (size_t)Q8S_STREAM_WGS * 4, "out"}};
    int rc;
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::stream_read_launch(buf, bytes, out, as_stream(stream)), fn);
}

size_t q8s_scratch_bytes(int fn, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act)
{
    if (rows <= 0 || E <= 0 || k <= 0 || d <= 0)
        return 0;
    switch (fn) {
    case Q8S_FN_ROUTE:
        return q8s::route_scratch_bytes(rows, E);
    case Q8S_FN_DOWN:
        return q8s::down_scratch_bytes(rows, d, dff, k, act);
    case Q8S_FN_BLOCK:
        return q8s::block_scratch_bytes(rows, d, dff, 0, E, k, act);
    case Q8S_FN_STACK:
        return q8s::stack_scratch_bytes(rows, d, dff, E, k, act);
    default:
        return 0;
    }
}

size_t q8s_block_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t sdff, int64_t E, int64_t k, int act)
{
    if (rows <= 0 || E <= 0 || k <= 0 || d <= 0 || dff <= 0 || sdff < 0)
        return 0;
    return q8s::block_scratch_bytes(rows, d, dff, sdff, E, k, act);
}

int q8s_moe_path(int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, int act)
{
    if (rows <= 0 || d <= 0 || dff <= 0 || E <= 0 || k <= 0 || k > E || act < 0 || act > 2)
        return Q8S_EINVAL;
    if (act == 0 || rows == 1 || !q8s::chunk_supported(d, dff))
        return Q8S_PATH_ROWS;
    return q8s::chunk_wide_sizes(rows, d, dff, E, k, act) ? Q8S_PATH_GROUPED_MFMA : Q8S_PATH_GROUPED;
}

int q8_gemv(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in, const float *x, const int8_t *xq,
            const float *xs, int64_t m, float *y, int act, void *stream)
{
    const char *fn = "q8_gemv";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_dim32(fn, "n_in", n_in)) ||
        (rc = check_count(fn, "n_out", n_out, INT32_MAX / 2)) || (rc = check_count(fn, "m", m, 65535)))
        return rc;
    const size_t nb = (size_t)(n_in / 32);
    std::vector<Span> ins = {{Wq, (size_t)(n_out * n_in), "Wq"}, {Ws, (size_t)n_out * nb * 4, "Ws"}};
    if (act == Q8S_ACT_F32) {
        ins.push_back({x, (size_t)(m * n_in) * 4, "x"});
    } else {
        ins.push_back({xq, (size_t)(m * n_in), "xq"});
        ins.push_back({xs, (size_t)m * nb * 4, "xs"});
    }
    std::vector<Span> outs = {{y, (size_t)(m * n_out) * 4, "y"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::GemvArgs a{Wq, Ws, n_out, n_in, act == 0 ? x : nullptr, act == 1 ? xq : nullptr, act == 1 ? xs : nullptr,
                    m, y, act};
    clear_stale();
    return launched(q8s::gemv_launch(a, as_stream(stream)), fn);
}

int q8_quantize_rows(const float *x, int64_t rows, int64_t n, int8_t *xq, float *xs, void *stream)
{
    const char *fn = "q8_quantize_rows";
    int rc;
    if ((rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "n", n)))
        return rc;
    std::vector<Span> ins = {{x, (size_t)(rows * n) * 4, "x"}};
    std::vector<Span> outs = {{xq, (size_t)(rows * n), "xq"}, {xs, (size_t)(rows * n / 32) * 4, "xs"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::quantize_launch(x, rows, n, xq, xs, as_stream(stream)), fn);
}

int q8_quantize_rows_x2(const float *x, int64_t rows, int64_t n, int8_t *xq, int8_t *xl, float *xs, void *stream)
{
    const char *fn = "q8_quantize_rows_x2";
    int rc;
    if ((rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "n", n)))
        return rc;
    std::vector<Span> ins = {{x, (size_t)(rows * n) * 4, "x"}};
    std::vector<Span> outs = {{xq, (size_t)(rows * n), "xq"}, {xl, (size_t)(rows * n), "xl"},
                              {xs, (size_t)(rows * n / 32) * 4, "xs"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::quantize_x2_launch(x, rows, n, xq, xl, xs, as_stream(stream)), fn);
}

int q8_gemv_x2(const int8_t *Wq, const float *Ws, int64_t n_out, int64_t n_in, const int8_t *xq, const int8_t *xl,
               const float *xs, int64_t m, float *y, void *stream)
{
    const char *fn = "q8_gemv_x2";
    int rc;
    if ((rc = check_dim32(fn, "n_in", n_in)) || (rc = check_count(fn, "n_out", n_out, INT32_MAX / 2)) ||
        (rc = check_count(fn, "m", m, 65535)))
        return rc;
    const size_t nb = (size_t)(n_in / 32);
    std::vector<Span> ins = {{Wq, (size_t)(n_out * n_in), "Wq"}, {Ws, (size_t)n_out * nb * 4, "Ws"},
                             {xq, (size_t)(m * n_in), "xq"}, {xl, (size_t)(m * n_in), "xl"},
                             {xs, (size_t)m * nb * 4, "xs"}};
    std::vector<Span> outs = {{y, (size_t)(m * n_out) * 4, "y"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::GemvArgs a{Wq, Ws, n_out, n_in, nullptr, xq, xs, m, y, 2, xl};
    clear_stale();
    return launched(q8s::gemv_launch(a, as_stream(stream)), fn);
}

int add_rmsnorm_q8(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps, float *sum,
                   float *y, int8_t *yq, float *ys, void *stream)
{
    const char *fn = "add_rmsnorm_q8";
    int rc;
    if ((rc = check_count(fn, "rows", rows, INT32_MAX)) || (rc = check_dim32(fn, "d", d)))
        return rc;
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    if ((yq == nullptr) != (ys == nullptr))
        return fail(Q8S_EINVAL, "%s: `yq` and `ys` are given together or not at all", fn);
    if (!y && !yq)
        return fail(Q8S_EINVAL, "%s: neither `y` nor `yq` is given -- the norm would write nothing but the sum", fn);
    const size_t n = (size_t)(rows * d);
    std::vector<Span> ins = {{h, n * 4, "h"}, {r, n * 4, "r"}, {w, (size_t)d * 4, "w"}};
    std::vector<Span> outs = {{sum, n * 4, "sum"}};
    if (y)
        outs.push_back({y, n * 4, "y"});
    if (yq) {
        outs.push_back({yq, n, "yq"});
        outs.push_back({ys, n / 32 * 4, "ys"});
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::add_rmsnorm_launch(h, r, w, rows, d, eps, sum, y, yq, ys, as_stream(stream)), fn);
}

int add_rmsnorm_q8_x2(const float *h, const float *r, const float *w, int64_t rows, int64_t d, float eps, float *sum,
                      float *y, int8_t *yq, int8_t *yl, float *ys, void *stream)
{
    const char *fn = "add_rmsnorm_q8_x2";
    int rc;
    if ((rc = check_count(fn, "rows", rows, INT32_MAX)) || (rc = check_dim32(fn, "d", d)))
        return rc;
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    const size_t n = (size_t)(rows * d);
    std::vector<Span> ins = {{h, n * 4, "h"}, {r, n * 4, "r"}, {w, (size_t)d * 4, "w"}};
    std::vector<Span> outs = {{sum, n * 4, "sum"}, {yq, n, "yq"}, {yl, n, "yl"}, {ys, n / 32 * 4, "ys"}};
    if (y)
        outs.push_back({y, n * 4, "y"});
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::add_rmsnorm_launch(h, r, w, rows, d, eps, sum, y, yq, ys, as_stream(stream), yl), fn);
}

int moe_route_topk(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                   float *wts, void *scratch, size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_route_topk";
    int rc;
    if ((rc = check_moe_shape(fn, rows, d, 32, E, k)))
        return rc;
    std::vector<Span> ins = {{x, (size_t)(rows * d) * 4, "x"}, {Wr, (size_t)(E * d) * 4, "Wr"}};
    std::vector<Span> outs = {{idx, (size_t)(rows * k) * 4, "idx"}, {wts, (size_t)(rows * k) * 4, "wts"}};
    const size_t need = q8s::route_scratch_bytes(rows, E);
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    if (!scratch || scratch_bytes < need)
        return fail(Q8S_ESCRATCH, "%s: scratch of %zu bytes given, %zu needed (logits and arrival counters)", fn,
                    scratch ? scratch_bytes : (size_t)0, need);
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
        return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
    outs.push_back({scratch, need, "scratch"});
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::route_launch(x, Wr, rows, d, E, k, idx, wts, scratch, as_stream(stream)), fn);
}

int moe_route_topk_gemv(const float *x, const float *Wr, int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx,
                        float *wts, const int8_t *Dq, const float *Ds, int64_t n_out, const int8_t *xq,
                        const int8_t *xl, const float *xs, float *y, int act, void *scratch, size_t scratch_bytes,
                        void *stream)
{
    const char *fn = "moe_route_topk_gemv";
    int rc;
    if (act != Q8S_ACT_INT8 && act != 2)
        return fail(act == Q8S_ACT_F32 ? Q8S_EUNSUPPORTED : Q8S_EINVAL,
                    "%s: act = %d: the projection reads the rows' Q8_0 form, in one word (act 1) or two (act 2)",
                    fn, act);
    if ((act == 2) != (xl != nullptr))
        return fail(Q8S_EINVAL, "%s: `xl` (the low words) is given for act 2 and only then", fn);
    if ((rc = check_moe_shape(fn, rows, d, 32, E, k)) || (rc = check_count(fn, "n_out", n_out, INT32_MAX / 2)))
        return rc;
    const size_t n = (size_t)(rows * d), nb = (size_t)(d / 32);
    std::vector<Span> ins = {{x, n * 4, "x"},
                             {Wr, (size_t)(E * d) * 4, "Wr"},
                             {Dq, (size_t)n_out * (size_t)d, "Dq"},
                             {Ds, (size_t)n_out * nb * 4, "Ds"},
                             {xq, n, "xq"},
                             {xs, (size_t)rows * nb * 4, "xs"}};
    if (act == 2)
        ins.push_back({xl, n, "xl"});
    std::vector<Span> outs = {{idx, (size_t)(rows * k) * 4, "idx"},
                              {wts, (size_t)(rows * k) * 4, "wts"},
                              {y, (size_t)rows * (size_t)n_out * 4, "y"}};
    const size_t need = q8s::route_scratch_bytes(rows, E);
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    if (!scratch || scratch_bytes < need)
        return fail(Q8S_ESCRATCH, "%s: scratch of %zu bytes given, %zu needed (the logits)", fn,
                    scratch ? scratch_bytes : (size_t)0, need);
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
        return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
    outs.push_back({scratch, need, "scratch"});
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    const hipStream_t st = as_stream(stream);
    const q8s::GemvArgs a{Dq, Ds, n_out, d, nullptr, xq, xs, rows, y, act, xl};
    double *logits = reinterpret_cast<double *>(scratch);
    if (!q8s::gemv_topk_fused(rows, E, act)) {
        const hipError_t err = q8s::route_launch(x, Wr, rows, d, E, k, idx, wts, scratch, st);
        return launched(err != hipSuccess ? err : q8s::gemv_launch(a, st), fn);
    }
    const hipError_t err = q8s::logits_launch(x, Wr, rows, d, E, logits, st);
    return launched(err != hipSuccess ? err : q8s::gemv_topk_launch(a, logits, rows, E, k, idx, wts, st), fn);
}

int moe_route_topk_q8(const float *x, const int8_t *xq, const float *xs, const int8_t *Wrq, const float *Wrs,
                      int64_t rows, int64_t d, int64_t E, int64_t k, int32_t *idx, float *wts, int act, void *scratch,
                      size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_route_topk_q8";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_moe_shape(fn, rows, d, 32, E, k)))
        return rc;
    std::vector<Span> ins = {{Wrq, (size_t)(E * d), "Wrq"}, {Wrs, (size_t)(E * d / 32) * 4, "Wrs"}};
    if (act == Q8S_ACT_F32) {
        ins.push_back({x, (size_t)(rows * d) * 4, "x"});
    } else {
        ins.push_back({xq, (size_t)(rows * d), "xq"});
        ins.push_back({xs, (size_t)(rows * d / 32) * 4, "xs"});
    }
    std::vector<Span> outs = {{idx, (size_t)(rows * k) * 4, "idx"}, {wts, (size_t)(rows * k) * 4, "wts"}};
    const size_t need = q8s::route_scratch_bytes(rows, E);
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    if (!scratch || scratch_bytes < need)
        return fail(Q8S_ESCRATCH, "%s: scratch of %zu bytes given, %zu needed (the logits)", fn,
                    scratch ? scratch_bytes : (size_t)0, need);
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
        return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
    outs.push_back({scratch, need, "scratch"});
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::route_q8_launch(act == 0 ? x : nullptr, act == 1 ? xq : nullptr, act == 1 ? xs : nullptr,
                                         Wrq, Wrs, rows, d, E, k, act, idx, wts, scratch, as_stream(stream)),
                    fn);
}

int moe_gate_up(const float *x, const int8_t *xq, const float *xs, const int8_t *Wgq, const float *Wgs,
                const int8_t *Wuq, const float *Wus, const int32_t *idx, int64_t rows, int64_t d, int64_t dff,
                int64_t E, int64_t k, float *h, int8_t *hq, float *hs, int act, void *stream)
{
    const char *fn = "moe_gate_up";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    const size_t nh = (size_t)(rows * k * dff);
    std::vector<Span> ins = {{Wgq, wq, "Wgq"}, {Wgs, wsb, "Wgs"}, {Wuq, wq, "Wuq"}, {Wus, wsb, "Wus"},
                             {idx, (size_t)(rows * k) * 4, "idx"}};
    std::vector<Span> outs;
    if (act == Q8S_ACT_F32) {
        ins.push_back({x, (size_t)(rows * d) * 4, "x"});
        outs.push_back({h, nh * 4, "h"});
    } else {
        if (rows > 1 && !h)
            return fail(Q8S_EINVAL, "%s: int8 numerics with rows > 1: `h` is required (the grouped chunk kernels "
                        "stage the float32 hidden rows there before forming their Q8_0 form)", fn);
        ins.push_back({xq, (size_t)(rows * d), "xq"});
        ins.push_back({xs, (size_t)(rows * d / 32) * 4, "xs"});
        // the grouped chunk kernels write the float32 hidden rows and then
        // form their Q8_0 form in a pass of their own, which a caller may
        // leave out (hq and hs both NULL) to quantise the rows itself
        const bool chunk = rows > 1 && q8s::chunk_supported(d, dff);
        if (!hq && !hs && !chunk)
            return fail(Q8S_EINVAL, "%s: int8 numerics: `hq`/`hs` are required (only a chunk of rows in the grouped "
                        "kernels may leave out the hidden rows' Q8_0 form)", fn);
        if (h)
            outs.push_back({h, nh * 4, "h"});
        if (hq || hs) {
            outs.push_back({hq, nh, "hq"});
            outs.push_back({hs, nh / 32 * 4, "hs"});
        }
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.x = act == 0 ? x : nullptr;
    a.xq = act == 1 ? xq : nullptr;
    a.xs = act == 1 ? xs : nullptr;
    a.Wgq = Wgq;
    a.Wgs = Wgs;
    a.Wuq = Wuq;
    a.Wus = Wus;
    a.idx = idx;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.h = h;
    a.hq = act == 1 ? hq : nullptr;
    a.hs = act == 1 ? hs : nullptr;
    a.act = act;
    clear_stale();
    return launched(q8s::gate_up_launch(a, as_stream(stream)), fn);
}

int moe_gate_up_x2(const int8_t *xq, const int8_t *xl, const float *xs, const int8_t *Wgq, const float *Wgs,
                   const int8_t *Wuq, const float *Wus, const int32_t *idx, int64_t rows, int64_t d, int64_t dff,
                   int64_t E, int64_t k, float *h, int8_t *hq, int8_t *hl, float *hs, void *stream)
{
    const char *fn = "moe_gate_up_x2";
    int rc;
    if ((rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    const size_t nh = (size_t)(rows * k * dff), nx = (size_t)(rows * d);
    const bool chunk = rows > 1 && q8s::chunk_supported(d, dff);
    if (chunk && !h)
        return fail(Q8S_EINVAL, "%s: a chunk of rows: `h` is required (the grouped chunk kernels stage the float32 "
                    "hidden rows there before forming their two-word form)", fn);
    const bool q = hq || hl || hs;
    if (!q && !chunk)
        return fail(Q8S_EINVAL, "%s: `hq`/`hl`/`hs` are required (only a chunk of rows in the grouped kernels may "
                    "leave out the hidden rows' two-word form)", fn);
    std::vector<Span> ins = {{Wgq, wq, "Wgq"}, {Wgs, wsb, "Wgs"}, {Wuq, wq, "Wuq"}, {Wus, wsb, "Wus"},
                             {idx, (size_t)(rows * k) * 4, "idx"}, {xq, nx, "xq"}, {xl, nx, "xl"},
                             {xs, nx / 32 * 4, "xs"}};
    std::vector<Span> outs;
    if (h)
        outs.push_back({h, nh * 4, "h"});
    if (q) {
        outs.push_back({hq, nh, "hq"});
        outs.push_back({hl, nh, "hl"});
        outs.push_back({hs, nh / 32 * 4, "hs"});
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.xq = xq;
    a.xl = xl;
    a.xs = xs;
    a.Wgq = Wgq;
    a.Wgs = Wgs;
    a.Wuq = Wuq;
    a.Wus = Wus;
    a.idx = idx;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.h = h;
    a.hq = hq;
    a.hl = hl;
    a.hs = hs;
    a.act = 2;
    clear_stale();
    return launched(q8s::gate_up_launch(a, as_stream(stream)), fn);
}

int moe_down_combine_x2(const int8_t *hq, const int8_t *hl, const float *hs, const int8_t *Wdq, const float *Wds,
                        const int32_t *idx, const float *wts, int64_t rows, int64_t d, int64_t dff, int64_t E,
                        int64_t k, float *y, void *scratch, size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_down_combine_x2";
    int rc;
    if ((rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    const size_t nh = (size_t)(rows * k * dff);
    std::vector<Span> ins = {{Wdq, (size_t)(E * d) * (size_t)dff, "Wdq"},
                             {Wds, (size_t)(E * d) * (size_t)(dff / 32) * 4, "Wds"},
                             {idx, (size_t)(rows * k) * 4, "idx"},
                             {wts, (size_t)(rows * k) * 4, "wts"},
                             {hq, nh, "hq"},
                             {hl, nh, "hl"},
                             {hs, nh / 32 * 4, "hs"}};
    std::vector<Span> outs = {{y, (size_t)(rows * d) * 4, "y"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    const size_t need = q8s::down_scratch_bytes(rows, d, dff, k, 2);
    if (need) {
        if (!scratch || scratch_bytes < need)
            return fail(Q8S_ESCRATCH, "%s: scratch of %zu bytes given, %zu needed (per-choice results)", fn,
                        scratch ? scratch_bytes : (size_t)0, need);
        if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
            return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
        outs.push_back({scratch, need, "scratch"});
    }
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.hq = const_cast<int8_t *>(hq);
    a.hl = const_cast<int8_t *>(hl);
    a.hs = const_cast<float *>(hs);
    a.Wdq = Wdq;
    a.Wds = Wds;
    a.idx = idx;
    a.wts = wts;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.y = y;
    a.act = 2;
    a.scratch = need ? scratch : nullptr;
    clear_stale();
    return launched(q8s::down_launch(a, as_stream(stream)), fn);
}

int moe_down_combine(const float *h, const int8_t *hq, const float *hs, const int8_t *Wdq, const float *Wds,
                     const int32_t *idx, const float *wts, int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k,
                     float *y, int act, void *scratch, size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_down_combine";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    const size_t nh = (size_t)(rows * k * dff);
    std::vector<Span> ins = {{Wdq, (size_t)(E * d) * (size_t)dff, "Wdq"},
                             {Wds, (size_t)(E * d) * (size_t)(dff / 32) * 4, "Wds"},
                             {idx, (size_t)(rows * k) * 4, "idx"},
                             {wts, (size_t)(rows * k) * 4, "wts"}};
    if (act == Q8S_ACT_F32) {
        ins.push_back({h, nh * 4, "h"});
    } else {
        ins.push_back({hq, nh, "hq"});
        ins.push_back({hs, nh / 32 * 4, "hs"});
    }
    std::vector<Span> outs = {{y, (size_t)(rows * d) * 4, "y"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    const size_t need = q8s::down_scratch_bytes(rows, d, dff, k, act);
    if (need) {
        if (!scratch || scratch_bytes < need)
            return fail(Q8S_ESCRATCH, "%s: scratch of %zu bytes given, %zu needed (per-choice results)", fn,
                        scratch ? scratch_bytes : (size_t)0, need);
        if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
            return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
        outs.push_back({scratch, need, "scratch"});
    }
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.h = act == 0 ? const_cast<float *>(h) : nullptr;
    a.hq = act == 1 ? const_cast<int8_t *>(hq) : nullptr;
    a.hs = act == 1 ? const_cast<float *>(hs) : nullptr;
    a.Wdq = Wdq;
    a.Wds = Wds;
    a.idx = idx;
    a.wts = wts;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.y = y;
    a.act = act;
    a.scratch = need ? scratch : nullptr;
    clear_stale();
    return launched(q8s::down_launch(a, as_stream(stream)), fn);
}

int add_rmsnorm_gemv(const float *h, const float *r, const float *w, float eps, const int8_t *Wq, const float *Ws,
                     int64_t rows, int64_t d, int64_t n_out, float *sum, float *y, int8_t *yq, float *ys, float *out,
                     int act, void *stream)
{
    const char *fn = "add_rmsnorm_gemv";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "d", d)) ||
        (rc = check_count(fn, "n_out", n_out, INT32_MAX / 2)))
        return rc;
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    if ((yq == nullptr) != (ys == nullptr))
        return fail(Q8S_EINVAL, "%s: `yq` and `ys` are given together or not at all", fn);
    if (act == Q8S_ACT_F32 && !y)
        return fail(Q8S_EINVAL, "%s: f32 numerics read the normed row: `y` is required", fn);
    if (act == Q8S_ACT_INT8 && !yq)
        return fail(Q8S_EINVAL, "%s: int8 numerics read the normed row's Q8_0 form: `yq`/`ys` are required", fn);
    const size_t n = (size_t)(rows * d);
    std::vector<Span> ins = {{h, n * 4, "h"},
                             {r, n * 4, "r"},
                             {w, (size_t)d * 4, "w"},
                             {Wq, (size_t)(n_out * d), "Wq"},
                             {Ws, (size_t)n_out * (size_t)(d / 32) * 4, "Ws"}};
    std::vector<Span> outs = {{sum, n * 4, "sum"}, {out, (size_t)(rows * n_out) * 4, "out"}};
    if (y)
        outs.push_back({y, n * 4, "y"});
    if (yq) {
        outs.push_back({yq, n, "yq"});
        outs.push_back({ys, n / 32 * 4, "ys"});
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    const hipStream_t st = as_stream(stream);
    if (q8s::norm_gemv_supported(rows, d)) {
        q8s::NormGemvArgs a{h, r, w, eps, Wq, Ws, d, n_out, sum, y, yq, ys, out, act};
        return launched(q8s::norm_gemv_launch(a, st), fn);
    }
    hipError_t e = q8s::add_rmsnorm_launch(h, r, w, rows, d, eps, sum, y, yq, ys, st);
    if (e == hipSuccess) {
        q8s::GemvArgs g{Wq, Ws, n_out, d, act == 0 ? y : nullptr, act == 1 ? yq : nullptr, act == 1 ? ys : nullptr,
                        rows, out, act};
        e = q8s::gemv_launch(g, st);
    }
    return launched(e, fn);
}

int add_rmsnorm_gemv_x2(const float *h, const float *r, const float *w, float eps, const int8_t *Wq,
                        const float *Ws, int64_t rows, int64_t d, int64_t n_out, float *sum, float *y, int8_t *yq,
                        int8_t *yl, float *ys, float *out, void *stream)
{
    const char *fn = "add_rmsnorm_gemv_x2";
    int rc;
    if ((rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "d", d)) ||
        (rc = check_count(fn, "n_out", n_out, INT32_MAX / 2)))
        return rc;
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    const size_t n = (size_t)(rows * d);
    std::vector<Span> ins = {{h, n * 4, "h"},
                             {r, n * 4, "r"},
                             {w, (size_t)d * 4, "w"},
                             {Wq, (size_t)(n_out * d), "Wq"},
                             {Ws, (size_t)n_out * (size_t)(d / 32) * 4, "Ws"}};
    std::vector<Span> outs = {{sum, n * 4, "sum"}, {out, (size_t)(rows * n_out) * 4, "out"}, {y, n * 4, "y"},
                              {yq, n, "yq"}, {yl, n, "yl"}, {ys, n / 32 * 4, "ys"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    const hipStream_t st = as_stream(stream);
    if (q8s::norm_gemv_supported(rows, d)) {
        q8s::NormGemvArgs a{h, r, w, eps, Wq, Ws, d, n_out, sum, y, yq, ys, out, 2, yl};
        return launched(q8s::norm_gemv_launch(a, st), fn);
    }
    hipError_t e = q8s::add_rmsnorm_launch(h, r, w, rows, d, eps, sum, y, yq, ys, st, yl);
    if (e == hipSuccess) {
        q8s::GemvArgs g{Wq, Ws, n_out, d, nullptr, yq, ys, rows, out, 2, yl};
        e = q8s::gemv_launch(g, st);
    }
    return launched(e, fn);
}

namespace {

int norm_router_common(const char *fn, const float *h, const float *r, const float *w, float eps,
                       const q8s::RouterRows &rt, int64_t rows, int64_t d, int64_t E, float *sum, float *x,
                       int8_t *xq, float *xs, double *logits, void *stream)
{
    int rc;
    if ((rc = check_count(fn, "rows", rows, 65535)) || (rc = check_dim32(fn, "d", d)) ||
        (rc = check_count(fn, "E", E, Q8S_MAX_E)))
        return rc;
    if (!q8s::norm_logits_supported(d))
        return fail(Q8S_EUNSUPPORTED, "%s: d = %lld exceeds the %lld values a fused norm + router row holds; use "
                    "add_rmsnorm_q8 then moe_route_topk", fn, (long long)d, (long long)q8s::NORM_LOGITS_MAX_D);
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    if ((xq == nullptr) != (xs == nullptr))
        return fail(Q8S_EINVAL, "%s: `xq` and `xs` are given together or not at all", fn);
    if (!x && !xq)
        return fail(Q8S_EINVAL, "%s: neither `x` nor `xq` is given -- the normed row would not be written", fn);
    const size_t n = (size_t)(rows * d);
    std::vector<Span> ins = {{h, n * 4, "h"}, {r, n * 4, "r"}, {w, (size_t)d * 4, "w"}};
    if (rt.Wrq) {
        ins.push_back({rt.Wrq, (size_t)(E * d), "Wrq"});
        ins.push_back({rt.Wrs, (size_t)(E * d / 32) * 4, "Wrs"});
    } else {
        ins.push_back({rt.Wr, (size_t)(E * d) * 4, "Wr"});
    }
    std::vector<Span> outs = {{sum, n * 4, "sum"}, {logits, (size_t)(rows * E) * 8, "logits"}};
    if (x)
        outs.push_back({x, n * 4, "x"});
    if (xq) {
        outs.push_back({xq, n, "xq"});
        outs.push_back({xs, n / 32 * 4, "xs"});
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    clear_stale();
    return launched(q8s::norm_logits_launch(h, r, w, rows, d, eps, rt, E, sum, x, xq, xs, logits, as_stream(stream)),
                    fn);
}

} // namespace

int add_rmsnorm_router(const float *h, const float *r, const float *w, float eps, const float *Wr, int64_t rows,
                       int64_t d, int64_t E, float *sum, float *x, int8_t *xq, float *xs, double *logits, void *stream)
{
    return norm_router_common("add_rmsnorm_router", h, r, w, eps, q8s::RouterRows{Wr, nullptr, nullptr, 0}, rows, d,
                              E, sum, x, xq, xs, logits, stream);
}

int add_rmsnorm_router_q8(const float *h, const float *r, const float *w, float eps, const int8_t *Wrq,
                          const float *Wrs, int64_t rows, int64_t d, int64_t E, float *sum, float *x, int8_t *xq,
                          float *xs, double *logits, int act, void *stream)
{
    const char *fn = "add_rmsnorm_router_q8";
    int rc;
    if ((rc = check_act(fn, act)))
        return rc;
    if (!Wrq)
        return fail(Q8S_EINVAL, "%s: `Wrq` is null", fn);
    return norm_router_common(fn, h, r, w, eps, q8s::RouterRows{nullptr, Wrq, Wrs, act}, rows, d, E, sum, x, xq, xs,
                              logits, stream);
}

namespace {

// The shared expert's arguments of a stage call: none (sdff 0, NULL
// matrices) or sdff a multiple of 32 fitting the down-combine's partials.
int check_shared(const char *fn, int64_t sdff, int64_t dff, int64_t k, std::initializer_list<const void *> mats)
{
    int rc;
    if (sdff < 0)
        return fail(Q8S_EINVAL, "%s: sdff = %lld is negative", fn, (long long)sdff);
    if (sdff == 0) {
        for (const void *p : mats)
            if (p)
                return fail(Q8S_EINVAL, "%s: shared-expert matrices given with sdff = 0", fn);
        return 0;
    }
    if ((rc = check_dim32(fn, "sdff", sdff)))
        return rc;
    if (!q8s::shared_fits(dff, sdff, k))
        return fail(Q8S_EUNSUPPORTED, "%s: a shared expert of sdff = %lld next to k = %lld experts of dff = %lld "
                    "exceeds the down-combine's 512 (slot, slice) partials", fn, (long long)sdff, (long long)k,
                    (long long)dff);
    return 0;
}

int topk_gate_up_common(const char *fn, const double *logits, const float *x, const int8_t *xq, const float *xs,
                        const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus, const int8_t *Sgq,
                        const float *Sgs, const int8_t *Suq, const float *Sus, int64_t sdff, int64_t rows, int64_t d,
                        int64_t dff, int64_t E, int64_t k, int32_t *idx, float *wts, float *h, int8_t *hq, float *hs,
                        int act, void *stream)
{
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_moe_shape(fn, rows, d, dff, E, k)) ||
        (rc = check_shared(fn, sdff, dff, k, {Sgq, Sgs, Suq, Sus})))
        return rc;
    if (E > q8s::ROUTE_FUSED_MAX_E)
        return fail(Q8S_EUNSUPPORTED, "%s: E = %lld experts exceed the %d a gate-up workgroup ranks itself; use "
                    "moe_route_topk then moe_gate_up", fn, (long long)E, q8s::ROUTE_FUSED_MAX_E);
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    const size_t nh = (size_t)(rows * (k * dff + sdff));
    std::vector<Span> ins = {{logits, (size_t)(rows * E) * 8, "logits"}, {Wgq, wq, "Wgq"}, {Wgs, wsb, "Wgs"},
                             {Wuq, wq, "Wuq"}, {Wus, wsb, "Wus"}};
    if (sdff > 0) {
        const size_t sq = (size_t)sdff * (size_t)d, ss = (size_t)sdff * (size_t)(d / 32) * 4;
        ins.push_back({Sgq, sq, "Sgq"});
        ins.push_back({Sgs, ss, "Sgs"});
        ins.push_back({Suq, sq, "Suq"});
        ins.push_back({Sus, ss, "Sus"});
    }
    std::vector<Span> outs = {{idx, (size_t)(rows * k) * 4, "idx"}, {wts, (size_t)(rows * k) * 4, "wts"}};
    if (act == Q8S_ACT_F32) {
        ins.push_back({x, (size_t)(rows * d) * 4, "x"});
        outs.push_back({h, nh * 4, "h"});
    } else {
        ins.push_back({xq, (size_t)(rows * d), "xq"});
        ins.push_back({xs, (size_t)(rows * d / 32) * 4, "xs"});
        // the grouped chunk kernels write the float32 hidden rows and then
        // form their Q8_0 form in a pass of their own, which a caller may
        // leave out (hq and hs both NULL) to quantise the rows itself
        const bool chunk = rows > 1 && q8s::chunk_supported(d, dff);
        if (!hq && !hs && !chunk)
            return fail(Q8S_EINVAL, "%s: int8 numerics: `hq`/`hs` are required (only a chunk of rows in the grouped "
                        "kernels may leave out the hidden rows' Q8_0 form)", fn);
        if (h)
            outs.push_back({h, nh * 4, "h"});
        if (hq || hs) {
            outs.push_back({hq, nh, "hq"});
            outs.push_back({hs, nh / 32 * 4, "hs"});
        }
    }
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.x = act == 0 ? x : nullptr;
    a.xq = act == 1 ? xq : nullptr;
    a.xs = act == 1 ? xs : nullptr;
    a.Wgq = Wgq;
    a.Wgs = Wgs;
    a.Wuq = Wuq;
    a.Wus = Wus;
    a.Sgq = Sgq;
    a.Sgs = Sgs;
    a.Suq = Suq;
    a.Sus = Sus;
    a.sdff = sdff;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.h = h;
    a.hq = act == 1 ? hq : nullptr;
    a.hs = act == 1 ? hs : nullptr;
    a.act = act;
    a.logits = logits;
    a.idx_w = idx;
    a.wts_w = wts;
    clear_stale();
    return launched(q8s::route_gate_up_launch(a, as_stream(stream)), fn);
}

} // namespace

int moe_topk_gate_up(const double *logits, const float *x, const int8_t *xq, const float *xs, const int8_t *Wgq,
                     const float *Wgs, const int8_t *Wuq, const float *Wus, int64_t rows, int64_t d, int64_t dff,
                     int64_t E, int64_t k, int32_t *idx, float *wts, float *h, int8_t *hq, float *hs, int act,
                     void *stream)
{
    return topk_gate_up_common("moe_topk_gate_up", logits, x, xq, xs, Wgq, Wgs, Wuq, Wus, nullptr, nullptr, nullptr,
                               nullptr, 0, rows, d, dff, E, k, idx, wts, h, hq, hs, act, stream);
}

int moe_topk_gate_up_x2(const double *logits, const int8_t *xq, const int8_t *xl, const float *xs,
                        const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus, int64_t rows,
                        int64_t d, int64_t dff, int64_t E, int64_t k, int32_t *idx, float *wts, int8_t *hq,
                        int8_t *hl, float *hs, void *stream)
{
    const char *fn = "moe_topk_gate_up_x2";
    int rc;
    if ((rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    if (E > q8s::ROUTE_FUSED_MAX_E)
        return fail(Q8S_EUNSUPPORTED, "%s: E = %lld experts exceed the %d a gate-up workgroup ranks itself", fn,
                    (long long)E, q8s::ROUTE_FUSED_MAX_E);
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    const size_t nh = (size_t)(rows * k * dff), nx = (size_t)(rows * d);
    std::vector<Span> ins = {{logits, (size_t)(rows * E) * 8, "logits"}, {Wgq, wq, "Wgq"}, {Wgs, wsb, "Wgs"},
                             {Wuq, wq, "Wuq"}, {Wus, wsb, "Wus"}, {xq, nx, "xq"}, {xl, nx, "xl"},
                             {xs, nx / 32 * 4, "xs"}};
    std::vector<Span> outs = {{idx, (size_t)(rows * k) * 4, "idx"}, {wts, (size_t)(rows * k) * 4, "wts"},
                              {hq, nh, "hq"}, {hl, nh, "hl"}, {hs, nh / 32 * 4, "hs"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.xq = xq;
    a.xl = xl;
    a.xs = xs;
    a.Wgq = Wgq;
    a.Wgs = Wgs;
    a.Wuq = Wuq;
    a.Wus = Wus;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.hq = hq;
    a.hl = hl;
    a.hs = hs;
    a.act = 2;
    a.logits = logits;
    a.idx_w = idx;
    a.wts_w = wts;
    clear_stale();
    return launched(q8s::route_gate_up_launch(a, as_stream(stream)), fn);
}

int moe_topk_gate_up_ex(const double *logits, const float *x, const int8_t *xq, const float *xs, const int8_t *Wgq,
                        const float *Wgs, const int8_t *Wuq, const float *Wus, const int8_t *Sgq, const float *Sgs,
                        const int8_t *Suq, const float *Sus, int64_t sdff, int64_t rows, int64_t d, int64_t dff,
                        int64_t E, int64_t k, int32_t *idx, float *wts, float *h, int8_t *hq, float *hs, int act,
                        void *stream)
{
    return topk_gate_up_common("moe_topk_gate_up_ex", logits, x, xq, xs, Wgq, Wgs, Wuq, Wus, Sgq, Sgs, Suq, Sus, sdff,
                               rows, d, dff, E, k, idx, wts, h, hq, hs, act, stream);
}

int moe_down_combine_ex(const float *h, const int8_t *hq, const float *hs, const int8_t *Wdq, const float *Wds,
                        const int8_t *Sdq, const float *Sds, int64_t sdff, const int32_t *idx, const float *wts,
                        int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, float *y, int act, void *stream)
{
    const char *fn = "moe_down_combine_ex";
    int rc;
    if ((rc = check_act(fn, act)) || (rc = check_moe_shape(fn, rows, d, dff, E, k)) ||
        (rc = check_shared(fn, sdff, dff, k, {Sdq, Sds})))
        return rc;
    const size_t nh = (size_t)(rows * (k * dff + sdff));
    std::vector<Span> ins = {{Wdq, (size_t)(E * d) * (size_t)dff, "Wdq"},
                             {Wds, (size_t)(E * d) * (size_t)(dff / 32) * 4, "Wds"},
                             {idx, (size_t)(rows * k) * 4, "idx"},
                             {wts, (size_t)(rows * k) * 4, "wts"}};
    if (sdff > 0) {
        ins.push_back({Sdq, (size_t)d * (size_t)sdff, "Sdq"});
        ins.push_back({Sds, (size_t)d * (size_t)(sdff / 32) * 4, "Sds"});
    }
    if (act == Q8S_ACT_F32) {
        ins.push_back({h, nh * 4, "h"});
    } else {
        ins.push_back({hq, nh, "hq"});
        ins.push_back({hs, nh / 32 * 4, "hs"});
    }
    std::vector<Span> outs = {{y, (size_t)(rows * d) * 4, "y"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)) || (rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::MoeArgs a{};
    a.h = act == 0 ? const_cast<float *>(h) : nullptr;
    a.hq = act == 1 ? const_cast<int8_t *>(hq) : nullptr;
    a.hs = act == 1 ? const_cast<float *>(hs) : nullptr;
    a.Wdq = Wdq;
    a.Wds = Wds;
    a.Sdq = Sdq;
    a.Sds = Sds;
    a.sdff = sdff;
    a.idx = idx;
    a.wts = wts;
    a.rows = rows;
    a.d = d;
    a.dff = dff;
    a.E = E;
    a.k = k;
    a.y = y;
    a.act = act;
    clear_stale();
    return launched(q8s::row_down_launch(a, as_stream(stream)), fn);
}

namespace {

int block_common(const char *fn, const float *h, const float *r, const float *w, float eps,
                 const q8s::RouterRows &rt, const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                 const int8_t *Wdq, const float *Wds, const int8_t *Sgq, const float *Sgs, const int8_t *Suq,
                 const float *Sus, const int8_t *Sdq, const float *Sds, int64_t sdff, int64_t rows, int64_t d,
                 int64_t dff, int64_t E, int64_t k, float *sum, int32_t *idx, float *wts, float *out, int act,
                 void *scratch, size_t scratch_bytes, void *stream)
{
    int rc;
    if ((act != 2 && (rc = check_act(fn, act))) || (rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    if (act == 2) {
        // two words: the three-launch form, or a chunk's grouped kernels
        if (!q8s::block_chunk(rows, d, dff, act) && !q8s::block_fused(rows, d, dff, E, act))
            return fail(Q8S_EUNSUPPORTED,
                        "%s: two-word numerics (act 2) need E <= %d and d <= %lld, or a chunk of rows with d <= 2048 "
                        "and dff <= 4096", fn, (int)q8s::ROUTE_FUSED_MAX_E, (long long)q8s::NORM_LOGITS_MAX_D);
    }
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    if ((rc = check_shared(fn, sdff, dff, k, {Sgq, Sgs, Suq, Sus, Sdq, Sds})))
        return rc;
    const size_t n = (size_t)(rows * d);
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    std::vector<Span> ins = {{h, n * 4, "h"},
                             {r, n * 4, "r"},
                             {w, (size_t)d * 4, "w"},
                             {Wgq, wq, "Wgq"},
                             {Wgs, wsb, "Wgs"},
                             {Wuq, wq, "Wuq"},
                             {Wus, wsb, "Wus"},
                             {Wdq, (size_t)(E * d) * (size_t)dff, "Wdq"},
                             {Wds, (size_t)(E * d) * (size_t)(dff / 32) * 4, "Wds"}};
    if (rt.Wrq) {
        ins.push_back({rt.Wrq, (size_t)(E * d), "Wrq"});
        ins.push_back({rt.Wrs, (size_t)(E * d / 32) * 4, "Wrs"});
    } else {
        ins.push_back({rt.Wr, (size_t)(E * d) * 4, "Wr"});
    }
    if (sdff > 0) {
        const size_t sq = (size_t)sdff * (size_t)d, ss = (size_t)sdff * (size_t)(d / 32) * 4;
        ins.push_back({Sgq, sq, "Sgq"});
        ins.push_back({Sgs, ss, "Sgs"});
        ins.push_back({Suq, sq, "Suq"});
        ins.push_back({Sus, ss, "Sus"});
        ins.push_back({Sdq, sq, "Sdq"});
        ins.push_back({Sds, (size_t)d * (size_t)(sdff / 32) * 4, "Sds"});
    }
    std::vector<Span> outs = {{sum, n * 4, "sum"},
                              {idx, (size_t)(rows * k) * 4, "idx"},
                              {wts, (size_t)(rows * k) * 4, "wts"},
                              {out, n * 4, "out"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    const size_t need = q8s::block_scratch_bytes(rows, d, dff, sdff, E, k, act);
    if (!scratch || scratch_bytes < need)
        return fail(Q8S_ESCRATCH,
                    "%s: scratch of %zu bytes given, %zu needed (logits, the normed row, the hidden rows)", fn,
                    scratch ? scratch_bytes : (size_t)0, need);
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
        return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
    outs.push_back({scratch, need, "scratch"});
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::BlockArgs b{h,    r,    w,  eps, rt,  Wgq, Wgs, Wuq, Wus, Wdq, Wds,     rows, d,   dff, E,   k,  sum,
                     idx,  wts,  out, act, scratch, Sgq, Sgs, Suq, Sus, Sdq, Sds, sdff};
    clear_stale();
    return launched(q8s::block_launch(b, as_stream(stream)), fn);
}

} // namespace

int moe_ffn_block(const float *h, const float *r, const float *w, float eps, const float *Wr, const int8_t *Wgq,
                  const float *Wgs, const int8_t *Wuq, const float *Wus, const int8_t *Wdq, const float *Wds,
                  int64_t rows, int64_t d, int64_t dff, int64_t E, int64_t k, float *sum, int32_t *idx, float *wts,
                  float *out, int act, void *scratch, size_t scratch_bytes, void *stream)
{
    return block_common("moe_ffn_block", h, r, w, eps, q8s::RouterRows{Wr, nullptr, nullptr, 0}, Wgq, Wgs, Wuq, Wus,
                        Wdq, Wds, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, rows, d, dff, E, k, sum, idx,
                        wts, out, act, scratch, scratch_bytes, stream);
}

int moe_ffn_stack(const float *h, const float *r, int64_t layers, const float *const *w, const float *const *Wr,
                  const int8_t *const *Wgq, const float *const *Wgs, const int8_t *const *Wuq,
                  const float *const *Wus, const int8_t *const *Wdq, const float *const *Wds, int64_t rows,
                  int64_t d, int64_t dff, int64_t E, int64_t k, float eps, float *out, int32_t *idx, float *wts,
                  int act, void *scratch, size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_ffn_stack";
    int rc;
    if ((act != 2 && (rc = check_act(fn, act))) || (rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    if (act == 2 && !q8s::block_chunk(rows, d, dff, act) && !q8s::block_fused(rows, d, dff, E, act))
        return fail(Q8S_EUNSUPPORTED,
                    "%s: two-word numerics (act 2) need E <= %d and d <= %lld, or a chunk of rows with d <= 2048 "
                    "and dff <= 4096", fn, (int)q8s::ROUTE_FUSED_MAX_E, (long long)q8s::NORM_LOGITS_MAX_D);
    if (layers < 1 || layers > 1024)
        return fail(layers < 1 ? Q8S_EINVAL : Q8S_EUNSUPPORTED, "%s: layers = %lld: 1 <= layers <= 1024", fn,
                    (long long)layers);
    if (!(eps >= 0.0f) || eps != eps)
        return fail(Q8S_EINVAL, "%s: eps must be a finite value >= 0", fn);
    if (!w || !Wr || !Wgq || !Wgs || !Wuq || !Wus || !Wdq || !Wds)
        return fail(Q8S_EINVAL, "%s: a per-layer pointer array (w, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds) is null", fn);
    const size_t n = (size_t)(rows * d);
    const size_t wq = (size_t)(E * dff) * (size_t)d, wsb = (size_t)(E * dff) * (size_t)(d / 32) * 4;
    const size_t dq = (size_t)(E * d) * (size_t)dff, dsb = (size_t)(E * d) * (size_t)(dff / 32) * 4;
    std::vector<Span> ins = {{h, n * 4, "h"}, {r, n * 4, "r"}};
    std::vector<std::string> names;
    names.reserve((size_t)layers * 8);
    for (int64_t l = 0; l < layers; l++) {
        const void *p[8] = {w[l], Wr[l], Wgq[l], Wgs[l], Wuq[l], Wus[l], Wdq[l], Wds[l]};
        const size_t b[8] = {(size_t)d * 4, (size_t)(E * d) * 4, wq, wsb, wq, wsb, dq, dsb};
        const char *nm[8] = {"w", "Wr", "Wgq", "Wgs", "Wuq", "Wus", "Wdq", "Wds"};
        for (int i = 0; i < 8; i++) {
            names.push_back(std::string(nm[i]) + "[" + std::to_string(l) + "]");
            ins.push_back({p[i], b[i], names.back().c_str()});
        }
    }
    std::vector<Span> outs = {{out, n * 4, "out"},
                              {idx, (size_t)(layers * rows * k) * 4, "idx"},
                              {wts, (size_t)(layers * rows * k) * 4, "wts"}};
    if ((rc = check_ptrs(fn, ins)) || (rc = check_ptrs(fn, outs)))
        return rc;
    const size_t need = q8s::stack_scratch_bytes(rows, d, dff, E, k, act);
    if (!scratch || scratch_bytes < need)
        return fail(Q8S_ESCRATCH,
                    "%s: scratch of %zu bytes given, %zu needed (a block's, and the residual stream between layers)",
                    fn, scratch ? scratch_bytes : (size_t)0, need);
    if (reinterpret_cast<uintptr_t>(scratch) % 256 != 0)
        return fail(Q8S_EALIGN, "%s: `scratch` is not 256-byte aligned", fn);
    outs.push_back({scratch, need, "scratch"});
    if ((rc = check_disjoint(fn, ins, outs)))
        return rc;
    q8s::StackArgs a{h, r, layers, w, Wr, Wgq, Wgs, Wuq, Wus, Wdq, Wds, rows, d, dff, E, k, eps, out, idx, wts, act,
                     scratch};
    clear_stale();
    return launched(q8s::stack_launch(a, as_stream(stream)), fn);
}

} // extern "C"

namespace {

// The allocation-free block's scratch: one fixed array in device memory,
// which every GPU the library runs on holds from the module's load to the
// end of the process.  In host code `scratch` names a host-side stand-in, not
// a device address: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[Q8S_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEV = 64;
void *g_noalloc_ptr[NOALLOC_MAX_DEV];
std::mutex g_noalloc_mu;

// This device's copy of the array, looked up on its first use; null (with a
// message) if the device or the lookup fails.
void *noalloc_scratch(const char *fn)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEV) {
        (void)hipGetLastError();
        fail(Q8S_ELAUNCH, "%s: no current HIP device (or device index %d beyond %d)", fn, dev, NOALLOC_MAX_DEV);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            fail(Q8S_ELAUNCH, "%s: hipGetSymbolAddress of the static scratch failed on device %d: %s", fn, dev,
                 hipGetErrorString(e));
            return nullptr;
        }
        g_noalloc_ptr[dev] = p;
    }
    return g_noalloc_ptr[dev];
}

} // namespace

extern "C" {

int moe_ffn_block_noalloc(const float *h, const float *r, const float *w, float eps, const float *Wr,
                          const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                          const int8_t *Wdq, const float *Wds, int64_t rows, int64_t d, int64_t dff, int64_t E,
                          int64_t k, float *sum, int32_t *idx, float *wts, float *out, int act, void *stream)
{
    const char *fn = "moe_ffn_block_noalloc";
    int rc;
    if ((act != 2 && (rc = check_act(fn, act))) || (rc = check_moe_shape(fn, rows, d, dff, E, k)))
        return rc;
    const size_t need = q8s::block_scratch_bytes(rows, d, dff, 0, E, k, act);
    if (need > (size_t)Q8S_NOALLOC_SCRATCH_BYTES)
        return fail(Q8S_EUNSUPPORTED,
                    "%s: these sizes need %zu bytes of scratch; the library's static scratch holds %zu "
                    "(use moe_ffn_block with a scratch of your own)",
                    fn, need, (size_t)Q8S_NOALLOC_SCRATCH_BYTES);
    void *p = noalloc_scratch(fn);
    if (!p)
        return Q8S_ELAUNCH;
    return block_common(fn, h, r, w, eps, q8s::RouterRows{Wr, nullptr, nullptr, 0}, Wgq, Wgs, Wuq, Wus, Wdq, Wds,
                        nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, rows, d, dff, E, k, sum, idx, wts,
                        out, act, p, (size_t)Q8S_NOALLOC_SCRATCH_BYTES, stream);
}

int moe_ffn_block_ex(const float *h, const float *r, const float *w, float eps, const float *Wr, const int8_t *Wrq,
                     const float *Wrs, const int8_t *Wgq, const float *Wgs, const int8_t *Wuq, const float *Wus,
                     const int8_t *Wdq, const float *Wds, const int8_t *Sgq, const float *Sgs, const int8_t *Suq,
                     const float *Sus, const int8_t *Sdq, const float *Sds, int64_t sdff, int64_t rows, int64_t d,
                     int64_t dff, int64_t E, int64_t k, float *sum, int32_t *idx, float *wts, float *out, int act,
                     void *scratch, size_t scratch_bytes, void *stream)
{
    const char *fn = "moe_ffn_block_ex";
    if ((Wr != nullptr) == (Wrq != nullptr))
        return fail(Q8S_EINVAL, "%s: give the router as float rows `Wr` or as Q8_0 rows `Wrq`/`Wrs`, exactly one", fn);
    return block_common(fn, h, r, w, eps, q8s::RouterRows{Wr, Wrq, Wrs, act}, Wgq, Wgs, Wuq, Wus, Wdq, Wds, Sgq, Sgs,
                        Suq, Sus, Sdq, Sds, sdff, rows, d, dff, E, k, sum, idx, wts, out, act, scratch, scratch_bytes,
                        stream);
}

} // extern "C"

namespace q8s {

int device_cus()
{
    constexpr int MAX_DEV = 64;
    static std::atomic<int> cache[MAX_DEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) {
        (void)hipGetLastError();
        return 256;
    }
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

} // namespace q8s
