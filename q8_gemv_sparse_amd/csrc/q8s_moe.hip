// q8s_moe.hip -- the sparse MoE FFN's gate-up and down-combine kernels.
//
// The block is fn emit_moe_forward's (codegen_cuda::qwen_emit module page):
// every kept expert's SwiGLU with an expert-indexed weight base, then the
// weighted combine.  The weights are struct MoeWeights' stacked Q8_0 rows:
// gate/up [E*dff, d] (expert e from row e*dff), down [E*d, dff] (from e*d).
// The expert index is read on the device, so the choices never travel to the
// host; an index outside [0, E) reads nothing and contributes zero.
//
// gate-up (one workgroup per tile of hidden outputs of one (row, slot)): each
//   wave streams gate and up rows side by side against the activation slice
//   in its registers and forms SiLU(g)*u; in int8 mode a tile is one 32-value
//   block, which the workgroup quantises once into the hidden row's Q8_0 form
//   (arena.rs fn scratch: hq/hs).
// These kernels serve one row at a time (a batch of rows in f32 numerics runs
// them row by row); a chunk of rows in int8 numerics goes to the grouped
// kernels of q8s_moe_chunk.hip.
// route + gate-up (the mixture block's fused path): the same tiles, each
//   workgroup first taking the row's top-K from the router logits itself.
// A shared expert (lane_link.rs fn class_launch, SharedExpertFusion arm: an
// always-on expert carried by the mixture's launch) adds its own tiles after
// the K slots' in the gate-up grid, its hidden row after the K routed ones
// (arena.rs fn scratch: K*dff + sdff hidden values a row), and its slices
// after the (slot, slice) pairs of the down-combine, summed with weight 1
// after the routed sum.
// down-combine (one workgroup per 8 outputs of one row): waves take
//   (slot, k-slice) pairs, so all K experts' rows of those outputs stream at
//   once; the partials meet in LDS and are weighted and summed in slot order.
#include "q8s_device.h"
#include "q8s_internal.h"

namespace q8s {


constexpr int DN_TILE = 8;
constexpr int MAX_KS = 16;
constexpr int GU_MAX_KS = 32;
constexpr int DN_MAX_WAVES = 8;
// (slot, slice) pairs a down-combine workgroup holds partials of
constexpr int DN_MAX_PAIRS = Q8S_MAX_K_DEV * MAX_KS;

// LDS of a gate-up workgroup: the slices' partial sums (rows cut into
// slices) and the tile's hidden values (int8 numerics).
template <int T>
struct GuLds {
    float gp[GU_MAX_KS][T];
    float up[GU_MAX_KS][T];
    float hv[T];
};

// One gate-up tile: the T hidden outputs from blockIdx.x*T of choice (row, j)
// of expert e.  With the row in one slice (ks == 1) each wave finishes its own
// outputs; otherwise the waves deal out (slice, step) items and the slices'
// partial sums meet in LDS.
// The tile's weight rows start at row rbase of the gate/up matrices given
// (an expert's or the shared expert's), its hidden values at hbase.
template <int ACT, int LPR, int C, int V>
Q8S_DEV void gate_up_tile(GuLds<GuShape<ACT, LPR, C, V>::T> &sm, bool valid, int64_t row, int64_t rbase, int64_t hbase,
                          const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xs,
                          const int8_t *__restrict__ Wgq, const float *__restrict__ Wgs,
                          const int8_t *__restrict__ Wuq, const float *__restrict__ Wus, int d, int ks,
                          float *__restrict__ h, int8_t *__restrict__ hq, float *__restrict__ hs,
                          const int8_t *__restrict__ xl, int8_t *__restrict__ hl)
{
    using S = GuShape<ACT, LPR, C, V>;
    constexpr int G = S::G, U = S::U, OPS = S::OPS, T = S::T, NW = S::NW;
    constexpr int STEPS = T / OPS;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, lig = lane % LPR, grp = lane / LPR;
    const int nch = d >> 4, nb = d >> 5;

    // A wave's items are wid, wid + NW, ... (ks of them: T = NW * OPS); item i
    // is slice i % ks of step i / ks.  For a row cut into slices, with ks
    // dividing NW, a wave's slice never changes, so its activation slice is
    // loaded once, before its first weight rows (waits on the vector-memory
    // counter are in issue order); reloading it for every item measured
    // several per cent slower on int8 rows cut into 4 slices.  Float32 slices
    // (16 registers a chunk) and waves with a single item load their weight
    // rows first: the activation slice then lives in registers for less time,
    // which for float32 decides occupancy.
    const int nitems = ks * STEPS;
    const bool fixed = ACT >= 1 && ks > 1 && (NW % ks) == 0;
    auto load_xs = [&](int s, XSlice<ACT, C> &xv) {
        const int ch0 = s * LPR * C;
        if constexpr (ACT == 2)
            load_x2<LPR, C>(xv, xq + row * d, xl + row * d, xs + row * nb, ch0, min(LPR * C, nch - ch0), lig);
        else
            load_x<LPR, C>(xv, ACT == 0 ? x + row * d : nullptr, ACT == 1 ? xq + row * d : nullptr,
                           ACT == 1 ? xs + row * nb : nullptr, ch0, min(LPR * C, nch - ch0), lig);
    };
    XSlice<ACT, C> xv;
    if (fixed && wid < nitems)
        load_xs(wid % ks, xv);
    for (int item = wid; item < nitems; item += NW) {
        const int s = item % ks, st = item / ks;
        const int ch0 = s * LPR * C;
        const int sl = min(LPR * C, nch - ch0);
        RowSlice<C> wg[U], wu[U];
        if (valid) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int64_t o = rbase + st * OPS + u * G + grp;
                load_row<LPR, C>(wg[u], Wgq + o * d, Wgs + o * nb, ch0, sl, lig);
                load_row<LPR, C>(wu[u], Wuq + o * d, Wus + o * nb, ch0, sl, lig);
            }
        }
        if (!fixed)
            load_xs(s, xv);
#pragma unroll
        for (int u = 0; u < U; u++) {
            float g = 0.0f, v = 0.0f;
            if (valid) {
                g = row_dot(wg[u], xv, lig);
                v = row_dot(wu[u], xv, lig);
            }
            g = group_sum<LPR>(g);
            v = group_sum<LPR>(v);
            const int ol = st * OPS + u * G + grp;
            if (lig == 0) {
                if (ks == 1) {
                    const float r = valid ? silu(g) * v : 0.0f;
                    if (ACT >= 1)
                        sm.hv[ol] = r;
                    if (h)
                        h[hbase + ol] = r;
                } else {
                    sm.gp[s][ol] = g;
                    sm.up[s][ol] = v;
                }
            }
        }
    }
    if (ks == 1 && ACT == 0)
        return;
    __syncthreads();
    if (ks > 1) {
        for (int t = threadIdx.x; t < T; t += blockDim.x) {
            float g = 0.0f, v = 0.0f;
            for (int s = 0; s < ks; s++) {
                g += sm.gp[s][t];
                v += sm.up[s][t];
            }
            const float r = valid ? silu(g) * v : 0.0f;
            if (ACT >= 1)
                sm.hv[t] = r;
            if (h)
                h[hbase + t] = r;
        }
        if (ACT >= 1)
            __syncthreads();
    }
    if (ACT >= 1 && wid == 0) {
        // the tile is one Q8_0 block of the hidden row: quantise it once
        const int t = lane & 31;
        const float v = sm.hv[t];
        float amax = fabsf(v);
        for (int off = 16; off >= 1; off >>= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
        const float dsc = q8_scale(amax);
        const float id = q8_inv(dsc);
        if (lane < 32) {
            const int q = q8_code(v, id);
            hq[hbase + t] = (int8_t)q;
            if (ACT == 2)
                hl[hbase + t] = (int8_t)q8_low(v, id, q);
        }
        if (lane == 0)
            hs[hbase / QB] = dsc;
    }
}

// The shared expert's matrices (none when sdff == 0): gate/up [sdff, d],
// down [d, sdff].
struct SharedW {
    const int8_t *gq;
    const float *gs;
    const int8_t *uq;
    const float *us;
    const int8_t *dq;
    const float *ds;
    int sdff;
};

// A row's gate-up workgroups: bx < k*tpe are slot bx/tpe's tile bx%tpe (tpe
// tiles of T an expert); the rest are the shared expert's tiles.
struct GuTile {
    int j, o0;
    bool shared;
};
template <bool SH>
Q8S_DEV GuTile gu_tile(int bx, int k, int tpe, int T)
{
    if (!SH || bx < k * tpe)
        return {bx / tpe, (bx % tpe) * T, false};
    return {k, (bx - k * tpe) * T, true};
}

// gate-up with the choices given: one workgroup per tile of one (row, slot),
// grid (k*dff/T + sdff/T, rows).  SH: with a shared expert (a kernel of its
// own, so the mixture without one runs the plain code).
template <int ACT, int LPR, int C, bool SH, int V>
__global__ void __launch_bounds__((GuShape<ACT, LPR, C, V>::NW * WAVE))
    k_gate_up(const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xs,
              const int8_t *__restrict__ Wgq, const float *__restrict__ Wgs, const int8_t *__restrict__ Wuq,
              const float *__restrict__ Wus, SharedW sw, const int32_t *__restrict__ idx, int d, int dff, int E,
              int k, int ks, float *__restrict__ h, int8_t *__restrict__ hq, float *__restrict__ hs,
              const int8_t *__restrict__ xl, int8_t *__restrict__ hl)
{
    constexpr int T = GuShape<ACT, LPR, C, V>::T;
    __shared__ GuLds<T> sm;
    const int64_t row = blockIdx.y;
    const GuTile t = gu_tile<SH>(blockIdx.x, k, dff / T, T);
    const int64_t hbase = row * ((int64_t)k * dff + (SH ? sw.sdff : 0)) + (int64_t)t.j * dff + t.o0;
    const int e = t.shared ? 0 : idx[row * k + t.j];
    const bool valid = t.shared || (e >= 0 && e < E);
    const int64_t rbase = t.shared ? t.o0 : (int64_t)(valid ? e : 0) * dff + t.o0;
    gate_up_tile<ACT, LPR, C, V>(sm, valid, row, rbase, hbase, x, xq, xs, t.shared ? sw.gq : Wgq,
                              t.shared ? sw.gs : Wgs, t.shared ? sw.uq : Wuq, t.shared ? sw.us : Wus, d, ks, h, hq,
                              hs, xl, hl);
}

// gate-up that first takes the row's top-K itself from the router logits:
// every routed workgroup ranks the row's E logits in LDS (topk_select), or
// for at most TOPK_WAVE_E experts in each wave's registers, and reads its
// expert from the result, so the choices need no launch of their own; the
// workgroup of tile 0, slot 0 writes the row's idx and wts for the
// down-combine launch.  The shared expert's workgroups need no ranking.
// (measured: the 8-expert block 70.97-71.10 -> 70.49-70.60 us a step; at 60
// experts the lanes' E compares cost more than the LDS pass, 24.45 against
// 23.77 us for the shared-expert block)
constexpr int TOPK_WAVE_E = 16;
template <int ACT, int LPR, int C, bool SH, int V>
__global__ void __launch_bounds__((GuShape<ACT, LPR, C, V>::NW * WAVE))
    k_route_gate_up(const double *__restrict__ logits, int32_t *__restrict__ idx, float *__restrict__ wts,
                    const float *__restrict__ x, const int8_t *__restrict__ xq, const float *__restrict__ xs,
                    const int8_t *__restrict__ Wgq, const float *__restrict__ Wgs, const int8_t *__restrict__ Wuq,
                    const float *__restrict__ Wus, SharedW sw, int d, int dff, int E, int k, int ks,
                    float *__restrict__ h, int8_t *__restrict__ hq, float *__restrict__ hs,
                    const int8_t *__restrict__ xl, int8_t *__restrict__ hl)
{
    static_assert(ROUTE_FUSED_MAX_E <= TOPK_LDS_E, "the row's logits fit the top-K LDS");
    constexpr int T = GuShape<ACT, LPR, C, V>::T;
    __shared__ GuLds<T> sm;
    __shared__ TopkLds tk;
    const int64_t row = blockIdx.y;
    const GuTile t = gu_tile<SH>(blockIdx.x, k, dff / T, T);
    const int64_t hbase = row * ((int64_t)k * dff + (SH ? sw.sdff : 0)) + (int64_t)t.j * dff + t.o0;
    if (t.shared) {
        gate_up_tile<ACT, LPR, C, V>(sm, true, row, t.o0, hbase, x, xq, xs, sw.gq, sw.gs, sw.uq, sw.us, d, ks, h, hq,
                                  hs, xl, hl);
        return;
    }
    const double *lr = logits + row * E;
    int e;
    if (E <= TOPK_WAVE_E) {
        // few experts: every wave ranks them itself, lane i logit i against
        // all E (the order of topk_select: code descending, index
        // ascending), and takes slot t.j's expert by ballot -- no LDS pass,
        // no barrier before the tile's first weight request
        const int lane = threadIdx.x & (WAVE - 1);
        const double li = lr[min(lane, E - 1)];
        const uint64_t ci = route_code(li);
        int rank = 0;
        for (int w = 0; w < E; w++) {
            const uint64_t cw = route_code(lr[w]);
            rank += (cw > ci || (cw == ci && w < lane)) ? 1 : 0;
        }
        const bool mine = lane < E;
        e = (int)__builtin_ctzll(__ballot(mine && rank == t.j));
        if (blockIdx.x == 0 && threadIdx.x < WAVE && mine && rank < k) {
            tk.ch[rank] = lane;  // for route_finish, read by this same wave
            tk.kl[rank] = li;
        }
    } else {
        topk_load(tk, lr, E);
        __syncthreads();
        topk_select(tk, E, k);
        __syncthreads();
        e = __builtin_amdgcn_readfirstlane(tk.ch[t.j]);
    }
    gate_up_tile<ACT, LPR, C, V>(sm, true, row, (int64_t)e * dff + t.o0, hbase, x, xq, xs, Wgq, Wgs, Wuq, Wus, d, ks, h,
                              hq, hs, xl, hl);
    // the choices and weights go out after the tile, off its critical path
    // (only the down-combine launch reads them)
    if (blockIdx.x == 0 && threadIdx.x < WAVE)
        route_finish(tk.kl, tk.ch, k, idx + row * k, wts + row * k);
}

// Rows a lane group takes per step of the down-combine (measured: one row a
// step for lane groups of 64 holding 4 chunks, e.g. 22 vs 23.4 us for the
// 8-expert block's int8 down projection; two for lane groups of 16 holding 3,
// so a wave's 8 rows of a 768-value hidden row load in one step: 18.25 vs
// 18.39 us for the 128-expert block; two for lane groups holding 2, in int8
// as in f32: 24.5 vs 25.2 us a step for the shared-expert block, whose
// 1408- and 5632-value hidden rows take lane groups of 64 holding 2).
template <int ACT, int LPR, int C>
constexpr int dn_unroll()
{
    if (ACT == 0)
        return C >= 3 ? 1 : (C == 2 ? 2 : (LPR == 16 ? 2 : 4));
    if (C == 3 && LPR == 16)
        return 2;
    return C >= 3 ? 1 : (C == 2 ? 2 : (LPR == 16 ? 2 : 4));
}

// Waves take (slot, slice) pairs: pairs j*ks + s for the K slots, then
// k*ks + s for the shared expert's kss slices of its sdff-long rows (the same
// lane shape).  The grid is (d / DN_TILE, rows).  With y_add the output is
// y_add + the mixture, one float32 add: the residual stream folded into the
// epilogue (forward_shim.rs module doc: the mixture's sum and what follows
// it fused), or, with y_add == y, the result added to what y holds.  SH: with
// a shared expert (a kernel of its own, so the mixture without one runs the
// plain code).
template <int ACT, int LPR, int C, bool SH>
__global__ void __launch_bounds__(DN_MAX_WAVES * WAVE) k_down(const float *__restrict__ h, const int8_t *__restrict__ hq,
                                                              const float *__restrict__ hs, const int8_t *__restrict__ Wdq,
                                                              const float *__restrict__ Wds, SharedW sw,
                                                              const int32_t *__restrict__ idx,
                                                              const float *__restrict__ wts, int d, int dff, int E, int k,
                                                              int ks, int kss, const float *y_add, float *y,
                                                              const int8_t *__restrict__ hl)
{
    constexpr int G = WAVE / LPR;
    constexpr int U = dn_unroll<ACT, LPR, C>();
    constexpr int OPS = G * U < DN_TILE ? G * U : DN_TILE;
    constexpr int STEPS = DN_TILE / OPS;
    static_assert(DN_TILE % OPS == 0 && OPS % G == 0, "steps tile the outputs");
    constexpr int UU = OPS / G;
    __shared__ float part[DN_MAX_PAIRS][DN_TILE];

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, lig = lane % LPR, grp = lane / LPR;
    const int nwaves = blockDim.x >> 6;
    const int o0 = blockIdx.x * DN_TILE;
    const int64_t row = blockIdx.y;
    const int64_t hw = (int64_t)k * dff + (SH ? sw.sdff : 0);
    const int rp = k * ks, pairs = rp + (SH ? kss : 0);

    for (int p = wid; p < pairs; p += nwaves) {
        const bool sh = SH && p >= rp;
        const int j = sh ? k : p / ks, s = sh ? p - rp : p % ks;
        const int e = sh ? 0 : idx[row * k + j];
        const bool valid = sh || (e >= 0 && e < E);
        const int n_in = sh ? sw.sdff : dff;
        const int nch = n_in >> 4, nb = n_in >> 5;
        const int8_t *wq = sh ? sw.dq : Wdq;
        const float *ws = sh ? sw.ds : Wds;
        const int ch0 = s * LPR * C;
        const int sl = min(LPR * C, nch - ch0);
        const int64_t hrow = row * hw + (int64_t)j * dff;
        const int64_t rbase = (int64_t)(valid && !sh ? e : 0) * d + o0;
        // Each step's weight rows are requested before the previous step is
        // reduced.  The loads are straight-line code (an invalid choice reads
        // expert 0's rows and is zeroed at the dot; chunks past the slice meet
        // zero activations), so the wait before a step's dots counts only
        // the next step's loads: with a branch in between the wait would
        // cover every load issued, the next step's included.
        auto load_step = [&](RowSlice<C>(&w)[UU], int st) {
#pragma unroll
            for (int u = 0; u < UU; u++) {
                const int64_t o = rbase + st * OPS + u * G + grp;
                load_row_flat<LPR, C>(w[u], wq + o * n_in, ws + o * nb, ch0, sl, lig);
            }
        };
        // The hidden row's chunks are requested first (they come from cache),
        // then the weight rows of step 0.
        XSlice<ACT, C> xv;
        if constexpr (ACT == 2)
            load_x2<LPR, C>(xv, hq + hrow, hl + hrow, hs + hrow / QB, ch0, sl, lig);
        else
            load_x<LPR, C>(xv, ACT == 0 ? h + hrow : nullptr, ACT == 1 ? hq + hrow : nullptr,
                           ACT == 1 ? hs + hrow / QB : nullptr, ch0, sl, lig);
        RowSlice<C> wa[UU], wb[UU];
        load_step(wa, 0);
#pragma unroll
        for (int st = 0; st < STEPS; st++) {
            if (st + 1 < STEPS)
                load_step((st & 1) ? wa : wb, st + 1);
            RowSlice<C>(&w)[UU] = (st & 1) ? wb : wa;
#pragma unroll
            for (int u = 0; u < UU; u++) {
                float a = valid ? row_dot(w[u], xv, lig) : 0.0f;
                a = group_sum<LPR>(a);
                if (lig == 0)
                    part[p][st * OPS + u * G + grp] = a;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < DN_TILE) {
        const int t = threadIdx.x;
        float acc = 0.0f;
        for (int j = 0; j < k; j++) {
            float dj = 0.0f;
            for (int s = 0; s < ks; s++)
                dj += part[j * ks + s][t];
            acc = __builtin_fmaf(wts[row * k + j], dj, acc);
        }
        if (SH && kss > 0) {
            float ds = 0.0f;
            for (int s = 0; s < kss; s++)
                ds += part[rp + s][t];
            acc += ds;
        }
        // a branch, not a select: the load happens only when asked for
        if (y_add)
            acc = y_add[row * d + o0 + t] + acc;
        y[row * d + o0 + t] = acc;
    }
}

// ---------------------------------------------------------------------------
// host dispatch

namespace {

SharedW shared_w(const MoeArgs &a)
{
    return SharedW{a.Sgq, a.Sgs, a.Suq, a.Sus, a.Sdq, a.Sds, (int)a.sdff};
}

template <int ACT, int LPR, int C, int V>
hipError_t gu_go(const MoeArgs &a, int ks, hipStream_t st)
{
    using S = GuShape<ACT, LPR, C, V>;
    dim3 grid((unsigned)((a.k * a.dff + a.sdff) / S::T), (unsigned)a.rows);
    if (a.sdff)
        hipLaunchKernelGGL((k_gate_up<ACT, LPR, C, true, V>), grid, dim3(S::NW * WAVE), 0, st, a.x, a.xq, a.xs, a.Wgq,
                           a.Wgs, a.Wuq, a.Wus, shared_w(a), a.idx, (int)a.d, (int)a.dff, (int)a.E, (int)a.k, ks, a.h,
                           a.hq, a.hs, a.xl, a.hl);
    else
        hipLaunchKernelGGL((k_gate_up<ACT, LPR, C, false, V>), grid, dim3(S::NW * WAVE), 0, st, a.x, a.xq, a.xs, a.Wgq,
                           a.Wgs, a.Wuq, a.Wus, shared_w(a), a.idx, (int)a.d, (int)a.dff, (int)a.E, (int)a.k, ks, a.h,
                           a.hq, a.hs, a.xl, a.hl);
    return hipGetLastError();
}

template <int ACT, int LPR, int C, int V>
hipError_t rgu_go(const MoeArgs &a, int ks, hipStream_t st)
{
    using S = GuShape<ACT, LPR, C, V>;
    static_assert(S::NW * WAVE >= ROUTE_FUSED_MAX_E, "one thread per logit at least");
    dim3 grid((unsigned)((a.k * a.dff + a.sdff) / S::T), (unsigned)a.rows);
    if (a.sdff)
        hipLaunchKernelGGL((k_route_gate_up<ACT, LPR, C, true, V>), grid, dim3(S::NW * WAVE), 0, st, a.logits, a.idx_w,
                           a.wts_w, a.x, a.xq, a.xs, a.Wgq, a.Wgs, a.Wuq, a.Wus, shared_w(a), (int)a.d, (int)a.dff,
                           (int)a.E, (int)a.k, ks, a.h, a.hq, a.hs, a.xl, a.hl);
    else
        hipLaunchKernelGGL((k_route_gate_up<ACT, LPR, C, false, V>), grid, dim3(S::NW * WAVE), 0, st, a.logits, a.idx_w,
                           a.wts_w, a.x, a.xq, a.xs, a.Wgq, a.Wgs, a.Wuq, a.Wus, shared_w(a), (int)a.d, (int)a.dff,
                           (int)a.E, (int)a.k, ks, a.h, a.hq, a.hs, a.xl, a.hl);
    return hipGetLastError();
}

// the shared expert's slices in a lane shape of LPR x C chunks
int shared_slices(int64_t sdff, int lpr, int c) { return (int)((sdff / 16 + lpr * c - 1) / (lpr * c)); }

template <int ACT, int LPR, int C>
hipError_t dn_go(const MoeArgs &a, int ks, hipStream_t st)
{
    const int kss = a.sdff ? shared_slices(a.sdff, LPR, C) : 0;
    const int pairs = (int)a.k * ks + kss;
    const int nw = std::min(DN_MAX_WAVES, pairs);
    dim3 grid((unsigned)(a.d / DN_TILE), (unsigned)a.rows);
    if (a.sdff)
        hipLaunchKernelGGL((k_down<ACT, LPR, C, true>), grid, dim3(64 * nw), 0, st, a.h, a.hq, a.hs, a.Wdq, a.Wds,
                           shared_w(a), a.idx, a.wts, (int)a.d, (int)a.dff, (int)a.E, (int)a.k, ks, kss,
                           a.acc_out ? a.y : a.resid, a.y, a.hl);
    else
        hipLaunchKernelGGL((k_down<ACT, LPR, C, false>), grid, dim3(64 * nw), 0, st, a.h, a.hq, a.hs, a.Wdq, a.Wds,
                           shared_w(a), a.idx, a.wts, (int)a.d, (int)a.dff, (int)a.E, (int)a.k, ks, kss,
                           a.acc_out ? a.y : a.resid, a.y, a.hl);
    return hipGetLastError();
}

template <int ACT, template <int, int, int> class F>
hipError_t by_shape(const MoeArgs &a, int64_t n_in, hipStream_t st)
{
    const SliceShape sh = slice_shape(n_in);
    if (sh.ks > 1)
        return F<ACT, 64, 4>::go(a, sh.ks, st);
    switch (sh.lpr * 8 + sh.c) {
    case 16 * 8 + 1:
        return F<ACT, 16, 1>::go(a, 1, st);
    case 16 * 8 + 3:
        return F<ACT, 16, 3>::go(a, 1, st);
    case 64 * 8 + 1:
        return F<ACT, 64, 1>::go(a, 1, st);
    case 64 * 8 + 2:
        return F<ACT, 64, 2>::go(a, 1, st);
    default:
        return F<ACT, 64, 4>::go(a, 1, st);
    }
}

// Whether an int8 gate-up with lane groups of 64 holding two chunks takes
// the 8-wave shape (V = 1): when its tiles outnumber the chip's CUs (256 on
// MI355X).  With one chunk a lane (the 8-expert block, 896 tiles) 8 waves of
// 4 pairs measured slower (45.5 vs 43.7 us), so V = 0 stays there.
inline bool gu_wide(const MoeArgs &a) { return a.rows * ((a.k * a.dff + a.sdff) / QB) > device_cus(); }
template <int ACT, int LPR, int C>
struct GU {
    static hipError_t go(const MoeArgs &a, int ks, hipStream_t st)
    {
        if constexpr (ACT >= 1 && LPR == 64 && C == 2)
            if (gu_wide(a))
                return gu_go<ACT, LPR, C, 1>(a, ks, st);
        return gu_go<ACT, LPR, C, 0>(a, ks, st);
    }
};
template <int ACT, int LPR, int C>
struct RGU {
    static hipError_t go(const MoeArgs &a, int ks, hipStream_t st)
    {
        if constexpr (ACT >= 1 && LPR == 64 && C == 2)
            if (gu_wide(a))
                return rgu_go<ACT, LPR, C, 1>(a, ks, st);
        return rgu_go<ACT, LPR, C, 0>(a, ks, st);
    }
};
template <int ACT, int LPR, int C>
struct DN {
    static hipError_t go(const MoeArgs &a, int ks, hipStream_t st) { return dn_go<ACT, LPR, C>(a, ks, st); }
};

} // namespace

namespace {

// The decode gate-up's int8 shapes (one or two words) for d, then the launch F.
template <int ACT, template <int, int, int> class F>
hipError_t gu_int8(const MoeArgs &a, hipStream_t st)
{
    // int8 rows past 2048: slices of 1024 values (lane groups of 64, one chunk
    // each; measured fastest at d 4096), or of 2048 past 32 slices
    const int64_t nch = a.d / 16;
    if (nch > 128 && nch <= 64 * GU_MAX_KS)
        return F<ACT, 64, 1>::go(a, (int)((nch + 63) / 64), st);
    if (nch > 128)
        return F<ACT, 64, 2>::go(a, (int)((nch + 127) / 128), st);
    const SliceShape sh = slice_shape(a.d);
    switch (sh.lpr * 8 + sh.c) {
    case 16 * 8 + 1:
        return F<ACT, 16, 1>::go(a, 1, st);
    case 16 * 8 + 3:
        return F<ACT, 16, 3>::go(a, 1, st);
    case 64 * 8 + 1:
        return F<ACT, 64, 1>::go(a, 1, st);
    default:
        return F<ACT, 64, 2>::go(a, 1, st);
    }
}

// The decode gate-up's shape for the mode and d, then the launch F.
template <template <int, int, int> class F>
hipError_t gu_dispatch(const MoeArgs &a, hipStream_t st)
{
    if (a.act == 0)
        return by_shape<0, F>(a, a.d, st);
    return a.act == 2 ? gu_int8<2, F>(a, st) : gu_int8<1, F>(a, st);
}

// The down-combine for the mode, over hidden rows of n_in values.
hipError_t dn_dispatch(const MoeArgs &a, int64_t n_in, hipStream_t st)
{
    if (a.act == 2)
        return by_shape<2, DN>(a, n_in, st);
    return a.act == 0 ? by_shape<0, DN>(a, n_in, st) : by_shape<1, DN>(a, n_in, st);
}

} // namespace

hipError_t gate_up_launch(const MoeArgs &a, hipStream_t st)
{
    if (a.act >= 1 && a.rows > 1 && chunk_supported(a.d, a.dff))
        return chunk_gate_up_launch(a, st);
    return gu_dispatch<GU>(a, st);
}

hipError_t route_gate_up_launch(const MoeArgs &a, hipStream_t st) { return gu_dispatch<RGU>(a, st); }

size_t down_scratch_bytes(int64_t rows, int64_t d, int64_t dff, int64_t k, int act)
{
    return (act >= 1 && rows > 1 && chunk_supported(d, dff)) ? chunk_down_scratch_bytes(rows, d, k) : 0;
}

hipError_t down_launch(const MoeArgs &a, hipStream_t st)
{
    if (a.act >= 1 && a.rows > 1 && chunk_supported(a.d, a.dff))
        return chunk_down_launch(a, st);
    return dn_dispatch(a, a.dff, st);
}

hipError_t row_down_launch(const MoeArgs &a, hipStream_t st) { return dn_dispatch(a, a.dff, st); }

int64_t down_pairs(int64_t dff, int64_t sdff, int64_t k)
{
    const SliceShape sh = slice_shape(dff);
    const int lpr = sh.ks > 1 ? 64 : sh.lpr, c = sh.ks > 1 ? 4 : sh.c;
    return k * sh.ks + (sdff ? shared_slices(sdff, lpr, c) : 0);
}

bool shared_fits(int64_t dff, int64_t sdff, int64_t k)
{
    return down_pairs(dff, sdff, k) <= DN_MAX_PAIRS && down_pairs(sdff, sdff, 0) <= DN_MAX_PAIRS;
}

hipError_t shared_launch(const MoeArgs &a, hipStream_t st)
{
    MoeArgs s = a;
    s.k = 0;
    s.acc_out = true;
    hipError_t err = gu_dispatch<GU>(s, st);
    if (err != hipSuccess)
        return err;
    return dn_dispatch(s, s.sdff, st);
}

} // namespace q8s
