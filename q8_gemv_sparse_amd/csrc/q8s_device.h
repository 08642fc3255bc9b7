// q8s_device.h -- device-side building blocks of the Q8_0 GEMV / MoE kernels
// for gfx950 (CDNA4, wave64).
//
// The weight stream is the whole cost of a batch-1 Q8_0 projection: its
// bytes, not its arithmetic, bound it (codegen_cuda::qwen_emit module page,
// enum Q8MatKind).  The pieces here are shaped for that:
//   * a row of quants is read as 16-byte chunks, chunk c of a row by lane
//     (c mod LPR) of an LPR-lane group, so each load instruction of a wave
//     covers LPR*16 contiguous bytes of every row it touches;
//   * the activation slice a lane multiplies against stays in registers for
//     every row the wave streams, so activations are read once per wave;
//   * partial sums are reduced across the lane group with DPP row operations,
//     no LDS round trip.
// A Q8_0 block (32 values, struct Q8Ref) is two chunks, held by lanes 2i and
// 2i+1 of a group; in int8 mode their exact int32 half-block sums are added
// across that lane pair before the block's two scales are applied.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8s {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QB = 32;  // values per Q8_0 block
constexpr int WAVE = 64;

#define Q8S_DEV __device__ __forceinline__

// ---------------------------------------------------------------------------
// loads

// A streamed (non-temporal) 16-byte load: weight rows are read once.
Q8S_DEV i32x4 ld_stream16(const int8_t *p) { return __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(p)); }
Q8S_DEV float ld_stream_f32(const float *p) { return __builtin_nontemporal_load(p); }
Q8S_DEV i32x4 ld16(const void *p) { return *reinterpret_cast<const i32x4 *>(p); }
Q8S_DEV f32x4 ldf4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// A raw buffer resource over n bytes from a wave-uniform base (held in
// scalar registers): its loads take a 32-bit byte offset a lane, so they keep
// no 64-bit address in vector registers; a load at or past n bytes returns
// zero.
typedef __amdgpu_buffer_rsrc_t BufRes;
Q8S_DEV BufRes buf_res(const void *p, uint32_t n)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n, 0x00020000);
}

// ---------------------------------------------------------------------------
// cross-lane reductions

// DPP controls (gfx9 encoding).
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within each 8
constexpr int DPP_MIRROR = 0x140;      // lane i <- lane 15-i within each 16

// (every control here is a whole permutation; a lane whose source is
// inactive reads 0, and no register needs clearing before the move)
template <int CTRL>
Q8S_DEV float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
Q8S_DEV int dpp_i(int v)
{
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Sum over each 16-lane row; every lane of the row receives the row's sum.
Q8S_DEV float sum16(float v)
{
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    return v;
}

// Sum over each group of LPR consecutive lanes (LPR = 16, 32 or 64); every
// lane of a group receives its group's sum.
template <int LPR>
Q8S_DEV float group_sum(float v)
{
    static_assert(LPR == 16 || LPR == 32 || LPR == 64, "lane group of 16, 32 or 64");
    v = sum16(v);
    if constexpr (LPR >= 32)
        v += __shfl_xor(v, 16);
    if constexpr (LPR >= 64)
        v += __shfl_xor(v, 32);
    return v;
}

Q8S_DEV float wave_max(float v)
{
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <int CTRL>
Q8S_DEV double dpp_d(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(b >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

Q8S_DEV double readlane_d(double v, int lane)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the whole wave (every lane active), the same value in every lane:
// DPP sums within each 16-lane row, then the four row sums in order.  No LDS
// traffic: the cross-lane permute of __shfl_xor goes through LDS and six
// dependent steps of it cost a few hundred cycles.
Q8S_DEV double wave_sum_f64(double v)
{
    v += dpp_d<DPP_XOR1>(v);
    v += dpp_d<DPP_XOR2>(v);
    v += dpp_d<DPP_HALF_MIRROR>(v);
    v += dpp_d<DPP_MIRROR>(v);
    return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

// ---------------------------------------------------------------------------
// the Q8_0 activation quantiser, float32 throughout:
//   d = amax/127; id = d ? 1/d : 0; q = clamp(round-half-away(v*id), +-127)
// The divisions are IEEE float32 divisions (the library is built with
// correctly rounded float32 division); roundf rounds halfway cases away
// from zero.

Q8S_DEV float q8_scale(float amax) { return amax / 127.0f; }
Q8S_DEV float q8_inv(float d) { return d != 0.0f ? 1.0f / d : 0.0f; }
Q8S_DEV int q8_code(float v, float id)
{
    float p = v * id;
    float r = roundf(p);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// The two-word activation's low word: the rest of v*id after the word q, in
// 128ths of a step, rounded half away from zero (v ~= d * (q + lo/128)).
// p - q is exact and 128 a power of two, so lo is the nearest 128th of the
// rest; |p - q| <= 1/2 keeps |lo| <= 64 (the clamp never binds).
Q8S_DEV int q8_low(float v, float id, int q)
{
    float p = v * id;
    float r = roundf((p - (float)q) * 128.0f);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Quantise 8 consecutive values held by one thread of a 4-thread group that
// owns one 32-value block (the group's lanes are neighbours within a quad):
// the 8 codes packed in two words, and the block scale.
Q8S_DEV uint2 quant8(const float (&v)[8], float &scale)
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp_f<DPP_XOR1>(amax));
    amax = fmaxf(amax, dpp_f<DPP_XOR2>(amax));
    const float d = q8_scale(amax);
    const float id = q8_inv(d);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo |= (uint32_t)(q8_code(v[i], id) & 0xFF) << (8 * i);
        hi |= (uint32_t)(q8_code(v[4 + i], id) & 0xFF) << (8 * i);
    }
    scale = d;
    return make_uint2(lo, hi);
}

// quant8, then the 8 codes written and, from the group's first thread, the
// block scale.
Q8S_DEV void quant8_store(const float (&v)[8], int8_t *q, float *scale, bool leader)
{
    float d;
    *reinterpret_cast<uint2 *>(q) = quant8(v, d);
    if (leader)
        *scale = d;
}

// The 8 low words of v whose words are w (quant8's packing) and scale d.
Q8S_DEV uint2 low8(const float (&v)[8], uint2 w, float d)
{
    const float id = q8_inv(d);
    uint32_t l0 = 0, l1 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int q0 = (int)(int8_t)((w.x >> (8 * i)) & 0xFF), q1 = (int)(int8_t)((w.y >> (8 * i)) & 0xFF);
        l0 |= (uint32_t)(q8_low(v[i], id, q0) & 0xFF) << (8 * i);
        l1 |= (uint32_t)(q8_low(v[4 + i], id, q1) & 0xFF) << (8 * i);
    }
    return make_uint2(l0, l1);
}

// quant8 in two words: the same words and scale, plus the 8 low words.
Q8S_DEV void quant8x2_store(const float (&v)[8], int8_t *q, int8_t *lo, float *scale, bool leader)
{
    float d;
    const uint2 w = quant8(v, d);
    *reinterpret_cast<uint2 *>(q) = w;
    *reinterpret_cast<uint2 *>(lo) = low8(v, w, d);
    if (leader)
        *scale = d;
}

// ---------------------------------------------------------------------------
// a lane's share of one row: C chunks of 16 bytes plus their block scales

template <int C>
struct RowSlice {
    i32x4 q[C];
    float s[C];
};

// The activation slice a lane multiplies against: float32 values, or Q8_0
// words + block scales.
template <int ACT, int C>
struct XSlice;
template <int C>
struct XSlice<0, C> {
    f32x4 v[C][4];
};
template <int C>
struct XSlice<1, C> {
    i32x4 q[C];
    float s[C];
};
// two-word int8: the words, the low words, one scale a block
template <int C>
struct XSlice<2, C> {
    i32x4 q[C];
    i32x4 l[C];
    float s[C];
};

// Chunk index (within the row) of a lane's c-th chunk: ch0 + c*LPR + lig.
// Chunks at or past `nch` (the slice's end) are masked to zero.
template <int LPR, int C>
Q8S_DEV void load_row(RowSlice<C> &w, const int8_t *__restrict__ rowq, const float *__restrict__ rows, int ch0, int nch,
                      int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        int ch = c * LPR + lig;
        if (ch < nch) {
            w.q[c] = ld_stream16(rowq + (int64_t)(ch0 + ch) * 16);
            w.s[c] = ld_stream_f32(rows + ((ch0 + ch) >> 1));
        } else {
            w.q[c] = i32x4{0, 0, 0, 0};
            w.s[c] = 0.0f;
        }
    }
}

// load_row without branches, for straight-line load sequences (the
// vector-memory wait before a use can then count exactly the loads issued
// after it): chunks past the slice read the slice's last chunk instead of
// zeros.  Only for use against an activation slice whose chunks past the
// slice are zero (load_x zeroes them), which makes those products vanish.
template <int LPR, int C>
Q8S_DEV void load_row_flat(RowSlice<C> &w, const int8_t *__restrict__ rowq, const float *__restrict__ rows, int ch0,
                           int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        const int ch = min(c * LPR + lig, nch - 1);
        w.q[c] = ld_stream16(rowq + (int64_t)(ch0 + ch) * 16);
        w.s[c] = ld_stream_f32(rows + ((ch0 + ch) >> 1));
    }
}

template <int LPR, int C>
Q8S_DEV void load_x(XSlice<0, C> &x, const float *__restrict__ xr, const int8_t *, const float *, int ch0, int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        int ch = c * LPR + lig;
        if (ch < nch) {
            const float *p = xr + (int64_t)(ch0 + ch) * 16;
#pragma unroll
            for (int i = 0; i < 4; i++)
                x.v[c][i] = ldf4(p + 4 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                x.v[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

template <int LPR, int C>
Q8S_DEV void load_x(XSlice<1, C> &x, const float *, const int8_t *__restrict__ xq, const float *__restrict__ xs, int ch0,
                    int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        int ch = c * LPR + lig;
        if (ch < nch) {
            x.q[c] = ld16(xq + (int64_t)(ch0 + ch) * 16);
            x.s[c] = xs[(ch0 + ch) >> 1];
        } else {
            x.q[c] = i32x4{0, 0, 0, 0};
            x.s[c] = 0.0f;
        }
    }
}

template <int LPR, int C>
Q8S_DEV void load_x2(XSlice<2, C> &x, const int8_t *__restrict__ xq, const int8_t *__restrict__ xl,
                     const float *__restrict__ xs, int ch0, int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        int ch = c * LPR + lig;
        if (ch < nch) {
            x.q[c] = ld16(xq + (int64_t)(ch0 + ch) * 16);
            x.l[c] = ld16(xl + (int64_t)(ch0 + ch) * 16);
            x.s[c] = xs[(ch0 + ch) >> 1];
        } else {
            x.q[c] = i32x4{0, 0, 0, 0};
            x.l[c] = i32x4{0, 0, 0, 0};
            x.s[c] = 0.0f;
        }
    }
}

// load_x for Q8_0 activations without branches: chunks past the slice read
// its last chunk and are zeroed by a select.
template <int LPR, int C>
Q8S_DEV void load_x_flat(XSlice<1, C> &x, const int8_t *__restrict__ xq, const float *__restrict__ xs, int ch0,
                         int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        const int ch = c * LPR + lig;
        const int cc = min(ch, nch - 1);
        const i32x4 q = ld16(xq + (int64_t)(ch0 + cc) * 16);
        const float sc = xs[(ch0 + cc) >> 1];
        x.q[c] = ch < nch ? q : i32x4{0, 0, 0, 0};
        x.s[c] = ch < nch ? sc : 0.0f;
    }
}

// Quantising an f32 activation slice on the spot, in two halves so the loads
// can be issued before other traffic (waits on the vector-memory counter are
// in issue order: a load issued after the weight rows could only be used once
// all of them had landed).
// Block b is chunks 2b, 2b+1, held by lanes 2i, 2i+1 of the group, so the
// block's absolute maximum is the pair's, one DPP step.  The scale and codes
// follow the float32 quantiser above, step for step, so they equal what
// q8_quantize_rows writes for the same values.
template <int C>
struct XRaw {
    f32x4 v[C][4];
};

template <int LPR, int C>
Q8S_DEV void load_x_raw(XRaw<C> &r, const float *__restrict__ xr, int ch0, int nch, int lig)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        const int ch = c * LPR + lig;
        if (ch < nch) {
            const float *p = xr + (int64_t)(ch0 + ch) * 16;
#pragma unroll
            for (int i = 0; i < 4; i++)
                r.v[c][i] = ldf4(p + 4 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                r.v[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

template <int C>
Q8S_DEV void quantize_slice(XSlice<1, C> &x, const XRaw<C> &r)
{
#pragma unroll
    for (int c = 0; c < C; c++) {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int b = 0; b < 4; b++)
                amax = fmaxf(amax, fabsf(r.v[c][i][b]));
        amax = fmaxf(amax, dpp_f<DPP_XOR1>(amax));
        const float d = q8_scale(amax);
        const float id = q8_inv(d);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t dw = 0;
#pragma unroll
            for (int b = 0; b < 4; b++)
                dw |= (uint32_t)(q8_code(r.v[c][i][b], id) & 0xFF) << (8 * b);
            x.q[c][i] = (int)dw;
        }
        x.s[c] = d;
    }
}

template <int C>
Q8S_DEV void raw_to_slice(XSlice<0, C> &x, const XRaw<C> &r)
{
#pragma unroll
    for (int c = 0; c < C; c++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            x.v[c][i] = r.v[c][i];
}

// sum_i q_i * x_i over one 16-byte chunk, float32 (each int8 converted
// exactly; the multiply-adds accumulate in float32).
Q8S_DEV float chunk_dot_f32(i32x4 q, const f32x4 (&x)[4])
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int dw = q[i];
#pragma unroll
        for (int b = 0; b < 4; b++)
            acc = __builtin_fmaf((float)(signed char)(dw >> (8 * b)), x[i][b], acc);
    }
    return acc;
}

// Exact int32 dot of two 16-byte int8 chunks (v_dot4_i32_i8).
Q8S_DEV int chunk_dot_i8(i32x4 a, i32x4 b)
{
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
        s = __builtin_amdgcn_sdot4(a[i], b[i], s, false);
    return s;
}

// The lane's partial of one row's dot with the activation slice.
//   f32 : sum_c s_c * sum_i q_i x_i
//   int8: sum over the lane's blocks of (ws*xs) * isum_block, where the
//         block's exact isum joins the half-block sums of lanes 2i, 2i+1; the
//         odd lane of the pair contributes nothing.
template <int C>
Q8S_DEV float row_dot(const RowSlice<C> &w, const XSlice<0, C> &x, int)
{
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < C; c++)
        acc = __builtin_fmaf(chunk_dot_f32(w.q[c], x.v[c]), w.s[c], acc);
    return acc;
}

template <int C>
Q8S_DEV float row_dot(const RowSlice<C> &w, const XSlice<1, C> &x, int lig)
{
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < C; c++) {
        int half = chunk_dot_i8(w.q[c], x.q[c]);
        int blk = half + dpp_i<DPP_XOR1>(half);
        float f = (float)blk * (w.s[c] * x.s[c]);
        acc += (lig & 1) ? 0.0f : f;
    }
    return acc;
}

// two words: the block's two exact dots joined as one int32,
// 128*isum_hi + isum_lo (|.| < 2^27), scaled by ws*xs/128
template <int C>
Q8S_DEV float row_dot(const RowSlice<C> &w, const XSlice<2, C> &x, int lig)
{
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < C; c++) {
        const int half = chunk_dot_i8(w.q[c], x.q[c]) * 128 + chunk_dot_i8(w.q[c], x.l[c]);
        const int blk = half + dpp_i<DPP_XOR1>(half);
        const float f = (float)blk * ((w.s[c] * x.s[c]) * 0.0078125f);
        acc += (lig & 1) ? 0.0f : f;
    }
    return acc;
}

// ---------------------------------------------------------------------------
// the MoE block's pieces shared by its decode and chunk kernels

// SiLU(z) = z / (1 + e^-z) with the hardware's exp2 and reciprocal (each
// within a couple of ulps: a few 1e-7 relative, far inside the float32
// tolerance; the library's correctly rounded division and exp cost ~40
// instructions, which the chunk gate-up, bound by its vector work, pays per
// hidden value).  Large |z| behaves: e^-z -> inf gives 0, e^-z -> 0 gives z.
Q8S_DEV float silu(float z)
{
    const float t = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    return z * __builtin_amdgcn_rcpf(1.0f + t);
}

// Decode gate-up launch shape per mode and row cut.  At these sizes the kernels are
// bound by memory latency more than by bandwidth: many waves with one or two
// rows' loads in flight each beat fewer waves with more (measured).
//   f32 : 8 waves, one gate/up pair per lane group (two for rows of one
//         chunk a lane, and for rows of four: 90.7 vs 93.8 us for the
//         8-expert block at d 4096, where tiles of 8 outputs made 3584
//         workgroups each paying the top-K; two pairs at d 2048 measured
//         20.4 vs 19.6 us, sixteen waves slower everywhere); tiles of 8 (or
//         16, 32) hidden outputs.
//   int8: a tile is one 32-value block, so the workgroup also writes the
//         block's Q8_0 form (the down projection's activation) once, in its
//         epilogue: 16 waves of 2 pairs (8 of 1 for lane groups of 16); rows
//         longer than 2048 are cut into 2048-value slices (gu_slices), which
//         keeps each wave at 8 loads in flight.
//   V = 1 (int8, lane groups of 64): the same 32-output tile in 8 waves of 4
//         pairs, for launches of more tiles than the chip has CUs, where
//         smaller workgroups share the CUs more evenly (the shared-expert
//         block's 352 tiles: 23.4 vs 24.6 us a step; the 128-expert block's
//         192 tiles: 18.7 vs 18.1 us, so V = 0 there).
template <int ACT, int LPR, int C, int V = 0>
struct GuShape {
    static_assert(V == 0 || (ACT >= 1 && LPR == 64), "the 8-wave int8 shape is for lane groups of 64");
    static constexpr int G = WAVE / LPR;
    static constexpr int NW = ACT >= 1 ? (LPR == 64 ? (V ? 8 : 16) : 8) : 8;
    static constexpr int U = ACT >= 1 ? (LPR == 64 ? (V ? 4 : 2) : 1) : ((LPR == 64 && (C == 1 || C == 4)) ? 2 : 1);
    static constexpr int OPS = G * U;
    static constexpr int T = NW * OPS;
    static_assert(QB % T == 0, "a tile divides a 32-value block, so it divides dff");
    static_assert(ACT == 0 || T == QB, "int8 tiles are whole blocks");
};

// ---------------------------------------------------------------------------
// top-K of one row's router logits, held in LDS (fn emit_moe_forward: the K
// largest by probability, which is monotone in the logit)


// LDS of the in-workgroup top-K, for rows of at most TOPK_LDS_E logits.
constexpr int TOPK_LDS_E = 256;
struct alignas(16) TopkLds {
    double L[TOPK_LDS_E];         // the row's logits
    uint32_t ck[TOPK_LDS_E + 4];  // codes' upper halves (coarse keys), padded with zeros to whole quads
    uint32_t lo[TOPK_LDS_E];      // codes' lower halves
    int ch[32];                   // the choices, in rank order
    double kl[32];                // their logits
};

// An order-preserving 64-bit code of a logit: its unsigned order is the order
// of the values (-0 taken as +0, so equal values get equal codes).  NaNs get
// codes too (above +inf or below -inf by their sign), so ranking by code is a
// strict total order with the index as tie-break and every rank is taken
// exactly once, whatever the logits hold.
Q8S_DEV uint64_t route_code(double v)
{
    // a select, not v + 0.0, so a NaN keeps its sign bit
    const uint64_t b = (uint64_t)__double_as_longlong(v == 0.0 ? 0.0 : v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// The code's upper half: a strictly greater key means a strictly greater
// logit; equal keys decide nothing.  Finite logits never get key 0.
Q8S_DEV uint32_t coarse_key(double v) { return (uint32_t)(route_code(v) >> 32); }

// Sum over each group of S consecutive lanes, S in {1, 2, 4, 8}, S uniform
// across the wave; every lane of a group receives its group's sum.
Q8S_DEV int sum_lanes8(int v, int S)
{
    if (S >= 2)
        v += dpp_i<DPP_XOR1>(v);
    if (S >= 4)
        v += dpp_i<DPP_XOR2>(v);
    if (S >= 8)
        v += dpp_i<DPP_HALF_MIRROR>(v);
    return v;
}

// Threads per item when `items` items share the workgroup: a power of two up
// to 8 with S * items <= blockDim.x.
Q8S_DEV int lanes_per_item(int items)
{
    int S = 1;
    while (S < 8 && S * 2 * items <= (int)blockDim.x)
        S *= 2;
    return S;
}

// Loads a row's E logits (E <= TOPK_LDS_E) and their codes; every thread
// calls it, and the caller synchronises before topk_select.
Q8S_DEV void topk_load(TopkLds &t, const double *__restrict__ lr, int E)
{
    for (int i = threadIdx.x; i < ((E + 3) & ~3); i += blockDim.x) {
        if (i < E) {
            const double v = lr[i];
            const uint64_t c = route_code(v);
            t.L[i] = v;
            t.ck[i] = (uint32_t)(c >> 32);
            t.lo[i] = (uint32_t)c;
        } else {
            t.ck[i] = 0u;
        }
    }
}

// The K best of the row's E <= blockDim.x logits by (logit descending, index
// ascending), in rank order, into t.ch / t.kl.  Every thread calls it; the
// caller synchronises before reading the choices.  Logit i's rank is the
// number of logits ranked before it, counted by S threads sharing the E keys
// in interleaved quads:
//   rank_i = #{w : key_w > key_i}
//          + #{w != i : key_w == key_i, and (lo_w > lo_i, or lo_w == lo_i and w < i)},
// which for non-NaN logits is #{w : l_w > l_i, or l_w == l_i and w < i}: the
// code is order-preserving, so a greater key is a greater logit and, on equal
// keys, the lower halves decide.  The second term is taken only for a logit
// whose key some other logit shares (the threads count equal keys alongside
// greater ones), which near-equal logits make rare.  The ranks are a
// permutation of 0..E-1, so each of the K slots gets exactly one writer.
// Ranking all E in one pass with no candidate list keeps it to one LDS pass
// between two barriers; an exact compare of all E^2 pairs in double measured
// several microseconds on a full workgroup.
// topk_load's LDS writes for one logit a thread, already in a register:
// thread t holds logit t (the workgroup has at least E threads).
Q8S_DEV void topk_put(TopkLds &t, double v, int E)
{
    const int i = threadIdx.x;
    if (i < E) {
        const uint64_t c = route_code(v);
        t.L[i] = v;
        t.ck[i] = (uint32_t)(c >> 32);
        t.lo[i] = (uint32_t)c;
    } else if (i < ((E + 3) & ~3)) {
        t.ck[i] = 0u;
    }
}

// The top-K of `rows` rows of E logits (E <= TOPK_LDS_E), ridden on another
// launch's workgroups; idx/wts as k_topk writes them.
struct TopkRider {
    const double *logits;
    int rows, E, k;
    int32_t *idx;
    float *wts;
};

// A row's kept choices and logits in rank order, for route_finish.
struct TopkKept {
    double kl[32];
    int ch[32];
};

Q8S_DEV void topk_select(TopkLds &t, int E, int k)
{
    const int S = lanes_per_item(E);
    const int i = threadIdx.x / S, part = threadIdx.x % S;
    int gt = 0, ge = 0;
    uint32_t ci = 0u;
    if (i < E) {
        ci = t.ck[i];
        const uint4 *q = reinterpret_cast<const uint4 *>(t.ck);
        const int nq = (E + 3) >> 2;
        for (int q0 = part; q0 < nq; q0 += 4 * S) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++)
                v[u] = q0 + u * S < nq ? q[q0 + u * S] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                gt += (v[u].x > ci) + (v[u].y > ci) + (v[u].z > ci) + (v[u].w > ci);
                ge += (v[u].x >= ci) + (v[u].y >= ci) + (v[u].z >= ci) + (v[u].w >= ci);
            }
        }
    }
    int r = sum_lanes8(gt, S);
    // ge counts the logit's own key; more than that is a coarse tie (every
    // lane of the item's group sees the same sum, so the group branches as one)
    const int eq = sum_lanes8(ge, S) - r;
    int extra = 0;
    if (i < E && eq > 1) {
        const uint32_t li = t.lo[i];
        for (int w = part; w < E; w += S)
            if (w != i && t.ck[w] == ci) {
                const uint32_t lw = t.lo[w];
                extra += (lw > li || (lw == li && w < i)) ? 1 : 0;
            }
    }
    r += sum_lanes8(extra, S);
    if (i < E && part == 0 && r < k) {
        t.ch[r] = i;
        t.kl[r] = t.L[i];
    }
}

// The kept weights: softmax over all E, then renormalised over the kept K,
//   w_j = p_j / sum_i p_i,  p_e = exp(l_e - m) / sum_all exp(l - m),
// where the all-expert denominator cancels; with m the largest logit (the
// rank-0 choice) this is w_j = exp(l_j - m) / sum_i exp(l_i - m), formed in
// double from the K kept logits only.  Called by one whole wave, lane j
// handling slot j.
Q8S_DEV void route_finish(const double *kl, const int *ch, int k, int32_t *idx_row, float *wts_row)
{
    const int j = threadIdx.x & (WAVE - 1);
    const double p = j < k ? exp(kl[j] - kl[0]) : 0.0;
    const double kept = wave_sum_f64(p);
    if (j < k) {
        idx_row[j] = ch[j];
        wts_row[j] = (float)(p / kept);
    }
}

} // namespace q8s
