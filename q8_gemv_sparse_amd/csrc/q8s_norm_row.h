// q8s_norm_row.h -- one row's residual add + RMSNorm as a 256-thread
// workgroup forms it, shared by every kernel that produces or consumes the
// normed row (forward_shim.rs module doc: the sum and the RMS norm of it as
// one row kernel writing the sum; a weighted norm scales and never shifts).
//
// A thread owns 8 consecutive values of every 2048-value segment, so four
// neighbouring threads own one Q8_0 block.  The mean square is summed in
// double (each thread's squares in order, then the wave sums, then the four
// waves in order) and the normalised value formed in double, then rounded to
// float32 once: every kernel using these helpers forms the same float32 row,
// bit for bit.
#pragma once

#include "q8s_device.h"

namespace q8s {

constexpr int NORM_THREADS = 256;
constexpr int NORM_SEG = NORM_THREADS * 8;

// A thread's share of one row for rows of at most SEGS 2048-value segments:
// its 8 values of each segment (the float32 sums) and their norm weights,
// kept in registers between the two passes.
template <int SEGS>
struct NormShare {
    f32x4 sv[SEGS][2], wv[SEGS][2];
};

// The row's raw h and r go into sv (as h) and a second array (r); norm_add
// forms the float32 sums.  Split so a caller can issue other loads between
// the two (no arithmetic waits on h and r before them).
template <int SEGS>
Q8S_DEV void norm_load_raw(NormShare<SEGS> &n, f32x4 (&rr4)[SEGS][2], const float *hr, const float *rr,
                           const float *w, int d, int t8)
{
    // no branches: a share past the row reads the row's last 8 values, which
    // the callers never use (their passes stop at base >= d)
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        const int base = min(t8 + g * NORM_SEG, d - 8);
        n.sv[g][0] = ldf4(hr + base);
        n.sv[g][1] = ldf4(hr + base + 4);
        rr4[g][0] = ldf4(rr + base);
        rr4[g][1] = ldf4(rr + base + 4);
        n.wv[g][0] = ldf4(w + base);
        n.wv[g][1] = ldf4(w + base + 4);
    }
}

// Unconditional (a share past the row adds values nobody reads): a branch
// here would let the compiler sink the loads of r into it, behind whatever the
// caller issued in between.
template <int SEGS>
Q8S_DEV void norm_add(NormShare<SEGS> &n, const f32x4 (&rr4)[SEGS][2], int, int)
{
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        n.sv[g][0] = n.sv[g][0] + rr4[g][0];
        n.sv[g][1] = n.sv[g][1] + rr4[g][1];
    }
}

template <int SEGS>
Q8S_DEV void norm_load(NormShare<SEGS> &n, const float *hr, const float *rr, const float *w, int d, int t8)
{
    f32x4 rr4[SEGS][2];
    norm_load_raw<SEGS>(n, rr4, hr, rr, w, d, t8);
    norm_add<SEGS>(n, rr4, d, t8);
}

// 1/sqrt(mean(sum^2) + eps) of the row, in double: each thread's squares in
// order, then the wave sums, then the four waves in order.  Every thread of
// the workgroup calls it (it synchronises the workgroup once).
Q8S_DEV double norm_inv(double ss, int d, float eps, double *wsum)
{
    ss = wave_sum_f64(ss);
    if ((threadIdx.x & 63) == 0)
        wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int i = 0; i < NORM_THREADS / WAVE; i++)
        tot += wsum[i];
    return 1.0 / sqrt(tot / (double)d + (double)eps);
}

template <int SEGS>
Q8S_DEV double norm_squares(const NormShare<SEGS> &n, int d, int t8)
{
    double ss = 0.0;
#pragma unroll
    for (int g = 0; g < SEGS; g++) {
        const bool in = t8 + g * NORM_SEG < d;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const double q = (double)n.sv[g][0][i] * (double)n.sv[g][0][i] + (double)n.sv[g][1][i] * (double)n.sv[g][1][i];
            ss += in ? q : 0.0;
        }
    }
    return ss;
}

// The normalised values of segment g, formed in double and rounded once.
Q8S_DEV void norm_values(f32x4 s0, f32x4 s1, f32x4 w0, f32x4 w1, double inv, float (&v)[8])
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[i] = (float)(((double)s0[i] * inv) * (double)w0[i]);
        v[4 + i] = (float)(((double)s1[i] * inv) * (double)w1[i]);
    }
}

} // namespace q8s
