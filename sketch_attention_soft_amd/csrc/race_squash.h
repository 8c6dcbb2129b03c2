// race_squash.h -- pieces shared by the bf16 chunk kernels: the host-fitted
// squash polynomial, the segment-state block index and the gradient of the
// Walsh features of one table.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (soft
// hashing with tanh-squashed projections and a temperature).
#pragma once
#include "race_common.h"

namespace race {

constexpr int MAXDEG = 16;  // coefficient slots reported by the diagnostic entry points
constexpr int DEG16 = 6;    // degree of the fp16 squash polynomials

// t = tanh(tanh(u') / tau) and dt/du' as polynomials in y = 2 exp(-2|u'|) - 1,
// evaluated by the bf16 kernels in fp16 pairs (deg < 0: the host fit missed
// its accuracy target and the kernels evaluate the functions directly).
struct Squash {
    uint32_t t16[DEG16 + 1];  // fp16 coefficients of |t|, each in both halves
    uint32_t c16[DEG16 + 1];  // fp16 coefficients of dt/du'
    int deg;
    float inv_tau;
};

// Segment state block of a workgroup: [wave][tile a][column tile ct][lane][4 floats]
// (at = tiles per wave).
__device__ __forceinline__ int64_t st_idx(int w, int a, int ct, int lane, int at)
{
    return ((((int64_t)w * at + a) * NT + ct) * 64 + lane) * 4;
}

// Gradient of the Walsh features of one table: with
// P(t) = sum_S dpsi_S prod_{p in S} t_p (the features without their common
// factor 1/4), dt[p] = dP/dt_p.  P is multilinear: contracting t_3, then t_2
// and t_1, yields the four partial derivatives in 24 fused multiply-adds.
// Returns P(t) itself (the gradient of a factor that multiplies every
// feature of the table).
__device__ __forceinline__ float walsh_grad(const float dp[16], const floatx4 &t, float dt[4])
{
    float a[8], c[4], b[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = fmaf(t[3], dp[i + 8], dp[i]);  // P with t_3 contracted
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = fmaf(t[2], dp[i + 12], dp[i + 8]);
    dt[3] = fmaf(t[0], fmaf(t[1], c[3], c[1]), fmaf(t[1], c[2], c[0]));
    dt[2] = fmaf(t[0], fmaf(t[1], a[7], a[5]), fmaf(t[1], a[6], a[4]));
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = fmaf(t[2], a[i + 4], a[i]);  // then t_2
    dt[1] = fmaf(t[0], b[3], b[2]);
    dt[0] = fmaf(t[1], b[3], b[1]);
    return fmaf(t[0], dt[0], fmaf(t[1], b[2], b[0]));  // b0 + t0 b1 + t1 b2 + t0 t1 b3
}

}  // namespace race
