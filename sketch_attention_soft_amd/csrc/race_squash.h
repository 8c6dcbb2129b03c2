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

// dt_p = d(sum_S dpsi_S psi_S)/dt_p for one table: the multilinear polynomial
// with coefficients dpsi_{S u p}, S over the other three bits, evaluated at t.
__device__ __forceinline__ void walsh_grad(const float dp[16], const floatx4 &t, float dt[4])
{
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        int o[3], n = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b != p) o[n++] = b;
        float m[4];
#pragma unroll
        for (int yz = 0; yz < 4; ++yz) {
            const int base = (1 << p) | ((yz & 1) << o[1]) | ((yz >> 1) << o[2]);
            m[yz] = fmaf(t[o[0]], dp[base | (1 << o[0])], dp[base]);
        }
        const float n0 = fmaf(t[o[1]], m[1], m[0]);
        const float n1 = fmaf(t[o[1]], m[3], m[2]);
        dt[p] = 0.25f * fmaf(t[o[2]], n1, n0);
    }
}

}  // namespace race
