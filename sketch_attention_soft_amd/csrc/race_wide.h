// race_wide.h -- the row-wise kernels of RACE attention for heads of 128
// elements (gfx950): hashing into the fused kernels' feature cache, the
// gradient values' last column, and the tail of the gradient (dx_hat = du W
// and the normalisation backward).
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (soft
// hashing of the normalised rows with Gaussian hyperplanes, tanh squash,
// temperature); gist.science/es/... §2 (the kernel on normalised vectors);
// differentiable end to end (es §2 item 3).
//
// A head of d = 128 runs the fused chunk kernels twice, on value columns
// 0..63 and 64..127 (the state of one pass, 64 features x 80 columns per
// wave, is what fits in registers).  Everything that needs the whole row
// happens here, once per row:
//   hash_rows_kernel  x / |x|, u = W x_hat, t = tanh(tanh(u) / tau) and
//                     dt/du (fp32), stored in fp16 in the cache layout the
//                     fused kernels read ([head][16-token tile][wave][lane][4],
//                     lane (g, c16) of wave w: table 4 w + g, token c16)
//   dm_rows_kernel    -(dO . o) / m over the whole row, the gradient values'
//                     last column (the first pass carries it, the second a
//                     zero column)
//   du_rows_kernel    du of the two passes added (the gradient is linear in
//                     the values' columns), dx_hat = du W, and
//                     dx = (dx_hat - x (x . dx_hat) / |x|^2) / |x|
// They take any d <= 128 (a multiple of 8); the host uses them for d = 128.
#pragma once
#include "race_walk.h"

namespace race {

constexpr int WD_MAX = 128;      // row length
constexpr int WROWS = 16;        // rows per workgroup
constexpr int WXS = WD_MAX + 1;  // staged row stride (fp32)
constexpr int WH_MAX = 128;      // internal hyperplane rows: 8 waves x 16

// the row's elements as floats (16-bit rows)
template <typename IO> __device__ __forceinline__ float io_f(IO v) { return (float)v; }

// rows r0 .. r0 + 15 of X ([rows][d], 16-bit) into xs[16][WXS] as fp32 (zero
// past the last row and past column d); 16 threads per row
template <typename IO>
__device__ __forceinline__ void stage_rows(const IO *__restrict__ X, int64_t r0, int64_t rows, int d,
                                           float *xs)
{
    for (int e = threadIdx.x; e < WROWS * WD_MAX; e += blockDim.x) {
        const int j = e / WD_MAX, c = e % WD_MAX;
        const int64_t r = r0 + j;
        xs[j * WXS + c] = r < rows && c < d ? io_f(X[r * d + c]) : 0.f;
    }
}

// internal hyperplane rows of W (the fused kernels' 4 per table, padding
// rows zero) into wl[nrows][WXS] as fp32
__device__ __forceinline__ void stage_w_rows(const float *__restrict__ W, int L, int P, int d, int nrows,
                                             float *wl)
{
    for (int e = threadIdx.x; e < nrows * WD_MAX; e += blockDim.x) {
        const int hp = e / WD_MAX, c = e % WD_MAX;
        wl[hp * WXS + c] = c < d ? w_elem(W, L, P, d, hp, c) : 0.f;
    }
}

// hash_rows_kernel: grid (16-token tiles of a head, heads); 256 threads.
// nwf: waves of the fused kernels (4 tables each).  Writes t (and with ct,
// dt/du) of every internal table 4 w + g < 4 nwf for the 16 tokens (tokens
// past N are not written).  inv_tau = 1 / tau.
template <typename IO>
__global__ __launch_bounds__(256) void hash_rows_kernel(const IO *__restrict__ X, int64_t N, int d,
                                                        const float *__restrict__ W, int L, int P,
                                                        float inv_tau, int nwf, int64_t tiles,
                                                        _Float16 *__restrict__ tt, _Float16 *__restrict__ ct)
{
    __shared__ float xs[WROWS * WXS];  // the rows (fp32)
    __shared__ float inv[WROWS];       // 1 / max(|x|, 1e-12)
    __shared__ float wl[WH_MAX * WXS];  // W rows of the internal hyperplanes
    const int64_t bh = blockIdx.y, tile = blockIdx.x;
    const int64_t r0 = bh * N + tile * WROWS;
    const int64_t nrow = min<int64_t>(WROWS, N - tile * WROWS);
    stage_rows(X, r0, bh * N + tile * WROWS + nrow, d, xs);
    stage_w_rows(W, L, P, d, nwf * 16, wl);
    __syncthreads();
    {
        // |x| of row j: 16 threads, 8 elements each, summed over the 16 lanes
        const int j = threadIdx.x >> 4, q = threadIdx.x & 15;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = xs[j * WXS + q * 8 + i];
            ss = fmaf(x, x, ss);
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) ss += __shfl_xor(ss, m);
        if (q == 0) inv[j] = 1.f / fmaxf(sqrtf(ss), 1e-12f);
    }
    __syncthreads();
    const int ntab = 4 * nwf;  // internal tables of the fused kernels (padding ones included)
    for (int e = threadIdx.x; e < WROWS * ntab; e += blockDim.x) {
        const int j = e % WROWS, it = e / WROWS;
        if (j >= nrow) continue;
        float tv[4], cv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hp = 4 * it + r;
            float u = 0.f;
            for (int c = 0; c < d; ++c) u = fmaf(wl[hp * WXS + c], xs[j * WXS + c], u);
            const float z = tanhf(u * inv[j]);
            const float t = tanhf(z * inv_tau);
            const bool pad = w_row(L, P, hp) < 0;  // padding rows: t = +0
            tv[r] = pad ? 0.f : t;
            cv[r] = pad ? 0.f : (1.f - t * t) * inv_tau * (1.f - z * z);
        }
        const int w = it >> 2, g = it & 3, tok = j;
        const int64_t idx = (((bh * tiles + tile) * nwf + w) * 64 + g * 16 + tok) * 4;
        const halfx4 th = {(_Float16)tv[0], (_Float16)tv[1], (_Float16)tv[2], (_Float16)tv[3]};
        *reinterpret_cast<halfx4 *>(tt + idx) = th;
        if (ct) {
            const halfx4 ch = {(_Float16)cv[0], (_Float16)cv[1], (_Float16)cv[2], (_Float16)cv[3]};
            *reinterpret_cast<halfx4 *>(ct + idx) = ch;
        }
    }
}

// dm_rows_kernel: dm[row] = -(dO . o) / m for rows of d elements; 16 threads
// per row (grid over all rows, 256 threads)
template <typename IO>
__global__ __launch_bounds__(256) void dm_rows_kernel(const IO *__restrict__ dO, const IO *__restrict__ O,
                                                      const float *__restrict__ den, int64_t rows, int d,
                                                      float *__restrict__ dm)
{
    const int64_t r = (int64_t)blockIdx.x * WROWS + (threadIdx.x >> 4);
    const int q = threadIdx.x & 15;
    float dot = 0.f;
    if (r < rows)
        for (int c = q; c < d; c += 16) dot = fmaf(io_f(dO[r * d + c]), io_f(O[r * d + c]), dot);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) dot += __shfl_xor(dot, m);
    if (r < rows && q == 0) dm[r] = -dot / den[r];
}

// du_rows_kernel: grid (16-row blocks of all rows); 256 threads = 16 rows x
// 16 threads of 8 columns.  du_a, du_b: the two passes' du, bf16
// [rows][nh] (nh = 16 nwf internal hyperplanes, at most WH_MAX).
template <typename IO>
__global__ __launch_bounds__(256) void du_rows_kernel(const IO *__restrict__ X, int64_t rows, int d,
                                                      const float *__restrict__ W, int L, int P, int nh,
                                                      const bf16 *__restrict__ du_a, const bf16 *__restrict__ du_b,
                                                      IO *__restrict__ dX)
{
    __shared__ float xs[WROWS * WXS];           // the rows (fp32)
    __shared__ float dul[WROWS * (WH_MAX + 1)];  // du of both passes, [16][nh + 1]
    __shared__ float wl[WH_MAX * WXS];          // W rows of the internal hyperplanes
    const int64_t r0 = (int64_t)blockIdx.x * WROWS;
    stage_rows(X, r0, rows, d, xs);
    stage_w_rows(W, L, P, d, nh, wl);
    for (int e = threadIdx.x; e < WROWS * nh; e += blockDim.x) {
        const int j = e / nh, h = e % nh;
        const int64_t r = r0 + j;
        dul[j * (nh + 1) + h] = r < rows ? (float)du_a[r * nh + h] + (float)du_b[r * nh + h] : 0.f;
    }
    __syncthreads();
    const int j = threadIdx.x >> 4, q = threadIdx.x & 15;
    const int64_t r = r0 + j;
    float dxh[8], xv[8], dot = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = q * 8 + i;
        float a = 0.f;
        for (int h = 0; h < nh; ++h) a = fmaf(dul[j * (nh + 1) + h], wl[h * WXS + c], a);
        dxh[i] = a;
        xv[i] = xs[j * WXS + c];
        dot = fmaf(a, xv[i], dot);
        ss = fmaf(xv[i], xv[i], ss);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
        dot += __shfl_xor(dot, m);
        ss += __shfl_xor(ss, m);
    }
    // dx = (dx_hat - x (x . dx_hat) / |x|^2) / |x| for |x| > 1e-12, else dx_hat 1e12
    const float invn = 1.f / fmaxf(sqrtf(ss), 1e-12f);
    const float coef = ss > 1e-24f ? dot * invn * invn : 0.f;
    if (r < rows)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = q * 8 + i;
            if (c < d) dX[r * d + c] = (IO)((dxh[i] - coef * xv[i]) * invn);
        }
}

}  // namespace race
