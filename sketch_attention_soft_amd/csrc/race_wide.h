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
//   hash_rows_kernel  u = W x on MFMA (W as bf16 hi + lo, as the fused
//                     kernels project), scaled by 1/|x|; t = tanh(tanh(u')/tau)
//                     and dt/du' in fp32, stored in fp16 in the cache layout
//                     the fused kernels read ([head][16-token tile][wave]
//                     [lane][4], lane (g, c16) of wave w: table 4 w + g, token
//                     c16)
//   dm_rows_kernel    -(dO . o) / m over the whole row, the gradient values'
//                     last column (the first pass carries it, the second a
//                     zero column)
//   du_rows_kernel    dx_hat = du W over both passes' du on MFMA (the
//                     gradient is linear in the values' columns), and
//                     dx = (dx_hat - x (x . dx_hat) / |x|^2) / |x|
// They take any d <= 128 (a multiple of 8); the host uses them for d = 128.
#pragma once
#include "race_walk.h"

namespace race {

constexpr int WD_MAX = 128;          // row length
constexpr int WROWS = 16;            // rows per tile (one MFMA column block)
constexpr int WH_MAX = 128;          // internal hyperplane rows: 8 waves x 16
constexpr int WKS = WD_MAX + 8;      // staged W row stride (bf16)
constexpr int WTS2 = WH_MAX + 8;     // staged W^T row stride (bf16)

// 8 elements of a 16-bit row as floats (exact) and as a bf16 operand
template <typename IO> struct Row8 {
    float f[8];
    bf16x8 b;
};
template <typename IO>
__device__ __forceinline__ Row8<IO> load_row8(const IO *__restrict__ p, bool ok)
{
    Row8<IO> r;
    const u32x4 v = ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.f[2 * i] = io_lo<IO>(v[i]);
        r.f[2 * i + 1] = io_hi<IO>(v[i]);
    }
    if constexpr (is_bf16<IO>)
        r.b = __builtin_bit_cast(bf16x8, v);
    else
        r.b = pk8(pk_bf16(r.f[0], r.f[1]), pk_bf16(r.f[2], r.f[3]), pk_bf16(r.f[4], r.f[5]),
                  pk_bf16(r.f[6], r.f[7]));
    return r;
}

// hash_rows_kernel: rows of d = 128 elements into the fused kernels' feature
// cache.  256 threads; the workgroup stages the internal hyperplane rows of
// W once (bf16 hi + lo, about 16 bits, as the fused kernels' projection),
// then every wave takes 16-token tiles of the cache (tiles per head x heads,
// in grid strides).  For fused wave w (tables 4 w .. 4 w + 3) the wave forms
// U^T = W x^T on MFMA (16 hyperplanes x 16 tokens, K = 128): lane (g, c16)
// then holds the 4 hyperplanes of table 4 w + g for token c16, which is the
// cache's layout, and stores t (and with ct, dt/du) as 4 fp16 values.
// Tokens past N get zeros (the fused kernels read whole tiles and multiply
// the features of those tokens by zero value rows, so they must be finite).
// inv_tau = 1 / tau; nwf: waves of the fused kernels.
template <typename IO>
__global__ __launch_bounds__(256) void hash_rows_kernel(const IO *__restrict__ X, int64_t N, int d,
                                                        const float *__restrict__ W, int L, int P,
                                                        float inv_tau, int nwf, int64_t tiles, int64_t nheads,
                                                        _Float16 *__restrict__ tt, _Float16 *__restrict__ ct)
{
    __shared__ __attribute__((aligned(16))) bf16 wl[2][WH_MAX * WKS];
    for (int e = threadIdx.x; e < nwf * 16 * WD_MAX; e += blockDim.x) {
        const int hp = e / WD_MAX, c = e % WD_MAX;
        const float v = w_elem(W, L, P, d, hp, c);
        const bf16 hi = (bf16)v;
        wl[0][hp * WKS + c] = hi;
        wl[1][hp * WKS + c] = (bf16)(v - (float)hi);
    }
    __syncthreads();
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    const int nwv = blockDim.x / 64;
    for (int64_t item = (int64_t)blockIdx.x * nwv + wave_id(); item < nheads * tiles;
         item += (int64_t)gridDim.x * nwv) {
        const int64_t bh = item / tiles, tok = (item % tiles) * WROWS + c16;
        const bool ok = tok < N;
        // the row of token c16 as four K = 32 operand blocks (lane group g
        // holds elements 32 k + 8 g .. + 7), and its squared norm
        bf16x8 xb[4];
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = 32 * k + 8 * g;
            const Row8<IO> r = load_row8<IO>(X + (bh * N + tok) * d + c, ok && c < d);
            xb[k] = r.b;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = fmaf(r.f[i], r.f[i], ss);
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
        for (int w = 0; w < nwf; ++w) {
            floatx4 u = {0.f, 0.f, 0.f, 0.f};
            const bf16 *wr = &wl[0][(16 * w + c16) * WKS + 8 * g];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                mma32(u, *reinterpret_cast<const bf16x8 *>(wr + 32 * k), xb[k]);
                mma32(u, *reinterpret_cast<const bf16x8 *>(wr + WH_MAX * WKS + 32 * k), xb[k]);
            }
            halfx4 th, ch;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = tanhf(u[r] * inv);
                const float t = tanhf(z * inv_tau);
                // padding rows and tokens past N: zeros
                const bool live = ok && w_row(L, P, 16 * w + 4 * g + r) >= 0;
                th[r] = (_Float16)(live ? t : 0.f);
                ch[r] = (_Float16)(live ? (1.f - t * t) * inv_tau * (1.f - z * z) : 0.f);
            }
            const int64_t idx = ((item * nwf + w) * 64 + lane) * 4;
            *reinterpret_cast<halfx4 *>(tt + idx) = th;
            if (ct) *reinterpret_cast<halfx4 *>(ct + idx) = ch;
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
        for (int c = 8 * q; c < d; c += 128) {
            const Row8<IO> a = load_row8<IO>(dO + r * d + c, true), b = load_row8<IO>(O + r * d + c, true);
#pragma unroll
            for (int i = 0; i < 8; ++i) dot = fmaf(a.f[i], b.f[i], dot);
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) dot += __shfl_xor(dot, m);
    if (r < rows && q == 0) dm[r] = -dot / den[r];
}

// du_rows_kernel: 256 threads; the workgroup stages W^T once (bf16, the
// precision of du), then every wave takes blocks of 16 rows (grid strides).
// dx_hat^T = W^T du^T on MFMA over both passes' du (16 dims x 16 rows per
// tile, K = the nh internal hyperplanes): lane (g, c16) holds dims
// 16 dt + 4 g .. + 3 of row c16, so the dots over the row are sums over the
// lane groups.  dx = (dx_hat - x (x . dx_hat) / |x|^2) / |x| for |x| > 1e-12,
// else dx_hat 1e12.  du_a, du_b: bf16 [rows][nh], nh = 16 nwf <= WH_MAX.
template <typename IO>
__global__ __launch_bounds__(256) void du_rows_kernel(const IO *__restrict__ X, int64_t rows, int d,
                                                      const float *__restrict__ W, int L, int P, int nh,
                                                      const bf16 *__restrict__ du_a, const bf16 *__restrict__ du_b,
                                                      IO *__restrict__ dX)
{
    __shared__ __attribute__((aligned(16))) bf16 wt[WD_MAX * WTS2];  // W^T: [dim][hyperplane]
    for (int e = threadIdx.x; e < nh * WD_MAX; e += blockDim.x) {
        const int hp = e / WD_MAX, c = e % WD_MAX;
        wt[c * WTS2 + hp] = (bf16)w_elem(W, L, P, d, hp, c);
    }
    __syncthreads();
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    const int nwv = blockDim.x / 64, nk = nh / 32;
    for (int64_t blk = (int64_t)blockIdx.x * nwv + wave_id(); blk * WROWS < rows;
         blk += (int64_t)gridDim.x * nwv) {
        const int64_t row = blk * WROWS + c16;
        const bool ok = row < rows;
        // du of both passes as K = 32 operand blocks (hyperplanes 32 k + 8 g .. + 7)
        bf16x8 ua[WH_MAX / 32], ub[WH_MAX / 32];
#pragma unroll
        for (int k = 0; k < WH_MAX / 32; ++k) {
            const bool in = ok && k < nk;
            const u32x4 z = {0u, 0u, 0u, 0u};
            ua[k] = __builtin_bit_cast(bf16x8, in ? *reinterpret_cast<const u32x4 *>(du_a + row * nh + 32 * k + 8 * g) : z);
            ub[k] = __builtin_bit_cast(bf16x8, in ? *reinterpret_cast<const u32x4 *>(du_b + row * nh + 32 * k + 8 * g) : z);
        }
        floatx4 dxh[WD_MAX / 16];
        float xv[WD_MAX / 16][4], dot = 0.f, ss = 0.f;
#pragma unroll
        for (int dt = 0; dt < WD_MAX / 16; ++dt) {
            dxh[dt] = {0.f, 0.f, 0.f, 0.f};
            const bf16 *wr = wt + (16 * dt + c16) * WTS2 + 8 * g;
#pragma unroll
            for (int k = 0; k < WH_MAX / 32; ++k) {
                if (k < nk) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(wr + 32 * k);
                    mma32(dxh[dt], a, ua[k]);
                    mma32(dxh[dt], a, ub[k]);
                }
            }
            const int c = 16 * dt + 4 * g;
            const u32x2 xw = ok && c < d ? *reinterpret_cast<const u32x2 *>(X + row * d + c) : u32x2{0u, 0u};
            xv[dt][0] = io_lo<IO>(xw[0]);
            xv[dt][1] = io_hi<IO>(xw[0]);
            xv[dt][2] = io_lo<IO>(xw[1]);
            xv[dt][3] = io_hi<IO>(xw[1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dot = fmaf(dxh[dt][r], xv[dt][r], dot);
                ss = fmaf(xv[dt][r], xv[dt][r], ss);
            }
        }
        dot += __shfl_xor(dot, 16);
        dot += __shfl_xor(dot, 32);
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float invn = 1.f / fmaxf(sqrtf(ss), 1e-12f);
        const float coef = ss > 1e-24f ? dot * invn * invn : 0.f;
#pragma unroll
        for (int dt = 0; dt < WD_MAX / 16; ++dt) {
            const int c = 16 * dt + 4 * g;
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (dxh[dt][r] - coef * xv[dt][r]) * invn;
            if (ok && c < d)
                *reinterpret_cast<u32x2 *>(dX + row * d + c) = u32x2{pk_io<IO>(o[0], o[1]), pk_io<IO>(o[2], o[3])};
        }
    }
}

}  // namespace race
