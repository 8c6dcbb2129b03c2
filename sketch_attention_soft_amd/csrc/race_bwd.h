// race_bwd.h -- backward kernels of RACE attention (gfx950).
//
// The pages state the method is differentiable end to end ("RACE Attention:
// A Strictly Linear-Time Attention for Long-Sequence Training",
// gist.science/es/paper/2510.04008 technical summary §2 item 3,
// gist.science/fr/... §3 item 3); the gradient below is the exact derivative
// of the forward of race_fwd.h.
//
// With m_i the readout denominator and g_i = dL/do_i, write the ratio-rule
// rows D_i = [g_i / m_i | -(g_i . o_i) / m_i] (80 columns with padding).
// With psi the Walsh features (race_common.h) and, in causal mode, sums over
// the visible pairs only (key j <= query i):
//   dpsi(q_i) = S_i D_i,            S_i = sum_{j <= i} psi(k_j)^T [v_j | 1]
//   dpsi(k_j) = G_j^T [v_j | 1],    G_j = sum_{i >= j} psi(q_i)^T D_i
//   dv_j      = psi(k_j) G_j[:, :d]
// then through the feature map, the squashes and the normalisation:
//   dt_p = sum_{S containing p} dpsi_S * dpsi_S/dt_p
//   du_p = dt_p * ((1 - t_p^2)/tau) * (1 - z_p^2)         (stored by hash_kernel<CHAIN>)
//   dxh  = du W          (K = L*P, MFMA)
//   dx   = (dxh - (dxh . xh) xh) / |x|                    (|x| > 1e-12; else dxh / 1e-12)
// dv is computed by readout_kernel<BWD = true>; dq and dk by dpsi_kernel.
#pragma once
#include "race_common.h"
#include "race_fwd.h"

namespace race {

// W^T in three forms for the dxh product: bf16 hi, bf16 lo (W = hi + lo) and
// fp32, each [HD][lp32] with hyperplanes beyond L*P zero.
static __global__ __launch_bounds__(256) void prep_wt_kernel(const float *__restrict__ W, int LP,
                                                      int lp32, char *__restrict__ wt)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= HD * lp32) return;
    const int col = e / lp32, hp = e % lp32;
    const float w = hp < LP ? W[hp * HD + col] : 0.f;
    const bf16 hi = (bf16)w;
    const bf16 lo = (bf16)(w - (float)hi);
    reinterpret_cast<bf16 *>(wt)[e] = hi;
    reinterpret_cast<bf16 *>(wt)[HD * lp32 + e] = lo;
    reinterpret_cast<float *>(wt + (size_t)HD * lp32 * 4)[e] = w;
}

// dpsi_kernel: gradient of the rows "r" that read a CxF state built from rows
// "w".  dQ: r = queries (values D), w = keys (values [v | 1]), token order,
// intra mask w <= r.  dK: r = keys (values [v | 1]), w = queries (values D),
// reverse token order, intra mask w >= r.  Then the hash backward of the r
// rows.  X: the raw r rows; t arrays hold 8 floats per table (t, dt/du).
template <typename T, int NW, int CAUSAL, bool REVERSE, bool READER_D>
__global__ __launch_bounds__(NW * 64) void dpsi_kernel(
    const T *__restrict__ X, const float *__restrict__ tr, const float *__restrict__ tw,
    ValSrc<T> vr_src, ValSrc<T> vw_src, const char *__restrict__ wt, int lp32, int64_t N, int L,
    int seg, int64_t nseg, const float *__restrict__ st, T *__restrict__ dX, Lens ls,
    Part prt = Part{nullptr, nullptr}, int pmode = PART_NONE)
{
    constexpr int F = NW * FPW;
    constexpr int TS = 2 * NP;
    constexpr int LPMAX = NW * TPW * NP;  // hyperplanes covered by the waves (multiple of 32)
    __shared__ __attribute__((aligned(16))) T pw[CAUSAL ? F * CH : 8];
    __shared__ __attribute__((aligned(16))) T yr[CH * NCOL];
    __shared__ __attribute__((aligned(16))) T yw[CAUSAL ? CH * NCOL : 8];
    __shared__ __attribute__((aligned(16))) T ywt[CAUSAL ? NCOL * CH : 8];
    __shared__ __attribute__((aligned(16))) float dpsi[CH * F];
    __shared__ __attribute__((aligned(16))) T dub[CH * LPMAX];
    __shared__ __attribute__((aligned(16))) float dxh[CH * HD];

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const T *Xh = X + bh * N * HD;
    const float *trh = tr + bh * N * L * TS;
    const float *twh = tw + bh * N * L * TS;
    ValSrc<T> vrh = vr_src, vwh = vw_src;
    vrh.V += bh * N * HD;
    vwh.V += bh * N * HD;
    if (READER_D) {
        vrh.O += bh * N * HD;
        vrh.den += bh * N;
    } else {
        vwh.O += bh * N * HD;
        vwh.den += bh * N;
    }
    T *dXh = dX + bh * N * HD;
    const bf16 *wt_hi = reinterpret_cast<const bf16 *>(wt);
    const bf16 *wt_lo = wt_hi + HD * lp32;
    const float *wt_f = reinterpret_cast<const float *>(wt + (size_t)HD * lp32 * 4);

    floatx4 acc[NT][MT];  // CxF state
    {
        const float *src = st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(F * NCOL);
#pragma unroll
        for (int ft = 0; ft < MT; ++ft)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                acc[ct][ft] = *reinterpret_cast<const floatx4 *>(src + st_index(w, ft, ct, lane));
    }
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(valid_rows(ls, bh, N), t_begin + seg);
    const int64_t nch = (t_end - t_begin + CH - 1) / CH;
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t tok0 = t_begin + (REVERSE ? nch - 1 - ci : ci) * CH;
        __syncthreads();
        load_vals<T, READER_D>(vrh, tok0, t_end, nullptr, yr);
        if (CAUSAL) {
            load_vals<T, !READER_D>(vwh, tok0, t_end, ywt, yw);
            expand_t<T>(twh, TS, tok0, t_end, L, pw);
        }
        __syncthreads();

        // E[i][j] = y_r(i) . y_w(j), computed transposed so that the
        // accumulator is directly the A operand of E psi_w (lane: row i, k = j)
        F4<T> efrag;
        if (CAUSAL) {
            floatx4 eacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < NT; ++kc) {
                const F4<T> a = ld4<T>(yw + c16 * NCOL + kc * 16 + g * 4);
                const F4<T> b = ld4<T>(yr + c16 * NCOL + kc * 16 + g * 4);
                mma(eacc, a, b);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = c16, j = g * 4 + r;
                const bool keep = REVERSE ? (j >= i) : (j <= i);
                efrag.v[r] = from_f32<T>(keep ? eacc[r] : 0.f);
            }
        }
        // dpsi_r = y_r S^T (+ E psi_w), wave's features; lane: feature column, rows i
#pragma unroll
        for (int ft = 0; ft < MT; ++ft) {
            floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < NT; ++kc) {
                const F4<T> a = ld4<T>(yr + c16 * NCOL + kc * 16 + g * 4);
                mma(d, a, acc2frag4<T>(acc[kc][ft]));
            }
            if (CAUSAL) {
                const F4<T> b = ld4<T>(pw + (w * FPW + ft * 16 + c16) * CH + g * 4);
                mma(d, efrag, b);
            }
            const int f = w * FPW + ft * 16 + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) dpsi[(g * 4 + r) * F + f] = d[r];
        }
        if (CAUSAL) update_cxf<T>(acc, pw, ywt);
        __syncthreads();

        // through the feature map: du for every (token, table)
        for (int e = threadIdx.x; e < CH * NW * TPW; e += NW * 64) {
            const int i = e / (NW * TPW), l = e % (NW * TPW);
            const int64_t tok = tok0 + i;
            float du[4] = {0.f, 0.f, 0.f, 0.f};
            if (l < L && tok < t_end) {
                const float *tp = trh + (tok * L + l) * TS;
                const floatx4 tv = *reinterpret_cast<const floatx4 *>(tp);
                const floatx4 sd = *reinterpret_cast<const floatx4 *>(tp + NP);
                const float *dp = dpsi + i * F + l * NR;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    floatx4 t1 = tv;
                    t1[p] = 1.f;
                    float part[16];
                    walsh16(t1, part);  // d psi_S / d t_p for S containing p
                    float acc_p = 0.f;
#pragma unroll
                    for (int S = 0; S < 16; ++S)
                        if (S & (1 << p)) acc_p += dp[S] * part[S];
                    du[p] = acc_p * sd[p];
                }
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) dub[i * LPMAX + l * NP + p] = from_f32<T>(du[p]);
        }
        __syncthreads();

        // dxh = du W: column tiles of d over the waves, K = hyperplanes
        for (int nt = w; nt < HD / 16; nt += NW) {
            floatx4 d = {0.f, 0.f, 0.f, 0.f};
            const int col = nt * 16 + c16;
            for (int kb = 0; kb < lp32 / 32; ++kb) {
                const F8<T> a = ld8<T>(dub + c16 * LPMAX + kb * 32 + g * 8);
                if constexpr (sizeof(T) == 2) {
                    mma(d, a, ld8<bf16>(wt_hi + col * lp32 + kb * 32 + g * 8));
                    mma(d, a, ld8<bf16>(wt_lo + col * lp32 + kb * 32 + g * 8));
                } else {
                    mma(d, a, ld8<float>(wt_f + col * lp32 + kb * 32 + g * 8));
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) dxh[(g * 4 + r) * HD + col] = d[r];
        }
        __syncthreads();

        // normalisation backward, 16 threads per row
        for (int base = 0; base < CH * 16; base += blockDim.x) {
            const int e = base + threadIdx.x;
            const int i = (e >> 4) & (CH - 1), part = e & 15;
            const int64_t tok = tok0 + i;
            const bool ok = (e < CH * 16) && tok < t_end;
            float x[4] = {0.f, 0.f, 0.f, 0.f}, dh[4] = {0.f, 0.f, 0.f, 0.f};
            if (ok) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    x[c] = to_f32(Xh[tok * HD + part * 4 + c]);
                    dh[c] = dxh[i * HD + part * 4 + c];
                }
            }
            // table passes (L > 32): dx_hat of the tables so far in fp32
            // partial rows; every pass but the last stores the sum and stops
            // before the normalisation backward (uniform per launch)
            if (pmode != PART_NONE) {
                float *pr = prt.v + (bh * N + tok) * HD + part * 4;
                if (ok && pmode != PART_OUT)
#pragma unroll
                    for (int c = 0; c < 4; ++c) dh[c] += pr[c];
                if (pmode != PART_IN) {
                    if (ok)
#pragma unroll
                        for (int c = 0; c < 4; ++c) pr[c] = dh[c];
                    continue;
                }
            }
            float ss = 0.f, dot = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                ss += x[c] * x[c];
                dot += dh[c] * x[c];
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                ss += __shfl_xor(ss, o);
                dot += __shfl_xor(dot, o);
            }
            const float nrm = sqrtf(ss);
            if (ok) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float r;
                    if (nrm > 1e-12f) {
                        const float inv = 1.0f / nrm;
                        r = (dh[c] - dot * inv * inv * x[c]) * inv;
                    } else {
                        r = dh[c] * 1e12f;
                    }
                    dXh[tok * HD + part * 4 + c] = from_f32<T>(r);
                }
            }
        }
    }
}

}  // namespace race
