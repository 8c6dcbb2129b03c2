// race_fused.h -- fused chunk kernels of RACE attention (gfx950): every
// kernel hashes its own rows (no hash features in HBM), keeps the sketch state
// in MFMA accumulators and prefetches the next chunk while computing one.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (soft
// hashing, bucket sums, ratio readout) and §2.3 (causal streaming sums); the
// es page §2 (angular kernel on normalised vectors).
//
// Hash of one row x (all in registers):
//   u = W x (MFMA; bf16 rows use W = W_hi + W_lo), x_hat scaling by 1/|x|,
//   t = tanh(tanh(u') / tau) = sign(u') h(e),  e = exp(-2|u'|),
//   h(e) = tanh(((1 - e)/(1 + e)) / tau) as a polynomial in y = 2e - 1 whose
//   coefficients the host fits for each tau by Chebyshev interpolation in
//   fp64 (deg < 0: evaluated directly with exp and reciprocal instead).
//
// Chunk of CT = 32 tokens.  Wave w owns HT hash tiles of 16 hyperplanes
// (4 tables each): tables l0 + 4h + g with l0 = 4 HT w, h < HT, g = lane/16.
//   projection accumulator: lane (token c16, hyperplanes 4g + p of tile h)
//     -> t of table l0+4h+g for token c16: the 16 Walsh features of that
//     table are a token-major operand fragment directly:
//     K-block (h, k): slot (g, i) <-> (table l0 + 4h + g, S = 8k + i).
//   feature-major fragments (for sums over tokens) read t back from LDS:
//     M-tile (h, s): row 4q + p <-> (table l0 + 4h + q, S = 4s + p),
//     K-slots = tokens 8g + i.
//   FxC state tile (h, s, ct): lane (column 16ct + c16, rows 4g + r) <->
//     features (table l0 + 4h + g, S = 4s + r); tiles (h, 2k) and (h, 2k+1)
//     form the B operand of K-block (h, k) of the readout.
// Segment state blocks in global memory: [wave][4 HT][5][64 lanes][4 floats].
#pragma once
#include "race_common.h"
#include "race_fwd.h"

namespace race {

constexpr int MAXDEG = 16;

// Polynomial degree of the squash per storage type (enough for its accuracy
// target at the temperatures in use; the host falls back to direct
// evaluation, deg < 0, when the fit misses the target).
template <typename T> struct SqDeg;
template <> struct SqDeg<bf16> { static constexpr int v = 8; };
template <> struct SqDeg<float> { static constexpr int v = 12; };

struct Squash {
    float c[MAXDEG + 1];  // monomial coefficients in y = 2e - 1
    int deg;              // < 0: direct evaluation
    float inv_tau;
};

// t = tanh(tanh(v) / tau) (and optionally dt/dv); polynomial of degree DEG
template <int DEG, bool CHAIN>
__device__ __forceinline__ float squash(float v, const Squash &sq, float *dtdv)
{
    const float av = fabsf(v);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * av);  // exp(-2|v|)
    float h;
    if (sq.deg >= 0) {
        const float y = 2.f * e - 1.f;
        h = sq.c[DEG];
#pragma unroll
        for (int k = DEG - 1; k >= 0; --k) h = fmaf(h, y, sq.c[k]);
    } else {
        const float z = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        const float e2 = __builtin_amdgcn_exp2f(-2.8853900817779268f * z * sq.inv_tau);
        h = (1.f - e2) * __builtin_amdgcn_rcpf(1.f + e2);
    }
    if (CHAIN) {
        // dt/dv = ((1 - t^2)/tau) (1 - z^2),  1 - z^2 = 4e / (1 + e)^2
        const float r = __builtin_amdgcn_rcpf(1.f + e);
        *dtdv = (1.f - h * h) * sq.inv_tau * 4.f * e * r * r;
    }
    return copysignf(h, v);
}

__device__ __forceinline__ int64_t st_idx(int w, int a, int ct, int lane, int at)
{
    return ((((int64_t)w * at + a) * NT + ct) * 64 + lane) * 4;
}

// W fragments of this wave's hyperplanes (A operand of U^T = W X^T)
template <typename T, int HT> struct WFrag;
template <int HT> struct WFrag<bf16, HT> {
    F8<bf16> hi[HT][2], lo[HT][2];
};
template <int HT> struct WFrag<float, HT> {
    F8<float> f[HT][2];
};

template <typename T, int HT>
__device__ __forceinline__ void load_wfrag(const float *__restrict__ W, int LP, WFrag<T, HT> &wf)
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const int hp = (w * HT + h) * 16 + c16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = hp < LP ? W[hp * HD + kb * 32 + g * 8 + i] : 0.f;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    wf.hi[h][kb].v[i] = (bf16)v[i];
                    wf.lo[h][kb].v[i] = (bf16)(v[i] - (float)wf.hi[h][kb].v[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) wf.f[h][kb].v[i] = v[i];
            }
        }
    }
}

// Row fragments of a token tile: lane holds x[tok][32kb + 8g + i] (zeros past tend)
template <typename T>
__device__ __forceinline__ void load_xfrag(const T *__restrict__ X, int64_t tok, int64_t tend,
                                           F8<T> (&xf)[2])
{
    const int g = lane_id() >> 4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (tok < tend) {
            xf[kb] = ld8<T>(X + tok * HD + kb * 32 + g * 8);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xf[kb].v[i] = from_f32<T>(0.f);
        }
    }
}

// t (and dt/du) of the lane's token for tables l0 + 4h + g, h < HT
template <typename T, int HT, bool CHAIN>
__device__ __forceinline__ void hash_tile(const F8<T> (&xf)[2], const WFrag<T, HT> &wf,
                                          const Squash &sq, floatx4 (&t)[HT], floatx4 (&sd)[HT])
{
    float ss = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = to_f32(xf[kb].v[i]);
            ss += x * x;
        }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float inv_norm = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));  // 1 / max(|x|, 1e-12)
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if constexpr (sizeof(T) == 2) {
                mma(u, wf.hi[h][kb], xf[kb]);
                mma(u, wf.lo[h][kb], xf[kb]);
            } else {
                mma(u, wf.f[h][kb], xf[kb]);
            }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float dd = 0.f;
            t[h][p] = squash<SqDeg<T>::v, CHAIN>(u[p] * inv_norm, sq, &dd);
            if (CHAIN) sd[h][p] = dd;
        }
    }
}

// token-major fragments of the 16 Walsh features of one table: S 0-7 and 8-15
// (zero for padding tables l >= L)
template <typename T>
__device__ __forceinline__ void walsh_frags(const floatx4 &t, bool on, F8<T> &lo, F8<T> &hi)
{
    float psi[16];
    walsh16(t, psi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        lo.v[i] = from_f32<T>(on ? psi[i] : 0.f);
        hi.v[i] = from_f32<T>(on ? psi[8 + i] : 0.f);
    }
}

// Feature-major fragments (M-tiles (h, s), K-slots tokens 8g + i) from t in
// LDS: tb[token * tstride + hyperplane-in-block].  Tables >= L give zeros
// (their t are zero, but the constant feature S = 0 is not).
template <typename T, int HT>
__device__ __forceinline__ void feat_frags(const float *tb, int tstride, int L, F8<T> (&pf)[HT][4])
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int q = c16 >> 2, p = c16 & 3;
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const int l = (w * HT + h) * 4 + q;
        const bool on = l < L;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const floatx4 t = *reinterpret_cast<const floatx4 *>(tb + (g * 8 + i) * tstride +
                                                                (w * HT + h) * 16 + q * 4);
            const float a = 0.25f * ((p & 1) ? t[0] : 1.f) * ((p & 2) ? t[1] : 1.f);
            const float b[4] = {a, a * t[2], a * t[3], a * t[2] * t[3]};
#pragma unroll
            for (int s = 0; s < 4; ++s) pf[h][s].v[i] = from_f32<T>(on ? b[s] : 0.f);
        }
    }
}

template <typename T> __device__ __forceinline__ void zero_frag(F8<T> &f)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = from_f32<T>(0.f);
}

// Value rows y_j of CT tokens: [v | 1 | 0] (DVAL = false) or the ratio-rule
// gradient rows [dO/m | -(dO . o)/m | 0] (DVAL = true, from dO, O and m).
// The CT x 8 (token, 8-column group) items are spread over the block's
// threads and staged in registers (prefetch of the next chunk); the store
// writes them column-major into vt[NCOL][CT] and/or token-major into
// vr[CT][VRS].  Rows past tend are zero.
constexpr int VRS = NCOL + 8;  // token-major value row stride

template <typename T, int CT, int NTHR, bool DVAL> struct VStage {
    static constexpr int ITEMS = (CT * 8 + NTHR - 1) / NTHR;
    F8<T> x[ITEMS];
    F8<T> o[DVAL ? ITEMS : 1];
    float m[ITEMS];
};

template <typename T, int CT, int NTHR, bool DVAL>
__device__ __forceinline__ void vstage_load(const ValSrc<T> &src, int64_t tok0, int64_t tend,
                                            VStage<T, CT, NTHR, DVAL> &vs)
{
#pragma unroll
    for (int it = 0; it < VStage<T, CT, NTHR, DVAL>::ITEMS; ++it) {
        const int e = threadIdx.x + it * NTHR;
        const int64_t tok = tok0 + (e >> 3);
        const int c0 = (e & 7) * 8;
        const bool ok = e < CT * 8 && tok < tend;
        vs.m[it] = 1.f;
        if (ok) {
            vs.x[it] = ld8<T>(src.V + tok * HD + c0);
        } else {
            zero_frag(vs.x[it]);
        }
        if constexpr (DVAL) {
            if (ok) {
                vs.o[it] = ld8<T>(src.O + tok * HD + c0);
                vs.m[it] = src.den[tok];
            } else {
                zero_frag(vs.o[it]);
            }
        }
    }
}

template <typename T, int CT, int NTHR, bool DVAL>
__device__ __forceinline__ void vstage_store(const VStage<T, CT, NTHR, DVAL> &vs, int64_t tok0,
                                             int64_t tend, T *vt, T *vr)
{
#pragma unroll
    for (int it = 0; it < VStage<T, CT, NTHR, DVAL>::ITEMS; ++it) {
        const int e = threadIdx.x + it * NTHR;
        const int j = (e >> 3) & (CT - 1), c0 = (e & 7) * 8;
        float y[8], extra;
        if constexpr (DVAL) {
            // the 8 items of a token sit in 8 consecutive lanes
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) dot += to_f32(vs.x[it].v[i]) * to_f32(vs.o[it].v[i]);
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 4);
            const float inv_m = __builtin_amdgcn_rcpf(vs.m[it]);
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = to_f32(vs.x[it].v[i]) * inv_m;
            extra = tok0 + j < tend ? -dot * inv_m : 0.f;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = to_f32(vs.x[it].v[i]);
            extra = tok0 + j < tend ? 1.f : 0.f;
        }
        if (e < CT * 8) {
            if (vt) {
#pragma unroll
                for (int i = 0; i < 8; ++i) vt[(c0 + i) * CT + j] = from_f32<T>(y[i]);
            }
            if (vr) {
                F8<T> f;
#pragma unroll
                for (int i = 0; i < 8; ++i) f.v[i] = from_f32<T>(y[i]);
                *reinterpret_cast<decltype(f.v) *>(vr + j * VRS + c0) = f.v;
            }
            if (c0 == 0) {
                // columns HD .. NCOL-1: the count (or dm) column, then zeros
#pragma unroll
                for (int c = HD; c < NCOL; ++c) {
                    const T val = from_f32<T>(c == HD ? extra : 0.f);
                    if (vt) vt[c * CT + j] = val;
                    if (vr) vr[j * VRS + c] = val;
                }
            }
        }
    }
}

// Feature-major fragments over one 16-token tile tj (K = 16: slots 4g + r).
template <typename T, int HT>
__device__ __forceinline__ void feat_frags4(const float *tb, int tstride, int L, int tj,
                                            F4<T> (&pf)[HT][4])
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int q = c16 >> 2, p = c16 & 3;
#pragma unroll
    for (int h = 0; h < HT; ++h) {
        const bool on = (w * HT + h) * 4 + q < L;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const floatx4 t = *reinterpret_cast<const floatx4 *>(
                tb + (tj * 16 + g * 4 + r) * tstride + (w * HT + h) * 16 + q * 4);
            const float a = 0.25f * ((p & 1) ? t[0] : 1.f) * ((p & 2) ? t[1] : 1.f);
            const float b[4] = {a, a * t[2], a * t[3], a * t[2] * t[3]};
#pragma unroll
            for (int s = 0; s < 4; ++s) pf[h][s].v[r] = from_f32<T>(on ? b[s] : 0.f);
        }
    }
}

// ---------------------------------------------------------------------------
// fused_sum_kernel: S_g = sum_{j in segment g} psi(x_j)^T y_j.
// LAYOUT bit 0: FxC state into st_f, bit 1: CxF state into st_c.
template <typename T, int NW, int HT, bool DVAL, int LAYOUT>
__global__ __launch_bounds__(NW * 64) void fused_sum_kernel(
    const T *__restrict__ X, ValSrc<T> vsrc, const float *__restrict__ W, int L, Squash sq,
    int64_t N, int seg, int64_t nseg, float *__restrict__ st_f, float *__restrict__ st_c)
{
    constexpr int CT = 32, NTT = 2;
    constexpr int TSTR = NW * HT * 16 + 4;
    constexpr bool FXC = LAYOUT & 1, CXF = LAYOUT & 2;
    __shared__ __attribute__((aligned(16))) float tb[CT * TSTR];
    __shared__ __attribute__((aligned(16))) T vt[NCOL * CT];
    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const T *Xh = X + bh * N * HD;
    ValSrc<T> vh = vsrc;
    vh.V += bh * N * HD;
    if (DVAL) {
        vh.O += bh * N * HD;
        vh.den += bh * N;
    }
    WFrag<T, HT> wf;
    load_wfrag<T, HT>(W, L * NP, wf);
    floatx4 af[FXC ? HT : 1][4][NT], ac[CXF ? HT : 1][4][NT];
#pragma unroll
    for (int h = 0; h < HT; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                if (FXC) af[h][s][ct] = {0.f, 0.f, 0.f, 0.f};
                if (CXF) ac[h][s][ct] = {0.f, 0.f, 0.f, 0.f};
            }
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(N, t_begin + seg);
    F8<T> xk[NTT][2];
    VStage<T, CT, NW * 64, DVAL> vs;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) load_xfrag<T>(Xh, t_begin + tt * 16 + c16, t_end, xk[tt]);
    vstage_load<T, CT, NW * 64, DVAL>(vh, t_begin, t_end, vs);
    for (int64_t tok0 = t_begin; tok0 < t_end; tok0 += CT) {
        floatx4 tk[NTT][HT], sd[HT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) hash_tile<T, HT, false>(xk[tt], wf, sq, tk[tt], sd);
        lds_barrier();  // previous chunk's LDS reads are done
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int h = 0; h < HT; ++h)
                *reinterpret_cast<floatx4 *>(tb + (tt * 16 + c16) * TSTR + (w * HT + h) * 16 +
                                             g * 4) = tk[tt][h];
        vstage_store<T, CT, NW * 64, DVAL>(vs, tok0, t_end, vt, nullptr);
        const int64_t nx = tok0 + CT;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) load_xfrag<T>(Xh, nx + tt * 16 + c16, t_end, xk[tt]);
        vstage_load<T, CT, NW * 64, DVAL>(vh, nx, t_end, vs);
        lds_barrier();
        // tokens past t_end have psi_0 = 1/4 but zero value rows
        F8<T> pf[HT][4];
        feat_frags<T, HT>(tb, TSTR, L, pf);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const F8<T> vb = ld8<T>(vt + (ct * 16 + c16) * CT + g * 8);
#pragma unroll
            for (int h = 0; h < HT; ++h)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (FXC) mma(af[h][s][ct], pf[h][s], vb);
                    if (CXF) mma(ac[h][s][ct], vb, pf[h][s]);
                }
        }
    }
    const int64_t blk = (bh * (nseg + 1) + sg) * (int64_t)(NW * HT * 64 * NCOL);
#pragma unroll
    for (int h = 0; h < HT; ++h)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const int64_t o = blk + st_idx(w, h * 4 + s, ct, lane, 4 * HT);
                if (FXC) *reinterpret_cast<floatx4 *>(st_f + o) = af[h][s][ct];
                if (CXF) *reinterpret_cast<floatx4 *>(st_c + o) = ac[h][s][ct];
            }
}

// ---------------------------------------------------------------------------
// fused_walk_kernel: rows "r" read an FxC state built from rows "w" and
// value rows y, in chunks of 32 tokens.
//   BWD = false: r = queries, w = keys, y = [v | 1]; token order; intra mask
//                w <= r; output O = n / m and den = m.
//   BWD = true:  r = keys, w = queries, y = [dO/m | dm]; reverse order; intra
//                mask w >= r; output dV = n[:, :d].
template <typename T, int NW, int HT, bool CAUSAL, bool BWD>
__global__ __launch_bounds__(NW * 64) void fused_walk_kernel(
    const T *__restrict__ R, const T *__restrict__ Wr, ValSrc<T> vsrc,
    const float *__restrict__ W, int L, Squash sq, int64_t N, int seg, int64_t nseg,
    const float *__restrict__ st, T *__restrict__ Out, float *__restrict__ den)
{
    constexpr int CT = 32, NTT = 2;
    constexpr int TSTR = NW * HT * 16 + 4;  // t rows (fp32)
    constexpr int ASTR = CT + 8;            // score rows (T)
    constexpr int SSTR = CT + 1;            // score partial rows (fp32)
    constexpr int RSTR = NCOL + 4;          // output partial rows (fp32)
    // score partials are written before a chunk's first barrier while other
    // waves may still read the previous chunk's output partials: no aliasing
    __shared__ __attribute__((aligned(16))) float tb[CAUSAL ? CT * TSTR : 4];
    __shared__ __attribute__((aligned(16))) T vt[CAUSAL ? NCOL * CT : 8];
    __shared__ __attribute__((aligned(16))) T abuf[CAUSAL ? CT * ASTR : 8];
    __shared__ __attribute__((aligned(16))) float scp[CAUSAL ? NW * CT * SSTR : 4];
    __shared__ __attribute__((aligned(16))) float red[NW * CT * RSTR];

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const T *Rh = R + bh * N * HD;
    const T *Wh = Wr + bh * N * HD;
    ValSrc<T> vh = vsrc;
    vh.V += bh * N * HD;
    if (BWD) {
        vh.O += bh * N * HD;
        vh.den += bh * N;
    }
    T *Oh = Out + bh * N * HD;
    float *denh = BWD ? nullptr : den + bh * N;
    WFrag<T, HT> wf;
    load_wfrag<T, HT>(W, L * NP, wf);
    floatx4 acc[HT][4][NT];
    {
        const float *src =
            st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(NW * HT * 64 * NCOL);
#pragma unroll
        for (int h = 0; h < HT; ++h)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    acc[h][s][ct] = *reinterpret_cast<const floatx4 *>(
                        src + st_idx(w, h * 4 + s, ct, lane, 4 * HT));
    }
    bool on[HT];
#pragma unroll
    for (int h = 0; h < HT; ++h) on[h] = (w * HT + h) * 4 + g < L;
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(N, t_begin + seg);
    const int64_t nch = (t_end - t_begin + CT - 1) / CT;
    auto chunk0 = [&](int64_t ci) { return t_begin + (BWD ? nch - 1 - ci : ci) * CT; };
    F8<T> xq[NTT][2], xk[NTT][2];
    VStage<T, CT, NW * 64, BWD> vs;
    {
        const int64_t c0 = chunk0(0);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            load_xfrag<T>(Rh, c0 + tt * 16 + c16, t_end, xq[tt]);
            if (CAUSAL) load_xfrag<T>(Wh, c0 + tt * 16 + c16, t_end, xk[tt]);
        }
        if (CAUSAL) vstage_load<T, CT, NW * 64, BWD>(vh, c0, t_end, vs);
    }

    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t tok0 = chunk0(ci);
        F8<T> psq[NTT][HT][2], psk[NTT][HT][2];
        {
            floatx4 tq[NTT][HT], tk[NTT][HT], sd[HT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                hash_tile<T, HT, false>(xq[tt], wf, sq, tq[tt], sd);
                if (CAUSAL) hash_tile<T, HT, false>(xk[tt], wf, sq, tk[tt], sd);
            }
            if (CAUSAL) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int h = 0; h < HT; ++h)
                        *reinterpret_cast<floatx4 *>(tb + (tt * 16 + c16) * TSTR +
                                                     (w * HT + h) * 16 + g * 4) = tk[tt][h];
                vstage_store<T, CT, NW * 64, BWD>(vs, tok0, t_end, vt, nullptr);
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int h = 0; h < HT; ++h) {
                    walsh_frags<T>(tq[tt][h], on[h], psq[tt][h][0], psq[tt][h][1]);
                    if (CAUSAL) walsh_frags<T>(tk[tt][h], on[h], psk[tt][h][0], psk[tt][h][1]);
                }
        }
        if (ci + 1 < nch) {  // prefetch the next chunk
            const int64_t nx = chunk0(ci + 1);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                load_xfrag<T>(Rh, nx + tt * 16 + c16, t_end, xq[tt]);
                if (CAUSAL) load_xfrag<T>(Wh, nx + tt * 16 + c16, t_end, xk[tt]);
            }
            if (CAUSAL) vstage_load<T, CT, NW * 64, BWD>(vh, nx, t_end, vs);
        }
        if (CAUSAL) {
            // intra-chunk scores s[i][j] (i: reader, j: writer), partial over this wave's tables
#pragma unroll
            for (int ti = 0; ti < NTT; ++ti)
#pragma unroll
                for (int tj = 0; tj < NTT; ++tj) {
                    if (BWD ? (tj < ti) : (tj > ti)) continue;
                    floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int h = 0; h < HT; ++h)
#pragma unroll
                        for (int k = 0; k < 2; ++k) mma(sacc, psq[ti][h][k], psk[tj][h][k]);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        scp[(w * CT + ti * 16 + g * 4 + r) * SSTR + tj * 16 + c16] = sacc[r];
                }
        }
        // inter-chunk readout, partial over this wave's tables
        floatx4 oacc[NTT][NT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) oacc[tt][ct] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < HT; ++h)
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const F8<T> b = acc2frag<T>(acc[h][2 * k][ct], acc[h][2 * k + 1][ct]);
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) mma(oacc[tt][ct], psq[tt][h][k], b);
                }
        lds_barrier();  // writer t, value rows and score partials are in LDS
        if (CAUSAL) {
            for (int e = threadIdx.x; e < CT * CT; e += NW * 64) {
                const int i = e / CT, j = e % CT;
                float s = 0.f;
                if (BWD ? (j >= i) : (j <= i)) {
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) s += scp[(ww * CT + i) * SSTR + j];
                }
                abuf[i * ASTR + j] = from_f32<T>(s);
            }
            lds_barrier();
            // masked scores x value rows: (token tile, column tile) pairs over the waves
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    if ((tt * NT + ct) % NW == w) {
                        const F8<T> a = ld8<T>(abuf + (tt * 16 + c16) * ASTR + g * 8);
                        const F8<T> b = ld8<T>(vt + (ct * 16 + c16) * CT + g * 8);
                        mma(oacc[tt][ct], a, b);
                    }
        }
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[(w * CT + tt * 16 + g * 4 + r) * RSTR + ct * 16 + c16] = oacc[tt][ct][r];
        if (CAUSAL) {
            // S += psi_w^T y
            F8<T> pf[HT][4];
            feat_frags<T, HT>(tb, TSTR, L, pf);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const F8<T> vb = ld8<T>(vt + (ct * 16 + c16) * CT + g * 8);
#pragma unroll
                for (int h = 0; h < HT; ++h)
#pragma unroll
                    for (int s = 0; s < 4; ++s) mma(acc[h][s][ct], pf[h][s], vb);
            }
        }
        lds_barrier();
        for (int e = threadIdx.x; e < CT * HD; e += NW * 64) {
            const int i = e / HD, c = e % HD;
            const int64_t tok = tok0 + i;
            if (tok < t_end) {
                float n = 0.f, m = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    n += red[(ww * CT + i) * RSTR + c];
                    if (!BWD) m += red[(ww * CT + i) * RSTR + HD];
                }
                if (BWD) {
                    Oh[tok * HD + c] = from_f32<T>(n);
                } else {
                    Oh[tok * HD + c] = from_f32<T>(n * __builtin_amdgcn_rcpf(m));
                    if (c == 0) denh[tok] = m;
                }
            }
        }
    }
}

// W fragments for dxh = du W (B operand, K = 16 hyperplanes of tile h:
// lane (d column 16 nt + c16, hyperplanes 4g + p)).
template <typename T, int HT> struct WBFrag;
template <int HT> struct WBFrag<bf16, HT> {
    F4<bf16> hi[HT][4], lo[HT][4];
};
template <int HT> struct WBFrag<float, HT> {
    F4<float> f[HT][4];
};

template <typename T, int HT>
__device__ __forceinline__ void load_wbfrag(const float *__restrict__ W, int LP, WBFrag<T, HT> &wb)
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int h = 0; h < HT; ++h)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int hp = (w * HT + h) * 16 + g * 4 + p;
                const float v = hp < LP ? W[hp * HD + nt * 16 + c16] : 0.f;
                if constexpr (sizeof(T) == 2) {
                    wb.hi[h][nt].v[p] = (bf16)v;
                    wb.lo[h][nt].v[p] = (bf16)(v - (float)wb.hi[h][nt].v[p]);
                } else {
                    wb.f[h][nt].v[p] = v;
                }
            }
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

// ---------------------------------------------------------------------------
// fused_dpsi_kernel: gradient of the rows "r" that read a CxF state built
// from rows "w" (values y_w), then back through the hash of the r rows.
//   dQ: r = queries (values D), w = keys (values [v | 1]), token order, mask w <= r.
//   dK: r = keys (values [v | 1]), w = queries (values D), reverse order, mask w >= r.
// Per chunk: dpsi_r = y_r S^T + E psi_w with E[i][j] = y_r(i) . y_w(j) masked;
// S += y_w^T psi_w; then dt, du = dt dt/du, dxh = du W and the normalisation.
template <typename T, int NW, int HT, bool CAUSAL, bool REVERSE, bool READER_D>
__global__ __launch_bounds__(NW * 64) void fused_dpsi_kernel(
    const T *__restrict__ Xr, const T *__restrict__ Xw, ValSrc<T> vr_src, ValSrc<T> vw_src,
    const float *__restrict__ W, int L, Squash sq, int64_t N, int seg, int64_t nseg,
    const float *__restrict__ st, T *__restrict__ dX)
{
    constexpr int CT = 32, NTT = 2;
    constexpr int TSTR = NW * HT * 16 + 4;
    constexpr int FW = 64 * HT;                      // features per wave
    constexpr int DSTR = (FW > HD ? FW : HD) + 4;    // per-wave dpsi / dxh rows (fp32)
    constexpr int XSTR = HD + 8;
    __shared__ __attribute__((aligned(16))) float tb[CAUSAL ? CT * TSTR : 4];
    __shared__ __attribute__((aligned(16))) T yr[CT * VRS];
    __shared__ __attribute__((aligned(16))) T yw[CAUSAL ? CT * VRS : 8];
    __shared__ __attribute__((aligned(16))) T ywt[CAUSAL ? NCOL * CT : 8];
    // raw reader rows, double-buffered: read after a chunk's last barrier
    __shared__ __attribute__((aligned(16))) T xbuf[2 * CT * XSTR];
    __shared__ __attribute__((aligned(16))) float dbuf[NW * CT * DSTR];

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const T *Rh = Xr + bh * N * HD;
    const T *Wh = Xw + bh * N * HD;
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
    float *db = dbuf + w * CT * DSTR;
    WFrag<T, HT> wf;
    load_wfrag<T, HT>(W, L * NP, wf);
    WBFrag<T, HT> wb;
    load_wbfrag<T, HT>(W, L * NP, wb);
    floatx4 acc[HT][4][NT];  // CxF state, tile (h, s, ct)
    {
        const float *src =
            st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(NW * HT * 64 * NCOL);
#pragma unroll
        for (int h = 0; h < HT; ++h)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    acc[h][s][ct] = *reinterpret_cast<const floatx4 *>(
                        src + st_idx(w, h * 4 + s, ct, lane, 4 * HT));
    }
    bool on[HT];
#pragma unroll
    for (int h = 0; h < HT; ++h) on[h] = (w * HT + h) * 4 + g < L;
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(N, t_begin + seg);
    const int64_t nch = (t_end - t_begin + CT - 1) / CT;
    auto chunk0 = [&](int64_t ci) { return t_begin + (REVERSE ? nch - 1 - ci : ci) * CT; };
    F8<T> xr[NTT][2], xw[NTT][2];
    VStage<T, CT, NW * 64, READER_D> vsr;
    VStage<T, CT, NW * 64, !READER_D> vsw;
    {
        const int64_t c0 = chunk0(0);
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            load_xfrag<T>(Rh, c0 + tt * 16 + c16, t_end, xr[tt]);
            if (CAUSAL) load_xfrag<T>(Wh, c0 + tt * 16 + c16, t_end, xw[tt]);
        }
        vstage_load<T, CT, NW * 64, READER_D>(vrh, c0, t_end, vsr);
        if (CAUSAL) vstage_load<T, CT, NW * 64, !READER_D>(vwh, c0, t_end, vsw);
    }
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t tok0 = chunk0(ci);
        floatx4 tr[NTT][HT], cr[NTT][HT];
        {
            floatx4 tw[NTT][HT], sd[HT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                hash_tile<T, HT, true>(xr[tt], wf, sq, tr[tt], cr[tt]);
                if (CAUSAL) hash_tile<T, HT, false>(xw[tt], wf, sq, tw[tt], sd);
            }
            if (CAUSAL) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int h = 0; h < HT; ++h)
                        *reinterpret_cast<floatx4 *>(tb + (tt * 16 + c16) * TSTR +
                                                     (w * HT + h) * 16 + g * 4) = tw[tt][h];
                vstage_store<T, CT, NW * 64, !READER_D>(vsw, tok0, t_end, ywt, yw);
            }
            vstage_store<T, CT, NW * 64, READER_D>(vsr, tok0, t_end, nullptr, yr);
            // raw reader rows for the normalisation backward (one wave stages them)
            if (w == 0) {
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
                        *reinterpret_cast<decltype(xr[tt][kb].v) *>(
                            xbuf + (ci & 1) * CT * XSTR + (tt * 16 + c16) * XSTR + kb * 32 +
                            g * 8) = xr[tt][kb].v;
            }
        }
        if (ci + 1 < nch) {  // prefetch the next chunk
            const int64_t nx = chunk0(ci + 1);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                load_xfrag<T>(Rh, nx + tt * 16 + c16, t_end, xr[tt]);
                if (CAUSAL) load_xfrag<T>(Wh, nx + tt * 16 + c16, t_end, xw[tt]);
            }
            vstage_load<T, CT, NW * 64, READER_D>(vrh, nx, t_end, vsr);
            if (CAUSAL) vstage_load<T, CT, NW * 64, !READER_D>(vwh, nx, t_end, vsw);
        }
        lds_barrier();

        // dpsi_r tiles (tt, h, s): lane (feature c16 of tile (h, s), reader tokens 4g + r)
        floatx4 dacc[NTT][HT][4];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int h = 0; h < HT; ++h)
#pragma unroll
                for (int s = 0; s < 4; ++s) dacc[tt][h][s] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            F4<T> ya[NTT];
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
                ya[tt] = ld4<T>(yr + (tt * 16 + c16) * VRS + ct * 16 + g * 4);
#pragma unroll
            for (int h = 0; h < HT; ++h)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const F4<T> b = acc2frag4<T>(acc[h][s][ct]);
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) mma(dacc[tt][h][s], ya[tt], b);
                }
        }
        if (CAUSAL) {
#pragma unroll
            for (int tj = 0; tj < NTT; ++tj) {
                F4<T> pf[HT][4];
                feat_frags4<T, HT>(tb, TSTR, L, tj, pf);
#pragma unroll
                for (int ti = 0; ti < NTT; ++ti) {
                    if (REVERSE ? (tj < ti) : (tj > ti)) continue;
                    // E^T tile: lane (reader token 16 ti + c16, writer tokens 16 tj + 4g + r)
                    floatx4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < NT; ++kc)
                        mma(e, ld4<T>(yw + (tj * 16 + c16) * VRS + kc * 16 + g * 4),
                            ld4<T>(yr + (ti * 16 + c16) * VRS + kc * 16 + g * 4));
                    F4<T> ef;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = ti * 16 + c16, j = tj * 16 + g * 4 + r;
                        ef.v[r] = from_f32<T>((REVERSE ? (j >= i) : (j <= i)) ? e[r] : 0.f);
                    }
#pragma unroll
                    for (int h = 0; h < HT; ++h)
#pragma unroll
                        for (int s = 0; s < 4; ++s) mma(dacc[ti][h][s], ef, pf[h][s]);
                }
                // S += y_w^T psi_w for the writer tokens of tile tj
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) {
                    const F4<T> a = ld4<T>(ywt + (ct * 16 + c16) * CT + tj * 16 + g * 4);
#pragma unroll
                    for (int h = 0; h < HT; ++h)
#pragma unroll
                        for (int s = 0; s < 4; ++s) mma(acc[h][s][ct], a, pf[h][s]);
                }
            }
        }
        // dpsi into this wave's LDS rows: row = reader token, column = 16 (table) + S
        {
            const int q = c16 >> 2, p = c16 & 3;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int h = 0; h < HT; ++h)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            db[(tt * 16 + g * 4 + r) * DSTR + h * 64 + q * 16 + s * 4 + p] =
                                dacc[tt][h][s][r];
        }
        // hash backward of the reader rows: lane (token c16, table g of tile h);
        // dxh partials over this wave's hyperplanes overwrite the same LDS
        // rows once every dpsi of the wave has been read
        floatx4 xacc[NTT][4];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            F4<T> duf[HT];
#pragma unroll
            for (int h = 0; h < HT; ++h) {
                float dp[16];
                const float *src = db + (tt * 16 + c16) * DSTR + h * 64 + g * 16;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const floatx4 v = *reinterpret_cast<const floatx4 *>(src + 4 * k);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dp[4 * k + i] = v[i];
                }
                float dt[4];
                walsh_grad(dp, tr[tt][h], dt);
#pragma unroll
                for (int p = 0; p < 4; ++p) duf[h].v[p] = from_f32<T>(on[h] ? dt[p] * cr[tt][h][p] : 0.f);
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                xacc[tt][nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int h = 0; h < HT; ++h) {
                    if constexpr (sizeof(T) == 2) {
                        mma(xacc[tt][nt], duf[h], wb.hi[h][nt]);
                        mma(xacc[tt][nt], duf[h], wb.lo[h][nt]);
                    } else {
                        mma(xacc[tt][nt], duf[h], wb.f[h][nt]);
                    }
                }
            }
        }
        // dxh partial over this wave's hyperplanes (same LDS rows, after the reads above)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    db[(tt * 16 + g * 4 + r) * DSTR + nt * 16 + c16] = xacc[tt][nt][r];
        lds_barrier();
        // sum over waves, then the normalisation backward (16 threads per row)
        for (int base = 0; base < CT * 16; base += NW * 64) {
            const int e = base + threadIdx.x;
            const int i = (e >> 4) & (CT - 1), part = e & 15;
            const int64_t tok = tok0 + i;
            const bool ok = e < CT * 16 && tok < t_end;
            float x[4], dh[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                x[c] = to_f32(xbuf[(ci & 1) * CT * XSTR + i * XSTR + part * 4 + c]);
                float sacc = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) sacc += dbuf[(ww * CT + i) * DSTR + part * 4 + c];
                dh[c] = sacc;
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
            if (ok) {
                const float nrm = sqrtf(ss);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float rv;
                    if (nrm > 1e-12f) {
                        const float inv = 1.0f / nrm;
                        rv = (dh[c] - dot * inv * inv * x[c]) * inv;
                    } else {
                        rv = dh[c] * 1e12f;
                    }
                    dXh[tok * HD + part * 4 + c] = from_f32<T>(rv);
                }
            }
        }
    }
}

}  // namespace race
