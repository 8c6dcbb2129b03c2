// race_fwd.h -- sketch kernels of RACE attention (gfx950): hashing, segment
// sums, the scan over segments and the chunked readout.  The backward reuses
// them with the roles of queries and keys swapped.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (soft
// hashing over hypercube corners, per-bucket sums A and B, the ratio readout)
// and §2.3 (causal streaming sums A_cum, B_cum); gist.science/es/... §2
// (kernel on normalised vectors).
//
// Forward pipeline (B*H heads of N tokens, segments of `seg` tokens):
//   hash_kernel     t = tanh(tanh(W x / |x|) / tau) for every row of Q and K
//   seg_sum_kernel  per segment g: S_g = sum_{j in g} psi(k_j)^T [v_j | 1]
//   scan_reduce_kernel / scan_apply_kernel
//                   exclusive prefix (or suffix) of S_g over the segments of a
//                   head, plus the head total (used by the non-causal readout),
//                   in groups of consecutive segments: group totals first,
//                   then each group rescans from the totals before it
//   readout_kernel  per segment, in sub-chunks of 16 tokens: the running state
//                   S (MFMA accumulators) is read by the chunk's queries, the
//                   causal intra-chunk term tril(psi_Q psi_K^T) [V | 1] is
//                   added, then S += psi_K^T [V | 1]; o = n / m, den = m.
// The chunked causal form is an exact re-association of the streaming
// recurrence: query i reads the sum over keys j <= i.
//
// Work split: wave w of a workgroup owns tables [8w, 8w+8), i.e. features
// [128w, 128w+128) and those rows of the state S[F][80] (80 = 64 value
// columns, the count column, zero padding).
//
// Layouts of the state in registers (16x16 accumulator tiles, 4 floats/lane):
//   "FxC"  tile (mt, nt): rows = features, columns = value columns
//          lane l holds feature 16*mt + 4*(l/16) + r, column 16*nt + l%16
//   "CxF"  tile (ct, ft): rows = value columns, columns = features
//          lane l holds column 16*ct + 4*(l/16) + r, feature 16*ft + l%16
// A segment state block in global memory is [wave][8][5][64 lanes][4 floats]
// in the producing kernel's layout; the scan is layout-agnostic.
#pragma once
#include "race_common.h"

namespace race {

// Value rows of the sketch.  With O == nullptr: [v | 1 | 0...] from V.
// Otherwise the ratio-rule gradient rows of the backward:
//   [dO/m | -(dO . o)/m | 0...] from V = dO, O and den = m.
template <typename T> struct ValSrc {
    const T *V;
    const T *O;
    const float *den;
    // rows of 128 elements (two passes of 64 value columns): the gradient
    // values' last column -(dO . o)/m over the whole row, precomputed, or null
    // (the pass without the column: zero)
    const float *dm = nullptr;
};

// ---------------------------------------------------------------------------
// hash_kernel: per row x of X and table l, t[p] = tanh(tanh(u_p / |x|) / tau)
// (inv_tau = 0: hard hashing, t[p] = +1 if u_p >= 0 else -1, the tau -> 0 limit)
// with u = W x (raw row; |x| clamped at 1e-12).  U^T = W X^T on MFMA
// (M = hyperplanes, N = 16 rows, K = d); bf16 inputs use W = W_hi + W_lo.
// CHAIN also stores dt/du = ((1 - t^2)/tau) (1 - z^2), z = tanh(u / |x|),
// after the 4 t values of each table (8 floats per table instead of 4).
template <typename T, bool CHAIN>
__global__ __launch_bounds__(256) void hash_kernel(const T *__restrict__ X, int64_t rows,
                                                   const float *__restrict__ W, int L,
                                                   float inv_tau, float *__restrict__ tout)
{
    constexpr int TS = CHAIN ? 2 * NP : NP;
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    const int64_t ntile = (rows + 15) / 16;
    const int LP = L * NP;
    const int mtiles = (LP + 15) / 16;
    for (int64_t tile = (int64_t)blockIdx.x * 4 + wave_id(); tile < ntile;
         tile += (int64_t)gridDim.x * 4) {
        const int64_t row = tile * 16 + c16;
        const bool valid = row < rows;
        F8<T> xb[2];
        float ss = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (valid) {
                xb[kb] = ld8<T>(X + row * HD + kb * 32 + g * 8);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xb[kb].v[i] = from_f32<T>(0.f);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = to_f32(xb[kb].v[i]);
                ss += x * x;
            }
        }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float inv_norm = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
        for (int mt = 0; mt < mtiles; ++mt) {
            const int hp = mt * 16 + c16;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float w[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    w[i] = hp < LP ? W[(int64_t)hp * HD + kb * 32 + g * 8 + i] : 0.f;
                if constexpr (sizeof(T) == 2) {
                    F8<bf16> hi, lo;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        hi.v[i] = (bf16)w[i];
                        lo.v[i] = (bf16)(w[i] - (float)hi.v[i]);
                    }
                    mma(acc, hi, xb[kb]);
                    mma(acc, lo, xb[kb]);
                } else {
                    F8<float> wf;
#pragma unroll
                    for (int i = 0; i < 8; ++i) wf.v[i] = w[i];
                    mma(acc, wf, xb[kb]);
                }
            }
            // acc[r]: hyperplane 16*mt + 4*g + r = table 4*mt + g, p = r, row c16
            const int l = mt * 4 + g;
            if (valid && l < L) {
                floatx4 t, sd;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float z = tanhf(acc[r] * inv_norm);
                    // inv_tau = 0: hard hashing, the tau -> 0 limit t = sign(z) (+1 at 0)
                    t[r] = inv_tau == 0.f ? (acc[r] >= 0.f ? 1.f : -1.f) : tanhf(z * inv_tau);
                    sd[r] = (1.f - t[r] * t[r]) * inv_tau * (1.f - z * z);
                }
                float *dst = tout + (row * L + l) * TS;
                *reinterpret_cast<floatx4 *>(dst) = t;
                if (CHAIN) *reinterpret_cast<floatx4 *>(dst + NP) = sd;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Shared pieces of the segment kernels.

// psi^T for the wave's tables into pt[F][CH] (feature-major), tokens
// tok0 .. tok0+15 of one head; tokens >= tend give zero columns.
// Lane = (table, feature group of 4, token half).
template <typename T>
__device__ __forceinline__ void expand_t(const float *__restrict__ t, int ts, int64_t tok0,
                                         int64_t tend, int L, T *pt)
{
    const int lane = lane_id(), w = wave_id();
    const int tl = lane >> 3, fg = (lane >> 1) & 3, th = lane & 1;
    const int l = w * TPW + tl;
    float vals[4][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t tok = tok0 + th * 8 + j;
        float psi[4] = {0.f, 0.f, 0.f, 0.f};
        if (l < L && tok < tend) {
            const floatx4 tv = *reinterpret_cast<const floatx4 *>(t + (tok * L + l) * ts);
            walsh4(tv, fg, psi);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) vals[s][j] = psi[s];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        T *dst = pt + (l * NR + fg * 4 + s) * CH + th * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[j] = from_f32<T>(vals[s][j]);
    }
}

// psi for the wave's tables into pr[CH][F] (token-major).  Lane = (token, table pair).
template <typename T>
__device__ __forceinline__ void expand_r(const float *__restrict__ t, int ts, int64_t tok0,
                                         int64_t tend, int L, int F, T *pr)
{
    const int lane = lane_id(), w = wave_id();
    const int tokl = lane >> 2, tp = lane & 3;
    const int64_t tok = tok0 + tokl;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int l = w * TPW + tp * 2 + h;
        float psi[16];
        if (l < L && tok < tend) {
            const floatx4 tv = *reinterpret_cast<const floatx4 *>(t + (tok * L + l) * ts);
            walsh16(tv, psi);
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) psi[s] = 0.f;
        }
        T *dst = pr + tokl * F + l * NR;
#pragma unroll
        for (int s = 0; s < 16; ++s) dst[s] = from_f32<T>(psi[s]);
    }
}

// Value rows of tokens tok0 .. tok0+15 into vt[NCOL][CH] (column-major,
// optional) and vr[CH][NCOL] (token-major, optional); tokens >= tend give
// zero rows.  16 threads per token, 4 value columns each.
template <typename T, bool DVAL>
__device__ __forceinline__ void load_vals(const ValSrc<T> &src, int64_t tok0, int64_t tend,
                                          T *vt, T *vr)
{
    for (int base = 0; base < CH * 16; base += blockDim.x) {
        const int e = base + threadIdx.x;
        const int j = (e >> 4) & (CH - 1), part = e & 15;
        const int64_t tok = tok0 + j;
        const bool ok = (e < CH * 16) && tok < tend;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        float extra = 0.f;  // column HD
        if (ok) {
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = to_f32(src.V[tok * HD + part * 4 + c]);
        }
        if (DVAL) {
            float dot = 0.f, inv_m = 0.f;
            if (ok) {
#pragma unroll
                for (int c = 0; c < 4; ++c) dot += x[c] * to_f32(src.O[tok * HD + part * 4 + c]);
                inv_m = 1.0f / src.den[tok];
            }
            dot += __shfl_xor(dot, 8);
            dot += __shfl_xor(dot, 4);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 1);
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] *= inv_m;
            extra = -dot * inv_m;
        } else {
            extra = ok ? 1.f : 0.f;
        }
        if (e < CH * 16) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int col = part * 4 + c;
                if (vt) vt[col * CH + j] = from_f32<T>(x[c]);
                if (vr) vr[j * NCOL + col] = from_f32<T>(x[c]);
            }
            // columns HD .. NCOL-1: part p covers column HD + p
            const int col = HD + part;
            const float y = part == 0 ? extra : 0.f;
            if (vt) vt[col * CH + j] = from_f32<T>(y);
            if (vr) vr[j * NCOL + col] = from_f32<T>(y);
        }
    }
}

// FxC state += psi^T Y (wave's feature rows): pt[F][CH], vt[NCOL][CH]
template <typename T>
__device__ __forceinline__ void update_fxc(floatx4 (&acc)[MT][NT], const T *pt, const T *vt)
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    F4<T> vb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vb[nt] = ld4<T>(vt + (nt * 16 + c16) * CH + g * 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const F4<T> a = ld4<T>(pt + (w * FPW + mt * 16 + c16) * CH + g * 4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) mma(acc[mt][nt], a, vb[nt]);
    }
}

// CxF state += Y^T psi (wave's feature columns): vt[NCOL][CH], pt[F][CH]
template <typename T>
__device__ __forceinline__ void update_cxf(floatx4 (&acc)[NT][MT], const T *pt, const T *vt)
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    F4<T> pb[MT];
#pragma unroll
    for (int ft = 0; ft < MT; ++ft) pb[ft] = ld4<T>(pt + (w * FPW + ft * 16 + c16) * CH + g * 4);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
        const F4<T> a = ld4<T>(vt + (ct * 16 + c16) * CH + g * 4);
#pragma unroll
        for (int ft = 0; ft < MT; ++ft) mma(acc[ct][ft], a, pb[ft]);
    }
}

__device__ __forceinline__ int64_t st_index(int w, int a, int b, int lane)
{
    return ((((int64_t)w * MT + a) * NT + b) * 64 + lane) * 4;
}

// ---------------------------------------------------------------------------
// seg_sum_kernel: S_g = sum_{j in segment g} psi(x_j)^T y_j, in layout FxC
// (CXF = false, stored as [w][mt][nt]) or CxF (CXF = true, stored [w][ft][ct]).
template <typename T, int NW, bool CXF, bool DVAL>
__global__ __launch_bounds__(NW * 64) void seg_sum_kernel(const float *__restrict__ t, int ts,
                                                          ValSrc<T> vs, int64_t N, int L,
                                                          int seg, int64_t nseg,
                                                          float *__restrict__ st, Lens ls)
{
    __shared__ __attribute__((aligned(16))) T pt[NW * FPW * CH];
    __shared__ __attribute__((aligned(16))) T vt[NCOL * CH];
    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id();
    const float *th = t + bh * N * L * ts;
    ValSrc<T> vh = vs;
    vh.V += bh * N * HD;
    if (DVAL) {
        vh.O += bh * N * HD;
        vh.den += bh * N;
    }
    floatx4 acc[MT][NT];  // CxF reuses it as [ft][ct]
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b) acc[a][b] = {0.f, 0.f, 0.f, 0.f};
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(valid_rows(ls, bh, N), t_begin + seg);
    for (int64_t tok0 = t_begin; tok0 < t_end; tok0 += CH) {
        __syncthreads();
        load_vals<T, DVAL>(vh, tok0, t_end, vt, nullptr);
        expand_t<T>(th, ts, tok0, t_end, L, pt);
        __syncthreads();
        if (CXF) {
            const int g = lane >> 4, c16 = lane & 15;
            F4<T> pb[MT];
#pragma unroll
            for (int ft = 0; ft < MT; ++ft)
                pb[ft] = ld4<T>(pt + (w * FPW + ft * 16 + c16) * CH + g * 4);
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const F4<T> a = ld4<T>(vt + (ct * 16 + c16) * CH + g * 4);
#pragma unroll
                for (int ft = 0; ft < MT; ++ft) mma(acc[ft][ct], a, pb[ft]);
            }
        } else {
            update_fxc<T>(acc, pt, vt);
        }
    }
    float *out = st + (bh * (nseg + 1) + sg) * (int64_t)(NW * FPW * NCOL);
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < NT; ++b)
            *reinterpret_cast<floatx4 *>(out + st_index(w, a, b, lane)) = acc[a][b];
}

// Scan over segments: per head, st[g] <- sum of st[g'] over g' < g
// (reverse = 0) or g' > g (reverse = 1); st[nseg] <- total.  The segments
// are split into G groups of consecutive segments; scan_reduce_kernel writes
// the group totals to tmp[head][G][elems], scan_apply_kernel rescans each
// group starting from the totals of the groups before (after) it.
static __global__ __launch_bounds__(256) void scan_reduce_kernel(const float *__restrict__ st,
                                                          float *__restrict__ tmp, int64_t nseg,
                                                          int64_t elems, int G)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= elems) return;
    const int grp = blockIdx.y;
    const int64_t bh = blockIdx.z;
    const float *p = st + bh * (nseg + 1) * elems + e;
    const int64_t s0 = grp * nseg / G, s1 = (grp + 1) * nseg / G;
    constexpr int U = 8;  // loads in flight per thread
    float sum = 0.f;
    int64_t g = s0;
    for (; g + U <= s1; g += U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[(g + u) * elems];
#pragma unroll
        for (int u = 0; u < U; ++u) sum += v[u];
    }
    for (; g < s1; ++g) sum += p[g * elems];
    tmp[(bh * G + grp) * elems + e] = sum;
}

static __global__ __launch_bounds__(256) void scan_apply_kernel(float *__restrict__ st,
                                                         const float *__restrict__ tmp,
                                                         int64_t nseg, int64_t elems, int G,
                                                         int reverse)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= elems) return;
    const int grp = blockIdx.y;
    const int64_t bh = blockIdx.z;
    float *p = st + bh * (nseg + 1) * elems + e;
    float run = 0.f;
    for (int q = 0; q < G; ++q)
        if (reverse ? q > grp : q < grp) run += tmp[(bh * G + q) * elems + e];
    const int64_t s0 = grp * nseg / G, s1 = (grp + 1) * nseg / G, n = s1 - s0;
    constexpr int U = 8;
    int64_t i = 0;
    for (; i + U <= n; i += U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = reverse ? s1 - 1 - (i + u) : s0 + i + u;
            v[u] = p[g * elems];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = reverse ? s1 - 1 - (i + u) : s0 + i + u;
            p[g * elems] = run;
            run += v[u];
        }
    }
    for (; i < n; ++i) {
        const int64_t g = reverse ? s1 - 1 - i : s0 + i;
        const float v = p[g * elems];
        p[g * elems] = run;
        run += v;
    }
    if (grp == (reverse ? 0 : G - 1)) p[nseg * elems] = run;
}

// ---------------------------------------------------------------------------
// readout_kernel: rows "r" read an FxC state built from rows "w" and values y.
//   BWD = false (forward): r = queries, w = keys, y = [v | 1], token order,
//            intra mask w <= r, output O = n / m and den = m.
//   BWD = true (dV):       r = keys, w = queries, y = [dO/m | dm], reverse
//            token order, intra mask w >= r, output n[:, :d] = dV.
template <typename T, int NW, bool CAUSAL, bool BWD>
__global__ __launch_bounds__(NW * 64) void readout_kernel(
    const float *__restrict__ tr, const float *__restrict__ tw, int ts, ValSrc<T> vs, int64_t N,
    int L, int seg, int64_t nseg, const float *__restrict__ st, T *__restrict__ Out,
    float *__restrict__ den, Lens ls, Part part = Part{nullptr, nullptr}, int pmode = PART_NONE)
{
    constexpr int F = NW * FPW;
    __shared__ __attribute__((aligned(16))) T pr[CH * F];
    __shared__ __attribute__((aligned(16))) T pw[CAUSAL ? F * CH : 8];
    __shared__ __attribute__((aligned(16))) T vt[CAUSAL ? NCOL * CH : 8];
    __shared__ __attribute__((aligned(16))) float scp[CAUSAL ? NW : 1][CH * CH];
    __shared__ __attribute__((aligned(16))) T abuf[CAUSAL ? CH * CH : 8];
    __shared__ __attribute__((aligned(16))) float red[NW][CH * NCOL];
    __shared__ float mrow[CH];  // table passes: each row's denominator, partial sums included

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const float *trh = tr + bh * N * L * ts;
    const float *twh = tw + bh * N * L * ts;
    ValSrc<T> vh = vs;
    vh.V += bh * N * HD;
    if (BWD) {
        vh.O += bh * N * HD;
        vh.den += bh * N;
    }
    T *Outh = Out + bh * N * HD;
    float *denh = BWD ? nullptr : den + bh * N;

    floatx4 acc[MT][NT];
    {
        const float *src = st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(F * NCOL);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[mt][nt] = *reinterpret_cast<const floatx4 *>(src + st_index(w, mt, nt, lane));
    }
    const int64_t t_begin = sg * seg, t_end = min<int64_t>(valid_rows(ls, bh, N), t_begin + seg);
    const int64_t nch = (t_end - t_begin + CH - 1) / CH;
    for (int64_t ci = 0; ci < nch; ++ci) {
        const int64_t tok0 = t_begin + (BWD ? nch - 1 - ci : ci) * CH;
        __syncthreads();
        if (CAUSAL) {
            load_vals<T, BWD>(vh, tok0, t_end, vt, nullptr);
            expand_t<T>(twh, ts, tok0, t_end, L, pw);
        }
        expand_r<T>(trh, ts, tok0, t_end, L, F, pr);
        __syncthreads();

        // inter-chunk readout: partial over this wave's features
        floatx4 oacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[nt] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < MT / 2; ++kb) {
            const T *row = pr + c16 * F + w * FPW + kb * 32 + g * 4;
            const F8<T> a = ld4x2<T>(row, row + 16);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const F8<T> b = acc2frag<T>(acc[2 * kb][nt], acc[2 * kb + 1][nt]);
                mma(oacc[nt], a, b);
            }
        }
        if (CAUSAL) {
            // intra-chunk scores s[i][j] = psi_r(i) . psi_w(j), partial over the wave's features
            floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < MT / 2; ++kb) {
                const int f0 = w * FPW + kb * 32 + g * 8;
                const F8<T> a = ld8<T>(pr + c16 * F + f0);
                const F8<T> b = ld8s<T>(pw + f0 * CH + c16, CH);
                mma(sacc, a, b);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) scp[w][(g * 4 + r) * CH + c16] = sacc[r];
            __syncthreads();
            for (int e = threadIdx.x; e < CH * CH; e += NW * 64) {
                const int i = e / CH, j = e % CH;
                float s = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) s += scp[ww][e];
                const bool keep = BWD ? (j >= i) : (j <= i);
                abuf[e] = from_f32<T>(keep ? s : 0.f);
            }
            __syncthreads();
            // Y = masked scores x values, column tiles spread over the waves
            for (int nt = w; nt < NT; nt += NW) {
                const F4<T> a = ld4<T>(abuf + c16 * CH + g * 4);
                const F4<T> b = ld4<T>(vt + (nt * 16 + c16) * CH + g * 4);
                mma(oacc[nt], a, b);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[w][(g * 4 + r) * NCOL + nt * 16 + c16] = oacc[nt][r];
        __syncthreads();
        // table passes (L > 32): n (and m) of the tables so far are added
        // from fp32 partial rows [rows][64] (and [rows]); the first pass
        // stores its sums there, middle passes add theirs, the last one adds
        // the stored sums and writes the outputs
        float *pv = pmode != PART_NONE ? part.v + bh * N * HD : nullptr;
        if (!BWD && pmode != PART_NONE) {
            // each row's m once, before any thread updates the stored one
            if (threadIdx.x < CH && tok0 + (int64_t)threadIdx.x < t_end) {
                const int64_t tok = tok0 + threadIdx.x;
                float m = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) m += red[ww][threadIdx.x * NCOL + HD];
                float *pm = part.m + bh * N;
                if (pmode != PART_OUT) m += pm[tok];
                if (pmode != PART_IN) pm[tok] = m;
                mrow[threadIdx.x] = m;
            }
            __syncthreads();
        }
        for (int e = threadIdx.x; e < CH * HD; e += NW * 64) {
            const int i = e / HD, c = e % HD;
            const int64_t tok = tok0 + i;
            if (tok < t_end) {
                float n = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) n += red[ww][i * NCOL + c];
                if (pmode != PART_NONE) {
                    if (pmode != PART_OUT) n += pv[tok * HD + c];
                    if (pmode != PART_IN) {
                        pv[tok * HD + c] = n;
                        continue;
                    }
                }
                if (BWD) {
                    Outh[tok * HD + c] = from_f32<T>(n);
                } else {
                    float m = 0.f;
                    if (pmode == PART_NONE) {
#pragma unroll
                        for (int ww = 0; ww < NW; ++ww) m += red[ww][i * NCOL + HD];
                    } else {
                        m = mrow[i];
                    }
                    // m = 0 only under hard hashing (no colliding key): o = 0
                    Outh[tok * HD + c] = from_f32<T>(m != 0.f ? n / m : 0.f);
                    if (c == 0) denh[tok] = m;
                }
            }
        }
        if (CAUSAL) update_fxc<T>(acc, pw, vt);
    }
}

}  // namespace race
