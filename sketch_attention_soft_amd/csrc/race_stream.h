// race_stream.h -- the streaming form of RACE attention (gfx950): a persistent
// per-head state that tokens are appended to and read from, for inference
// (decode) after a prompt.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.3 (causal
// mode keeps running bucket sums and reads them at every step, so each step
// costs the same however long the prefix) and §2.2 (bucket sums A and B, the
// ratio readout).
//
// State of one head: S[f][c] for f < F = 16 L, c <= d (fp32, [F][d + 1]),
// d <= 64 (rows and W are read with their own length d; lane c < d of a wave
// holds column c):
//   S[f][c] = sum_j psi_f(k_j) v_j[c] (c < d),  S[f][d] = sum_j psi_f(k_j),
//   psi_{16 l + s}(x) = 2^(-P/2) prod_{p in s} t_{lp}(x)  (s: a subset of the
//   table's hyperplanes, bit p set when p is in it; 1/4 for P = 4),
//   t_{lp}(x) = tanh(tanh(<w_lp, x / max(|x|, 1e-12)>) / tau).
// For P < 4 the kernel keeps 16 rows per table: hyperplanes p >= P have zero
// W rows, so t = tanh(0) = 0 exactly and every row whose s contains one is
// zero.
// The corner weights of the pages are phi_lr = prod_p (1 + c_rp t_lp) / 2, so
// psi is their Walsh-Hadamard transform and psi(q).psi(k) = phi(q).phi(k): S
// holds the pages' bucket sums A and B in that basis, and a readout is
// [n | m] = psi(q) S, o = n / m, den = m.
//
// One kernel in three modes, over the tokens [b blk, (b + 1) blk) of a head:
//   ADD      S_b = sum over the block (from zero), to a partial buffer; the
//            partials are then added to the state in block order.
//   DECODE   token by token: S += psi(k_i)^T [v_i | 1], then o_i from
//            psi(q_i) S (one workgroup per head, the causal recurrence).
//   READOUT  o_i from psi(q_i) S for a fixed S (no append).
// Wave g of a workgroup owns the features [g FPT, (g + 1) FPT): lane c keeps
// S[f][c] of those features in registers for the whole block, and the count
// column S[f][d] is spread over the wave's lanes (feature g FPT + 64 z + lane
// in slot z).  Tokens go in tiles of TT: rows staged in LDS, projections and
// features of the tile in LDS, then every wave applies the tile to its slice
// of S.  The per-token work is the F x (d + 1) update and readout, in fp32
// vector arithmetic; the state (133 KB per head at L = 32) is read and
// written once per call.
#pragma once
#include "race_common.h"
#include "race_walk.h"

namespace race {

constexpr int SM_ADD = 0, SM_DECODE = 1, SM_READOUT = 2;
constexpr int S_XS = HD + 1;     // LDS row stride of staged rows and W (odd: no bank conflicts)

template <typename T> __device__ __forceinline__ float sload(const T *p) { return (float)*p; }

// sum over the 64 lanes of a wave (every lane active): rows of 16 through
// DPP, then the four row sums read out of lanes 0, 16, 32, 48 (uniform)
__device__ __forceinline__ float wave_sum(float x)
{
    const int r = __builtin_bit_cast(int, sum16(x));
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(r, 48)));
}

// MAXT threads = MAXT / 64 waves of FPT features: F <= FMAX = FPT MAXT / 64
// and L P <= FMAX P / 16 (the launch picks the instance that fits).  Tiles
// of S_TT tokens: TT, or with TT = 0 eight (four for L > 32 decode, for LDS);
// a decode of one token per head takes TT = 1, so that the projections of a
// tile are not formed for tokens it does not have.
template <typename T, int MODE, int FPT, int MAXT, int TT = 0>
__global__ __launch_bounds__(MAXT)
__attribute__((amdgpu_waves_per_eu(MODE != SM_DECODE && MAXT <= 512 ? 4 : 1))) void stream_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
    const float *__restrict__ W, int L, int P, int d, float inv_tau, int64_t N, int64_t blk,
    float *__restrict__ state, float *__restrict__ part, T *__restrict__ O, float *__restrict__ den)
{
    constexpr bool UPD = MODE != SM_READOUT, RD = MODE != SM_ADD;
    constexpr int NS = (UPD ? 1 : 0) + (RD ? 1 : 0);  // row sides: queries (if RD), then keys (if UPD)
    constexpr int KS = RD ? 1 : 0;                     // side of the keys
    constexpr int NWV = MAXT / 64, FMAX = FPT * NWV, LPMAX = FMAX / NR * NP;
    constexpr int ZP = (FPT + 63) / 64;                // count-column slots per lane
    constexpr int S_TT = TT > 0 ? TT : NS == 2 && FMAX > 512 ? 4 : 8;  // tokens per tile
    __shared__ float wl[LPMAX * S_XS];                 // W rows
    __shared__ float xr[NS][S_TT][S_XS];               // staged rows
    __shared__ float yv[UPD ? S_TT : 1][HD];           // staged v rows
    __shared__ float inrm[NS][S_TT];                   // 1 / max(|x|, 1e-12)
    __shared__ float tv[NS][S_TT][LPMAX];              // squashed projections t
    __shared__ float ps[NS][S_TT][FMAX];               // features psi (zero past F)
    __shared__ float pn[RD ? S_TT : 1][NWV][HD];       // partial readouts n of the waves
    __shared__ float pm[RD ? S_TT : 1][NWV];           // and of m

    const int LP = L * NP, F = L * NR, sc = d + 1;  // sc: state columns
    const float fscale = __builtin_sqrtf(__builtin_ldexpf(1.f, -P));  // 2^(-P/2): 1/4 for P = 4
    const int QN = (F + FPT - 1) / FPT;
    const int nthr = blockDim.x, tid = threadIdx.x;
    const int c = tid & 63, grp = tid >> 6, f0 = grp * FPT;
    const int64_t bh = blockIdx.y;
    const int64_t t_begin = (int64_t)blockIdx.x * blk, t_end = min(N, t_begin + blk);
    const int64_t row0 = bh * N;
    float *sh = state + bh * (int64_t)F * sc;
    // One decode token per head (TT = 1 instances, launched for N = 1 only):
    // the single tile's row elements are loaded first, beside W, and the
    // state after the rows are staged, so that one memory round trip comes
    // before the first barrier and the state arrives while the token is
    // hashed; the state is stored as soon as it is updated, under the readout.
    constexpr bool ONE = MODE == SM_DECODE && TT == 1;
    float r1q = 0.f, r1k = 0.f, r1v = 0.f;
    if constexpr (ONE) {
        if (tid < d && t_begin < t_end) {
            const int64_t off = (row0 + t_begin) * d + tid;
            r1q = sload(Q + off);
            r1k = sload(K + off);
            r1v = sload(V + off);
        }
    }

    // W rows in LDS: each thread issues all its loads before its stores, so
    // the staging costs one memory round trip (LP HD <= WPT nthr, since nthr =
    // 64 ceil(16 L / FPT))
    constexpr int WPT = FPT / 4;
    {
        float wv[WPT];
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            // internal hyperplane h = 4 l + p <- W row P l + p (p < P), else zero
            const int e = tid + j * nthr, h = e / HD, k = e % HD, p = h & 3;
            wv[j] = (e < LP * HD && k < d && p < P) ? W[((h >> 2) * P + p) * d + k] : 0.f;
        }
        // (e / HD < WPT nthr / 64 <= LPMAX: every store is in the array, and
        // those past L P rows store zeros)
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            const int e = tid + j * nthr;
            wl[(e / HD) * S_XS + e % HD] = wv[j];
        }
    }
    // The head's state through a buffer resource: row f, column c at byte
    // 4 (f sc + c).  Lanes c >= d take an offset past the resource, and rows
    // f >= F fall past it (F sc floats), so loads read zero and stores are
    // dropped without branches; the row step is a scalar offset.
    const int lane_off = c < d ? (f0 * sc + c) * 4 : OOB, rstep = sc * 4;
    const Rsrc rs = make_rsrc(sh, F * sc * 4);
    auto z_off = [&](int z) {
        const int f = f0 + 64 * z + c;
        return 64 * z + c < FPT && f < F ? (f * sc + d) * 4 : OOB;
    };
    float S[FPT], Z[ZP];
    auto load_state = [&]() {
#pragma unroll
        for (int i = 0; i < FPT; ++i)
            S[i] = MODE != SM_ADD
                       ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lane_off, i * rstep, 0))
                       : 0.f;
#pragma unroll
        for (int z = 0; z < ZP; ++z) Z[z] = MODE != SM_ADD ? bldf(rs, z_off(z)) : 0.f;
    };
    float *dst = MODE == SM_DECODE ? sh
                 : MODE == SM_ADD    ? part + ((int64_t)bh * gridDim.x + blockIdx.x) * (int64_t)F * sc
                                     : nullptr;
    auto store_state = [&]() {
        const Rsrc rd = make_rsrc(dst, F * sc * 4);
#pragma unroll
        for (int i = 0; i < FPT; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, S[i]), rd, lane_off, i * rstep, 0);
#pragma unroll
        for (int z = 0; z < ZP; ++z) bstf(Z[z], rd, z_off(z));
    };
    if constexpr (!ONE) load_state();

    for (int64_t tile = t_begin; tile < t_end; tile += S_TT) {
        const int nt = (int)min<int64_t>(S_TT, t_end - tile);
        // rows of the tile (zeros past the end)
        if constexpr (ONE) {
            if (tid < HD) {
                xr[0][0][tid] = r1q;
                xr[KS][0][tid] = r1k;
                yv[0][tid] = r1v;
            }
        } else
        for (int e = tid; e < S_TT * HD; e += nthr) {
            const int t = e / HD, k = e % HD;
            float q = 0.f, kk = 0.f, v = 0.f;
            if (t < nt && k < d) {  // zeros past column d
                const int64_t off = (row0 + tile + t) * d + k;
                if (RD) q = sload(Q + off);
                if (UPD) {
                    kk = sload(K + off);
                    v = sload(V + off);
                }
            }
            if (RD) xr[0][t][k] = q;
            if (UPD) {
                xr[KS][t][k] = kk;
                yv[t][k] = v;
            }
        }
        __syncthreads();
        if constexpr (ONE) load_state();
        // squared norms: wave w takes rows w, w + NWV, ...; lane k one element
        for (int r = grp; r < NS * nt; r += nthr >> 6) {
            const int side = r / nt, t = r % nt;
            const float ss = wave_sum(xr[side][t][c] * xr[side][t][c]);
            if (c == 0) inrm[side][t] = 1.f / fmaxf(sqrtf(ss), 1e-12f);
        }
        __syncthreads();
        // projections: thread (side, h) for all tokens of the tile
        for (int j = tid; j < NS * LP; j += nthr) {
            const int side = j / LP, h = j % LP;
            float u[S_TT];
#pragma unroll
            for (int t = 0; t < S_TT; ++t) u[t] = 0.f;
#pragma unroll 8
            for (int k = 0; k < HD; ++k) {
                const float wk = wl[h * S_XS + k];
#pragma unroll
                for (int t = 0; t < S_TT; ++t) u[t] = fmaf(wk, xr[side][t][k], u[t]);
            }
#pragma unroll
            for (int t = 0; t < S_TT; ++t)
                if (t < nt) tv[side][t][h] = tanhf(tanhf(u[t] * inrm[side][t]) * inv_tau);
        }
        __syncthreads();
        // features of the tile's tokens, zero past F up to the waves' end
        for (int e = tid; e < NS * nt * QN * FPT; e += nthr) {
            const int side = e / (nt * QN * FPT), r = e % (nt * QN * FPT);
            const int t = r / (QN * FPT), f = r % (QN * FPT);
            float p = 0.f;
            if (f < F) {
                const float *tl = &tv[side][t][(f >> 4) * NP];
                p = fscale;
#pragma unroll
                for (int b = 0; b < NP; ++b)
                    if ((f >> b) & 1) p *= tl[b];
            }
            ps[side][t][f] = p;
        }
        __syncthreads();
#pragma unroll 1
        for (int t = 0; t < nt; ++t) {
            if (UPD) {
                const float y = yv[t][c];
#pragma unroll
                for (int i = 0; i < FPT; ++i) S[i] = fmaf(ps[KS][t][f0 + i], y, S[i]);
#pragma unroll
                for (int z = 0; z < ZP; ++z)
                    if (64 * z + c < FPT) Z[z] += ps[KS][t][f0 + 64 * z + c];
            }
            if (RD) {
                float n = 0.f, m = 0.f;
#pragma unroll
                for (int i = 0; i < FPT; ++i) n = fmaf(ps[0][t][f0 + i], S[i], n);
#pragma unroll
                for (int z = 0; z < ZP; ++z)
                    if (64 * z + c < FPT) m = fmaf(ps[0][t][f0 + 64 * z + c], Z[z], m);
                pn[t][grp][c] = n;
                m = wave_sum(m);
                if (c == 0) pm[t][grp] = m;
            }
        }
        if constexpr (ONE) store_state();
        __syncthreads();
        if (RD) {
            for (int e = tid; e < nt * (d + 1); e += nthr) {
                const int t = e / (d + 1), col = e % (d + 1);
                float n = 0.f, m = 0.f;
                for (int g = 0; g < QN; ++g) {
                    if (col < d) n += pn[t][g][col];
                    m += pm[t][g];
                }
                const int64_t row = row0 + tile + t;
                if (col < d)
                    O[row * d + col] = (T)(n / m);
                else
                    den[row] = m;
            }
            __syncthreads();  // the tile's LDS is rewritten next
        }
    }
    if (MODE != SM_READOUT && !ONE) store_state();
}

// state[head] += sum over the blocks b = 0, 1, ... of part[head][b] (in that
// order, so the result does not depend on the launch)
static __global__ __launch_bounds__(256) void stream_reduce_kernel(const float *__restrict__ part, int nblk,
                                                            int64_t elems, float *__restrict__ state)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= elems) return;
    const int64_t bh = blockIdx.y;
    float acc = state[bh * elems + e];
    const float *p = part + bh * (int64_t)nblk * elems + e;
    for (int b = 0; b < nblk; ++b) acc += p[(int64_t)b * elems];
    state[bh * elems + e] = acc;
}

}  // namespace race

namespace race {

// state[head] += scale x (the key-state total of a fused segment sum).  The
// total is slot nseg of the head's segment states, FxC blocks
// [wave][s][ct][lane][4]: element (w, s, ct, lane (g, c16), r) is feature
// 16 (4 w + g) + 4 s + r (table 4 w + g, Walsh subset 4 s + r) and value
// column 16 ct + c16, column HD being the count column.  Tables >= L and the
// padding columns are skipped.  scale = 2^(P/2): the fused writer features
// are 2^-P prod t, the streaming state's 2^(-P/2) prod t.
static __global__ __launch_bounds__(256) void stream_from_sums_kernel(const float *__restrict__ st,
                                                               int64_t nseg, int nwaves, int L,
                                                               int d, float scale,
                                                               float *__restrict__ state)
{
    const int per_wave = 4 * NT * 64 * 4;
    const int total = nwaves * per_wave;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= total) return;
    const int64_t bh = blockIdx.y;
    const int r = e & 3, lane = (e >> 2) & 63, wsct = e >> 8;
    const int ct = wsct % NT, s = (wsct / NT) & 3, w = wsct / (NT * 4);
    const int g = lane >> 4, c16 = lane & 15;
    const int table = 4 * w + g, col = 16 * ct + c16;
    const int c = col < d ? col : col == HD ? d : -1;
    if (table >= L || c < 0) return;
    const int sc = d + 1, f = 16 * table + 4 * s + r;
    const float v = st[(bh * (nseg + 1) + nseg) * (int64_t)total + e];
    float *dst = state + bh * (int64_t)(16 * L) * sc + (int64_t)f * sc + c;
    *dst += scale * v;
}

}  // namespace race
