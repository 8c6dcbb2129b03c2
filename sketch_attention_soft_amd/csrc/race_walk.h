// race_walk.h -- block-staged chunk kernels of RACE attention for bf16 rows
// (gfx950), built so that almost all arithmetic per chunk is MFMA work.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (soft
// hashing, bucket sums, ratio readout) and §2.3 (causal streaming sums); the
// es page §2 (angular kernel on normalised vectors).
//
// Staging.  Each chunk of 32 tokens is loaded once per workgroup: every
// thread fetches one 16-byte piece of a row (the next chunk's, while the
// current one is computed) and writes it to LDS, where the eight threads of a
// row also form its squared norm.  Value rows go to LDS column by column (and
// row by row where needed), so that any wave reads them as MFMA operands.
// All chunk loads and stores go through buffer resources sized to the chunk's
// valid rows, so ragged ends need neither clamping nor branches.
//
// Hash-feature cache.  Each row is hashed once per pass: the kernel that
// hashes it stores t = tanh(tanh(u')/tau) (and dt/du') in fp16 in the
// kernels' register layout, and later kernels read it instead of hashing.
//
// Per wave (4 tables = 16 hyperplanes = 64 features, all in registers):
//   U^T = W x^T (MFMA, W = W_hi + W_lo) -> lane (table g, token c16) holds
//   t_0..3 of its table -> the 16 Walsh features of that table are two
//   token-major K-blocks (slots (g, i) <-> S = 8k + i);
//   feature-major fragments (K = tokens) come from the token-major ones by a
//   0/1 selection MFMA, which moves every bf16 value exactly;
//   intra-chunk scores are formed per wave over its own features and
//   multiplied into the wave's partial output, so the only cross-wave sum is
//   the one of the partial outputs.
// FxC state tile (s, ct): lane (rows 4g + r, column 16 ct + c16) <-> features
// (table 4w + g, S = 4s + r), stored in global memory as [wave][s][ct][lane][4].
#pragma once
#include "race_common.h"
#include "race_fwd.h"
#include "race_squash.h"

namespace race {

constexpr int WCT = 32;      // tokens per chunk
constexpr int XRS = HD + 8;  // staged row stride (bf16 elements)
constexpr int YCS = WCT + 8; // staged value column stride (tokens)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ halfx4 to_h4(const floatx4 &v)
{
    const halfx4 r = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    return r;
}
__device__ __forceinline__ floatx4 to_f4(const halfx4 &v)
{
    const floatx4 r = {(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    return r;
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    const bf16x2 v = {(bf16)a, (bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
typedef _Float16 f16;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Rows in global memory are bf16 or fp16 (IO); what is staged in LDS and
// every MFMA operand is bf16.  One 32-bit word holds two row elements:
// io_lo / io_hi give them as floats (exact), io_bf16w as bf16 bits (as they
// are for bf16 rows, rounded to nearest even for fp16 rows), and pk_io packs
// two floats as IO (round to nearest even).
template <typename IO> inline constexpr bool is_bf16 = false;
template <> inline constexpr bool is_bf16<bf16> = true;
template <typename IO> __device__ __forceinline__ float io_lo(uint32_t w)
{
    if constexpr (is_bf16<IO>) return __builtin_bit_cast(float, w << 16);
    else return (float)__builtin_bit_cast(half2v, w)[0];
}
template <typename IO> __device__ __forceinline__ float io_hi(uint32_t w)
{
    if constexpr (is_bf16<IO>) return __builtin_bit_cast(float, w & 0xffff0000u);
    else return (float)__builtin_bit_cast(half2v, w)[1];
}
template <typename IO> __device__ __forceinline__ uint32_t io_bf16w(uint32_t w)
{
    if constexpr (is_bf16<IO>) return w;
    else return pk_bf16(io_lo<IO>(w), io_hi<IO>(w));
}
template <typename IO> __device__ __forceinline__ uint32_t pk_io(float a, float b)
{
    if constexpr (is_bf16<IO>) {
        return pk_bf16(a, b);
    } else {
        const half2v v = {(f16)a, (f16)b};
        return __builtin_bit_cast(uint32_t, v);
    }
}
__device__ __forceinline__ bf16x8 pk8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ bf16x4 pk4(uint32_t a, uint32_t b)
{
    const u32x2 v = {a, b};
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 lo4(bf16x8 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 hi4(bf16x8 v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }
__device__ __forceinline__ bf16x4 acc2bf4(const floatx4 &a)
{
    return pk4(pk_bf16(a[0], a[1]), pk_bf16(a[2], a[3]));
}

__device__ __forceinline__ void mma32(floatx4 &acc, bf16x8 a, bf16x8 b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// Sums over aligned groups of 8 / 16 lanes (DPP within a row).
__device__ __forceinline__ float dpp_add(float x, int ctrl_sel)
{
    int y;
    switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false); break;
    case 1: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false); break;
    case 2: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false); break;
    default: y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false); break;
    }
    return x + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float sum8(float x)
{
    x = dpp_add(x, 0);  // quad_perm [1,0,3,2]
    x = dpp_add(x, 1);  // quad_perm [2,3,0,1]
    return dpp_add(x, 2);  // row_half_mirror: the other quad of the 8
}
__device__ __forceinline__ float sum16(float x) { return dpp_add(sum8(x), 3); }  // row_ror:8

// ---------------------------------------------------------------------------
// Buffer resources.  The rows of one chunk are addressed through a resource
// whose base is the chunk's first row and whose size covers its valid rows
// only: loads past the size return zeros and stores past it are dropped.  So
// the loop needs no clamping and no per-row branches, lane offsets are loop
// constants, and the chunk position lives in scalar registers.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, int bytes)
{
    // the arguments are wave-uniform; reading them through the first lane
    // keeps the descriptor in scalar registers whichever unit computed them
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    // dword 3: 32-bit data format, the raw-buffer setting of this GPU family
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(lo | (hi << 32)), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
constexpr int OOB = 0x7ffffff0;  // a lane offset past every resource: the access is skipped

__device__ __forceinline__ u32x4 bld128(Rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ u32x2 bld64(Rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }
__device__ __forceinline__ float bldf(Rsrc r, int off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void bst64(u32x2 v, Rsrc r, int off) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0); }
__device__ __forceinline__ void bst128(u32x4 v, Rsrc r, int off) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0); }
__device__ __forceinline__ void bstf(float v, Rsrc r, int off)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}

// Wave priority: the two waves of a SIMD leave a chunk's barrier together
// and would reach their matrix-product blocks together; raising a wave's
// priority for its products lets the other one issue its vector work in
// between (measured: 2-3% off the walk kernels and the hashing sum, nothing
// or worse on the gradient kernels, which do without).
template <int P> __device__ __forceinline__ void prio() { __builtin_amdgcn_s_setprio(P); }

// Keeps the loads issued above it in place: the scheduler would otherwise
// sink prefetches towards the end of the loop body, next to their first use.
__device__ __forceinline__ void pin_loads() { __builtin_amdgcn_sched_barrier(0); }

// A chunk of a segment: first token (segment-relative) and valid rows (0 for
// chunk indices past the end, whose accesses are all skipped).
struct Chunk {
    int tok0, nv;
};

// chunk loop unrolled by two so that the parity of the chunk, which selects a
// double buffer, is a compile-time constant: body(ci, Par<ci & 1>{})
template <int P> struct Par {
    static constexpr int v = P;
};
template <class F>
__device__ __forceinline__ void for_chunks2(int n, F &&body)
{
    for (int ci = 0; ci < n; ci += 2) {
        body(ci, Par<0>{});
        if (ci + 1 < n) body(ci + 1, Par<1>{});
    }
}

// rows of a [token][D] array of 16-bit elements (D = d: 64, or 32 staged
// into the 64 columns of the kernels with zeros past column D)
template <int D, typename IO> __device__ __forceinline__ Rsrc row_res(const IO *seg_rows, const Chunk &c)
{
    return make_rsrc(seg_rows + c.tok0 * D, c.nv * D * 2);
}

// ---------------------------------------------------------------------------
// Staging of raw rows of one chunk: item e = threadIdx.x + it NTHR (< 256)
// -> token e >> 3, columns (e & 7) * 8 .. + 8 (byte offset 16 e).
template <int NTHR> struct XStage {
    static constexpr int ITEMS = (WCT * 8 + NTHR - 1) / NTHR;
    u32x4 v[ITEMS];
};

// Row piece of this thread.  UP (the gradient kernels, whose value rows cost
// the most) with 512 threads: the rows go to the upper four waves, so that the
// value rows (items of the lower four) and the rows are staged by different
// waves of each SIMD.
template <int NTHR, bool UP> __device__ __forceinline__ int xitem(int it)
{
    return (UP && NTHR == 512 ? (int)threadIdx.x ^ 256 : (int)threadIdx.x) + it * NTHR;
}

template <int NTHR, bool UP, int D>
__device__ __forceinline__ void xstage_load(Rsrc r, XStage<NTHR> &xs)
{
#pragma unroll
    for (int it = 0; it < XStage<NTHR>::ITEMS; ++it) {
        const int e = xitem<NTHR, UP>(it);
        if constexpr (D == HD)
            xs.v[it] = bld128(r, e < WCT * 8 ? e * 16 : OOB);
        else  // columns past D read as zeros
            xs.v[it] = bld128(r, e < WCT * 8 && (e & 7) * 8 < D ? (e >> 3) * (D * 2) + (e & 7) * 16 : OOB);
    }
}

// rows -> xb[token][XRS] (rows past the chunk's end were loaded as zeros);
// kb[token] = -2 log2(e) / max(|x|, 1e-12) (NORM2: the squared norm |x|^2;
// the pieces are those of xstage_load<NTHR, NORM2>)
template <int NTHR, bool NORM2, typename IO>
__device__ __forceinline__ void xstage_store(const XStage<NTHR> &xs, bf16 *xb, float *kb)
{
#pragma unroll
    for (int it = 0; it < XStage<NTHR>::ITEMS; ++it) {
        const int e = xitem<NTHR, NORM2>(it);
        if (e < WCT * 8) {  // uniform per wave
            const int j = e >> 3;
            float ss = 0.f;
            if constexpr (is_bf16<IO>) {
                const bf16x8 v = __builtin_bit_cast(bf16x8, xs.v[it]);
                *reinterpret_cast<bf16x8 *>(xb + j * XRS + (e & 7) * 8) = v;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float x = (float)v[i];
                    ss = fmaf(x, x, ss);
                }
            } else {
                // the norm from the exact values, the staged row rounded to bf16
                float x[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = io_lo<IO>(xs.v[it][i]);
                    x[2 * i + 1] = io_hi<IO>(xs.v[it][i]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
                *reinterpret_cast<bf16x8 *>(xb + j * XRS + (e & 7) * 8) =
                    pk8(pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3]), pk_bf16(x[4], x[5]), pk_bf16(x[6], x[7]));
            }
            ss = sum8(ss);
            if ((e & 7) == 0)
                kb[j] = NORM2 ? ss : -2.8853900817779268f * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
        }
    }
}

// Staging of value rows y_j: [v | 1] (DVAL = false) or [dO/m | -(dO . o)/m]
// (DVAL = true).  Item e < 256 -> tokens 2 (e >> 4) and 2 (e >> 4) + 1,
// columns (e & 15) * 4 .. + 4.
//
// Rows of D = 128 elements run in two passes of 64 value columns (the value
// pointers point at the pass's first column, rows keep their stride): the
// gradient values' last column comes precomputed over the whole row (dm), or
// is zero in the pass without it.
struct YRes {
    Rsrc v, o, d, dm;
};
template <bool DVAL, int D, typename IO>
__device__ __forceinline__ YRes yres(const ValSrc<IO> &s, const Chunk &c)
{
    YRes r;
    r.v = row_res<D>(s.V, c);
    if constexpr (DVAL) {
        r.o = D > HD ? r.v : row_res<D>(s.O, c);
        r.d = make_rsrc(s.den + c.tok0, c.nv * 4);
        // (a pass without the column: an empty resource, loads read zero)
        r.dm = D > HD ? make_rsrc(s.dm ? s.dm + c.tok0 : s.den, s.dm ? c.nv * 4 : 0) : r.d;
    } else {
        r.o = r.v;
        r.d = r.v;
        r.dm = r.v;
    }
    return r;
}

template <int NTHR, bool DVAL> struct YStage {
    static constexpr int ITEMS = (WCT * 8 + NTHR - 1) / NTHR;
    u32x2 x[ITEMS][2];
    u32x2 o[DVAL ? ITEMS : 1][2];
    float m[DVAL ? ITEMS : 1][2];
};

template <int NTHR, bool DVAL, int D>
__device__ __forceinline__ void ystage_load(const YRes &r, YStage<NTHR, DVAL> &ys)
{
#pragma unroll
    for (int it = 0; it < YStage<NTHR, DVAL>::ITEMS; ++it) {
        const int e = threadIdx.x + it * NTHR;
        const bool act = e < WCT * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tok = 2 * (e >> 4) + h;
            // columns past D read as zeros (m is read with the row)
            const int off = act && (D == HD || (e & 15) * 4 < D) ? tok * (D * 2) + (e & 15) * 8 : OOB;
            ys.x[it][h] = bld64(r.v, off);
            if constexpr (DVAL) {
                if constexpr (D > HD)  // the last column, precomputed
                    ys.o[it][h] = u32x2{__builtin_bit_cast(uint32_t, bldf(r.dm, act ? tok * 4 : OOB)), 0u};
                else
                    ys.o[it][h] = bld64(r.o, off);
                ys.m[it][h] = bldf(r.d, act ? tok * 4 : OOB);
            }
        }
    }
}

// token-major value rows: columns 0 .. NCOL + 15 (three K = 32 operand groups,
// zero past column HD) and 8 of padding
constexpr int YRC = NCOL + 16;
constexpr int YRS = YRC + 8;

// yc: column-major [NCOL][YCS] and / or yr: token-major [WCT][YRS] (either may
// be null); nv = valid rows of the chunk (the others are staged as zeros)
template <int NTHR, bool DVAL, typename IO, int D = HD>
__device__ __forceinline__ void ystage_store(const YStage<NTHR, DVAL> &ys, int nv, bf16 *yc,
                                             bf16 *yr = nullptr)
{
#pragma unroll
    for (int it = 0; it < YStage<NTHR, DVAL>::ITEMS; ++it) {
        const int e = threadIdx.x + it * NTHR;
        if (e < WCT * 8) {  // uniform per wave
            const int jp = e >> 4, c0 = (e & 15) * 4;
            if constexpr (!DVAL) {
                // [v | 1]: the loaded bits are staged as they are (bf16 rows) or
                // rounded to bf16; the column layout pairs tokens 2jp, 2jp + 1 of
                // each column by byte permutes
                u32x2 yx[2] = {ys.x[it][0], ys.x[it][1]};
                if constexpr (!is_bf16<IO>)
#pragma unroll
                    for (int h = 0; h < 2; ++h) yx[h] = u32x2{io_bf16w<IO>(yx[h][0]), io_bf16w<IO>(yx[h][1])};
                if (yc) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        *reinterpret_cast<uint32_t *>(yc + (c0 + i) * YCS + 2 * jp) =
                            __builtin_amdgcn_perm(yx[1][i >> 1], yx[0][i >> 1],
                                                  (i & 1) ? 0x07060302u : 0x05040100u);
                    if (c0 == 0)
                        *reinterpret_cast<uint32_t *>(yc + HD * YCS + 2 * jp) =
                            pk_bf16(2 * jp < nv ? 1.f : 0.f, 2 * jp + 1 < nv ? 1.f : 0.f);
                }
                if (yr) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *reinterpret_cast<u32x2 *>(yr + (2 * jp + h) * YRS + c0) = yx[h];
                        if (c0 == 0) yr[(2 * jp + h) * YRS + HD] = (bf16)(2 * jp + h < nv ? 1.f : 0.f);
                    }
                }
                continue;
            }
            float y[2][4], extra[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = 2 * jp + h < nv;
                float xv[4], ov[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    xv[2 * i] = io_lo<IO>(ys.x[it][h][i]);
                    xv[2 * i + 1] = io_hi<IO>(ys.x[it][h][i]);
                    ov[2 * i] = io_lo<IO>(ys.o[it][h][i]);
                    ov[2 * i + 1] = io_hi<IO>(ys.o[it][h][i]);
                }
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) dot = fmaf(xv[i], ov[i], dot);
                dot = sum16(dot);
                // rows past the end read m = 0: their D row is zero
                const float inv_m = ok ? __builtin_amdgcn_rcpf(ys.m[it][h]) : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[h][i] = xv[i] * inv_m;
                extra[h] = -dot * inv_m;
                if constexpr (D > HD) extra[h] = __builtin_bit_cast(float, ys.o[it][h][0]);
            }
            if (yc) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint32_t *>(yc + (c0 + i) * YCS + 2 * jp) = pk_bf16(y[0][i], y[1][i]);
                if (c0 == 0) *reinterpret_cast<uint32_t *>(yc + HD * YCS + 2 * jp) = pk_bf16(extra[0], extra[1]);
            }
            if (yr) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    *reinterpret_cast<bf16x4 *>(yr + (2 * jp + h) * YRS + c0) =
                        pk4(pk_bf16(y[h][0], y[h][1]), pk_bf16(y[h][2], y[h][3]));
                    if (c0 == 0) yr[(2 * jp + h) * YRS + HD] = (bf16)extra[h];
                }
            }
        }
    }
}

// value columns HD+1 .. NCOL-1 are zero for every chunk
template <int NTHR> __device__ __forceinline__ void ystage_zero_pad(bf16 *yc)
{
    for (int e = threadIdx.x; e < (NCOL - HD - 1) * WCT / 2; e += NTHR) {
        const int c = HD + 1 + e / (WCT / 2), jp = e % (WCT / 2);
        *reinterpret_cast<uint32_t *>(yc + c * YCS + 2 * jp) = 0u;
    }
}
template <int NTHR> __device__ __forceinline__ void yrow_zero_pad(bf16 *yr)
{
    for (int e = threadIdx.x; e < (YRC - HD - 1) * WCT; e += NTHR) {
        const int c = HD + 1 + e % (YRC - HD - 1), j = e / (YRC - HD - 1);
        yr[j * YRS + c] = (bf16)0.f;
    }
}

// ---------------------------------------------------------------------------
// Hyperplanes per table P <= 4.  The kernels always work with 4 hyperplanes
// (16 Walsh features) per table; for P < 4, hyperplanes p >= P are padding:
// their W rows are zero and their t is +0 exactly, so every feature that
// contains one vanishes on the writer side, and with writer features scaled by
// 2^-P each table's kernel is prod_{p < P} (1 + t_p t'_p) / 2^P, the P-plane
// corner product.  W is [L][P][d]: internal hyperplane 4 l + p <- row P l + p.
//
// P = 5, 6: a table of 2^P features is V = 2^(P-4) virtual tables of 16.
// Its features prod_{p in S} t_p, S a subset of {0..P-1}, split as S = A + B
// with A in {0..3} and B in {4, 5}: virtual table B (b = bit mask of B) holds
// the 16 Walsh features of t_0..t_3 times tau_b = prod_{p in B} t_p, so the
// sum over the virtual tables of their kernels is the real table's,
// prod_{p < P} (1 + t_p t'_p) / 2^P.  Internal rows: virtual table 0 projects
// hyperplanes 0..3, virtual table 1 hyperplanes 4 (and 5), the others none
// (zero rows, t = +0); vt_expand moves t_0..t_3 and t_4, t_5 between the
// lanes of a real table, vt_reduce adds the virtual tables' gradients back.
// Virtual table 4 w + g of a wave is real table (4 w + g) >> (P - 4), b = g & (V - 1).
__device__ __forceinline__ int vt_shift(int P) { return P > NP ? P - NP : 0; }
// internal tables of L real ones
__device__ __forceinline__ int vtables(int L, int P) { return L << vt_shift(P); }
// row of W [L][P][d] of internal hyperplane hp, or -1 (padding)
__device__ __forceinline__ int w_row(int L, int P, int hp)
{
    int l = hp >> 2, p = hp & 3;
    if (P > NP) {
        const int sh = P - NP, b = l & ((1 << sh) - 1);
        l >>= sh;
        p = b == 0 ? p : b == 1 ? NP + p : P;
    }
    return l < L && p < P ? l * P + p : -1;
}
__device__ __forceinline__ float w_elem(const float *__restrict__ W, int L, int P, int D, int hp, int c)
{
    const int r = w_row(L, P, hp);
    return r >= 0 && c < D ? W[r * D + c] : 0.f;
}
// masks of |t| for the fp16 pairs (p = 0, 1) and (2, 3): zero for padding
// hyperplanes (P > 4: of this lane's virtual table)
struct TMask {
    uint32_t m[2];
};
template <bool PV = false> __device__ __forceinline__ TMask t_mask(int P)
{
    int n = P;  // hyperplanes of this lane's table that are not padding
    if (PV) {
        const int b = (lane_id() >> 4) & ((1 << (P - NP)) - 1);
        n = b == 0 ? NP : b == 1 ? P - NP : 0;
    }
    TMask t;
#pragma unroll
    for (int q = 0; q < 2; ++q)
        t.m[q] = (2 * q < n ? 0x7fffu : 0u) | (2 * q + 1 < n ? 0x7fff0000u : 0u);
    return t;
}
// writer feature scale 2^-P (padding tables: 0)
__device__ __forceinline__ float writer_scale(int P, bool table_in_use)
{
    return table_in_use ? __builtin_ldexpf(1.f, -P) : 0.f;
}

// t_0..t_3 of this lane's table, with (P > 4) the factor tau_b of its
// virtual table b and t_4, t_5 of the real table
struct VT {
    floatx4 t;
    float tau, t4, t5;
    int b;
};
// P > 4: from the per-row t of the lanes of virtual tables 0 (t_0..t_3) and
// 1 (t_4, t_5) of the same token; P <= 4: t itself, tau = 1.
template <bool PV> __device__ __forceinline__ VT vt_expand(const halfx4 &raw, int P)
{
    VT v;
    if constexpr (!PV) {
        v.t = to_f4(raw);
        v.tau = 1.f;
        v.t4 = v.t5 = 0.f;
        v.b = 0;
    } else {
        const int lane = lane_id();
        v.b = (lane >> 4) & ((1 << (P - NP)) - 1);
        const u32x2 r = __builtin_bit_cast(u32x2, raw);
        const int src = (lane - 16 * v.b) * 4;  // byte address of the lane of virtual table 0
        const u32x2 t03 = {(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)r[0]),
                           (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)r[1])};
        const half2v t45 = __builtin_bit_cast(half2v, __builtin_amdgcn_ds_bpermute(src + 64, (int)r[0]));
        v.t = to_f4(__builtin_bit_cast(halfx4, t03));
        v.t4 = (float)t45[0];
        v.t5 = (float)t45[1];
        v.tau = v.b == 0 ? 1.f : v.b == 1 ? v.t4 : v.b == 2 ? v.t5 : v.t4 * v.t5;
    }
    return v;
}
// P > 4: dt holds the gradient of this lane's 16 features with respect to
// t_0..t_3 of its table without the factor tau_b, dtau the gradient with
// respect to tau_b.  Sums the shares of the V virtual tables of the real
// table and leaves in dt the gradient of this lane's own rows: t_0..t_3
// (virtual table 0), t_4, t_5 (virtual table 1), zero (the others).
template <bool PV> __device__ __forceinline__ void vt_reduce(const VT &v, int P, float dtau, float (&dt)[4])
{
    if constexpr (PV) {
        float x[6];
#pragma unroll
        for (int p = 0; p < 4; ++p) x[p] = v.tau * dt[p];
        x[4] = v.b == 1 ? dtau : v.b == 3 ? dtau * v.t5 : 0.f;  // d tau_b / d t_4
        x[5] = v.b == 2 ? dtau : v.b == 3 ? dtau * v.t4 : 0.f;  // d tau_b / d t_5
        for (int m = 16; m < (16 << (P - NP)); m <<= 1)
#pragma unroll
            for (int i = 0; i < 6; ++i) x[i] += __shfl_xor(x[i], m);
#pragma unroll
        for (int p = 0; p < 4; ++p)
            dt[p] = v.b == 0 ? x[p] : v.b == 1 && p < 2 ? x[4 + p] : 0.f;
    }
}

// W rows of this wave's 16 hyperplanes as the A operand of U^T = W x^T.
struct WRows {
    bf16x8 hi[2], lo[2];
};

template <int D>
__device__ __forceinline__ void load_wrows(const float *__restrict__ W, int L, int P, WRows &wr)
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int hp = w * 16 + c16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = w_elem(W, L, P, D, hp, kb * 32 + g * 8 + i);
            wr.hi[kb][i] = (bf16)v;
            wr.lo[kb][i] = (bf16)(v - (float)wr.hi[kb][i]);
        }
}

// 0/1 selection operand: column rho of FxC row-tile s takes token-major slot
// (g = rho / 4, i = 4 (s & 1) + rho % 4) of K-block s / 2.
__device__ __forceinline__ bf16x8 selection(int par)
{
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)((g == (c16 >> 2) && i == 4 * par + (c16 & 3)) ? 1.f : 0.f);
    return f;
}

// W rows (hi, lo) of all waves staged once per workgroup, wl[2][NW * 16][XRS]
template <int NW, int D>
__device__ __forceinline__ void stage_wrows(const float *__restrict__ W, int L, int P, bf16 *wl)
{
    for (int e = threadIdx.x; e < NW * 16 * HD; e += NW * 64) {
        const int hp = e / HD, c = e % HD;
        const float v = w_elem(W, L, P, D, hp, c);
        const bf16 hi = (bf16)v;
        wl[hp * XRS + c] = hi;
        wl[(NW * 16 + hp) * XRS + c] = (bf16)(v - (float)hi);
    }
}
// the two selection operands, sl[2][64 lanes][8]
__device__ __forceinline__ void stage_sel(bf16 *sl)
{
    if (threadIdx.x < 64) {
        *reinterpret_cast<bf16x8 *>(sl + threadIdx.x * 8) = selection(0);
        *reinterpret_cast<bf16x8 *>(sl + (64 + threadIdx.x) * 8) = selection(1);
    }
}
template <int NW> __device__ __forceinline__ void wrows_lds(const bf16 *wl, WRows &wr)
{
    const int lane = lane_id(), g = lane >> 4, hp = wave_id() * 16 + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        wr.hi[kb] = *reinterpret_cast<const bf16x8 *>(wl + hp * XRS + kb * 32 + g * 8);
        wr.lo[kb] = *reinterpret_cast<const bf16x8 *>(wl + (NW * 16 + hp) * XRS + kb * 32 + g * 8);
    }
}
__device__ __forceinline__ void sel_lds(const bf16 *sl, bf16x8 (&sel)[2])
{
    sel[0] = *reinterpret_cast<const bf16x8 *>(sl + lane_id() * 8);
    sel[1] = *reinterpret_cast<const bf16x8 *>(sl + (64 + lane_id()) * 8);
}

// Squash of the projections u of tables 4w + g (lane (g, c16)) for token
// 16 tt + c16 of the staged rows xb: t = tanh(tanh(u') / tau) with u' = u / |x|,
// and with CHAIN also dt/du' = ((1 - t^2) / tau) (1 - z^2), z = tanh(|u'|),
// 1 - z^2 = 4e / (1 + e)^2, e = exp(-2|u'|) = exp2(|u| kb).  Both are returned
// in fp16, the precision the hash-feature cache keeps.
//   POLY: |t| and dt/du' as degree-DEG16 polynomials in y = 2e - 1, evaluated
//         in fp16 pairs (two values per instruction); the sign of u is copied
//         onto the pair's sign bits.
//   else: the functions themselves in fp32.
// Padding hyperplanes (tm) get t = +0.
__device__ __forceinline__ half2v horner16(const uint32_t (&cf)[DEG16 + 1], half2v y)
{
    half2v h = __builtin_bit_cast(half2v, cf[DEG16]);
#pragma unroll
    for (int k = DEG16 - 1; k >= 0; --k) h = __builtin_elementwise_fma(h, y, __builtin_bit_cast(half2v, cf[k]));
    return h;
}
// the sign bits of a and b in the sign bits of an fp16 pair (low, high)
__device__ __forceinline__ uint32_t sign_pair(float a, float b)
{
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a), 0x07000300u) &
           0x80008000u;
}

template <bool POLY, bool CHAIN>
__device__ __forceinline__ void hash_staged(const bf16 *xb, const float *kb, int tt, const WRows &wr,
                                            const Squash &sq, const TMask &tm, halfx4 &t, halfx4 &c)
{
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    const int row = tt * 16 + c16;
    const bf16x8 x0 = *reinterpret_cast<const bf16x8 *>(xb + row * XRS + g * 8);
    const bf16x8 x1 = *reinterpret_cast<const bf16x8 *>(xb + row * XRS + 32 + g * 8);
    floatx4 u = {0.f, 0.f, 0.f, 0.f};
    mma32(u, wr.hi[0], x0);
    mma32(u, wr.lo[0], x0);
    mma32(u, wr.hi[1], x1);
    mma32(u, wr.lo[1], x1);
    const float kf = kb[row];
    if constexpr (POLY) {
        uint32_t tp[2], cp[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float e0 = __builtin_amdgcn_exp2f(fabsf(u[2 * q]) * kf);
            const float e1 = __builtin_amdgcn_exp2f(fabsf(u[2 * q + 1]) * kf);
            const half2v y = {(_Float16)fmaf(2.f, e0, -1.f), (_Float16)fmaf(2.f, e1, -1.f)};
            const uint32_t h = __builtin_bit_cast(uint32_t, horner16(sq.t16, y));
            tp[q] = (h & tm.m[q]) | sign_pair(u[2 * q], u[2 * q + 1]);  // padding: +0
            if constexpr (CHAIN) cp[q] = __builtin_bit_cast(uint32_t, horner16(sq.c16, y));
        }
        const u32x2 tv = {tp[0], tp[1]};
        t = __builtin_bit_cast(halfx4, tv);
        if constexpr (CHAIN) {
            const u32x2 cv = {cp[0], cp[1]};
            c = __builtin_bit_cast(halfx4, cv);
        }
    } else {
        floatx4 tf, cf;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float e = __builtin_amdgcn_exp2f(fabsf(u[p]) * kf);
            const float z = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
            const float e2 = __builtin_amdgcn_exp2f(-2.8853900817779268f * z * sq.inv_tau);
            const float h = (1.f - e2) * __builtin_amdgcn_rcpf(1.f + e2);
            tf[p] = (tm.m[p >> 1] >> (16 * (p & 1))) & 1u ? copysignf(h, u[p]) : 0.f;
            if constexpr (CHAIN) {
                const float r = __builtin_amdgcn_rcpf(1.f + e);
                cf[p] = (1.f - h * h) * (4.f * sq.inv_tau) * e * r * r;
            }
        }
        t = to_h4(tf);
        if constexpr (CHAIN) c = to_h4(cf);
    }
}

// token-major Walsh features of one table, q prod_{p in S} t_p: lo = S 0..7,
// hi = S 8..15.  The features are 2^(-P/2) prod t_p (1/4 for P = 4); the
// kernels form reader features with q = 1 and writer features with q = 2^-P
// (0 for padding tables), which gives every score and state product its
// factor 2^-P exactly (powers of two) and saves the reader side four products.
__device__ __forceinline__ void walsh_tm(const floatx4 &t, float q, bf16x8 &lo, bf16x8 &hi)
{
    const float a1 = q * t[0], a2 = q * t[1], a3 = a1 * t[1], b3 = t[2] * t[3];
    lo = pk8(pk_bf16(q, a1), pk_bf16(a2, a3), pk_bf16(q * t[2], a1 * t[2]),
             pk_bf16(a2 * t[2], a3 * t[2]));
    hi = pk8(pk_bf16(q * t[3], a1 * t[3]), pk_bf16(a2 * t[3], a3 * t[3]), pk_bf16(q * b3, a1 * b3),
             pk_bf16(a2 * b3, a3 * b3));
}

// feature-major fragments of the 4 FxC row tiles over the chunk's 32 tokens
// (K-slots (g, r) <-> token 4g + r, (g, 4 + r) <-> token 16 + 4g + r)
__device__ __forceinline__ void feat_major(const bf16x8 (&ptm)[2][2], const bf16x8 (&sel)[2],
                                           bf16x8 (&pfm)[4])
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x4 half[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            floatx4 d = {0.f, 0.f, 0.f, 0.f};
            mma32(d, ptm[tt][s >> 1], sel[s & 1]);
            half[tt] = acc2bf4(d);
        }
        pfm[s] = cat8(half[0], half[1]);
    }
}

// The same features of a writer row in fp16, formed from the fp16 t with
// packed multiplies (two features per instruction, no conversion): feature
// pairs (S, S + 1) differ in t_0 only, so pair m is g_m (1, t_0) with g_m the
// product over the bits of S = 2m in t_1..t_3.  The selection product below
// moves them to the feature-major operand, rounded there to bf16.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void walsh_tm16(const halfx4 &t, _Float16 q, halfx8 &lo, halfx8 &hi)
{
    const half2v u = half2v{q, q} * half2v{(_Float16)1.f, t[0]};  // S = 0, 1
    const half2v p2 = u * t[1];                                    // S = 2, 3
    const half2v p4 = u * t[2];                                    // S = 4, 5
    const half2v p6 = p2 * t[2];                                   // S = 6, 7
    const half2v p8 = u * t[3], p10 = p2 * t[3], p12 = p4 * t[3], p14 = p6 * t[3];
    const halfx4 a = __builtin_shufflevector(u, p2, 0, 1, 2, 3), b = __builtin_shufflevector(p4, p6, 0, 1, 2, 3);
    const halfx4 c = __builtin_shufflevector(p8, p10, 0, 1, 2, 3), e = __builtin_shufflevector(p12, p14, 0, 1, 2, 3);
    lo = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    hi = __builtin_shufflevector(c, e, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ halfx8 selection16(int par)
{
    const int lane = lane_id(), g = lane >> 4, c16 = lane & 15;
    halfx8 f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (g == (c16 >> 2) && i == 4 * par + (c16 & 3)) ? (_Float16)1.f : (_Float16)0.f;
    return f;
}
__device__ __forceinline__ void feat_major16(const halfx8 (&ptm)[2][2], const halfx8 (&sel)[2], bf16x8 (&pfm)[4])
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x4 half[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            floatx4 d = {0.f, 0.f, 0.f, 0.f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ptm[tt][s >> 1], sel[s & 1], d, 0, 0, 0);
            half[tt] = acc2bf4(d);
        }
        pfm[s] = cat8(half[0], half[1]);
    }
}
// the fp16 selection operands, sl[2][64 lanes][8]
__device__ __forceinline__ void stage_sel16(_Float16 *sl)
{
    if (threadIdx.x < 64) {
        *reinterpret_cast<halfx8 *>(sl + threadIdx.x * 8) = selection16(0);
        *reinterpret_cast<halfx8 *>(sl + (64 + threadIdx.x) * 8) = selection16(1);
    }
}
__device__ __forceinline__ void sel_lds16(const _Float16 *sl, halfx8 (&sel)[2])
{
    sel[0] = *reinterpret_cast<const halfx8 *>(sl + lane_id() * 8);
    sel[1] = *reinterpret_cast<const halfx8 *>(sl + (64 + lane_id()) * 8);
}
// Writer features of one chunk (two token tiles, cached or freshly hashed t)
// in the feature-major layout of the state update.  P <= 4 take the fp16
// route above; P > 4 (virtual tables, t moved between lanes) the fp32 one.
template <bool PV>
__device__ __forceinline__ void writer_fm(const halfx4 (&t)[2], int P, float qw, const bf16x8 (&sel)[2],
                                          const halfx8 (&sel16)[2], bf16x8 (&pfm)[4])
{
    if constexpr (PV) {
        bf16x8 ptm[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const VT vt = vt_expand<PV>(t[tt], P);
            walsh_tm(vt.t, qw * vt.tau, ptm[tt][0], ptm[tt][1]);
        }
        feat_major(ptm, sel, pfm);
    } else {
        halfx8 ptm[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) walsh_tm16(t[tt], (_Float16)qw, ptm[tt][0], ptm[tt][1]);
        feat_major16(ptm, sel16, pfm);
    }
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte reads of lanes 4j + i / 4,
// j = 0..3 (four consecutive 16-bit values read by four lanes become one
// lane's four values).
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr16(const bf16 *p)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p)));
}

// value-column operand over the chunk's tokens (same K-slot order as feat_major)
__device__ __forceinline__ bf16x8 ycol_frag(const bf16 *yc, int col)
{
    const int g = lane_id() >> 4;
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(yc + col * YCS + 4 * g);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(yc + col * YCS + 16 + 4 * g);
    return cat8(a, b);
}

// CxF register tiles of a state stored as FxC blocks [wave][s][ct][lane][4]:
// CxF (s, ct) lane (g, c16) reg r = column 16 ct + 4g + r of feature row c16.
__device__ __forceinline__ void load_state_cxf(const float *__restrict__ src, floatx4 (&acc)[4][NT])
{
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[s][ct][r] = src[(((w * 4 + s) * NT + ct) * 64 + (c16 >> 2) * 16 + 4 * g + r) * 4 + (c16 & 3)];
}

// value-row operand of 16 tokens (token-major): columns 32k + 4g + r (slots
// r < 4) and 32k + 16 + 4g + r (slots 4 + r), k = 0, 1, 2 (zero past column HD)
__device__ __forceinline__ void yrow_frags(const bf16 *yr, int row, bf16x8 (&f8)[3])
{
    const int g = lane_id() >> 4;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        f8[k] = cat8(*reinterpret_cast<const bf16x4 *>(yr + row * YRS + 32 * k + 4 * g),
                     *reinterpret_cast<const bf16x4 *>(yr + row * YRS + 32 * k + 16 + 4 * g));
}



// ---------------------------------------------------------------------------
// Hash-feature cache: fp16 t (and dt/du') of every row, in the kernels'
// register layout [head][token tile of 16][wave][lane][4]: lane (g, c16) of
// wave w holds the 4 values of table 4w + g for token 16 * tile + c16.

struct HCache {
    _Float16 *t;    // t values (null: not stored / not read)
    _Float16 *c;    // dt/du' values (null: not stored / not read)
    int64_t tiles;  // token tiles per head (2 per 32-token chunk)
};

// first element of the cache of a segment (t_begin: a multiple of 32)
template <int NW>
__device__ __forceinline__ int64_t hc_seg(const HCache &h, int64_t bh, int64_t t_begin)
{
    return (bh * h.tiles + t_begin / 16) * (int64_t)(NW * 64 * 4);
}
// the two tiles of a chunk (tiles past its valid rows are skipped)
template <int NW>
__device__ __forceinline__ Rsrc hc_res(const _Float16 *seg, const Chunk &c)
{
    return make_rsrc(seg + (c.tok0 / 16) * (NW * 64 * 4), (c.nv + 15) / 16 * (NW * 64 * 8));
}
// byte offset of this lane's 4 values in tile tt of the chunk
template <int NW> __device__ __forceinline__ int hc_lane(int tt)
{
    return ((tt * NW + wave_id()) * 64 + lane_id()) * 8;
}
template <int NW>
__device__ __forceinline__ void hc_load(Rsrc r, halfx4 (&v)[2])
{
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) v[tt] = __builtin_bit_cast(halfx4, bld64(r, hc_lane<NW>(tt)));
}
template <int NW>
__device__ __forceinline__ void hc_store(Rsrc r, int tt, const halfx4 &v)
{
    bst64(__builtin_bit_cast(u32x2, v), r, hc_lane<NW>(tt));
}

// ---------------------------------------------------------------------------
// sum_kernel: S_g = sum_{j in segment g} psi(x_j)^T y_j over the segment's
// writer rows (FxC state blocks [wave][s][ct][lane][4]).
//   SRC = 0: the rows X are hashed here; WR bit 0 / bit 1 store their t /
//            dt/du' into the cache `co`.
//   SRC = 1: t comes from the cache `ci_` (X is not read).
template <int NW, bool DVAL, int SRC, int WR, bool POLY, typename IO, int D, bool PV = false>
__global__ __launch_bounds__(NW * 64, 2) void sum_kernel(
    const IO *__restrict__ X, ValSrc<IO> vsrc, const float *__restrict__ W, int L, int P, Squash sq,
    int64_t N, int seg, int64_t nseg, HCache ci_, HCache co, float *__restrict__ st, Lens ls)
{
    constexpr int NTHR = NW * 64;
    constexpr bool HASH = SRC == 0;
    static_assert(!(HASH && D > HD), "rows of 128 elements are hashed by hash_rows_kernel");
    // double-buffered: chunk c is hashed and summed while chunk c + 1 is staged
    __shared__ __attribute__((aligned(16))) bf16 xbuf[2][HASH ? WCT * XRS : 8];
    __shared__ __attribute__((aligned(16))) float kbuf[2][WCT];
    __shared__ __attribute__((aligned(16))) bf16 ycol[2][NCOL * YCS];

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4;
    // segment-relative row pointers; chunk positions go into buffer resources
    const int64_t t_begin = sg * seg, row0 = row_base(ls, bh, N) + t_begin;
    const int tend = (int)max<int64_t>(0, min<int64_t>(valid_rows(ls, bh, N), t_begin + seg) - t_begin);
    const int nch = (tend + WCT - 1) / WCT;
    const IO *Xs = X + row0 * D;
    ValSrc<IO> vh = vsrc;
    vh.V += row0 * D;
    if (DVAL) {
        vh.O += row0 * D;
        vh.den += row0;
        if (vh.dm) vh.dm += row0;
    }
    const _Float16 *cin_t = HASH ? nullptr : ci_.t + hc_seg<NW>(ci_, bh, t_begin);
    _Float16 *cout_t = co.t ? co.t + hc_seg<NW>(co, bh, t_begin) : nullptr;
    _Float16 *cout_c = co.c ? co.c + hc_seg<NW>(co, bh, t_begin) : nullptr;
    WRows wr;
    if (HASH) load_wrows<D>(W, L, P, wr);
    const TMask tm = t_mask<PV>(P);
    const bf16x8 sel[2] = {selection(0), selection(1)};
    const halfx8 sel16[2] = {selection16(0), selection16(1)};
    const float qw = writer_scale(P, 4 * w + g < vtables(L, P));  // writer features: 2^-P, padding 0
    floatx4 af[4][NT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) af[s][ct] = {0.f, 0.f, 0.f, 0.f};
    auto chunk = [&](int ci) -> Chunk {
        if (ci >= nch) return Chunk{0, 0};
        return Chunk{ci * WCT, min(WCT, tend - ci * WCT)};
    };
    XStage<NTHR> xs;
    YStage<NTHR, DVAL> ys;
    halfx4 tc[2];
    ystage_zero_pad<NTHR>(ycol[0]);
    ystage_zero_pad<NTHR>(ycol[1]);
    const Chunk c0 = chunk(0), c1 = chunk(1);
    ystage_load<NTHR, DVAL, D>(yres<DVAL, D>(vh, c0), ys);
    if (HASH) {
        xstage_load<NTHR, false, D>(row_res<D>(Xs, c0), xs);
        xstage_store<NTHR, false, IO>(xs, xbuf[0], kbuf[0]);
    } else {
        hc_load<NW>(hc_res<NW>(cin_t, c0), tc);
    }
    ystage_store<NTHR, DVAL, IO, D>(ys, c0.nv, ycol[0]);
    if (HASH) xstage_load<NTHR, false, D>(row_res<D>(Xs, c1), xs);
    ystage_load<NTHR, DVAL, D>(yres<DVAL, D>(vh, c1), ys);
    lds_barrier();
    vm_drain();
    for_chunks2(nch, [&](int ci, auto par) {
        constexpr int b = decltype(par)::v;
        const Chunk cc = chunk(ci);
        // stage chunk ci + 1 (loaded one iteration ago) into the other buffers,
        // which were last read before the previous barrier, then prefetch ci + 2
        if (ci + 1 < nch) {
            if (HASH) xstage_store<NTHR, false, IO>(xs, xbuf[b ^ 1], kbuf[b ^ 1]);
            ystage_store<NTHR, DVAL, IO, D>(ys, chunk(ci + 1).nv, ycol[b ^ 1]);
        }
        const halfx4 tcur[2] = {tc[0], tc[1]};
        if (HASH)
            xstage_load<NTHR, false, D>(row_res<D>(Xs, chunk(ci + 2)), xs);
        else
            hc_load<NW>(hc_res<NW>(cin_t, chunk(ci + 1)), tc);
        ystage_load<NTHR, DVAL, D>(yres<DVAL, D>(vh, chunk(ci + 2)), ys);
        if (!HASH) pin_loads();
        bf16x8 pfm[4];
        Rsrc rto, rco;
        if constexpr (HASH && (WR & 1) != 0) rto = hc_res<NW>(cout_t, cc);
        if constexpr (HASH && (WR & 2) != 0) rco = hc_res<NW>(cout_c, cc);
        halfx4 tw[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            if constexpr (HASH) {
                halfx4 c;
                hash_staged<POLY, (WR & 2) != 0>(xbuf[b], kbuf[b], tt, wr, sq, tm, tw[tt], c);
                if constexpr ((WR & 2) != 0) hc_store<NW>(rco, tt, c);
                if constexpr ((WR & 1) != 0) hc_store<NW>(rto, tt, tw[tt]);
            } else {
                tw[tt] = tcur[tt];
            }
        }
        if constexpr (HASH) prio<1>();
        writer_fm<PV>(tw, P, qw, sel, sel16, pfm);
        // tokens past the end have psi_0 = 1/4 but zero value rows
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            const bf16x8 yb = ycol_frag(ycol[b], ct * 16 + (lane & 15));
#pragma unroll
            for (int s = 0; s < 4; ++s) mma32(af[s][ct], pfm[s], yb);
        }
        if constexpr (HASH) prio<0>();
        lds_barrier();
    });
    const int64_t blk = (bh * (nseg + 1) + sg) * (int64_t)(NW * 64 * NCOL);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
            *reinterpret_cast<floatx4 *>(st + blk + st_idx(w, s, ct, lane, 4)) = af[s][ct];
}

// ---------------------------------------------------------------------------
// walk_kernel: reader rows read an FxC state built from writer rows, in
// chunks of 32 tokens, NW waves of 4 tables each.
//   BWD = false: readers = queries, writers = keys, y = [v | 1]; token order;
//                intra mask j <= i; output O = n / m and den = m.
//   BWD = true:  readers = keys, writers = queries, y = [dO/m | dm]; reverse
//                order; intra mask j >= i; output dV = n[:, :d].
//   Readers: RSRC = 0 hashes the rows R (RWR bit 0 / 1 store t / dt/du' into
//   the cache rc); RSRC = 1 reads t from rc.  Writers: t from the cache wc.
// Outputs are formed transposed (value columns x tokens: the state and value
// operands are the A side of the MFMAs), so that a lane ends up with four
// consecutive columns of one token.
// One barrier per chunk: staging buffers and the partial outputs are double
// buffered, and the partial outputs of chunk c are summed after the barrier
// of chunk c + 1, beside that chunk's products.
template <int NW, bool CAUSAL, bool BWD, int RSRC, int RWR, bool POLY, typename IO, int D,
          int PART = PART_NONE, bool PV = false>
__global__ __launch_bounds__(NW * 64, 2) void walk_kernel(
    const IO *__restrict__ R, ValSrc<IO> vsrc, const float *__restrict__ W, int L, int P, Squash sq,
    int64_t N, int seg, int64_t nseg, const float *__restrict__ st, HCache rc, HCache wc,
    IO *__restrict__ Out, float *__restrict__ den, Lens ls, Part part)
{
    constexpr int NTHR = NW * 64;
    constexpr bool HASH = RSRC == 0;
    static_assert(!(HASH && D > HD), "rows of 128 elements are hashed by hash_rows_kernel");
    constexpr int RSLOTS = 2 * 4 * 64;  // (token tile, value column tile < 4, lane) output slots
    constexpr int RIT = (RSLOTS + NTHR - 1) / NTHR;
    constexpr int REDN = NW * 2 * 4 * 64 * 4;  // partial outputs: value columns (4 tiles) of every wave
    constexpr int REDM = NW * 2 * 64;          // and their count column
    // Workgroups of 8 waves fill a compute unit (two waves per SIMD at up to
    // 256 registers) and double-buffer the partial outputs, so that a chunk
    // needs one barrier.  Narrower workgroups (fewer tables) run two or more
    // per compute unit, which LDS allows only with one buffer: the chunk then
    // takes a second barrier before it overwrites the sums the previous
    // chunk's finish reads.
    constexpr int NRED = NW >= 8 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) bf16 xbuf[2][HASH ? WCT * XRS : 8];
    __shared__ __attribute__((aligned(16))) float kbuf[2][WCT];
    __shared__ __attribute__((aligned(16))) bf16 ycol[2][CAUSAL ? NCOL * YCS : 8];
    // [NRED][REDN + REDM]; before the loop the forward's W rows are staged here
    __shared__ __attribute__((aligned(16))) float red[NRED * (REDN + REDM)];
    __shared__ __attribute__((aligned(16))) bf16 sl[2 * 64 * 8];
    static_assert(!HASH || 2 * NW * 16 * XRS * 2 <= NRED * (REDN + REDM) * 4, "W rows fit the partial-output buffer");

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    // segment-relative row pointers; chunk positions go into buffer resources
    const int64_t t_begin = sg * seg, row0 = row_base(ls, bh, N) + t_begin;
    const int tend = (int)max<int64_t>(0, min<int64_t>(valid_rows(ls, bh, N), t_begin + seg) - t_begin);
    const int nch = (tend + WCT - 1) / WCT;
    const IO *Rs = R + row0 * D;
    ValSrc<IO> vh = vsrc;
    vh.V += row0 * D;
    if (BWD) {
        vh.O += row0 * D;
        vh.den += row0;
        if (vh.dm) vh.dm += row0;
    }
    IO *Os = Out + row0 * D;
    float *pv = PART != PART_NONE ? part.v + row0 * HD : nullptr;
    float *pm = PART != PART_NONE && !BWD ? part.m + row0 : nullptr;
    float *dens = BWD ? nullptr : den + row0;
    const _Float16 *rt_seg = rc.t ? rc.t + hc_seg<NW>(rc, bh, t_begin) : nullptr;
    const _Float16 *rc_seg = rc.c ? rc.c + hc_seg<NW>(rc, bh, t_begin) : nullptr;
    const _Float16 *wt_seg = wc.t ? wc.t + hc_seg<NW>(wc, bh, t_begin) : nullptr;

    WRows wr;  // the forward's W rows (hi, lo), kept in registers
    if (HASH) stage_wrows<NW, D>(W, L, P, reinterpret_cast<bf16 *>(red));
    const TMask tm = t_mask<PV>(P);
    stage_sel(sl);
    __syncthreads();
    // red is next written after two more barriers
    if (HASH) wrows_lds<NW>(reinterpret_cast<const bf16 *>(red), wr);
    const float qw = writer_scale(P, 4 * w + g < vtables(L, P));  // writer features: 2^-P, padding 0
    floatx4 acc[4][NT];
    {
        const float *src = st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(NW * 64 * NCOL);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct)
                acc[s][ct] = *reinterpret_cast<const floatx4 *>(src + st_idx(w, s, ct, lane, 4));
    }
    // chunks in walk order
    auto chunk = [&](int ci) -> Chunk {
        if (ci < 0 || ci >= nch) return Chunk{0, 0};
        const int t0 = (BWD ? nch - 1 - ci : ci) * WCT;
        return Chunk{t0, min(WCT, tend - t0)};
    };

    XStage<NTHR> xs;
    YStage<NTHR, BWD> ys;
    halfx4 rt[2], wt[2];
    const Chunk c0 = chunk(0);
    if (CAUSAL) {
        ystage_zero_pad<NTHR>(ycol[0]);
        ystage_zero_pad<NTHR>(ycol[1]);
        ystage_load<NTHR, BWD, D>(yres<BWD, D>(vh, c0), ys);
        hc_load<NW>(hc_res<NW>(wt_seg, c0), wt);
    }
    if (HASH) {
        xstage_load<NTHR, false, D>(row_res<D>(Rs, c0), xs);
        xstage_store<NTHR, false, IO>(xs, xbuf[0], kbuf[0]);
        xstage_load<NTHR, false, D>(row_res<D>(Rs, chunk(1)), xs);
    } else {
        hc_load<NW>(hc_res<NW>(rt_seg, c0), rt);
    }
    lds_barrier();

    // Walsh features of chunk ci's readers: hashed from the rows staged in
    // buffer xb (storing t and dt/du' to the cache as asked), or from the
    // cached t of the chunk (rt, which then takes the next chunk's t)
    auto reader_feats = [&](int ci, const bf16 *xb, const float *kb, bf16x8 (&pr)[2][2]) {
        const Chunk c = chunk(ci);
        Rsrc rto, rco;
        if constexpr (HASH && (RWR & 1) != 0) rto = hc_res<NW>(rt_seg, c);
        if constexpr (HASH && (RWR & 2) != 0) rco = hc_res<NW>(rc_seg, c);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            halfx4 t;
            if constexpr (HASH) {
                halfx4 cd;
                hash_staged<POLY, (RWR & 2) != 0>(xb, kb, tt, wr, sq, tm, t, cd);
                if constexpr ((RWR & 2) != 0) hc_store<NW>(rco, tt, cd);
                if constexpr ((RWR & 1) != 0) hc_store<NW>(rto, tt, t);
            } else {
                t = rt[tt];
            }
            const VT vt = vt_expand<PV>(t, P);
            walsh_tm(vt.t, vt.tau, pr[tt][0], pr[tt][1]);
        }
        if (!HASH) hc_load<NW>(hc_res<NW>(rt_seg, chunk(ci + 1)), rt);
    };
    // Reader features from the cache are formed one chunk ahead, beside the
    // products of the chunk before (this helps there but not where the rows
    // are hashed, which happens before the chunk's barrier)
    constexpr bool PIPE = !HASH;
    bf16x8 prc[2][2];  // reader features of the current chunk
    if constexpr (PIPE) reader_feats(0, xbuf[0], kbuf[0], prc);

    // Sum of the partial outputs of chunk c (buffer c & 1) and its output
    // rows: O = n / m (m formed per token from the count column) and den = m,
    // or dV = n.  Thread slot: token tile tt, column tile ct, lane (g, c16).
    auto finish = [&](int ci, int pb) {
        const Chunk c = chunk(ci);
        const float *rn = red + (NRED == 2 ? pb : 0) * (REDN + REDM), *rm = rn + REDN;
        const Rsrc ro = row_res<D>(Os, c);
#pragma unroll
        for (int it = 0; it < RIT; ++it) {
            const int sl_ = threadIdx.x + it * NTHR;
            // branch-free where every slot is taken, so that this joins the
            // block of the products
            if (RSLOTS % NTHR == 0 || sl_ < RSLOTS) {
                const int tt = sl_ >> 8, ct = (sl_ >> 6) & 3, ln = sl_ & 63;
                floatx4 n = *reinterpret_cast<const floatx4 *>(rn + ((tt * 4 + ct) * 64 + ln) * 4);
#pragma unroll
                for (int ww = 1; ww < NW; ++ww)
                    n += *reinterpret_cast<const floatx4 *>(rn + (((ww * 2 + tt) * 4 + ct) * 64 + ln) * 4);
                const int col = 16 * ct + 4 * (ln >> 4);  // columns past D are not stored
                const int off = (D == HD || col < D) ? (tt * 16 + (ln & 15)) * (D * 2) + col * 2 : OOB;
                const int tok = tt * 16 + (ln & 15);
                if constexpr (PART != PART_NONE) {
                    const Rsrc rp = make_rsrc(pv + c.tok0 * HD, c.nv * HD * 4);
                    if constexpr (PART != PART_OUT)
                        n += __builtin_bit_cast(floatx4, bld128(rp, tok * (HD * 4) + col * 4));
                    if constexpr (PART == PART_OUT || PART == PART_MID)
                        bst128(__builtin_bit_cast(u32x4, n), rp, tok * (HD * 4) + col * 4);
                }
                if (BWD) {
                    if constexpr (PART == PART_NONE || PART == PART_IN)
                        bst64(u32x2{pk_io<IO>(n[0], n[1]), pk_io<IO>(n[2], n[3])}, ro, off);
                } else {
                    float m = rm[tt * 64 + (ln & 15)];
#pragma unroll
                    for (int ww = 1; ww < NW; ++ww) m += rm[(ww * 2 + tt) * 64 + (ln & 15)];
                    const int moff = (ct == 0 && ln < 16) ? tok * 4 : OOB;
                    if constexpr (PART == PART_OUT || PART == PART_MID) {
                        if constexpr (PART == PART_MID) m += bldf(make_rsrc(pm + c.tok0, c.nv * 4), tok * 4);
                        bstf(m, make_rsrc(pm + c.tok0, c.nv * 4), moff);
                    } else {
                        if constexpr (PART == PART_IN) m += bldf(make_rsrc(pm + c.tok0, c.nv * 4), tok * 4);
                        // m = 0 only under hard hashing (no colliding key): o = 0
                        const float inv = m != 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
                        bst64(u32x2{pk_io<IO>(n[0] * inv, n[1] * inv), pk_io<IO>(n[2] * inv, n[3] * inv)}, ro, off);
                        bstf(m, make_rsrc(dens + c.tok0, c.nv * 4), moff);
                    }
                }
            }
        }
    };

    vm_drain();
    for_chunks2(nch, [&](int ci, auto par) {
        constexpr int b = decltype(par)::v;
        const Chunk cc = chunk(ci), cn = chunk(ci + 1);
        if (CAUSAL) {
            ystage_store<NTHR, BWD, IO, D>(ys, cc.nv, ycol[b]);
            ystage_load<NTHR, BWD, D>(yres<BWD, D>(vh, cn), ys);
        }
        bf16x8 pr[2][2];
        if constexpr (PIPE) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int k = 0; k < 2; ++k) pr[tt][k] = prc[tt][k];
        } else {
            reader_feats(ci, xbuf[b], kbuf[b], pr);
        }
        bf16x8 pfm[4];
        bf16x8 kA1;   // single-tile scores (fwd: reader tile 0, bwd: reader tile 1)
        bf16x8 kA8;   // two-tile scores (fwd: reader tile 1, bwd: reader tile 0)
        if (HASH) {  // the next chunk's rows into the other buffer (last read before the previous barrier)
            if (ci + 1 < nch) xstage_store<NTHR, false, IO>(xs, xbuf[b ^ 1], kbuf[b ^ 1]);
            xstage_load<NTHR, false, D>(row_res<D>(Rs, chunk(ci + 2)), xs);
        }
        lds_barrier();  // value columns and next rows staged; partial outputs of chunk ci - 1 in LDS
        finish(ci - 1, b ^ 1);  // (none before the first chunk: its stores are dropped)
        __builtin_amdgcn_sched_barrier(0);
        prio<1>();
        // the next chunk's reader features, computed beside this chunk's
        // products (past the last chunk: nothing is read or stored)
        if constexpr (PIPE) reader_feats(ci + 1, xbuf[b ^ 1], kbuf[b ^ 1], prc);
        // writer features, masked scores and feature-major operands, next to
        // the MFMA-bound products that consume them
        if (CAUSAL) {
            bf16x8 pw[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const VT vt = vt_expand<PV>(wt[tt], P);
                walsh_tm(vt.t, qw * vt.tau, pw[tt][0], pw[tt][1]);
            }
            hc_load<NW>(hc_res<NW>(wt_seg, cn), wt);
            // scores^T tiles D[j][i] = psi_w(j) . psi_r(i) over this wave's tables
            constexpr int TJ[3] = {0, BWD ? 1 : 0, 1}, TI[3] = {0, BWD ? 0 : 1, 1};
            floatx4 sc[3];
#pragma unroll
            for (int pi = 0; pi < 3; ++pi) {
                sc[pi] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 2; ++k) mma32(sc[pi], pw[TJ[pi]][k], pr[TI[pi]][k]);
            }
            // diagonal tiles: keep j <= i (fwd) or j >= i (bwd); lane (j = 4g + r, i = c16)
#pragma unroll
            for (int pi = 0; pi < 3; pi += 2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = BWD ? (4 * g + r >= c16) : (4 * g + r <= c16);
                    sc[pi][r] = keep ? sc[pi][r] : 0.f;
                }
            // operands over both writer tiles (the masked-out tile is zero)
            const bf16x4 z4 = pk4(0, 0);
            if (BWD) {
                kA8 = cat8(acc2bf4(sc[0]), acc2bf4(sc[1]));  // reader tile 0: writer tiles 0, 1
                kA1 = cat8(z4, acc2bf4(sc[2]));              // reader tile 1: writer tile 1
            } else {
                kA1 = cat8(acc2bf4(sc[0]), z4);              // reader tile 0: writer tile 0
                kA8 = cat8(acc2bf4(sc[1]), acc2bf4(sc[2]));  // reader tile 1: writer tiles 0, 1
            }
            bf16x8 sel[2];
            sel_lds(sl, sel);
            feat_major(pw, sel, pfm);
        }
        // O^T tiles (tt, ct): lane (columns 16 ct + 4g + r, token 16 tt + c16)
        floatx4 oacc[2][NT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) oacc[tt][ct] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            // inter-chunk readout with the state before this chunk
            bf16x8 sf[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) sf[k] = cat8(acc2bf4(acc[2 * k][ct]), acc2bf4(acc[2 * k + 1][ct]));
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma32(oacc[tt][ct], sf[k], pr[tt][k]);
            if (CAUSAL) {
                const bf16x8 yb = ycol_frag(ycol[b], ct * 16 + c16);
                mma32(oacc[0][ct], yb, BWD ? kA8 : kA1);
                mma32(oacc[1][ct], yb, BWD ? kA1 : kA8);
#pragma unroll
                for (int s = 0; s < 4; ++s) mma32(acc[s][ct], pfm[s], yb);
            }
        }
        // ask the scheduler to interleave the products with the vector work of
        // this block (writer features, score masks, state conversions): one
        // MFMA, then up to three VALU instructions, which co-issue with it
#pragma unroll
        for (int i = 0; i < 40; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
        if constexpr (NRED == 1) lds_barrier();  // every finish(ci - 1) has read the sums
        float *rn = red + (NRED == 2 ? b : 0) * (REDN + REDM), *rm = rn + REDN;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                *reinterpret_cast<floatx4 *>(rn + (((w * 2 + tt) * 4 + ct) * 64 + lane) * 4) = oacc[tt][ct];
            // the count column (64) is row 0 of column tile 4: register 0 of lanes
            // 0..15 (the other lanes' values are not read)
            if (!BWD) rm[(w * 2 + tt) * 64 + lane] = oacc[tt][4][0];
        }
        prio<0>();
    });
    if (nch > 0) {
        lds_barrier();
        finish(nch - 1, (nch - 1) & 1);
    }
}

// ---------------------------------------------------------------------------
// grad_kernel: gradient of the reader rows, which read a state built from the
// writer rows, and back through the readers' hash.
//   dQ (REVERSE = false): readers = queries with values D = [dO/m | dm],
//       writers = keys with values [v | 1]; token order; mask j <= i.
//   dK (REVERSE = true): readers = keys with values [v | 1], writers =
//       queries with values D; reverse order; mask j >= i.
// Reader t and dt/du' come from the cache rc, writer t from wc; the raw
// reader rows are staged for the normalisation backward.
// Per chunk: dpsi_r(i)[f] = sum_c S[f][c] y_r(i)[c] + sum_j E[i][j] psi_w(j)[f]
// with E[i][j] = y_r(i) . y_w(j) (masked), computed transposed (rows f) so
// that a lane holds all 16 features of its table; S += psi_w^T y_w; then the
// Walsh gradient, du = dt dt/du', dxh = du W and the normalisation backward.
// DW: also the gradient of the projection, dW = sum over the reader rows of
// du x_hat^T: per chunk and wave, [16 hyperplanes x 32 tokens] x [32 tokens x
// 64 dims] on MFMA (both operands read transposed from du and the staged
// rows), summed in LDS, and the workgroup's sum written to dwp[workgroup]
// ([NW * 16][64] fp32) for a reduction over segments.
// D = 128 (rows of 128 elements, in two passes of 64 value columns): the
// kernel stops at du, which it stores (bf16, [row][NW * 16], at dwp) for
// du_rows_kernel, which adds the passes and forms dx_hat = du W and the
// normalisation backward over the whole row.
template <int NW, bool CAUSAL, bool REVERSE, bool DW, typename IO, int D, int PART = PART_NONE,
          bool PV = false>
__global__ __launch_bounds__(NW * 64, 2) void grad_kernel(
    const IO *__restrict__ Xr, ValSrc<IO> vr_src, ValSrc<IO> vw_src,
    const float *__restrict__ W, int L, int P, int64_t N, int seg, int64_t nseg,
    const float *__restrict__ st, HCache rc, HCache wc, IO *__restrict__ dX,
    float *__restrict__ dwp, Lens ls, Part part)
{
    constexpr bool RD = !REVERSE;  // the readers carry the gradient values D
    constexpr bool DUO = D > HD;   // store du, no dx_hat here
    static_assert(!DUO || (!DW && PART == PART_NONE), "rows of 128: du only");
    constexpr int NTHR = NW * 64;
    constexpr int DUS = NW * 16 + 8;  // du row stride (bf16)
    constexpr int TPWV = 8 / NW;      // dxh tiles per wave
    constexpr int WTS = NW * 16 + 8;  // staged W^T row stride
    // staging buffers, du and the partial dots are double buffered: one
    // barrier per chunk
    __shared__ __attribute__((aligned(16))) bf16 xbuf[2][WCT * XRS];
    __shared__ __attribute__((aligned(16))) float kbuf[2][WCT];
    __shared__ __attribute__((aligned(16))) bf16 yrow_r[2][WCT * YRS];
    __shared__ __attribute__((aligned(16))) bf16 yrow_w[2][CAUSAL ? WCT * YRS : 8];
    __shared__ __attribute__((aligned(16))) bf16 ycol_w[2][CAUSAL ? NCOL * YCS : 8];
    __shared__ __attribute__((aligned(16))) bf16 du_l[2][WCT * DUS];
    // partial x . dxh [token][nt][g]; rows of 20 words, so that the 16 tokens
    // of a tile fall in different banks (rows of 16 put them in 2)
    constexpr int DPS = 20;
    __shared__ __attribute__((aligned(16))) float dotp[2][WCT * DPS];
    __shared__ __attribute__((aligned(16))) bf16 wt_l[HD * WTS];     // W^T (bf16): [dim][hyperplane]
    // this block's dW as [hyperplane / 4][column][hyperplane % 4]: a lane's
    // four accumulator values are one 16-byte word (each wave owns its rows)
    __shared__ __attribute__((aligned(16))) float dwl[DW ? NW * 16 * HD : 4];
    __shared__ __attribute__((aligned(16))) bf16 sl[2 * 64 * 8];

    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    // segment-relative row pointers; chunk positions go into buffer resources
    const int64_t t_begin = sg * seg, row0 = row_base(ls, bh, N) + t_begin;
    const int tend = (int)max<int64_t>(0, min<int64_t>(valid_rows(ls, bh, N), t_begin + seg) - t_begin);
    const int nch = (tend + WCT - 1) / WCT;
    const IO *Rs = Xr + row0 * D;
    ValSrc<IO> vrh = vr_src, vwh = vw_src;
    vrh.V += row0 * D;
    vwh.V += row0 * D;
    if (RD) {
        vrh.O += row0 * D;
        vrh.den += row0;
        if (vrh.dm) vrh.dm += row0;
    } else {
        vwh.O += row0 * D;
        vwh.den += row0;
        if (vwh.dm) vwh.dm += row0;
    }
    IO *dXs = dX + row0 * D;
    bf16 *dug = DUO ? reinterpret_cast<bf16 *>(dwp) + row0 * (NW * 16) : nullptr;
    float *pv = PART != PART_NONE ? part.v + row0 * HD : nullptr;
    const _Float16 *rt_seg = rc.t + hc_seg<NW>(rc, bh, t_begin);
    const _Float16 *rc_seg = rc.c + hc_seg<NW>(rc, bh, t_begin);
    const _Float16 *wt_seg = wc.t ? wc.t + hc_seg<NW>(wc, bh, t_begin) : nullptr;

    // W^T and the selection operands, once per workgroup.  dxh = du W takes W
    // in bf16, the precision of du itself (the forward projection keeps W to
    // about 16 bits as bf16 hi + lo).  With writer features scaled by 2^-P and
    // reader features by 1, the products below give the gradient with respect
    // to the unscaled reader features prod t_p, so that walsh_grad yields dt
    // itself.
    if constexpr (!DUO)
        for (int e = threadIdx.x; e < NW * 16 * HD; e += NTHR) {
            const int hp = e / HD, c = e % HD;
            wt_l[c * WTS + hp] = (bf16)w_elem(W, L, P, D, hp, c);
        }
    if constexpr (DW)
        for (int e = threadIdx.x; e < NW * 16 * HD; e += NTHR) dwl[e] = 0.f;
    if constexpr (PV)
        stage_sel(sl);
    else
        stage_sel16(reinterpret_cast<_Float16 *>(sl));
    // the selection operands are read in the first chunk before its barrier
    // (and a wave whose W rows are all padding reaches that read early)
    __syncthreads();
    const float qw = writer_scale(P, 4 * w + g < vtables(L, P));  // writer features: 2^-P, padding 0
    floatx4 acc[4][NT];  // CxF state
    load_state_cxf(st + (bh * (nseg + 1) + (CAUSAL ? sg : nseg)) * (int64_t)(NW * 64 * NCOL), acc);

    auto chunk = [&](int ci) -> Chunk {
        if (ci < 0 || ci >= nch) return Chunk{0, 0};
        const int t0 = (REVERSE ? nch - 1 - ci : ci) * WCT;
        return Chunk{t0, min(WCT, tend - t0)};
    };

    XStage<NTHR> xs;
    YStage<NTHR, RD> ysr;
    YStage<NTHR, !RD> ysw;
    halfx4 rt[2], rcv[2], wt[2];
    const Chunk c0 = chunk(0);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
        yrow_zero_pad<NTHR>(yrow_r[pb]);
        if (CAUSAL) {
            yrow_zero_pad<NTHR>(yrow_w[pb]);
            ystage_zero_pad<NTHR>(ycol_w[pb]);
        }
    }
    if (CAUSAL) {
        ystage_load<NTHR, !RD, D>(yres<!RD, D>(vwh, c0), ysw);
        hc_load<NW>(hc_res<NW>(wt_seg, c0), wt);
    }
    ystage_load<NTHR, RD, D>(yres<RD, D>(vrh, c0), ysr);
    hc_load<NW>(hc_res<NW>(rt_seg, c0), rt);
    hc_load<NW>(hc_res<NW>(rc_seg, c0), rcv);
    if constexpr (!DUO) xstage_load<NTHR, true, D>(row_res<D>(Rs, c0), xs);

    // dxh = du W of chunk ci (du in buffer pb) for this wave's tiles; the
    // partial dots with x go to dotp[pb], dxh, x and |x|^2 stay in registers
    // until every wave's dots are in LDS.  Tile (tt, nt) = wave + NW i; lane
    // (g, c16): token 16 tt + c16, dims 16 nt + 4g + r.
    floatx4 dxh[TPWV];
    bf16x4 xkeep[TPWV];
    float sskeep[TPWV];
    // (ci: the chunk whose du is in buffer pb, for the partial sums of dx_hat)
    auto dxh_tiles = [&](int pb, int ci) {
        Rsrc rp;
        if constexpr (PART != PART_NONE) {
            const Chunk c = chunk(ci);
            rp = make_rsrc(pv + c.tok0 * HD, c.nv * HD * 4);
        }
#pragma unroll
        for (int i = 0; i < TPWV; ++i) {
            const int tile = w + NW * i, tt = tile >> 2, nt = tile & 3, tok = tt * 16 + c16;
            floatx4 xa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NW / 2; ++k) {
                const bf16x8 dub = *reinterpret_cast<const bf16x8 *>(du_l[pb] + tok * DUS + 32 * k + 8 * g);
                const bf16 *wrow = wt_l + (nt * 16 + c16) * WTS + 32 * k + 8 * g;
                mma32(xa, *reinterpret_cast<const bf16x8 *>(wrow), dub);
            }
            if constexpr (PART == PART_IN || PART == PART_MID)
                xa += __builtin_bit_cast(floatx4, bld128(rp, tok * (HD * 4) + (nt * 16 + 4 * g) * 4));
            if constexpr (PART == PART_OUT || PART == PART_MID) {
                bst128(__builtin_bit_cast(u32x4, xa), rp, tok * (HD * 4) + (nt * 16 + 4 * g) * 4);
                continue;
            }
            const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xbuf[pb] + tok * XRS + nt * 16 + 4 * g);
            float dot = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) dot = fmaf(xa[r], (float)xv[r], dot);
            dotp[pb][tok * DPS + nt * 4 + g] = dot;
            dxh[i] = xa;
            xkeep[i] = xv;
            sskeep[i] = kbuf[pb][tok];
        }
    };
    // dW of chunk ci's rows (du in buffer pb, rows in xbuf[pb]): A = du^T
    // scaled per token by 1 / max(|x|, 1e-12) (x_hat = x / that), K-slot
    // (g, j) <-> token 8g + j for both operands
    auto dw_tiles = [&](int pb) {
        const int tq = c16 & 3, tj = c16 >> 2;
        const bf16 *da = du_l[pb] + (8 * g + tj) * DUS + w * 16 + 4 * tq;
        bf16x8 a = cat8(lds_tr16(da), lds_tr16(da + 4 * DUS));
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float ss = kbuf[pb][8 * g + j];
            a[j] = (bf16)((float)a[j] * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)));
        }
        const bf16 *xa = xbuf[pb] + (8 * g + tj) * XRS + 4 * tq;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const bf16x8 bx = cat8(lds_tr16(xa + 16 * nt), lds_tr16(xa + 16 * nt + 4 * XRS));
            // rows 4g + r of this wave's 16, column 16 nt + c16
            floatx4 *acc4 = reinterpret_cast<floatx4 *>(dwl + ((w * 4 + g) * HD + 16 * nt + c16) * 4);
            floatx4 v = *acc4;
            mma32(v, a, bx);
            *acc4 = v;
        }
    };
    // the normalisation backward of chunk ci from the registers above and the
    // dots in dotp[pb]: dx = (dxh - x (x . dxh) / |x|^2) / |x| for
    // |x| > 1e-12, else dxh 1e12
    auto finish = [&](int ci, int pb) {
        if constexpr (PART == PART_OUT || PART == PART_MID) return;  // dx_hat went to the partial sums
        const Rsrc rdx = row_res<D>(dXs, chunk(ci));
#pragma unroll
        for (int i = 0; i < TPWV; ++i) {
            const int tile = w + NW * i, tt = tile >> 2, nt = tile & 3, tok = tt * 16 + c16;
            float dot = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const floatx4 v = *reinterpret_cast<const floatx4 *>(dotp[pb] + tok * DPS + 4 * q);
                dot += (v[0] + v[1]) + (v[2] + v[3]);
            }
            const float ss = sskeep[i];
            const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
            const float coef = ss > 1e-24f ? dot * inv * inv : 0.f;
            float rv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) rv[r] = (dxh[i][r] - coef * (float)xkeep[i][r]) * inv;
            const u32x2 v = {pk_io<IO>(rv[0], rv[1]), pk_io<IO>(rv[2], rv[3])};
            const int col = nt * 16 + 4 * g;  // columns past D are not stored
            bst64(v, rdx, (D == HD || col < D) ? tok * (D * 2) + col * 2 : OOB);
        }
    };

    // Chunk ci: its value rows are staged before the barrier; after it, the
    // normalisation backward of chunk ci - 2 (whose dots are complete), chunk
    // ci's rows and products, and last dxh of chunk ci - 1 (whose du is
    // complete).
    vm_drain();
    for (int ci = 0; ci < nch; ++ci) {
        const int b = ci & 1;
        const Chunk cc = chunk(ci), cn = chunk(ci + 1);
        ystage_store<NTHR, RD, IO, D>(ysr, cc.nv, nullptr, yrow_r[b]);
        if (CAUSAL) ystage_store<NTHR, !RD, IO, D>(ysw, cc.nv, ycol_w[b], yrow_w[b]);
        ystage_load<NTHR, RD, D>(yres<RD, D>(vrh, cn), ysr);
        if (CAUSAL) ystage_load<NTHR, !RD, D>(yres<!RD, D>(vwh, cn), ysw);
        const halfx4 trh[2] = {rt[0], rt[1]}, crh[2] = {rcv[0], rcv[1]};
        hc_load<NW>(hc_res<NW>(rt_seg, cn), rt);
        hc_load<NW>(hc_res<NW>(rc_seg, cn), rcv);
        bf16x8 pfm[4];
        if (CAUSAL) {
            const halfx4 wcur[2] = {wt[0], wt[1]};
            hc_load<NW>(hc_res<NW>(wt_seg, cn), wt);
            bf16x8 sel[2];
            halfx8 sel16[2];
            if constexpr (PV)
                sel_lds(sl, sel);
            else
                sel_lds16(reinterpret_cast<const _Float16 *>(sl), sel16);
            writer_fm<PV>(wcur, P, qw, sel, sel16, pfm);
        }
        lds_barrier();  // value rows of this chunk; du and rows of ci - 1; dots of ci - 2
        if constexpr (!DUO) {
            finish(ci - 2, b);  // (branch-free: before the first chunks the stores are dropped)
            // this chunk's raw rows (the buffer was last read by dxh of ci - 2)
            xstage_store<NTHR, true, IO>(xs, xbuf[b], kbuf[b]);
            xstage_load<NTHR, true, D>(row_res<D>(Rs, cn), xs);
        }
        // reader value rows as B operands (token-major)
        bf16x8 yb8[2][3];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) yrow_frags(yrow_r[b], tt * 16 + c16, yb8[tt]);
        floatx4 dps[4][2];  // dpsi^T tiles (s, tt): lane (rows 4g + r <-> S = 4s + r of table 4w + g, token c16)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) dps[s][tt] = {0.f, 0.f, 0.f, 0.f};
        bf16x8 eb8, eb1;
        if (CAUSAL) {
            // E^T tiles D[j][i] = y_w(j) . y_r(i) over all value columns
            constexpr int TJ[3] = {0, REVERSE ? 1 : 0, 1}, TI[3] = {0, REVERSE ? 0 : 1, 1};
            floatx4 et[3];
#pragma unroll
            for (int pi = 0; pi < 3; ++pi) et[pi] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tj = 0; tj < 2; ++tj) {
                bf16x8 wa8[3];
                yrow_frags(yrow_w[b], tj * 16 + c16, wa8);
#pragma unroll
                for (int pi = 0; pi < 3; ++pi) {
                    if (TJ[pi] != tj) continue;
#pragma unroll
                    for (int k = 0; k < 3; ++k) mma32(et[pi], wa8[k], yb8[TI[pi]][k]);
                }
            }
#pragma unroll
            for (int pi = 0; pi < 3; pi += 2)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool keep = REVERSE ? (4 * g + r >= c16) : (4 * g + r <= c16);
                    et[pi][r] = keep ? et[pi][r] : 0.f;
                }
            // operands over both writer tiles (the masked-out tile is zero)
            const bf16x4 z4 = pk4(0, 0);
            if (REVERSE) {
                eb8 = cat8(acc2bf4(et[0]), acc2bf4(et[1]));  // reader tile 0: writer tiles 0, 1
                eb1 = cat8(z4, acc2bf4(et[2]));              // reader tile 1: writer tile 1
            } else {
                eb1 = cat8(acc2bf4(et[0]), z4);              // reader tile 0: writer tile 0
                eb8 = cat8(acc2bf4(et[1]), acc2bf4(et[2]));  // reader tile 1: writer tiles 0, 1
            }
        }
        // inter-chunk part with the state before this chunk (consecutive
        // products go to the two token tiles' independent accumulators)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 sa[3];
            sa[0] = cat8(acc2bf4(acc[s][0]), acc2bf4(acc[s][1]));
            sa[1] = cat8(acc2bf4(acc[s][2]), acc2bf4(acc[s][3]));
            // columns 80 .. 95 of the value rows are zero: any finite upper half
            const bf16x4 s4 = acc2bf4(acc[s][4]);
            sa[2] = cat8(s4, s4);
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma32(dps[s][tt], sa[k], yb8[tt][k]);
            if (CAUSAL) {
                mma32(dps[s][0], pfm[s], REVERSE ? eb8 : eb1);
                mma32(dps[s][1], pfm[s], REVERSE ? eb1 : eb8);
            }
        }
        if (CAUSAL) {
            // S += psi_w^T y_w (after every read of the state above)
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                const bf16x8 ya = ycol_frag(ycol_w[b], ct * 16 + c16);  // rows = value columns
#pragma unroll
                for (int s = 0; s < 4; ++s) mma32(acc[s][ct], ya, pfm[s]);
            }
        }
        // Walsh gradient -> du of this wave's 16 hyperplanes (token-major, LDS)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float dp[16], dt[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) dp[4 * s + r] = dps[s][tt][r];
            const VT vt = vt_expand<PV>(trh[tt], P);
            const float dtau = walsh_grad(dp, vt.t, dt);
            vt_reduce<PV>(vt, P, dtau, dt);
            const floatx4 cr = to_f4(crh[tt]);
            const bf16x4 du = pk4(pk_bf16(dt[0] * cr[0], dt[1] * cr[1]), pk_bf16(dt[2] * cr[2], dt[3] * cr[3]));
            if constexpr (DUO)  // rows past the chunk's end are dropped
                bst64(__builtin_bit_cast(u32x2, du), make_rsrc(dug + cc.tok0 * (NW * 16), cc.nv * (NW * 16) * 2),
                      ((tt * 16 + c16) * (NW * 16) + w * 16 + 4 * g) * 2);
            else
                *reinterpret_cast<bf16x4 *>(du_l[b] + (tt * 16 + c16) * DUS + w * 16 + 4 * g) = du;
        }
        if constexpr (!DUO) {
            dxh_tiles(b ^ 1, ci - 1);  // (before the first chunk: unused values)
            if constexpr (DW) {
                if (ci >= 1) dw_tiles(b ^ 1);
            }
        }
    }
    if (!DUO && nch > 0) {
        const int pl = (nch - 1) & 1;  // buffers of the last chunk
        lds_barrier();
        if (nch >= 2) finish(nch - 2, pl ^ 1);
        dxh_tiles(pl, nch - 1);
        if constexpr (DW) dw_tiles(pl);
        lds_barrier();
        finish(nch - 1, pl);
    }
    if constexpr (DW) {
        __syncthreads();
        float *dst = dwp + blockIdx.x * (int64_t)(NW * 16 * HD);
        for (int e = threadIdx.x; e < NW * 16 * HD; e += NTHR) {
            const int hp = e / HD, col = e % HD;
            dst[e] = dwl[((hp >> 2) * HD + col) * 4 + (hp & 3)];
        }
    }
}

// dW[hp][c] = sum over the nparts partial blocks [rows][HD] for hp < LP; rows
// >= LP of the blocks (padding hyperplanes) are zero.  A workgroup takes 32
// consecutive entries; its 8 thread groups sum every 8th block (in order),
// then the 8 group sums are added in group order (a fixed order, whatever the
// launch).
static __global__ __launch_bounds__(256) void dw_reduce_kernel(const float *__restrict__ part, int64_t nparts,
                                                        int rows, int LP, int L, int P, int d,
                                                        float *__restrict__ dW)
{
    __shared__ float gs[8][32];
    const int grp = threadIdx.x >> 5, j = threadIdx.x & 31;
    const int e = blockIdx.x * 32 + j;
    float acc = 0.f;
    if (e < LP * HD) {
        const float *p = part + e;
        for (int64_t b = grp; b < nparts; b += 8) acc += p[b * (int64_t)rows * HD];
    }
    gs[grp][j] = acc;
    __syncthreads();
    if (grp == 0 && e < LP * HD) {
        float t = gs[0][j];
#pragma unroll
        for (int g2 = 1; g2 < 8; ++g2) t += gs[g2][j];
        // dW is [L][P][d]: padding hyperplanes and columns past d of the
        // blocks are dropped
        const int hp = e / HD, c = e % HD, r = w_row(L, P, hp);
        if (r >= 0 && c < d) dW[r * d + c] = t;
    }
}

}  // namespace race
