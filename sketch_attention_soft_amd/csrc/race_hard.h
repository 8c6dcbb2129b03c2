// race_hard.h -- hard-hash RACE attention for gfx950: integer bucket ids per
// (row, table), int32 bucket counts and fp32 value sums.
//
// Pages: "RACE Attention: A Strictly Linear-Time Attention for Long-Sequence
// Training", gist.science/zh/paper/2510.04008, technical summary §2.2 (the
// original RACE count arrays, which the soft hash makes differentiable) and
// §3; gist.science/es/paper/2510.04008, technical summary §2 item 3 (hard,
// YOSO-style hashing as the contrast).  With tau -> 0 the corner softmax of
// table l becomes one corner, r_l(x) = sum_p [u_lp >= 0] 2^p with u = W x
// (x / |x| has the same signs), and the bucket statistics are true counts
// A_l[r] and value sums B_l[r].
//
// Bucket ids.  A sign decided in floating point is exact unless the sum is
// within its rounding error of zero.  Here every product is exact: W is
// split into three bf16 terms that add up to the fp32 value exactly, and
// a row into one (bf16), two (fp16) or three (fp32) bf16 terms, so every
// product of terms is exact in the fp32 MFMA accumulators; only the fp32
// additions round, and the decision differs from the exact sign only when
// |sum_t W_t x_t| is within n 2^-24 sum_t |W_t x_t|, n the number of terms.
#pragma once
#include "race_walk.h"

namespace race {

// W [L][P][d] fp32 -> three bf16 terms [3][LPpad][Dpad] (zero padding), with
// W = t0 + t1 + t2 exactly: each term is the previous remainder rounded to
// bf16, and after two roundings at most 8 significant bits remain.
static __global__ __launch_bounds__(256) void hard_wsplit_kernel(const float *__restrict__ W, int LP,
                                                                 int d, int LPpad, int Dpad,
                                                                 bf16 *__restrict__ out)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= LPpad * Dpad) return;
    const int hp = e / Dpad, c = e % Dpad;
    const float w = hp < LP && c < d ? W[hp * d + c] : 0.f;
    const bf16 a = (bf16)w;
    const float r1 = w - (float)a;
    const bf16 b = (bf16)r1;
    const bf16 c2 = (bf16)(r1 - (float)b);
    const int n = LPpad * Dpad;
    out[e] = a;
    out[n + e] = b;
    out[2 * n + e] = c2;
}

// bf16 terms of eight row elements: XT terms, x = sum of the terms exactly
template <typename IO> struct XTerms;
template <> struct XTerms<bf16> {
    static constexpr int N = 1;
    static __device__ __forceinline__ void split(u32x4 raw, bf16x8 (&t)[1]) { t[0] = __builtin_bit_cast(bf16x8, raw); }
};
template <> struct XTerms<_Float16> {
    static constexpr int N = 2;
    static __device__ __forceinline__ void split(u32x4 raw, bf16x8 (&t)[2])
    {
        const halfx4 *h = reinterpret_cast<const halfx4 *>(&raw);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = (float)h[i >> 2][i & 3];
            const bf16 a = (bf16)x;
            t[0][i] = a;
            t[1][i] = (bf16)(x - (float)a);
        }
    }
};
template <> struct XTerms<float> {
    static constexpr int N = 3;
    static __device__ __forceinline__ void split(const float (&x)[8], bf16x8 (&t)[3])
    {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bf16 a = (bf16)x[i];
            const float r1 = x[i] - (float)a;
            const bf16 b = (bf16)r1;
            t[0][i] = a;
            t[1][i] = b;
            t[2][i] = (bf16)(r1 - (float)b);
        }
    }
};

// hard_ids_kernel: ids[row][l] = sum_p [u_lp >= 0] 2^p, u = W x, for `rows`
// rows of d elements (d a multiple of 8, at most 32 NKB).  Persistent: each
// workgroup loops over blocks of ids_rows() rows (256, fewer for wide rows),
// loading the next block into registers while the current one, staged in
// LDS, is multiplied; wave w keeps the W terms of the hyperplane words w,
// w + 4, ... (32 hyperplanes each) in registers and runs the block's row
// tiles of 16 through them: U^T tiles of 16 hyperplanes x 16 rows on MFMA (W terms x row
// terms, every product exact).  The signs are gathered into a bit mask per
// row in LDS, then one thread per row cuts the row's L ids out of its mask
// and stores them.
constexpr int HARD_MAXW = 24;  // 32-bit mask words per row: L P <= 768
template <typename IO, int NKB> constexpr int ids_rows()
{
    // at most 32 KB of staged rows per workgroup, whole row tiles of 16
    return 32768 / (NKB * 32 * (int)sizeof(IO)) >= 256 ? 256 : 32768 / (NKB * 32 * (int)sizeof(IO)) / 16 * 16;
}

// bf16 terms of one lane's 8 elements of a staged row
template <typename IO, int NKB>
__device__ __forceinline__ void ids_row_terms(const uint8_t *xs, int stride, int rr, int g,
                                              bf16x8 (&xt)[NKB][XTerms<IO>::N])
{
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const uint8_t *src = xs + rr * stride + (kb * 32 + 8 * g) * (int)sizeof(IO);
        if constexpr (sizeof(IO) == 2) {
            XTerms<IO>::split(*reinterpret_cast<const u32x4 *>(src), xt[kb]);
        } else {
            const floatx4 a = *reinterpret_cast<const floatx4 *>(src);
            const floatx4 b = *reinterpret_cast<const floatx4 *>(src + 16);
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = a[i];
                x[4 + i] = b[i];
            }
            XTerms<IO>::split(x, xt[kb]);
        }
    }
}

// vshift > 0 (P = 5, 6 in the hard forward): each table of 2^P buckets is
// written as 2^vshift virtual tables of 16 buckets: bucket r becomes bucket
// r & 15 of virtual table r >> 4 and id 16 (none) of the others, L 2^vshift
// ids per row.
template <typename IO, int NKB>
__global__ __launch_bounds__(256) void hard_ids_kernel(const IO *__restrict__ X, int64_t rows, int d,
                                                       const bf16 *__restrict__ wsp, int L, int P,
                                                       int LPpad, int Dpad, uint8_t *__restrict__ ids,
                                                       int vshift)
{
    constexpr int XT = XTerms<IO>::N, ROWS = ids_rows<IO, NKB>(), NRT = ROWS / 16;
    constexpr int RB = NKB * 32 * (int)sizeof(IO);  // bytes of a staged row
    constexpr int STRIDE = RB + 16;                 // (padding: conflict-free 16-byte reads)
    constexpr int PIECES = ROWS * RB / 16, PER = (PIECES + 255) / 256;
    __shared__ __attribute__((aligned(16))) uint8_t xs[ROWS * STRIDE];
    __shared__ uint32_t mask[ROWS][HARD_MAXW + 1];
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int nht = LPpad / 16, nwd = (nht + 1) / 2, nterm = LPpad * Dpad;
    const int64_t nblk = (rows + ROWS - 1) / ROWS;
    // a block's rows into registers, every load in flight at once (zeros
    // past d and past the rows); then into LDS
    u32x4 v[PER];
    auto load_block = [&](int64_t blk) {
        const int64_t r0 = blk * ROWS;
        const int nv = (int)min<int64_t>(ROWS, rows - r0);
        const Rsrc rx = make_rsrc(X + r0 * d, (int)(nv * d * sizeof(IO)));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * 256, rr = e / (RB / 16), pc = e % (RB / 16);
            const int col = pc * 16 / (int)sizeof(IO);
            v[i] = bld128(rx, e < PIECES && col < d ? (int)((rr * d + col) * sizeof(IO)) : OOB);
        }
    };
    // the W terms of a hyperplane word: two tiles of 16 hyperplanes
    bf16x8 wa[2][NKB][3];
    auto load_w = [&](int wd) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int ht = min(2 * wd + h2, nht - 1);  // (a missing second tile is not used)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    wa[h2][kb][t] = *reinterpret_cast<const bf16x8 *>(wsp + t * nterm + (ht * 16 + c16) * Dpad +
                                                                      kb * 32 + 8 * g);
        }
    };
    // with at most 4 words (L P <= 128) each wave keeps its word's W terms
    // for every block; otherwise it loads them per word and block
    const bool resident = nwd <= 4;
    if (resident && w < nwd) load_w(w);
    if ((int64_t)blockIdx.x < nblk) load_block(blockIdx.x);
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t r0 = blk * ROWS;
        const int nv = (int)min<int64_t>(ROWS, rows - r0);
        // the previous block's products and ids are done with xs and mask
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * 256, rr = e / (RB / 16), pc = e % (RB / 16);
            if (e < PIECES) *reinterpret_cast<u32x4 *>(xs + rr * STRIDE + pc * 16) = v[i];
        }
        if (blk + gridDim.x < nblk) load_block(blk + gridDim.x);
        // the words are OR-ed together below: clear them (their last reads,
        // the previous block's ids, came before the barrier above)
        for (int e = threadIdx.x; e < ROWS * nwd; e += 256) mask[e / nwd][e % nwd] = 0u;
        __syncthreads();
        // pairs of hyperplane tiles make one 32-bit word: lane group g holds
        // the nibbles at bits 4 g (tile 2 wd) and 16 + 4 g (tile 2 wd + 1)
        for (int wd = w; wd < nwd; wd += 4) {
            if (!resident) load_w(wd);
            const bool two = 2 * wd + 1 < nht;
#pragma unroll 4
            for (int rt = 0; rt < NRT; ++rt) {
                bf16x8 xt[NKB][XT];
                ids_row_terms<IO, NKB>(xs, STRIDE, rt * 16 + c16, g, xt);
                uint32_t word = 0;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    if (h2 == 1 && !two) break;
                    floatx4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int t = 0; t < 3; ++t)
#pragma unroll
                            for (int s = 0; s < XT; ++s) mma32(u, wa[h2][kb][t], xt[kb][s]);
                    // u[r]: hyperplane 16 (2 wd + h2) + 4 g + r of row c16;
                    // u = 0 counts as >= 0
                    uint32_t nib = 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) nib |= (u[r] >= 0.f ? 1u : 0u) << r;
                    word |= nib << (16 * h2 + 4 * g);
                }
                // the four lane groups' nibbles meet in LDS (an OR that
                // returns nothing, so the next tile does not wait on it)
                atomicOr(&mask[rt * 16 + c16][wd], word);
            }
        }
        __syncthreads();
        // one thread per row: bits l P .. l P + P - 1 of its mask (P <= 8, so
        // at most two words) are id l; ids are stored four to a dword when the
        // rows' byte offsets allow it (L a multiple of 4), else byte by byte
        const int rr = threadIdx.x;
        if (rr < ROWS) {
            const int Lv = L << vshift;  // ids per row written
            const Rsrc ro = make_rsrc(ids + r0 * Lv, nv * Lv);
            const uint32_t pm = (1u << P) - 1u;
            auto id = [&](int e) -> uint32_t {
                const int l = e >> vshift, b0 = l * P, wi = b0 >> 5;
                const uint32_t lo = mask[rr][wi], hi = wi + 1 < HARD_MAXW ? mask[rr][wi + 1] : 0u;
                const uint32_t r = __builtin_amdgcn_alignbit(hi, lo, b0 & 31) & pm;
                if (vshift == 0) return r;
                return (r >> 4) == (uint32_t)(e & ((1 << vshift) - 1)) ? (r & 15u) : 16u;
            };
            if ((Lv & 3) == 0) {
                for (int e = 0; e < Lv; e += 4) {
                    const uint32_t val = id(e) | id(e + 1) << 8 | id(e + 2) << 16 | id(e + 3) << 24;
                    __builtin_amdgcn_raw_buffer_store_b32(val, ro, rr < nv ? rr * Lv + e : OOB, 0, 0);
                }
            } else {
                for (int e = 0; e < Lv; ++e)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)id(e), ro, rr < nv ? rr * Lv + e : OOB, 0, 0);
            }
        }
    }
}

}  // namespace race

namespace race {

// ---------------------------------------------------------------------------
// Hard-hash sums and readout on the bucket ids (L <= 32, P <= 4, 16-bit rows).
// The work split is the soft kernels': a workgroup per (head, segment), NW
// waves of 4 tables each, chunks of 32 tokens.  A wave keeps the value sums
// of its 4 tables as 4 MFMA tiles of 16 buckets x 64 value columns (fp32);
// the one-hot operands built from the ids make every product 0 or a value,
// exact.  Counts are integers: the 4 tables x 16 buckets of a wave are one
// per lane, so each lane keeps its bucket's count in a register and adds the
// number of the chunk's keys in that bucket (the population count of the
// bucket's token mask); a query reads its buckets' counts from the wave's
// copy in LDS and adds the keys of its own chunk that come before it.
constexpr int HNT = 4;  // value column tiles (64 columns)

// bf16 one-hot quadruples: entry n holds 1.0 in slot i when bit i of n is set
__device__ __forceinline__ void stage_lut(uint32_t *lut)
{
    if (threadIdx.x < 16) {
        const uint32_t n = threadIdx.x;
        lut[2 * n] = (n & 1 ? 0x3F80u : 0u) | (n & 2 ? 0x3F800000u : 0u);
        lut[2 * n + 1] = (n & 4 ? 0x3F80u : 0u) | (n & 8 ? 0x3F800000u : 0u);
    }
}
__device__ __forceinline__ bf16x4 lut4(const uint32_t *lut, uint32_t nib)
{
    return __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(lut + 2 * nib));
}
// token-major one-hot operand (lane group g: buckets 4g .. 4g + 3 of tables
// t0 then t1, the K-slot order of the state operands); id 16 (none) gives zeros
// (ids of valid rows are 0 .. 16: the bit of id 16 lies past every group's
// nibble, bits 4 g .. 4 g + 3 with g <= 3, so it needs no test; bytes past a
// chunk's valid rows only reach tokens whose scores are masked out or whose
// value rows and outputs are zero or dropped)
__device__ __forceinline__ uint32_t onehot_nib(uint32_t id, int g)
{
    return __builtin_amdgcn_ubfe(1u << (id & 31u), 4 * g, 4);
}
__device__ __forceinline__ bf16x8 onehot_tm(const uint32_t *lut, uint32_t id0, uint32_t id1, int g)
{
    return cat8(lut4(lut, onehot_nib(id0, g)), lut4(lut, onehot_nib(id1, g)));
}
// feature-major one-hot operand of one table from its bucket's token mask
// (bit j: token j of the chunk falls in the bucket); K-slots (g, r) <-> token
// 4g + r, (g, 4 + r) <-> token 16 + 4g + r, as ycol_frag
__device__ __forceinline__ bf16x8 onehot_fm(const uint32_t *lut, uint32_t m, int g)
{
    return cat8(lut4(lut, __builtin_amdgcn_ubfe(m, 4 * g, 4)), lut4(lut, __builtin_amdgcn_ubfe(m, 16 + 4 * g, 4)));
}

// ids of one chunk's rows: rsrc over its nv rows of L bytes, rounded up to
// whole dwords (a dword past the range reads as zero; the id arrays carry
// padding, and bytes past the valid rows are never counted)
__device__ __forceinline__ Rsrc id_res(const uint8_t *seg_ids, int L, const Chunk &c)
{
    return make_rsrc(seg_ids + (int64_t)c.tok0 * L, (c.nv * L + 3) & ~3);
}
// the chunk's 32 L id bytes as dwords: thread e < 8 L loads dword e (zeros
// past the valid rows), and later stores it to LDS.  Every launch has at
// least 8 L threads (2 waves per 8 tables).
__device__ __forceinline__ uint32_t load_ids(Rsrc r, int L)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)threadIdx.x < 8 * L ? 4 * (int)threadIdx.x : OOB, 0, 0);
}
__device__ __forceinline__ void store_ids(uint32_t v, int L, uint32_t *dst)
{
    if ((int)threadIdx.x < 8 * L) dst[threadIdx.x] = v;
}
// ids of tables 4 w .. 4 w + 3 of one token (bytes 0..3; the bytes of tables
// past L are not ids and must not be used): one funnel shift over the two
// dwords that hold them (the id arrays in LDS carry one dword of padding)
__device__ __forceinline__ uint32_t ids4_at(const uint32_t *ids, int L, int tok, int w)
{
    const int b = tok * L + 4 * w;
    return __builtin_amdgcn_alignbit(ids[(b >> 2) + 1], ids[b >> 2], 8 * (b & 3));
}
__device__ __forceinline__ uint32_t byte_of(uint32_t v, int i) { return (v >> (8 * i)) & 0xffu; }

// The bucket token masks of this wave's tables for one chunk: bm[16 s + r]
// bit j is set when key j of the chunk falls in bucket r of table 4 w + s.
// Only the wave itself reads them, so no workgroup barrier is needed: its
// LDS operations complete in program order.
__device__ __forceinline__ void wave_masks(uint32_t *bm, const uint32_t *kid, int L, int nv, int w)
{
    const int lane = lane_id();
    bm[lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    // lanes take tokens, the two halves of the wave two tables each
    const int j = lane & 31;
    const uint32_t k4 = ids4_at(kid, L, j, w);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int s = (lane >> 5) + 2 * it, T = 4 * w + s;
        const uint32_t id = byte_of(k4, s);  // (16: no bucket in this virtual table)
        if (T < L && j < nv && id < 16u) atomicOr(&bm[s * 16 + id], 1u << j);
    }
    __builtin_amdgcn_wave_barrier();
}

// hard_sum_kernel: per (head, segment) the value sums B[l][r][:] (FxC
// tiles, stored as the soft kernels' state blocks) and the int32 counts
// A[l][r] of the segment's keys.
template <int NW, typename IO, int D>
__global__ __launch_bounds__(NW * 64) void hard_sum_kernel(
    const IO *__restrict__ V, const uint8_t *__restrict__ idk, int L, int64_t N, int seg,
    int64_t nseg, float *__restrict__ st, int *__restrict__ cst, Lens ls)
{
    constexpr int NTHR = NW * 64;
    __shared__ __attribute__((aligned(16))) bf16 ycol[2][NCOL * YCS];
    __shared__ uint32_t ids[2][8 * 32 + 1];
    __shared__ uint32_t bmw[NW][64];
    __shared__ uint32_t lut[32];
    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int64_t t_begin = sg * seg, row0 = row_base(ls, bh, N) + t_begin;
    const int tend = (int)max<int64_t>(0, min<int64_t>(valid_rows(ls, bh, N), t_begin + seg) - t_begin);
    const int nch = (tend + WCT - 1) / WCT;
    ValSrc<IO> vh{V + row0 * D, nullptr, nullptr};
    const uint8_t *ids_seg = idk + row0 * L;
    uint32_t *bm = bmw[w];
    stage_lut(lut);
    floatx4 acc[4][HNT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < HNT; ++ct) acc[s][ct] = {0.f, 0.f, 0.f, 0.f};
    uint32_t cnt = 0;  // keys in bucket (lane & 15) of table 4 w + lane / 16
    auto chunk = [&](int ci) -> Chunk {
        if (ci >= nch) return Chunk{0, 0};
        return Chunk{ci * WCT, min(WCT, tend - ci * WCT)};
    };
    // chunk ci + 1 is loaded into registers while chunk ci is summed
    YStage<NTHR, false> ys;
    uint32_t kid = 0;
    if (nch > 0) {
        kid = load_ids(id_res(ids_seg, L, chunk(0)), L);
        ystage_load<NTHR, false, D>(yres<false, D>(vh, chunk(0)), ys);
    }
    for (int ci = 0; ci < nch; ++ci) {
        const int b = ci & 1;
        const Chunk cc = chunk(ci), cn = chunk(ci + 1);
        // stage ids and [v | 1] of chunk ci (buffers last read before the
        // previous barrier), then start loading chunk ci + 1
        store_ids(kid, L, ids[b]);
        ystage_store<NTHR, false, IO>(ys, cc.nv, ycol[b]);
        if (ci + 1 < nch) {
            kid = load_ids(id_res(ids_seg, L, cn), L);
            ystage_load<NTHR, false, D>(yres<false, D>(vh, cn), ys);
        }
        __syncthreads();
        wave_masks(bm, ids[b], L, cc.nv, w);
        cnt += __builtin_popcount(bm[lane]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int T = 4 * w + s;
            const bf16x8 a = onehot_fm(lut, T < L ? bm[s * 16 + c16] : 0u, g);
#pragma unroll
            for (int ct = 0; ct < HNT; ++ct) mma32(acc[s][ct], a, ycol_frag(ycol[b], ct * 16 + c16));
        }
    }
    const int64_t blk = bh * (nseg + 1) + sg;
    float *vdst = st + blk * (int64_t)(NW * 4 * HNT * 64 * 4);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ct = 0; ct < HNT; ++ct)
            *reinterpret_cast<floatx4 *>(vdst + (((w * 4 + s) * HNT + ct) * 64 + lane) * 4) = acc[s][ct];
    // count block [32 tables][16 buckets]: this wave's 64, zeros past the
    // waves' tables
    int *cdst = cst + blk * (int64_t)(32 * 16);
    cdst[w * 64 + lane] = (int)cnt;
    for (int e = NW * 64 + (int)threadIdx.x; e < 32 * 16; e += NTHR) cdst[e] = 0;
}

// Scan of the int32 count blocks over segments (exclusive prefix, head
// total at index nseg), one thread per count, in segment order.
static __global__ __launch_bounds__(256) void hard_count_scan_kernel(int *__restrict__ cst, int64_t nseg,
                                                                     int elems)
{
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= elems) return;
    int *p = cst + blockIdx.y * (nseg + 1) * (int64_t)elems + e;
    int run = 0;
    constexpr int U = 8;  // loads in flight per thread
    int64_t g = 0;
    for (; g + U <= nseg; g += U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[(g + u) * elems];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            p[(g + u) * elems] = run;
            run += v[u];
        }
    }
    for (; g < nseg; ++g) {
        const int v = p[g * elems];
        p[g * elems] = run;
        run += v;
    }
    p[nseg * elems] = run;
}

// hard_walk_kernel: o_i = sum_l B_l[r_l(q_i)] / sum_l A_l[r_l(q_i)] over the
// keys j <= i (causal) or all keys, from the segment's prefix state (values:
// fp32 tiles read as bf16 MFMA operands; counts: integers, exact), the
// chunks before i in the segment, and the chunk's own keys j <= i.  den =
// the count (as fp32) and, when count is not null, the count itself (int32).
// Two barriers per chunk: after staging, and after the partial outputs.
template <int NW, bool CAUSAL, typename IO, int D>
__global__ __launch_bounds__(NW * 64) void hard_walk_kernel(
    const IO *__restrict__ V, const uint8_t *__restrict__ idq, const uint8_t *__restrict__ idk,
    int L, int64_t N, int seg, int64_t nseg, const float *__restrict__ st,
    const int *__restrict__ cst, IO *__restrict__ Out, float *__restrict__ den,
    int *__restrict__ count, Lens ls)
{
    constexpr int NTHR = NW * 64;
    constexpr int REDN = NW * 2 * HNT * 64 * 4;  // partial outputs of every wave
    // 8-wave workgroups (one per compute unit) double-buffer the partial
    // outputs and counts, so that a chunk needs one barrier: chunk c's are
    // summed after the barrier of chunk c + 1.  Narrower ones run two per
    // compute unit, which LDS allows only with one buffer and a second
    // barrier per chunk.
    constexpr int NRED = NW >= 8 ? 2 : 1;
    __shared__ __attribute__((aligned(16))) bf16 ycol[2][CAUSAL ? NCOL * YCS : 8];
    __shared__ uint32_t qids[2][8 * 32 + 1];
    __shared__ uint32_t kids[2][CAUSAL ? 8 * 32 + 1 : 1];
    __shared__ uint32_t bmw[CAUSAL ? NW : 1][64];  // this chunk's bucket token masks, per wave
    __shared__ uint32_t cntw[NW][64];              // counts of the keys before the chunk, per wave
    __shared__ uint32_t lut[32];
    __shared__ __attribute__((aligned(16))) float red[NRED][REDN];
    __shared__ uint32_t redm[NRED][NW][32];        // each wave's count of every query
    const int64_t bh = blockIdx.x / nseg, sg = blockIdx.x % nseg;
    const int lane = lane_id(), w = wave_id(), g = lane >> 4, c16 = lane & 15;
    const int64_t t_begin = sg * seg, row0 = row_base(ls, bh, N) + t_begin;
    const int tend = (int)max<int64_t>(0, min<int64_t>(valid_rows(ls, bh, N), t_begin + seg) - t_begin);
    const int nch = (tend + WCT - 1) / WCT;
    ValSrc<IO> vh{V + row0 * D, nullptr, nullptr};
    const uint8_t *q_seg = idq + row0 * L, *k_seg = idk + row0 * L;
    IO *Os = Out + row0 * D;
    float *dens = den + row0;
    int *cnts = count ? count + row0 : nullptr;
    uint32_t *bm = bmw[CAUSAL ? w : 0], *cw = cntw[w];
    stage_lut(lut);
    const int64_t sidx = bh * (nseg + 1) + (CAUSAL ? sg : nseg);
    // counts before the segment (all keys: non-causal), one bucket per lane
    uint32_t cnt = (uint32_t)cst[sidx * (int64_t)(32 * 16) + w * 64 + lane];
    cw[lane] = cnt;
    if (CAUSAL) {
        ystage_zero_pad<NTHR>(ycol[0]);
        ystage_zero_pad<NTHR>(ycol[1]);
    }
    floatx4 acc[4][HNT];
    {
        const float *src = st + sidx * (int64_t)(NW * 4 * HNT * 64 * 4);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int ct = 0; ct < HNT; ++ct)
                acc[s][ct] = *reinterpret_cast<const floatx4 *>(src + (((w * 4 + s) * HNT + ct) * 64 + lane) * 4);
    }
    auto chunk = [&](int ci) -> Chunk {
        if (ci >= nch) return Chunk{0, 0};
        return Chunk{ci * WCT, min(WCT, tend - ci * WCT)};
    };
    // chunk ci + 1 is loaded into registers while chunk ci is read out
    YStage<NTHR, false> ys;
    uint32_t qid = 0, kid = 0;
    if (nch > 0) {
        qid = load_ids(id_res(q_seg, L, chunk(0)), L);
        if (CAUSAL) {
            kid = load_ids(id_res(k_seg, L, chunk(0)), L);
            ystage_load<NTHR, false, D>(yres<false, D>(vh, chunk(0)), ys);
        }
    }
    // outputs of chunk ci from the partial sums in buffer pb: thread slot
    // (token tile tt, column tile ct, lane)
    auto finish = [&](int ci, int pb) {
        const Chunk cc = chunk(ci);
        const Rsrc ro = row_res<D>(Os, cc);
        const float *rd = red[NRED == 2 ? pb : 0];
        const uint32_t(*rm)[32] = redm[NRED == 2 ? pb : 0];
        for (int sl = threadIdx.x; sl < 2 * HNT * 64; sl += NTHR) {
            const int tt = sl >> 8, ct = (sl >> 6) & 3, ln = sl & 63, tok = tt * 16 + (ln & 15);
            floatx4 n = *reinterpret_cast<const floatx4 *>(rd + ((tt * HNT + ct) * 64 + ln) * 4);
            uint32_t m = rm[0][tok];
            for (int ww = 1; ww < NW; ++ww) {
                n += *reinterpret_cast<const floatx4 *>(rd + (((ww * 2 + tt) * HNT + ct) * 64 + ln) * 4);
                m += rm[ww][tok];
            }
            // a query that meets no visible key in any table: an empty sum,
            // o = 0 (n is 0 too)
            const float inv = m > 0 ? __builtin_amdgcn_rcpf((float)m) : 0.f;
            const int col = 16 * ct + 4 * (ln >> 4);
            const int off = (D == HD || col < D) ? tok * (D * 2) + col * 2 : OOB;
            bst64(u32x2{pk_io<IO>(n[0] * inv, n[1] * inv), pk_io<IO>(n[2] * inv, n[3] * inv)}, ro, off);
            if (ct == 0 && ln < 16) {
                bstf((float)m, make_rsrc(dens + cc.tok0, cc.nv * 4), tok * 4);
                if (cnts)
                    __builtin_amdgcn_raw_buffer_store_b32(m, make_rsrc(cnts + cc.tok0, cc.nv * 4), tok * 4,
                                                          0, 0);
            }
        }
    };
    for_chunks2(nch, [&](int ci, auto par) {
        constexpr int b = decltype(par)::v;
        const Chunk cc = chunk(ci), cn = chunk(ci + 1);
        // stage ids (and keys' [v | 1]) of chunk ci into buffers last read
        // before the previous barrier, then start loading chunk ci + 1
        store_ids(qid, L, qids[b]);
        if (CAUSAL) {
            store_ids(kid, L, kids[b]);
            ystage_store<NTHR, false, IO>(ys, cc.nv, ycol[b]);
        }
        if (ci + 1 < nch) {
            qid = load_ids(id_res(q_seg, L, cn), L);
            if (CAUSAL) {
                kid = load_ids(id_res(k_seg, L, cn), L);
                ystage_load<NTHR, false, D>(yres<false, D>(vh, cn), ys);
            }
        }
        __syncthreads();
        // (the previous chunk's partial sums, in the other buffer)
        if (NRED == 2 && ci > 0) finish(ci - 1, b ^ 1);
        if (CAUSAL) wave_masks(bm, kids[b], L, cc.nv, w);
        {
            // this wave's count of each query: its buckets' counts before the
            // chunk, and (causal) the chunk's keys j <= i in them; lanes take
            // tokens, the two halves of the wave two tables each
            const int tok = lane & 31;
            const uint32_t q4 = ids4_at(qids[b], L, tok, w);
            uint32_t m = 0;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int s = 2 * (lane >> 5) + h, T = 4 * w + s;
                const uint32_t id = byte_of(q4, s);
                if (T < L && id < 16u) {
                    m += cw[s * 16 + id];
                    if (CAUSAL) m += __builtin_popcount(bm[s * 16 + id] & ((2u << tok) - 1u));
                }
            }
            m += __shfl_xor(m, 32);
            if (lane < 32) redm[NRED == 2 ? b : 0][w][tok] = m;
        }
        if (CAUSAL) {
            // the chunk's keys join the counts (after the reads above: this
            // wave's LDS operations complete in order)
            cnt += __builtin_popcount(bm[lane]);
            __builtin_amdgcn_wave_barrier();
            cw[lane] = cnt;
        }
        // one-hot operands of this wave's tables 4w .. 4w + 3 (16: none)
        bf16x8 pr[2][2], pw[2][2], pfm[4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int tok = 16 * tt + c16;
            const uint32_t q4 = ids4_at(qids[b], L, tok, w);
            const uint32_t k4 = CAUSAL ? ids4_at(kids[b], L, tok, w) : 0u;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int t0 = 4 * w + 2 * k;
                const uint32_t q0 = t0 < L ? byte_of(q4, 2 * k) : 16u;
                const uint32_t q1 = t0 + 1 < L ? byte_of(q4, 2 * k + 1) : 16u;
                pr[tt][k] = onehot_tm(lut, q0, q1, g);
                if (CAUSAL) {
                    const uint32_t k0 = t0 < L ? byte_of(k4, 2 * k) : 16u;
                    const uint32_t k1 = t0 + 1 < L ? byte_of(k4, 2 * k + 1) : 16u;
                    pw[tt][k] = onehot_tm(lut, k0, k1, g);
                }
            }
        }
        if (CAUSAL)
#pragma unroll
            for (int s = 0; s < 4; ++s) pfm[s] = onehot_fm(lut, 4 * w + s < L ? bm[s * 16 + c16] : 0u, g);
        floatx4 oacc[2][HNT];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ct = 0; ct < HNT; ++ct) oacc[tt][ct] = {0.f, 0.f, 0.f, 0.f};
        // the state of the keys before the chunk (value columns)
#pragma unroll
        for (int ct = 0; ct < HNT; ++ct) {
            bf16x8 sf[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) sf[k] = cat8(acc2bf4(acc[2 * k][ct]), acc2bf4(acc[2 * k + 1][ct]));
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) mma32(oacc[tt][ct], sf[k], pr[tt][k]);
        }
        if (CAUSAL) {
            // collision counts D[j][i] of writer j and reader i over the wave's
            // tables (exact small integers), keys j <= i only
            constexpr int TJ[3] = {0, 0, 1}, TI[3] = {0, 1, 1};
            floatx4 sc[3];
#pragma unroll
            for (int pi = 0; pi < 3; ++pi) {
                sc[pi] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 2; ++k) mma32(sc[pi], pw[TJ[pi]][k], pr[TI[pi]][k]);
            }
#pragma unroll
            for (int pi = 0; pi < 3; pi += 2)
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[pi][r] = 4 * g + r <= c16 ? sc[pi][r] : 0.f;
            const bf16x4 z4 = pk4(0, 0);
            const bf16x8 kA1 = cat8(acc2bf4(sc[0]), z4);              // reader tile 0: writer tile 0
            const bf16x8 kA8 = cat8(acc2bf4(sc[1]), acc2bf4(sc[2]));  // reader tile 1: writer tiles 0, 1
#pragma unroll
            for (int ct = 0; ct < HNT; ++ct) {
                const bf16x8 yb = ycol_frag(ycol[b], ct * 16 + c16);
                mma32(oacc[0][ct], yb, kA1);
                mma32(oacc[1][ct], yb, kA8);
#pragma unroll
                for (int s = 0; s < 4; ++s) mma32(acc[s][ct], pfm[s], yb);
            }
        }
        // partial outputs of this wave
        float *rd = red[NRED == 2 ? b : 0];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ct = 0; ct < HNT; ++ct)
                *reinterpret_cast<floatx4 *>(rd + (((w * 2 + tt) * HNT + ct) * 64 + lane) * 4) = oacc[tt][ct];
        if constexpr (NRED == 1) {
            __syncthreads();
            finish(ci, 0);
        }
    });
    if (NRED == 2 && nch > 0) {
        __syncthreads();
        finish(nch - 1, (nch - 1) & 1);
    }
}

}  // namespace race
