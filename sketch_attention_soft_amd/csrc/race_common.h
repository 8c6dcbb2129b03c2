// race_common.h -- shared device helpers for the RACE attention kernels (gfx950).
//
// Feature map.  The corner softmax of one table factorises over its P
// hyperplanes, and for P = 4 the inner product of two soft assignments is
//   sum_r phi_r(q) phi_r(k) = prod_p (1 + t_p(q) t_p(k)) / 2,  t = tanh(z / tau),
// which expands into the 16 Walsh monomials of t:
//   = sum_S psi_S(q) psi_S(k),   psi_S = (1/4) prod_{p in S} t_p,   S subset of {0..3}.
// The corner basis and this basis differ by an orthogonal (Hadamard) change
// of basis per table, so every sketch, readout and gradient of the method is
// the same; the monomials need 16 multiplies per table instead of a softmax.
// Feature f = 16 * l + S, where bit p of S selects t_p.
//
// MFMA fragments.  A K-block of 32 (F8) or 16 (F4) along a contraction
// dimension: lane l holds k = 8*(l/16) + i (F8) or 4*(l/16) + i (F4) of row
// (A operand) or column (B operand) l % 16.  Both operands of one product use
// the same k-slots, so the fp32 path issues one 16x16x4 MFMA per slot i and
// the bf16 path one 16x16x32 (or 16x16x16) MFMA per block.  Accumulators use
// the 16x16 output layout: lane l holds rows 4*(l/16) + r, column l % 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace race {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int HD = 64;          // head dimension d
constexpr int NP = 4;           // hyperplanes per table P
constexpr int NR = 16;          // corners (features) per table R = 2^P
constexpr int NCOL = 80;        // d value columns + count column, padded to 5 tiles
constexpr int NT = NCOL / 16;   // column tiles
constexpr int CH = 16;          // tokens per sub-chunk
constexpr int TPW = 8;          // tables per wave
constexpr int FPW = TPW * NR;   // features per wave (128)
constexpr int MT = FPW / 16;    // feature tiles per wave (8)

template <typename T> struct F8;
template <> struct F8<bf16> { bf16x8 v; };
template <> struct F8<float> { floatx8 v; };
template <typename T> struct F4;
template <> struct F4<bf16> { bf16x4 v; };
template <> struct F4<float> { floatx4 v; };

__device__ __forceinline__ void mma(floatx4 &acc, const F8<bf16> &a, const F8<bf16> &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4 &acc, const F8<float> &a, const F8<float> &b)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4 &acc, const F4<bf16> &a, const F4<bf16> &b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a.v),
                                                    __builtin_bit_cast(shortx4, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4 &acc, const F4<float> &a, const F4<float> &b)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// 4 / 8 consecutive elements from LDS or global memory
template <typename T> __device__ __forceinline__ F4<T> ld4(const T *p);
template <> __device__ __forceinline__ F4<bf16> ld4<bf16>(const bf16 *p)
{
    F4<bf16> f;
    f.v = *reinterpret_cast<const bf16x4 *>(p);
    return f;
}
template <> __device__ __forceinline__ F4<float> ld4<float>(const float *p)
{
    F4<float> f;
    f.v = *reinterpret_cast<const floatx4 *>(p);
    return f;
}
template <typename T> __device__ __forceinline__ F8<T> ld8(const T *p);
template <> __device__ __forceinline__ F8<bf16> ld8<bf16>(const bf16 *p)
{
    F8<bf16> f;
    f.v = *reinterpret_cast<const bf16x8 *>(p);
    return f;
}
template <> __device__ __forceinline__ F8<float> ld8<float>(const float *p)
{
    F8<float> f;
    f.v = *reinterpret_cast<const floatx8 *>(p);
    return f;
}
// two groups of 4 consecutive elements -> one F8 (slots 0-3 from p, 4-7 from q)
template <typename T> __device__ __forceinline__ F8<T> ld4x2(const T *p, const T *q)
{
    F4<T> a = ld4<T>(p), b = ld4<T>(q);
    F8<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = a.v[i];
        f.v[4 + i] = b.v[i];
    }
    return f;
}
// 8 elements at a stride
template <typename T> __device__ __forceinline__ F8<T> ld8s(const T *p, int stride)
{
    F8<T> f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f.v[i] = p[i * stride];
    return f;
}
// accumulator tiles -> operand fragment (slots 0-3 from a, 4-7 from b)
template <typename T> __device__ __forceinline__ F8<T> acc2frag(const floatx4 &a, const floatx4 &b)
{
    F8<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = from_f32<T>(a[i]);
        f.v[4 + i] = from_f32<T>(b[i]);
    }
    return f;
}
template <typename T> __device__ __forceinline__ F4<T> acc2frag4(const floatx4 &a)
{
    F4<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = from_f32<T>(a[i]);
    return f;
}

// Workgroup barrier that orders LDS only: global loads in flight (prefetches
// of the next chunk) are not waited for, unlike __syncthreads().
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until every global load and store this wave has issued is complete.
// Placed before a chunk loop: memory operations complete in order, and where
// the prologue issues its loads in another order than the loop body, the
// compiler's wait at the loop head has to cover both paths and becomes a wait
// for everything outstanding -- in every iteration, the prefetch of the next
// chunk's rows included.  With nothing outstanding on entry, the waits inside
// the loop follow the loop's own issue order.
__device__ __forceinline__ void vm_drain()
{
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt, lgkmcnt unchanged
}

// Rows of head bh = b H + h that exist: N, or for right-padded batches the
// length of its batch, len[b] clamped to [0, N] (rows past it are neither
// read nor written: the sums skip them and their outputs are left as they
// are).  Packed batches (cu != null): the sequences of head h lie back to
// back in rows [h T, (h + 1) T), sequence b at rows cu[b] .. cu[b + 1] of
// them; its length is clamped to [0, N] and to the T rows.
struct Lens {
    const int *len;
    int H;
    const int *cu = nullptr;  // cu_seqlens [B + 1] (packed batches) or null
    int64_t T = 0;            // rows per head of a packed batch
};
__device__ __forceinline__ void packed_range(const Lens &ls, int64_t bh, int64_t N, int64_t &start,
                                             int64_t &len)
{
    const int64_t b = bh / ls.H;
    int64_t s0 = ls.cu[b], s1 = ls.cu[b + 1];
    s0 = s0 < 0 ? 0 : s0 < ls.T ? s0 : ls.T;
    s1 = s1 < s0 ? s0 : s1 < ls.T ? s1 : ls.T;
    start = s0;
    len = s1 - s0 < N ? s1 - s0 : N;
}
__device__ __forceinline__ int64_t valid_rows(const Lens &ls, int64_t bh, int64_t N)
{
    if (ls.cu) {
        int64_t s, n;
        packed_range(ls, bh, N, s, n);
        return n;
    }
    if (!ls.len) return N;
    const int64_t n = ls.len[bh / ls.H];
    return n < 0 ? 0 : n < N ? n : N;
}
// First row of head bh in the [rows][d] tensors: bh N, or h T + cu[b] for
// packed batches.
__device__ __forceinline__ int64_t row_base(const Lens &ls, int64_t bh, int64_t N)
{
    if (ls.cu) {
        int64_t s, n;
        packed_range(ls, bh, N, s, n);
        return (bh % ls.H) * ls.T + s;
    }
    return bh * N;
}

// Tables in passes of at most 32 (L > 32: tables 0..31, 32..63, ...).  The
// outputs are sums over tables before the last, nonlinear step, so the first
// pass stores its sums in fp32 (PART_OUT), the middle ones add theirs to the
// stored sums (PART_MID) and the last adds the stored sums to its own
// (PART_IN): the readout's n and m before o = n / m, dV, and dx_hat before
// the normalisation backward.  Partial rows are [token][64] fp32 (and m
// [token]).
constexpr int PART_NONE = 0, PART_OUT = 1, PART_IN = 2, PART_MID = 3;
struct Part {
    float *v;  // [rows][64]
    float *m;  // [rows] (readout denominators) or null
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// The 16 Walsh features of one table from its t_0..t_3: psi[S] = (1/4) prod_{p in S} t_p.
__device__ __forceinline__ void walsh16(const floatx4 &t, float psi[16])
{
    const float a0 = 0.25f, a1 = 0.25f * t[0], a2 = 0.25f * t[1], a3 = a1 * t[1];
    const float b1 = t[2], b2 = t[3], b3 = t[2] * t[3];
    psi[0] = a0; psi[1] = a1; psi[2] = a2; psi[3] = a3;
    psi[4] = a0 * b1; psi[5] = a1 * b1; psi[6] = a2 * b1; psi[7] = a3 * b1;
    psi[8] = a0 * b2; psi[9] = a1 * b2; psi[10] = a2 * b2; psi[11] = a3 * b2;
    psi[12] = a0 * b3; psi[13] = a1 * b3; psi[14] = a2 * b3; psi[15] = a3 * b3;
}

// Features 4*fg .. 4*fg+3 of one table (bits 2,3 of S fixed to fg).
__device__ __forceinline__ void walsh4(const floatx4 &t, int fg, float psi[4])
{
    const float b = fg == 0 ? 0.25f : fg == 1 ? 0.25f * t[2] : fg == 2 ? 0.25f * t[3] : 0.25f * t[2] * t[3];
    psi[0] = b;
    psi[1] = b * t[0];
    psi[2] = b * t[1];
    psi[3] = psi[1] * t[1];
}

}  // namespace race
