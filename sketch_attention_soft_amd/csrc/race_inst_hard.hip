// race_inst_hard.hip -- launch sequences of the hard-hash kernels
// (race_hard.h), compiled apart from the other race_inst_*.hip files so that
// the library builds in parallel.
#include <algorithm>

#include "race_host.h"

namespace race_host {

template <typename IO, int NKB>
static void hard_ids_nkb(const IO *X, int64_t rows, int d, const bf16 *wsp, int L, int P, int LPpad,
                         int Dpad, uint8_t *ids, hipStream_t s, int vshift)
{
    // persistent workgroups: two per compute unit (256 CUs), or one per block
    constexpr int R = race::ids_rows<IO, NKB>();
    const int64_t blocks = (rows + R - 1) / R;
    const dim3 grid((unsigned)std::min<int64_t>(blocks, 512));
    hipLaunchKernelGGL((race::hard_ids_kernel<IO, NKB>), grid, dim3(256), 0, s, X, rows, d, wsp, L, P, LPpad,
                       Dpad, ids, vshift);
}
template <typename IO>
static void hard_ids_t(const IO *X, int64_t rows, int d, const bf16 *wsp, int L, int P, int LPpad,
                       int Dpad, uint8_t *ids, hipStream_t s, int vshift)
{
    switch (Dpad / 32) {
    case 1: hard_ids_nkb<IO, 1>(X, rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift); break;
    case 2: hard_ids_nkb<IO, 2>(X, rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift); break;
    case 3: hard_ids_nkb<IO, 3>(X, rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift); break;
    default: hard_ids_nkb<IO, 4>(X, rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift); break;
    }
}

void hard_ids_launch(const void *X, int64_t rows, int d, race_dtype_t dt, const float *W, int L,
                     int P, uint8_t *ids, char *ws, hipStream_t s, int vshift)
{
    const int LPpad = hard_lppad(L, P), Dpad = hard_dpad(d);
    bf16 *wsp = reinterpret_cast<bf16 *>(ws);
    hipLaunchKernelGGL(race::hard_wsplit_kernel, dim3((LPpad * Dpad + 255) / 256), dim3(256), 0, s, W,
                       L * P, d, LPpad, Dpad, wsp);
    if (rows == 0) return;
    if (dt == RACE_BF16)
        hard_ids_t(static_cast<const bf16 *>(X), rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift);
    else if (dt == RACE_F16)
        hard_ids_t(static_cast<const _Float16 *>(X), rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift);
    else
        hard_ids_t(static_cast<const float *>(X), rows, d, wsp, L, P, LPpad, Dpad, ids, s, vshift);
}

template <typename T, int NW, int D>
static void hard_forward_t(const Plan &p, const HardPlan &h, const T *Q, const T *K, const T *V,
                           int causal, T *O, float *den, int *count, char *ws, hipStream_t s)
{
    const uint8_t *idq = reinterpret_cast<const uint8_t *>(ws + h.o_idq);
    const uint8_t *idk = reinterpret_cast<const uint8_t *>(ws + h.o_idk);
    float *vst = reinterpret_cast<float *>(ws + h.o_v);
    int *cst = reinterpret_cast<int *>(ws + h.o_c);
    float *tmp = reinterpret_cast<float *>(ws + h.o_scan);
    const dim3 nblk((unsigned)(p.BH * p.nseg));
    hipLaunchKernelGGL((race::hard_sum_kernel<NW, T, D>), nblk, dim3(NW * 64), 0, s, V, idk, p.L, p.N,
                       (int)p.seg, p.nseg, vst, cst, p.lens);
    const dim3 sg((unsigned)((h.velems + 255) / 256), (unsigned)p.scan_groups, (unsigned)p.BH);
    hipLaunchKernelGGL(race::scan_reduce_kernel, sg, dim3(256), 0, s, vst, tmp, p.nseg, h.velems,
                       p.scan_groups);
    hipLaunchKernelGGL(race::scan_apply_kernel, sg, dim3(256), 0, s, vst, tmp, p.nseg, h.velems,
                       p.scan_groups, 0);
    hipLaunchKernelGGL(race::hard_count_scan_kernel, dim3(2, (unsigned)p.BH), dim3(256), 0, s, cst,
                       p.nseg, 32 * 16);
    if (causal)
        hipLaunchKernelGGL((race::hard_walk_kernel<NW, true, T, D>), nblk, dim3(NW * 64), 0, s, V, idq,
                           idk, p.L, p.N, (int)p.seg, p.nseg, vst, cst, O, den, count, p.lens);
    else
        hipLaunchKernelGGL((race::hard_walk_kernel<NW, false, T, D>), nblk, dim3(NW * 64), 0, s, V, idq,
                           idk, p.L, p.N, (int)p.seg, p.nseg, vst, cst, O, den, count, p.lens);
}

template <typename T, int D>
static void hard_forward_d(const Plan &p, const HardPlan &h, const void *Q, const void *K,
                           const void *V, int causal, void *O, float *den, int *count, char *ws,
                           hipStream_t s)
{
    auto q = static_cast<const T *>(Q), k = static_cast<const T *>(K), v = static_cast<const T *>(V);
    auto o = static_cast<T *>(O);
    switch (h.hw) {
    case 2: hard_forward_t<T, 2, D>(p, h, q, k, v, causal, o, den, count, ws, s); break;
    case 4: hard_forward_t<T, 4, D>(p, h, q, k, v, causal, o, den, count, ws, s); break;
    default: hard_forward_t<T, 8, D>(p, h, q, k, v, causal, o, den, count, ws, s); break;
    }
}

void hard_forward_launch(const Plan &p, int Lr, int Pr, race_dtype_t dt, const void *Q, const void *K,
                         const void *V, const float *W, int causal, void *O, float *den, int *count,
                         char *ws, hipStream_t s)
{
    const HardPlan h = hard_plan(p, Lr, Pr);
    // the bucket ids of every row of Q and of K (P = 5, 6: as 2^(P-4)
    // virtual tables of 16 buckets per table, the p.L tables the kernels see)
    const int vshift = Pr > 4 ? Pr - 4 : 0;
    const int64_t rows = p.lens.cu ? (int64_t)p.lens.H * p.lens.T : p.rows;
    hard_ids_launch(Q, rows, p.d, dt, W, Lr, Pr, reinterpret_cast<uint8_t *>(ws + h.o_idq), ws + h.o_w, s,
                    vshift);
    hard_ids_launch(K, rows, p.d, dt, W, Lr, Pr, reinterpret_cast<uint8_t *>(ws + h.o_idk), ws + h.o_w, s,
                    vshift);
    if (dt == RACE_BF16) {
        if (p.d == 32) hard_forward_d<bf16, 32>(p, h, Q, K, V, causal, O, den, count, ws, s);
        else hard_forward_d<bf16, race::HD>(p, h, Q, K, V, causal, O, den, count, ws, s);
    } else {
        if (p.d == 32) hard_forward_d<_Float16, 32>(p, h, Q, K, V, causal, O, den, count, ws, s);
        else hard_forward_d<_Float16, race::HD>(p, h, Q, K, V, causal, O, den, count, ws, s);
    }
}

}  // namespace race_host
