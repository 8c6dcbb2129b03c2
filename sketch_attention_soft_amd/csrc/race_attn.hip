// race_attn.hip -- C ABI of the RACE attention library (declared in include/race_attn.h).
//
// Host side: argument validation, workspace planning and kernel sequencing
// on the caller's stream.  No allocation, no synchronisation, no global
// mutable state.
#include "race_attn.h"

#include <cmath>
#include <cstring>

#include "race_bwd.h"
#include "race_common.h"
#include "race_fwd.h"

namespace {

using race::bf16;

constexpr int64_t kMaxN = (int64_t)1 << 40;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Plan {
    int64_t BH, N, rows;
    int L, nw, F, LP;
    int64_t seg, nseg;
    size_t st_bytes;   // one set of segment states (nseg + 1 per head)
    size_t t_bytes;    // forward hash features of Q or K
    size_t tb_bytes;   // backward hash features (t and dt/du) of Q or K
    size_t wt_bytes;   // transposed projection for the backward
    // forward layout
    size_t f_tq, f_tk, f_st, f_total;
    // backward layout
    size_t b_tq, b_tk, b_s, b_gt, b_g, b_wt, b_total;
};

race_status_t make_plan(int B, int H, int64_t N, int d, int L, int P, int chunk,
                        race_dtype_t dt, Plan *p)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || L < 1 || P < 1) return RACE_ERR_SHAPE;
    if (N > kMaxN || (int64_t)B * H > 65535) return RACE_ERR_SHAPE;
    if (dt != RACE_F32 && dt != RACE_BF16) return RACE_ERR_UNSUPPORTED;
    if (d != race::HD || P != race::NP) return RACE_ERR_UNSUPPORTED;
    if (L > 64 || (dt == RACE_F32 && L > 32)) return RACE_ERR_UNSUPPORTED;
    if (chunk < 0 || chunk % race::CH != 0) return RACE_ERR_CHUNK;
    p->BH = (int64_t)B * H;
    p->N = N;
    p->rows = p->BH * N;
    p->L = L;
    p->nw = L <= 8 ? 1 : L <= 16 ? 2 : L <= 32 ? 4 : 8;
    p->F = p->nw * race::FPW;
    p->LP = L * race::NP;
    const int64_t n16 = (N + 15) / 16 * 16;
    int64_t seg = chunk;
    if (seg == 0) {
        // about 2048 workgroups in total, segments of 64 .. 8192 tokens
        const int64_t want = (p->rows + 2047) / 2048;
        seg = (want + 15) / 16 * 16;
        if (seg < 64) seg = 64;
        if (seg > 8192) seg = 8192;
    }
    if (seg > n16) seg = n16;
    p->seg = seg;
    p->nseg = (N + seg - 1) / seg;
    if (p->BH * p->nseg > 0x7fffffffLL) return RACE_ERR_SHAPE;
    p->st_bytes = align256((size_t)p->BH * (p->nseg + 1) * p->F * race::NCOL * sizeof(float));
    p->t_bytes = align256((size_t)p->rows * L * race::NP * sizeof(float));
    p->tb_bytes = align256((size_t)p->rows * L * 2 * race::NP * sizeof(float));
    const int lp32 = (p->LP + 31) / 32 * 32;
    p->wt_bytes = align256((size_t)race::HD * lp32 * (2 * sizeof(bf16) + sizeof(float)));
    p->f_tq = 0;
    p->f_tk = p->f_tq + p->t_bytes;
    p->f_st = p->f_tk + p->t_bytes;
    p->f_total = p->f_st + p->st_bytes;
    p->b_tq = 0;
    p->b_tk = p->b_tq + p->tb_bytes;
    p->b_s = p->b_tk + p->tb_bytes;
    p->b_gt = p->b_s + p->st_bytes;
    p->b_g = p->b_gt + p->st_bytes;
    p->b_wt = p->b_g + p->st_bytes;
    p->b_total = p->b_wt + p->wt_bytes;
    return RACE_OK;
}

race_status_t check_tau(float tau)
{
    return (std::isfinite(tau) && tau > 0.f) ? RACE_OK : RACE_ERR_TAU;
}

race_status_t check_ws(const Plan &p, size_t need, const void *ws, size_t ws_bytes)
{
    if (ws_bytes < need) return RACE_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255) != 0) return RACE_ERR_WORKSPACE;
    (void)p;
    return RACE_OK;
}

int hash_grid(int64_t rows)
{
    const int64_t tiles = (rows + 15) / 16;
    const int64_t blocks = (tiles + 3) / 4;
    return (int)(blocks < 16384 ? blocks : 16384);
}

template <typename T, int NW>
void launch_forward(const Plan &p, const T *Q, const T *K, const T *V, const float *W, float tau,
                    int causal, T *O, float *den, char *ws, hipStream_t s)
{
    float *tq = reinterpret_cast<float *>(ws + p.f_tq);
    float *tk = reinterpret_cast<float *>(ws + p.f_tk);
    float *st = reinterpret_cast<float *>(ws + p.f_st);
    const float inv_tau = 1.0f / tau;
    const int hg = hash_grid(p.rows);
    hipLaunchKernelGGL((race::hash_kernel<T, false>), dim3(hg), dim3(256), 0, s, Q, p.rows, W,
                       p.L, inv_tau, tq);
    hipLaunchKernelGGL((race::hash_kernel<T, false>), dim3(hg), dim3(256), 0, s, K, p.rows, W,
                       p.L, inv_tau, tk);
    const race::ValSrc<T> vs{V, nullptr, nullptr};
    const int nblk = (int)(p.BH * p.nseg);
    hipLaunchKernelGGL((race::seg_sum_kernel<T, NW, false, false>), dim3(nblk), dim3(NW * 64), 0,
                       s, tk, race::NP, vs, p.N, p.L, (int)p.seg, p.nseg, st);
    const int64_t elems = (int64_t)p.F * race::NCOL;
    hipLaunchKernelGGL(race::scan_kernel, dim3((unsigned)((elems + 255) / 256), (unsigned)p.BH),
                       dim3(256), 0, s, st, p.nseg, elems, 0);
    if (causal)
        hipLaunchKernelGGL((race::readout_kernel<T, NW, true, false>), dim3(nblk), dim3(NW * 64),
                           0, s, tq, tk, race::NP, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den);
    else
        hipLaunchKernelGGL((race::readout_kernel<T, NW, false, false>), dim3(nblk), dim3(NW * 64),
                           0, s, tq, tk, race::NP, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den);
}

template <typename T, int NW>
void launch_backward(const Plan &p, const T *Q, const T *K, const T *V, const float *W,
                     const T *O, const float *den, const T *dO, float tau, int causal, T *dQ,
                     T *dK, T *dV, char *ws, hipStream_t s)
{
    float *tq = reinterpret_cast<float *>(ws + p.b_tq);
    float *tk = reinterpret_cast<float *>(ws + p.b_tk);
    float *sS = reinterpret_cast<float *>(ws + p.b_s);    // key state, [80 x F] layout
    float *sGt = reinterpret_cast<float *>(ws + p.b_gt);  // gradient state, [80 x F] layout
    float *sG = reinterpret_cast<float *>(ws + p.b_g);    // gradient state, [F x 80] layout
    char *wt = ws + p.b_wt;
    const float inv_tau = 1.0f / tau;
    const int hg = hash_grid(p.rows);
    const int lp32 = (p.LP + 31) / 32 * 32;
    hipLaunchKernelGGL(race::prep_wt_kernel, dim3((race::HD * lp32 + 255) / 256), dim3(256), 0, s,
                       W, p.LP, lp32, wt);
    hipLaunchKernelGGL((race::hash_kernel<T, true>), dim3(hg), dim3(256), 0, s, Q, p.rows, W,
                       p.L, inv_tau, tq);
    hipLaunchKernelGGL((race::hash_kernel<T, true>), dim3(hg), dim3(256), 0, s, K, p.rows, W,
                       p.L, inv_tau, tk);
    const race::ValSrc<T> vv{V, nullptr, nullptr};     // [v | 1]
    const race::ValSrc<T> vd{dO, O, den};              // [dO/m | -(dO.o)/m]
    const int nblk = (int)(p.BH * p.nseg);
    const int64_t elems = (int64_t)p.F * race::NCOL;
    const dim3 sgrid((unsigned)((elems + 255) / 256), (unsigned)p.BH);
    const int ts = 2 * race::NP;
    // key-side state S^T (for dQ), prefix over segments
    hipLaunchKernelGGL((race::seg_sum_kernel<T, NW, true, false>), dim3(nblk), dim3(NW * 64), 0,
                       s, tk, ts, vv, p.N, p.L, (int)p.seg, p.nseg, sS);
    hipLaunchKernelGGL(race::scan_kernel, sgrid, dim3(256), 0, s, sS, p.nseg, elems, 0);
    // query-side gradient states G^T (for dK) and G (for dV), suffix over segments
    hipLaunchKernelGGL((race::seg_sum_kernel<T, NW, true, true>), dim3(nblk), dim3(NW * 64), 0,
                       s, tq, ts, vd, p.N, p.L, (int)p.seg, p.nseg, sGt);
    hipLaunchKernelGGL(race::scan_kernel, sgrid, dim3(256), 0, s, sGt, p.nseg, elems, 1);
    hipLaunchKernelGGL((race::seg_sum_kernel<T, NW, false, true>), dim3(nblk), dim3(NW * 64), 0,
                       s, tq, ts, vd, p.N, p.L, (int)p.seg, p.nseg, sG);
    hipLaunchKernelGGL(race::scan_kernel, sgrid, dim3(256), 0, s, sG, p.nseg, elems, 1);
    // dQ: readers Q (values D), writers K (values [v|1]), forward order
    // dK: readers K (values [v|1]), writers Q (values D), reverse order
    if (causal) {
        hipLaunchKernelGGL((race::dpsi_kernel<T, NW, 1, false, true>), dim3(nblk), dim3(NW * 64),
                           0, s, Q, tq, tk, vd, vv, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sS, dQ);
        hipLaunchKernelGGL((race::dpsi_kernel<T, NW, 1, true, false>), dim3(nblk), dim3(NW * 64),
                           0, s, K, tk, tq, vv, vd, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sGt, dK);
        hipLaunchKernelGGL((race::readout_kernel<T, NW, true, true>), dim3(nblk), dim3(NW * 64), 0,
                           s, tk, tq, ts, vd, p.N, p.L, (int)p.seg, p.nseg, sG, dV, nullptr);
    } else {
        hipLaunchKernelGGL((race::dpsi_kernel<T, NW, 0, false, true>), dim3(nblk), dim3(NW * 64),
                           0, s, Q, tq, tk, vd, vv, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sS, dQ);
        hipLaunchKernelGGL((race::dpsi_kernel<T, NW, 0, true, false>), dim3(nblk), dim3(NW * 64),
                           0, s, K, tk, tq, vv, vd, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sGt, dK);
        hipLaunchKernelGGL((race::readout_kernel<T, NW, false, true>), dim3(nblk), dim3(NW * 64),
                           0, s, tk, tq, ts, vd, p.N, p.L, (int)p.seg, p.nseg, sG, dV, nullptr);
    }
}

template <typename T>
void dispatch_forward(const Plan &p, const void *Q, const void *K, const void *V, const float *W,
                      float tau, int causal, void *O, float *den, char *ws, hipStream_t s)
{
    auto q = static_cast<const T *>(Q);
    auto k = static_cast<const T *>(K);
    auto v = static_cast<const T *>(V);
    auto o = static_cast<T *>(O);
    switch (p.nw) {
    case 1: launch_forward<T, 1>(p, q, k, v, W, tau, causal, o, den, ws, s); break;
    case 2: launch_forward<T, 2>(p, q, k, v, W, tau, causal, o, den, ws, s); break;
    case 4: launch_forward<T, 4>(p, q, k, v, W, tau, causal, o, den, ws, s); break;
    default:
        if constexpr (sizeof(T) == 2) launch_forward<T, 8>(p, q, k, v, W, tau, causal, o, den, ws, s);
        break;
    }
}

template <typename T>
void dispatch_backward(const Plan &p, const void *Q, const void *K, const void *V,
                       const float *W, const void *O, const float *den, const void *dO,
                       float tau, int causal, void *dQ, void *dK, void *dV, char *ws,
                       hipStream_t s)
{
    auto q = static_cast<const T *>(Q);
    auto k = static_cast<const T *>(K);
    auto v = static_cast<const T *>(V);
    auto o = static_cast<const T *>(O);
    auto go = static_cast<const T *>(dO);
    auto dq = static_cast<T *>(dQ);
    auto dk = static_cast<T *>(dK);
    auto dv = static_cast<T *>(dV);
    switch (p.nw) {
    case 1: launch_backward<T, 1>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, s); break;
    case 2: launch_backward<T, 2>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, s); break;
    case 4: launch_backward<T, 4>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, s); break;
    default:
        if constexpr (sizeof(T) == 2)
            launch_backward<T, 8>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, s);
        break;
    }
}

}  // namespace

extern "C" {

race_status_t race_attn_workspace_bytes(int B, int H, int64_t N, int d, int L, int P,
                                        int causal, int chunk, race_dtype_t dt,
                                        int for_backward, size_t *bytes)
{
    (void)causal;
    if (!bytes) return RACE_ERR_NULL;
    Plan p;
    const race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    *bytes = for_backward ? p.b_total : p.f_total;
    return RACE_OK;
}

race_status_t race_attn_forward(const void *Q, const void *K, const void *V, const float *W,
                                int L, int P, float tau, int causal, int B, int H, int64_t N,
                                int d, race_dtype_t dt, int chunk, void *O, float *den,
                                void *workspace, size_t ws_bytes, void *stream)
{
    if (!Q || !K || !V || !W || !O || !den || !workspace) return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (dt == RACE_BF16)
        dispatch_forward<bf16>(p, Q, K, V, W, tau, causal, O, den, ws, s);
    else
        dispatch_forward<float>(p, Q, K, V, W, tau, causal, O, den, ws, s);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_backward(const void *Q, const void *K, const void *V, const float *W,
                                 const void *O, const float *den, const void *dO, int L,
                                 int P, float tau, int causal, int B, int H, int64_t N, int d,
                                 race_dtype_t dt, int chunk, void *dQ, void *dK, void *dV,
                                 void *workspace, size_t ws_bytes, void *stream)
{
    if (!Q || !K || !V || !W || !O || !den || !dO || !dQ || !dK || !dV || !workspace)
        return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, p.b_total, workspace, ws_bytes)) != RACE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (dt == RACE_BF16)
        dispatch_backward<bf16>(p, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, s);
    else
        dispatch_backward<float>(p, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, s);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

const char *race_attn_status_string(race_status_t status)
{
    switch (status) {
    case RACE_OK: return "success";
    case RACE_ERR_NULL: return "a required pointer is NULL";
    case RACE_ERR_SHAPE: return "B, H, N, d, L or P out of range";
    case RACE_ERR_UNSUPPORTED: return "unsupported configuration (d, P, L or dtype)";
    case RACE_ERR_TAU: return "tau must be finite and > 0";
    case RACE_ERR_CHUNK: return "chunk must be 0 or a positive multiple of 16";
    case RACE_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case RACE_ERR_HIP: return "HIP kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
