// race_host.h -- host-side planning and kernel sequencing of the RACE
// attention library, shared by the C ABI (race_attn.hip) and the files that
// instantiate the launch sequences per row type (race_inst_*.hip), which are
// compiled in parallel.
#pragma once
#include "race_attn.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <type_traits>

#include "race_bwd.h"
#include "race_common.h"
#include "race_fwd.h"
#include "race_stream.h"
#include "race_walk.h"
#include "race_hard.h"
#include "race_wide.h"

namespace race_host {

using race::bf16;

constexpr int64_t kMaxN = (int64_t)1 << 40;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Records caller-owned events around each launch when a trace is given.
struct Tracer {
    race_trace_t *t;
    hipStream_t s;
    void begin(const char *name) const
    {
        if (t && t->count < t->capacity) {
            t->name[t->count] = name;
            (void)hipEventRecord(static_cast<hipEvent_t>(t->start[t->count]), s);
        }
    }
    void end() const
    {
        if (t && t->count < t->capacity) {
            (void)hipEventRecord(static_cast<hipEvent_t>(t->stop[t->count]), s);
            t->count++;
        }
    }
};

#define LAUNCH(tr, name, kern, grid, block, ...)                                   \
    do {                                                                          \
        (tr).begin(name);                                                         \
        hipLaunchKernelGGL(kern, grid, block, 0, (tr).s, __VA_ARGS__);            \
        (tr).end();                                                               \
    } while (0)

struct Plan {
    int64_t BH, N, rows;
    int L, nw, F, LP;
    int d;             // head dimension (64, or 32 on the fused path)
    int P;             // hyperplanes per table (4, or 1..3 on the fused path)
    race::Lens lens;   // per-batch valid rows (right-padded batches), or none
    // L > 32 with 16-bit rows: two fused passes over 32 and L - 32 tables
    // (the sizes below are then those of both passes and the partial sums)
    bool split;
    int part_mode;     // PART_NONE, or this pass's PART_OUT / PART_IN
    race::Part part_o, part_dq, part_dk, part_dv;
    bool fused;        // bf16 and L <= 32: kernels hash their own rows
    bool wide;         // d = 128 (16-bit rows, L <= 32, P <= 4): two passes of 64 value columns
    int64_t seg, nseg;
    size_t st_bytes;   // one set of segment states (nseg + 1 per head)
    size_t t_bytes;    // forward hash features of Q or K
    size_t tb_bytes;   // backward hash features (t and dt/du) of Q or K
    size_t wt_bytes;   // transposed projection for the backward
    int scan_groups;   // segment groups of the two-pass scan
    size_t scan_bytes; // group totals of the scan
    int64_t hc_tiles;  // hash-feature cache: 16-token tiles per head (bf16 path)
    size_t hc_bytes;   // one cache array (t or dt/du' of Q or K), fp16
    // forward layout (hc: t of K)
    size_t f_tq, f_tk, f_st, f_hc, f_scan, f_total;
    // backward layout (hc: t, dt/du' of K then of Q)
    size_t b_tq, b_tk, b_s, b_gt, b_g, b_wt, b_hc, b_scan, b_total;
    size_t b_dw, dw_total;  // backward with dW (bf16, L <= 32): partials after b_total
    // saved buffer (bf16 path): key state, then t, dt/du' of K and of Q
    size_t s_hc, s_total;
    // d = 128, backward: du of Q and K per pass (bf16 [rows][16 * waves]),
    // the gradient values' last column (fp32 [rows])
    size_t w_du, w_du_bytes, w_dm;
};

race_status_t make_plan(int B, int H, int64_t N, int d, int L, int P, int chunk,
                        race_dtype_t dt, Plan *p);
race::Squash fit_squash(float tau, race_dtype_t dt);
race::Squash hard_squash();

inline int hash_grid(int64_t rows)
{
    const int64_t tiles = (rows + 15) / 16;
    const int64_t blocks = (tiles + 3) / 4;
    return (int)(blocks < 16384 ? blocks : 16384);
}

// exclusive prefix (reverse = 0) or suffix (reverse = 1) of the segment
// states of every head, plus the head totals
inline void launch_scan(const Tracer &tr, const char *name, const Plan &p, float *st, float *tmp,
                 int reverse)
{
    const int64_t elems = (int64_t)p.F * race::NCOL;
    const dim3 grid((unsigned)((elems + 255) / 256), (unsigned)p.scan_groups, (unsigned)p.BH);
    tr.begin(name);
    hipLaunchKernelGGL(race::scan_reduce_kernel, grid, dim3(256), 0, tr.s, st, tmp, p.nseg, elems,
                       p.scan_groups);
    hipLaunchKernelGGL(race::scan_apply_kernel, grid, dim3(256), 0, tr.s, st, tmp, p.nseg, elems,
                       p.scan_groups, reverse);
    tr.end();
}

// hash-feature cache arrays (t, dt/du') at base, in units of hc_bytes
inline race::HCache hcache(const Plan &p, char *base, int it, int ic)
{
    race::HCache h;
    h.t = it >= 0 ? reinterpret_cast<_Float16 *>(base + it * p.hc_bytes) : nullptr;
    h.c = ic >= 0 ? reinterpret_cast<_Float16 *>(base + ic * p.hc_bytes) : nullptr;
    h.tiles = p.hc_tiles;
    return h;
}

// segment sums: hashing (SRC = 0, squash polynomial or direct) or from the cache
template <int NW, bool DVAL, int SRC, int WR, int D, typename T>
void launch_sum(const Tracer &tr, const char *name, dim3 grid, const race::Squash &sq, const T *X,
                const race::ValSrc<T> &vs, const float *W, const Plan &p, const race::HCache &cin,
                const race::HCache &cout, float *st)
{
    if constexpr (sizeof(T) == 2) {
        auto go = [&](auto pv_c) {
            constexpr bool PV = decltype(pv_c)::value;
            if (SRC == 1 || sq.deg >= 0)
                LAUNCH(tr, name, (race::sum_kernel<NW, DVAL, SRC, WR, true, T, D, PV>), grid, dim3(NW * 64),
                       X, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, cin, cout, st, p.lens);
            else
                LAUNCH(tr, name, (race::sum_kernel<NW, DVAL, SRC, WR, false, T, D, PV>), grid, dim3(NW * 64),
                       X, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, cin, cout, st, p.lens);
        };
        // P = 5, 6 (virtual tables): d = 64 only
        if constexpr (D == race::HD) {
            if (p.P > race::NP) return go(std::true_type{});
        }
        go(std::false_type{});
    }
}

// chunk walk: readers hashed (RSRC = 0) or from the cache, writers from the cache
template <int NW, bool CAUSAL, bool BWD, int RSRC, int RWR, int D, typename T>
void launch_walk(const Tracer &tr, const char *name, dim3 grid, const race::Squash &sq, const T *R,
                 const race::ValSrc<T> &vs, const float *W, const Plan &p, const float *st,
                 const race::HCache &rc, const race::HCache &wc, T *out, float *den)
{
    if constexpr (sizeof(T) == 2) {
        const race::Part pt = BWD ? p.part_dv : p.part_o;
        auto go2 = [&](auto part_c, auto pv_c) {
            constexpr int PT = decltype(part_c)::value;
            constexpr bool PV = decltype(pv_c)::value;
            if (RSRC == 1 || sq.deg >= 0)
                LAUNCH(tr, name, (race::walk_kernel<NW, CAUSAL, BWD, RSRC, RWR, true, T, D, PT, PV>), grid,
                       dim3(NW * 64), R, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, st, rc, wc, out,
                       den, p.lens, pt);
            else
                LAUNCH(tr, name, (race::walk_kernel<NW, CAUSAL, BWD, RSRC, RWR, false, T, D, PT, PV>), grid,
                       dim3(NW * 64), R, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, st, rc, wc, out,
                       den, p.lens, pt);
        };
        // P = 5, 6 (virtual tables): d = 64 only
        auto go = [&](auto part_c) {
            if constexpr (D == race::HD) {
                if (p.P > race::NP) return go2(part_c, std::true_type{});
            }
            go2(part_c, std::false_type{});
        };
        // every pass but the last has 32 tables (NW = 8); split runs have d = 64
        if (p.part_mode == race::PART_NONE) {
            go(std::integral_constant<int, race::PART_NONE>{});
        } else if constexpr (D == race::HD) {
            if (p.part_mode == race::PART_IN) {
                go(std::integral_constant<int, race::PART_IN>{});
            } else if constexpr (NW == 8) {
                if (p.part_mode == race::PART_OUT)
                    go(std::integral_constant<int, race::PART_OUT>{});
                else
                    go(std::integral_constant<int, race::PART_MID>{});
            }
        }
    }
}

template <int NW, bool CAUSAL, bool REVERSE, int D, typename T>
void launch_grad(const Tracer &tr, const char *name, dim3 grid, const T *Xr,
                 const race::ValSrc<T> &vr, const race::ValSrc<T> &vw, const float *W,
                 const Plan &p, const float *st, const race::HCache &rc, const race::HCache &wc,
                 T *dX, float *dwp)
{
    if constexpr (sizeof(T) == 2) {
        const race::Part pt = REVERSE ? p.part_dk : p.part_dq;
        auto go2 = [&](auto part_c, auto pv_c) {
            constexpr int PT = decltype(part_c)::value;
            constexpr bool PV = decltype(pv_c)::value;
            if constexpr (D > race::HD)  // rows of 128: dwp takes du
                LAUNCH(tr, name, (race::grad_kernel<NW, CAUSAL, REVERSE, false, T, D, PT, PV>), grid,
                       dim3(NW * 64), Xr, vr, vw, W, p.L, p.P, p.N, (int)p.seg, p.nseg, st, rc, wc, dX,
                       dwp, p.lens, pt);
            else if (dwp)
                LAUNCH(tr, name, (race::grad_kernel<NW, CAUSAL, REVERSE, true, T, D, PT, PV>), grid,
                       dim3(NW * 64), Xr, vr, vw, W, p.L, p.P, p.N, (int)p.seg, p.nseg, st, rc, wc, dX,
                       dwp, p.lens, pt);
            else
                LAUNCH(tr, name, (race::grad_kernel<NW, CAUSAL, REVERSE, false, T, D, PT, PV>), grid,
                       dim3(NW * 64), Xr, vr, vw, W, p.L, p.P, p.N, (int)p.seg, p.nseg, st, rc, wc, dX,
                       nullptr, p.lens, pt);
        };
        // P = 5, 6 (virtual tables): d = 64 only
        auto go = [&](auto part_c) {
            if constexpr (D == race::HD) {
                if (p.P > race::NP) return go2(part_c, std::true_type{});
            }
            go2(part_c, std::false_type{});
        };
        if (p.part_mode == race::PART_NONE) {
            go(std::integral_constant<int, race::PART_NONE>{});
        } else if constexpr (D == race::HD) {
            if (p.part_mode == race::PART_IN) {
                go(std::integral_constant<int, race::PART_IN>{});
            } else if constexpr (NW == 8) {
                if (p.part_mode == race::PART_OUT)
                    go(std::integral_constant<int, race::PART_OUT>{});
                else
                    go(std::integral_constant<int, race::PART_MID>{});
            }
        }
    }
}

// D = d: 64, or 32 on the fused path (bf16 / fp16 rows, L <= 32)
template <typename T, int NW, int D>
void launch_forward(const Plan &p, const T *Q, const T *K, const T *V, const float *W, float tau,
                    int causal, T *O, float *den, char *ws, float *saved, const Tracer &tr)
{
    float *tq = reinterpret_cast<float *>(ws + p.f_tq);
    float *tk = reinterpret_cast<float *>(ws + p.f_tk);
    // key state: into the caller's saved buffer when given (bf16 path)
    float *st = saved ? saved : reinterpret_cast<float *>(ws + p.f_st);
    float *scan_tmp = reinterpret_cast<float *>(ws + p.f_scan);
    // tau = 0 (race_attn_forward_hard only): hard hashing
    const bool hard = tau == 0.f;
    const float inv_tau = hard ? 0.f : 1.0f / tau;
    const dim3 hg(hash_grid(p.rows)), b256(256), bw(NW * 64);
    if constexpr (sizeof(T) == 2 && NW <= 4) {
        // bf16 path: 2 NW waves of 4 tables each (16 hyperplanes, 64 features)
        constexpr int WS = 2 * NW, WW = 2 * NW;
        const race::Squash sq = hard ? hard_squash() : fit_squash(tau, RACE_BF16);
        const dim3 nblk((unsigned)(p.BH * p.nseg));
        const race::ValSrc<T> vv{V, nullptr, nullptr};
        // hash features: K (t) in the workspace, or K and Q (t, dt/du') in the saved buffer
        char *sb = reinterpret_cast<char *>(saved);
        const race::HCache hk = saved ? hcache(p, sb + p.s_hc, 0, 1) : hcache(p, ws + p.f_hc, 0, -1);
        const race::HCache hq = saved ? hcache(p, sb + p.s_hc, 2, 3) : hcache(p, nullptr, -1, -1);
        const race::HCache none = hcache(p, nullptr, -1, -1);
        if (saved)
            launch_sum<WS, false, 0, 3, D>(tr, "sum_kv", nblk, sq, K, vv, W, p, none, hk, st);
        else
            launch_sum<WS, false, 0, 1, D>(tr, "sum_kv", nblk, sq, K, vv, W, p, none, hk, st);
        launch_scan(tr, "scan_kv", p, st, scan_tmp, 0);
        if (causal) {
            if (saved)
                launch_walk<WW, true, false, 0, 3, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O, den);
            else
                launch_walk<WW, true, false, 0, 0, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O, den);
        } else {
            if (saved)
                launch_walk<WW, false, false, 0, 3, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O, den);
            else
                launch_walk<WW, false, false, 0, 0, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O, den);
        }
        return;
    }
    if constexpr (!std::is_same<T, _Float16>::value && D == race::HD) {  // fp16 rows, d = 32: fused path only
    // fp32 rows: t of Q and K in the workspace, or t and dt/du' (the
    // backward's chain rows, 8 floats per table) in the saved buffer
    int ts = race::NP;
    if (saved) {
        tq = saved;
        tk = reinterpret_cast<float *>(reinterpret_cast<char *>(saved) + p.tb_bytes);
        ts = 2 * race::NP;
        st = reinterpret_cast<float *>(ws + p.f_st);
        LAUNCH(tr, "hash_q", (race::hash_kernel<T, true>), hg, b256, Q, p.rows, W, p.L, inv_tau, tq);
        LAUNCH(tr, "hash_k", (race::hash_kernel<T, true>), hg, b256, K, p.rows, W, p.L, inv_tau, tk);
    } else {
        LAUNCH(tr, "hash_q", (race::hash_kernel<T, false>), hg, b256, Q, p.rows, W, p.L, inv_tau, tq);
        LAUNCH(tr, "hash_k", (race::hash_kernel<T, false>), hg, b256, K, p.rows, W, p.L, inv_tau, tk);
    }
    const race::ValSrc<T> vs{V, nullptr, nullptr};
    const dim3 nblk((unsigned)(p.BH * p.nseg));
    LAUNCH(tr, "seg_sum_kv", (race::seg_sum_kernel<T, NW, false, false>), nblk, bw, tk, ts,
           vs, p.N, p.L, (int)p.seg, p.nseg, st, p.lens);
    launch_scan(tr, "scan_kv", p, st, scan_tmp, 0);
    if (causal)
        LAUNCH(tr, "readout_o", (race::readout_kernel<T, NW, true, false>), nblk, bw, tq, tk,
               ts, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den, p.lens, p.part_o, p.part_mode);
    else
        LAUNCH(tr, "readout_o", (race::readout_kernel<T, NW, false, false>), nblk, bw, tq, tk,
               ts, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den, p.lens, p.part_o, p.part_mode);
    }
}

template <typename T, int NW, int CAUSAL, int D>
void launch_backward_body(const Plan &p, const T *Q, const T *K, const T *V, const float *W,
                          const T *O, const float *den, const T *dO, float tau, T *dQ, T *dK,
                          T *dV, char *ws, const float *saved, const Tracer &tr, float *dW)
{
    float *tq = reinterpret_cast<float *>(ws + p.b_tq);
    float *tk = reinterpret_cast<float *>(ws + p.b_tk);
    float *sS = reinterpret_cast<float *>(ws + p.b_s);    // key state (CxF; FxC on the bf16 path)
    float *sGt = reinterpret_cast<float *>(ws + p.b_gt);  // gradient state, CxF layout (fp32 / L > 32)
    float *sG = reinterpret_cast<float *>(ws + p.b_g);    // gradient state, FxC layout
    char *wt = ws + p.b_wt;
    float *scan_tmp = reinterpret_cast<float *>(ws + p.b_scan);
    const float inv_tau = 1.0f / tau;
    const int lp32 = (p.LP + 31) / 32 * 32;
    const dim3 hg(hash_grid(p.rows)), b256(256), bw(NW * 64);
    if constexpr (sizeof(T) == 2 && NW <= 4) {
        // bf16 path: 2 NW waves of 4 tables each (16 hyperplanes, 64 features)
        constexpr int WS = 2 * NW, WW = 2 * NW, WD = 2 * NW;
        const race::Squash sq = fit_squash(tau, RACE_BF16);
        const race::ValSrc<T> vv{V, nullptr, nullptr};  // [v | 1]
        const race::ValSrc<T> vd{dO, O, den};           // [dO/m | -(dO.o)/m]
        const dim3 nblk((unsigned)(p.BH * p.nseg));
        // key state S (FxC, read transposed by dQ) and the hash features of K
        // and Q (t, dt/du'): the forward's saved copies, or recomputed
        const float *sK;
        race::HCache hk, hq;
        const race::HCache none = hcache(p, nullptr, -1, -1);
        if (saved) {
            const char *sb = reinterpret_cast<const char *>(saved);
            sK = saved;
            hk = hcache(p, const_cast<char *>(sb) + p.s_hc, 0, 1);
            hq = hcache(p, const_cast<char *>(sb) + p.s_hc, 2, 3);
            // gradient state G (FxC; read transposed by dK): suffix over segments
            launch_sum<WS, true, 1, 0, D>(tr, "sum_qd", nblk, sq, Q, vd, W, p, hq, none, sG);
        } else {
            hk = hcache(p, ws + p.b_hc, 0, 1);
            hq = hcache(p, ws + p.b_hc, 2, 3);
            launch_sum<WS, false, 0, 3, D>(tr, "sum_kv_t", nblk, sq, K, vv, W, p, none, hk, sS);
            launch_scan(tr, "scan_kv_t", p, sS, scan_tmp, 0);
            sK = sS;
            launch_sum<WS, true, 0, 3, D>(tr, "sum_qd", nblk, sq, Q, vd, W, p, none, hq, sG);
        }
        launch_scan(tr, "scan_qd", p, sG, scan_tmp, 1);
        // dW (when asked): partial sums of the dQ and dK workgroups, then their sum
        float *dwp = dW ? reinterpret_cast<float *>(ws + p.b_dw) : nullptr;
        const int64_t dwb = p.BH * p.nseg * (int64_t)(WD * 16 * race::HD);
        launch_grad<WD, CAUSAL != 0, false, D>(tr, "dq", nblk, Q, vd, vv, W, p, sK, hq, hk, dQ, dwp);
        launch_grad<WD, CAUSAL != 0, true, D>(tr, "dk", nblk, K, vv, vd, W, p, sG, hk, hq, dK,
                                           dwp ? dwp + dwb : nullptr);
        if (dW)
            LAUNCH(tr, "dw_reduce", race::dw_reduce_kernel, dim3((p.LP * race::HD + 31) / 32),
                   dim3(256), dwp, 2 * p.BH * p.nseg, WD * 16, p.LP, p.L, p.P, D, dW);
        launch_walk<WW, CAUSAL != 0, true, 1, 0, D>(tr, "dv", nblk, sq, K, vd, W, p, sG, hk, hq, dV,
                                                 nullptr);
        return;
    }
    if constexpr (!std::is_same<T, _Float16>::value && D == race::HD) {  // fp16 rows, d = 32: fused path only
    LAUNCH(tr, "prep_wt", race::prep_wt_kernel, dim3((race::HD * lp32 + 255) / 256), b256, W,
           p.LP, lp32, wt);
    // t and dt/du' of Q and K: the forward's saved rows, or hashed here
    if (saved) {
        tq = const_cast<float *>(saved);
        tk = reinterpret_cast<float *>(reinterpret_cast<char *>(const_cast<float *>(saved)) + p.tb_bytes);
    } else {
        LAUNCH(tr, "hash_q_chain", (race::hash_kernel<T, true>), hg, b256, Q, p.rows, W, p.L,
               inv_tau, tq);
        LAUNCH(tr, "hash_k_chain", (race::hash_kernel<T, true>), hg, b256, K, p.rows, W, p.L,
               inv_tau, tk);
    }
    const race::ValSrc<T> vv{V, nullptr, nullptr};  // [v | 1]
    const race::ValSrc<T> vd{dO, O, den};           // [dO/m | -(dO.o)/m]
    const dim3 nblk((unsigned)(p.BH * p.nseg));
    const int ts = 2 * race::NP;
    // key-side state S (CxF, for dQ): prefix over segments
    LAUNCH(tr, "seg_sum_kv_t", (race::seg_sum_kernel<T, NW, true, false>), nblk, bw, tk, ts, vv,
           p.N, p.L, (int)p.seg, p.nseg, sS, p.lens);
    launch_scan(tr, "scan_kv_t", p, sS, scan_tmp, 0);
    // query-side gradient states G (CxF for dK, FxC for dV): suffix over segments
    LAUNCH(tr, "seg_sum_qd_t", (race::seg_sum_kernel<T, NW, true, true>), nblk, bw, tq, ts, vd,
           p.N, p.L, (int)p.seg, p.nseg, sGt, p.lens);
    launch_scan(tr, "scan_qd_t", p, sGt, scan_tmp, 1);
    LAUNCH(tr, "seg_sum_qd", (race::seg_sum_kernel<T, NW, false, true>), nblk, bw, tq, ts, vd,
           p.N, p.L, (int)p.seg, p.nseg, sG, p.lens);
    launch_scan(tr, "scan_qd", p, sG, scan_tmp, 1);
    // dQ: readers Q (values D), writers K (values [v|1]), token order
    LAUNCH(tr, "dpsi_q", (race::dpsi_kernel<T, NW, CAUSAL, false, true>), nblk, bw, Q, tq, tk, vd,
           vv, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sS, dQ, p.lens, p.part_dq, p.part_mode);
    // dK: readers K (values [v|1]), writers Q (values D), reverse order
    LAUNCH(tr, "dpsi_k", (race::dpsi_kernel<T, NW, CAUSAL, true, false>), nblk, bw, K, tk, tq, vv,
           vd, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sGt, dK, p.lens, p.part_dk, p.part_mode);
    // dV: keys read the FxC gradient state, reverse order
    LAUNCH(tr, "readout_dv", (race::readout_kernel<T, NW, CAUSAL != 0, true>), nblk, bw, tk, tq,
           ts, vd, p.N, p.L, (int)p.seg, p.nseg, sG, dV, nullptr, p.lens, p.part_dv, p.part_mode);
    }
}

template <typename T, int NW, int D>
void launch_backward(const Plan &p, const T *Q, const T *K, const T *V, const float *W,
                     const T *O, const float *den, const T *dO, float tau, int causal, T *dQ,
                     T *dK, T *dV, char *ws, const float *saved, const Tracer &tr, float *dW)
{
    if (causal)
        launch_backward_body<T, NW, 1, D>(p, Q, K, V, W, O, den, dO, tau, dQ, dK, dV, ws, saved, tr, dW);
    else
        launch_backward_body<T, NW, 0, D>(p, Q, K, V, W, O, den, dO, tau, dQ, dK, dV, ws, saved, tr, dW);
}

// Heads of d = 128 (16-bit rows, up to 32 tables, P <= 4).  The rows are
// hashed once into the feature cache (hash_rows_kernel); the fused kernels
// then run twice from the cache, on value columns 0..63 and 64..127 (both
// passes carry the count column, so each finds m).  In the backward both
// passes end at du (the first with the gradient values' last column, the
// second with a zero column: the gradient is linear in the values'
// columns), and du_rows_kernel adds them and forms dx_hat = du W and the
// normalisation backward over the whole row.
template <typename T>
void launch_hash_rows(const Tracer &tr, const char *name, const Plan &p, const T *X, const float *W,
                      float tau, const race::HCache &h)
{
    // every tile the chunk kernels read, a tile per wave at a time; two
    // workgroups per compute unit (the staged W takes 70 KB of LDS)
    const int64_t items = p.hc_tiles * p.BH;
    const dim3 grid((unsigned)std::min<int64_t>((items + 3) / 4, 512));
    LAUNCH(tr, name, race::hash_rows_kernel<T>, grid, dim3(256), X, p.N, p.d, W, p.L, p.P, 1.0f / tau,
           2 * p.nw, p.hc_tiles, p.BH, h.t, h.c);
}

// saved (optional): t and dt/du of K and Q, kept for the backward
template <typename T, int NW>
void launch_forward_wide(const Plan &p, const T *Q, const T *K, const T *V, const float *W, float tau,
                         int causal, T *O, float *den, char *ws, float *saved, const Tracer &tr)
{
    if constexpr (sizeof(T) == 2) {
        constexpr int WS = 2 * NW, D = 2 * race::HD;
        const race::Squash sq = fit_squash(tau, RACE_BF16);  // (not evaluated: t comes from the cache)
        const dim3 nblk((unsigned)(p.BH * p.nseg));
        float *st = reinterpret_cast<float *>(ws + p.f_st);
        float *scan_tmp = reinterpret_cast<float *>(ws + p.f_scan);
        char *sb = reinterpret_cast<char *>(saved);
        const race::HCache hk = saved ? hcache(p, sb + p.s_hc, 0, 1) : hcache(p, ws + p.f_hc, 0, -1);
        const race::HCache hq = saved ? hcache(p, sb + p.s_hc, 2, 3) : hcache(p, ws + p.f_hc, 1, -1);
        const race::HCache none = hcache(p, nullptr, -1, -1);
        launch_hash_rows(tr, "hash_k", p, K, W, tau, hk);
        launch_hash_rows(tr, "hash_q", p, Q, W, tau, hq);
        for (int c0 = 0; c0 < D; c0 += race::HD) {
            const race::ValSrc<T> vv{V + c0, nullptr, nullptr};
            launch_sum<WS, false, 1, 0, D>(tr, "sum_kv", nblk, sq, K, vv, W, p, hk, none, st);
            launch_scan(tr, "scan_kv", p, st, scan_tmp, 0);
            if (causal)
                launch_walk<WS, true, false, 1, 0, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O + c0, den);
            else
                launch_walk<WS, false, false, 1, 0, D>(tr, "fwd_o", nblk, sq, Q, vv, W, p, st, hq, hk, O + c0, den);
        }
    }
}

// saved (optional): the forward's t and dt/du of K and Q (else rehashed)
template <typename T, int NW, int CAUSAL>
void launch_backward_wide(const Plan &p, const T *Q, const T *K, const T *V, const float *W, const T *O,
                          const float *den, const T *dO, float tau, T *dQ, T *dK, T *dV, char *ws,
                          const float *saved, const Tracer &tr)
{
    if constexpr (sizeof(T) == 2) {
        constexpr int WS = 2 * NW, D = 2 * race::HD;
        const race::Squash sq = fit_squash(tau, RACE_BF16);
        const dim3 nblk((unsigned)(p.BH * p.nseg));
        float *sS = reinterpret_cast<float *>(ws + p.b_s);
        float *sG = reinterpret_cast<float *>(ws + p.b_g);
        float *scan_tmp = reinterpret_cast<float *>(ws + p.b_scan);
        char *hb = saved ? const_cast<char *>(reinterpret_cast<const char *>(saved)) + p.s_hc : ws + p.b_hc;
        const race::HCache hk = hcache(p, hb, 0, 1), hq = hcache(p, hb, 2, 3);
        const race::HCache none = hcache(p, nullptr, -1, -1);
        // du of Q for passes 0, 1, then of K
        bf16 *du[4];
        for (int i = 0; i < 4; ++i) du[i] = reinterpret_cast<bf16 *>(ws + p.w_du + i * p.w_du_bytes);
        float *dm = reinterpret_cast<float *>(ws + p.w_dm);
        if (!saved) {
            launch_hash_rows(tr, "hash_k_chain", p, K, W, tau, hk);
            launch_hash_rows(tr, "hash_q_chain", p, Q, W, tau, hq);
        }
        LAUNCH(tr, "dm_rows", race::dm_rows_kernel<T>, dim3((unsigned)((p.rows + race::WROWS - 1) / race::WROWS)),
               dim3(256), dO, O, den, p.rows, p.d, dm);
        for (int pass = 0; pass < 2; ++pass) {
            const int c0 = pass * race::HD;
            const race::ValSrc<T> vv{V + c0, nullptr, nullptr};                      // [v | 1]
            const race::ValSrc<T> vd{dO + c0, O + c0, den, pass == 0 ? dm : nullptr};  // [dO/m | dm or 0]
            launch_sum<WS, false, 1, 0, D>(tr, "sum_kv_t", nblk, sq, K, vv, W, p, hk, none, sS);
            launch_scan(tr, "scan_kv_t", p, sS, scan_tmp, 0);
            launch_sum<WS, true, 1, 0, D>(tr, "sum_qd", nblk, sq, Q, vd, W, p, hq, none, sG);
            launch_scan(tr, "scan_qd", p, sG, scan_tmp, 1);
            launch_grad<WS, CAUSAL != 0, false, D>(tr, "dq", nblk, Q, vd, vv, W, p, sS, hq, hk, dQ,
                                                   reinterpret_cast<float *>(du[pass]));
            launch_grad<WS, CAUSAL != 0, true, D>(tr, "dk", nblk, K, vv, vd, W, p, sG, hk, hq, dK,
                                                  reinterpret_cast<float *>(du[2 + pass]));
            launch_walk<WS, CAUSAL != 0, true, 1, 0, D>(tr, "dv", nblk, sq, K, vd, W, p, sG, hk, hq, dV + c0,
                                                        nullptr);
        }
        // blocks of 16 rows, one per wave at a time; four workgroups per compute unit
        const dim3 rg((unsigned)std::min<int64_t>(((p.rows + race::WROWS - 1) / race::WROWS + 3) / 4, 1024));
        LAUNCH(tr, "du_rows_q", race::du_rows_kernel<T>, rg, dim3(256), Q, p.rows, p.d, W, p.L, p.P, WS * 16,
               du[0], du[1], dQ);
        LAUNCH(tr, "du_rows_k", race::du_rows_kernel<T>, rg, dim3(256), K, p.rows, p.d, W, p.L, p.P, WS * 16,
               du[2], du[3], dK);
    }
}

template <typename T>
void dispatch_forward(const Plan &p, const void *Q, const void *K, const void *V, const float *W,
                      float tau, int causal, void *O, float *den, char *ws, float *saved,
                      const Tracer &tr)
{
    auto q = static_cast<const T *>(Q);
    auto k = static_cast<const T *>(K);
    auto v = static_cast<const T *>(V);
    auto o = static_cast<T *>(O);
    if constexpr (sizeof(T) == 2) {
        if (p.wide) {
            switch (p.nw) {
            case 1: launch_forward_wide<T, 1>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            case 2: launch_forward_wide<T, 2>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            default: launch_forward_wide<T, 4>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            }
            return;
        }
        if (p.d == 32) {  // the fused path only (L <= 32)
            switch (p.nw) {
            case 1: launch_forward<T, 1, 32>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            case 2: launch_forward<T, 2, 32>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            default: launch_forward<T, 4, 32>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
            }
            return;
        }
    }
    constexpr int D = race::HD;
    switch (p.nw) {
    case 1: launch_forward<T, 1, D>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
    case 2: launch_forward<T, 2, D>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
    default: launch_forward<T, 4, D>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
    }
}

template <typename T>
void dispatch_backward(const Plan &p, const void *Q, const void *K, const void *V,
                       const float *W, const void *O, const float *den, const void *dO,
                       float tau, int causal, void *dQ, void *dK, void *dV, char *ws,
                       const float *saved, const Tracer &tr, float *dW)
{
    auto q = static_cast<const T *>(Q);
    auto k = static_cast<const T *>(K);
    auto v = static_cast<const T *>(V);
    auto o = static_cast<const T *>(O);
    auto go = static_cast<const T *>(dO);
    auto dq = static_cast<T *>(dQ);
    auto dk = static_cast<T *>(dK);
    auto dv = static_cast<T *>(dV);
    if constexpr (sizeof(T) == 2) {
        if (p.wide) {
            auto run = [&](auto nw_c) {
                constexpr int NW = decltype(nw_c)::value;
                if (causal)
                    launch_backward_wide<T, NW, 1>(p, q, k, v, W, o, den, go, tau, dq, dk, dv, ws, saved, tr);
                else
                    launch_backward_wide<T, NW, 0>(p, q, k, v, W, o, den, go, tau, dq, dk, dv, ws, saved, tr);
            };
            switch (p.nw) {
            case 1: run(std::integral_constant<int, 1>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            default: run(std::integral_constant<int, 4>{}); break;
            }
            return;
        }
        if (p.d == 32) {  // the fused path only (L <= 32)
            switch (p.nw) {
            case 1: launch_backward<T, 1, 32>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
            case 2: launch_backward<T, 2, 32>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
            default: launch_backward<T, 4, 32>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
            }
            return;
        }
    }
    constexpr int D = race::HD;
    switch (p.nw) {
    case 1: launch_backward<T, 1, D>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
    case 2: launch_backward<T, 2, D>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
    default: launch_backward<T, 4, D>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
    }
}

// L > 32 with 16-bit rows: passes over tables 0..31, 32..63, ... (the last
// pass takes the rest) over the same rows.  The first pass stores its sums in
// fp32 (the readout's n and m; dx_hat of Q and of K; dV) in partial arrays
// after every pass's buffers, the middle passes add theirs, the last adds the
// stored sums before its last step.  Each pass has its own buffers and saved
// state; dW rows are those of its tables.
// 2^vt_shift(P) virtual tables per table (P = 5, 6)
inline int vt_shift(int P) { return P > race::NP ? P - race::NP : 0; }
// real tables per pass: 32 virtual tables
inline int split_step(int P) { return 32 >> vt_shift(P); }
inline int split_passes(int L, int P) { return (L + split_step(P) - 1) / split_step(P); }
inline int split_tables(int L, int P, int pass) { return std::min(split_step(P), L - split_step(P) * pass); }
inline int split_mode(int L, int P, int pass)
{
    return pass == 0 ? race::PART_OUT : pass + 1 == split_passes(L, P) ? race::PART_IN : race::PART_MID;
}
constexpr int kMaxPasses = 16;  // L <= 128 tables, up to 4 virtual tables each

template <typename T>
void split_forward(const Plan &p, int B, int H, int chunk, race_dtype_t dt, const void *Q,
                   const void *K, const void *V, const float *W, float tau, int causal, void *O,
                   float *den, char *ws, float *saved, const Tracer &tr)
{
    const int np = split_passes(p.L, p.P), step = split_step(p.P);
    Plan q[kMaxPasses];
    size_t fw = 0, sv = 0;
    for (int i = 0; i < np; ++i) {
        make_plan(B, H, p.N, p.d, split_tables(p.L, p.P, i), p.P, chunk, dt, &q[i]);
        fw += q[i].f_total;
    }
    float *pv = reinterpret_cast<float *>(ws + fw);
    float *pm = reinterpret_cast<float *>(reinterpret_cast<char *>(pv) +
                                          align256((size_t)p.rows * race::HD * sizeof(float)));
    size_t off = 0;
    for (int i = 0; i < np; ++i) {
        q[i].lens = p.lens;
        q[i].part_o = race::Part{pv, pm};
        q[i].part_mode = split_mode(p.L, p.P, i);
        float *sb = saved ? reinterpret_cast<float *>(reinterpret_cast<char *>(saved) + sv) : nullptr;
        dispatch_forward<T>(q[i], Q, K, V, W + step * i * p.P * p.d, tau, causal, O, den, ws + off, sb, tr);
        off += q[i].f_total;
        sv += q[i].s_total;
    }
}

template <typename T>
void split_backward(const Plan &p, int B, int H, int chunk, race_dtype_t dt, const void *Q,
                    const void *K, const void *V, const float *W, const void *O, const float *den,
                    const void *dO, float tau, int causal, void *dQ, void *dK, void *dV, char *ws,
                    const float *saved, const Tracer &tr, float *dW)
{
    const int np = split_passes(p.L, p.P), step = split_step(p.P);
    Plan q[kMaxPasses];
    size_t bw = 0;
    for (int i = 0; i < np; ++i) {
        make_plan(B, H, p.N, p.d, split_tables(p.L, p.P, i), p.P, chunk, dt, &q[i]);
        bw += dW ? q[i].dw_total : q[i].b_total;
    }
    const size_t pvb = align256((size_t)p.rows * race::HD * sizeof(float));
    char *pbase = ws + bw;
    const race::Part pq{reinterpret_cast<float *>(pbase), nullptr};
    const race::Part pk{reinterpret_cast<float *>(pbase + pvb), nullptr};
    const race::Part pd{reinterpret_cast<float *>(pbase + 2 * pvb), nullptr};
    size_t off = 0, sv = 0;
    for (int i = 0; i < np; ++i) {
        q[i].lens = p.lens;
        q[i].part_dq = pq;
        q[i].part_dk = pk;
        q[i].part_dv = pd;
        q[i].part_mode = split_mode(p.L, p.P, i);
        const float *sb =
            saved ? reinterpret_cast<const float *>(reinterpret_cast<const char *>(saved) + sv) : nullptr;
        dispatch_backward<T>(q[i], Q, K, V, W + step * i * p.P * p.d, O, den, dO, tau, causal, dQ, dK,
                             dV, ws + off, sb, tr, dW ? dW + step * i * p.P * p.d : nullptr);
        off += dW ? q[i].dw_total : q[i].b_total;
        sv += q[i].s_total;
    }
}

// Bulk add through the fused segment sum (16-bit rows, L <= 32): the keys'
// segment sums and their scan give the head total, which is added into the
// streaming state in its own layout and scale.
template <typename T, int NW, int D>
void fused_state_add(const Plan &p, const T *K, const T *V, const float *W, float tau, char *ws,
                     float *state, const Tracer &tr)
{
    constexpr int WS = 2 * NW;
    const race::Squash sq = fit_squash(tau, RACE_BF16);
    const dim3 nblk((unsigned)(p.BH * p.nseg));
    const race::ValSrc<T> vv{V, nullptr, nullptr};
    // workspace: the segment states, then the scan's group totals (no
    // hash-feature cache: nothing reads the keys' t again)
    float *st = reinterpret_cast<float *>(ws);
    const race::HCache none = hcache(p, nullptr, -1, -1);
    launch_sum<WS, false, 0, 0, D>(tr, "sum_kv", nblk, sq, K, vv, W, p, none, none, st);
    launch_scan(tr, "scan_kv", p, st, reinterpret_cast<float *>(ws + p.st_bytes), 0);
    const int total = WS * 4 * race::NT * 64 * 4;
    tr.begin("state_from_sums");
    hipLaunchKernelGGL(race::stream_from_sums_kernel, dim3((total + 255) / 256, (unsigned)p.BH),
                       dim3(256), 0, tr.s, st, p.nseg, WS, p.L, p.d, std::sqrt(std::ldexp(1.f, p.P)),
                       state);
    tr.end();
}

template <typename T>
void dispatch_fused_state_add(const Plan &p, const void *K, const void *V, const float *W,
                              float tau, char *ws, float *state, const Tracer &tr)
{
    auto k = static_cast<const T *>(K);
    auto v = static_cast<const T *>(V);
    if (p.d == 32) {
        switch (p.nw) {
        case 1: fused_state_add<T, 1, 32>(p, k, v, W, tau, ws, state, tr); break;
        case 2: fused_state_add<T, 2, 32>(p, k, v, W, tau, ws, state, tr); break;
        default: fused_state_add<T, 4, 32>(p, k, v, W, tau, ws, state, tr); break;
        }
    } else {
        switch (p.nw) {
        case 1: fused_state_add<T, 1, race::HD>(p, k, v, W, tau, ws, state, tr); break;
        case 2: fused_state_add<T, 2, race::HD>(p, k, v, W, tau, ws, state, tr); break;
        default: fused_state_add<T, 4, race::HD>(p, k, v, W, tau, ws, state, tr); break;
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming state (race_stream.h)

struct StreamPlan {
    int BH, L, P, d, F, fpt, nthr;
    int64_t elems;  // floats of one head's state
};

// token blocks per head for the parallel modes: about 1024 workgroups in all,
// at least 64 tokens per block
inline int64_t stream_blocks(const StreamPlan &sp, int64_t N)
{
    const int64_t want = (1024 + sp.BH - 1) / sp.BH;
    return std::max<int64_t>(1, std::min<int64_t>(want, (N + 63) / 64));
}

template <typename T, int MODE>
void launch_stream(const StreamPlan &sp, const void *Q, const void *K, const void *V,
                   const float *W, float tau, int64_t N, int64_t nblk, float *state, float *part,
                   void *O, float *den, hipStream_t s)
{
    const int64_t blk = (N + nblk - 1) / nblk;
    const dim3 grid((unsigned)nblk, (unsigned)sp.BH);
    // 32 or 64 features per wave; up to 8 waves (256 registers per lane), or
    // 16 for L > 32 (128 registers)
    // one token per head (decode): tiles of one token
    const bool one = MODE == race::SM_DECODE && N == 1;
    auto k = sp.fpt == 32     ? (one ? race::stream_kernel<T, MODE, 32, 512, 1> : race::stream_kernel<T, MODE, 32, 512>)
             : sp.nthr <= 512 ? (one ? race::stream_kernel<T, MODE, 64, 512, 1> : race::stream_kernel<T, MODE, 64, 512>)
                              : (one ? race::stream_kernel<T, MODE, 64, 1024, 1> : race::stream_kernel<T, MODE, 64, 1024>);
    hipLaunchKernelGGL(k, grid, dim3(sp.nthr), 0, s, static_cast<const T *>(Q),
                       static_cast<const T *>(K), static_cast<const T *>(V), W, sp.L, sp.P, sp.d, 1.f / tau,
                       N, blk, state, part, static_cast<T *>(O), den);
}

// Hard hashing (race_hard.h, launched from race_inst_hard.hip).  Workspace of
// the bucket ids: the three bf16 terms of W, [3][LPpad][Dpad].
inline int hard_lppad(int L, int P) { return (L * P + 31) / 32 * 32; }
inline int hard_dpad(int d) { return (d + 31) / 32 * 32; }
inline size_t hard_ids_ws(int L, int P, int d)
{
    return align256((size_t)3 * hard_lppad(L, P) * hard_dpad(d) * sizeof(bf16));
}
void hard_ids_launch(const void *X, int64_t rows, int d, race_dtype_t dt, const float *W, int L,
                     int P, uint8_t *ids, char *ws, hipStream_t s, int vshift = 0);

// Hard forward on the bucket ids (16-bit rows, L <= 32, P <= 4, d = 32 or 64).
// Workspace: ids of Q and K (padded), the W terms, value states, count
// states and the value scan's group totals.
struct HardPlan {
    size_t ids_bytes, wsplit, vstate, cstate, scan, total;
    size_t o_idq, o_idk, o_w, o_v, o_c, o_scan;
    int hw;            // waves per workgroup (4 tables each)
    int64_t velems;    // floats of one value state block
};
// p: the plan of the tables the sum and walk kernels see (for P = 5, 6 the
// L 2^(P-4) virtual tables of 4 planes); Lr, Pr: the real tables, whose W
// the id kernel splits
inline HardPlan hard_plan(const Plan &p, int Lr, int Pr)
{
    HardPlan h;
    h.hw = 2 * p.nw;
    h.velems = (int64_t)h.hw * 4 * race::HNT * 64 * 4;
    h.ids_bytes = align256((size_t)p.rows * p.L + 4);
    h.wsplit = hard_ids_ws(Lr, Pr, p.d);
    h.vstate = align256((size_t)p.BH * (p.nseg + 1) * h.velems * sizeof(float));
    h.cstate = align256((size_t)p.BH * (p.nseg + 1) * 32 * 16 * sizeof(int));
    h.scan = align256((size_t)p.BH * p.scan_groups * h.velems * sizeof(float));
    h.o_idq = 0;
    h.o_idk = h.o_idq + h.ids_bytes;
    h.o_w = h.o_idk + h.ids_bytes;
    h.o_v = h.o_w + h.wsplit;
    h.o_c = h.o_v + h.vstate;
    h.o_scan = h.o_c + h.cstate;
    h.total = h.o_scan + h.scan;
    return h;
}
inline bool hard_fused(const Plan &p, race_dtype_t dt)
{
    // (int32 counts: every count is at most N L)
    return (dt == RACE_BF16 || dt == RACE_F16) && p.L <= 32 && p.P <= 4 && (p.d == 64 || p.d == 32) &&
           (int64_t)p.N * p.L < ((int64_t)1 << 31);
}
void hard_forward_launch(const Plan &p, int Lr, int Pr, race_dtype_t dt, const void *Q, const void *K,
                         const void *V, const float *W, int causal, void *O, float *den, int *count,
                         char *ws, hipStream_t s);

// Launch sequences instantiated in race_inst_*.hip (one file per row type
// and direction), not in the files that call them.
#define RACE_FWD_INST(EXT, T)                                                                     \
    EXT template void dispatch_forward<T>(const Plan &, const void *, const void *, const void *, \
                                          const float *, float, int, void *, float *, char *,     \
                                          float *, const Tracer &)
#define RACE_SPLIT_FWD_INST(EXT, T)                                                               \
    EXT template void split_forward<T>(const Plan &, int, int, int, race_dtype_t, const void *,   \
                                       const void *, const void *, const float *, float, int,     \
                                       void *, float *, char *, float *, const Tracer &)
#define RACE_BWD_INST(EXT, T)                                                                     \
    EXT template void dispatch_backward<T>(const Plan &, const void *, const void *, const void *,\
                                           const float *, const void *, const float *,            \
                                           const void *, float, int, void *, void *, void *,      \
                                           char *, const float *, const Tracer &, float *)
#define RACE_SPLIT_BWD_INST(EXT, T)                                                               \
    EXT template void split_backward<T>(const Plan &, int, int, int, race_dtype_t, const void *,  \
                                        const void *, const void *, const float *, const void *,  \
                                        const float *, const void *, float, int, void *, void *,  \
                                        void *, char *, const float *, const Tracer &, float *)
#define RACE_STATE_ADD_INST(EXT, T)                                                               \
    EXT template void dispatch_fused_state_add<T>(const Plan &, const void *, const void *,       \
                                                  const float *, float, char *, float *,         \
                                                  const Tracer &)
#define RACE_STREAM_INST(EXT, T, MODE)                                                            \
    EXT template void launch_stream<T, MODE>(const StreamPlan &, const void *, const void *,      \
                                             const void *, const float *, float, int64_t,         \
                                             int64_t, float *, float *, void *, float *,          \
                                             hipStream_t)

RACE_FWD_INST(extern, bf16);
RACE_FWD_INST(extern, _Float16);
RACE_FWD_INST(extern, float);
RACE_SPLIT_FWD_INST(extern, bf16);
RACE_SPLIT_FWD_INST(extern, _Float16);
RACE_SPLIT_FWD_INST(extern, float);
RACE_BWD_INST(extern, bf16);
RACE_BWD_INST(extern, _Float16);
RACE_BWD_INST(extern, float);
RACE_SPLIT_BWD_INST(extern, bf16);
RACE_SPLIT_BWD_INST(extern, _Float16);
RACE_SPLIT_BWD_INST(extern, float);
RACE_STATE_ADD_INST(extern, bf16);
RACE_STATE_ADD_INST(extern, _Float16);
RACE_STREAM_INST(extern, bf16, race::SM_ADD);
RACE_STREAM_INST(extern, bf16, race::SM_DECODE);
RACE_STREAM_INST(extern, bf16, race::SM_READOUT);
RACE_STREAM_INST(extern, _Float16, race::SM_ADD);
RACE_STREAM_INST(extern, _Float16, race::SM_DECODE);
RACE_STREAM_INST(extern, _Float16, race::SM_READOUT);
RACE_STREAM_INST(extern, float, race::SM_ADD);
RACE_STREAM_INST(extern, float, race::SM_DECODE);
RACE_STREAM_INST(extern, float, race::SM_READOUT);

}  // namespace race_host
