// race_attn.hip -- C ABI of the RACE attention library (declared in include/race_attn.h).
//
// Host side: argument validation, workspace planning and kernel sequencing
// on the caller's stream.  No allocation, no synchronisation, no global
// mutable state.
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

namespace {

using race::bf16;

constexpr int64_t kMaxN = (int64_t)1 << 40;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

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
};

race_status_t make_plan(int B, int H, int64_t N, int d, int L, int P, int chunk,
                        race_dtype_t dt, Plan *p)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || L < 1 || P < 1) return RACE_ERR_SHAPE;
    if (N > kMaxN || (int64_t)B * H > 65535) return RACE_ERR_SHAPE;
    if (dt != RACE_F32 && dt != RACE_BF16 && dt != RACE_F16) return RACE_ERR_UNSUPPORTED;
    if (P > race::NP) return RACE_ERR_UNSUPPORTED;
    if (L > 64 || (dt == RACE_F32 && L > 32)) return RACE_ERR_UNSUPPORTED;
    // 16-bit rows with L > 32: two fused passes, d = 64 only
    if (dt != RACE_F32 && L > 32 && d != race::HD) return RACE_ERR_UNSUPPORTED;
    // d = 64 and P = 4, or d = 32 and P < 4 on the fused path (16-bit rows, L <= 32)
    const bool fusable = dt != RACE_F32 && L <= 32;
    if (d != race::HD && !(d == 32 && fusable)) return RACE_ERR_UNSUPPORTED;
    if (P != race::NP && dt == RACE_F32) return RACE_ERR_UNSUPPORTED;
    if (chunk < 0 || chunk % race::CH != 0) return RACE_ERR_CHUNK;
    p->BH = (int64_t)B * H;
    p->d = d;
    p->P = P;
    p->lens = race::Lens{nullptr, H};
    p->split = false;
    p->part_mode = race::PART_NONE;
    p->part_o = p->part_dq = p->part_dk = p->part_dv = race::Part{nullptr, nullptr};
    p->N = N;
    p->rows = p->BH * N;
    p->L = L;
    p->nw = L <= 8 ? 1 : L <= 16 ? 2 : L <= 32 ? 4 : 8;
    p->F = p->nw * race::FPW;
    p->LP = L * race::NP;
    const int64_t n16 = (N + 15) / 16 * 16;
    int64_t seg = chunk;
    if (seg == 0) {
        // one workgroup per compute unit (MI355X: 256 CUs; every segment
        // kernel keeps one workgroup per CU resident), segments >= 64 tokens
        const int64_t want = (p->rows + 255) / 256;
        seg = (want + 31) / 32 * 32;
        if (seg < 64) seg = 64;
    }
    if (seg > n16) seg = n16;
    seg = (seg + 31) / 32 * 32;  // whole 32-token sub-chunks per segment
    p->seg = seg;
    p->nseg = (N + seg - 1) / seg;
    if (p->BH * p->nseg > 0x7fffffffLL) return RACE_ERR_SHAPE;
    p->fused = (dt == RACE_BF16 || dt == RACE_F16) && L <= 32;
    p->st_bytes = align256((size_t)p->BH * (p->nseg + 1) * p->F * race::NCOL * sizeof(float));
    // the fused kernels keep hash features on chip: no per-row buffers
    p->t_bytes = p->fused ? 0 : align256((size_t)p->rows * L * race::NP * sizeof(float));
    p->tb_bytes = p->fused ? 0 : align256((size_t)p->rows * L * 2 * race::NP * sizeof(float));
    const int lp32 = (p->LP + 31) / 32 * 32;
    p->wt_bytes = p->fused ? 0 : align256((size_t)race::HD * lp32 * (2 * sizeof(bf16) + sizeof(float)));
    // groups of at least 16 segments, at most 64 groups
    const int64_t groups = p->nseg / 16;
    p->scan_groups = (int)(groups < 1 ? 1 : groups > 64 ? 64 : groups);
    p->scan_bytes = align256((size_t)p->BH * p->scan_groups * p->F * race::NCOL * sizeof(float));
    p->hc_tiles = (N + 31) / 32 * 2;
    // per 16-token tile: 2 nw waves x 64 lanes x 4 fp16 values
    p->hc_bytes = p->fused ? align256((size_t)p->BH * p->hc_tiles * (2 * p->nw) * 64 * 4 * 2) : 0;
    p->f_tq = 0;
    p->f_tk = p->f_tq + p->t_bytes;
    p->f_st = p->f_tk + p->t_bytes;
    p->f_hc = p->f_st + p->st_bytes;
    p->f_scan = p->f_hc + p->hc_bytes;
    p->f_total = p->f_scan + p->scan_bytes;
    p->s_hc = p->st_bytes;
    p->s_total = p->fused ? p->s_hc + 4 * p->hc_bytes : 0;
    p->b_tq = 0;
    p->b_tk = p->b_tq + p->tb_bytes;
    p->b_s = p->b_tk + p->tb_bytes;
    p->b_gt = p->b_s + p->st_bytes;
    // the bf16 kernels read the gradient state transposed from its FxC copy
    p->b_g = p->b_gt + (p->fused ? 0 : p->st_bytes);
    p->b_wt = p->b_g + p->st_bytes;
    p->b_hc = p->b_wt + p->wt_bytes;
    p->b_scan = p->b_hc + 4 * p->hc_bytes;
    p->b_total = p->b_scan + p->scan_bytes;
    // backward with dW: one [hyperplane rows][d] fp32 block per workgroup of dQ and of dK
    p->b_dw = p->b_total;
    p->dw_total = p->fused ? p->b_dw + align256((size_t)2 * p->BH * p->nseg * (2 * p->nw * 16) *
                                                race::HD * sizeof(float))
                           : 0;
    if (dt != RACE_F32 && L > 32) {
        // two fused passes (the first 32 tables, then the other L - 32): both
        // passes' buffers, then the fp32 partial sums
        Plan a, b;
        race_status_t st = make_plan(B, H, N, d, 32, P, chunk, dt, &a);
        if (st != RACE_OK) return st;
        if ((st = make_plan(B, H, N, d, L - 32, P, chunk, dt, &b)) != RACE_OK) return st;
        const size_t pv = align256((size_t)p->rows * race::HD * sizeof(float));
        const size_t pm = align256((size_t)p->rows * sizeof(float));
        p->split = true;
        p->f_total = a.f_total + b.f_total + pv + pm;
        p->b_total = a.b_total + b.b_total + 3 * pv;
        p->dw_total = a.dw_total + b.dw_total + 3 * pv;
        p->s_total = a.s_total + b.s_total;
    }
    return RACE_OK;
}

// h(e) = tanh(((1 - e)/(1 + e)) / tau) on e in [0, 1], the outer tanh of
// t = tanh(tanh(v) / tau) written through e = exp(-2|v|); g(e) = dt/dv there,
// ((1 - h^2) / tau) (1 - z^2) with z = (1 - e)/(1 + e) = tanh(|v|).
double squash_ref(double e, double tau) { return std::tanh(((1.0 - e) / (1.0 + e)) / tau); }
double squash_deriv_ref(double e, double tau)
{
    const double z = (1.0 - e) / (1.0 + e), h = std::tanh(z / tau);
    return (1.0 - h * h) / tau * (1.0 - z * z);
}

// x rounded to the nearest fp16 value (ties to even; fp16 normals have 11
// significant bits, subnormals a quantum of 2^-24)
double round_f16(double x)
{
    if (x == 0.0 || !std::isfinite(x)) return x;
    int ex;
    std::frexp(x, &ex);
    const double q = std::ldexp(1.0, std::max(ex - 11, -24));
    return std::nearbyint(x / q) * q;
}

// IEEE binary16 bits of a value that is exactly representable in fp16
uint32_t f16_bits(double v)
{
    uint32_t sign = std::signbit(v) ? 0x8000u : 0u;
    v = std::fabs(v);
    if (v == 0.0) return sign;
    int ex;
    const double m = std::frexp(v, &ex);  // v = m 2^ex, m in [0.5, 1)
    const int be = ex - 1 + 15;           // biased exponent of 1.f x 2^(ex - 1)
    if (be >= 1) return sign | ((uint32_t)be << 10) | (uint32_t)std::lround((2.0 * m - 1.0) * 1024.0);
    return sign | (uint32_t)std::lround(v * 16777216.0);  // subnormal: v / 2^-24
}

// Chebyshev interpolation of f(., tau) at the Chebyshev nodes of y = 2e - 1,
// in fp64, converted to monomial coefficients in y.
void cheb_mono(double (*f)(double, double), double tau, int deg, double *mono)
{
    const int n = deg + 1;
    double fk[race::MAXDEG + 1], a[race::MAXDEG + 1];
    for (int k = 0; k < n; ++k) fk[k] = f(0.5 * (std::cos(M_PI * (k + 0.5) / n) + 1.0), tau);
    for (int j = 0; j < n; ++j) {
        double sum = 0.0;
        for (int k = 0; k < n; ++k) sum += fk[k] * std::cos(M_PI * j * (k + 0.5) / n);
        a[j] = (j == 0 ? 1.0 : 2.0) * sum / n;
    }
    // T_0 = 1, T_1 = y, T_{j+1} = 2y T_j - T_{j-1}
    double tm1[race::MAXDEG + 2] = {0}, t0[race::MAXDEG + 2] = {0}, t1[race::MAXDEG + 2] = {0};
    for (int i = 0; i <= deg; ++i) mono[i] = 0.0;
    t0[0] = 1.0;
    for (int j = 0; j < n; ++j) {
        for (int i = 0; i <= j; ++i) mono[i] += a[j] * t0[i];
        for (int i = 0; i <= j + 1; ++i) {
            const double up = i > 0 ? t0[i - 1] : 0.0;
            t1[i] = j == 0 ? up : 2.0 * up - (i <= j - 1 ? tm1[i] : 0.0);
        }
        for (int i = 0; i <= j + 1; ++i) {
            tm1[i] = t0[i];
            t0[i] = t1[i];
        }
    }
}

// The bf16 kernels' squash: |t| and dt/dv as degree-DEG16 polynomials in
// y = 2e - 1 with fp16 coefficients, evaluated in fp16 (Horner with fused
// multiply-adds, y rounded from fp32).  The fit is kept when that evaluation,
// emulated here on a dense grid, is within 1.5e-3 of t and within
// 1.5e-3 max(1, 1/tau) of dt/dv (fp16 keeps t to 2.4e-4 and the bf16 Walsh
// features to 2e-3 relative anyway); otherwise deg = -1 and the kernels
// evaluate both functions directly in fp32.  The fp32 kernels always
// evaluate directly.
race::Squash fit_squash(float tau, race_dtype_t dt)
{
    race::Squash sq;
    std::memset(&sq, 0, sizeof sq);
    sq.inv_tau = 1.0f / tau;
    sq.deg = -1;
    if (dt != RACE_BF16) return sq;
    constexpr int D = race::DEG16;
    double mt[race::MAXDEG + 1], mc[race::MAXDEG + 1];
    cheb_mono(squash_ref, tau, D, mt);
    cheb_mono(squash_deriv_ref, tau, D, mc);
    for (int i = 0; i <= D; ++i) {
        mt[i] = round_f16(mt[i]);
        mc[i] = round_f16(mc[i]);
    }
    constexpr int NG = 4001;
    double et = 0.0, ec = 0.0;
    for (int k = 0; k < NG; ++k) {
        const double e = (double)k / (NG - 1);
        const double y = round_f16((double)std::fma(2.0f, (float)e, -1.0f));
        double h = mt[D], c = mc[D];
        for (int i = D - 1; i >= 0; --i) {
            h = round_f16(h * y + mt[i]);
            c = round_f16(c * y + mc[i]);
        }
        et = std::fmax(et, std::fabs(std::fabs(h) - squash_ref(e, tau)));
        ec = std::fmax(ec, std::fabs(c - squash_deriv_ref(e, tau)));
    }
    if (et <= 1.5e-3 && ec <= 1.5e-3 * std::fmax(1.0, 1.0 / tau)) {
        for (int i = 0; i <= D; ++i) {
            sq.t16[i] = f16_bits(mt[i]) * 0x10001u;
            sq.c16[i] = f16_bits(mc[i]) * 0x10001u;
        }
        sq.deg = D;
    }
    return sq;
}

// Hard hashing (the tau -> 0 limit, t = sign(u), +1 at 0) in the polynomial
// form the bf16 kernels evaluate: |t| = 1 (the constant polynomial) with the
// sign of u, and dt/du' = 0.
race::Squash hard_squash()
{
    race::Squash sq;
    std::memset(&sq, 0, sizeof sq);
    sq.inv_tau = 0.f;
    sq.deg = race::DEG16;
    sq.t16[0] = f16_bits(1.0) * 0x10001u;
    return sq;
}

// value of an fp16 pair's low half
double f16_value(uint32_t bits)
{
    const uint32_t b = bits & 0xffffu, e = (b >> 10) & 31u, m = b & 1023u;
    const double v = e == 0 ? std::ldexp((double)m, -24) : std::ldexp(1.0 + m / 1024.0, (int)e - 15);
    return (b & 0x8000u) ? -v : v;
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

// exclusive prefix (reverse = 0) or suffix (reverse = 1) of the segment
// states of every head, plus the head totals
void launch_scan(const Tracer &tr, const char *name, const Plan &p, float *st, float *tmp,
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
race::HCache hcache(const Plan &p, char *base, int it, int ic)
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
        if (SRC == 1 || sq.deg >= 0)
            LAUNCH(tr, name, (race::sum_kernel<NW, DVAL, SRC, WR, true, T, D>), grid, dim3(NW * 64), X, vs,
                   W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, cin, cout, st, p.lens);
        else
            LAUNCH(tr, name, (race::sum_kernel<NW, DVAL, SRC, WR, false, T, D>), grid, dim3(NW * 64), X, vs,
                   W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, cin, cout, st, p.lens);
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
        auto go = [&](auto part_c) {
            constexpr int PT = decltype(part_c)::value;
            if (RSRC == 1 || sq.deg >= 0)
                LAUNCH(tr, name, (race::walk_kernel<NW, CAUSAL, BWD, RSRC, RWR, true, T, D, PT>), grid,
                       dim3(NW * 64), R, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, st, rc, wc, out,
                       den, p.lens, pt);
            else
                LAUNCH(tr, name, (race::walk_kernel<NW, CAUSAL, BWD, RSRC, RWR, false, T, D, PT>), grid,
                       dim3(NW * 64), R, vs, W, p.L, p.P, sq, p.N, (int)p.seg, p.nseg, st, rc, wc, out,
                       den, p.lens, pt);
        };
        // the first of two passes always has 32 tables (NW = 8); split runs have d = 64
        if (p.part_mode == race::PART_NONE) {
            go(std::integral_constant<int, race::PART_NONE>{});
        } else if constexpr (D == race::HD) {
            if (p.part_mode == race::PART_IN)
                go(std::integral_constant<int, race::PART_IN>{});
            else if constexpr (NW == 8)
                go(std::integral_constant<int, race::PART_OUT>{});
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
        auto go = [&](auto part_c) {
            constexpr int PT = decltype(part_c)::value;
            if (dwp)
                LAUNCH(tr, name, (race::grad_kernel<NW, CAUSAL, REVERSE, true, T, D, PT>), grid,
                       dim3(NW * 64), Xr, vr, vw, W, p.L, p.P, p.N, (int)p.seg, p.nseg, st, rc, wc, dX,
                       dwp, p.lens, pt);
            else
                LAUNCH(tr, name, (race::grad_kernel<NW, CAUSAL, REVERSE, false, T, D, PT>), grid,
                       dim3(NW * 64), Xr, vr, vw, W, p.L, p.P, p.N, (int)p.seg, p.nseg, st, rc, wc, dX,
                       nullptr, p.lens, pt);
        };
        if (p.part_mode == race::PART_NONE) {
            go(std::integral_constant<int, race::PART_NONE>{});
        } else if constexpr (D == race::HD) {
            if (p.part_mode == race::PART_IN)
                go(std::integral_constant<int, race::PART_IN>{});
            else if constexpr (NW == 8)
                go(std::integral_constant<int, race::PART_OUT>{});
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
    LAUNCH(tr, "hash_q", (race::hash_kernel<T, false>), hg, b256, Q, p.rows, W, p.L, inv_tau, tq);
    LAUNCH(tr, "hash_k", (race::hash_kernel<T, false>), hg, b256, K, p.rows, W, p.L, inv_tau, tk);
    const race::ValSrc<T> vs{V, nullptr, nullptr};
    const dim3 nblk((unsigned)(p.BH * p.nseg));
    LAUNCH(tr, "seg_sum_kv", (race::seg_sum_kernel<T, NW, false, false>), nblk, bw, tk, race::NP,
           vs, p.N, p.L, (int)p.seg, p.nseg, st, p.lens);
    launch_scan(tr, "scan_kv", p, st, scan_tmp, 0);
    if (causal)
        LAUNCH(tr, "readout_o", (race::readout_kernel<T, NW, true, false>), nblk, bw, tq, tk,
               race::NP, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den, p.lens);
    else
        LAUNCH(tr, "readout_o", (race::readout_kernel<T, NW, false, false>), nblk, bw, tq, tk,
               race::NP, vs, p.N, p.L, (int)p.seg, p.nseg, st, O, den, p.lens);
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
                   dim3(256), dwp, 2 * p.BH * p.nseg, WD * 16, p.LP, p.P, D, dW);
        launch_walk<WW, CAUSAL != 0, true, 1, 0, D>(tr, "dv", nblk, sq, K, vd, W, p, sG, hk, hq, dV,
                                                 nullptr);
        return;
    }
    if constexpr (!std::is_same<T, _Float16>::value && D == race::HD) {  // fp16 rows, d = 32: fused path only
    LAUNCH(tr, "prep_wt", race::prep_wt_kernel, dim3((race::HD * lp32 + 255) / 256), b256, W,
           p.LP, lp32, wt);
    LAUNCH(tr, "hash_q_chain", (race::hash_kernel<T, true>), hg, b256, Q, p.rows, W, p.L,
           inv_tau, tq);
    LAUNCH(tr, "hash_k_chain", (race::hash_kernel<T, true>), hg, b256, K, p.rows, W, p.L,
           inv_tau, tk);
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
           vv, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sS, dQ, p.lens);
    // dK: readers K (values [v|1]), writers Q (values D), reverse order
    LAUNCH(tr, "dpsi_k", (race::dpsi_kernel<T, NW, CAUSAL, true, false>), nblk, bw, K, tk, tq, vv,
           vd, wt, lp32, p.N, p.L, (int)p.seg, p.nseg, sGt, dK, p.lens);
    // dV: keys read the FxC gradient state, reverse order
    LAUNCH(tr, "readout_dv", (race::readout_kernel<T, NW, CAUSAL != 0, true>), nblk, bw, tk, tq,
           ts, vd, p.N, p.L, (int)p.seg, p.nseg, sG, dV, nullptr, p.lens);
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
    case 4: launch_forward<T, 4, D>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr); break;
    default:
        if constexpr (std::is_same<T, bf16>::value)
            launch_forward<T, 8, D>(p, q, k, v, W, tau, causal, o, den, ws, saved, tr);
        break;
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
    case 4: launch_backward<T, 4, D>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW); break;
    default:
        if constexpr (std::is_same<T, bf16>::value)
            launch_backward<T, 8, D>(p, q, k, v, W, o, den, go, tau, causal, dq, dk, dv, ws, saved, tr, dW);
        break;
    }
}

// L > 32 with 16-bit rows: the first 32 tables, then the other L - 32, as two
// fused passes over the same rows.  The first stores its sums in fp32 (the
// readout's n and m; dx_hat of Q and of K; dV) in partial arrays after both
// passes' buffers, the second adds them before its last step.  Each pass has
// its own buffers and saved state; dW rows are those of its tables.
template <typename T>
void split_forward(const Plan &p, int B, int H, int chunk, race_dtype_t dt, const void *Q,
                   const void *K, const void *V, const float *W, float tau, int causal, void *O,
                   float *den, char *ws, float *saved, const Tracer &tr)
{
    Plan a, b;
    make_plan(B, H, p.N, p.d, 32, p.P, chunk, dt, &a);
    make_plan(B, H, p.N, p.d, p.L - 32, p.P, chunk, dt, &b);
    a.lens = b.lens = p.lens;
    float *pv = reinterpret_cast<float *>(ws + a.f_total + b.f_total);
    float *pm = reinterpret_cast<float *>(reinterpret_cast<char *>(pv) +
                                          align256((size_t)p.rows * race::HD * sizeof(float)));
    a.part_o = b.part_o = race::Part{pv, pm};
    a.part_mode = race::PART_OUT;
    b.part_mode = race::PART_IN;
    float *sb = saved ? reinterpret_cast<float *>(reinterpret_cast<char *>(saved) + a.s_total) : nullptr;
    dispatch_forward<T>(a, Q, K, V, W, tau, causal, O, den, ws, saved, tr);
    dispatch_forward<T>(b, Q, K, V, W + 32 * p.P * p.d, tau, causal, O, den, ws + a.f_total, sb, tr);
}

template <typename T>
void split_backward(const Plan &p, int B, int H, int chunk, race_dtype_t dt, const void *Q,
                    const void *K, const void *V, const float *W, const void *O, const float *den,
                    const void *dO, float tau, int causal, void *dQ, void *dK, void *dV, char *ws,
                    const float *saved, const Tracer &tr, float *dW)
{
    Plan a, b;
    make_plan(B, H, p.N, p.d, 32, p.P, chunk, dt, &a);
    make_plan(B, H, p.N, p.d, p.L - 32, p.P, chunk, dt, &b);
    a.lens = b.lens = p.lens;
    const size_t ta = dW ? a.dw_total : a.b_total, tb = dW ? b.dw_total : b.b_total;
    const size_t pvb = align256((size_t)p.rows * race::HD * sizeof(float));
    char *pbase = ws + ta + tb;
    const race::Part pq{reinterpret_cast<float *>(pbase), nullptr};
    const race::Part pk{reinterpret_cast<float *>(pbase + pvb), nullptr};
    const race::Part pd{reinterpret_cast<float *>(pbase + 2 * pvb), nullptr};
    a.part_dq = b.part_dq = pq;
    a.part_dk = b.part_dk = pk;
    a.part_dv = b.part_dv = pd;
    a.part_mode = race::PART_OUT;
    b.part_mode = race::PART_IN;
    const float *sb =
        saved ? reinterpret_cast<const float *>(reinterpret_cast<const char *>(saved) + a.s_total) : nullptr;
    dispatch_backward<T>(a, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, saved, tr, dW);
    dispatch_backward<T>(b, Q, K, V, W + 32 * p.P * p.d, O, den, dO, tau, causal, dQ, dK, dV, ws + ta,
                         sb, tr, dW ? dW + 32 * p.P * p.d : nullptr);
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
    float *st = reinterpret_cast<float *>(ws + p.f_st);
    const race::HCache hk = hcache(p, ws + p.f_hc, 0, -1), none = hcache(p, nullptr, -1, -1);
    launch_sum<WS, false, 0, 1, D>(tr, "sum_kv", nblk, sq, K, vv, W, p, none, hk, st);
    launch_scan(tr, "scan_kv", p, st, reinterpret_cast<float *>(ws + p.f_scan), 0);
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

race_status_t check_trace(race_trace_t *trace)
{
    if (!trace) return RACE_OK;
    if (trace->capacity < 0 || trace->capacity > RACE_TRACE_MAX) return RACE_ERR_SHAPE;
    for (int i = 0; i < trace->capacity; ++i)
        if (!trace->start[i] || !trace->stop[i]) return RACE_ERR_NULL;
    trace->count = 0;
    return RACE_OK;
}

// ---------------------------------------------------------------------------
// Streaming state (race_stream.h)

struct StreamPlan {
    int BH, L, P, d, F, fpt, nthr;
    int64_t elems;  // floats of one head's state
};

race_status_t stream_plan(int B, int H, int64_t N, int d, int L, int P, race_dtype_t dt,
                          StreamPlan *sp)
{
    if (B < 1 || H < 1 || N < 0 || d < 1 || L < 1 || P < 1) return RACE_ERR_SHAPE;
    if (d > race::HD || P > race::NP || L > 64) return RACE_ERR_UNSUPPORTED;
    if (dt != RACE_F32 && dt != RACE_BF16 && dt != RACE_F16) return RACE_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH > 65535) return RACE_ERR_UNSUPPORTED;  // heads go to the second grid dimension
    if (N > ((int64_t)1 << 62) / (BH * d)) return RACE_ERR_SHAPE;
    sp->BH = (int)BH;
    sp->L = L;
    sp->P = P;
    sp->d = d;
    sp->F = L * race::NR;
    sp->fpt = sp->F > 256 ? 64 : 32;
    sp->nthr = 64 * ((sp->F + sp->fpt - 1) / sp->fpt);  // one wave per feature group
    sp->elems = (int64_t)sp->F * (d + 1);
    return RACE_OK;
}

// token blocks per head for the parallel modes: about 1024 workgroups in all,
// at least 64 tokens per block
int64_t stream_blocks(const StreamPlan &sp, int64_t N)
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
    if (for_backward == 2 && !p.fused && !p.split) return RACE_ERR_UNSUPPORTED;
    *bytes = for_backward == 2 ? p.dw_total : for_backward ? p.b_total : p.f_total;
    return RACE_OK;
}

race_status_t race_attn_saved_bytes(int B, int H, int64_t N, int d, int L, int P, int causal,
                                    int chunk, race_dtype_t dt, size_t *bytes)
{
    (void)causal;
    if (!bytes) return RACE_ERR_NULL;
    Plan p;
    const race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    *bytes = p.s_total;
    return RACE_OK;
}

// forward / backward of every variant; lens: per-batch valid rows (device
// int32 [B]) or NULL; dW: the projection gradient (fused path) or NULL
static race_status_t forward_impl(const void *Q, const void *K, const void *V, const float *W,
                                  int L, int P, float tau, int causal, int B, int H, int64_t N,
                                  int d, race_dtype_t dt, int chunk, void *O, float *den,
                                  void *workspace, size_t ws_bytes, void *stream, void *saved,
                                  race_trace_t *trace, const int *lens)
{
    if (!Q || !K || !V || !W || !O || !den || !workspace) return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
    if ((st = check_trace(trace)) != RACE_OK) return st;
    if (saved && ((uintptr_t)saved & 255) != 0) return RACE_ERR_WORKSPACE;
    p.lens.len = lens;
    float *sv = p.fused || p.split ? static_cast<float *>(saved) : nullptr;
    const Tracer tr{trace, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (p.split && dt == RACE_BF16)
        split_forward<bf16>(p, B, H, chunk, dt, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else if (p.split)
        split_forward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else if (dt == RACE_BF16)
        dispatch_forward<bf16>(p, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else if (dt == RACE_F16)
        dispatch_forward<_Float16>(p, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else
        dispatch_forward<float>(p, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

static race_status_t backward_impl(const void *Q, const void *K, const void *V, const float *W,
                                   const void *O, const float *den, const void *dO, int L, int P,
                                   float tau, int causal, int B, int H, int64_t N, int d,
                                   race_dtype_t dt, int chunk, void *dQ, void *dK, void *dV,
                                   float *dW, void *workspace, size_t ws_bytes, void *stream,
                                   const void *saved, race_trace_t *trace, const int *lens)
{
    if (!Q || !K || !V || !W || !O || !den || !dO || !dQ || !dK || !dV || !workspace)
        return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if (dW && !p.fused && !p.split) return RACE_ERR_UNSUPPORTED;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, dW ? p.dw_total : p.b_total, workspace, ws_bytes)) != RACE_OK) return st;
    if ((st = check_trace(trace)) != RACE_OK) return st;
    if (saved && ((uintptr_t)saved & 255) != 0) return RACE_ERR_WORKSPACE;
    p.lens.len = lens;
    const float *sv = p.fused || p.split ? static_cast<const float *>(saved) : nullptr;
    const Tracer tr{trace, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (p.split && dt == RACE_BF16)
        split_backward<bf16>(p, B, H, chunk, dt, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr, dW);
    else if (p.split)
        split_backward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr,
                                 dW);
    else if (dt == RACE_BF16)
        dispatch_backward<bf16>(p, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr, dW);
    else if (dt == RACE_F16)
        dispatch_backward<_Float16>(p, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr, dW);
    else
        dispatch_backward<float>(p, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr, dW);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_forward_ex(const void *Q, const void *K, const void *V, const float *W,
                                   int L, int P, float tau, int causal, int B, int H, int64_t N,
                                   int d, race_dtype_t dt, int chunk, void *O, float *den,
                                   void *workspace, size_t ws_bytes, void *stream, void *saved,
                                   race_trace_t *trace)
{
    return forward_impl(Q, K, V, W, L, P, tau, causal, B, H, N, d, dt, chunk, O, den, workspace,
                        ws_bytes, stream, saved, trace, nullptr);
}

race_status_t race_attn_forward_padded(const void *Q, const void *K, const void *V,
                                       const float *W, int L, int P, float tau, int causal, int B,
                                       int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                       const int *seqlens, void *O, float *den, void *workspace,
                                       size_t ws_bytes, void *stream)
{
    if (!seqlens) return RACE_ERR_NULL;
    return forward_impl(Q, K, V, W, L, P, tau, causal, B, H, N, d, dt, chunk, O, den, workspace,
                        ws_bytes, stream, nullptr, nullptr, seqlens);
}

race_status_t race_attn_forward_hard(const void *Q, const void *K, const void *V,
                                     const float *W, int L, int P, int causal, int B, int H,
                                     int64_t N, int d, race_dtype_t dt, int chunk, void *O,
                                     float *den, void *workspace, size_t ws_bytes, void *stream)
{
    if (!Q || !K || !V || !W || !O || !den || !workspace) return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
    const Tracer tr{nullptr, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (p.split && dt == RACE_BF16)
        split_forward<bf16>(p, B, H, chunk, dt, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
    else if (p.split)
        split_forward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
    else if (dt == RACE_BF16)
        dispatch_forward<bf16>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
    else if (dt == RACE_F16)
        dispatch_forward<_Float16>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
    else
        dispatch_forward<float>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_forward(const void *Q, const void *K, const void *V, const float *W,
                                int L, int P, float tau, int causal, int B, int H, int64_t N,
                                int d, race_dtype_t dt, int chunk, void *O, float *den,
                                void *workspace, size_t ws_bytes, void *stream)
{
    return race_attn_forward_ex(Q, K, V, W, L, P, tau, causal, B, H, N, d, dt, chunk, O, den,
                                workspace, ws_bytes, stream, nullptr, nullptr);
}

race_status_t race_attn_backward_ex(const void *Q, const void *K, const void *V,
                                    const float *W, const void *O, const float *den,
                                    const void *dO, int L, int P, float tau, int causal, int B,
                                    int H, int64_t N, int d, race_dtype_t dt, int chunk, void *dQ,
                                    void *dK, void *dV, void *workspace, size_t ws_bytes,
                                    void *stream, const void *saved, race_trace_t *trace)
{
    return backward_impl(Q, K, V, W, O, den, dO, L, P, tau, causal, B, H, N, d, dt, chunk, dQ, dK,
                         dV, nullptr, workspace, ws_bytes, stream, saved, trace, nullptr);
}

race_status_t race_attn_backward_dw(const void *Q, const void *K, const void *V,
                                    const float *W, const void *O, const float *den,
                                    const void *dO, int L, int P, float tau, int causal, int B,
                                    int H, int64_t N, int d, race_dtype_t dt, int chunk, void *dQ,
                                    void *dK, void *dV, float *dW, void *workspace,
                                    size_t ws_bytes, void *stream, const void *saved,
                                    race_trace_t *trace)
{
    if (!dW) return RACE_ERR_NULL;
    return backward_impl(Q, K, V, W, O, den, dO, L, P, tau, causal, B, H, N, d, dt, chunk, dQ, dK,
                         dV, dW, workspace, ws_bytes, stream, saved, trace, nullptr);
}

race_status_t race_attn_backward_padded(const void *Q, const void *K, const void *V,
                                        const float *W, const void *O, const float *den,
                                        const void *dO, int L, int P, float tau, int causal, int B,
                                        int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                        const int *seqlens, void *dQ, void *dK, void *dV,
                                        float *dW, void *workspace, size_t ws_bytes, void *stream)
{
    if (!seqlens) return RACE_ERR_NULL;
    return backward_impl(Q, K, V, W, O, den, dO, L, P, tau, causal, B, H, N, d, dt, chunk, dQ, dK,
                         dV, dW, workspace, ws_bytes, stream, nullptr, nullptr, seqlens);
}

race_status_t race_attn_backward(const void *Q, const void *K, const void *V, const float *W,
                                 const void *O, const float *den, const void *dO, int L,
                                 int P, float tau, int causal, int B, int H, int64_t N, int d,
                                 race_dtype_t dt, int chunk, void *dQ, void *dK, void *dV,
                                 void *workspace, size_t ws_bytes, void *stream)
{
    return race_attn_backward_ex(Q, K, V, W, O, den, dO, L, P, tau, causal, B, H, N, d, dt, chunk,
                                 dQ, dK, dV, workspace, ws_bytes, stream, nullptr, nullptr);
}

static race_status_t squash_coeffs(float tau, race_dtype_t dt, float *coef, int *deg, bool deriv)
{
    if (!coef || !deg) return RACE_ERR_NULL;
    race_status_t st = check_tau(tau);
    if (st != RACE_OK) return st;
    if (dt != RACE_F32 && dt != RACE_BF16 && dt != RACE_F16) return RACE_ERR_UNSUPPORTED;
    // fp16 rows take the bf16 path's squash (its operands are bf16)
    const race::Squash sq = fit_squash(tau, dt == RACE_F16 ? RACE_BF16 : dt);
    for (int i = 0; i <= race::MAXDEG; ++i)
        coef[i] = (sq.deg >= 0 && i <= sq.deg) ? (float)f16_value(deriv ? sq.c16[i] : sq.t16[i]) : 0.f;
    *deg = sq.deg;
    return RACE_OK;
}

race_status_t race_attn_squash_coeffs(float tau, race_dtype_t dt, float *coef, int *deg)
{
    return squash_coeffs(tau, dt, coef, deg, false);
}

race_status_t race_attn_squash_deriv_coeffs(float tau, race_dtype_t dt, float *coef, int *deg)
{
    return squash_coeffs(tau, dt, coef, deg, true);
}

race_status_t race_attn_state_bytes(int B, int H, int d, int L, int P, size_t *bytes)
{
    if (!bytes) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, 1, d, L, P, RACE_F32, &sp);
    if (st != RACE_OK) return st;
    *bytes = (size_t)sp.BH * sp.elems * sizeof(float);
    return RACE_OK;
}

race_status_t race_attn_state_add_workspace_bytes(int B, int H, int64_t N, int d, int L, int P,
                                                  size_t *bytes)
{
    if (!bytes) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, N, d, L, P, RACE_F32, &sp);
    if (st != RACE_OK) return st;
    *bytes = N == 0 ? 0 : (size_t)sp.BH * stream_blocks(sp, N) * sp.elems * sizeof(float);
    return RACE_OK;
}

race_status_t race_attn_state_add(const void *K, const void *V, const float *W, int L, int P,
                                  float tau, int B, int H, int64_t N, int d, race_dtype_t dt,
                                  float *state, void *workspace, size_t ws_bytes, void *stream)
{
    if (!W || !state) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, N, d, L, P, dt, &sp);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if (N == 0) return RACE_OK;  // the row pointers may be NULL then
    if (!K || !V) return RACE_ERR_NULL;
    const int64_t nblk = stream_blocks(sp, N);
    if (!workspace) return RACE_ERR_NULL;
    if (ws_bytes < (size_t)sp.BH * nblk * sp.elems * sizeof(float) || ((uintptr_t)workspace & 255))
        return RACE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *part = static_cast<float *>(workspace);
    (void)hipGetLastError();
    if (dt == RACE_BF16)
        launch_stream<bf16, race::SM_ADD>(sp, nullptr, K, V, W, tau, N, nblk, state, part, nullptr,
                                          nullptr, s);
    else if (dt == RACE_F16)
        launch_stream<_Float16, race::SM_ADD>(sp, nullptr, K, V, W, tau, N, nblk, state, part,
                                              nullptr, nullptr, s);
    else
        launch_stream<float, race::SM_ADD>(sp, nullptr, K, V, W, tau, N, nblk, state, part,
                                           nullptr, nullptr, s);
    hipLaunchKernelGGL(race::stream_reduce_kernel, dim3((unsigned)((sp.elems + 255) / 256), sp.BH),
                       dim3(256), 0, s, part, (int)nblk, sp.elems, state);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_state_add_fast(const void *K, const void *V, const float *W, int L, int P,
                                       float tau, int B, int H, int64_t N, int d,
                                       race_dtype_t dt, float *state, void *workspace,
                                       size_t ws_bytes, void *stream)
{
    if (!W || !state) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, N, d, L, P, dt, &sp);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if (N == 0) return RACE_OK;  // the row pointers may be NULL then
    if (!K || !V) return RACE_ERR_NULL;
    Plan p;
    if ((st = make_plan(B, H, N, d, L, P, 0, dt, &p)) != RACE_OK) return st;
    if (!p.fused) return RACE_ERR_UNSUPPORTED;
    if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
    const Tracer tr{nullptr, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (dt == RACE_BF16)
        dispatch_fused_state_add<bf16>(p, K, V, W, tau, ws, state, tr);
    else
        dispatch_fused_state_add<_Float16>(p, K, V, W, tau, ws, state, tr);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_decode(const void *Q, const void *K, const void *V, const float *W,
                               int L, int P, float tau, int B, int H, int64_t T, int d,
                               race_dtype_t dt, float *state, void *O, float *den, void *stream)
{
    if (!W || !state) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, T, d, L, P, dt, &sp);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if (T == 0) return RACE_OK;  // the row pointers may be NULL then
    if (!Q || !K || !V || !O || !den) return RACE_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dt == RACE_BF16)
        launch_stream<bf16, race::SM_DECODE>(sp, Q, K, V, W, tau, T, 1, state, nullptr, O, den, s);
    else if (dt == RACE_F16)
        launch_stream<_Float16, race::SM_DECODE>(sp, Q, K, V, W, tau, T, 1, state, nullptr, O, den, s);
    else
        launch_stream<float, race::SM_DECODE>(sp, Q, K, V, W, tau, T, 1, state, nullptr, O, den, s);
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_state_readout(const void *Q, const float *W, int L, int P, float tau,
                                      int B, int H, int64_t T, int d, race_dtype_t dt,
                                      const float *state, void *O, float *den, void *stream)
{
    if (!W || !state) return RACE_ERR_NULL;
    StreamPlan sp;
    race_status_t st = stream_plan(B, H, T, d, L, P, dt, &sp);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if (T == 0) return RACE_OK;  // the row pointers may be NULL then
    if (!Q || !O || !den) return RACE_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *sv = const_cast<float *>(state);  // read only in this mode
    (void)hipGetLastError();
    const int64_t nblk = stream_blocks(sp, T);
    if (dt == RACE_BF16)
        launch_stream<bf16, race::SM_READOUT>(sp, Q, nullptr, nullptr, W, tau, T, nblk, sv,
                                              nullptr, O, den, s);
    else if (dt == RACE_F16)
        launch_stream<_Float16, race::SM_READOUT>(sp, Q, nullptr, nullptr, W, tau, T, nblk, sv,
                                                  nullptr, O, den, s);
    else
        launch_stream<float, race::SM_READOUT>(sp, Q, nullptr, nullptr, W, tau, T, nblk, sv,
                                               nullptr, O, den, s);
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
