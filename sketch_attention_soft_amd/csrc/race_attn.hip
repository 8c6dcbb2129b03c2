// race_attn.hip -- C ABI of the RACE attention library (declared in include/race_attn.h).
//
// Host side: argument validation, workspace planning and kernel sequencing
// on the caller's stream.  No allocation and no synchronisation; the only
// global state is the per-device address of the allocation-free forward's
// scratch array, looked up once per device.
#include "race_attn.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "race_host.h"

// Workspace of race_attn_forward_noalloc: one copy per GPU, allocated when the
// code object is loaded on that device and held until the process ends.  In
// host code this name is a host-side stand-in; the device address comes from
// hipGetSymbolAddress (scratch_address below).
__device__ __align__(256) char scratch[RACE_NOALLOC_SCRATCH_BYTES];

namespace race_host {

race_status_t make_plan(int B, int H, int64_t N, int d, int L, int P, int chunk,
                        race_dtype_t dt, Plan *p)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || L < 1 || P < 1) return RACE_ERR_SHAPE;
    if (N > kMaxN || (int64_t)B * H > 65535) return RACE_ERR_SHAPE;
    if (dt != RACE_F32 && dt != RACE_BF16 && dt != RACE_F16) return RACE_ERR_UNSUPPORTED;
    if (P > 6) return RACE_ERR_UNSUPPORTED;
    if (L > 128) return RACE_ERR_UNSUPPORTED;
    // P = 5, 6: 2^(P-4) virtual tables of 4 planes per table, on the fused
    // kernels (16-bit rows, d = 64)
    const int vs = vt_shift(P), Lv = L << vs;
    if (vs && (dt == RACE_F32 || d != race::HD)) return RACE_ERR_UNSUPPORTED;
    // 16-bit rows with more than 32 (virtual) tables: fused passes of up to
    // 32, d = 64 only
    if (dt != RACE_F32 && Lv > 32 && d != race::HD) return RACE_ERR_UNSUPPORTED;
    // d = 64 and P = 4, or d = 32 and P < 4 on the fused path (16-bit rows, L <= 32);
    // d = 128 in two passes of 64 value columns (16-bit rows, L <= 32, P <= 4)
    const bool fusable = dt != RACE_F32 && Lv <= 32;
    const bool wide = d == 2 * race::HD && fusable && P <= race::NP;
    if (d != race::HD && !(d == 32 && fusable) && !wide) return RACE_ERR_UNSUPPORTED;
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
    p->nw = Lv <= 8 ? 1 : Lv <= 16 ? 2 : Lv <= 32 ? 4 : 8;
    p->F = p->nw * race::FPW;
    p->LP = Lv * race::NP;  // internal hyperplane rows
    const int64_t n16 = (N + 15) / 16 * 16;
    int64_t seg = chunk;
    if (seg == 0) {
        // one round of workgroups over the compute units (MI355X: 256 CUs):
        // one 8-wave workgroup per CU (32 tables), two 4-wave ones (16
        // tables), four 2-wave ones; segments >= 32 tokens (short sequences:
        // more, shorter segments, for latency)
        const int64_t wgs = 256 * (4 / std::min(p->nw, 4));
        const int64_t want = (p->rows + wgs - 1) / wgs;
        seg = (want + 31) / 32 * 32;
        if (seg < 32) seg = 32;
    }
    if (seg > n16) seg = n16;
    seg = (seg + 31) / 32 * 32;  // whole 32-token sub-chunks per segment
    p->seg = seg;
    p->nseg = (N + seg - 1) / seg;
    if (p->BH * p->nseg > 0x7fffffffLL) return RACE_ERR_SHAPE;
    p->wide = wide;
    p->fused = (dt == RACE_BF16 || dt == RACE_F16) && Lv <= 32 && !wide;
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
    p->hc_bytes = p->fused || wide ? align256((size_t)p->BH * p->hc_tiles * (2 * p->nw) * 64 * 4 * 2) : 0;
    p->f_tq = 0;
    p->f_tk = p->f_tq + p->t_bytes;
    p->f_st = p->f_tk + p->t_bytes;
    p->f_hc = p->f_st + p->st_bytes;
    p->f_scan = p->f_hc + p->hc_bytes;
    p->f_total = p->f_scan + p->scan_bytes;
    p->s_hc = p->st_bytes;
    // saved state: the key state and the fp16 hash features of Q and K (fused
    // path); t and dt/du' of Q and of K in fp32 (fp32 rows, whose backward
    // reads them instead of hashing again)
    p->s_total = p->fused ? p->s_hc + 4 * p->hc_bytes : dt == RACE_F32 ? 2 * p->tb_bytes : 0;
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
    p->w_du = p->w_du_bytes = p->w_dm = 0;
    if (wide) {
        // forward: the segment states, the scan's totals, t of K and of Q;
        // backward: key and gradient states, the scan's totals, t and dt/du
        // of K and of Q, du of Q and K for both passes, the values' last
        // column.  The saved buffer keeps t and dt/du of K and Q (the
        // backward rehashes without it); no dW.
        p->w_du_bytes = align256((size_t)p->rows * (2 * p->nw) * 16 * sizeof(bf16));
        p->f_st = 0;
        p->f_scan = p->f_st + p->st_bytes;
        p->f_hc = p->f_scan + p->scan_bytes;
        p->f_total = p->f_hc + 2 * p->hc_bytes;
        p->b_s = 0;
        p->b_g = p->b_s + p->st_bytes;
        p->b_scan = p->b_g + p->st_bytes;
        p->b_hc = p->b_scan + p->scan_bytes;
        p->w_du = p->b_hc + 4 * p->hc_bytes;
        p->w_dm = p->w_du + 4 * p->w_du_bytes;
        p->b_total = p->w_dm + align256((size_t)p->rows * sizeof(float));
        p->dw_total = 0;
        p->s_hc = 0;
        p->s_total = 4 * p->hc_bytes;
    }
    if (Lv > 32) {
        // passes over tables 0..31, 32..63, ... (split_passes; the fused
        // kernels for 16-bit rows, the unfused ones for fp32; 32 virtual
        // tables for P = 5, 6): every pass's buffers, then the fp32 partial
        // sums
        const size_t pv = align256((size_t)p->rows * race::HD * sizeof(float));
        const size_t pm = align256((size_t)p->rows * sizeof(float));
        p->split = true;
        p->f_total = pv + pm;
        p->b_total = p->dw_total = 3 * pv;
        p->s_total = 0;
        for (int i = 0; i < split_passes(L, P); ++i) {
            Plan a;
            race_status_t st = make_plan(B, H, N, d, split_tables(L, P, i), P, chunk, dt, &a);
            if (st != RACE_OK) return st;
            p->f_total += a.f_total;
            p->b_total += a.b_total;
            p->dw_total += a.dw_total;
            p->s_total += a.s_total;
        }
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

}  // namespace race_host

namespace {

using namespace race_host;

// Device address of `scratch` on the current device, looked up on the first
// call with that device current and kept per device.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

race_status_t scratch_address(char **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RACE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return RACE_ERR_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *out = static_cast<char *>(g_scratch[dev]);
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

// Packed batches run on the fused kernels only (16-bit rows); the T rows of
// every head must fit the B N rows the plan sizes its partial sums for.
race_status_t check_packed(const Plan &p, int B, int64_t N, int64_t T)
{
    if (!p.fused && !p.split) return RACE_ERR_UNSUPPORTED;
    if (T < 1 || T > (int64_t)B * N) return RACE_ERR_SHAPE;
    return RACE_OK;
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

// The hard forward's plan: P = 5, 6 run on the id path only, as L 2^(P-4)
// virtual tables of 4 planes (16 buckets each) for the sum and walk kernels;
// ids_path tells whether the id kernels run (else the soft kernels with
// t = +-1 on the real tables).
race_status_t hard_forward_plan(int B, int H, int64_t N, int d, int L, int P, int chunk,
                                race_dtype_t dt, Plan *p, bool *ids_path)
{
    const int vs = P > race::NP && P <= 6 ? P - race::NP : 0;
    if (vs) {
        if (L < 1) return RACE_ERR_SHAPE;
        if (L > 128) return RACE_ERR_UNSUPPORTED;
        const race_status_t st = make_plan(B, H, N, d, L << vs, race::NP, chunk, dt, p);
        if (st != RACE_OK) return st;
        if (!hard_fused(*p, dt)) return RACE_ERR_UNSUPPORTED;
        *ids_path = true;
        return RACE_OK;
    }
    const race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, p);
    if (st != RACE_OK) return st;
    if (p->wide) return RACE_ERR_UNSUPPORTED;  // d = 128: the soft path only
    *ids_path = hard_fused(*p, dt);
    return RACE_OK;
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
    if (for_backward == 4) {
        bool ids_path = false;
        const race_status_t st = hard_forward_plan(B, H, N, d, L, P, chunk, dt, &p, &ids_path);
        if (st != RACE_OK) return st;
        *bytes = ids_path ? hard_plan(p, L, P).total : p.f_total;
        return RACE_OK;
    }
    const race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if (for_backward == 2 && (dt == RACE_F32 || (!p.fused && !p.split))) return RACE_ERR_UNSUPPORTED;
    if (for_backward == 3 && !p.fused) return RACE_ERR_UNSUPPORTED;
    if (for_backward < 0 || for_backward > 4) return RACE_ERR_SHAPE;
    *bytes = for_backward == 3   ? p.st_bytes + p.scan_bytes
             : for_backward == 2 ? p.dw_total
             : for_backward      ? p.b_total
                                 : p.f_total;
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
                                  race_trace_t *trace, const int *lens, const int *cu = nullptr,
                                  int64_t T = 0)
{
    if (!Q || !K || !V || !W || !O || !den || !workspace) return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if (cu && (st = check_packed(p, B, N, T)) != RACE_OK) return st;
    if (p.wide && (lens || cu)) return RACE_ERR_UNSUPPORTED;  // d = 128: dense heads only
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
    if ((st = check_trace(trace)) != RACE_OK) return st;
    if (saved && ((uintptr_t)saved & 255) != 0) return RACE_ERR_WORKSPACE;
    p.lens.len = lens;
    p.lens.cu = cu;
    p.lens.T = T;
    float *sv = p.s_total > 0 ? static_cast<float *>(saved) : nullptr;
    const Tracer tr{trace, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (p.split && dt == RACE_BF16)
        split_forward<bf16>(p, B, H, chunk, dt, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else if (p.split && dt == RACE_F16)
        split_forward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
    else if (p.split)
        split_forward<float>(p, B, H, chunk, dt, Q, K, V, W, tau, causal, O, den, ws, sv, tr);
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
                                   const void *saved, race_trace_t *trace, const int *lens,
                                   const int *cu = nullptr, int64_t T = 0)
{
    if (!Q || !K || !V || !W || !O || !den || !dO || !dQ || !dK || !dV || !workspace)
        return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if (cu && (st = check_packed(p, B, N, T)) != RACE_OK) return st;
    if (p.wide && (lens || cu)) return RACE_ERR_UNSUPPORTED;  // d = 128: dense heads only
    if (dW && (dt == RACE_F32 || (!p.fused && !p.split))) return RACE_ERR_UNSUPPORTED;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if ((st = check_ws(p, dW ? p.dw_total : p.b_total, workspace, ws_bytes)) != RACE_OK) return st;
    if ((st = check_trace(trace)) != RACE_OK) return st;
    if (saved && ((uintptr_t)saved & 255) != 0) return RACE_ERR_WORKSPACE;
    p.lens.len = lens;
    p.lens.cu = cu;
    p.lens.T = T;
    const float *sv = p.s_total > 0 ? static_cast<const float *>(saved) : nullptr;
    const Tracer tr{trace, static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();
    char *ws = static_cast<char *>(workspace);
    if (p.split && dt == RACE_BF16)
        split_backward<bf16>(p, B, H, chunk, dt, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr, dW);
    else if (p.split && dt == RACE_F16)
        split_backward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr,
                                 dW);
    else if (p.split)
        split_backward<float>(p, B, H, chunk, dt, Q, K, V, W, O, den, dO, tau, causal, dQ, dK, dV, ws, sv, tr,
                              nullptr);
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

// Hard hashing: the bucket-id kernels for 16-bit rows with L <= 32, P <= 4,
// d = 32 or 64; otherwise the chunked soft kernels with t = +-1 (no int32
// counts there).
static race_status_t hard_impl(const void *Q, const void *K, const void *V, const float *W, int L,
                               int P, int causal, int B, int H, int64_t N, int d, race_dtype_t dt,
                               int chunk, void *O, float *den, int32_t *count, void *workspace,
                               size_t ws_bytes, void *stream)
{
    if (!Q || !K || !V || !W || !O || !den || !workspace) return RACE_ERR_NULL;
    Plan p;
    bool ids_path = false;
    race_status_t st = hard_forward_plan(B, H, N, d, L, P, chunk, dt, &p, &ids_path);
    if (st != RACE_OK) return st;
    if (!ids_path) {
        // tau = 0 selects hard hashing in the soft kernels
        if (count) return RACE_ERR_UNSUPPORTED;
        if ((st = check_ws(p, p.f_total, workspace, ws_bytes)) != RACE_OK) return st;
        const Tracer tr{nullptr, static_cast<hipStream_t>(stream)};
        (void)hipGetLastError();
        char *ws = static_cast<char *>(workspace);
        if (p.split && dt == RACE_BF16)
            split_forward<bf16>(p, B, H, chunk, dt, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        else if (p.split && dt == RACE_F16)
            split_forward<_Float16>(p, B, H, chunk, dt, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        else if (p.split)
            split_forward<float>(p, B, H, chunk, dt, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        else if (dt == RACE_BF16)
            dispatch_forward<bf16>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        else if (dt == RACE_F16)
            dispatch_forward<_Float16>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        else
            dispatch_forward<float>(p, Q, K, V, W, 0.f, causal, O, den, ws, nullptr, tr);
        return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
    }
    const HardPlan h = hard_plan(p, L, P);
    if (ws_bytes < h.total || ((uintptr_t)workspace & 255)) return RACE_ERR_WORKSPACE;
    (void)hipGetLastError();
    hard_forward_launch(p, L, P, dt, Q, K, V, W, causal, O, den, count, static_cast<char *>(workspace),
                        static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? RACE_OK : RACE_ERR_HIP;
}

race_status_t race_attn_forward_hard(const void *Q, const void *K, const void *V,
                                     const float *W, int L, int P, int causal, int B, int H,
                                     int64_t N, int d, race_dtype_t dt, int chunk, void *O,
                                     float *den, void *workspace, size_t ws_bytes, void *stream)
{
    return hard_impl(Q, K, V, W, L, P, causal, B, H, N, d, dt, chunk, O, den, nullptr, workspace,
                     ws_bytes, stream);
}

race_status_t race_attn_forward_hard_counts(const void *Q, const void *K, const void *V,
                                            const float *W, int L, int P, int causal, int B, int H,
                                            int64_t N, int d, race_dtype_t dt, int chunk, void *O,
                                            float *den, int32_t *count, void *workspace,
                                            size_t ws_bytes, void *stream)
{
    if (!count) return RACE_ERR_NULL;
    return hard_impl(Q, K, V, W, L, P, causal, B, H, N, d, dt, chunk, O, den, count, workspace,
                     ws_bytes, stream);
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

race_status_t race_attn_forward_varlen(const void *Q, const void *K, const void *V,
                                       const float *W, int L, int P, float tau, int causal, int B,
                                       int H, int64_t T, int64_t max_seqlen, int d,
                                       race_dtype_t dt, int chunk, const int *cu_seqlens, void *O,
                                       float *den, void *workspace, size_t ws_bytes, void *stream)
{
    if (!cu_seqlens) return RACE_ERR_NULL;
    return forward_impl(Q, K, V, W, L, P, tau, causal, B, H, max_seqlen, d, dt, chunk, O, den,
                        workspace, ws_bytes, stream, nullptr, nullptr, nullptr, cu_seqlens, T);
}

race_status_t race_attn_backward_varlen(const void *Q, const void *K, const void *V,
                                        const float *W, const void *O, const float *den,
                                        const void *dO, int L, int P, float tau, int causal, int B,
                                        int H, int64_t T, int64_t max_seqlen, int d,
                                        race_dtype_t dt, int chunk, const int *cu_seqlens,
                                        void *dQ, void *dK, void *dV, float *dW, void *workspace,
                                        size_t ws_bytes, void *stream)
{
    if (!cu_seqlens) return RACE_ERR_NULL;
    return backward_impl(Q, K, V, W, O, den, dO, L, P, tau, causal, B, H, max_seqlen, d, dt,
                         chunk, dQ, dK, dV, dW, workspace, ws_bytes, stream, nullptr, nullptr,
                         nullptr, cu_seqlens, T);
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
    if ((st = check_ws(p, p.st_bytes + p.scan_bytes, workspace, ws_bytes)) != RACE_OK) return st;
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

race_status_t race_attn_forward_noalloc(const void *Q, const void *K, const void *V,
                                        const float *W, int L, int P, float tau, int causal,
                                        int B, int H, int64_t N, int d, race_dtype_t dt, int chunk,
                                        void *O, float *den, void *stream)
{
    if (!Q || !K || !V || !W || !O || !den) return RACE_ERR_NULL;
    Plan p;
    race_status_t st = make_plan(B, H, N, d, L, P, chunk, dt, &p);
    if (st != RACE_OK) return st;
    if ((st = check_tau(tau)) != RACE_OK) return st;
    if (p.f_total > RACE_NOALLOC_SCRATCH_BYTES) return RACE_ERR_WORKSPACE;
    char *ws = nullptr;
    if ((st = scratch_address(&ws)) != RACE_OK) return st;
    return forward_impl(Q, K, V, W, L, P, tau, causal, B, H, N, d, dt, chunk, O, den, ws,
                        RACE_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr);
}

race_status_t race_attn_hash_ids_workspace_bytes(int L, int P, int d, size_t *bytes)
{
    if (!bytes) return RACE_ERR_NULL;
    if (L < 1 || P < 1 || d < 1) return RACE_ERR_SHAPE;
    if (L > 128 || P > 6 || d > 128 || d % 8 != 0) return RACE_ERR_UNSUPPORTED;
    *bytes = hard_ids_ws(L, P, d);
    return RACE_OK;
}

race_status_t race_attn_hash_ids(const void *X, int64_t rows, int d, race_dtype_t dt,
                                 const float *W, int L, int P, uint8_t *ids, void *workspace,
                                 size_t ws_bytes, void *stream)
{
    size_t need = 0;
    race_status_t st = race_attn_hash_ids_workspace_bytes(L, P, d, &need);
    if (st != RACE_OK) return st;
    if (rows < 0 || rows > ((int64_t)1 << 40)) return RACE_ERR_SHAPE;
    if (dt != RACE_F32 && dt != RACE_BF16 && dt != RACE_F16) return RACE_ERR_UNSUPPORTED;
    if (rows == 0) return RACE_OK;
    if (!X || !W || !ids || !workspace) return RACE_ERR_NULL;
    if (ws_bytes < need || ((uintptr_t)workspace & 255)) return RACE_ERR_WORKSPACE;
    (void)hipGetLastError();
    hard_ids_launch(X, rows, d, dt, W, L, P, ids, static_cast<char *>(workspace),
                    static_cast<hipStream_t>(stream));
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
