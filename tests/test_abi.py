"""The C ABI without a GPU: loading, exported symbols, argument validation,
workspace sizing, status strings and the host-fitted squash polynomial.

Every call here returns before the library touches the HIP runtime (the
documented validation order), so no device is needed.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from sketch_attention_soft_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "race_attn.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_TAU, E_CHUNK, E_WS, E_HIP = range(8)
F32, BF16, F16 = 0, 1, 2


# the library under test: the built one, or another build of the same
# sources (tests/test_sanitizers.py runs this file against a host build with
# AddressSanitizer and UndefinedBehaviorSanitizer)
LIB_UNDER_TEST = os.environ.get("RACE_ABI_TEST_LIB") or hip_build.LIB


@pytest.fixture(scope="module")
def lib():
    if LIB_UNDER_TEST == hip_build.LIB and not os.path.exists(hip_build.LIB):
        hip_build.build()
    L = ctypes.CDLL(LIB_UNDER_TEST)
    i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    L.race_attn_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(sz)]
    L.race_attn_forward.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i32, i64, i32, i32,
                                    i32, vp, vp, vp, sz, vp]
    L.race_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, i32, i32, i32,
                                     i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.race_attn_status_string.argtypes = [i32]
    L.race_attn_status_string.restype = ctypes.c_char_p
    for fn in (L.race_attn_squash_coeffs, L.race_attn_squash_deriv_coeffs):
        fn.argtypes = [f32, i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]
    return L


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(race_attn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert {"race_attn_forward", "race_attn_backward", "race_attn_workspace_bytes",
            "race_attn_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_lists_the_header(lib):
    from sketch_attention_soft_amd import binding
    assert set(binding.EXPORTS) <= set(header_functions())


def ws_bytes(lib, B=1, H=1, N=1024, d=64, L=8, P=4, causal=1, chunk=0, dt=BF16, bwd=0):
    out = ctypes.c_size_t(0)
    st = lib.race_attn_workspace_bytes(B, H, N, d, L, P, causal, chunk, dt, bwd,
                                       ctypes.byref(out))
    return st, out.value


def test_workspace_sizes(lib):
    st, f = ws_bytes(lib)
    assert st == OK and f > 0 and f % 256 == 0
    st, b = ws_bytes(lib, bwd=1)
    assert st == OK and b >= f
    # grows with N and with the table count
    assert ws_bytes(lib, N=1 << 20)[1] > f
    assert ws_bytes(lib, L=32)[1] > f
    # fp32 keeps per-row hash buffers, bf16 (fused) does not
    assert ws_bytes(lib, dt=F32, N=1 << 16)[1] > ws_bytes(lib, dt=BF16, N=1 << 16)[1]
    # fp16 rows take the bf16 (fused) path: the same workspace
    for bwd in (0, 1, 2):
        assert ws_bytes(lib, dt=F16, L=32, bwd=bwd) == ws_bytes(lib, dt=BF16, L=32, bwd=bwd)
    # the 75M-token workload fits comfortably in one GPU's HBM: segment states
    # plus four fp16 hash-feature arrays (t, dt/du' of Q and K), 512 B per row
    st, b75 = ws_bytes(lib, N=75_000_064, L=16, bwd=1)
    assert st == OK and b75 < 75_000_064 * 16 * 4 * 2 * 4 + (4 << 30)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), E_SHAPE), (dict(H=-1), E_SHAPE), (dict(N=0), E_SHAPE), (dict(L=0), E_SHAPE),
    (dict(d=48), E_UNSUP), (dict(d=96), E_UNSUP), (dict(d=128, dt=F32), E_UNSUP),
    (dict(d=128, L=33), E_UNSUP), (dict(d=128, P=5), E_UNSUP), (dict(d=128, bwd=2), E_UNSUP),
    (dict(d=256), E_UNSUP), (dict(d=32, dt=F32), E_UNSUP),
    (dict(d=32, L=33), E_UNSUP), (dict(P=7), E_UNSUP), (dict(P=3, dt=F32), E_UNSUP),
    (dict(P=5, dt=F32), E_UNSUP), (dict(P=6, d=32), E_UNSUP), (dict(P=6, L=129), E_UNSUP),
    (dict(P=0), E_SHAPE), (dict(L=129), E_UNSUP), (dict(L=129, dt=F32), E_UNSUP),
    (dict(L=33, dt=F32, bwd=2), E_UNSUP), (dict(L=8, dt=F32, bwd=2), E_UNSUP),
    (dict(d=32, L=33, dt=F16), E_UNSUP), (dict(dt=5), E_UNSUP),
    (dict(chunk=17), E_CHUNK), (dict(chunk=-16), E_CHUNK),
])
def test_workspace_validation(lib, kw, code):
    assert ws_bytes(lib, **kw)[0] == code


def test_head_dim_128(lib):
    """d = 128 on 16-bit rows (up to 32 tables, P <= 4): two passes of 64 value
    columns; the backward keeps du of both passes, so it needs more room than
    d = 64; the saved buffer holds the hash features of Q and K only."""
    for dt in (BF16, F16):
        for L in (1, 8, 32):
            for bwd in (0, 1):
                st, b = ws_bytes(lib, d=128, L=L, dt=dt, bwd=bwd, N=3000)
                assert st == OK and b > 0, (dt, L, bwd)
        assert ws_bytes(lib, d=128, dt=dt, bwd=1, N=3000)[1] > ws_bytes(lib, d=64, dt=dt, bwd=1, N=3000)[1]
    out = ctypes.c_size_t(7)
    assert lib.race_attn_saved_bytes(1, 1, 3000, 128, 8, 4, 1, 0, BF16, ctypes.byref(out)) == OK
    s128 = out.value
    assert lib.race_attn_saved_bytes(1, 1, 3000, 64, 8, 4, 1, 0, BF16, ctypes.byref(out)) == OK
    assert 0 < s128 < out.value  # no key state


def test_virtual_tables(lib):
    """P = 5, 6 on 16-bit rows: 2^(P-4) virtual tables of 16 features per
    table, in passes of 32 virtual tables when there are more."""
    for P in (5, 6):
        prev = 0
        for L in (1, 4, 8, 9, 16, 17, 33, 128):
            for bwd in (0, 1, 2):
                st, b = ws_bytes(lib, L=L, P=P, bwd=bwd, N=3000)
                assert st == OK and b > 0, (P, L, bwd)
            st, b = ws_bytes(lib, L=L, P=P, N=3000)
            assert b >= prev
            prev = b
        # a P = 6 table takes the room of four P = 4 tables
        assert ws_bytes(lib, L=8, P=6, N=3000)[1] == ws_bytes(lib, L=32, P=4, N=3000)[1]


def test_tables_in_passes(lib):
    """16-bit rows with L > 32 run as passes of up to 32 tables: the workspace
    grows with every pass plus the partial sums, up to L = 128."""
    prev = 0
    for L in (32, 33, 64, 65, 96, 97, 128):
        for bwd in (0, 1, 2):
            st, b = ws_bytes(lib, L=L, bwd=bwd, N=5000)
            assert st == OK and b > 0, (L, bwd)
        st, b = ws_bytes(lib, L=L, N=5000)
        assert b > prev
        prev = b
    # fp32 rows: passes of the unfused kernels; the saved state is t and
    # dt/du' of Q and K per pass (8 fp32 per row and table, each array
    # 256-byte aligned)
    prev = 0
    for L in (32, 33, 64, 65, 128):
        for bwd in (0, 1):
            st, b = ws_bytes(lib, L=L, bwd=bwd, N=5000, dt=F32)
            assert st == OK and b > 0, (L, bwd)
        st, b = ws_bytes(lib, L=L, N=5000, dt=F32)
        assert b > prev
        prev = b
        sz0 = ctypes.c_size_t(1)
        assert lib.race_attn_saved_bytes(1, 1, 5000, 64, L, 4, 1, 0, F32, ctypes.byref(sz0)) == OK
        passes = [min(32, L - 32 * i) for i in range((L + 31) // 32)]
        assert sz0.value == sum(2 * ((5000 * lp * 32 + 255) // 256 * 256) for lp in passes), L
    # a saved state for every pass
    sz = ctypes.c_size_t(0)
    sizes = []
    for L in (32, 64, 96, 128):
        assert lib.race_attn_saved_bytes(1, 1, 5000, 64, L, 4, 1, 0, BF16, ctypes.byref(sz)) == OK
        sizes.append(sz.value)
    assert sizes[1] == 2 * sizes[0] and sizes[3] == 4 * sizes[0] and sizes[2] == 3 * sizes[0]


def test_fewer_hyperplanes(lib):
    # P = 1..3 run the fused kernels with padding hyperplanes: the same
    # workspace as P = 4 for 16-bit rows and L <= 32
    for P in (1, 2, 3):
        for dt in (BF16, F16):
            for bwd in (0, 1, 2):
                st, b = ws_bytes(lib, P=P, L=32, dt=dt, bwd=bwd)
                assert st == OK and (st, b) == ws_bytes(lib, P=4, L=32, dt=dt, bwd=bwd)


def test_head_dim_32(lib):
    # d = 32 runs the fused kernels with rows zero-padded on chip: the same
    # workspace as d = 64 for 16-bit rows and L <= 32
    for dt in (BF16, F16):
        for bwd in (0, 1, 2):
            st, b = ws_bytes(lib, d=32, L=32, dt=dt, bwd=bwd)
            assert st == OK and b > 0 and (st, b) == ws_bytes(lib, d=64, L=32, dt=dt, bwd=bwd)


def test_saved_bytes(lib):
    fn = lib.race_attn_saved_bytes
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.POINTER(ctypes.c_size_t)]
    out = ctypes.c_size_t(7)
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, BF16, ctypes.byref(out)) == OK
    assert out.value > 0 and out.value % 256 == 0
    # one fp32 state of F x 80 per segment plus the head total
    assert out.value >= 2 * 512 * 80 * 4
    # fp32 rows: t and dt/du' of Q and K, 8 fp32 per row and table
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, F32, ctypes.byref(out)) == OK
    assert out.value == 2 * (1 << 16) * 32 * 8 * 4
    # fp16 rows save the same state as bf16 rows
    o16, ob = ctypes.c_size_t(0), ctypes.c_size_t(1)
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, F16, ctypes.byref(o16)) == OK
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, BF16, ctypes.byref(ob)) == OK
    assert o16.value == ob.value > 0
    # L > 32 (two passes of the fused kernels): both passes' saved states
    o32, o64 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, BF16, ctypes.byref(o32)) == OK
    assert fn(1, 1, 1 << 16, 64, 64, 4, 1, 0, BF16, ctypes.byref(o64)) == OK
    assert o64.value == 2 * o32.value
    assert fn(1, 1, 1 << 16, 64, 32, 4, 1, 0, BF16, None) == E_NULL
    assert fn(1, 1, 0, 64, 32, 4, 1, 0, BF16, ctypes.byref(out)) == E_SHAPE


def test_saved_alignment(lib):
    i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    lib.race_attn_forward_ex.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i32, i64, i32,
                                         i32, i32, vp, vp, vp, sz, vp, vp, vp]
    lib.race_attn_backward_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, i32, i32,
                                          i32, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp, vp, vp]
    st = lib.race_attn_forward_ex(FAKE, FAKE, FAKE, FAKE, 8, 4, 1.0, 1, 1, 1, 64, 64, BF16, 0, FAKE,
                                  FAKE, FAKE * 16, 1 << 30, None, FAKE * 16 + 4, None)
    assert st == E_WS
    st = lib.race_attn_backward_ex(*([FAKE] * 7), 8, 4, 1.0, 1, 1, 1, 64, 64, BF16, 0, FAKE, FAKE,
                                   FAKE, FAKE * 16, 1 << 30, None, FAKE * 16 + 4, None)
    assert st == E_WS


def test_workspace_null(lib):
    assert lib.race_attn_workspace_bytes(1, 1, 16, 64, 8, 4, 1, 0, BF16, 0, None) == E_NULL


FAKE = 0x1000  # never dereferenced: validation fails first


def fwd(lib, ptrs=(FAKE,) * 7, L=8, P=4, tau=1.0, causal=1, B=1, H=1, N=64, d=64, dt=BF16,
        chunk=0, ws_bytes=1 << 30, ws=FAKE * 16):
    q, k, v, W, o, den, _ = ptrs
    return lib.race_attn_forward(q, k, v, W, L, P, tau, causal, B, H, N, d, dt, chunk, o, den, ws,
                                 ws_bytes, None)


def test_forward_validation(lib):
    assert fwd(lib, ptrs=(None,) + (FAKE,) * 6) == E_NULL
    assert fwd(lib, ws=None) == E_NULL
    assert fwd(lib, N=0) == E_SHAPE
    assert fwd(lib, d=96) == E_UNSUP
    assert fwd(lib, d=128, dt=F32) == E_UNSUP
    assert fwd(lib, d=128, L=33) == E_UNSUP
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert fwd(lib, tau=bad) == E_TAU
    assert fwd(lib, chunk=24) == E_CHUNK
    assert fwd(lib, ws_bytes=16) == E_WS
    assert fwd(lib, ws=FAKE * 16 + 8) == E_WS  # not 256-byte aligned


def test_backward_validation(lib):
    args = [FAKE] * 7 + [8, 4, 1.0, 1, 1, 1, 64, 64, BF16, 0] + [FAKE] * 3 + [FAKE * 16, 16,
                                                                            None]
    assert lib.race_attn_backward(*args) == E_WS
    a = list(args)
    a[6] = None  # dO
    assert lib.race_attn_backward(*a) == E_NULL
    a = list(args)
    a[9] = 0.0  # tau
    a[-2] = 1 << 30
    assert lib.race_attn_backward(*a) == E_TAU


def test_status_strings(lib):
    seen = set()
    for code in range(8):
        s = lib.race_attn_status_string(code).decode()
        assert s and s not in seen
        seen.add(s)
    assert lib.race_attn_status_string(99).decode() == "unknown status"


def f16_eval(coef, deg, v):
    """The kernels' fp16 evaluation: y = 2 exp(-2|v|) - 1 formed in fp32 and
    rounded to fp16, then Horner with fused multiply-adds rounded to fp16."""
    v = v.astype(np.float32)
    e = np.exp(np.float32(-2.0) * np.abs(v)).astype(np.float32)
    y = (np.float32(2) * e - np.float32(1)).astype(np.float32).astype(np.float16).astype(np.float64)
    c = np.asarray(coef, dtype=np.float64)
    assert np.all(c.astype(np.float16).astype(np.float64) == c)  # fp16 coefficients
    h = np.full_like(y, c[deg])
    for k in range(deg - 1, -1, -1):
        h = (h * y + c[k]).astype(np.float16).astype(np.float64)
    return h


def coeffs(lib, fn, tau, dt):
    coef = (ctypes.c_float * 17)()
    deg = ctypes.c_int(0)
    assert fn(tau, dt, coef, ctypes.byref(deg)) == OK
    return np.array(coef[:], dtype=np.float64), deg.value


V_GRID = np.concatenate([np.linspace(-12, 12, 200001), [0.0, 1e-30, -1e-30, 1e-6, 40.0]])


@pytest.mark.parametrize("tau", [0.1, 0.25, 0.5, 1.0, 2.0, 8.0])
def test_squash_polynomial_against_numpy_tanh(lib, tau):
    coef, deg = coeffs(lib, lib.race_attn_squash_coeffs, tau, BF16)
    if tau >= 0.5:
        assert deg > 0  # the polynomial, not the fallback, at the workloads' tau
    if deg < 0:
        return
    ref = np.tanh(np.tanh(V_GRID) / tau)
    got = np.copysign(np.abs(f16_eval(coef, deg, V_GRID)), V_GRID)
    assert np.abs(got - ref).max() <= 1.5e-3 + 1e-6, (deg, np.abs(got - ref).max())


@pytest.mark.parametrize("tau", [0.1, 0.25, 0.5, 1.0, 2.0, 8.0])
def test_squash_derivative_against_numpy(lib, tau):
    coef, deg = coeffs(lib, lib.race_attn_squash_deriv_coeffs, tau, BF16)
    tdeg = coeffs(lib, lib.race_attn_squash_coeffs, tau, BF16)[1]
    assert deg == tdeg
    if deg < 0:
        return
    z = np.tanh(V_GRID)
    t = np.tanh(z / tau)
    ref = (1 - t * t) / tau * (1 - z * z)  # d/dv tanh(tanh(v) / tau)
    # the same derivative by central differences of the closed form
    h = 1e-5
    fd = (np.tanh(np.tanh(V_GRID + h) / tau) - np.tanh(np.tanh(V_GRID - h) / tau)) / (2 * h)
    assert np.abs(fd - ref).max() < 1e-8
    got = f16_eval(coef, deg, V_GRID)
    assert np.abs(got - ref).max() <= 1.5e-3 * max(1.0, 1.0 / tau) + 1e-6


def test_squash_f32_is_direct(lib):
    for fn in (lib.race_attn_squash_coeffs, lib.race_attn_squash_deriv_coeffs):
        coef, deg = coeffs(lib, fn, 1.0, F32)
        assert deg == -1 and not coef.any()


def test_squash_rejects_bad_tau(lib):
    coef = (ctypes.c_float * 17)()
    deg = ctypes.c_int(0)
    assert lib.race_attn_squash_coeffs(0.0, BF16, coef, ctypes.byref(deg)) == E_TAU
    assert lib.race_attn_squash_coeffs(1.0, BF16, None, ctypes.byref(deg)) == E_NULL


# ---------------------------------------------------------------------------
# Streaming state entry points (validation and sizes only: no kernel runs)

def _stream_lib(lib):
    i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    lib.race_attn_state_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.race_attn_state_add_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32,
                                                        ctypes.POINTER(sz)]
    lib.race_attn_state_add.argtypes = [vp, vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                        vp, sz, vp]
    lib.race_attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                     vp, vp, vp]
    lib.race_attn_state_readout.argtypes = [vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                            vp, vp, vp]
    return lib


def test_state_bytes(lib):
    L = _stream_lib(lib)
    out = ctypes.c_size_t(0)
    # [B][H][16 L][d + 1] fp32
    assert L.race_attn_state_bytes(2, 3, 64, 32, 4, ctypes.byref(out)) == OK
    assert out.value == 2 * 3 * 512 * 65 * 4
    assert L.race_attn_state_bytes(1, 1, 64, 5, 4, ctypes.byref(out)) == OK
    assert out.value == 80 * 65 * 4
    assert L.race_attn_state_bytes(1, 1, 64, 32, 4, None) == E_NULL
    # P < 4 keeps 16 rows per table
    assert L.race_attn_state_bytes(1, 1, 64, 8, 3, ctypes.byref(out)) == OK and out.value == 128 * 65 * 4
    # any d <= 64: [16 L][d + 1]
    assert L.race_attn_state_bytes(1, 2, 32, 8, 4, ctypes.byref(out)) == OK
    assert out.value == 2 * 128 * 33 * 4
    assert L.race_attn_state_bytes(1, 1, 1, 8, 4, ctypes.byref(out)) == OK and out.value == 128 * 2 * 4
    for args, code in (((0, 1, 64, 8, 4), E_SHAPE), ((1, 1, 65, 8, 4), E_UNSUP),
                       ((1, 1, 0, 8, 4), E_SHAPE),
                       ((1, 1, 64, 8, 5), E_UNSUP), ((1, 1, 64, 65, 4), E_UNSUP),
                       ((1, 1, 64, 0, 4), E_SHAPE), ((65536, 1, 64, 8, 4), E_UNSUP)):
        assert L.race_attn_state_bytes(*args, ctypes.byref(out)) == code, args


def test_state_add_workspace(lib):
    L = _stream_lib(lib)
    out = ctypes.c_size_t(7)
    assert L.race_attn_state_add_workspace_bytes(1, 1, 0, 64, 32, 4, ctypes.byref(out)) == OK
    assert out.value == 0
    # block partials of one state each, at most about 1024 blocks in all
    assert L.race_attn_state_add_workspace_bytes(1, 1, 1 << 22, 64, 32, 4, ctypes.byref(out)) == OK
    assert out.value == 1024 * 512 * 65 * 4
    assert L.race_attn_state_add_workspace_bytes(64, 1, 100, 64, 32, 4, ctypes.byref(out)) == OK
    assert out.value == 64 * 2 * 512 * 65 * 4
    assert L.race_attn_state_add_workspace_bytes(1, 1, -1, 64, 32, 4, ctypes.byref(out)) == E_SHAPE


def test_stream_validation(lib):
    L = _stream_lib(lib)
    F = FAKE
    # state_add: nulls, tau, dtype, workspace size and alignment
    assert L.race_attn_state_add(None, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, F, F, 1 << 30, None) == E_NULL
    assert L.race_attn_state_add(F, F, None, 8, 4, 1.0, 1, 1, 0, 64, BF16, F, F, 1 << 30, None) == E_NULL
    assert L.race_attn_state_add(F, F, F, 8, 4, 0.0, 1, 1, 64, 64, BF16, F, F, 1 << 30, None) == E_TAU
    assert L.race_attn_state_add(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, 7, F, F, 1 << 30, None) == E_UNSUP
    assert L.race_attn_state_add(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, F, F, 16, None) == E_WS
    assert L.race_attn_state_add(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, F, F + 4, 1 << 30, None) == E_WS
    assert L.race_attn_state_add(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, F, None, 1 << 30, None) == E_NULL
    # N = 0 is a no-op that needs no workspace
    assert L.race_attn_state_add(F, F, F, 8, 4, 1.0, 1, 1, 0, 64, BF16, F, None, 0, None) == OK
    # decode / readout
    assert L.race_attn_decode(F, F, F, F, 8, 4, 1.0, 1, 1, 4, 64, BF16, None, F, F, None) == E_NULL
    assert L.race_attn_decode(F, F, F, F, 8, 4, float("nan"), 1, 1, 4, 64, BF16, F, F, F, None) == E_TAU
    assert L.race_attn_decode(F, F, F, F, 8, 4, 1.0, 1, 1, -1, 64, BF16, F, F, F, None) == E_SHAPE
    assert L.race_attn_decode(F, F, F, F, 8, 4, 1.0, 1, 1, 4, 128, BF16, F, F, F, None) == E_UNSUP
    assert L.race_attn_decode(None, None, None, F, 8, 4, 1.0, 1, 1, 0, 64, BF16, F, None, None, None) == OK
    assert L.race_attn_decode(F, None, F, F, 8, 4, 1.0, 1, 1, 3, 64, BF16, F, F, F, None) == E_NULL
    assert L.race_attn_state_readout(F, F, 8, 4, 1.0, 1, 1, 4, 64, BF16, F, None, F, None) == E_NULL
    assert L.race_attn_state_readout(F, F, 8, 5, 1.0, 1, 1, 4, 64, BF16, F, F, F, None) == E_UNSUP
    assert L.race_attn_state_readout(None, F, 8, 4, 1.0, 1, 1, 0, 64, BF16, F, None, None, None) == OK
    assert L.race_attn_state_readout(F, F, 8, 4, 1.0, 1, 1, 2, 64, BF16, None, F, F, None) == E_NULL


def test_backward_dw_validation(lib):
    i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    fn = lib.race_attn_backward_dw
    fn.argtypes = [vp] * 7 + [i32, i32, f32, i32, i32, i32, i64, i32, i32, i32, vp, vp, vp, vp,
                              vp, sz, vp, vp, vp]
    F = FAKE
    # the workspace with dW is larger than the plain backward's, bf16 with L <= 32 only
    st1, b1 = ws_bytes(lib, L=32, bwd=1)
    st2, b2 = ws_bytes(lib, L=32, bwd=2)
    assert st1 == OK and st2 == OK and b2 > b1
    assert ws_bytes(lib, L=32, dt=F32, bwd=2)[0] == E_UNSUP
    assert ws_bytes(lib, L=64, bwd=2)[0] == OK and ws_bytes(lib, L=64, dt=F32, bwd=2)[0] == E_UNSUP
    args = [F] * 7 + [32, 4, 1.0, 1, 1, 1, 1024, 64, BF16, 0, F, F, F, F, F * 16, 1 << 40, None,
                      None, None]
    bad = list(args)
    bad[20] = None  # dW
    assert fn(*bad) == E_NULL
    bad = list(args)
    bad[15] = F32
    assert fn(*bad) == E_UNSUP
    bad = list(args)
    bad[14] = 128  # d = 128: no dW
    assert fn(*bad) == E_UNSUP
    bad = list(args)
    bad[22] = 16  # workspace too small
    assert fn(*bad) == E_WS


def test_forward_hard_validation(lib):
    i32, i64, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    fn = lib.race_attn_forward_hard
    fn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    F = FAKE
    assert fn(None, F, F, F, 8, 4, 1, 1, 1, 64, 64, BF16, 0, F, F, F, 1 << 30, None) == E_NULL
    assert fn(F, F, F, F, 8, 7, 1, 1, 1, 64, 64, BF16, 0, F, F, F, 1 << 30, None) == E_UNSUP
    assert fn(F, F, F, F, 17, 5, 1, 1, 1, 64, 64, BF16, 0, F, F, F, 1 << 30, None) == E_UNSUP
    assert fn(F, F, F, F, 8, 5, 1, 1, 1, 64, 64, F32, 0, F, F, F, 1 << 30, None) == E_UNSUP
    # P = 5 is accepted on 16-bit rows: refused here only for the workspace
    assert fn(F, F, F, F, 8, 5, 1, 1, 1, 64, 64, BF16, 0, F, F, F * 16, 16, None) == E_WS
    assert fn(F, F, F, F, 8, 4, 1, 1, 1, 64, 64, BF16, 17, F, F, F, 1 << 30, None) == E_CHUNK
    assert fn(F, F, F, F, 8, 4, 1, 1, 1, 64, 64, BF16, 0, F, F, F * 16, 16, None) == E_WS


def test_padded_validation(lib):
    i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                             ctypes.c_size_t)
    F = FAKE
    fwd = lib.race_attn_forward_padded
    fwd.argtypes = [vp] * 4 + [i32, i32, f32, i32, i32, i32, i64, i32, i32, i32, vp, vp, vp, vp,
                               sz, vp]
    args = [F] * 4 + [8, 4, 1.0, 0, 2, 1, 1024, 64, BF16, 0, F, F, F, F * 16, 1 << 40, None]
    bad = list(args)
    bad[14] = None  # seqlens
    assert fwd(*bad) == E_NULL
    bad = list(args)
    bad[6] = 0.0  # tau
    assert fwd(*bad) == E_TAU
    bad = list(args)
    bad[18] = 16  # workspace too small
    assert fwd(*bad) == E_WS
    bad = list(args)
    bad[11] = 128  # d = 128: dense heads only
    assert fwd(*bad) == E_UNSUP
    bwd = lib.race_attn_backward_padded
    bwd.argtypes = [vp] * 7 + [i32, i32, f32, i32, i32, i32, i64, i32, i32, i32, vp, vp, vp, vp,
                               vp, vp, sz, vp]
    args = [F] * 7 + [8, 4, 1.0, 0, 2, 1, 1024, 64, BF16, 0, F, F, F, F, F, F * 16, 1 << 40,
                      None]
    bad = list(args)
    bad[17] = None  # seqlens
    assert bwd(*bad) == E_NULL
    bad = list(args)
    bad[15] = F32  # dW (not NULL) needs the fused path
    assert bwd(*bad) == E_UNSUP
    bad = list(args)
    bad[23] = 16  # workspace too small
    assert bwd(*bad) == E_WS
    # dW = NULL is allowed: then only the workspace of the plain backward is needed
    ok = list(args)
    ok[21] = None
    ok[15] = 7  # unsupported dtype code: rejected before anything is enqueued
    assert bwd(*ok) == E_UNSUP


def test_state_add_fast_validation(lib):
    L = _stream_lib(lib)
    F = FAKE
    fn = lib.race_attn_state_add_fast
    fn.argtypes = L.race_attn_state_add.argtypes
    assert fn(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, None, F, 1 << 30, None) == E_NULL
    assert fn(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, F32, F, F, 1 << 30, None) == E_UNSUP   # fp32 rows
    assert fn(F, F, F, 33, 4, 1.0, 1, 1, 64, 64, BF16, F, F, 1 << 30, None) == E_UNSUP  # L > 32
    assert fn(F, F, F, 8, 4, 0.0, 1, 1, 64, 64, BF16, F, F, 1 << 30, None) == E_TAU
    assert fn(F, F, F, 8, 4, 1.0, 1, 1, 64, 64, BF16, F, F, 16, None) == E_WS
    assert fn(None, None, F, 8, 4, 1.0, 1, 1, 0, 64, BF16, F, None, 0, None) == OK      # N = 0


def test_state_add_fast_workspace(lib):
    """for_backward = 3 sizes race_attn_state_add_fast: the segment states and
    the scan's group totals only, less than the forward's workspace (which
    also holds the keys' hash-feature cache)."""
    L = _stream_lib(lib)
    sz = ctypes.c_size_t(0)
    ws = lib.race_attn_workspace_bytes
    for (N, Lt, dt) in ((4096, 8, BF16), (1 << 20, 32, BF16), (70000, 16, 2)):
        assert ws(1, 2, N, 64, Lt, 4, 1, 0, dt, 3, ctypes.byref(sz)) == OK
        fast = sz.value
        assert ws(1, 2, N, 64, Lt, 4, 1, 0, dt, 0, ctypes.byref(sz)) == OK
        assert 0 < fast < sz.value
        fn = lib.race_attn_state_add_fast
        fn.argtypes = L.race_attn_state_add.argtypes
        assert fn(FAKE, FAKE, FAKE, Lt, 4, 1.0, 1, 2, N, 64, dt, FAKE, FAKE, fast - 1, None) == E_WS
    assert ws(1, 1, 4096, 64, 8, 4, 1, 0, F32, 3, ctypes.byref(sz)) == E_UNSUP
    assert ws(1, 1, 4096, 64, 40, 4, 1, 0, BF16, 3, ctypes.byref(sz)) == E_UNSUP
    assert ws(1, 1, 4096, 64, 8, 4, 1, 0, BF16, 5, ctypes.byref(sz)) != OK    # no such code


def test_hard_forward_workspace(lib):
    """for_backward = 4 sizes race_attn_forward_hard(_counts): on the
    bucket-id shapes the ids of Q and K (one byte per row and table) and the
    value and count states; elsewhere the soft forward's workspace."""
    sz = ctypes.c_size_t(0)
    ws = lib.race_attn_workspace_bytes
    for (N, Lt) in ((4096, 8), (1 << 20, 32), (70000, 16)):
        assert ws(1, 2, N, 64, Lt, 4, 1, 0, BF16, 4, ctypes.byref(sz)) == OK
        assert sz.value >= 2 * 2 * N * Lt    # the two id arrays
    # P = 5, 6 (16-bit rows, L 2^(P-4) <= 32): virtual tables of 16 buckets,
    # one id byte per row and virtual table
    for (Lt, P) in ((8, 5), (16, 5), (8, 6), (3, 6)):
        assert ws(1, 2, 4096, 64, Lt, P, 1, 0, BF16, 4, ctypes.byref(sz)) == OK
        assert sz.value >= 2 * 2 * 4096 * Lt * 2 ** (P - 4)
    for (Lt, P, dt) in ((17, 5, BF16), (9, 6, BF16), (8, 5, F32), (8, 7, BF16)):
        assert ws(1, 1, 4096, 64, Lt, P, 1, 0, dt, 4, ctypes.byref(sz)) == E_UNSUP
    # d = 128: the soft path only
    assert ws(1, 1, 4096, 128, 8, 4, 1, 0, BF16, 4, ctypes.byref(sz)) == E_UNSUP
    # fp32 rows: the soft kernels with t = +-1, the forward's workspace
    assert ws(1, 1, 4096, 64, 8, 4, 1, 0, F32, 4, ctypes.byref(sz)) == OK
    hard = sz.value
    assert ws(1, 1, 4096, 64, 8, 4, 1, 0, F32, 0, ctypes.byref(sz)) == OK
    assert hard == sz.value


def test_varlen_validation(lib):
    """Packed batches: cu_seqlens required, 16-bit rows only, T <= B max_seqlen."""
    f = lib.race_attn_forward_varlen
    i32, i64, f32, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    f.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i32, i64, i64, i32, i32, i32, vp, vp, vp,
                  vp, sz, vp]
    F = FAKE
    # B = 2, H = 1, T = 100, max_seqlen = 60
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 100, 60, 64, BF16, 0, None, F, F, F, 1 << 40, None) == E_NULL
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 100, 60, 64, F32, 0, F, F, F, F, 1 << 40, None) == E_UNSUP
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 100, 60, 128, BF16, 0, F, F, F, F, 1 << 40, None) == E_UNSUP
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 121, 60, 64, BF16, 0, F, F, F, F, 1 << 40, None) == E_SHAPE
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 0, 60, 64, BF16, 0, F, F, F, F, 1 << 40, None) == E_SHAPE
    assert f(F, F, F, F, 8, 4, 1.0, 1, 2, 1, 100, 60, 64, BF16, 0, F, F, F, F, 16, None) == E_WS
