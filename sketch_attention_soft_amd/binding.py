"""Thin ctypes binding of librace_attn.so (declared in include/race_attn.h).

Argument marshalling only: shape/dtype/device checks, workspace allocation
through torch, and the current HIP stream.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librace_attn.so")

RACE_F32, RACE_BF16, RACE_F16 = 0, 1, 2
STATUS = {
    0: "RACE_OK", 1: "RACE_ERR_NULL", 2: "RACE_ERR_SHAPE", 3: "RACE_ERR_UNSUPPORTED",
    4: "RACE_ERR_TAU", 5: "RACE_ERR_CHUNK", 6: "RACE_ERR_WORKSPACE", 7: "RACE_ERR_HIP",
}
EXPORTS = ("race_attn_workspace_bytes", "race_attn_saved_bytes", "race_attn_forward",
           "race_attn_backward", "race_attn_forward_ex", "race_attn_backward_ex",
           "race_attn_backward_dw", "race_attn_forward_hard", "race_attn_forward_padded",
           "race_attn_backward_padded",
           "race_attn_squash_coeffs", "race_attn_squash_deriv_coeffs",
           "race_attn_state_bytes", "race_attn_state_add_workspace_bytes", "race_attn_state_add",
           "race_attn_state_add_fast",
           "race_attn_decode", "race_attn_state_readout", "race_attn_status_string",
           "race_attn_forward_noalloc", "race_attn_forward_varlen", "race_attn_backward_varlen",
           "race_attn_hash_ids_workspace_bytes", "race_attn_hash_ids",
           "race_attn_forward_hard_counts")
TRACE_MAX = 24


class _RaceTrace(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int), ("count", ctypes.c_int),
                ("start", ctypes.c_void_p * TRACE_MAX), ("stop", ctypes.c_void_p * TRACE_MAX),
                ("name", ctypes.c_char_p * TRACE_MAX)]


class Trace:
    """Caller-owned HIP events that the *_ex entry points record around
    every kernel they enqueue (see race_trace_t in include/race_attn.h)."""

    def __init__(self, capacity: int = TRACE_MAX):
        self.events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(capacity)]
        for a, b in self.events:  # materialise the underlying hipEvent_t
            a.record()
            b.record()
        self.st = _RaceTrace()
        self.st.capacity = capacity
        for i, (a, b) in enumerate(self.events):
            self.st.start[i] = a.cuda_event
            self.st.stop[i] = b.cuda_event

    def results(self):
        """[(kernel name, milliseconds)] of the last traced call (after a sync)."""
        return [(self.st.name[i].decode(), self.events[i][0].elapsed_time(self.events[i][1]))
                for i in range(self.st.count)]

_lib = None


class RaceError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def lib():
    """Load librace_attn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, f32, vp, sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                 ctypes.c_size_t)
        L.race_attn_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32, i32,
                                                ctypes.POINTER(sz)]
        L.race_attn_workspace_bytes.restype = i32
        L.race_attn_forward.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i32, i64, i32,
                                        i32, i32, vp, vp, vp, sz, vp]
        L.race_attn_forward.restype = i32
        L.race_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, i32, i32, i32,
                                         i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.race_attn_backward.restype = i32
        L.race_attn_forward_hard.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i32,
                                             i32, i32, vp, vp, vp, sz, vp]
        L.race_attn_forward_hard.restype = i32
        L.race_attn_forward_hard_counts.argtypes = L.race_attn_forward_hard.argtypes[:15] + [vp, vp, sz, vp]
        L.race_attn_forward_hard_counts.restype = i32
        L.race_attn_saved_bytes.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(sz)]
        L.race_attn_saved_bytes.restype = i32
        tp = ctypes.POINTER(_RaceTrace)
        L.race_attn_forward_ex.argtypes = L.race_attn_forward.argtypes + [vp, tp]
        L.race_attn_forward_ex.restype = i32
        L.race_attn_backward_ex.argtypes = L.race_attn_backward.argtypes + [vp, tp]
        L.race_attn_backward_ex.restype = i32
        L.race_attn_backward_dw.argtypes = (L.race_attn_backward.argtypes[:20] + [vp]
                                            + L.race_attn_backward.argtypes[20:] + [vp, tp])
        L.race_attn_backward_dw.restype = i32
        L.race_attn_forward_padded.argtypes = (L.race_attn_forward.argtypes[:14] + [vp]
                                               + L.race_attn_forward.argtypes[14:])
        L.race_attn_forward_padded.restype = i32
        L.race_attn_backward_padded.argtypes = (L.race_attn_backward.argtypes[:17] + [vp]
                                                + L.race_attn_backward.argtypes[17:20] + [vp]
                                                + L.race_attn_backward.argtypes[20:])
        L.race_attn_backward_padded.restype = i32
        L.race_attn_forward_varlen.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i32, i64,
                                               i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.race_attn_forward_varlen.restype = i32
        L.race_attn_backward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, f32, i32,
                                                i32, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp,
                                                vp, vp, sz, vp]
        L.race_attn_backward_varlen.restype = i32
        L.race_attn_hash_ids_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
        L.race_attn_hash_ids_workspace_bytes.restype = i32
        L.race_attn_hash_ids.argtypes = [vp, i64, i32, i32, vp, i32, i32, vp, vp, sz, vp]
        L.race_attn_hash_ids.restype = i32
        L.race_attn_state_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
        L.race_attn_state_bytes.restype = i32
        L.race_attn_state_add_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32,
                                                          ctypes.POINTER(sz)]
        L.race_attn_state_add_workspace_bytes.restype = i32
        L.race_attn_state_add.argtypes = [vp, vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                          vp, sz, vp]
        L.race_attn_state_add.restype = i32
        L.race_attn_state_add_fast.argtypes = L.race_attn_state_add.argtypes
        L.race_attn_state_add_fast.restype = i32
        L.race_attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                       vp, vp, vp]
        L.race_attn_decode.restype = i32
        L.race_attn_state_readout.argtypes = [vp, vp, i32, i32, f32, i32, i32, i64, i32, i32, vp,
                                              vp, vp, vp]
        L.race_attn_state_readout.restype = i32
        L.race_attn_forward_noalloc.argtypes = L.race_attn_forward.argtypes[:16] + [vp]
        L.race_attn_forward_noalloc.restype = i32
        L.race_attn_status_string.argtypes = [i32]
        L.race_attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(code: int) -> None:
    if code != 0:
        raise RaceError(code, lib().race_attn_status_string(code).decode())


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return RACE_F32
    if dtype == torch.bfloat16:
        return RACE_BF16
    if dtype == torch.float16:
        return RACE_F16
    raise TypeError(f"unsupported dtype {dtype}")


def workspace_bytes(B, H, N, d, L, P, causal, chunk, dtype, for_backward) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_workspace_bytes(B, H, N, d, L, P, int(causal), chunk,
                                           dtype_code(dtype), int(for_backward),
                                           ctypes.byref(out)))
    return out.value


def saved_bytes(B, H, N, d, L, P, causal, chunk, dtype) -> int:
    """Bytes of the key-state buffer a forward can save for its backward (0: unused)."""
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_saved_bytes(B, H, N, d, L, P, int(causal), chunk, dtype_code(dtype),
                                       ctypes.byref(out)))
    return out.value


def new_saved(q: torch.Tensor, W: torch.Tensor, causal: bool, chunk: int = 0):
    """A saved-state buffer for forward(..., saved=) / backward(..., saved=), or None."""
    B, H, N, d = q.shape
    L, P, _ = W.shape
    n = saved_bytes(B, H, N, d, L, P, causal, chunk, q.dtype)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _shape(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return q.shape


def _check_tensors(ref: torch.Tensor, *ts: torch.Tensor) -> None:
    for t in ts:
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("Q, K, V (and O, dO) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _require_gpu(ref: torch.Tensor) -> None:
    """Last check before the library is called: every argument check above
    it runs on any device, so that mistakes are reported the same way
    everywhere."""
    if ref.device.type != "cuda":
        raise ValueError("tensors must be on a GPU")


def _check_out(t, shape, dtype, device, name):
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or t.device != device or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device}")


def _outputs_fwd(q, out, alloc=torch.empty):
    """(o, den) for a forward or readout over the rows of q: new, or out checked."""
    B, H, N, _ = q.shape
    if out is None:
        return alloc(q.shape, dtype=q.dtype, device=q.device), alloc(
            (B, H, N), dtype=torch.float32, device=q.device)
    o, den = out
    _check_out(o, q.shape, q.dtype, q.device, "o")
    _check_out(den, (B, H, N), torch.float32, q.device, "den")
    return o, den


def _outputs_bwd(q, out, alloc):
    if out is None:
        return alloc(q), alloc(q), alloc(q)
    for t, n in zip(out, ("dq", "dk", "dv")):
        _check_out(t, q.shape, q.dtype, q.device, n)
    return tuple(out)


def _check_den(den, q):
    B, H, N, _ = q.shape
    _check_out(den, (B, H, N), torch.float32, q.device, "den")


def _check_saved(saved, B, H, N, d, L, P, causal, chunk, q):
    """A saved-state buffer must be a uint8 device tensor of at least
    saved_bytes(...) bytes (the library cannot check its size)."""
    if saved is None:
        return
    need = saved_bytes(B, H, N, d, L, P, causal, chunk, q.dtype)
    if (not isinstance(saved, torch.Tensor) or saved.dtype != torch.uint8
            or saved.device != q.device or not saved.is_contiguous() or saved.numel() < need):
        raise ValueError(f"saved must be a contiguous uint8 tensor of at least {need} bytes "
                         f"on {q.device} (new_saved)")


def _workspace(ws, nbytes, device):
    """The caller's workspace as bytes when it is a contiguous tensor on the
    device with at least nbytes bytes, else a new one."""
    if (ws is not None and ws.device == device and ws.is_contiguous()
            and ws.numel() * ws.element_size() >= nbytes):
        return ws.reshape(-1).view(torch.uint8)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _tp(trace):
    return ctypes.byref(trace.st) if trace is not None else None


def forward(q, k, v, W, tau: float, causal: bool, chunk: int = 0, workspace=None, out=None,
            trace: Trace | None = None, saved=None):
    """RACE attention forward; returns (o, den).  out = (o, den) reuses buffers;
    saved (from new_saved) receives the key state for the backward."""
    B, H, N, d = _shape(q)
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    o, den = _outputs_fwd(q, out)
    _check_saved(saved, B, H, N, d, L, P, causal, chunk, q)
    nbytes = workspace_bytes(B, H, N, d, L, P, causal, chunk, q.dtype, False)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib().race_attn_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), L,
                                      P, float(tau), int(causal), B, H, N, d,
                                      dtype_code(q.dtype), chunk, o.data_ptr(), den.data_ptr(),
                                      workspace.data_ptr(), workspace.numel(), _stream(),
                                      _ptr(saved), _tp(trace)))
    return o, den


def forward_noalloc(q, k, v, W, tau: float, causal: bool, chunk: int = 0, out=None):
    """race_attn_forward_noalloc: the forward with the library's per-GPU scratch
    array as its workspace (nothing is allocated for it); returns (o, den).
    Calls on one GPU share that array and must not overlap."""
    B, H, N, d = _shape(q)
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    o, den = _outputs_fwd(q, out)
    _require_gpu(q)
    _check(lib().race_attn_forward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           W.data_ptr(), L, P, float(tau), int(causal), B, H, N,
                                           d, dtype_code(q.dtype), chunk, o.data_ptr(),
                                           den.data_ptr(), _stream()))
    return o, den


NOALLOC_SCRATCH_BYTES = 128 << 20


def forward_hard(q, k, v, W, causal: bool, chunk: int = 0, workspace=None, out=None,
                 counts: bool = False):
    """Hard-hash forward (one bucket per table and row, true counts): (o, den),
    and the int32 counts last with counts=True (race_attn_forward_hard_counts)."""
    B, H, N, d = _shape(q)
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    o, den = _outputs_fwd(q, out)
    cnt = torch.empty((B, H, N), dtype=torch.int32, device=q.device) if counts else None
    nbytes = workspace_bytes(B, H, N, d, L, P, causal, chunk, q.dtype, 4)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), L, P, int(causal), B, H, N, d,
            dtype_code(q.dtype), chunk, o.data_ptr(), den.data_ptr())
    if counts:
        _check(lib().race_attn_forward_hard_counts(*args, cnt.data_ptr(), workspace.data_ptr(),
                                                   workspace.numel(), _stream()))
        return o, den, cnt
    _check(lib().race_attn_forward_hard(*args, workspace.data_ptr(), workspace.numel(), _stream()))
    return o, den


def backward(q, k, v, W, o, den, do, tau: float, causal: bool, chunk: int = 0, workspace=None,
             out=None, trace: Trace | None = None, saved=None, dw: bool = False):
    """RACE attention backward; returns (dq, dk, dv), and dW last with dw=True
    (race_attn_backward_dw: bf16 or fp16 rows).  out = (dq, dk, dv) reuses buffers;
    saved: the buffer the forward of the same inputs filled, or None."""
    B, H, N, d = _shape(q)
    _check_tensors(q, k, v, o, do)
    _check_den(den, q)
    L, P = _check_w(W, q)
    _check_saved(saved, B, H, N, d, L, P, causal, chunk, q)
    dq, dk, dv = _outputs_bwd(q, out, torch.empty_like)
    nbytes = workspace_bytes(B, H, N, d, L, P, causal, chunk, q.dtype, 2 if dw else 1)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    if dw:
        gW = torch.empty_like(W)
        _check(lib().race_attn_backward_dw(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), o.data_ptr(), den.data_ptr(),
            do.data_ptr(), L, P, float(tau), int(causal), B, H, N, d, dtype_code(q.dtype), chunk,
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), gW.data_ptr(), workspace.data_ptr(),
            workspace.numel(), _stream(), _ptr(saved), _tp(trace)))
        return dq, dk, dv, gW
    _check(lib().race_attn_backward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(),
                                       o.data_ptr(), den.data_ptr(), do.data_ptr(), L, P,
                                       float(tau), int(causal), B, H, N, d, dtype_code(q.dtype),
                                       chunk, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       workspace.data_ptr(), workspace.numel(), _stream(),
                                       _ptr(saved), _tp(trace)))
    return dq, dk, dv


def _check_lens(seqlens, q):
    B = q.shape[0]
    if (seqlens.dtype != torch.int32 or seqlens.shape != (B,) or not seqlens.is_contiguous()
            or seqlens.device != q.device):
        raise ValueError("seqlens must be a contiguous int32 [B] tensor on the same device")


def padded_chunk(B: int, H: int, N: int) -> int:
    """Segment length for right-padded batches: about eight segments per compute
    unit over the padded rows (the library's default aims at one), so that
    sequences of unequal lengths leave few workgroups without work (best of
    2, 4, 8 and 16 per unit for four sequences of 4M to 1M tokens)."""
    return max(64, -(-(B * H * N) // 2048 // 32) * 32)


def forward_padded(q, k, v, W, seqlens, tau: float, causal: bool, chunk: int | None = None,
                   workspace=None, out=None):
    """Forward over right-padded batches: batch b has seqlens[b] rows.  Returns
    (o, den) with zeros on the padding rows (out = (o, den): buffers to reuse,
    whose padding rows are left as they are).  chunk None: padded_chunk."""
    B, H, N, d = _shape(q)
    chunk = padded_chunk(B, H, N) if chunk is None else chunk
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    _check_lens(seqlens, q)
    o, den = _outputs_fwd(q, out, torch.zeros)
    nbytes = workspace_bytes(B, H, N, d, L, P, causal, chunk, q.dtype, False)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib().race_attn_forward_padded(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(),
                                          L, P, float(tau), int(causal), B, H, N, d,
                                          dtype_code(q.dtype), chunk, seqlens.data_ptr(),
                                          o.data_ptr(), den.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream()))
    return o, den


def backward_padded(q, k, v, W, o, den, do, seqlens, tau: float, causal: bool,
                    chunk: int | None = None, workspace=None, dw: bool = False, out=None):
    """Backward over right-padded batches; returns (dq, dk, dv) with zeros on
    the padding rows, and dW last with dw=True (out = (dq, dk, dv): buffers to
    reuse, whose padding rows are left as they are).  chunk None: padded_chunk
    (it must be the forward's)."""
    B, H, N, d = _shape(q)
    chunk = padded_chunk(B, H, N) if chunk is None else chunk
    _check_tensors(q, k, v, o, do)
    L, P = _check_w(W, q)
    _check_den(den, q)
    _check_lens(seqlens, q)
    dq, dk, dv = _outputs_bwd(q, out, torch.zeros_like)
    gW = torch.empty_like(W) if dw else None
    nbytes = workspace_bytes(B, H, N, d, L, P, causal, chunk, q.dtype, 2 if dw else 1)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib().race_attn_backward_padded(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), o.data_ptr(), den.data_ptr(),
        do.data_ptr(), L, P, float(tau), int(causal), B, H, N, d, dtype_code(q.dtype), chunk,
        seqlens.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _ptr(gW),
        workspace.data_ptr(), workspace.numel(), _stream()))
    return (dq, dk, dv, gW) if dw else (dq, dk, dv)


def _check_cu(cu_seqlens, T, ref):
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or not cu_seqlens.is_contiguous()
            or cu_seqlens.device != ref.device):
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor on the rows' device")
    return cu_seqlens.numel() - 1


def _packed_shape(q):
    if q.dim() != 3:
        raise ValueError("packed batches take [H, T, d] tensors")
    return q.shape


def forward_varlen(q, k, v, W, cu_seqlens, max_seqlen: int, tau: float, causal: bool,
                   chunk: int | None = None, workspace=None, out=None):
    """Forward over packed batches: q, k, v [H, T, d], sequence b at rows
    cu_seqlens[b] .. cu_seqlens[b + 1] of every head, none longer than
    max_seqlen.  Returns (o [H, T, d], den [H, T]).  chunk None: padded_chunk."""
    H, T, d = _packed_shape(q)
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    B = _check_cu(cu_seqlens, T, q)
    chunk = padded_chunk(B, H, max_seqlen) if chunk is None else chunk
    if out is None:
        o = torch.empty_like(q)
        den = torch.empty((H, T), dtype=torch.float32, device=q.device)
    else:
        o, den = out
        _check_out(o, q.shape, q.dtype, q.device, "o")
        _check_out(den, (H, T), torch.float32, q.device, "den")
    nbytes = workspace_bytes(B, H, max_seqlen, d, L, P, causal, chunk, q.dtype, False)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib().race_attn_forward_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(),
                                          L, P, float(tau), int(causal), B, H, T, int(max_seqlen),
                                          d, dtype_code(q.dtype), chunk, cu_seqlens.data_ptr(),
                                          o.data_ptr(), den.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream()))
    return o, den


def backward_varlen(q, k, v, W, o, den, do, cu_seqlens, max_seqlen: int, tau: float,
                    causal: bool, chunk: int | None = None, workspace=None, dw: bool = False,
                    out=None):
    """Backward over packed batches ([H, T, d] tensors, den [H, T]); returns
    (dq, dk, dv), and dW last with dw=True.  chunk None: padded_chunk (it must
    be the forward's)."""
    H, T, d = _packed_shape(q)
    _check_tensors(q, k, v, o, do)
    L, P = _check_w(W, q)
    B = _check_cu(cu_seqlens, T, q)
    _check_out(den, (H, T), torch.float32, q.device, "den")
    chunk = padded_chunk(B, H, max_seqlen) if chunk is None else chunk
    dq, dk, dv = _outputs_bwd(q, out, torch.empty_like)
    gW = torch.empty_like(W) if dw else None
    nbytes = workspace_bytes(B, H, max_seqlen, d, L, P, causal, chunk, q.dtype, 2 if dw else 1)
    _require_gpu(q)
    workspace = _workspace(workspace, nbytes, q.device)
    _check(lib().race_attn_backward_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), o.data_ptr(), den.data_ptr(),
        do.data_ptr(), L, P, float(tau), int(causal), B, H, T, int(max_seqlen),
        d, dtype_code(q.dtype), chunk, cu_seqlens.data_ptr(), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), _ptr(gW), workspace.data_ptr(), workspace.numel(), _stream()))
    return (dq, dk, dv, gW) if dw else (dq, dk, dv)


def hash_ids(x, W, workspace=None, out=None):
    """Hard-hash bucket ids of the rows of x (any shape [..., d]): uint8
    [..., L], ids[..., l] = sum_p [u_lp >= 0] 2^p with u = W x
    (race_attn_hash_ids)."""
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [..., d] tensor")
    L, P = _check_w(W, x)
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if out is None:
        ids = torch.empty((*x.shape[:-1], L), dtype=torch.uint8, device=x.device)
    else:
        ids = out
        _check_out(ids, (*x.shape[:-1], L), torch.uint8, x.device, "ids")
    nb = ctypes.c_size_t(0)
    _check(lib().race_attn_hash_ids_workspace_bytes(L, P, d, ctypes.byref(nb)))
    _require_gpu(x)
    workspace = _workspace(workspace, nb.value, x.device)
    _check(lib().race_attn_hash_ids(x.data_ptr(), rows, d, dtype_code(x.dtype), W.data_ptr(), L, P,
                                    ids.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                    _stream()))
    return ids


class RaceAttention(torch.autograd.Function):
    """Autograd wrapper: o = race_attention(q, k, v, W).  W gets a gradient when
    it requires one (learned hyperplanes; bf16 or fp16 inputs)."""

    @staticmethod
    def forward(ctx, q, k, v, W, tau, causal, chunk=0):
        saved = new_saved(q, W, causal, chunk)
        o, den = forward(q, k, v, W, tau, causal, chunk, saved=saved)
        ctx.save_for_backward(q, k, v, W, o, den)
        ctx.key_state = saved
        ctx.cfg = (tau, causal, chunk)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, W, o, den = ctx.saved_tensors
        tau, causal, chunk = ctx.cfg
        grads = backward(q, k, v, W, o, den, do.contiguous(), tau, causal, chunk,
                         saved=ctx.key_state, dw=ctx.needs_input_grad[3])
        ctx.key_state = None
        dW = grads[3] if ctx.needs_input_grad[3] else None
        return grads[0], grads[1], grads[2], dW, None, None, None


def race_attention(q, k, v, W, tau: float = 1.0, causal: bool = True, chunk: int = 0):
    return RaceAttention.apply(q, k, v, W, tau, causal, chunk)


class RaceAttentionLayer(torch.nn.Module):
    """Drop-in attention core on [B, H, N, d] tensors: o = race_attention(q, k, v, W)
    with W [L, P, d] drawn from N(0, 1) (the pages' random hyperplanes), kept as a
    buffer, or as a parameter with learn_projection=True (bf16 or fp16)."""

    def __init__(self, d: int = 64, L: int = 32, P: int = 4, tau: float = 1.0,
                 causal: bool = True, chunk: int = 0, learn_projection: bool = False,
                 generator: torch.Generator | None = None):
        super().__init__()
        W = torch.randn((L, P, d), generator=generator, dtype=torch.float32)
        if learn_projection:
            self.W = torch.nn.Parameter(W)
        else:
            self.register_buffer("W", W)
        self.tau, self.causal, self.chunk = tau, causal, chunk

    def forward(self, q, k, v):
        return RaceAttention.apply(q, k, v, self.W.contiguous(), self.tau, self.causal, self.chunk)


# ---------------------------------------------------------------------------
# Streaming state (race_attn_state_* / race_attn_decode in include/race_attn.h)

def _check_w(W, ref):
    """W must be a contiguous fp32 [L, P, d] tensor on the rows' device, with
    d the rows' width (the library takes no width for W)."""
    if (W.dtype != torch.float32 or W.dim() != 3 or not W.is_contiguous()
            or W.device != ref.device or W.shape[2] != ref.shape[-1]):
        raise ValueError("W must be a contiguous fp32 [L, P, d] tensor on the rows' device, "
                         "with d the rows' width")
    return W.shape[0], W.shape[1]


def state_bytes(B, H, d, L, P) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_state_bytes(B, H, d, L, P, ctypes.byref(out)))
    return out.value


def new_state(B, H, d, L, P, device) -> torch.Tensor:
    """Zeroed states [B, H, 16 L, d + 1] (fp32): the empty prefix of every head."""
    state_bytes(B, H, d, L, P)  # validates the shape
    return torch.zeros((B, H, 16 * L, d + 1), dtype=torch.float32, device=device)


def _check_state(state, B, H, d, L, P, ref):
    if (state.dtype != torch.float32 or state.shape != (B, H, 16 * L, d + 1)
            or not state.is_contiguous() or state.device != ref.device):
        raise ValueError("state must be a contiguous fp32 [B, H, 16 L, d + 1] tensor")


def state_add_workspace_bytes(B, H, N, d, L, P) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().race_attn_state_add_workspace_bytes(B, H, N, d, L, P, ctypes.byref(out)))
    return out.value


def state_add(state, k, v, W, tau: float, workspace=None, fast: bool = False):
    """state += the sums of the rows of k, v ([B, H, N, d]); returns state.
    fast: through the fused matrix-core kernels (race_attn_state_add_fast:
    bf16 / fp16 rows, L <= 32; the forward's bf16 precision)."""
    B, H, N, d = _shape(k)
    _check_tensors(k, v)
    L, P = _check_w(W, k)
    _check_state(state, B, H, d, L, P, k)
    if fast:
        nbytes = workspace_bytes(B, H, max(N, 1), d, L, P, True, 0, k.dtype, 3)
        fn = lib().race_attn_state_add_fast
    else:
        nbytes = state_add_workspace_bytes(B, H, N, d, L, P)
        fn = lib().race_attn_state_add
    _require_gpu(k)
    workspace = _workspace(workspace, nbytes, k.device)
    _check(fn(k.data_ptr(), v.data_ptr(), W.data_ptr(), L, P, float(tau), B, H, N, d,
              dtype_code(k.dtype), state.data_ptr(), workspace.data_ptr(), workspace.numel(),
              _stream()))
    return state


def decode(state, q, k, v, W, tau: float, out=None):
    """Appends the T tokens of q, k, v ([B, H, T, d]) to state in order; returns
    their causal outputs (o, den)."""
    B, H, T, d = _shape(q)
    _check_tensors(q, k, v)
    L, P = _check_w(W, q)
    _check_state(state, B, H, d, L, P, q)
    o, den = _outputs_fwd(q, out)
    _require_gpu(q)
    _check(lib().race_attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), W.data_ptr(), L, P,
                                  float(tau), B, H, T, d, dtype_code(q.dtype), state.data_ptr(),
                                  o.data_ptr(), den.data_ptr(), _stream()))
    return o, den


def state_readout(state, q, W, tau: float, out=None):
    """Readout of the rows of q ([B, H, T, d]) from state (not modified): (o, den)."""
    B, H, T, d = _shape(q)
    _check_tensors(q)
    L, P = _check_w(W, q)
    _check_state(state, B, H, d, L, P, q)
    o, den = _outputs_fwd(q, out)
    _require_gpu(q)
    _check(lib().race_attn_state_readout(q.data_ptr(), W.data_ptr(), L, P, float(tau), B, H, T,
                                         d, dtype_code(q.dtype), state.data_ptr(), o.data_ptr(),
                                         den.data_ptr(), _stream()))
    return o, den
