"""Argument checks of the Python binding, on the CPU.

Every check runs before the library is called and before the GPU is
required, so each mistake raises its own ValueError here; correct arguments
get as far as the final "must be on a GPU" check.
"""
import pytest
import torch

from sketch_attention_soft_amd import binding

B, H, N, d, L, P = 1, 2, 40, 64, 8, 4


def _rows(dtype=torch.bfloat16, n=N, dd=d):
    return torch.zeros((B, H, n, dd), dtype=dtype)


def _args(dtype=torch.bfloat16):
    q, k, v = _rows(dtype), _rows(dtype), _rows(dtype)
    W = torch.zeros((L, P, d), dtype=torch.float32)
    return q, k, v, W


def _gpu_only(fn, *a, **kw):
    with pytest.raises(ValueError, match="on a GPU"):
        fn(*a, **kw)


def test_correct_arguments_reach_the_gpu_check():
    q, k, v, W = _args()
    _gpu_only(binding.forward, q, k, v, W, 1.0, True)
    o, den = torch.zeros_like(q), torch.ones((B, H, N))
    _gpu_only(binding.backward, q, k, v, W, o, den, q, 1.0, True)
    _gpu_only(binding.forward_hard, q, k, v, W, True)
    lens = torch.full((B,), N, dtype=torch.int32)
    _gpu_only(binding.forward_padded, q, k, v, W, lens, 1.0, True)
    _gpu_only(binding.backward_padded, q, k, v, W, o, den, q, lens, 1.0, True)


@pytest.mark.parametrize("W", [
    torch.zeros((L, P, 32)),                       # narrower than the rows: read past its end
    torch.zeros((L, P, 128)),
    torch.zeros((L, P, d), dtype=torch.float64),
    torch.zeros((L, P * d)),
    torch.zeros((L, d, P)).transpose(1, 2),        # not contiguous
], ids=["d32", "d128", "f64", "2d", "strided"])
def test_bad_w_rejected_everywhere(W):
    q, k, v, _ = _args()
    o, den = torch.zeros_like(q), torch.ones((B, H, N))
    lens = torch.full((B,), N, dtype=torch.int32)
    for call in (lambda: binding.forward(q, k, v, W, 1.0, True),
                 lambda: binding.backward(q, k, v, W, o, den, q, 1.0, True),
                 lambda: binding.backward(q, k, v, W, o, den, q, 1.0, True, dw=True),
                 lambda: binding.forward_hard(q, k, v, W, True),
                 lambda: binding.forward_padded(q, k, v, W, lens, 1.0, True),
                 lambda: binding.backward_padded(q, k, v, W, o, den, q, lens, 1.0, True)):
        with pytest.raises(ValueError, match="W must be"):
            call()


@pytest.mark.parametrize("den", [
    torch.ones((B, H, N - 1)),
    torch.ones((B, H, N), dtype=torch.bfloat16),
    torch.ones((B, H, 2 * N))[..., ::2],
], ids=["short", "bf16", "strided"])
def test_bad_den_rejected(den):
    q, k, v, W = _args()
    o = torch.zeros_like(q)
    lens = torch.full((B,), N, dtype=torch.int32)
    with pytest.raises(ValueError, match="den must be"):
        binding.backward(q, k, v, W, o, den, q, 1.0, True)
    with pytest.raises(ValueError, match="den must be"):
        binding.backward_padded(q, k, v, W, o, den, q, lens, 1.0, True)


def test_bad_forward_outputs_rejected():
    q, k, v, W = _args()
    good_o, good_den = torch.zeros_like(q), torch.zeros((B, H, N))
    for o, den, what in ((_rows(torch.float32), good_den, "o must be"),
                         (_rows(n=N - 1), good_den, "o must be"),
                         (good_o, torch.zeros((B, H, N - 1)), "den must be"),
                         (good_o, torch.zeros((B, H, N), dtype=torch.float16), "den must be")):
        with pytest.raises(ValueError, match=what):
            binding.forward(q, k, v, W, 1.0, True, out=(o, den))
        with pytest.raises(ValueError, match=what):
            binding.forward_hard(q, k, v, W, True, out=(o, den))


def test_bad_backward_outputs_rejected():
    q, k, v, W = _args()
    o, den = torch.zeros_like(q), torch.ones((B, H, N))
    good = torch.zeros_like(q)
    for i, name in enumerate(("dq", "dk", "dv")):
        outs = [good, good, good]
        outs[i] = _rows(torch.float16)
        with pytest.raises(ValueError, match=f"{name} must be"):
            binding.backward(q, k, v, W, o, den, q, 1.0, True, out=tuple(outs))
        outs[i] = _rows(n=N + 1)
        with pytest.raises(ValueError, match=f"{name} must be"):
            binding.backward(q, k, v, W, o, den, q, 1.0, True, out=tuple(outs))


def test_saved_buffer_checked():
    q, k, v, W = _args()
    o, den = torch.zeros_like(q), torch.ones((B, H, N))
    need = binding.saved_bytes(B, H, N, d, L, P, True, 0, q.dtype)
    assert need > 0
    for bad in (torch.zeros(need - 1, dtype=torch.uint8),
                torch.zeros(need, dtype=torch.float32),
                torch.zeros(2 * need, dtype=torch.uint8)[::2]):
        with pytest.raises(ValueError, match="saved must be"):
            binding.forward(q, k, v, W, 1.0, True, saved=bad)
        with pytest.raises(ValueError, match="saved must be"):
            binding.backward(q, k, v, W, o, den, q, 1.0, True, saved=bad)
    _gpu_only(binding.forward, q, k, v, W, 1.0, True, saved=torch.zeros(need, dtype=torch.uint8))


def test_stream_entry_points_checked():
    q, k, v, W = _args()
    state = binding.new_state(B, H, d, L, P, "cpu")
    with pytest.raises(ValueError, match="W must be"):
        binding.decode(state, q, k, v, torch.zeros((L, P, 32)), 1.0)
    with pytest.raises(ValueError, match="W must be"):
        binding.state_readout(state, q, torch.zeros((L, P, 32)), 1.0)
    with pytest.raises(ValueError, match="W must be"):
        binding.state_add(state, k, v, torch.zeros((L, P, 32)), 1.0)
    with pytest.raises(ValueError, match="o must be"):
        binding.decode(state, q, k, v, W, 1.0, out=(_rows(n=N - 1), torch.zeros((B, H, N))))
    with pytest.raises(ValueError, match="den must be"):
        binding.state_readout(state, q, W, 1.0, out=(torch.zeros_like(q), torch.zeros((B, H))))
    _gpu_only(binding.decode, state, q, k, v, W, 1.0)
    _gpu_only(binding.state_readout, state, q, W, 1.0)
    _gpu_only(binding.state_add, state, k, v, W, 1.0)


def test_mismatched_rows_rejected():
    q, k, v, W = _args()
    with pytest.raises(ValueError, match="share shape"):
        binding.forward(q, k[..., :N - 1, :], v, W, 1.0, True)
    with pytest.raises(ValueError, match="share shape"):
        binding.forward(q, k.float(), v, W, 1.0, True)


def test_varlen_checks():
    H, T = 2, 50
    q = torch.zeros((H, T, d), dtype=torch.bfloat16)
    W = torch.zeros((L, P, d), dtype=torch.float32)
    cu = torch.tensor([0, 20, 50], dtype=torch.int32)
    _gpu_only(binding.forward_varlen, q, q, q, W, cu, 30, 1.0, True)
    with pytest.raises(ValueError, match="cu_seqlens"):
        binding.forward_varlen(q, q, q, W, cu.long(), 30, 1.0, True)
    with pytest.raises(ValueError, match="packed"):
        binding.forward_varlen(q[None], q[None], q[None], W, cu, 30, 1.0, True)
    den = torch.ones((H, T))
    _gpu_only(binding.backward_varlen, q, q, q, W, q, den, q, cu, 30, 1.0, True)
    with pytest.raises(ValueError, match="den must be"):
        binding.backward_varlen(q, q, q, W, q, den[:, 1:], q, cu, 30, 1.0, True)
