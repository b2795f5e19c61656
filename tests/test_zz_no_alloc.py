"""m2rnn_gate_rmsnorm_backward_noalloc, the allocation-free variant of the
output-gate + RMSNorm backward (slide "Backup: RMSNormTP synchronizes
per-token statistics", paper App. C), called through the C ABI: its dy, dg
and dw must equal those of m2rnn_gate_rmsnorm_backward on the same inputs,
bit for bit (the two share their kernels; only where the dw partial sums
live differs).  Two calls in a row share the library's scratch array, the
second with a smaller input, so stale partials of the first would show."""
import ctypes

import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def run_pair(B, T, N, dtype, eps, seed):
    print(f"noalloc case B{B} T{T} N{N} {dtype} eps {eps}", flush=True)
    x = {k: v.cuda() for k, v in m2rnn_inputs.make_epilogue(B, T, N, dtype, seed=seed).items()}
    ref = m2.gate_rmsnorm_backward(x["y"], x["g"], x["w"], x["dout"], eps=eps)
    dy = torch.full_like(x["y"], float("nan"))
    dg = torch.full_like(x["y"], float("nan"))
    dw = torch.full((N * 16,), float("nan"), device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = m2.lib.m2rnn_gate_rmsnorm_backward_noalloc(B, T, N, 16, m2.M2RNN_BF16 if dtype == "bf16" else m2.M2RNN_F32,
                                                    _p(x["y"]), _p(x["g"]), _p(x["w"]), ctypes.c_float(eps),
                                                    _p(x["dout"]), _p(dy), _p(dg), _p(dw), stream)
    assert st == m2.M2RNN_OK, m2.m2rnn_last_error()
    torch.cuda.synchronize()
    for name, got, want in (("dy", dy, ref[0]), ("dg", dg, ref[1]), ("dw", dw, ref[2])):
        assert torch.equal(got, want), name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    # the largest scratch use first (1024 dw partial rows of d = 2048), then a smaller call
    run_pair(2, 2048, 128, dtype, 0.0, seed=3)
    run_pair(2, 50, 16, dtype, 1e-3, seed=4)


def test_noalloc_repeated_small_after_large():
    run_pair(4, 300, 64, "bf16", 0.0, seed=5)
    run_pair(1, 7, 4, "bf16", 0.0, seed=6)
    run_pair(1, 7, 4, "bf16", 0.0, seed=6)
