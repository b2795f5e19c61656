"""Forward scan on the GPU (through the C ABI) against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
from gpu_common import TOL, batch_rows, chain_slice, make, max_abs, oracle_forward, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def run(x, ckpt_every=0):
    g = to_gpu(x)
    out = m2.forward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], ckpt_every=ckpt_every)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N", [(1, 256, 4), (2, 100, 5), (3, 37, 1), (1, 65, 2), (2, 33, 3), (1, 1, 4)])
def test_forward_parity_small(dtype, B, T, N):
    """Shapes spanning several 32-step chunks with a ragged tail, and head
    counts that do not fill a 4-head workgroup."""
    x = make(B, T, N, dtype, seed=B * 1000 + T + N)
    y, HT = run(x)
    yr, HTr = oracle_forward(x)
    ey, eh = max_abs(y, yr), max_abs(HT, HTr)
    print(f"{dtype} B{B} T{T} N{N}: max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N", [(2, 70, 64), (1, 101, 128), (1, 45, 129), (1, 70, 512), (3, 40, 201),
                                   (2, 20, 801), (1, 45, 1600)])
def test_forward_parity_launch_shapes(dtype, B, T, N):
    """Chain counts B*N in each launch shape the forward picks: at most 128
    (the row-split forward, one state element per lane, four workgroups per
    head; 128 is its largest), up to 512 (one head per workgroup, one tile per
    wave; 129 its smallest), up to 1536 (two heads of two waves each, with a
    head count that leaves the last workgroup half empty) and above (four
    heads, one per wave, the last group partly empty)."""
    x = make(B, T, N, dtype, seed=B * 7 + T + N)
    y, HT = run(x)
    yr, HTr = oracle_forward(x)
    ey, eh = max_abs(y, yr), max_abs(HT, HTr)
    print(f"{dtype} B{B} T{T} N{N} (B*N={B * N}): max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def test_forward_bf16_weight_range():
    """bf16 W of order 1e-5 with entries down to 5e-7, below fp16's normal
    range, where the fp16 A operand rounds to within 2^-25: y and H_T still
    meet the bf16 bar.  (Large W is no test of precision: the saturated
    recurrence then amplifies any rounding difference, the oracle's own
    included.)"""
    x = make(2, 100, 5, "bf16", seed=43)
    W = x["W"].float() * 1e-5
    W[0, 0, :4] = torch.tensor([1e-6, -3e-6, 5e-7, 2e-5])   # below 2^-14
    x["W"] = W.to(torch.bfloat16)
    y, HT = run(x)
    yr, HTr = oracle_forward(x)
    ey, eh = max_abs(y, yr), max_abs(HT, HTr)
    print(f"bf16 small W: max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
    assert ey <= TOL["bf16"] and eh <= TOL["bf16"]


def test_forward_config_fp32_B1_T256_N4():
    """The float32 workload B=1, T=256, N=4 (seed 0), element by element."""
    w = m2rnn_inputs.WORKLOADS["fwd_f32_B1_T256_N4"]
    x = m2rnn_inputs.make_workload(w)
    y, HT = run(x)
    yr, HTr = oracle_forward(x)
    ey, eh = max_abs(y, yr), max_abs(HT, HTr)
    print(f"fp32 B1 T256 N4: max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
    assert ey <= 1e-4 and eh <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_checkpoints(dtype):
    x = make(2, 150, 3, dtype, seed=7)
    y, HT, ck = run(x, ckpt_every=64)
    yr, HTr, ckr = oracle_forward(x, ckpt_every=64)
    assert ck.shape == (2, 3, 3, 64, 16)
    assert np.all(ck[:, :, 0] == 0.0)
    assert max_abs(ck, ckr) <= TOL[dtype]
    assert max_abs(y, yr) <= TOL[dtype]
    # checkpointing does not change the trajectory
    y2, HT2 = run(x)
    assert np.array_equal(y, y2) and np.array_equal(HT, HT2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_f_one_is_exact(dtype):
    """f = 1 keeps H = 0, so H_T = 0 and y = w_r * v, bit-exact."""
    x = make(2, 70, 5, dtype, seed=3)
    x["f"] = torch.ones_like(x["f"])
    y, HT = run(x)
    assert np.all(HT == 0.0)
    expect = (x["wr"].float()[None, None] * x["v"].float()).numpy()
    assert np.array_equal(y, expect)


def test_forward_state_bound():
    """|H| <= 1 (convex combination of values in [-1, 1]), up to fp32 rounding."""
    x = make(2, 300, 4, "f32", seed=11)
    x["k"] = x["k"] * 8
    x["v"] = x["v"] * 8
    x["W"] = x["W"] * 6
    _, HT, ck = run(x, ckpt_every=1)
    assert np.max(np.abs(ck)) <= 1.0 + 2.0 ** -22
    assert np.max(np.abs(HT)) <= 1.0 + 2.0 ** -22
    assert np.max(np.abs(HT)) > 0.9


def test_forward_rnn_embedding():
    """f = 0, w_r = 0, q = k = e_1: y_t = h_t of the Elman RNN (textbook form,
    computed by torch.nn.RNN in float64 on the CPU)."""
    B, T, N = 2, 50, 3
    x = make(B, T, N, "f32", seed=5)
    q = torch.zeros(B, T, 64)
    q[:, :, 0] = 1.0
    x["q"], x["k"] = q, q.clone()
    x["f"] = torch.zeros(B, T, N)
    x["wr"] = torch.zeros(N, 16)
    y, _ = run(x)
    for n in range(N):
        rnn = torch.nn.RNN(16, 16, nonlinearity="tanh", bias=False, batch_first=True).double()
        with torch.no_grad():
            rnn.weight_ih_l0.copy_(torch.eye(16, dtype=torch.float64))
            rnn.weight_hh_l0.copy_(x["W"][n].double().T)
            h, _ = rnn(x["v"][:, :, n].double())
        assert max_abs(y[:, :, n], h.numpy()) <= 1e-4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_zero_w_zero_f_closed_form(dtype):
    """W = 0 and f = 0: every step forgets the past, so H_t = tanh(k_t v_t^T)
    elementwise and y_t = H_t^T q_t + w_r v_t, written out in float64 from the
    same (bf16-rounded) inputs; on the launch shape of four heads per
    workgroup with a ragged chunk."""
    B, T, N = 4, 77, 300
    x = make(B, T, N, dtype, seed=23)
    x["W"] = torch.zeros_like(x["W"])
    x["f"] = torch.zeros_like(x["f"])
    y, HT, ck = run(x, ckpt_every=16)
    q, k, v, wr = (x[n].double() for n in ("q", "k", "v", "wr"))
    H = torch.tanh(k[:, :, None, :, None] * v[:, :, :, None, :])        # [B,T,N,K,V]
    y_ref = torch.einsum("btnkv,btk->btnv", H, q) + wr * v
    tol = TOL[dtype]
    assert max_abs(y, y_ref.numpy()) <= tol
    assert max_abs(HT, H[:, -1].numpy()) <= tol
    assert max_abs(ck[:, :, 1:], H[:, 15:T - 1:16].permute(0, 2, 1, 3, 4).numpy()) <= tol
    assert np.all(ck[:, :, 0] == 0.0)


def test_forward_deterministic():
    x = make(2, 200, 8, "bf16", seed=2)
    a = run(x)
    b = run(x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_forward_empty_and_zero_length():
    x = make(2, 5, 3, "bf16")
    g = to_gpu(x)
    # T = 0: y is empty and H_T = H_0 = 0
    y, HT = m2.forward(g["q"][:, :0].contiguous(), g["k"][:, :0].contiguous(), g["v"][:, :0].contiguous(),
                       g["f"][:, :0].contiguous(), g["W"], g["wr"])
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 3, 16) and torch.all(HT == 0)
    # B = 0: nothing to do
    y, HT = m2.forward(g["q"][:0], g["k"][:0], g["v"][:0], g["f"][:0], g["W"], g["wr"])
    torch.cuda.synchronize()
    assert y.numel() == 0 and HT.numel() == 0


def test_forward_rejects_bad_arguments():
    x = to_gpu(make(1, 4, 2, "f32"))
    dev = x["q"].device
    y = torch.empty(1, 4, 2, 16, device=dev)
    H = torch.empty(1, 2, 64, 16, device=dev)
    P = m2._ptr
    s = m2._stream(dev)
    args = [P(x[n]) for n in ("q", "k", "v", "f", "W", "wr")]
    assert m2.m2rnn_forward(1, 4, 2, 32, 16, 0, *args, None, P(y), P(H), None, 0, None, 0, s) == m2.M2RNN_ERR_UNSUPPORTED
    assert m2.m2rnn_forward(1, 4, 2, 64, 16, 7, *args, None, P(y), P(H), None, 0, None, 0, s) == m2.M2RNN_ERR_INVALID_ARG
    assert m2.m2rnn_forward(-1, 4, 2, 64, 16, 0, *args, None, P(y), P(H), None, 0, None, 0, s) == m2.M2RNN_ERR_INVALID_ARG
    bad = list(args)
    bad[0] = None
    assert m2.m2rnn_forward(1, 4, 2, 64, 16, 0, *bad, None, P(y), P(H), None, 0, None, 0, s) == m2.M2RNN_ERR_INVALID_ARG
    assert "q" in m2.m2rnn_last_error()
    mis = torch.empty(1, 4, 2, 16 + 1, device=dev)
    assert m2.m2rnn_forward(1, 4, 2, 64, 16, 0, *args, None, ctypes.c_void_p(mis.data_ptr() + 4), P(H), None, 0, None, 0,
                            s) == m2.M2RNN_ERR_INVALID_ARG
    # checkpoint pointer without an interval
    assert m2.m2rnn_forward(1, 4, 2, 64, 16, 0, *args, None, P(y), P(H), P(H), 0, None, 0, s) == m2.M2RNN_ERR_INVALID_ARG


@pytest.mark.parametrize("name,rows", [
    ("fwd_bf16_B8_T2048_N16", None),
    ("fwd_bf16_B2_T32768_N32", None),
    ("fwd_bf16_B32_T4096_N64", [(0, 4), (15, 17), (28, 32)]),
])
def test_forward_full_size(name, rows):
    """Full-size workloads in the launch configuration the benchmark times,
    against the oracle element by element: every y and H_T element of the
    B=8, T=2048, N=16 and B=2, T=32768, N=32 workloads, and every element of
    eight whole batch rows (all 64 heads, first, middle and last) of the
    B=32, T=4096, N=64 one; every output is finite with |H_T| <= 1."""
    w = m2rnn_inputs.WORKLOADS[name]
    x = m2rnn_inputs.make_workload(w)
    g = to_gpu(x)
    y, HT = m2.forward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and float(HT.abs().max()) <= 1.0 + 2.0 ** -22
    for b0, b1 in rows or [(0, w.B)]:
        yr, HTr = oracle_forward(batch_rows(x, b0, b1))
        ey = max_abs(y[b0:b1].cpu().numpy(), yr)
        eh = max_abs(HT[b0:b1].cpu().numpy(), HTr)
        print(f"{name} rows {b0}..{b1 - 1}: max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
        assert ey <= TOL[w.dtype] and eh <= TOL[w.dtype]
