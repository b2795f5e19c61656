"""Causal Conv1D (width 4) and SiLU before the scan, on the GPU through the C
ABI, against the fp64 oracle (slide "Most of the block can be computed before
recurrence", paper Fig. 2).

The pages state no tolerance for this step.  The kernels compute in fp32 on
inputs exact in fp32: float32 outputs are held to 1e-5 * max(1, max|ref|);
bfloat16 outputs are the nearest-even rounding of such a value, so each is
held to 2^-8 |ref| + 1e-5.  Gradients (float32) per tensor to
1e-4 * max(1, max|ref|)."""
import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
import oracle
from gpu_common import make, max_abs, to_gpu

pytestmark = pytest.mark.gpu


def f64(t):
    return None if t is None else t.double().cpu().numpy()


def scaled_err(got, ref):
    ref = np.asarray(ref)
    if ref.size == 0:
        return 0.0
    return max_abs(got, ref) / max(1.0, float(np.max(np.abs(ref))))


def check_forward(z, ref, dtype, label):
    z = z.double().cpu().numpy()
    if dtype == "bf16":
        excess = np.abs(z - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5)
        worst = float(np.max(excess)) if excess.size else -1.0
        assert worst <= 0.0, f"{label}: bf16 output off by {worst:.3e} beyond one rounding"
    else:
        e = scaled_err(z, ref)
        assert e <= 1e-5, f"{label}: {e:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,C", [(2, 37, 64), (1, 100, 80), (3, 5, 4), (2, 1, 16), (1, 70, 1024), (2, 17, 8)])
@pytest.mark.parametrize("use_bias", [True, False])
def test_conv_parity(dtype, B, T, C, use_bias):
    """Ragged strips (T not a multiple of 16 or 8, T < 3, T = 1) and channel
    counts from one group of four up to N V = 1024."""
    x = m2rnn_inputs.make_conv(B, T, C, dtype, seed=B * 1000 + T + C)
    bias = x["bias"] if use_bias else None
    g = {k: v.cuda() for k, v in x.items()}
    gb = g["bias"] if use_bias else None
    z = m2.conv_silu_forward(g["u"], g["w"], gb)
    du, dw, db = m2.conv_silu_backward(g["u"], g["w"], gb, g["dz"])
    torch.cuda.synchronize()
    zr = oracle.conv_silu_forward(f64(x["u"]), f64(x["w"]), f64(bias))
    rdu, rdw, rdb = oracle.conv_silu_backward(f64(x["u"]), f64(x["w"]), f64(bias), f64(x["dz"]))
    label = f"conv {dtype} B{B} T{T} C{C} bias={use_bias}"
    check_forward(z, zr, dtype, label)
    errs = {"du": scaled_err(du.cpu().numpy(), rdu), "dw": scaled_err(dw.cpu().numpy(), rdw),
            "dbias": scaled_err(db.cpu().numpy(), rdb)}
    print(label + ": " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 1e-4, (label, k, v)


def test_conv_empty_and_deterministic():
    """T = 0 sets dw and dbias to zero; two backward runs agree bit for bit."""
    x = {k: v.cuda() for k, v in m2rnn_inputs.make_conv(2, 0, 16, "bf16", seed=1).items()}
    dw = torch.full((16, 4), 3.0, device="cuda")
    db = torch.full((16,), 3.0, device="cuda")
    z = m2.conv_silu_forward(x["u"], x["w"], x["bias"])
    m2.conv_silu_backward(x["u"], x["w"], x["bias"], x["dz"], out=(torch.empty(2, 0, 16, device="cuda"), dw, db))
    torch.cuda.synchronize()
    assert z.numel() == 0 and torch.all(dw == 0) and torch.all(db == 0)
    x = {k: v.cuda() for k, v in m2rnn_inputs.make_conv(4, 300, 256, "bf16", seed=2).items()}
    r1 = m2.conv_silu_backward(x["u"], x["w"], x["bias"], x["dz"])
    r2 = m2.conv_silu_backward(x["u"], x["w"], x["bias"], x["dz"])
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_conv_then_scan():
    """The block's order on a small case: q, k and v through the conv and
    SiLU, then the scan, and back: the scan's dq, dk, dv feed the conv
    backward.  Each stage is checked against the oracle run on the previous
    stage's GPU output (bf16 inputs; the scan's 5e-3 bar)."""
    B, T, N, ck = 2, 50, 3, 16
    base = make(B, T, N, "bf16", seed=31, with_dy=True)
    cq = m2rnn_inputs.make_conv(B, T, 64, "bf16", seed=1)
    ck_ = m2rnn_inputs.make_conv(B, T, 64, "bf16", seed=2)
    cv = m2rnn_inputs.make_conv(B, T, N * 16, "bf16", seed=3)
    convs = {"q": cq, "k": ck_, "v": cv}
    gpu = {n: {k: t.cuda() for k, t in c.items()} for n, c in convs.items()}
    z = {n: m2.conv_silu_forward(c["u"], c["w"], c["bias"]) for n, c in gpu.items()}
    z["v"] = z["v"].view(B, T, N, 16)
    gb = to_gpu(base)
    y, _, Hck = m2.forward(z["q"], z["k"], z["v"], gb["f"], gb["W"], gb["wr"], ckpt_every=ck)
    grads = m2.backward(z["q"], z["k"], z["v"], gb["f"], gb["W"], gb["wr"], Hck, ck, gb["dy"])
    dz = {"q": grads["dq"], "k": grads["dk"], "v": grads["dv"].reshape(B, T, N * 16)}
    back = {n: m2.conv_silu_backward(gpu[n]["u"], gpu[n]["w"], gpu[n]["bias"], dz[n]) for n in gpu}
    torch.cuda.synchronize()
    ins = [f64(z["q"]), f64(z["k"]), f64(z["v"]), f64(base["f"]), f64(base["W"]), f64(base["wr"])]
    yr, _ = oracle.forward(*ins)
    assert max_abs(y.cpu().numpy(), yr) <= 5e-3
    gr = oracle.backward(*ins, f64(base["dy"]))
    for n, rn in (("dq", "dq"), ("dk", "dk"), ("dv", "dv")):
        assert scaled_err(grads[n].cpu().numpy(), gr[rn]) <= 5e-3, n
    for n in ("q", "k", "v"):
        c = convs[n]
        rdu, rdw, rdb = oracle.conv_silu_backward(f64(c["u"]), f64(c["w"]), f64(c["bias"]), f64(dz[n]))
        assert scaled_err(back[n][0].cpu().numpy(), rdu) <= 1e-4, n
        assert scaled_err(back[n][1].cpu().numpy(), rdw) <= 1e-4, n
        assert scaled_err(back[n][2].cpu().numpy(), rdb) <= 1e-4, n


def test_conv_full_size_sampled():
    """v's channels at the B=32, T=4096, N=64 shape (C = 1024, bf16) in the
    launch configuration the benchmark times: sampled (batch row, 8-channel)
    slices against the oracle run on that slice alone (each channel's conv
    runs along its own time axis), and dw, dbias (sums over all 131072
    tokens) against a float64 torch computation over the whole tensor."""
    B, T, C = 32, 4096, 1024
    x = m2rnn_inputs.make_conv(B, T, C, "bf16", seed=7)
    g = {k: v.cuda() for k, v in x.items()}
    z = m2.conv_silu_forward(g["u"], g["w"], g["bias"])
    du, dw, db = m2.conv_silu_backward(g["u"], g["w"], g["bias"], g["dz"])
    torch.cuda.synchronize()
    for b, c0 in ((0, 0), (31, 1016), (17, 512)):
        sl = slice(c0, c0 + 8)
        zr = oracle.conv_silu_forward(f64(x["u"][b:b + 1, :, sl]), f64(x["w"][sl]), f64(x["bias"][sl]))
        check_forward(z[b:b + 1, :, sl], zr, "bf16", f"full-size conv ({b},{c0})")
        rdu, _, _ = oracle.conv_silu_backward(f64(x["u"][b:b + 1, :, sl]), f64(x["w"][sl]), f64(x["bias"][sl]),
                                              f64(x["dz"][b:b + 1, :, sl]))
        assert scaled_err(du[b:b + 1, :, sl].cpu().numpy(), rdu) <= 1e-4
    up = torch.nn.functional.pad(g["u"].double(), (0, 0, 3, 0))   # [B, T + 3, C], zero history
    w = g["w"].double()
    a = g["bias"].double() + sum(w[:, j] * up[:, j:j + T] for j in range(4))
    s = torch.sigmoid(a)
    da = g["dz"].double() * s * (1.0 + a * (1.0 - s))
    dw_ref = torch.stack([(da * up[:, j:j + T]).sum(dim=(0, 1)) for j in range(4)], dim=1)
    db_ref = da.sum(dim=(0, 1))
    e_w = float((dw.double() - dw_ref).abs().max()) / max(1.0, float(dw_ref.abs().max()))
    e_b = float((db.double() - db_ref).abs().max()) / max(1.0, float(db_ref.abs().max()))
    print(f"full-size conv dw {e_w:.2e} dbias {e_b:.2e}")
    assert e_w <= 1e-4 and e_b <= 1e-4
