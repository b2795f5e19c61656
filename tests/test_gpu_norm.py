"""Output gate and RMSNorm after the readout, on the GPU through the C ABI,
against the fp64 oracle (slide "Most of the block can be computed before
recurrence", paper Fig. 2; statistic and backward of slide "Backup: RMSNormTP
synchronizes per-token statistics", paper App. C, Eqs. (26)-(33)).

The pages state no tolerance for this step.  The kernels compute in fp32 on
inputs that are exact in fp32 (bf16 inputs are widened exactly), so each
output is a few fp32 roundings plus a sum of d <= 2048 products away from the
fp64 value: the bar is max|out - ref| <= 1e-4 * max(1, max|ref|) per tensor,
for both input dtypes."""
import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
import oracle
from gpu_common import make, max_abs, to_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-4


def inputs(B, T, N, dtype, seed):
    x = m2rnn_inputs.make_epilogue(B, T, N, dtype, seed=seed)
    return x["y"], x["g"], x["w"], x["dout"]


def f64(t):
    return t.double().numpy()


def scaled_err(got, ref):
    ref = np.asarray(ref)
    if ref.size == 0:
        return 0.0
    return max_abs(got, ref) / max(1.0, float(np.max(np.abs(ref))))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N", [(2, 37, 5), (1, 100, 16), (3, 20, 64), (1, 7, 128), (2, 50, 1)])
@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_norm_parity(dtype, B, T, N, eps):
    """Feature rows that fill 1, 2, 4 or 8 chunks of 256 and rows that leave
    most of a chunk idle (d = 80, d = 16)."""
    y, g, w, dout = inputs(B, T, N, dtype, seed=B * 100 + T + N)
    rstd = torch.empty(B, T, device="cuda")
    out = m2.gate_rmsnorm_forward(y.cuda(), g.cuda(), w.cuda(), eps, rstd=rstd)
    dy, dg, dw = m2.gate_rmsnorm_backward(y.cuda(), g.cuda(), w.cuda(), dout.cuda(), eps)
    torch.cuda.synchronize()
    d = N * 16
    ro, rs = oracle.gate_rmsnorm_forward(f64(y).reshape(-1, d), f64(g).reshape(-1, d), f64(w).reshape(d), eps)
    rdy, rdg, rdw = oracle.gate_rmsnorm_backward(f64(y).reshape(-1, d), f64(g).reshape(-1, d), f64(w).reshape(d),
                                                 f64(dout).reshape(-1, d), eps)
    errs = {"out": scaled_err(out.cpu().numpy().reshape(-1, d), ro),
            "rstd": scaled_err(rstd.cpu().numpy().reshape(-1), rs),
            "dy": scaled_err(dy.cpu().numpy().reshape(-1, d), rdy),
            "dg": scaled_err(dg.cpu().numpy().reshape(-1, d), rdg),
            "dw": scaled_err(dw.cpu().numpy(), rdw)}
    print(f"norm {dtype} B{B} T{T} N{N} eps{eps}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL, (k, v)


def test_norm_in_place_and_deterministic():
    """out may overwrite y and dy may overwrite dout; two backward runs agree
    bit for bit (fixed-order sums, no atomics)."""
    y, g, w, dout = [t.cuda() for t in inputs(2, 300, 64, "bf16", seed=3)]
    ref = m2.gate_rmsnorm_forward(y, g, w)
    yy = y.clone()
    got = m2.gate_rmsnorm_forward(yy, g, w, out=yy)
    r1 = m2.gate_rmsnorm_backward(y, g, w, dout)
    r2 = m2.gate_rmsnorm_backward(y, g, w, dout)
    dd = dout.clone()
    r3 = m2.gate_rmsnorm_backward(y, g, w, dd, out=(dd, torch.empty_like(dd), torch.empty(1024, device="cuda")))
    torch.cuda.synchronize()
    assert got.data_ptr() == yy.data_ptr() and torch.equal(got, ref)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    assert torch.equal(r3[0], r1[0]) and torch.equal(r3[1], r1[1]) and torch.equal(r3[2], r1[2])


def test_norm_empty():
    """No tokens: the forward does nothing and the backward sets dw = 0."""
    y, g, w, dout = [t.cuda() for t in inputs(2, 0, 5, "f32", seed=1)]
    out = m2.gate_rmsnorm_forward(y, g, w)
    dw = torch.full((80,), 7.0, device="cuda")
    m2.gate_rmsnorm_backward(y, g, w, dout, out=(torch.empty_like(y), torch.empty_like(y), dw))
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.all(dw == 0)


def test_norm_chained_with_scan():
    """The block's order on a small case: scan forward, gate and RMSNorm, then
    the RMSNorm backward feeds dy of the scan backward.  Every gradient against
    the oracle composed the same way (bf16 inputs; the scan's 5e-3 bar)."""
    B, T, N, ck = 2, 70, 5, 16
    x = make(B, T, N, "bf16", seed=21)
    _, g, w, dout = inputs(B, T, N, "bf16", seed=22)
    gx = to_gpu(x)
    y, _, Hck = m2.forward(gx["q"], gx["k"], gx["v"], gx["f"], gx["W"], gx["wr"], ckpt_every=ck)
    o = m2.gate_rmsnorm_forward(y, g.cuda(), w.cuda())
    dy, dg, dw = m2.gate_rmsnorm_backward(y, g.cuda(), w.cuda(), dout.cuda())
    grads = m2.backward(gx["q"], gx["k"], gx["v"], gx["f"], gx["W"], gx["wr"], Hck, ck, dy)
    torch.cuda.synchronize()
    ins = [f64(x[n]) for n in ("q", "k", "v", "f", "W", "wr")]
    yr, _ = oracle.forward(*ins)
    d = N * 16
    ro, _ = oracle.gate_rmsnorm_forward(yr.reshape(-1, d), f64(g).reshape(-1, d), f64(w).reshape(d))
    rdy, rdg, rdw = oracle.gate_rmsnorm_backward(yr.reshape(-1, d), f64(g).reshape(-1, d), f64(w).reshape(d),
                                                 f64(dout).reshape(-1, d))
    gr = oracle.backward(*ins, rdy.reshape(B, T, N, 16))
    assert scaled_err(o.cpu().numpy().reshape(-1, d), ro) <= 5e-3
    assert scaled_err(dg.cpu().numpy().reshape(-1, d), rdg) <= 5e-3
    assert scaled_err(dw.cpu().numpy(), rdw) <= 5e-3
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("df", "df"), ("dW", "dW"), ("dw_r", "dwr")):
        e = scaled_err(grads[name].cpu().numpy(), gr[rname])
        print(f"chained {name}: {e:.2e}")
        assert e <= 5e-3, name


def test_norm_full_size_sampled():
    """The B=32, T=4096, N=64 feature rows (d = 1024) in the launch
    configuration the benchmark times: sampled tokens against the oracle, and
    dw (a sum over all 131072 tokens) against a float64 torch sum of
    dout * x * s over the whole tensor."""
    B, T, N = 32, 4096, 64
    y, g, w, dout = [t.cuda() for t in inputs(B, T, N, "bf16", seed=5)]
    rstd = torch.empty(B, T, device="cuda")
    out = m2.gate_rmsnorm_forward(y, g, w, rstd=rstd)
    dy, dg, dw = m2.gate_rmsnorm_backward(y, g, w, dout)
    torch.cuda.synchronize()
    d = N * 16
    for b, t in ((0, 0), (31, 4095), (17, 1234), (5, 4000)):
        yy, gg, dd = f64(y[b, t].cpu()).reshape(1, d), f64(g[b, t].cpu()).reshape(1, d), f64(dout[b, t].cpu())
        ro, rs = oracle.gate_rmsnorm_forward(yy, gg, f64(w.cpu()).reshape(d))
        rdy, rdg, _ = oracle.gate_rmsnorm_backward(yy, gg, f64(w.cpu()).reshape(d), dd.reshape(1, d))
        assert scaled_err(out[b, t].cpu().numpy().reshape(1, d), ro) <= TOL
        assert abs(float(rstd[b, t]) - rs[0]) <= TOL * max(1.0, rs[0])
        assert scaled_err(dy[b, t].cpu().numpy().reshape(1, d), rdy) <= TOL
        assert scaled_err(dg[b, t].cpu().numpy().reshape(1, d), rdg) <= TOL
    x = y.double() * g.double()
    s = 1.0 / torch.sqrt((x * x).mean(dim=(2, 3), keepdim=True))
    dw_ref = (dout.double() * x * s).sum(dim=(0, 1)).reshape(-1)
    e = float((dw.double() - dw_ref).abs().max()) / max(1.0, float(dw_ref.abs().max()))
    print(f"full-size dw scaled err {e:.2e}")
    assert e <= TOL
