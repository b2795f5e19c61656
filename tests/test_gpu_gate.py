"""The gated scan on the GPU through the C ABI: the forget gate computed in the
kernels from a pre-activation (slide "The gate preserves a direct path
through time", paper Eqs. (13), (17)), f = exp(-alpha softplus(a + beta)),
and its backward into (da, dalpha, dbeta).

The reference is the fp64 oracle composed: its gate forward gives f, its
scan forward/backward gives y, H_T and df, and its gate backward carries df
to (da, dalpha, dbeta).  Bars as for the plain scan: max-abs 1e-4 (float32
inputs) and 5e-3 (bfloat16 inputs) on y and H_T; per gradient tensor
max|g - g_ref| <= tol * max(1, max|g_ref|)."""
import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
import oracle
from gpu_common import TOL, make, max_abs, to_gpu

pytestmark = pytest.mark.gpu

GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("da", "da"), ("dalpha", "dalpha"), ("dbeta", "dbeta"),
         ("dW", "dW"), ("dw_r", "dwr"), ("dH_0", "dH_0"))


def inputs(B, T, N, dtype, seed, with_dy=False, **gate_kw):
    x = make(B, T, N, dtype, seed=seed, with_dy=with_dy)
    del x["f"]
    x.update(m2rnn_inputs.make_gate(B, T, N, dtype, seed=seed, **gate_kw))
    return x


def f64(t):
    return None if t is None else t.double().numpy()


def ref_forward(x, H_0=None, ckpt_every=0):
    f = oracle.gate_forward(f64(x["a"]), f64(x["alpha"]), f64(x["beta"]))
    return oracle.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f, f64(x["W"]), f64(x["wr"]),
                          ckpt_every=ckpt_every, H_0=f64(H_0))


def ref_backward(x, H_0=None, dH_T=None):
    a, al, be = f64(x["a"]), f64(x["alpha"]), f64(x["beta"])
    f = oracle.gate_forward(a, al, be)
    gr = oracle.backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f, f64(x["W"]), f64(x["wr"]), f64(x["dy"]),
                         f64(dH_T), H_0=f64(H_0))
    gr["da"], gr["dalpha"], gr["dbeta"] = oracle.gate_backward(a, al, be, gr["df"])
    return gr


def gpu_forward(g, H_0=None, ckpt_every=0):
    return m2.forward_gated(g["q"], g["k"], g["v"], g["a"], g["alpha"], g["beta"], g["W"], g["wr"],
                            ckpt_every=ckpt_every, H_0=H_0)


def gpu_grads(x, ck, H_0=None, dH_T=None):
    g = to_gpu(x)
    H0 = None if H_0 is None else H_0.cuda()
    _, _, Hck = gpu_forward(g, H_0=H0, ckpt_every=ck)
    out = m2.backward_gated(g["q"], g["k"], g["v"], g["a"], g["alpha"], g["beta"], g["W"], g["wr"], Hck, ck,
                            g["dy"], dH_T=None if dH_T is None else dH_T.cuda(), want_dH_0=True)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in out.items()}


def check(gg, gr, tol, label):
    worst = 0.0
    for name, rname in GRADS:
        ref = gr[rname]
        err = float(np.max(np.abs(gg[name] - ref))) if ref.size else 0.0
        scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
        worst = max(worst, err / scale)
        assert err <= tol * scale, f"{label} {name}: max abs err {err:.3e} > {tol * scale:.3e}"
    print(f"{label}: worst scaled err {worst:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N", [(1, 256, 4), (2, 100, 5), (3, 37, 1), (2, 70, 9), (3, 1, 2), (3, 30, 201),
                                   (2, 20, 801)])
def test_gated_forward_parity(dtype, B, T, N):
    """Ragged lengths and head counts that leave part of a workgroup idle,
    from a given initial state, with checkpoints."""
    x = inputs(B, T, N, dtype, seed=500 + B + T + N)
    H0 = m2rnn_inputs.make_state(B, N, seed=N)
    y, HT, Hck = gpu_forward(to_gpu(x), H_0=H0.cuda(), ckpt_every=16)
    torch.cuda.synchronize()
    yr, HTr, ckr = ref_forward(x, H_0=H0, ckpt_every=16)
    ey, eh = max_abs(y.cpu().numpy(), yr), max_abs(HT.cpu().numpy(), HTr)
    ec = max_abs(Hck.cpu().numpy(), ckr)
    print(f"gated {dtype} B{B} T{T} N{N}: max|dy|={ey:.3e} max|dH_T|={eh:.3e} max|dH_ckpt|={ec:.3e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype] and ec <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_forward_alpha_zero_is_f_one(dtype):
    """alpha = 0 gives f = 1 exactly, so the gated scan reproduces the plain
    scan run with f = 1 bit for bit (the state stays at H_0, up to the
    rounding of the kernels' internal state scaling)."""
    B, T, N = 2, 50, 5
    x = to_gpu(inputs(B, T, N, dtype, seed=3))
    x["alpha"] = torch.zeros_like(x["alpha"])
    H0 = m2rnn_inputs.make_state(B, N, seed=4).cuda()
    y, HT = gpu_forward(x, H_0=H0)
    ones = torch.ones_like(x["a"])
    y1, HT1 = m2.forward(x["q"], x["k"], x["v"], ones, x["W"], x["wr"], H_0=H0)
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(HT, HT1)
    assert float((HT - H0).abs().max()) <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_forward_saturated_gate(dtype):
    """Pre-activations far out on both sides (softplus near 0 and near its
    argument; f near 1 and underflowing to 0) against the oracle."""
    B, T, N = 2, 64, 4
    x = inputs(B, T, N, dtype, seed=8, mu=0.0)
    x["a"] = (x["a"].float() * 30.0).to(x["a"].dtype)
    y, HT = gpu_forward(to_gpu(x))
    torch.cuda.synchronize()
    yr, HTr = ref_forward(x)
    assert bool(torch.isfinite(y).all())
    assert max_abs(y.cpu().numpy(), yr) <= TOL[dtype] and max_abs(HT.cpu().numpy(), HTr) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N,ck", [(2, 37, 3, 1), (1, 70, 5, 16), (2, 150, 6, 64), (1, 45, 9, 8), (1, 3, 2, 64),
                                      (2, 20, 301, 16), (1, 13, 1031, 4)])
def test_gated_backward_parity(dtype, B, T, N, ck):
    """From a given initial state with dH_T; checkpoint intervals below, at
    and above the replay window; head counts that do not fill a workgroup."""
    x = inputs(B, T, N, dtype, seed=600 + B + T + N + ck, with_dy=True)
    H0 = m2rnn_inputs.make_state(B, N, seed=T)
    dHT = m2rnn_inputs.make_state(B, N, seed=T + 1)
    check(gpu_grads(x, ck, H0, dHT), ref_backward(x, H0, dHT), TOL[dtype], f"gated {dtype} B{B} T{T} N{N} ck{ck}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_backward_saturated_gate(dtype):
    B, T, N, ck = 2, 64, 4, 16
    x = inputs(B, T, N, dtype, seed=9, with_dy=True, mu=0.0)
    x["a"] = (x["a"].float() * 30.0).to(x["a"].dtype)
    check(gpu_grads(x, ck), ref_backward(x), TOL[dtype], f"gated saturated {dtype}")


def test_gated_backward_alpha_zero():
    """alpha = 0: f = 1 whatever a and beta, so da = 0 and dbeta = 0 exactly,
    dalpha = -sum df softplus(a + beta) (oracle), and every other gradient is
    the plain backward's with f = 1, bit for bit."""
    B, T, N, ck = 2, 90, 5, 16
    x = inputs(B, T, N, "f32", seed=12, with_dy=True)
    x["alpha"] = torch.zeros_like(x["alpha"])
    gg = gpu_grads(x, ck)
    assert np.all(gg["da"] == 0) and np.all(gg["dbeta"] == 0)
    gr = ref_backward(x)
    assert max_abs(gg["dalpha"], gr["dalpha"]) <= 1e-4 * max(1.0, float(np.max(np.abs(gr["dalpha"]))))
    g = to_gpu(x)
    ones = torch.ones_like(g["a"])
    _, _, Hck = m2.forward(g["q"], g["k"], g["v"], ones, g["W"], g["wr"], ckpt_every=ck)
    pl = m2.backward(g["q"], g["k"], g["v"], ones, g["W"], g["wr"], Hck, ck, g["dy"], want_dH_0=True)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dW", "dw_r", "dH_0"):
        assert np.array_equal(gg[name], pl[name].cpu().numpy()), name


def test_gated_backward_zero_length():
    """T = 0: dalpha, dbeta, dW, dw_r are zero and dH_0 = dH_T."""
    x = to_gpu(inputs(2, 3, 3, "bf16", seed=2, with_dy=True))
    e = {n: x[n][:, :0].contiguous() for n in ("q", "k", "v", "a", "dy")}
    Hck = torch.empty(2, 3, 0, 64, 16, device="cuda")
    dHT = m2rnn_inputs.make_state(2, 3, seed=9).cuda()
    out = m2.backward_gated(e["q"], e["k"], e["v"], e["a"], x["alpha"], x["beta"], x["W"], x["wr"], Hck, 64,
                            e["dy"], dH_T=dHT, want_dH_0=True)
    out["dalpha"].fill_(7.0)
    out["dbeta"].fill_(7.0)
    m2.backward_gated(e["q"], e["k"], e["v"], e["a"], x["alpha"], x["beta"], x["W"], x["wr"], Hck, 64, e["dy"],
                      dH_T=dHT, out=out)
    torch.cuda.synchronize()
    assert torch.all(out["dalpha"] == 0) and torch.all(out["dbeta"] == 0)
    assert torch.all(out["dW"] == 0) and torch.all(out["dw_r"] == 0) and torch.equal(out["dH_0"], dHT)


def test_gated_backward_deterministic():
    x = to_gpu(inputs(2, 200, 7, "bf16", seed=5, with_dy=True))
    _, _, Hck = gpu_forward(x, ckpt_every=64)
    outs = [m2.backward_gated(x["q"], x["k"], x["v"], x["a"], x["alpha"], x["beta"], x["W"], x["wr"], Hck, 64,
                              x["dy"]) for _ in range(2)]
    torch.cuda.synchronize()
    for name in outs[0]:
        assert torch.equal(outs[0][name], outs[1][name]), name


def test_gated_full_size_sampled():
    """The B=32, T=4096, N=64 gated forward + backward in the benchmark's
    launch configuration (bf16 inputs, checkpoints every 64 steps).  Sampled
    (b, n) chains: y, H_T, dv and da against the oracle run on that chain
    alone.  Whole tensors: finiteness, 0 <= |H_T| <= 1, and dbeta = sum over
    b, t of da (the chain rule through a + beta, which holds at any size)."""
    w = m2rnn_inputs.WORKLOADS["fwdbwd_bf16_B32_T4096_N64"]
    x = inputs(w.B, w.T, w.N, w.dtype, seed=1, with_dy=True)
    g = to_gpu(x)
    y, HT, Hck = gpu_forward(g, ckpt_every=w.ckpt_every)
    out = m2.backward_gated(g["q"], g["k"], g["v"], g["a"], g["alpha"], g["beta"], g["W"], g["wr"], Hck,
                            w.ckpt_every, g["dy"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and float(HT.abs().max()) <= 1.0 + 2.0 ** -22
    for name in out:
        assert bool(torch.isfinite(out[name]).all()), name
    dbeta = out["da"].double().sum(dim=(0, 1))
    assert float((out["dbeta"].double() - dbeta).abs().max()) <= 1e-4 * max(1.0, float(dbeta.abs().max()))
    for b, n in ((0, 0), (31, 63), (17, 42)):
        sl = {nm: x[nm][b:b + 1] for nm in ("q", "k")}
        sl.update({nm: x[nm][b:b + 1, :, n:n + 1] for nm in ("v", "a", "dy")})
        sl.update({nm: x[nm][n:n + 1] for nm in ("W", "wr", "alpha", "beta")})
        yr, HTr = ref_forward(sl)
        gr = ref_backward(sl)
        ey = max_abs(y[b:b + 1, :, n:n + 1].cpu().numpy(), yr)
        eh = max_abs(HT[b:b + 1, n:n + 1].cpu().numpy(), HTr)
        assert ey <= TOL["bf16"] and eh <= TOL["bf16"], (b, n, ey, eh)
        for name in ("dv", "da"):
            got = out[name][b:b + 1, :, n:n + 1].cpu().numpy()
            ref = gr[name]
            err = max_abs(got, ref)
            scale = max(1.0, float(np.max(np.abs(ref))))
            print(f"gated chain ({b},{n}) {name}: max err {err:.3e} (scale {scale:.2f})")
            assert err <= 5e-3 * scale
