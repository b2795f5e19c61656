"""Initial state H_0, its gradient dH_0 and the one-token decode step, on the
GPU through the C ABI, against the fp64 oracle (which takes the same H_0)."""
import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
import oracle
from gpu_common import TOL, make, max_abs, to_f64, to_gpu

pytestmark = pytest.mark.gpu

GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("df", "df"), ("dW", "dW"), ("dw_r", "dwr"), ("dH_0", "dH_0"))
BTOL = {"f32": 1e-4, "bf16": 5e-3}


def fwd(g, H_0=None, ckpt_every=0, out=None):
    return m2.forward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], ckpt_every=ckpt_every, out=out, H_0=H_0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N", [(2, 100, 5), (1, 37, 3), (3, 1, 2)])
def test_forward_from_initial_state(dtype, B, T, N):
    x = make(B, T, N, dtype, seed=300 + T)
    H0 = m2rnn_inputs.make_state(B, N, seed=T)
    y, HT = fwd(to_gpu(x), H_0=H0.cuda())
    torch.cuda.synchronize()
    yr, HTr = oracle.forward(*to_f64(x), H_0=H0.double().numpy())
    ey, eh = max_abs(y.cpu().numpy(), yr), max_abs(HT.cpu().numpy(), HTr)
    print(f"{dtype} B{B} T{T} N{N} from H_0: max|dy|={ey:.3e} max|dH_T|={eh:.3e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_split_sequence(dtype):
    """Two launches (T1 steps, then the rest from the first H_T) give the one
    launch's outputs; the hand-over goes through the fp32 state, so they agree
    to fp32 rounding of the state."""
    B, T, N, T1 = 2, 150, 3, 61
    x = to_gpu(make(B, T, N, dtype, seed=11))
    y, HT = fwd(x)
    a = {n: (t[:, :T1].contiguous() if n in ("q", "k", "v", "f") else t) for n, t in x.items()}
    z = {n: (t[:, T1:].contiguous() if n in ("q", "k", "v", "f") else t) for n, t in x.items()}
    ya, HA = fwd(a)
    yb, HB = fwd(z, H_0=HA)
    torch.cuda.synchronize()
    assert max_abs(torch.cat([ya, yb], dim=1).cpu().numpy(), y.cpu().numpy()) <= 1e-5
    assert max_abs(HB.cpu().numpy(), HT.cpu().numpy()) <= 1e-5


def test_forward_state_in_place_and_zero_length():
    """H_T may overwrite H_0; with T = 0, H_T = H_0."""
    B, T, N = 2, 40, 3
    x = to_gpu(make(B, T, N, "bf16", seed=5))
    H0 = m2rnn_inputs.make_state(B, N, seed=1).cuda()
    y1, HT1 = fwd(x, H_0=H0)
    H = H0.clone()
    y2, HT2 = fwd(x, H_0=H, out=(torch.empty_like(y1), H))
    torch.cuda.synchronize()
    assert HT2.data_ptr() == H.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(HT1, H)
    e = {n: (t[:, :0].contiguous() if n in ("q", "k", "v", "f") else t) for n, t in x.items()}
    _, HT0 = fwd(e, H_0=H0)
    torch.cuda.synchronize()
    assert torch.equal(HT0, H0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_match_forward(dtype):
    """T calls of the one-token decode step from H_0 reproduce the T-step
    forward from H_0 (same kernel arithmetic, state carried in fp32)."""
    B, T, N = 3, 12, 4
    x = to_gpu(make(B, T, N, dtype, seed=21))
    H0 = m2rnn_inputs.make_state(B, N, seed=2).cuda()
    y, HT = fwd(x, H_0=H0)
    H = H0.clone()
    ys = []
    for t in range(T):
        ys.append(m2.decode(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(), x["v"][:, t].contiguous(),
                            x["f"][:, t].contiguous(), x["W"], x["wr"], H))
    torch.cuda.synchronize()
    assert max_abs(torch.stack(ys, dim=1).cpu().numpy(), y.cpu().numpy()) <= 1e-5
    assert max_abs(H.cpu().numpy(), HT.cpu().numpy()) <= 1e-5


def _decode(x, H, t=0):
    return m2.decode(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(), x["v"][:, t].contiguous(),
                     x["f"][:, t].contiguous(), x["W"], x["wr"], H)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_bit_identical_to_forward_first_step(dtype):
    """At more than 1536 chains the forward runs four heads of one wave each;
    the decode kernel runs the same arithmetic in the same order, so one
    decode step from H_0 equals that forward's T = 1 outputs bit for bit."""
    B, N = 32, 64
    x = to_gpu(make(B, 1, N, dtype, seed=31))
    H0 = m2rnn_inputs.make_state(B, N, seed=3).cuda()
    y, HT = fwd(x, H_0=H0)
    H = H0.clone()
    yd = _decode(x, H)
    torch.cuda.synchronize()
    assert torch.equal(yd, y[:, 0]) and torch.equal(H, HT)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,N", [(3, 5), (1, 1), (2, 130)])
def test_decode_against_oracle(dtype, B, N):
    """One decode step from H_0 against the oracle's one-step forward from H_0,
    for head counts that leave the last workgroup partly empty (15, 1, 260)."""
    x = make(B, 1, N, dtype, seed=40 + N)
    H0 = m2rnn_inputs.make_state(B, N, seed=N)
    H = H0.clone().cuda()
    y = _decode(to_gpu(x), H)
    torch.cuda.synchronize()
    yr, HTr = oracle.forward(*to_f64(x), H_0=H0.double().numpy())
    ey, eh = max_abs(y.cpu().numpy(), yr[:, 0]), max_abs(H.cpu().numpy(), HTr)
    print(f"decode {dtype} B{B} N{N}: max|dy|={ey:.3e} max|dH|={eh:.3e}")
    assert ey <= TOL[dtype] and eh <= TOL[dtype]


def _check(gg, gr, tol, label):
    worst = 0.0
    for name, rname in GRADS:
        ref = gr[rname]
        err = float(np.max(np.abs(gg[name] - ref)))
        scale = max(1.0, float(np.max(np.abs(ref))))
        worst = max(worst, err / scale)
        assert err <= tol * scale, f"{label} {name}: max abs err {err:.3e} > {tol * scale:.3e}"
    print(f"{label}: worst scaled err {worst:.3e}")


def _gpu_grads(x, H0, ck, dHT):
    g = to_gpu(x)
    _, _, Hck = fwd(g, H_0=H0.cuda(), ckpt_every=ck)
    out = m2.backward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], Hck, ck, g["dy"],
                      dH_T=dHT.cuda(), want_dH_0=True)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy() for n, t in out.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,N,ck", [(2, 37, 3, 1), (1, 70, 5, 16), (2, 150, 2, 64), (1, 3, 2, 64)])
def test_backward_initial_state_gradient(dtype, B, T, N, ck):
    x = make(B, T, N, dtype, seed=400 + T + ck, with_dy=True)
    H0 = m2rnn_inputs.make_state(B, N, seed=T)
    dHT = m2rnn_inputs.make_state(B, N, seed=T + 1)
    gg = _gpu_grads(x, H0, ck, dHT)
    gr = oracle.backward(*to_f64(x), x["dy"].double().numpy(), dHT.double().numpy(), H_0=H0.double().numpy())
    _check(gg, gr, BTOL[dtype], f"{dtype} B{B} T{T} N{N} ck{ck} from H_0")


def test_backward_split_sequence():
    """The backward of two launches, chained through dH_0 -> dH_T, gives the
    one launch's gradients (float32 inputs)."""
    B, T, N, T1, ck = 2, 130, 3, 50, 16
    x = make(B, T, N, "f32", seed=31, with_dy=True)
    g = to_gpu(x)
    cut = lambda t, lo, hi: t[:, lo:hi].contiguous()
    parts = []
    for lo, hi in ((0, T1), (T1, T)):
        parts.append({n: (cut(t, lo, hi) if n in ("q", "k", "v", "f", "dy") else t) for n, t in g.items()})
    _, HA, ckA = fwd(parts[0], ckpt_every=ck)
    _, _, ckB = fwd(parts[1], H_0=HA, ckpt_every=ck)
    _, _, ck_full = fwd(g, ckpt_every=ck)
    full = m2.backward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], ck_full, ck, g["dy"], want_dH_0=True)
    p = parts[1]
    gb = m2.backward(p["q"], p["k"], p["v"], p["f"], p["W"], p["wr"], ckB, ck, p["dy"], want_dH_0=True)
    p = parts[0]
    ga = m2.backward(p["q"], p["k"], p["v"], p["f"], p["W"], p["wr"], ckA, ck, p["dy"], dH_T=gb["dH_0"],
                     want_dH_0=True)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "df"):
        got = torch.cat([ga[name], gb[name]], dim=1)
        scale = max(1.0, float(full[name].abs().max()))
        assert float((got - full[name]).abs().max()) <= 1e-5 * scale, name
    for name in ("dW", "dw_r"):
        scale = max(1.0, float(full[name].abs().max()))
        assert float((ga[name] + gb[name] - full[name]).abs().max()) <= 1e-5 * scale, name
    assert float((ga["dH_0"] - full["dH_0"]).abs().max()) <= 1e-5 * max(1.0, float(full["dH_0"].abs().max()))


def test_backward_zero_length_passes_dH_T():
    """T = 0: dH_0 = dH_T (zero without dH_T)."""
    x = to_gpu(make(2, 3, 2, "bf16", with_dy=True))
    e = {k: v[:, :0].contiguous() for k, v in x.items() if k in ("q", "k", "v", "f", "dy")}
    Hck = torch.empty(2, 2, 0, 64, 16, device="cuda")
    dHT = m2rnn_inputs.make_state(2, 2, seed=9).cuda()
    out = m2.backward(e["q"], e["k"], e["v"], e["f"], x["W"], x["wr"], Hck, 64, e["dy"], dH_T=dHT, want_dH_0=True)
    out2 = m2.backward(e["q"], e["k"], e["v"], e["f"], x["W"], x["wr"], Hck, 64, e["dy"], want_dH_0=True)
    torch.cuda.synchronize()
    assert torch.equal(out["dH_0"], dHT) and torch.all(out2["dH_0"] == 0)
