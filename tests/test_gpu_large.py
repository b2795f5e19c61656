"""Tensors of more than 2^31 elements (slide "Write, transform, retain, and
read a matrix state", paper Eqs. (10)-(12), at sizes past 32-bit offsets):
the kernels form every global offset in 64 bits.  Inputs are drawn on the
GPU (make_inputs_on); sampled chains are copied back and checked against the
oracle run on those chains alone, to the bf16 bar of 5e-3."""
import numpy as np
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2
import oracle
from gpu_common import chain_slice, to_f64

pytestmark = pytest.mark.gpu

TOL = 5e-3


def scaled(got, ref):
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / max(1.0, float(np.max(np.abs(ref))))


def host_slice(x, b, n, with_dy=False):
    sl = {k: t.cpu() for k, t in chain_slice(x, b, n).items()}
    if with_dy:
        sl["dy"] = x["dy"][b:b + 1, :, n:n + 1].cpu()
    return sl


def test_forward_beyond_2_31_elements():
    """B=40, T=4096, N=1024: y and the checkpoints every 64 steps each hold
    40 * 4096 * 1024 * 16 = 2.68e9 elements; the last chain's outputs sit past
    offset 2^31."""
    B, T, N, ck = 40, 4096, 1024, 64
    print(f"large forward B{B} T{T} N{N}", flush=True)
    x = m2rnn_inputs.make_inputs_on("cuda", B, T, N, dtype="bf16", seed=71)
    y, HT, Hck = m2.forward(x["q"], x["k"], x["v"], x["f"], x["W"], x["wr"], ckpt_every=ck)
    torch.cuda.synchronize()
    assert y.numel() > 2 ** 31 and Hck.numel() > 2 ** 31
    for b, n in ((B - 1, N - 1), (B - 1, 0), (0, N - 1), (23, 517), (0, 0)):
        ry, rHT, rck = oracle.forward(*to_f64(host_slice(x, b, n)), ckpt_every=ck)
        errs = (scaled(y[b:b + 1, :, n:n + 1].cpu(), ry), scaled(HT[b:b + 1, n:n + 1].cpu(), rHT),
                scaled(Hck[b:b + 1, n:n + 1].cpu(), rck))
        print(f"chain ({b},{n}): y {errs[0]:.2e} H_T {errs[1]:.2e} H_ckpt {errs[2]:.2e}")
        assert max(errs) <= TOL


def test_backward_beyond_2_31_elements():
    """B=40, T=4096, N=64 with checkpoints every 64 steps: the backward's
    replayed states every 4 steps hold 40 * 64 * 1024 * 1024 = 2.68e9 floats.
    dv and df of sampled chains and dq, dk of the last batch row against the
    oracle; dw_r against its closed form sum over b, t of dy * v."""
    B, T, N, ck = 40, 4096, 64, 64
    print(f"large backward B{B} T{T} N{N}", flush=True)
    x = m2rnn_inputs.make_inputs_on("cuda", B, T, N, dtype="bf16", seed=72, with_dy=True)
    _, _, Hck = m2.forward(x["q"], x["k"], x["v"], x["f"], x["W"], x["wr"], ckpt_every=ck)
    out = m2.backward(x["q"], x["k"], x["v"], x["f"], x["W"], x["wr"], Hck, ck, x["dy"])
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "df", "dW", "dw_r"):
        assert bool(torch.isfinite(out[name]).all()), name
    dwr_ref = (x["dy"].double() * x["v"].double()).sum(dim=(0, 1))
    assert float((out["dw_r"].double() - dwr_ref).abs().max()) <= 1e-3 * max(1.0, float(dwr_ref.abs().max()))
    for b, n in ((B - 1, N - 1), (B - 1, 0), (17, 33), (0, 0)):
        sl = host_slice(x, b, n, with_dy=True)
        gr = oracle.backward(*to_f64(sl), sl["dy"].double().numpy())
        ev = scaled(out["dv"][b:b + 1, :, n:n + 1].cpu(), gr["dv"])
        ef = scaled(out["df"][b:b + 1, :, n:n + 1].cpu(), gr["df"])
        print(f"chain ({b},{n}): dv {ev:.2e} df {ef:.2e}")
        assert ev <= TOL and ef <= TOL
    # dq, dk of the last batch row (sums over its 64 heads), against the oracle
    # on that row; where the row's own half-ulp sensitivity s reaches 1e-3 (a
    # chain whose gradients explode backward in time), the bar is 10 s
    b = B - 1
    row = {k: t[b:b + 1].cpu() for k, t in x.items() if k in ("q", "k", "v", "f", "dy")}
    row.update(W=x["W"].cpu(), wr=x["wr"].cpu())
    ins = to_f64(row)
    gr = oracle.backward(*ins, row["dy"].double().numpy())
    rng = np.random.default_rng(0)
    moved = [a * (1.0 + 2.0 ** -24 * rng.choice([-1.0, 1.0], size=a.shape)) if i in (0, 1, 2, 4) else a
             for i, a in enumerate(ins)]
    gm = oracle.backward(*moved, row["dy"].double().numpy())
    for name in ("dq", "dk"):
        scale = max(1.0, float(np.max(np.abs(gr[name]))))
        sens = float(np.max(np.abs(gm[name] - gr[name]))) / scale
        err = scaled(out[name][b:b + 1].cpu(), gr[name])
        print(f"row {b} {name}: scaled err {err:.2e}, half-ulp sensitivity {sens:.2e}")
        assert err <= (TOL if sens < 1e-3 else 10.0 * sens)
