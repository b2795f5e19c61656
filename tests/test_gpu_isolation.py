"""A non-finite value in one (b, n) chain stays in that chain.

Each (batch row, head) chain of the recurrence (slide "Write, transform,
retain, and read a matrix state", paper Eqs. (10)-(12)) depends on nothing
but its own inputs, q and k of its batch row, and its head's W and w_r.  So a
NaN or an infinity in one chain's v, f or dy may reach that chain's outputs
and the sums it takes part in (dq and dk of its batch row, summed over heads;
dW and dw_r of its head, summed over batch rows), and nothing else: every
other output must be bit-identical to a run without it.  The shape puts the
poisoned head in a four-head sweep workgroup and a two-head forward
workgroup with clean neighbours."""
import numpy as np
import pytest
import torch

import non_linear_matrix_amd as m2
from gpu_common import make, to_gpu

pytestmark = pytest.mark.gpu

B, T, N, CK = 2, 40, 520, 16
B0, N0 = 1, 5   # the poisoned chain


def run(x):
    g = to_gpu(x)
    y, HT, Hck = m2.forward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], ckpt_every=CK)
    out = m2.backward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"], Hck, CK, g["dy"])
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in out.items()}
    res.update(y=y.cpu(), H_T=HT.cpu(), H_ckpt=Hck.cpu())
    return res


def clean_mask(name, shape):
    """True where an output does not depend on chain (B0, N0)."""
    m = torch.ones(shape, dtype=torch.bool)
    if name in ("y", "dv", "df"):
        m[B0, :, N0] = False
    elif name in ("H_T", "H_ckpt"):
        m[B0, N0] = False
    elif name in ("dq", "dk"):
        m[B0] = False
    elif name in ("dW", "dw_r"):
        m[N0] = False
    return m


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_nonfinite_chain_is_isolated(dtype, bad):
    print(f"isolation {dtype} bad={bad}", flush=True)
    x = make(B, T, N, dtype, seed=61, with_dy=True)
    # the clean run holds 0 where the poisoned one holds `bad`, so that the
    # largest finite |dy| (the bf16 backward's gradient scale) is the same in both
    x["dy"][B0, 30, N0, 3] = 0.0
    base = run(x)
    p = {k: v.clone() for k, v in x.items()}
    p["v"][B0, 10:12, N0, :] = bad
    p["f"][B0, 20, N0] = bad
    p["dy"][B0, 30, N0, 3] = bad
    got = run(p)
    for name, t in base.items():
        m = clean_mask(name, t.shape)
        same = torch.equal(got[name][m], t[m])
        assert same, f"{name}: an output outside chain ({B0}, {N0}) changed"
    # the poison did reach its own chain
    assert not bool(torch.isfinite(got["y"][B0, :, N0]).all())
    assert bool(torch.isfinite(base["y"]).all())
