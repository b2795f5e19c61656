"""The GPU's tanh, through the C ABI.

The candidate Z_t = tanh(H_{t-1} W + k_t v_t^T) (slide "Write, transform,
retain, and read a matrix state", paper Eq. (10)) is computed in the kernels
as 1 - 2 / (1 + 2^{x 2/ln 2}) with v_exp_f32 and v_rcp_f32, folded into the
gate.  With T = 1, f = 0 and W = 0 the state after one step is
H_1 = tanh(k v^T) exactly, so H_T pins that formula against the oracle's
libm tanh in double: on a dense grid of arguments over [-10, 10], on
|x| < 1e-3 (where 1 - 2r cancels), and for |x| >= 20 (saturation, including
arguments whose exponential overflows fp32)."""
import numpy as np
import pytest
import torch

import non_linear_matrix_amd as m2
import oracle

pytestmark = pytest.mark.gpu

B, N = 8, 16
BOUND = 1e-6


def tanh_inputs(dtype):
    """k[b, 0, :] holds the arguments' first factor per batch row, v[b, 0, n, :]
    = 1 + (16 n + j) / 4096 the second, so each row spans its range 256 times
    with small shifts."""
    k = np.zeros((B, 1, 64))
    for b in range(4):   # rows 0..3: a 256-point grid over [-10, 10], interleaved
        k[b, 0] = -10.0 + 20.0 * (4 * np.arange(64) + b) / 255.0
    k[4, 0] = np.linspace(-1e-3, 1e-3, 64)
    k[5, 0] = np.linspace(20.0, 100.0, 64)
    k[6, 0] = -np.linspace(20.0, 100.0, 64)
    special = [0.0, 1e-30, -1e-30, 1e-8, -1e-8, 44.3, -44.3, 44.5, -44.5, 88.7, -88.7, 200.0, -200.0, 1e4, -1e4,
               3e38, -3e38, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 5.0, -5.0]
    k[7, 0, :len(special)] = special
    j = np.arange(16)
    v = np.zeros((B, 1, N, 16))
    for n in range(N):
        v[:, 0, n, :] = 1.0 + (16 * n + j) / 4096.0
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    x = dict(q=torch.zeros(B, 1, 64), k=torch.from_numpy(k).float(), v=torch.from_numpy(v).float(),
             f=torch.zeros(B, 1, N), W=torch.zeros(N, 16, 16), wr=torch.zeros(N, 16))
    return {n: t.to(td).contiguous() for n, t in x.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tanh_bound(dtype):
    x = tanh_inputs(dtype)
    g = {n: t.cuda() for n, t in x.items()}
    _, HT = m2.forward(g["q"], g["k"], g["v"], g["f"], g["W"], g["wr"])
    torch.cuda.synchronize()
    HT = HT.cpu().numpy().astype(np.float64)
    _, ref = oracle.forward(*[x[n].double().numpy() for n in ("q", "k", "v", "f", "W", "wr")])
    err = np.abs(HT - ref)
    for name, rows in (("grid [-10, 10]", slice(0, 4)), ("|x| < 1e-3", slice(4, 5)), ("|x| >= 20", slice(5, 7)),
                       ("special", slice(7, 8))):
        print(f"{dtype} {name}: max |H_T - tanh| = {err[rows].max():.3e}")
    assert err.max() <= BOUND
    assert np.abs(HT).max() <= 1.0
    # exact saturation where 2^{x 2/ln 2} overflows or dwarfs 1, and an exact zero at x = 0
    kk = x["k"].double().numpy()[:, 0, :]                                  # [B, 64]
    vv = x["v"].double().numpy()[:, 0, :, :]                               # [B, N, 16]
    xs = kk[:, None, :, None] * vv[:, :, None, :]                          # [B, N, 64, 16]
    assert np.all(HT[np.abs(xs) >= 20.0] == np.sign(xs[np.abs(xs) >= 20.0]))
    assert np.all(HT[xs == 0.0] == 0.0)
