"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU, run
the oracle on the same (bf16-rounded) values, compare."""
import numpy as np
import torch

import m2rnn_inputs
import oracle

NAMES = ("q", "k", "v", "f", "W", "wr")
# parity bars: max-abs on y and H_T, 1e-4 for float32 inputs, 5e-3 for bfloat16
TOL = {"f32": 1e-4, "bf16": 5e-3}


def to_gpu(x):
    return {n: t.cuda() for n, t in x.items()}


def to_f64(x, names=NAMES):
    return [x[n].double().numpy() for n in names]


def chain_slice(x, b, n):
    """Inputs of the single chain (b, n): the recurrence of one head of one
    batch row depends on nothing else."""
    return dict(q=x["q"][b:b + 1], k=x["k"][b:b + 1], v=x["v"][b:b + 1, :, n:n + 1],
                f=x["f"][b:b + 1, :, n:n + 1], W=x["W"][n:n + 1], wr=x["wr"][n:n + 1])


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def make(B, T, N, dtype="f32", f_mu=2.0, seed=0, with_dy=False):
    return m2rnn_inputs.make_inputs(B, T, N, dtype=dtype, f_mu=f_mu, seed=seed, with_dy=with_dy)


def oracle_forward(x, ckpt_every=0):
    return oracle.forward(*to_f64(x), ckpt_every=ckpt_every)


def batch_rows(x, b0, b1, with_dy=False):
    """Inputs of batch rows b0 .. b1-1 with every head (rows never interact
    in the forward; W and w_r are shared and kept whole)."""
    out = dict(q=x["q"][b0:b1], k=x["k"][b0:b1], v=x["v"][b0:b1], f=x["f"][b0:b1], W=x["W"], wr=x["wr"])
    if with_dy:
        out["dy"] = x["dy"][b0:b1]
    return out
