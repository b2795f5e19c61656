"""Seeded synthetic inputs for the M2RNN scan (shared by the oracle side and the
HIP side of every test and of the benchmark).

This module holds none of the method's arithmetic: it only draws random
tensors.  The distributions stand in for the activations the paper's layer
feeds the scan (slide "Most of the block can be computed before recurrence",
paper Fig. 2: q, k, v come out of a SiLU; the forget gate lies in [0, 1]):

    q, k = SiLU(N(0,1))            [B, T, K]   shared by the N value heads
    v    = SiLU(N(0,1))            [B, T, N, V]
    f    = sigmoid(N(mu, 1))       [B, T, N]   mu = 2 (mu = 3: long retention)
    W    = N(0, 1/16)              [N, V, V]   (standard deviation 0.25)
    w_r  = N(0, 1)                 [N, V]
    dy   = N(0, 1)                 [B, T, N, V]  (float32, backward only)

For the gated scan (f computed in the kernel from a pre-activation, slide
"The gate preserves a direct path through time", paper Eqs. (13), (17)),
make_gate draws, from its own generator:

    a     = N(-mu, 1)              [B, T, N]   mu = 2: with alpha = 1, beta = 0
                                               f has the distribution above
    alpha = U[0.5, 2)              [N]
    beta  = U[-1, 1)               [N]

For the output gate and RMSNorm after the readout (slide "Most of the block
can be computed before recurrence", paper Fig. 2), make_epilogue draws, from
its own generator, in this order:

    y    = 3 N(0, 1)               [B, T, N, V]  float32 (the scale of a readout)
    g    = sigmoid(N(0, 1))        [B, T, N, V]  output gate
    w    = 1 + N(0, 1/100)         [N, V]        RMSNorm weight
    dout = N(0, 1)                 [B, T, N, V]  float32

For the causal Conv1D and SiLU before the scan, make_conv draws, from its own
generator, in this order (the taps and bias as a width-4 conv layer's default
initialisation, U(-1/2, 1/2)):

    u    = N(0, 1)                 [B, T, C]   projected q, k or v
    w    = U(-1/2, 1/2)            [C, 4]
    bias = U(-1/2, 1/2)            [C]
    dz   = N(0, 1)                 [B, T, C]   float32

Draw order is fixed (q, k, v, f, W, w_r, dy) from one CPU torch.Generator
seeded with `seed`; every tensor is drawn in float32 and, for bfloat16
workloads, rounded to bfloat16 with round-to-nearest-even.  dy stays float32.
"""
from dataclasses import dataclass

import torch

K_DIM = 64
V_DIM = 16


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    N: int
    dtype: str = "f32"      # dtype of q, k, v, f, W, w_r: "f32" or "bf16"
    f_mu: float = 2.0       # mean of the pre-sigmoid forget-gate logits
    backward: bool = False  # also draw dy
    ckpt_every: int = 0     # state checkpoint interval for the backward
    K: int = K_DIM
    V: int = V_DIM

    @property
    def head_tokens(self):
        return self.B * self.T * self.N


WORKLOADS = {
    "fwd_f32_B1_T256_N4": Workload("fwd_f32_B1_T256_N4", 1, 256, 4, "f32"),
    "fwd_bf16_B8_T2048_N16": Workload("fwd_bf16_B8_T2048_N16", 8, 2048, 16, "bf16"),
    "fwd_bf16_B2_T32768_N32": Workload("fwd_bf16_B2_T32768_N32", 2, 32768, 32, "bf16", f_mu=3.0),
    "fwd_bf16_B32_T4096_N64": Workload("fwd_bf16_B32_T4096_N64", 32, 4096, 64, "bf16"),
    "fwdbwd_bf16_B8_T2048_N16": Workload("fwdbwd_bf16_B8_T2048_N16", 8, 2048, 16, "bf16",
                                         backward=True, ckpt_every=64),
    # the headline shape, forward + backward
    "fwdbwd_bf16_B32_T4096_N64": Workload("fwdbwd_bf16_B32_T4096_N64", 32, 4096, 64, "bf16",
                                          backward=True, ckpt_every=64),
}


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(B, T, N, K=K_DIM, V=V_DIM, dtype="f32", f_mu=2.0, seed=0, with_dy=False):
    """Draw one seeded input set.  Returns a dict of CPU tensors: q, k, v, f, W,
    wr in `dtype` (float32 or bfloat16) and, if `with_dy`, dy in float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    td = torch_dtype(dtype)

    def draw(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32)

    out = {}
    out["q"] = torch.nn.functional.silu(draw(B, T, K))
    out["k"] = torch.nn.functional.silu(draw(B, T, K))
    out["v"] = torch.nn.functional.silu(draw(B, T, N, V))
    out["f"] = torch.sigmoid(draw(B, T, N) + f_mu)
    out["W"] = draw(N, V, V) * 0.25
    out["wr"] = draw(N, V)
    for name in ("q", "k", "v", "f", "W", "wr"):
        out[name] = out[name].to(td).contiguous()
    if with_dy:
        out["dy"] = draw(B, T, N, V).contiguous()
    return out


def make_inputs_on(device, B, T, N, K=K_DIM, V=V_DIM, dtype="f32", f_mu=2.0, seed=0, with_dy=False):
    """make_inputs drawn on `device` from a generator of that device: the same
    distributions and draw order (on the CPU the same numbers; a GPU's
    generator gives another stream).  For sizes too large to draw on the host
    (tensors of billions of elements)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    td = torch_dtype(dtype)

    def draw(*shape):
        return torch.randn(*shape, generator=g, dtype=torch.float32, device=device)

    out = {}
    out["q"] = torch.nn.functional.silu(draw(B, T, K)).to(td)
    out["k"] = torch.nn.functional.silu(draw(B, T, K)).to(td)
    out["v"] = torch.nn.functional.silu(draw(B, T, N, V)).to(td)
    out["f"] = torch.sigmoid(draw(B, T, N) + f_mu).to(td)
    out["W"] = (draw(N, V, V) * 0.25).to(td)
    out["wr"] = draw(N, V).to(td)
    if with_dy:
        out["dy"] = draw(B, T, N, V)
    return {n: t.contiguous() for n, t in out.items()}


def make_workload(w: Workload, seed=0, with_dy=None):
    return make_inputs(w.B, w.T, w.N, w.K, w.V, w.dtype, w.f_mu, seed,
                       w.backward if with_dy is None else with_dy)


def make_state(B, N, K=K_DIM, V=V_DIM, seed=0):
    """A seeded float32 state [B,N,K,V] drawn uniformly from [-1, 1) (the range
    every state takes when f lies in [0, 1]): an initial state H_0, or a
    gradient dH_T, for the resumable scan."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.rand(B, N, K, V, generator=g, dtype=torch.float32) * 2.0 - 1.0).contiguous()


def make_gate(B, T, N, dtype="f32", mu=2.0, seed=0):
    """Seeded gate inputs for the gated scan: dict of CPU tensors a [B,T,N],
    alpha [N], beta [N] in `dtype` (drawn in float32, then rounded)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    td = torch_dtype(dtype)
    a = torch.randn(B, T, N, generator=g, dtype=torch.float32) - mu
    alpha = torch.rand(N, generator=g, dtype=torch.float32) * 1.5 + 0.5
    beta = torch.rand(N, generator=g, dtype=torch.float32) * 2.0 - 1.0
    return {"a": a.to(td).contiguous(), "alpha": alpha.to(td).contiguous(), "beta": beta.to(td).contiguous()}


def make_epilogue(B, T, N, dtype="f32", seed=0, V=V_DIM):
    """Seeded inputs of the output gate and RMSNorm: dict of CPU tensors y,
    dout (float32) and g, w in `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 104729)
    td = torch_dtype(dtype)
    y = torch.randn(B, T, N, V, generator=g, dtype=torch.float32) * 3.0
    gate = torch.sigmoid(torch.randn(B, T, N, V, generator=g, dtype=torch.float32))
    w = 1.0 + 0.1 * torch.randn(N, V, generator=g, dtype=torch.float32)
    dout = torch.randn(B, T, N, V, generator=g, dtype=torch.float32)
    return {"y": y.contiguous(), "g": gate.to(td).contiguous(), "w": w.to(td).contiguous(), "dout": dout.contiguous()}


def make_conv(B, T, C, dtype="f32", seed=0):
    """Seeded inputs of the causal Conv1D and SiLU: dict of CPU tensors u, w,
    bias in `dtype` and dz in float32."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 1299709)
    td = torch_dtype(dtype)
    u = torch.randn(B, T, C, generator=g, dtype=torch.float32)
    w = torch.rand(C, 4, generator=g, dtype=torch.float32) - 0.5
    bias = torch.rand(C, generator=g, dtype=torch.float32) - 0.5
    dz = torch.randn(B, T, C, generator=g, dtype=torch.float32)
    return {"u": u.to(td).contiguous(), "w": w.to(td).contiguous(), "bias": bias.to(td).contiguous(),
            "dz": dz.contiguous()}
