"""The Python binding checks every tensor before it hands a pointer to the C
ABI: the library sees raw addresses only, so a tensor of another dtype,
shape or device, or a non-contiguous view, would be read as the wrong bytes
(or past the end of its buffer) on the GPU.  On the CPU, with the library
replaced by an object that fails on any use, each mismatch must raise
ValueError before a call is made."""
import pytest
import torch

import m2rnn_inputs
import non_linear_matrix_amd as m2


class NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the C ABI was reached ({name}) before the arguments were checked")


@pytest.fixture
def nolib(monkeypatch):
    monkeypatch.setattr(m2, "lib", NoCalls())


def scan(dtype="bf16", B=2, T=10, N=3):
    x = m2rnn_inputs.make_inputs(B, T, N, dtype=dtype, seed=1, with_dy=True)
    return x


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_forward_checks(nolib):
    x = scan()
    args = [x[n] for n in ("q", "k", "v", "f", "W", "wr")]
    raises("must be on a GPU", m2.forward, *args)
    bad = list(args)
    bad[3] = x["f"].float()                          # f in float32 next to bf16 q
    raises("f has dtype", m2.forward, *bad)
    bad = list(args)
    bad[0] = torch.cat([x["q"], x["q"]], dim=2).chunk(2, dim=2)[0]   # a non-contiguous view
    raises("q must be contiguous", m2.forward, *bad)
    bad = list(args)
    bad[1] = x["k"][:, :5].contiguous()
    raises("k has shape", m2.forward, *bad)
    bad = list(args)
    bad[4] = x["W"][:2].contiguous()
    raises("W has shape", m2.forward, *bad)
    raises("inputs must be float32 or bfloat16", m2.forward, x["q"].double(), *args[1:])
    raises("H_0 has dtype", m2.forward, *args, H_0=torch.zeros(2, 3, 64, 16, dtype=torch.bfloat16))
    raises("H_0 has shape", m2.forward, *args, H_0=torch.zeros(2, 3, 64, 8))
    y, HT = torch.empty(2, 10, 3, 16), torch.empty(2, 3, 64, 16)
    raises("y has shape", m2.forward, *args, out=(torch.empty(2, 10, 3, 8), HT))
    raises("H_T has dtype", m2.forward, *args, out=(y, HT.double()))
    # checkpoints of another interval: ceil(10 / 4) = 3 slots, not ceil(10 / 2) = 5
    raises("H_ckpt has shape", m2.forward, *args, ckpt_every=2, out=(y, HT, torch.empty(2, 3, 3, 64, 16)))
    raises("out holds H_ckpt exactly", m2.forward, *args, ckpt_every=2, out=(y, HT))
    raises("ckpt_every must be >= 0", m2.forward, *args, ckpt_every=-1)


def test_forward_gated_checks(nolib):
    x = scan()
    gt = m2rnn_inputs.make_gate(2, 10, 3, "bf16", seed=1)
    raises("alpha has shape", m2.forward_gated, x["q"], x["k"], x["v"], gt["a"], gt["alpha"][:2].contiguous(),
           gt["beta"], x["W"], x["wr"])
    raises("beta has dtype", m2.forward_gated, x["q"], x["k"], x["v"], gt["a"], gt["alpha"], gt["beta"].float(),
           x["W"], x["wr"])
    raises("must be on a GPU", m2.forward_gated, x["q"], x["k"], x["v"], gt["a"], gt["alpha"], gt["beta"], x["W"],
           x["wr"])


def test_backward_checks(nolib):
    x = scan()
    args = [x[n] for n in ("q", "k", "v", "f", "W", "wr")]
    Hck = torch.zeros(2, 3, 3, 64, 16)          # ckpt_every = 4
    raises("must be on a GPU", m2.backward, *args, Hck, 4, x["dy"])
    raises("H_ckpt has shape", m2.backward, *args, Hck, 2, x["dy"])
    raises("ckpt_every must be >= 1", m2.backward, *args, Hck, 0, x["dy"])
    raises("dy has dtype", m2.backward, *args, Hck, 4, x["dy"].bfloat16())
    raises("dH_T has shape", m2.backward, *args, Hck, 4, x["dy"], dH_T=torch.zeros(2, 3, 64, 15))
    out = dict(dq=torch.empty(2, 10, 64), dk=torch.empty(2, 10, 64), dv=torch.empty(2, 10, 3, 16),
               dW=torch.empty(3, 16, 16), dw_r=torch.empty(3, 16))
    raises("out has no df", m2.backward, *args, Hck, 4, x["dy"], out=out)
    out["df"] = torch.empty(2, 10, 3, dtype=torch.bfloat16)
    raises("df has dtype", m2.backward, *args, Hck, 4, x["dy"], out=out)
    out["df"] = torch.empty(2, 10, 3)
    out["dH_0"] = torch.empty(2, 3, 64, 16).transpose(2, 3).contiguous().transpose(2, 3)
    raises("dH_0 must be contiguous", m2.backward, *args, Hck, 4, x["dy"], out=out)
    bad = list(args)
    bad[2] = x["v"].float()
    raises("v has dtype", m2.backward, *bad, Hck, 4, x["dy"])


def test_decode_checks(nolib):
    x = scan()
    q, k = x["q"][:, 0].contiguous(), x["k"][:, 0].contiguous()
    v, f = x["v"][:, 0].contiguous(), x["f"][:, 0].contiguous()
    raises("H has shape", m2.decode, q, k, v, f, x["W"], x["wr"], torch.zeros(2, 3, 64, 8))
    raises("H has dtype", m2.decode, q, k, v, f, x["W"], x["wr"], torch.zeros(2, 3, 64, 16, dtype=torch.bfloat16))
    raises("f has shape", m2.decode, q, k, v, f[:, :2].contiguous(), x["W"], x["wr"], torch.zeros(2, 3, 64, 16))
    raises("must be on a GPU", m2.decode, q, k, v, f, x["W"], x["wr"], torch.zeros(2, 3, 64, 16))


def test_epilogue_checks(nolib):
    e = m2rnn_inputs.make_epilogue(2, 5, 4, "bf16", seed=1)
    raises("must be on a GPU", m2.gate_rmsnorm_forward, e["y"], e["g"], e["w"])
    raises("g has shape", m2.gate_rmsnorm_forward, e["y"], e["g"][:, :4].contiguous(), e["w"])
    raises("y has dtype", m2.gate_rmsnorm_forward, e["y"].bfloat16(), e["g"], e["w"])
    raises("w has dtype", m2.gate_rmsnorm_forward, e["y"], e["g"], e["w"].float())
    raises("w has shape", m2.gate_rmsnorm_forward, e["y"], e["g"], e["w"].reshape(-1)[:60].contiguous())
    raises("rstd has shape", m2.gate_rmsnorm_forward, e["y"], e["g"], e["w"], rstd=torch.empty(2, 4))
    raises("dout has dtype", m2.gate_rmsnorm_backward, e["y"], e["g"], e["w"], e["dout"].double())
    raises("dg has shape", m2.gate_rmsnorm_backward, e["y"], e["g"], e["w"], e["dout"],
           out=(torch.empty(2, 5, 4, 16), torch.empty(2, 5, 4, 8), torch.empty(64)))
    raises("must be on a GPU", m2.gate_rmsnorm_backward_noalloc, e["y"], e["g"], e["w"], e["dout"])


def test_prologue_checks(nolib):
    c = m2rnn_inputs.make_conv(2, 9, 8, "bf16", seed=1)
    raises("must be on a GPU", m2.conv_silu_forward, c["u"], c["w"], c["bias"])
    raises("w has shape", m2.conv_silu_forward, c["u"], c["w"][:, :3].contiguous(), c["bias"])
    raises("bias has dtype", m2.conv_silu_forward, c["u"], c["w"], c["bias"].float())
    raises("dz has dtype", m2.conv_silu_backward, c["u"], c["w"], c["bias"], c["dz"].bfloat16())
    raises("du has shape", m2.conv_silu_backward, c["u"], c["w"], c["bias"], c["dz"],
           out=(torch.empty(2, 9, 4), torch.empty(8, 4), torch.empty(8)))
