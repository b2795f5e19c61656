"""Sizes the M2RNN slides print, against the input generator and the oracle."""
import json
import os

import numpy as np

import m2rnn_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def facts():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_state_and_transition_sizes():
    fx = facts()
    assert m2rnn_inputs.K_DIM == fx["K"] and m2rnn_inputs.V_DIM == fx["V"]
    assert fx["K"] * fx["V"] == fx["state_elements_per_head"]
    assert fx["V"] ** 2 == fx["transition_parameters_per_head"]
    x = m2rnn_inputs.make_inputs(1, 3, 2)
    assert tuple(x["W"].shape[1:]) == (fx["V"], fx["V"])
    # one q and one k per token, shared by every value head
    assert tuple(x["q"].shape) == (1, 3, fx["K"]) and tuple(x["k"].shape) == (1, 3, fx["K"])
    _, HT = oracle.get().forward(*(x[n].double().numpy() for n in ("q", "k", "v", "f", "W", "wr")))
    assert HT.shape == (1, 2, fx["K"], fx["V"])


def test_initial_state_is_zero():
    """H_0 = 0: the checkpoint at t = 0 is exactly the printed initial state."""
    x = m2rnn_inputs.make_inputs(2, 5, 3)
    ins = [x[n].double().numpy() for n in ("q", "k", "v", "f", "W", "wr")]
    _, _, ck = oracle.get().forward(*ins, ckpt_every=2)
    assert np.all(ck[:, :, 0] == facts()["initial_state"])


def test_generator_is_seeded_and_rounded():
    a = m2rnn_inputs.make_inputs(1, 4, 2, dtype="bf16", seed=3, with_dy=True)
    b = m2rnn_inputs.make_inputs(1, 4, 2, dtype="bf16", seed=3, with_dy=True)
    for n in a:
        assert a[n].equal(b[n])
    assert a["q"].dtype.is_floating_point and str(a["q"].dtype) == "torch.bfloat16"
    assert str(a["dy"].dtype) == "torch.float32"
    f32 = m2rnn_inputs.make_inputs(1, 4, 2, dtype="f32", seed=3)
    assert f32["q"].to(a["q"].dtype).equal(a["q"])  # bf16 = RNE rounding of the same draws
    assert float(a["f"].float().min()) > 0.0 and float(a["f"].float().max()) < 1.0
