"""Plant plausible slips in copies of the oracle source and check that the pins
catch every one (CPU only; the real oracle is never modified).

Each mutant is one textual edit of oracle/m2rnn_ref.c, compiled with gcc into a
temporary library and run through the pin suite of tests/oracle_pins.py.  A
mutant that passes every pin would mean the pins cannot tell that slip from the
method, so the test fails.
"""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SRC = oracle_build.SRC

# (id, text in the oracle, replacement): one slip each
MUTANTS = [
    ("drop_rank1_write", "A[i * V + j] = s + kt[i] * vt[j];", "A[i * V + j] = s;"),
    ("transposed_W_forward", "s += Hp[i * V + l] * Wn[l * V + j];", "s += Hp[i * V + l] * Wn[j * V + l];"),
    ("gate_swapped", "Hn[e] = ft * Hp[e] + (1.0 - ft) * Z[e];", "Hn[e] = (1.0 - ft) * Hp[e] + ft * Z[e];"),
    ("gate_drops_history", "Hn[e] = ft * Hp[e] + (1.0 - ft) * Z[e];", "Hn[e] = (1.0 - ft) * Z[e];"),
    ("readout_of_old_state", "memcpy(H, Hn, sizeof(double) * S);\n      readout(J, b, n, t, H);",
     "readout(J, b, n, t, H);\n      memcpy(H, Hn, sizeof(double) * S);"),
    ("drop_value_residual", "yt[j] = s + wrn[j] * vt[j];", "yt[j] = s;"),
    ("readout_uses_k", "const double* qt = J->q + ((size_t)b * T + t) * K;\n  const double* vt",
     "const double* qt = J->k + ((size_t)b * T + t) * K;\n  const double* vt"),
    ("ckpt_after_step", "memcpy(dst, H, sizeof(double) * S);", "memcpy(dst, H, sizeof(double) * S); dst[0] += 1e-3;"),
    ("R_drops_future_gradient", "R[i * V + j] = C[i * V + j] + qt[i] * u[j];", "R[i * V + j] = qt[i] * u[j];"),
    ("C_drops_DW", "C[i * V + l] = ft * R[i * V + l] + a;", "C[i * V + l] = ft * R[i * V + l];"),
    ("C_drops_direct_path", "C[i * V + l] = ft * R[i * V + l] + a;", "C[i * V + l] = a;"),
    ("C_transposed_W", "a += D[i * V + j] * Wn[l * V + j];", "a += D[i * V + j] * Wn[j * V + l];"),
    ("D_drops_gate", "D[e] = ((1.0 - ft) * R[e]) * (1.0 - Z[e] * Z[e]);", "D[e] = R[e] * (1.0 - Z[e] * Z[e]);"),
    ("D_wrong_tanh_derivative", "D[e] = ((1.0 - ft) * R[e]) * (1.0 - Z[e] * Z[e]);",
     "D[e] = ((1.0 - ft) * R[e]) * (1.0 - Z[e]);"),
    ("df_wrong_sign", "s += R[e] * (Hp[e] - Z[e]);", "s += R[e] * (Z[e] - Hp[e]);"),
    ("df_uses_new_state", "s += R[e] * (Hp[e] - Z[e]);", "s += R[e] * (Hc[e] - Z[e]);"),
    ("dW_uses_new_state", "a += Hp[i * V + l] * D[i * V + j];", "a += Hc[i * V + l] * D[i * V + j];"),
    ("dW_transposed", "dWc[l * V + j] += a;", "dWc[j * V + l] += a;"),
    ("dq_uses_old_state", "a += Hc[i * V + j] * u[j];", "a += Hp[i * V + j] * u[j];"),
    ("dk_drops_v", "a += D[i * V + j] * vt[j];", "a += D[i * V + j];"),
    ("dv_drops_residual", "dvt[j] = a + wrn[j] * u[j];", "dvt[j] = a;"),
    ("dwr_drops_v", "dwrc[j] += u[j] * vt[j];", "dwrc[j] += u[j];"),
    ("ignores_dH_T", "if (J->dH_T) memcpy(C,", "if (0) memcpy(C,"),
    ("dq_keeps_last_head", "sq += J.dq_part", "sq = J.dq_part"),
    ("dk_keeps_last_head", "sk += J.dk_part", "sk = J.dk_part"),
    ("dW_keeps_last_batch", "s += J.dW_part", "s = J.dW_part"),
    ("forward_ignores_H0", "if (J->H_0) memcpy(H, J->H_0", "if (0) memcpy(H, J->H_0"),
    ("backward_replay_ignores_H0", "if (J->H_0) memcpy(Hs, J->H_0", "if (0) memcpy(Hs, J->H_0"),
    ("dH0_is_R", "if (J->dH_0) memcpy(J->dH_0 + ((size_t)b * N + n) * S, C,",
     "if (J->dH_0) memcpy(J->dH_0 + ((size_t)b * N + n) * S, R,"),
    ("H0_of_wrong_head", "memcpy(H, J->H_0 + ((size_t)b * N + n) * S", "memcpy(H, J->H_0 + ((size_t)b * N + (n + 1) % N) * S"),
    ("softplus_naive", "return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));", "return log(1.0 + exp(x));"),
    ("softplus_drops_linear_part", "return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));", "return log1p(exp(-fabs(x)));"),
    ("gate_sign", "f[i] = exp(-alpha[n] * softplus(a[i] + beta[n]));", "f[i] = exp(alpha[n] * softplus(a[i] + beta[n]));"),
    ("gate_beta_subtracted", "f[i] = exp(-alpha[n] * softplus(a[i] + beta[n]));", "f[i] = exp(-alpha[n] * softplus(a[i] - beta[n]));"),
    ("da_drops_f", "da[i] = df[i] * f * (-alpha[n]) * sig;", "da[i] = df[i] * (-alpha[n]) * sig;"),
    ("da_wrong_derivative", "da[i] = df[i] * f * (-alpha[n]) * sig;", "da[i] = df[i] * f * (-alpha[n]) * (1.0 - sig);"),
    ("dalpha_drops_f", "dalpha[n] += df[i] * f * (-sp);", "dalpha[n] += df[i] * (-sp);"),
    ("dbeta_is_df", "dbeta[n] += da[i];", "dbeta[n] += df[i];"),
    ("norm_drops_mean", "const double s = 1.0 / sqrt(ss / d + eps);\n    for (int j = 0; j < d; ++j) o[",
     "const double s = 1.0 / sqrt(ss + eps);\n    for (int j = 0; j < d; ++j) o["),
    ("norm_eps_outside_root", "const double s = 1.0 / sqrt(ss / d + eps);\n    for (int j = 0; j < d; ++j) o[",
     "const double s = 1.0 / sqrt(ss / d) + eps;\n    for (int j = 0; j < d; ++j) o["),
    ("norm_forward_drops_gate", "o[(size_t)t * d + j] = w[j] * (yt[j] * gt[j]) * s;", "o[(size_t)t * d + j] = w[j] * yt[j] * s;"),
    ("norm_forward_drops_weight", "o[(size_t)t * d + j] = w[j] * (yt[j] * gt[j]) * s;",
     "o[(size_t)t * d + j] = (yt[j] * gt[j]) * s;"),
    ("norm_dx_drops_r", "const double dx = s * (w[j] * dt[j]) - r * s * s * s * x[j] / d;",
     "const double dx = s * (w[j] * dt[j]);"),
    ("norm_dx_s_squared", "const double dx = s * (w[j] * dt[j]) - r * s * s * s * x[j] / d;",
     "const double dx = s * (w[j] * dt[j]) - r * s * s * x[j] / d;"),
    ("norm_dx_drops_weight", "const double dx = s * (w[j] * dt[j]) - r * s * s * s * x[j] / d;",
     "const double dx = s * dt[j] - r * s * s * s * x[j] / d;"),
    ("norm_r_drops_weight", "r += (w[j] * dt[j]) * x[j];", "r += dt[j] * x[j];"),
    ("norm_dy_uses_y", "dy[(size_t)t * d + j] = dx * gt[j];", "dy[(size_t)t * d + j] = dx * yt[j];"),
    ("norm_dg_uses_g", "dg[(size_t)t * d + j] = dx * yt[j];", "dg[(size_t)t * d + j] = dx * gt[j];"),
    ("norm_dw_drops_s", "dw[j] += dt[j] * x[j] * s;", "dw[j] += dt[j] * x[j];"),
    ("norm_dw_uses_y", "dw[j] += dt[j] * x[j] * s;", "dw[j] += dt[j] * yt[j] * s;"),
    ("conv_taps_reversed", "if (ts >= 0) a += w[c * CONV_W + j] * u[((size_t)b * T + ts) * C + c];",
     "if (ts >= 0) a += w[c * CONV_W + (CONV_W - 1 - j)] * u[((size_t)b * T + ts) * C + c];"),
    ("conv_not_causal", "    const int ts = t - (CONV_W - 1) + j;\n    if (ts >= 0) a +=",
     "    const int ts = t + j;\n    if (ts < T) a +="),
    ("conv_drops_bias", "double a = bias ? bias[c] : 0.0;", "double a = 0.0;"),
    ("conv_sigmoid_for_silu", "z[((size_t)b * T + t) * C + c] = a / (1.0 + exp(-a));",
     "z[((size_t)b * T + t) * C + c] = 1.0 / (1.0 + exp(-a));"),
    ("conv_silu_derivative_is_sigmoid", "da[t] = dz[((size_t)b * T + t) * C + c] * s * (1.0 + a * (1.0 - s));",
     "da[t] = dz[((size_t)b * T + t) * C + c] * s;"),
    ("conv_du_forward_taps", "const int to = t + (CONV_W - 1) - j;", "const int to = t + j;"),
    ("conv_dw_wrong_shift", "          const int ts = t - (CONV_W - 1) + j;\n          if (ts >= 0) dw[",
     "          const int ts = t - j;\n          if (ts >= 0) dw["),
    ("conv_dbias_is_dz", "if (dbias) dbias[c] += da[t];", "if (dbias) dbias[c] += dz[((size_t)b * T + t) * C + c];"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as fh:
        return fh.read()


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, mid, old, new):
    assert source.count(old) == 1, f"mutation anchor for {mid} must occur exactly once in the oracle"
    mutated = source.replace(old, new)
    src = tmp_path / "m2rnn_ref.c"
    src.write_text(mutated)
    # the header sits next to the real source
    lib = oracle_build.build(str(src), str(tmp_path / f"lib_{mid}.so"),
                             extra_flags=("-I" + os.path.dirname(SRC),))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError as exc:
            caught.append(f"{pin.__name__}: {exc}")
            break
    assert caught, f"mutant {mid} passed every pin"
