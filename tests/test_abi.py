"""The C-ABI library on the CPU: it loads, exports every entry point that
include/m2rnn.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "m2rnn.h")


def declared():
    with open(HEADER) as fh:
        src = fh.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(m2rnn_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def m2():
    import non_linear_matrix_amd
    return non_linear_matrix_amd


def test_header_declares_the_entry_points():
    assert declared() == ["m2rnn_backward", "m2rnn_backward_gated", "m2rnn_backward_workspace_bytes",
                          "m2rnn_conv_silu_backward", "m2rnn_conv_silu_backward_workspace_bytes",
                          "m2rnn_conv_silu_forward", "m2rnn_decode", "m2rnn_forward", "m2rnn_forward_gated",
                          "m2rnn_forward_workspace_bytes",
                          "m2rnn_gate_rmsnorm_backward", "m2rnn_gate_rmsnorm_backward_noalloc",
                          "m2rnn_gate_rmsnorm_backward_workspace_bytes", "m2rnn_gate_rmsnorm_forward",
                          "m2rnn_last_error"]


def test_library_exports_every_declared_symbol(m2):
    lib = ctypes.CDLL(m2.LIB_PATH)
    for name in declared():
        assert hasattr(lib, name), name


def test_workspace_query(m2):
    ws = m2.m2rnn_backward_workspace_bytes
    assert ws(2, 100, 5, 64, 16, 64) > 0
    assert ws(2, 100, 5, 64, 16, 64) % 256 == 0
    # the 4-step replay states are only needed when checkpoints are sparser
    assert ws(2, 100, 5, 64, 16, 4) < ws(2, 100, 5, 64, 16, 8) == ws(2, 100, 5, 64, 16, 64)
    assert ws(2, 100, 5, 64, 16, 1) == ws(2, 100, 5, 64, 16, 4)
    assert ws(2, 100, 5, 32, 16, 64) == 0 and ws(2, 100, 5, 64, 16, 0) == 0 and ws(0, 100, 5, 64, 16, 64) == 0


def test_forward_workspace(m2):
    """Few chains (B N <= 128) take the row-split forward, whose readout
    partials need B N T 256 bytes of workspace; more chains need none.  A
    missing or short workspace is refused before anything is launched."""
    ws = m2.m2rnn_forward_workspace_bytes
    assert ws(1, 4, 2) == 1 * 2 * 4 * 256 and ws(8, 2048, 16) == 8 * 16 * 2048 * 256
    assert ws(1, 4, 129) == 0 and ws(129, 4, 1) == 0 and ws(32, 4096, 64) == 0
    assert ws(0, 4, 2) == 0 and ws(1, 0, 2) == 0 and ws(1, 4, 2, 32, 16) == 0
    dummy = ctypes.c_void_p(256)   # never dereferenced: the workspace check fails first
    f = m2.lib.m2rnn_forward
    assert f(1, 4, 2, 64, 16, 0, *[dummy] * 6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_WORKSPACE
    assert "workspace" in m2.m2rnn_last_error()
    assert f(1, 4, 2, 64, 16, 0, *[dummy] * 6, None, dummy, dummy, None, 0, dummy, 2047, None) == \
        m2.M2RNN_ERR_WORKSPACE
    assert f(1, 4, 2, 64, 16, 0, *[dummy] * 6, None, dummy, dummy, None, 0, ctypes.c_void_p(256 + 16), 2048, None) == \
        m2.M2RNN_ERR_INVALID_ARG   # 256-byte alignment
    fg = m2.lib.m2rnn_forward_gated
    assert fg(1, 4, 2, 64, 16, 0, *[dummy] * 8, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_WORKSPACE


def test_argument_errors_without_launch(m2):
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    args6 = [dummy] * 6
    f = m2.lib.m2rnn_forward
    assert f(1, 4, 2, 32, 16, 0, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert "K=64" in m2.m2rnn_last_error()
    assert f(1, 4, 2, 64, 8, 0, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert f(1, 4, 2, 64, 16, 5, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert f(-1, 4, 2, 64, 16, 0, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert f(1, 4, 2, 64, 16, 0, None, *args6[1:], None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "q" in m2.m2rnn_last_error()
    odd = ctypes.c_void_p(256 + 4)   # y must be 16-byte aligned
    assert f(1, 4, 2, 64, 16, 0, *args6, None, odd, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert f(1, 4, 2, 64, 16, 0, *args6, None, dummy, dummy, dummy, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert f(1, 4, 2, 64, 16, 0, *args6, None, dummy, dummy, None, -3, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert f(1, 4, 2, 64, 16, 0, *args6, odd, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "H_0" in m2.m2rnn_last_error()
    d = m2.lib.m2rnn_decode
    assert d(1, 2, 64, 16, 0, *args6, None, dummy, None) == m2.M2RNN_ERR_INVALID_ARG   # H is required
    assert d(1, 2, 32, 16, 0, *args6, dummy, dummy, None) == m2.M2RNN_ERR_UNSUPPORTED
    b = m2.lib.m2rnn_backward
    grads = [dummy] * 6
    assert b(1, 4, 2, 64, 16, 0, *args6, dummy, 0, dummy, None, *grads, None, dummy, 1 << 30, None) == \
        m2.M2RNN_ERR_INVALID_ARG          # ckpt_every must be >= 1
    assert b(1, 4, 2, 64, 16, 0, *args6, dummy, 64, dummy, None, *grads, None, dummy, 16, None) == \
        m2.M2RNN_ERR_WORKSPACE            # too small
    assert "workspace" in m2.m2rnn_last_error()
    assert b(1, 4, 2, 64, 16, 0, *args6, dummy, 64, dummy, None, *grads, None, None, 0, None) == m2.M2RNN_ERR_WORKSPACE


def test_size_limits_without_launch(m2):
    """Sizes whose launches would not fit 2^32 work-items are refused before
    anything runs; the largest accepted sizes pass validation (they then fail
    on the missing workspace, not on size)."""
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    args6 = [dummy] * 6
    f = m2.lib.m2rnn_forward
    # B ceil(N/4) < 2^22
    assert f(1 << 20, 1, 16, 64, 16, 0, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert "2^22" in m2.m2rnn_last_error()
    assert f((1 << 20) - 1, 1, 16, 64, 16, 1, *args6, None, None, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "y must" in m2.m2rnn_last_error()
    # B T N V <= 2^40
    assert f(1 << 10, 1 << 20, 128, 64, 16, 0, *args6, None, dummy, dummy, None, 0, None, 0, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert "too large" in m2.m2rnn_last_error()
    d = m2.lib.m2rnn_decode
    assert d(1 << 22, 4, 64, 16, 0, *args6, dummy, dummy, None) == m2.M2RNN_ERR_UNSUPPORTED
    # the backward's replay: B ceil(N/4) ceil(T/ckpt_every) < 2^24 once ckpt_every > 4
    b = m2.lib.m2rnn_backward
    grads = [dummy] * 6
    assert b(1 << 10, 1 << 20, 4, 64, 16, 0, *args6, dummy, 64, dummy, None, *grads, None, dummy, 16, None) == \
        m2.M2RNN_ERR_UNSUPPORTED
    assert "2^24" in m2.m2rnn_last_error()
    assert b(1 << 10, (1 << 20) - 64, 4, 64, 16, 0, *args6, dummy, 64, dummy, None, *grads, None, dummy, 16,
             None) == m2.M2RNN_ERR_WORKSPACE
    assert b(1 << 10, 1 << 20, 4, 64, 16, 0, *args6, dummy, 4, dummy, None, *grads, None, dummy, 16, None) == \
        m2.M2RNN_ERR_WORKSPACE   # states every 4 steps are given: no replay
    ws = m2.m2rnn_backward_workspace_bytes
    assert ws(1 << 20, 1, 16, 64, 16, 64) == 0 and ws((1 << 20) - 1, 1, 16, 64, 16, 64) > 0
    assert ws(1 << 10, 1 << 20, 128, 64, 16, 64) == 0


def test_gated_argument_errors_without_launch(m2):
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    q3 = [dummy] * 3
    fg = m2.lib.m2rnn_forward_gated
    # q, k, v, a, alpha, beta, W, w_r
    assert fg(1, 4, 2, 64, 16, 0, *q3, None, dummy, dummy, dummy, dummy, None, dummy, dummy, None, 0, None, 0, None) \
        == m2.M2RNN_ERR_INVALID_ARG
    assert "a must" in m2.m2rnn_last_error()
    assert fg(1, 4, 2, 64, 16, 0, *q3, dummy, None, dummy, dummy, dummy, None, dummy, dummy, None, 0, None, 0, None) \
        == m2.M2RNN_ERR_INVALID_ARG
    assert "alpha" in m2.m2rnn_last_error()
    assert fg(1, 4, 2, 64, 16, 1, *q3, dummy, dummy, ctypes.c_void_p(257), dummy, dummy, None, dummy, dummy,
              None, 0, None, 0, None, 0, None) == m2.M2RNN_ERR_INVALID_ARG   # bf16 beta needs 2-byte alignment
    assert "beta" in m2.m2rnn_last_error()
    bg = m2.lib.m2rnn_backward_gated
    g3 = [dummy] * 3
    # ... H_ckpt, ckpt_every, dy, dH_T, dq, dk, dv, da, dalpha, dbeta, dW, dw_r, dH_0, ws, bytes, stream
    assert bg(1, 4, 2, 64, 16, 0, *q3, dummy, dummy, dummy, dummy, dummy, dummy, 64, dummy, None, *g3, dummy,
              None, dummy, dummy, dummy, None, dummy, 1 << 30, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "dalpha" in m2.m2rnn_last_error()
    assert bg(1, 4, 2, 64, 16, 0, *q3, dummy, dummy, dummy, dummy, dummy, dummy, 64, dummy, None, *g3, None,
              dummy, dummy, dummy, dummy, None, dummy, 1 << 30, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "da must" in m2.m2rnn_last_error()
    assert bg(1, 4, 2, 64, 16, 0, *q3, dummy, dummy, dummy, dummy, dummy, dummy, 64, dummy, None, *g3, dummy,
              dummy, dummy, dummy, dummy, None, dummy, 16, None) == m2.M2RNN_ERR_WORKSPACE


def test_gate_rmsnorm_argument_errors_without_launch(m2):
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    fwd = m2.lib.m2rnn_gate_rmsnorm_forward
    # B, T, N, V, dtype, y, g, w, eps, out, rstd, stream
    assert fwd(2, 3, 5, 16, 0, dummy, dummy, dummy, ctypes.c_float(-1.0), dummy, None, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "eps" in m2.m2rnn_last_error()
    assert fwd(2, 3, 129, 16, 0, dummy, dummy, dummy, 0.0, dummy, None, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert fwd(2, 3, 1, 3, 0, dummy, dummy, dummy, 0.0, dummy, None, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert fwd(2, 3, 5, 16, 2, dummy, dummy, dummy, 0.0, dummy, None, None) == m2.M2RNN_ERR_INVALID_ARG
    assert fwd(2, 3, 5, 16, 0, None, dummy, dummy, 0.0, dummy, None, None) == m2.M2RNN_ERR_INVALID_ARG
    assert fwd(2, 3, 5, 16, 1, dummy, ctypes.c_void_p(260), dummy, 0.0, dummy, None, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "g must be 8-byte aligned" in m2.m2rnn_last_error()
    assert fwd(2, 3, 5, 16, 0, dummy, dummy, dummy, 0.0, dummy, ctypes.c_void_p(258), None) == \
        m2.M2RNN_ERR_INVALID_ARG
    ws = m2.m2rnn_gate_rmsnorm_backward_workspace_bytes
    # one dw partial row per workgroup of four token rows (at most 1024), then 32 second-level rows
    assert ws(2, 3, 5, 16) == (2 + 32) * 80 * 4 and ws(2, 3, 5, 3) == 0 and ws(0, 3, 5, 16) == 0
    assert ws(64, 4096, 64, 16) == (1024 + 32) * 1024 * 4 and ws(64, 4096, 8, 16) == (1024 + 32) * 128 * 4
    bwd = m2.lib.m2rnn_gate_rmsnorm_backward
    # ..., dout, dy, dg, dw, workspace, bytes, stream
    assert bwd(2, 3, 5, 16, 0, dummy, dummy, dummy, 0.0, dummy, dummy, dummy, dummy, dummy, 16, None) == \
        m2.M2RNN_ERR_WORKSPACE
    assert bwd(2, 3, 5, 16, 0, dummy, dummy, dummy, 0.0, dummy, dummy, None, dummy, dummy, 1 << 20, None) == \
        m2.M2RNN_ERR_INVALID_ARG
    assert "dg" in m2.m2rnn_last_error()
    # the variant without a workspace validates the same way, before it looks up its scratch array
    na = m2.lib.m2rnn_gate_rmsnorm_backward_noalloc
    assert na(2, 3, 5, 16, 0, dummy, dummy, dummy, 0.0, dummy, dummy, None, dummy, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "dg" in m2.m2rnn_last_error()
    assert na(2, 3, 129, 16, 0, dummy, dummy, dummy, 0.0, dummy, dummy, dummy, dummy, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert na(2, 3, 5, 16, 0, dummy, dummy, dummy, ctypes.c_float(-1.0), dummy, dummy, dummy, dummy, None) == \
        m2.M2RNN_ERR_INVALID_ARG
    # its scratch array covers the largest workspace: 1024 partial rows and 32 second-level rows of 2048 floats
    assert ws(64, 4096, 128, 16) == (1024 + 32) * 2048 * 4 == 8650752


def test_conv_silu_argument_errors_without_launch(m2):
    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    fwd = m2.lib.m2rnn_conv_silu_forward
    # B, T, C, dtype, u, w, bias, z, stream
    assert fwd(2, 3, 6, 0, dummy, dummy, None, dummy, None) == m2.M2RNN_ERR_UNSUPPORTED
    assert fwd(2, 3, 8, 3, dummy, dummy, None, dummy, None) == m2.M2RNN_ERR_INVALID_ARG
    assert fwd(-1, 3, 8, 0, dummy, dummy, None, dummy, None) == m2.M2RNN_ERR_INVALID_ARG
    assert fwd(2, 3, 8, 0, None, dummy, None, dummy, None) == m2.M2RNN_ERR_INVALID_ARG
    assert fwd(2, 3, 8, 1, dummy, dummy, ctypes.c_void_p(260), dummy, None) == m2.M2RNN_ERR_INVALID_ARG
    assert "bias" in m2.m2rnn_last_error()
    assert fwd(2, 3, 8, 0, dummy, dummy, None, ctypes.c_void_p(264), None) == m2.M2RNN_ERR_INVALID_ARG
    ws = m2.m2rnn_conv_silu_backward_workspace_bytes
    # R = max(1, min(262144 / (C/4), B * ceil(T/8) / 4)) worker rows, then 32 second-level rows, of 5 C floats
    assert ws(2, 3, 8) == (1 + 32) * 40 * 4 and ws(2, 3, 6) == 0 and ws(0, 3, 8) == 0
    assert ws(32, 4096, 1024) == (1024 + 32) * 5120 * 4 and ws(32, 4096, 64) == (4096 + 32) * 320 * 4
    bwd = m2.lib.m2rnn_conv_silu_backward
    # ..., dz, du, dw, dbias, workspace, bytes, stream
    assert bwd(2, 3, 8, 0, dummy, dummy, None, dummy, dummy, dummy, None, dummy, 16, None) == m2.M2RNN_ERR_WORKSPACE
    assert bwd(2, 3, 8, 0, dummy, dummy, None, dummy, None, dummy, None, dummy, 1 << 20, None) == \
        m2.M2RNN_ERR_INVALID_ARG
    assert "du" in m2.m2rnn_last_error()
    assert bwd(2, 3, 8, 0, dummy, dummy, None, dummy, dummy, dummy, ctypes.c_void_p(260), dummy, 1 << 20, None) == \
        m2.M2RNN_ERR_INVALID_ARG


def test_size_validation_property(m2):
    """Random and extreme sizes: the backward's validation gives the status
    that follows from the documented rules, computed here in Python integers
    (no overflow), and never reaches a launch.  The workspace offered is
    always 16 bytes, so every size that passes validation stops at
    M2RNN_ERR_WORKSPACE (or succeeds without a launch when there are no
    steps to run, which needs an empty tensor)."""
    from hypothesis import given, settings, strategies as st

    dummy = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    args6 = [dummy] * 6
    grads = [dummy] * 6
    big = st.one_of(st.integers(-2, 70), st.integers(0, 2 ** 31 - 1), st.sampled_from([2 ** 20, 2 ** 22, 2 ** 24]))

    def expected(B, T, N, K, V, dtype, ck):
        if B < 0 or T < 0 or N < 0:
            return m2.M2RNN_ERR_INVALID_ARG
        if K != 64 or V != 16:
            return m2.M2RNN_ERR_UNSUPPORTED
        if dtype not in (0, 1):
            return m2.M2RNN_ERR_INVALID_ARG
        if B * T * N * V > 2 ** 40 or B * ((N + 3) // 4) > 2 ** 22 - 1:
            return m2.M2RNN_ERR_UNSUPPORTED
        if ck < 1:
            return m2.M2RNN_ERR_INVALID_ARG
        if ck > 4 and B * ((N + 3) // 4) * ((T + ck - 1) // ck) > 2 ** 24 - 1:
            return m2.M2RNN_ERR_UNSUPPORTED
        if B * T * N == 0:
            return None   # the empty-tensor path: zero fills only, not reached here
        return m2.M2RNN_ERR_WORKSPACE

    @settings(max_examples=400, deadline=None)
    @given(B=big, T=big, N=big, K=st.sampled_from([64, 64, 32]), V=st.sampled_from([16, 16, 8]),
           dtype=st.sampled_from([0, 1, 2]), ck=st.one_of(st.integers(-1, 80), st.sampled_from([2 ** 30])))
    def check(B, T, N, K, V, dtype, ck):
        want = expected(B, T, N, K, V, dtype, ck)
        if want is None:
            return
        got = m2.lib.m2rnn_backward(B, T, N, K, V, dtype, *args6, dummy, ck, dummy, None, *grads, None, dummy, 16,
                                    None)
        assert got == want, (B, T, N, K, V, dtype, ck, got, want, m2.m2rnn_last_error())

    check()
