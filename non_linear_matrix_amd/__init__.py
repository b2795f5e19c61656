"""Python binding of libm2rnn.so, the MI355X M2RNN scan (C ABI in include/m2rnn.h).

Argument marshalling only: every step of the scan runs in the HIP kernels of
libm2rnn.so.  PyTorch provides device memory and the current HIP stream.  If
the library is missing or fails to load, importing this package raises: there
is no CPU fallback.

    import non_linear_matrix_amd as m2
    y, H_T = m2.forward(q, k, v, f, W, w_r)                    # H_0 = 0 (workspace allocated if needed)
    y, H_T, H_ckpt = m2.forward(q, k, v, f, W, w_r, ckpt_every=64)
    grads = m2.backward(q, k, v, f, W, w_r, H_ckpt, 64, dy)     # dict
    y2, H_T2 = m2.forward(q2, k2, v2, f2, W, w_r, H_0=H_T)     # resume
    y_t = m2.decode(q_t, k_t, v_t, f_t, W, w_r, H)              # one token, H updated
    y, H_T = m2.forward_gated(q, k, v, a, alpha, beta, W, w_r)  # f from the gate
    grads = m2.backward_gated(q, k, v, a, alpha, beta, W, w_r, H_ckpt, 64, dy)
    q = m2.conv_silu_forward(q_proj, w_cq, b_cq)                # SiLU(causal conv4(q_proj))
    o = m2.gate_rmsnorm_forward(y, g, w_o)                      # RMSNorm(y * g) * w_o
    dy, dg, dw_o = m2.gate_rmsnorm_backward(y, g, w_o, do)

Shapes (K = 64, V = 16): q, k [B,T,K]; v [B,T,N,V]; f [B,T,N]; W [N,V,V];
w_r [N,V]; gate pre-activation a [B,T,N] and alpha, beta [N] in place of f;
all inputs float32 or all bfloat16, contiguous, on one GPU.
Outputs and gradients are float32.
"""
import ctypes
import os

import torch

K = 64
V = 16
_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libm2rnn.so")

M2RNN_OK = 0
M2RNN_ERR_INVALID_ARG = -1
M2RNN_ERR_UNSUPPORTED = -2
M2RNN_ERR_WORKSPACE = -3
M2RNN_ERR_HIP = -4
M2RNN_F32 = 0
M2RNN_BF16 = 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python non_linear_matrix_amd/build.py`")
lib = ctypes.CDLL(LIB_PATH)

_i = ctypes.c_int
_p = ctypes.c_void_p
lib.m2rnn_forward.restype = _i
lib.m2rnn_forward.argtypes = [_i] * 6 + [_p] * 7 + [_p, _p, _p, _i] + [_p, ctypes.c_size_t, _p]
lib.m2rnn_forward_workspace_bytes.restype = ctypes.c_size_t
lib.m2rnn_forward_workspace_bytes.argtypes = [_i] * 5
lib.m2rnn_backward_workspace_bytes.restype = ctypes.c_size_t
lib.m2rnn_backward_workspace_bytes.argtypes = [_i] * 6
lib.m2rnn_backward.restype = _i
lib.m2rnn_backward.argtypes = [_i] * 6 + [_p] * 6 + [_p, _i] + [_p, _p] + [_p] * 7 + [_p, ctypes.c_size_t, _p]
lib.m2rnn_forward_gated.restype = _i
lib.m2rnn_forward_gated.argtypes = [_i] * 6 + [_p] * 9 + [_p, _p, _p, _i] + [_p, ctypes.c_size_t, _p]
lib.m2rnn_backward_gated.restype = _i
lib.m2rnn_backward_gated.argtypes = ([_i] * 6 + [_p] * 8 + [_p, _i] + [_p, _p] + [_p] * 9
                                     + [_p, ctypes.c_size_t, _p])
lib.m2rnn_conv_silu_forward.restype = _i
lib.m2rnn_conv_silu_forward.argtypes = [_i] * 4 + [_p] * 4 + [_p]
lib.m2rnn_conv_silu_backward_workspace_bytes.restype = ctypes.c_size_t
lib.m2rnn_conv_silu_backward_workspace_bytes.argtypes = [_i] * 3
lib.m2rnn_conv_silu_backward.restype = _i
lib.m2rnn_conv_silu_backward.argtypes = [_i] * 4 + [_p] * 7 + [_p, ctypes.c_size_t, _p]
lib.m2rnn_gate_rmsnorm_forward.restype = _i
lib.m2rnn_gate_rmsnorm_forward.argtypes = [_i] * 5 + [_p] * 3 + [ctypes.c_float] + [_p, _p, _p]
lib.m2rnn_gate_rmsnorm_backward_workspace_bytes.restype = ctypes.c_size_t
lib.m2rnn_gate_rmsnorm_backward_workspace_bytes.argtypes = [_i] * 4
lib.m2rnn_gate_rmsnorm_backward.restype = _i
lib.m2rnn_gate_rmsnorm_backward.argtypes = ([_i] * 5 + [_p] * 3 + [ctypes.c_float] + [_p] * 4
                                            + [_p, ctypes.c_size_t, _p])
lib.m2rnn_gate_rmsnorm_backward_noalloc.restype = _i
lib.m2rnn_gate_rmsnorm_backward_noalloc.argtypes = [_i] * 5 + [_p] * 3 + [ctypes.c_float] + [_p] * 4 + [_p]
lib.m2rnn_decode.restype = _i
lib.m2rnn_decode.argtypes = [_i] * 5 + [_p] * 6 + [_p, _p, _p]
lib.m2rnn_last_error.restype = ctypes.c_char_p
lib.m2rnn_last_error.argtypes = []


class M2RNNError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"m2rnn status {status}: {msg}")
        self.status = status


def _check(status):
    if status != M2RNN_OK:
        raise M2RNNError(status, lib.m2rnn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return M2RNN_F32
    if t.dtype == torch.bfloat16:
        return M2RNN_BF16
    raise TypeError(f"inputs must be float32 or bfloat16, got {t.dtype}")


def _tensor(t, name, shape, dtype, device):
    """Raise ValueError unless t is a contiguous tensor of this shape, dtype
    and device: the C ABI sees only the data pointer, so a mismatch would be
    read as the wrong bytes (or past the end of the buffer) on the GPU."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (all tensors on one device)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name, shape, dtype, device):
    return None if t is None else _tensor(t, name, shape, dtype, device)


def _gpu(device):
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {device}")


def _in_dtype(t, name):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"inputs must be float32 or bfloat16, got {name} in {t.dtype}")
    return t.dtype


def _scan_inputs(q, k, v, f, W, w_r, f_name="f", alpha=None, beta=None):
    """Checks the scan's inputs (all of q's dtype, contiguous, on q's device)
    and returns B, T, N, K, V and the device."""
    dt = _in_dtype(q, "q")
    if q.dim() != 3:
        raise ValueError(f"q must be [B, T, K], got shape {tuple(q.shape)}")
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a 4-D tensor [B, T, N, V]")
    B, T, Kq = q.shape
    N, Vv = v.shape[2], v.shape[3]
    dev = q.device
    _tensor(q, "q", (B, T, Kq), dt, dev)
    _tensor(k, "k", (B, T, Kq), dt, dev)
    _tensor(v, "v", (B, T, N, Vv), dt, dev)
    _tensor(f, f_name, (B, T, N), dt, dev)
    _tensor(W, "W", (N, Vv, Vv), dt, dev)
    _tensor(w_r, "w_r", (N, Vv), dt, dev)
    if alpha is not None or beta is not None:
        _tensor(alpha, "alpha", (N,), dt, dev)
        _tensor(beta, "beta", (N,), dt, dev)
    return B, T, N, Kq, Vv, dev


def _n_ckpt(T, ckpt_every):
    return (T + ckpt_every - 1) // ckpt_every if ckpt_every > 0 else 0


def m2rnn_forward(B, T, N, K_, V_, dtype, q, k, v, f, W, w_r, H_0, y, H_T, H_ckpt, ckpt_every, workspace,
                  workspace_bytes, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_forward(B, T, N, K_, V_, dtype, q, k, v, f, W, w_r, H_0, y, H_T, H_ckpt, ckpt_every, workspace,
                             workspace_bytes, stream)


def m2rnn_forward_workspace_bytes(B, T, N, K_=K, V_=V):
    return int(lib.m2rnn_forward_workspace_bytes(B, T, N, K_, V_))


def m2rnn_backward(B, T, N, K_, V_, dtype, q, k, v, f, W, w_r, H_ckpt, ckpt_every, dy, dH_T,
                   dq, dk, dv, df, dW, dw_r, dH_0, workspace, workspace_bytes, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_backward(B, T, N, K_, V_, dtype, q, k, v, f, W, w_r, H_ckpt, ckpt_every, dy, dH_T,
                              dq, dk, dv, df, dW, dw_r, dH_0, workspace, workspace_bytes, stream)


def m2rnn_forward_gated(B, T, N, K_, V_, dtype, q, k, v, a, alpha, beta, W, w_r, H_0, y, H_T, H_ckpt, ckpt_every,
                        workspace, workspace_bytes, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_forward_gated(B, T, N, K_, V_, dtype, q, k, v, a, alpha, beta, W, w_r, H_0, y, H_T, H_ckpt,
                                   ckpt_every, workspace, workspace_bytes, stream)


def m2rnn_backward_gated(B, T, N, K_, V_, dtype, q, k, v, a, alpha, beta, W, w_r, H_ckpt, ckpt_every, dy, dH_T,
                         dq, dk, dv, da, dalpha, dbeta, dW, dw_r, dH_0, workspace, workspace_bytes, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_backward_gated(B, T, N, K_, V_, dtype, q, k, v, a, alpha, beta, W, w_r, H_ckpt, ckpt_every,
                                    dy, dH_T, dq, dk, dv, da, dalpha, dbeta, dW, dw_r, dH_0, workspace,
                                    workspace_bytes, stream)


def m2rnn_decode(B, N, K_, V_, dtype, q, k, v, f, W, w_r, H, y, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_decode(B, N, K_, V_, dtype, q, k, v, f, W, w_r, H, y, stream)


def m2rnn_backward_workspace_bytes(B, T, N, K_=K, V_=V, ckpt_every=64):
    return int(lib.m2rnn_backward_workspace_bytes(B, T, N, K_, V_, ckpt_every))


def m2rnn_last_error():
    return lib.m2rnn_last_error().decode()


def _fwd_outputs(B, T, N, Kq, Vv, dev, ckpt_every, out, H_0):
    f32 = torch.float32
    if int(ckpt_every) < 0:
        raise ValueError("ckpt_every must be >= 0")
    _opt(H_0, "H_0", (B, N, Kq, Vv), f32, dev)
    shape_ck = (B, N, _n_ckpt(T, ckpt_every), Kq, Vv)
    if out is None:
        _gpu(dev)
        y = torch.empty((B, T, N, Vv), device=dev, dtype=f32)
        H_T = torch.empty((B, N, Kq, Vv), device=dev, dtype=f32)
        H_ck = torch.empty(shape_ck, device=dev, dtype=f32) if ckpt_every > 0 else None
    else:
        y, H_T = out[0], out[1]
        H_ck = out[2] if len(out) > 2 else None
        if (H_ck is None) != (ckpt_every <= 0):
            raise ValueError("out holds H_ckpt exactly when ckpt_every > 0")
        _tensor(y, "y", (B, T, N, Vv), f32, dev)
        _tensor(H_T, "H_T", (B, N, Kq, Vv), f32, dev)
        _opt(H_ck, "H_ckpt", shape_ck, f32, dev)
    _gpu(dev)
    return y, H_T, H_ck


def _fwd_workspace(B, T, N, Kq, Vv, dev, workspace):
    nbytes = int(lib.m2rnn_forward_workspace_bytes(B, T, N, Kq, Vv))
    if workspace is None:
        if nbytes > 0:
            workspace = torch.empty((nbytes,), device=dev, dtype=torch.uint8)
    else:
        _tensor(workspace, "workspace", (workspace.numel(),), workspace.dtype, dev)
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def forward(q, k, v, f, W, w_r, ckpt_every=0, out=None, H_0=None, workspace=None):
    """y [B,T,N,V], H_T [B,N,K,V] (float32) and, if ckpt_every > 0,
    H_ckpt [B,N,ceil(T/ckpt_every),K,V].  `out` may pass preallocated
    (y, H_T[, H_ckpt]) tensors; H_0 [B,N,K,V] float32 is the initial state
    (None: zero) and may be the same tensor as H_T.  `workspace` may pass
    m2rnn_forward_workspace_bytes(B, T, N) bytes of device memory (allocated
    here when needed and not given)."""
    B, T, N, Kq, Vv, dev = _scan_inputs(q, k, v, f, W, w_r)
    y, H_T, H_ck = _fwd_outputs(B, T, N, Kq, Vv, dev, ckpt_every, out, H_0)
    workspace, wbytes = _fwd_workspace(B, T, N, Kq, Vv, dev, workspace)
    _check(lib.m2rnn_forward(B, T, N, Kq, Vv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W),
                             _ptr(w_r), _ptr(H_0), _ptr(y), _ptr(H_T), _ptr(H_ck), int(ckpt_every),
                             _ptr(workspace), wbytes, _stream(q.device)))
    return (y, H_T) if H_ck is None else (y, H_T, H_ck)


def forward_gated(q, k, v, a, alpha, beta, W, w_r, ckpt_every=0, out=None, H_0=None, workspace=None):
    """forward() with f = exp(-alpha[n] softplus(a + beta[n])) computed in the
    kernel from the gate pre-activation a [B,T,N] and alpha, beta [N]."""
    B, T, N, Kq, Vv, dev = _scan_inputs(q, k, v, a, W, w_r, f_name="a", alpha=alpha, beta=beta)
    y, H_T, H_ck = _fwd_outputs(B, T, N, Kq, Vv, dev, ckpt_every, out, H_0)
    workspace, wbytes = _fwd_workspace(B, T, N, Kq, Vv, dev, workspace)
    _check(lib.m2rnn_forward_gated(B, T, N, Kq, Vv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                   _ptr(alpha), _ptr(beta), _ptr(W), _ptr(w_r), _ptr(H_0), _ptr(y), _ptr(H_T),
                                   _ptr(H_ck), int(ckpt_every), _ptr(workspace), wbytes, _stream(q.device)))
    return (y, H_T) if H_ck is None else (y, H_T, H_ck)


def _bwd_outputs(B, T, N, Kq, Vv, dev, H_ckpt, ckpt_every, dy, dH_T, out, want_dH_0, df_name):
    f32 = torch.float32
    if int(ckpt_every) < 1:
        raise ValueError("ckpt_every must be >= 1 for the backward")
    _tensor(H_ckpt, "H_ckpt", (B, N, _n_ckpt(T, ckpt_every), Kq, Vv), f32, dev)
    _tensor(dy, "dy", (B, T, N, Vv), f32, dev)
    _opt(dH_T, "dH_T", (B, N, Kq, Vv), f32, dev)
    shapes = dict(dq=(B, T, Kq), dk=(B, T, Kq), dv=(B, T, N, Vv), dW=(N, Vv, Vv), dw_r=(N, Vv))
    shapes[df_name] = (B, T, N)
    if df_name == "da":
        shapes.update(dalpha=(N,), dbeta=(N,))
    if out is not None:
        for n, sh in shapes.items():
            if n not in out:
                raise ValueError(f"out has no {n}")
            _tensor(out[n], n, sh, f32, dev)
        _opt(out.get("dH_0"), "dH_0", (B, N, Kq, Vv), f32, dev)
    _gpu(dev)
    if out is None:
        out = {n: torch.empty(sh, device=dev, dtype=f32) for n, sh in shapes.items()}
        if want_dH_0:
            out["dH_0"] = torch.empty((B, N, Kq, Vv), device=dev, dtype=f32)
    return out


def _bwd_workspace(B, T, N, Kq, Vv, dev, ckpt_every, workspace):
    nbytes = int(lib.m2rnn_backward_workspace_bytes(B, T, N, Kq, Vv, int(ckpt_every)))
    if workspace is None:
        if nbytes > 0:
            workspace = torch.empty((nbytes,), device=dev, dtype=torch.uint8)
    else:
        _tensor(workspace, "workspace", (workspace.numel(),), workspace.dtype, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, wbytes


def backward(q, k, v, f, W, w_r, H_ckpt, ckpt_every, dy, dH_T=None, out=None, workspace=None, want_dH_0=False):
    """Gradients of sum(y*dy) + sum(H_T*dH_T): dict dq, dk [B,T,K]; dv [B,T,N,V];
    df [B,T,N]; dW [N,V,V]; dw_r [N,V] and, with want_dH_0 (or a "dH_0"
    entry in `out`), dH_0 [B,N,K,V] (float32)."""
    B, T, N, Kq, Vv, dev = _scan_inputs(q, k, v, f, W, w_r)
    out = _bwd_outputs(B, T, N, Kq, Vv, dev, H_ckpt, ckpt_every, dy, dH_T, out, want_dH_0, "df")
    workspace, wbytes = _bwd_workspace(B, T, N, Kq, Vv, dev, ckpt_every, workspace)
    _check(lib.m2rnn_backward(B, T, N, Kq, Vv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W),
                              _ptr(w_r), _ptr(H_ckpt), int(ckpt_every), _ptr(dy), _ptr(dH_T),
                              _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["df"]),
                              _ptr(out["dW"]), _ptr(out["dw_r"]), _ptr(out.get("dH_0")), _ptr(workspace), wbytes,
                              _stream(dev)))
    return out


def backward_gated(q, k, v, a, alpha, beta, W, w_r, H_ckpt, ckpt_every, dy, dH_T=None, out=None, workspace=None,
                   want_dH_0=False):
    """backward() of forward_gated(): the dict holds da [B,T,N] and dalpha,
    dbeta [N] in place of df."""
    B, T, N, Kq, Vv, dev = _scan_inputs(q, k, v, a, W, w_r, f_name="a", alpha=alpha, beta=beta)
    out = _bwd_outputs(B, T, N, Kq, Vv, dev, H_ckpt, ckpt_every, dy, dH_T, out, want_dH_0, "da")
    workspace, wbytes = _bwd_workspace(B, T, N, Kq, Vv, dev, ckpt_every, workspace)
    _check(lib.m2rnn_backward_gated(B, T, N, Kq, Vv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                    _ptr(alpha), _ptr(beta), _ptr(W), _ptr(w_r), _ptr(H_ckpt), int(ckpt_every),
                                    _ptr(dy), _ptr(dH_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                    _ptr(out["da"]), _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dW"]),
                                    _ptr(out["dw_r"]), _ptr(out.get("dH_0")), _ptr(workspace), wbytes,
                                    _stream(dev)))
    return out


def decode(q, k, v, f, W, w_r, H, y=None):
    """One token for every (b, n): q, k [B,K]; v [B,N,V]; f [B,N]; H [B,N,K,V]
    float32, advanced in place.  Returns y [B,N,V] float32."""
    dt = _in_dtype(q, "q")
    if q.dim() != 2 or not isinstance(v, torch.Tensor) or v.dim() != 3:
        raise ValueError("decode takes q, k [B, K] and v [B, N, V]")
    B, Kq = q.shape
    N, Vv = v.shape[1], v.shape[2]
    dev = q.device
    _tensor(q, "q", (B, Kq), dt, dev)
    _tensor(k, "k", (B, Kq), dt, dev)
    _tensor(v, "v", (B, N, Vv), dt, dev)
    _tensor(f, "f", (B, N), dt, dev)
    _tensor(W, "W", (N, Vv, Vv), dt, dev)
    _tensor(w_r, "w_r", (N, Vv), dt, dev)
    _tensor(H, "H", (B, N, Kq, Vv), torch.float32, dev)
    _opt(y, "y", (B, N, Vv), torch.float32, dev)
    _gpu(dev)
    if y is None:
        y = torch.empty((B, N, Vv), device=dev, dtype=torch.float32)
    _check(lib.m2rnn_decode(B, N, Kq, Vv, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r),
                            _ptr(H), _ptr(y), _stream(q.device)))
    return y


def m2rnn_gate_rmsnorm_forward(B, T, N, V_, dtype, y, g, w, eps, out, rstd, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_gate_rmsnorm_forward(B, T, N, V_, dtype, y, g, w, eps, out, rstd, stream)


def m2rnn_gate_rmsnorm_backward(B, T, N, V_, dtype, y, g, w, eps, dout, dy, dg, dw, workspace, workspace_bytes,
                                stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_gate_rmsnorm_backward(B, T, N, V_, dtype, y, g, w, eps, dout, dy, dg, dw, workspace,
                                           workspace_bytes, stream)


def m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, V_=V):
    return int(lib.m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, V_))


def _norm_inputs(y, g, w):
    """Checks y (float32 [B,T,N,V]), g (y's shape, the input dtype) and w
    ([N,V] or [N*V], g's dtype); returns B, T, N, V and the device."""
    if not isinstance(y, torch.Tensor) or y.dim() != 4:
        raise ValueError("y must be a 4-D tensor [B, T, N, V]")
    B, T, N, Vv = y.shape
    dev = y.device
    dt = _in_dtype(g, "g")
    _tensor(y, "y", (B, T, N, Vv), torch.float32, dev)
    _tensor(g, "g", (B, T, N, Vv), dt, dev)
    _tensor(w, "w", (N, Vv) if isinstance(w, torch.Tensor) and w.dim() == 2 else (N * Vv,), dt, dev)
    return B, T, N, Vv, dev


def gate_rmsnorm_forward(y, g, w, eps=0.0, out=None, rstd=None):
    """out = w * x * s with x = y * g and s = (mean over the N*V features of
    x^2 + eps)^-1/2, per token.  y [B,T,N,V] float32; g like y and w [N,V]
    (or [N*V]) in the input dtype.  Returns out [B,T,N,V] float32 (`out` may
    be y itself); `rstd` [B,T] float32, if given, receives s."""
    B, T, N, Vv, dev = _norm_inputs(y, g, w)
    _opt(out, "out", (B, T, N, Vv), torch.float32, dev)
    _opt(rstd, "rstd", (B, T), torch.float32, dev)
    _gpu(dev)
    if out is None:
        out = torch.empty_like(y, dtype=torch.float32)
    _check(lib.m2rnn_gate_rmsnorm_forward(B, T, N, Vv, _dtype_code(g), _ptr(y), _ptr(g), _ptr(w), float(eps),
                                          _ptr(out), _ptr(rstd), _stream(y.device)))
    return out


def _norm_grads(B, T, N, Vv, dev, dout, out):
    f32 = torch.float32
    _tensor(dout, "dout", (B, T, N, Vv), f32, dev)
    if out is not None:
        _tensor(out[0], "dy", (B, T, N, Vv), f32, dev)
        _tensor(out[1], "dg", (B, T, N, Vv), f32, dev)
        _tensor(out[2], "dw", (N, Vv) if isinstance(out[2], torch.Tensor) and out[2].dim() == 2 else (N * Vv,), f32,
                dev)
    _gpu(dev)
    if out is None:
        out = (torch.empty((B, T, N, Vv), device=dev, dtype=f32), torch.empty((B, T, N, Vv), device=dev, dtype=f32),
               torch.empty((N * Vv,), device=dev, dtype=f32))
    return out


def gate_rmsnorm_backward(y, g, w, dout, eps=0.0, out=None, workspace=None):
    """Gradients of sum(out * dout) for gate_rmsnorm_forward: (dy [B,T,N,V],
    dg [B,T,N,V], dw [N*V]) float32.  `out` may pass (dy, dg, dw)."""
    B, T, N, Vv, dev = _norm_inputs(y, g, w)
    out = _norm_grads(B, T, N, Vv, dev, dout, out)
    nbytes = int(lib.m2rnn_gate_rmsnorm_backward_workspace_bytes(B, T, N, Vv))
    if workspace is None and nbytes > 0:
        workspace = torch.empty((nbytes,), device=dev, dtype=torch.uint8)
    elif workspace is not None:
        _tensor(workspace, "workspace", (workspace.numel(),), workspace.dtype, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m2rnn_gate_rmsnorm_backward(B, T, N, Vv, _dtype_code(g), _ptr(y), _ptr(g), _ptr(w), float(eps),
                                           _ptr(dout), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(workspace),
                                           wbytes, _stream(dev)))
    return out


def m2rnn_gate_rmsnorm_backward_noalloc(B, T, N, V_, dtype, y, g, w, eps, dout, dy, dg, dw, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_gate_rmsnorm_backward_noalloc(B, T, N, V_, dtype, y, g, w, eps, dout, dy, dg, dw, stream)


def gate_rmsnorm_backward_noalloc(y, g, w, dout, eps=0.0, out=None):
    """gate_rmsnorm_backward without a workspace: the library's own scratch
    array on the GPU holds the dw partial sums (calls on one GPU must be
    ordered on one stream).  Returns (dy, dg, dw) float32; `out` may pass
    them."""
    B, T, N, Vv, dev = _norm_inputs(y, g, w)
    out = _norm_grads(B, T, N, Vv, dev, dout, out)
    _check(lib.m2rnn_gate_rmsnorm_backward_noalloc(B, T, N, Vv, _dtype_code(g), _ptr(y), _ptr(g), _ptr(w), float(eps),
                                                   _ptr(dout), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                                                   _stream(dev)))
    return out


def m2rnn_conv_silu_forward(B, T, C, dtype, u, w, bias, z, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_conv_silu_forward(B, T, C, dtype, u, w, bias, z, stream)


def m2rnn_conv_silu_backward(B, T, C, dtype, u, w, bias, dz, du, dw, dbias, workspace, workspace_bytes, stream):
    """Raw C-ABI call with ctypes pointers; returns the status code."""
    return lib.m2rnn_conv_silu_backward(B, T, C, dtype, u, w, bias, dz, du, dw, dbias, workspace, workspace_bytes,
                                        stream)


def m2rnn_conv_silu_backward_workspace_bytes(B, T, C):
    return int(lib.m2rnn_conv_silu_backward_workspace_bytes(B, T, C))


def _conv_shape(u):
    """u [B, T, C] or [B, T, N, V] (treated as C = N V)."""
    if not isinstance(u, torch.Tensor) or u.dim() not in (3, 4):
        raise ValueError("u must be [B, T, C] or [B, T, N, V]")
    C = 1
    for s in u.shape[2:]:
        C *= s
    return u.shape[0], u.shape[1], C


def _conv_inputs(u, w, bias):
    B, T, C = _conv_shape(u)
    dt = _in_dtype(u, "u")
    dev = u.device
    _tensor(u, "u", tuple(u.shape), dt, dev)
    _tensor(w, "w", (C, 4), dt, dev)
    _opt(bias, "bias", (C,), dt, dev)
    return B, T, C, dev


def conv_silu_forward(u, w, bias=None, out=None):
    """z = SiLU(bias + causal depthwise conv of width 4 over time) with taps
    w [C, 4] in torch conv1d order (the last tap on the current step).  u is
    [B, T, C] or [B, T, N, V]; z has u's shape and dtype."""
    B, T, C, dev = _conv_inputs(u, w, bias)
    _opt(out, "z", tuple(u.shape), u.dtype, dev)
    _gpu(dev)
    if out is None:
        out = torch.empty_like(u)
    _check(lib.m2rnn_conv_silu_forward(B, T, C, _dtype_code(u), _ptr(u), _ptr(w), _ptr(bias), _ptr(out),
                                       _stream(u.device)))
    return out


def conv_silu_backward(u, w, bias, dz, out=None, workspace=None, want_dbias=True):
    """Gradients of sum(z * dz) for conv_silu_forward: (du like u in float32,
    dw [C, 4], dbias [C] or None) float32.  `out` may pass (du, dw, dbias)."""
    B, T, C, dev = _conv_inputs(u, w, bias)
    f32 = torch.float32
    _tensor(dz, "dz", tuple(u.shape), f32, dev)
    if out is not None:
        _tensor(out[0], "du", tuple(u.shape), f32, dev)
        _tensor(out[1], "dw", (C, 4), f32, dev)
        _opt(out[2], "dbias", (C,), f32, dev)
    _gpu(dev)
    if out is None:
        out = (torch.empty(u.shape, device=dev, dtype=f32), torch.empty((C, 4), device=dev, dtype=f32),
               torch.empty((C,), device=dev, dtype=f32) if want_dbias else None)
    nbytes = int(lib.m2rnn_conv_silu_backward_workspace_bytes(B, T, C))
    if workspace is None and nbytes > 0:
        workspace = torch.empty((nbytes,), device=dev, dtype=torch.uint8)
    elif workspace is not None:
        _tensor(workspace, "workspace", (workspace.numel(),), workspace.dtype, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.m2rnn_conv_silu_backward(B, T, C, _dtype_code(u), _ptr(u), _ptr(w), _ptr(bias), _ptr(dz),
                                        _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(workspace), wbytes,
                                        _stream(dev)))
    return out
