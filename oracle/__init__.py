"""Python handle on the fp64 CPU oracle of the M2RNN scan (oracle/m2rnn_ref.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  The HIP library
(``non_linear_matrix_amd``) never imports it and shares no code with it.

What the oracle computes follows the M2RNN paper-discussion slides (reading of
arXiv:2603.14360v2): slide "Write, transform, retain, and read a matrix state"
(paper Eqs. (10)-(12)) for the forward recurrence and slide "Backup: the
recurrent gradient needs both paths" for the backward; q and k are shared by
the value heads (slide "Shared queries and keys buy more recurrent capacity",
paper Alg. 1).  Inputs are upcast exactly to float64; outputs are float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_dbl_p = ctypes.POINTER(ctypes.c_double)


class Oracle:
    """ctypes binding of one compiled copy of the oracle source."""

    def __init__(self, lib_path):
        self.path = lib_path
        self.lib = ctypes.CDLL(lib_path)
        fwd = self.lib.m2rnn_ref_forward
        fwd.restype = ctypes.c_int
        fwd.argtypes = [ctypes.c_int] * 5 + [_dbl_p] * 7 + [_dbl_p, _dbl_p, _dbl_p, ctypes.c_int, ctypes.c_int]
        bwd = self.lib.m2rnn_ref_backward
        bwd.restype = ctypes.c_int
        bwd.argtypes = [ctypes.c_int] * 5 + [_dbl_p] * 7 + [_dbl_p, _dbl_p] + [_dbl_p] * 7 + [ctypes.c_int]

        gf = self.lib.m2rnn_ref_gate_forward
        gf.restype = ctypes.c_int
        gf.argtypes = [ctypes.c_int] * 3 + [_dbl_p] * 4
        gb = self.lib.m2rnn_ref_gate_backward
        gb.restype = ctypes.c_int
        gb.argtypes = [ctypes.c_int] * 3 + [_dbl_p] * 7
        nf = self.lib.m2rnn_ref_gate_rmsnorm_forward
        nf.restype = ctypes.c_int
        nf.argtypes = [ctypes.c_int] * 2 + [_dbl_p] * 3 + [ctypes.c_double] + [_dbl_p] * 2
        cf = self.lib.m2rnn_ref_conv_silu_forward
        cf.restype = ctypes.c_int
        cf.argtypes = [ctypes.c_int] * 3 + [_dbl_p] * 4
        cb = self.lib.m2rnn_ref_conv_silu_backward
        cb.restype = ctypes.c_int
        cb.argtypes = [ctypes.c_int] * 3 + [_dbl_p] * 7
        nb = self.lib.m2rnn_ref_gate_rmsnorm_backward
        nb.restype = ctypes.c_int
        nb.argtypes = [ctypes.c_int] * 2 + [_dbl_p] * 3 + [ctypes.c_double] + [_dbl_p] * 4

    @staticmethod
    def _arr(x, shape=None):
        a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        if shape is not None and a.shape != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
        return a

    @staticmethod
    def _p(a):
        return a.ctypes.data_as(_dbl_p) if a is not None else None

    def _inputs(self, q, k, v, f, W, wr):
        q = self._arr(q)
        B, T, K = q.shape
        v = self._arr(v)
        N, V = v.shape[2], v.shape[3]
        k = self._arr(k, (B, T, K))
        v = self._arr(v, (B, T, N, V))
        f = self._arr(f, (B, T, N))
        W = self._arr(W, (N, V, V))
        wr = self._arr(wr, (N, V))
        return (B, T, N, K, V), (q, k, v, f, W, wr)

    def forward(self, q, k, v, f, W, wr, ckpt_every=0, nthreads=0, H_0=None):
        """Returns (y [B,T,N,V], H_T [B,N,K,V]) or, with ckpt_every > 0,
        (y, H_T, H_ckpt [B,N,ceil(T/ckpt_every),K,V]).  H_0 [B,N,K,V] is the
        initial state (None: zero)."""
        (B, T, N, K, V), ins = self._inputs(q, k, v, f, W, wr)
        h0 = None if H_0 is None else self._arr(H_0, (B, N, K, V))
        y = np.empty((B, T, N, V))
        HT = np.empty((B, N, K, V))
        ck = None
        if ckpt_every > 0:
            ck = np.empty((B, N, (T + ckpt_every - 1) // ckpt_every, K, V))
        st = self.lib.m2rnn_ref_forward(B, T, N, K, V, *[self._p(a) for a in ins], self._p(h0),
                                        self._p(y), self._p(HT), self._p(ck), int(ckpt_every), int(nthreads))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_forward failed with status {st}")
        return (y, HT) if ck is None else (y, HT, ck)

    def backward(self, q, k, v, f, W, wr, dy, dH_T=None, nthreads=0, H_0=None):
        """Gradients of sum(y*dy) + sum(H_T*dH_T) for the run from H_0 (None:
        zero): dict with dq, dk, dv, df, dW, dwr and dH_0."""
        (B, T, N, K, V), ins = self._inputs(q, k, v, f, W, wr)
        h0 = None if H_0 is None else self._arr(H_0, (B, N, K, V))
        dy = self._arr(dy, (B, T, N, V))
        dHT = None if dH_T is None else self._arr(dH_T, (B, N, K, V))
        out = dict(dq=np.empty((B, T, K)), dk=np.empty((B, T, K)), dv=np.empty((B, T, N, V)),
                   df=np.empty((B, T, N)), dW=np.empty((N, V, V)), dwr=np.empty((N, V)),
                   dH_0=np.empty((B, N, K, V)))
        st = self.lib.m2rnn_ref_backward(B, T, N, K, V, *[self._p(a) for a in ins], self._p(h0),
                                         self._p(dy), self._p(dHT),
                                         *[self._p(out[n]) for n in ("dq", "dk", "dv", "df", "dW", "dwr", "dH_0")],
                                         int(nthreads))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_backward failed with status {st}")
        return out


    def gate_forward(self, a, alpha, beta):
        """f = exp(-alpha[n] softplus(a + beta[n])) for a [B,T,N], alpha, beta [N]."""
        a = self._arr(a)
        B, T, N = a.shape
        alpha = self._arr(alpha, (N,))
        beta = self._arr(beta, (N,))
        f = np.empty((B, T, N))
        st = self.lib.m2rnn_ref_gate_forward(B, T, N, self._p(a), self._p(alpha), self._p(beta), self._p(f))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_gate_forward failed with status {st}")
        return f

    def conv_silu_forward(self, u, w, bias=None):
        """Causal depthwise Conv1D (width 4) and SiLU over time: u [B, T, C],
        w [C, 4], bias [C] or None.  Returns z [B, T, C]."""
        u = self._arr(u)
        B, T, C = u.shape
        w = self._arr(w, (C, 4))
        bias = None if bias is None else self._arr(bias, (C,))
        z = np.empty((B, T, C))
        st = self.lib.m2rnn_ref_conv_silu_forward(B, T, C, self._p(u), self._p(w), self._p(bias), self._p(z))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_conv_silu_forward failed with status {st}")
        return z

    def conv_silu_backward(self, u, w, bias, dz):
        """(du [B, T, C], dw [C, 4], dbias [C]) from dz [B, T, C]."""
        u = self._arr(u)
        B, T, C = u.shape
        w = self._arr(w, (C, 4))
        bias = None if bias is None else self._arr(bias, (C,))
        dz = self._arr(dz, (B, T, C))
        du, dw, db = np.empty((B, T, C)), np.empty((C, 4)), np.empty(C)
        st = self.lib.m2rnn_ref_conv_silu_backward(B, T, C, self._p(u), self._p(w), self._p(bias), self._p(dz),
                                                   self._p(du), self._p(dw), self._p(db))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_conv_silu_backward failed with status {st}")
        return du, dw, db

    def gate_rmsnorm_forward(self, y, g, w, eps=0.0):
        """Output gate and RMSNorm over the last axis: y, g [..., d], w [d].
        Returns (o [..., d], rstd [...])."""
        y = self._arr(y)
        d = y.shape[-1]
        g = self._arr(g, y.shape)
        w = self._arr(w, (d,))
        ntok = y.size // d
        o, rstd = np.empty(y.shape), np.empty(y.shape[:-1])
        st = self.lib.m2rnn_ref_gate_rmsnorm_forward(ntok, d, self._p(y), self._p(g), self._p(w), float(eps),
                                                     self._p(o), self._p(rstd))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_gate_rmsnorm_forward failed with status {st}")
        return o, rstd

    def gate_rmsnorm_backward(self, y, g, w, dout, eps=0.0):
        """(dy [..., d], dg [..., d], dw [d]) from dout [..., d]."""
        y = self._arr(y)
        d = y.shape[-1]
        g = self._arr(g, y.shape)
        w = self._arr(w, (d,))
        dout = self._arr(dout, y.shape)
        ntok = y.size // d
        dy, dg, dw = np.empty(y.shape), np.empty(y.shape), np.empty(d)
        st = self.lib.m2rnn_ref_gate_rmsnorm_backward(ntok, d, self._p(y), self._p(g), self._p(w), float(eps),
                                                      self._p(dout), self._p(dy), self._p(dg), self._p(dw))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_gate_rmsnorm_backward failed with status {st}")
        return dy, dg, dw

    def gate_backward(self, a, alpha, beta, df):
        """(da [B,T,N], dalpha [N], dbeta [N]) from df [B,T,N]."""
        a = self._arr(a)
        B, T, N = a.shape
        alpha = self._arr(alpha, (N,))
        beta = self._arr(beta, (N,))
        df = self._arr(df, (B, T, N))
        da, dal, dbe = np.empty((B, T, N)), np.empty(N), np.empty(N)
        st = self.lib.m2rnn_ref_gate_backward(B, T, N, self._p(a), self._p(alpha), self._p(beta), self._p(df),
                                              self._p(da), self._p(dal), self._p(dbe))
        if st != 0:
            raise RuntimeError(f"m2rnn_ref_gate_backward failed with status {st}")
        return da, dal, dbe


_default = None


def get(rebuild=False):
    """The oracle built from oracle/m2rnn_ref.c (compiled on first use)."""
    global _default
    if _default is None or rebuild:
        if rebuild or not os.path.exists(_build.LIB) or \
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def forward(*args, **kw):
    return get().forward(*args, **kw)


def backward(*args, **kw):
    return get().backward(*args, **kw)


def conv_silu_forward(*args, **kw):
    return get().conv_silu_forward(*args, **kw)


def conv_silu_backward(*args, **kw):
    return get().conv_silu_backward(*args, **kw)


def gate_rmsnorm_forward(*args, **kw):
    return get().gate_rmsnorm_forward(*args, **kw)


def gate_rmsnorm_backward(*args, **kw):
    return get().gate_rmsnorm_backward(*args, **kw)


def gate_forward(*args, **kw):
    return get().gate_forward(*args, **kw)


def gate_backward(*args, **kw):
    return get().gate_backward(*args, **kw)
