"""Pins of the fp64 oracle to facts fixed by the M2RNN slides and by mathematics.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees.  The pins are chosen so that a plausible slip anywhere in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a stale state)
fails at least one of them; tests/test_oracle_mutants.py plants such slips in
copies of the oracle source and checks exactly that.

Sources (M2RNN paper-discussion slides, reading of arXiv:2603.14360v2):
  [EQ]  slide "Write, transform, retain, and read a matrix state",
        paper Eqs. (10)-(12): the recurrence, H_0 = 0, f in [0, 1].
  [SH]  slide "Shared queries and keys buy more recurrent capacity",
        paper Alg. 1 / App. A: q, k shared by the value heads.
  [RNN] slide "Backup: embedding a vector RNN in one matrix row",
        paper App. B, Eq. (25): f = 0, w_r = 0, q = k = e_1 turns row 1 of
        the state into the Elman RNN h_t = tanh(W^T h_{t-1} + v_t), y_t = h_t.
  [BW]  slide "Backup: the recurrent gradient needs both paths".
  [H0]  a caller-given initial state: the recurrence of [EQ] resumed from a
        stored state, and its gradient dL/dH_0 = C_0, where the recursion of
        [BW] for C ends.
  [GT]  slide "The gate preserves a direct path through time", paper Sec. 3.1,
        Eqs. (13), (17): f = exp(-alpha softplus(a + beta)), alpha >= 0.
  [CNV] slide "Most of the block can be computed before recurrence", paper
        Fig. 2: q, k, v pass a causal Conv1D of width 4 and a SiLU before the
        scan (depthwise over time per channel, zero input before t = 0).
  [NRM] slide "Most of the block can be computed before recurrence", paper
        Fig. 2 (after the readout: times the output gate, then RMSNorm), with
        the statistic and backward of slide "Backup: RMSNormTP synchronizes
        per-token statistics", paper App. C, Eqs. (26)-(33).
"""
import numpy as np
import torch

RNG_SEED = 1234


def _rand_inputs(rng, B, T, N, K, V, f_lo=0.0, f_hi=1.0, scale=1.0):
    q = rng.standard_normal((B, T, K)) * scale
    k = rng.standard_normal((B, T, K)) * scale
    v = rng.standard_normal((B, T, N, V)) * scale
    f = rng.uniform(f_lo, f_hi, (B, T, N))
    W = rng.standard_normal((N, V, V)) * 0.4
    wr = rng.standard_normal((N, V))
    return q, k, v, f, W, wr


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- forward pins

def pin_t1_closed_form(o):
    """[EQ] with T = 1 and H_0 = 0: H_1 = (1 - f) tanh(k v^T) (the H W term
    vanishes) and y_1 = H_1^T q + w_r * v."""
    rng = np.random.default_rng(RNG_SEED)
    B, T, N, K, V = 2, 1, 3, 5, 4
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V)
    y, HT = o.forward(q, k, v, f, W, wr)
    for b in range(B):
        for n in range(N):
            H1 = (1 - f[b, 0, n]) * np.tanh(np.outer(k[b, 0], v[b, 0, n]))
            _close(HT[b, n], H1, 1e-15, "T=1 H_1")
            _close(y[b, 0, n], H1.T @ q[b, 0] + wr[n] * v[b, 0, n], 1e-14, "T=1 y_1")


def pin_zero_w_zero_f_forward(o):
    """[EQ] with W = 0 and f = 0: every step forgets, so H_t = tanh(k_t v_t^T)
    exactly and y_t = tanh(k_t v_t^T)^T q_t + w_r * v_t."""
    rng = np.random.default_rng(RNG_SEED + 1)
    B, T, N, K, V = 2, 6, 2, 64, 16
    q, k, v, _, _, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.zeros((B, T, N))
    W = np.zeros((N, V, V))
    y, HT = o.forward(q, k, v, f, W, wr)
    for b in range(B):
        for n in range(N):
            for t in range(T):
                Z = np.tanh(np.outer(k[b, t], v[b, t, n]))
                _close(y[b, t, n], Z.T @ q[b, t] + wr[n] * v[b, t, n], 1e-13, "W=0,f=0 y")
            _close(HT[b, n], np.tanh(np.outer(k[b, T - 1], v[b, T - 1, n])), 1e-15, "W=0,f=0 H_T")


def pin_f_one_forward(o):
    """[EQ] with f = 1: H_t = H_{t-1} = H_0 = 0 for all t, so H_T = 0 and
    y_t = w_r * v_t, bit-exact."""
    rng = np.random.default_rng(RNG_SEED + 2)
    B, T, N, K, V = 2, 7, 3, 64, 16
    q, k, v, _, W, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.ones((B, T, N))
    y, HT = o.forward(q, k, v, f, W, wr)
    assert np.array_equal(HT, np.zeros_like(HT)), "f=1 must keep H = 0"
    assert np.array_equal(y, wr[None, None] * v), "f=1 must give y = w_r * v exactly"


def pin_rnn_embedding_forward_backward(o):
    """[RNN]: f = 0, w_r = 0, q = k = e_1 gives y_t = h_t of the textbook Elman
    RNN h_t = tanh(W^T h_{t-1} + v_t), i.e. torch.nn.RNN with weight_ih = I and
    weight_hh = W^T.  Its autograd gradient of sum(y * dy) pins the oracle's dv
    (= dL/dx) and dW (= (dL/dweight_hh)^T) too."""
    rng = np.random.default_rng(RNG_SEED + 3)
    B, T, N, K, V = 2, 9, 2, 64, 16
    _, _, v, _, W, _ = _rand_inputs(rng, B, T, N, K, V)
    W = W * 2.0  # strong recurrence, so an orientation slip shows
    q = np.zeros((B, T, K))
    q[:, :, 0] = 1.0
    k = q.copy()
    f = np.zeros((B, T, N))
    wr = np.zeros((N, V))
    dy = rng.standard_normal((B, T, N, V))
    y, _ = o.forward(q, k, v, f, W, wr)
    g = o.backward(q, k, v, f, W, wr, dy)
    for n in range(N):
        rnn = torch.nn.RNN(V, V, nonlinearity="tanh", bias=False, batch_first=True).double()
        with torch.no_grad():
            rnn.weight_ih_l0.copy_(torch.eye(V, dtype=torch.float64))
            rnn.weight_hh_l0.copy_(torch.from_numpy(W[n].T.copy()))
        x = torch.from_numpy(v[:, :, n].copy()).requires_grad_(True)
        h, _ = rnn(x)
        _close(y[:, :, n], h.detach().numpy(), 1e-13, "RNN embedding y")
        (h * torch.from_numpy(dy[:, :, n].copy())).sum().backward()
        _close(g["dv"][:, :, n], x.grad.numpy(), 1e-12, "RNN embedding dv")
        _close(g["dW"][n], rnn.weight_hh_l0.grad.numpy().T, 1e-11, "RNN embedding dW")


def pin_convex_bound(o):
    """[EQ]: H_t is a convex combination of H_{t-1} and tanh(.) in [-1, 1], so
    |H_t| <= 1 elementwise for f in [0, 1], even for large inputs."""
    rng = np.random.default_rng(RNG_SEED + 4)
    B, T, N, K, V = 2, 40, 3, 64, 16
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V, scale=4.0)
    W = W * 5.0
    f[:, ::3] = 0.0
    f[:, 1::7] = 1.0
    _, HT, ck = o.forward(q, k, v, f, W, wr, ckpt_every=1)
    assert np.all(np.abs(ck) <= 1.0) and np.all(np.abs(HT) <= 1.0), "|H| must stay <= 1"
    assert np.max(np.abs(HT)) > 0.5, "bound test must reach the saturated regime"


def pin_checkpoints(o):
    """H_ckpt[j] is the state after j*c steps (H_0 = 0 for j = 0): it must equal
    H_T of the same recurrence run for j*c steps."""
    rng = np.random.default_rng(RNG_SEED + 5)
    B, T, N, K, V = 1, 11, 2, 8, 4
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V)
    c = 4
    _, HT, ck = o.forward(q, k, v, f, W, wr, ckpt_every=c)
    assert ck.shape == (B, N, 3, K, V)
    assert np.array_equal(ck[:, :, 0], np.zeros((B, N, K, V))), "ckpt 0 must be H_0 = 0"
    for j in (1, 2):
        _, HTj = o.forward(q[:, :j * c], k[:, :j * c], v[:, :j * c], f[:, :j * c], W, wr)
        assert np.array_equal(ck[:, :, j], HTj), f"ckpt {j} != H after {j * c} steps"


def pin_permutations(o):
    """Symmetries of [EQ] and [SH]:
    - permuting the K index of q and k together permutes the rows of H_T and
      leaves y unchanged (dq, dk permute the same way, the rest is unchanged);
    - permuting the value channels of v, w_r and both indices of W permutes the
      columns of H_T and the channels of y;
    - permuting heads or batch rows permutes the outputs."""
    rng = np.random.default_rng(RNG_SEED + 6)
    B, T, N, K, V = 3, 6, 4, 8, 5
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V)
    dy = rng.standard_normal((B, T, N, V))
    y, HT = o.forward(q, k, v, f, W, wr)
    g = o.backward(q, k, v, f, W, wr, dy)
    tol = 1e-13

    p = rng.permutation(K)
    y2, HT2 = o.forward(q[..., p], k[..., p], v, f, W, wr)
    _close(y2, y, tol, "row perm y")
    _close(HT2, HT[:, :, p, :], tol, "row perm H_T")
    g2 = o.backward(q[..., p], k[..., p], v, f, W, wr, dy)
    _close(g2["dq"], g["dq"][..., p], tol, "row perm dq")
    _close(g2["dk"], g["dk"][..., p], tol, "row perm dk")
    for name in ("dv", "df", "dW", "dwr"):
        _close(g2[name], g[name], tol, f"row perm {name}")

    s = rng.permutation(V)
    y3, HT3 = o.forward(q, k, v[..., s], f, W[:, s][:, :, s], wr[:, s])
    _close(y3, y[..., s], tol, "value perm y")
    _close(HT3, HT[..., s], tol, "value perm H_T")

    h = rng.permutation(N)
    y4, HT4 = o.forward(q, k, v[:, :, h], f[:, :, h], W[h], wr[h])
    _close(y4, y[:, :, h], tol, "head perm y")
    _close(HT4, HT[:, h], tol, "head perm H_T")
    g4 = o.backward(q, k, v[:, :, h], f[:, :, h], W[h], wr[h], dy[:, :, h])
    _close(g4["dq"], g["dq"], tol, "head perm dq")
    _close(g4["dk"], g["dk"], tol, "head perm dk")
    _close(g4["dW"], g["dW"][h], tol, "head perm dW")

    bp = rng.permutation(B)
    y5, HT5 = o.forward(q[bp], k[bp], v[bp], f[bp], W, wr)
    _close(y5, y[bp], tol, "batch perm y")
    _close(HT5, HT[bp], tol, "batch perm H_T")


def pin_readout_linear_in_q(o):
    """[EQ]: q enters only through the readout, so y - w_r * v is linear in q."""
    rng = np.random.default_rng(RNG_SEED + 7)
    B, T, N, K, V = 2, 5, 2, 8, 4
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V)
    q2 = rng.standard_normal(q.shape)
    base = wr[None, None] * v
    ya, _ = o.forward(q, k, v, f, W, wr)
    yb, _ = o.forward(q2, k, v, f, W, wr)
    yc, _ = o.forward(q + 2.0 * q2, k, v, f, W, wr)
    _close(yc - base, (ya - base) + 2.0 * (yb - base), 1e-13, "linearity in q")


# --------------------------------------------------------------- backward pins

def pin_f_one_backward(o):
    """[BW] with f = 1: D_t = 0, so C_{t-1} = R_t and C_t = dH_T + sum_{s>t}
    q_s u_s^T.  Hence dW = dk = dq = 0, dv = w_r * u, dw_r = sum_t u * v and
    df_t = <dH_T + sum_{s>=t} q_s u_s^T, 0 - tanh(k_t v_t^T)>."""
    rng = np.random.default_rng(RNG_SEED + 8)
    B, T, N, K, V = 2, 6, 3, 8, 5
    q, k, v, _, W, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.ones((B, T, N))
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    g = o.backward(q, k, v, f, W, wr, dy, dHT)
    for name in ("dW", "dk", "dq"):
        assert np.array_equal(g[name], np.zeros_like(g[name])), f"f=1: {name} must be 0"
    _close(g["dv"], wr[None, None] * dy, 0.0, "f=1 dv")
    _close(g["dwr"], np.einsum("btnj,btnj->nj", dy, v), 1e-12, "f=1 dwr")
    for b in range(B):
        for n in range(N):
            acc = dHT[b, n].copy()
            for t in range(T - 1, -1, -1):
                acc = acc + np.outer(q[b, t], dy[b, t, n])
                Z = np.tanh(np.outer(k[b, t], v[b, t, n]))
                _close(g["df"][b, t, n], -np.sum(acc * Z), 1e-12, "f=1 df")


def pin_zero_w_zero_f_backward(o):
    """[BW] with W = 0, f = 0 and no dH_T: C_{t-1} = f R_t + D_t W^T = 0, so
    R_t = q_t u_t^T, H_t = Z_t = tanh(k_t v_t^T), D_t = R_t * (1 - Z_t^2), and
    df_t = <R_t, Z_{t-1} - Z_t>, dW = sum_t Z_{t-1}^T D_t, dk_t = sum_n D_t v_t,
    dv_t = D_t^T k_t + w_r * u_t, dq_t = sum_n Z_t u_t."""
    rng = np.random.default_rng(RNG_SEED + 9)
    B, T, N, K, V = 2, 5, 3, 8, 4
    q, k, v, _, _, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.zeros((B, T, N))
    W = np.zeros((N, V, V))
    dy = rng.standard_normal((B, T, N, V))
    g = o.backward(q, k, v, f, W, wr, dy)
    dW = np.zeros((N, V, V))
    for b in range(B):
        dq = np.zeros((T, K))
        dk = np.zeros((T, K))
        for n in range(N):
            Zprev = np.zeros((K, V))
            for t in range(T):
                Z = np.tanh(np.outer(k[b, t], v[b, t, n]))
                R = np.outer(q[b, t], dy[b, t, n])
                D = R * (1 - Z * Z)
                _close(g["df"][b, t, n], np.sum(R * (Zprev - Z)), 1e-12, "W=0,f=0 df")
                _close(g["dv"][b, t, n], D.T @ k[b, t] + wr[n] * dy[b, t, n], 1e-12, "W=0,f=0 dv")
                dW[n] += Zprev.T @ D
                dk[t] += D @ v[b, t, n]
                dq[t] += Z @ dy[b, t, n]
                Zprev = Z
        _close(g["dq"][b], dq, 1e-12, "W=0,f=0 dq")
        _close(g["dk"][b], dk, 1e-12, "W=0,f=0 dk")
    _close(g["dW"], dW, 1e-12, "W=0,f=0 dW")


def _loss(o, ins, dy, dHT):
    y, HT = o.forward(*ins)
    return float(np.sum(y * dy) + np.sum(HT * dHT))


def _fd_check(o, B, T, N, K, V, seed, tol=1e-6, h=1e-6):
    rng = np.random.default_rng(seed)
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V, f_lo=0.05, f_hi=0.95)
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    ins = [q, k, v, f, W, wr]
    g = o.backward(*ins, dy, dHT)
    names = ["dq", "dk", "dv", "df", "dW", "dwr"]
    for idx, name in enumerate(names):
        x = ins[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            orig = x[mi]
            x[mi] = orig + h
            lp = _loss(o, ins, dy, dHT)
            x[mi] = orig - h
            lm = _loss(o, ins, dy, dHT)
            x[mi] = orig
            fd[mi] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(fd - g[name])))
        assert err <= tol * scale, f"FD {name}: max abs diff {err:.3e} > {tol * scale:.1e}"


def pin_finite_differences_small(o):
    """[BW] against brute force: central differences of
    L = sum(y * dy) + sum(H_T * dH_T) over every element of q, k, v, f, W, w_r,
    at B=2, T=5, N=3, K=4, V=3."""
    _fd_check(o, 2, 5, 3, 4, 3, RNG_SEED + 10)


def pin_finite_differences_full_state(o):
    """Same brute-force check at the real state shape K=64, V=16 (B=1, T=3, N=2)."""
    _fd_check(o, 1, 3, 2, 64, 16, RNG_SEED + 11)


def pin_thread_invariance(o):
    """Outputs do not depend on the number of host threads (fixed summation
    order over heads and batch rows)."""
    rng = np.random.default_rng(RNG_SEED + 12)
    B, T, N, K, V = 3, 7, 5, 8, 4
    ins = _rand_inputs(rng, B, T, N, K, V)
    dy = rng.standard_normal((B, T, N, V))
    y1, H1 = o.forward(*ins, nthreads=1)
    y4, H4 = o.forward(*ins, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(H1, H4)
    g1 = o.backward(*ins, dy, nthreads=1)
    g4 = o.backward(*ins, dy, nthreads=4)
    for name in g1:
        assert np.array_equal(g1[name], g4[name]), name


# ---------------------------------------------------------- initial-state pins

def _rand_state(rng, B, N, K, V):
    return np.tanh(rng.standard_normal((B, N, K, V)))   # a reachable state, |H| < 1


def pin_initial_state_f_one(o):
    """[H0] with f = 1 the state never moves: H_T = H_0 and
    y_t = H_0^T q_t + w_r * v_t; D_t = 0, so dW = dk = 0,
    dq_t = sum_n H_0 u_t and dH_0 = C_0 = dH_T + sum_t q_t u_t^T."""
    rng = np.random.default_rng(RNG_SEED + 20)
    B, T, N, K, V = 2, 5, 3, 6, 4
    q, k, v, _, W, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.ones((B, T, N))
    H0 = _rand_state(rng, B, N, K, V)
    y, HT = o.forward(q, k, v, f, W, wr, H_0=H0)
    assert np.array_equal(HT, H0), "f=1: H_T must equal H_0"
    _close(y, np.einsum("bnkv,btk->btnv", H0, q) + wr[None, None] * v, 1e-13, "f=1 y from H_0")
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    g = o.backward(q, k, v, f, W, wr, dy, dHT, H_0=H0)
    for name in ("dW", "dk"):
        assert np.array_equal(g[name], np.zeros_like(g[name])), f"f=1: {name} must be 0"
    _close(g["dq"], np.einsum("bnkv,btnv->btk", H0, dy), 1e-12, "f=1 dq from H_0")
    _close(g["dH_0"], dHT + np.einsum("btk,btnv->bnkv", q, dy), 1e-12, "f=1 dH_0")


def pin_initial_state_forgotten(o):
    """[H0] with W = 0 and f = 0 the first step forgets H_0 entirely
    (H_1 = tanh(k_1 v_1^T)): every output equals that of the H_0 = 0 run and
    dH_0 = f_1 R_1 + D_1 W^T = 0."""
    rng = np.random.default_rng(RNG_SEED + 21)
    B, T, N, K, V = 2, 4, 2, 5, 3
    q, k, v, _, _, wr = _rand_inputs(rng, B, T, N, K, V)
    f = np.zeros((B, T, N))
    W = np.zeros((N, V, V))
    H0 = _rand_state(rng, B, N, K, V)
    y0, H0T = o.forward(q, k, v, f, W, wr)
    y1, H1T = o.forward(q, k, v, f, W, wr, H_0=H0)
    assert np.array_equal(y0, y1) and np.array_equal(H0T, H1T)
    dy = rng.standard_normal((B, T, N, V))
    g = o.backward(q, k, v, f, W, wr, dy, H_0=H0)
    assert np.array_equal(g["dH_0"], np.zeros_like(g["dH_0"])), "W=0, f=0: dH_0 must be 0"


def pin_split_sequence(o):
    """[H0]: a run over T steps equals a run over the first T1 steps followed by
    one over the rest started from its H_T (the state carries everything); in
    the backward, dH_0 of the second part is the dH_T of the first, and the two
    parts together give the full run's gradients."""
    rng = np.random.default_rng(RNG_SEED + 22)
    B, T, N, K, V, T1 = 2, 9, 3, 6, 4, 4
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V)
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    a = lambda x: x[:, :T1]
    z = lambda x: x[:, T1:]
    y, HT = o.forward(q, k, v, f, W, wr)
    ya, HA = o.forward(a(q), a(k), a(v), a(f), W, wr)
    yb, HB = o.forward(z(q), z(k), z(v), z(f), W, wr, H_0=HA)
    assert np.array_equal(np.concatenate([ya, yb], axis=1), y) and np.array_equal(HB, HT)
    g = o.backward(q, k, v, f, W, wr, dy, dHT)
    gb = o.backward(z(q), z(k), z(v), z(f), W, wr, z(dy), dHT, H_0=HA)
    ga = o.backward(a(q), a(k), a(v), a(f), W, wr, a(dy), gb["dH_0"])
    for name in ("dq", "dk", "dv", "df"):
        _close(np.concatenate([ga[name], gb[name]], axis=1), g[name], 1e-12, f"split {name}")
    for name in ("dW", "dwr"):
        _close(ga[name] + gb[name], g[name], 1e-12, f"split {name}")
    _close(ga["dH_0"], g["dH_0"], 1e-12, "split dH_0")


def pin_finite_differences_initial_state(o):
    """[BW] and [H0] against brute force, with a non-zero H_0: central
    differences of L = sum(y * dy) + sum(H_T * dH_T) over every element of H_0
    and of q, k, v, f, W, w_r (B=2, T=4, N=2, K=4, V=3)."""
    rng = np.random.default_rng(RNG_SEED + 23)
    B, T, N, K, V = 2, 4, 2, 4, 3
    q, k, v, f, W, wr = _rand_inputs(rng, B, T, N, K, V, f_lo=0.05, f_hi=0.95)
    H0 = _rand_state(rng, B, N, K, V)
    dy = rng.standard_normal((B, T, N, V))
    dHT = rng.standard_normal((B, N, K, V))
    ins = [q, k, v, f, W, wr, H0]
    g = o.backward(q, k, v, f, W, wr, dy, dHT, H_0=H0)

    def loss():
        y, HT = o.forward(*ins[:6], H_0=ins[6])
        return float(np.sum(y * dy) + np.sum(HT * dHT))

    h = 1e-6
    for idx, name in enumerate(["dq", "dk", "dv", "df", "dW", "dwr", "dH_0"]):
        x = ins[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            orig = x[mi]
            x[mi] = orig + h
            lp = loss()
            x[mi] = orig - h
            lm = loss()
            x[mi] = orig
            fd[mi] = (lp - lm) / (2 * h)
        scale = max(1.0, float(np.max(np.abs(fd))))
        err = float(np.max(np.abs(fd - g[name])))
        assert err <= 1e-6 * scale, f"FD {name} (H_0 != 0): max abs diff {err:.3e}"



# ----------------------------------------------------------------- gate pins

def _gate_inputs(rng, B, T, N):
    a = rng.standard_normal((B, T, N)) * 2.0
    a[0, 0, :] = [50.0, -50.0, 0.0][:N] + [0.0] * max(0, N - 3)   # saturated arguments
    alpha = rng.uniform(0.2, 2.5, N)
    beta = rng.uniform(-3.0, 1.0, N)
    return a, alpha, beta


def pin_gate_sigmoid_identity(o):
    """[GT] with alpha = 1: exp(-softplus(x)) = 1 / (1 + e^x), here via
    scipy's expit, including saturated arguments x = +-50."""
    from scipy.special import expit
    rng = np.random.default_rng(RNG_SEED + 30)
    a, _, beta = _gate_inputs(rng, 2, 7, 3)
    f = o.gate_forward(a, np.ones(3), beta)
    _close(f, expit(-(a + beta)), 1e-15, "gate alpha=1")


def pin_gate_alpha_zero(o):
    """[GT] alpha = 0 keeps the state (f = 1, the slide's endpoint): da = 0,
    dbeta = 0 and dalpha = -sum df * softplus(a + beta) (numpy's logaddexp)."""
    rng = np.random.default_rng(RNG_SEED + 31)
    a, _, beta = _gate_inputs(rng, 2, 5, 3)
    alpha = np.zeros(3)
    assert np.array_equal(o.gate_forward(a, alpha, beta), np.ones_like(a))
    df = rng.standard_normal(a.shape)
    da, dal, dbe = o.gate_backward(a, alpha, beta, df)
    assert np.array_equal(da, np.zeros_like(da)) and np.array_equal(dbe, np.zeros_like(dbe))
    _close(dal, -np.sum(df * np.logaddexp(0.0, a + beta), axis=(0, 1)), 1e-12, "gate alpha=0 dalpha")


def pin_gate_power_law_and_range(o):
    """[GT]: f(alpha) = f(1)^alpha, and alpha >= 0 keeps f in [0, 1]."""
    rng = np.random.default_rng(RNG_SEED + 32)
    a, alpha, beta = _gate_inputs(rng, 3, 6, 4)
    f = o.gate_forward(a, alpha, beta)
    f1 = o.gate_forward(a, np.ones(4), beta)
    _close(f, f1 ** alpha, 1e-14, "gate power law")
    assert np.all(f >= 0.0) and np.all(f <= 1.0)


def pin_gate_large_arguments(o):
    """[GT] for x = a + beta >= 40, softplus(x) = x in double precision, so
    f = exp(-alpha x) exactly; with a small alpha f stays well above zero even
    where e^x overflows (x = 750), and the gradients stay finite."""
    a = np.array([[[40.0, 300.0, 750.0]]])
    alpha = np.array([0.5, 0.02, 0.01])
    beta = np.zeros(3)
    f = o.gate_forward(a, alpha, beta)
    _close(f, np.exp(-alpha * a), 1e-15, "gate large x")
    da, dal, dbe = o.gate_backward(a, alpha, beta, np.ones_like(a))
    assert np.all(np.isfinite(da)) and np.all(np.isfinite(dal)) and np.all(np.isfinite(dbe))
    _close(dal, -(np.exp(-alpha * a) * a)[0, 0], 1e-12, "gate large x dalpha")


def pin_gate_finite_differences(o):
    """[GT] backward against central differences of L = sum(f * df) over every
    element of a, alpha and beta."""
    rng = np.random.default_rng(RNG_SEED + 33)
    B, T, N = 2, 4, 3
    a = rng.standard_normal((B, T, N)) * 2.0
    alpha = rng.uniform(0.2, 2.5, N)
    beta = rng.uniform(-3.0, 1.0, N)
    df = rng.standard_normal((B, T, N))
    da, dal, dbe = o.gate_backward(a, alpha, beta, df)
    h = 1e-6
    ins = [a, alpha, beta]
    for idx, got in enumerate([da, dal, dbe]):
        x = ins[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            orig = x[mi]
            x[mi] = orig + h
            lp = float(np.sum(o.gate_forward(*ins) * df))
            x[mi] = orig - h
            lm = float(np.sum(o.gate_forward(*ins) * df))
            x[mi] = orig
            fd[mi] = (lp - lm) / (2 * h)
        _close(got, fd, 1e-7 * max(1.0, float(np.max(np.abs(fd)))), f"gate FD {['da', 'dalpha', 'dbeta'][idx]}")


def _norm_inputs(rng, ntok, d):
    y = rng.standard_normal((ntok, d))
    g = rng.standard_normal((ntok, d))
    w = rng.standard_normal(d)
    return y, g, w


def pin_norm_torch_rms_norm(o):
    """[NRM] against torch.nn.functional.rms_norm in float64 applied to the
    gated features y * g, forward and (through torch autograd, including the
    product with g) backward, with and without eps."""
    rng = np.random.default_rng(RNG_SEED + 40)
    y, g, w = _norm_inputs(rng, 6, 48)
    dout = rng.standard_normal(y.shape)
    for eps in (0.0, 1e-3):
        out, rstd = o.gate_rmsnorm_forward(y, g, w, eps)
        ty = torch.tensor(y, requires_grad=True)
        tg = torch.tensor(g, requires_grad=True)
        tw = torch.tensor(w, requires_grad=True)
        ref = torch.nn.functional.rms_norm(ty * tg, (48,), weight=tw, eps=eps)
        (ref * torch.tensor(dout)).sum().backward()
        _close(out, ref.detach().numpy(), 1e-13, f"rmsnorm eps={eps}")
        _close(rstd, 1.0 / np.sqrt(np.mean((y * g) ** 2, axis=-1) + eps), 1e-13, f"rstd eps={eps}")
        dy, dg, dw = o.gate_rmsnorm_backward(y, g, w, dout, eps)
        _close(dy, ty.grad.numpy(), 1e-12, f"rmsnorm dy eps={eps}")
        _close(dg, tg.grad.numpy(), 1e-12, f"rmsnorm dg eps={eps}")
        _close(dw, tw.grad.numpy(), 1e-12, f"rmsnorm dw eps={eps}")


def pin_norm_invariances(o):
    """[NRM] at eps = 0: the output does not change when a token's y is scaled
    by c > 0 and flips sign with it; o / w has unit mean square per token; and
    the gradient is orthogonal to the scaling direction (sum_j dy_j y_j = 0 and
    sum_j dg_j g_j = 0 per token)."""
    rng = np.random.default_rng(RNG_SEED + 41)
    y, g, w = _norm_inputs(rng, 5, 32)
    out, _ = o.gate_rmsnorm_forward(y, g, w)
    c = np.array([0.01, 1.0, 3.0, 250.0, 7.5])[:, None]
    _close(o.gate_rmsnorm_forward(y * c, g, w)[0], out, 1e-13, "rmsnorm scale invariance")
    _close(o.gate_rmsnorm_forward(-y, g, w)[0], -out, 1e-15, "rmsnorm odd")
    _close(np.mean((out / w) ** 2, axis=-1), np.ones(5), 1e-13, "rmsnorm unit rms")
    dy, dg, _ = o.gate_rmsnorm_backward(y, g, w, rng.standard_normal(y.shape))
    _close(np.sum(dy * y, axis=-1), np.zeros(5), 1e-12, "rmsnorm dy orthogonal to y")
    _close(np.sum(dg * g, axis=-1), np.zeros(5), 1e-12, "rmsnorm dg orthogonal to g")


def pin_norm_constant_token(o):
    """[NRM] a token whose gated features all equal c: s = 1/|c| and
    o = w sign(c) (eps = 0); with eps, s = 1/sqrt(c^2 + eps)."""
    d = 20
    y = np.array([[0.5] * d, [-4.0] * d])
    g = np.array([[3.0] * d, [0.25] * d])
    w = np.linspace(-1.0, 2.0, d)
    out, rstd = o.gate_rmsnorm_forward(y, g, w)
    _close(out, np.stack([w, -w]), 1e-15, "rmsnorm constant token")
    _close(rstd, np.array([1.0 / 1.5, 1.0]), 1e-15, "rmsnorm constant rstd")
    _, rstd = o.gate_rmsnorm_forward(y, g, w, 0.75)
    _close(rstd, np.array([1.0 / np.sqrt(1.5 ** 2 + 0.75), 1.0 / np.sqrt(1.0 + 0.75)]), 1e-15, "rmsnorm eps rstd")


def pin_norm_finite_differences(o):
    """[NRM] backward against central differences of L = sum(o * dout) over
    every element of y, g and w (eps = 1e-3)."""
    rng = np.random.default_rng(RNG_SEED + 42)
    y, g, w = _norm_inputs(rng, 3, 8)
    dout = rng.standard_normal(y.shape)
    eps = 1e-3
    dy, dg, dw = o.gate_rmsnorm_backward(y, g, w, dout, eps)
    ins = [y, g, w]
    h = 1e-6
    for idx, got in enumerate([dy, dg, dw]):
        x = ins[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            orig = x[mi]
            x[mi] = orig + h
            lp = float(np.sum(o.gate_rmsnorm_forward(*ins, eps)[0] * dout))
            x[mi] = orig - h
            lm = float(np.sum(o.gate_rmsnorm_forward(*ins, eps)[0] * dout))
            x[mi] = orig
            fd[mi] = (lp - lm) / (2 * h)
        _close(got, fd, 1e-7 * max(1.0, float(np.max(np.abs(fd)))), f"rmsnorm FD {['dy', 'dg', 'dw'][idx]}")


def _conv_inputs(rng, B, T, C):
    u = rng.standard_normal((B, T, C)) * 1.5
    w = rng.standard_normal((C, 4)) * 0.6
    bias = rng.standard_normal(C) * 0.5
    return u, w, bias


def pin_conv_torch_conv1d(o):
    """[CNV] against torch.nn.functional.conv1d (groups = C, padding 3, the
    first T outputs) and torch.nn.functional.silu in float64, forward and,
    through torch autograd, du, dw and dbias; with and without a bias."""
    rng = np.random.default_rng(RNG_SEED + 50)
    B, T, C = 2, 11, 5
    u, w, bias = _conv_inputs(rng, B, T, C)
    dz = rng.standard_normal((B, T, C))
    for use_bias in (True, False):
        b = bias if use_bias else None
        tu = torch.tensor(u, requires_grad=True)
        tw = torch.tensor(w, requires_grad=True)
        tb = torch.tensor(bias, requires_grad=True) if use_bias else None
        a = torch.nn.functional.conv1d(tu.transpose(1, 2), tw.unsqueeze(1), tb, padding=3, groups=C)[..., :T]
        ref = torch.nn.functional.silu(a).transpose(1, 2)
        (ref * torch.tensor(dz)).sum().backward()
        _close(o.conv_silu_forward(u, w, b), ref.detach().numpy(), 1e-13, f"conv silu bias={use_bias}")
        du, dw, db = o.conv_silu_backward(u, w, b, dz)
        _close(du, tu.grad.numpy(), 1e-12, f"conv du bias={use_bias}")
        _close(dw, tw.grad.numpy(), 1e-12, f"conv dw bias={use_bias}")
        if use_bias:
            _close(db, tb.grad.numpy(), 1e-12, "conv dbias")


def pin_conv_impulse_and_causality(o):
    """[CNV] a unit impulse at (t0, c) gives a = bias + w[c][3 - (t - t0)] for
    t0 <= t <= t0 + 3 and a = bias elsewhere (closed form, silu written out
    with numpy); a change of u at t0 leaves every z before t0 unchanged."""
    rng = np.random.default_rng(RNG_SEED + 51)
    B, T, C, t0, c = 1, 12, 3, 5, 1
    _, w, bias = _conv_inputs(rng, B, T, C)
    u = np.zeros((B, T, C))
    u[0, t0, c] = 1.0
    a = np.tile(bias, (B, T, 1))
    for t in range(t0, min(T, t0 + 4)):
        a[0, t, c] += w[c, 3 - (t - t0)]
    _close(o.conv_silu_forward(u, w, bias), a / (1.0 + np.exp(-a)), 1e-15, "conv impulse")
    u2, _, _ = _conv_inputs(rng, 2, T, C)
    z1 = o.conv_silu_forward(u2, w, bias)
    u3 = u2.copy()
    u3[:, t0:] += rng.standard_normal((2, T - t0, C))
    z2 = o.conv_silu_forward(u3, w, bias)
    assert np.array_equal(z1[:, :t0], z2[:, :t0]), "conv is not causal"
    assert not np.allclose(z1[:, t0:], z2[:, t0:])


def pin_conv_identity_taps(o):
    """[CNV] taps (0, 0, 0, 1) and no bias make z = silu(u) exactly, and the
    gradient du = dz silu'(u) with silu'(x) = s (1 + x (1 - s))."""
    rng = np.random.default_rng(RNG_SEED + 52)
    u, _, _ = _conv_inputs(rng, 2, 7, 4)
    w = np.zeros((4, 4))
    w[:, 3] = 1.0
    s = 1.0 / (1.0 + np.exp(-u))
    _close(o.conv_silu_forward(u, w), u * s, 1e-15, "conv identity taps")
    dz = rng.standard_normal(u.shape)
    du, _, _ = o.conv_silu_backward(u, w, None, dz)
    _close(du, dz * s * (1.0 + u * (1.0 - s)), 1e-14, "conv identity du")


def pin_conv_finite_differences(o):
    """[CNV] backward against central differences of L = sum(z * dz) over every
    element of u, w and bias."""
    rng = np.random.default_rng(RNG_SEED + 53)
    u, w, bias = _conv_inputs(rng, 2, 6, 3)
    dz = rng.standard_normal(u.shape)
    du, dw, db = o.conv_silu_backward(u, w, bias, dz)
    ins = [u, w, bias]
    h = 1e-6
    for idx, got in enumerate([du, dw, db]):
        x = ins[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            orig = x[mi]
            x[mi] = orig + h
            lp = float(np.sum(o.conv_silu_forward(*ins) * dz))
            x[mi] = orig - h
            lm = float(np.sum(o.conv_silu_forward(*ins) * dz))
            x[mi] = orig
            fd[mi] = (lp - lm) / (2 * h)
        _close(got, fd, 1e-7 * max(1.0, float(np.max(np.abs(fd)))), f"conv FD {['du', 'dw', 'dbias'][idx]}")


FORWARD_PINS = [pin_t1_closed_form, pin_f_one_forward, pin_zero_w_zero_f_forward, pin_readout_linear_in_q,
                pin_checkpoints, pin_convex_bound, pin_permutations, pin_rnn_embedding_forward_backward]
BACKWARD_PINS = [pin_f_one_backward, pin_zero_w_zero_f_backward, pin_finite_differences_small,
                 pin_finite_differences_full_state]
INITIAL_STATE_PINS = [pin_initial_state_f_one, pin_initial_state_forgotten, pin_split_sequence,
                      pin_finite_differences_initial_state]
GATE_PINS = [pin_gate_sigmoid_identity, pin_gate_alpha_zero, pin_gate_power_law_and_range,
             pin_gate_large_arguments, pin_gate_finite_differences]
NORM_PINS = [pin_norm_torch_rms_norm, pin_norm_invariances, pin_norm_constant_token, pin_norm_finite_differences]
CONV_PINS = [pin_conv_torch_conv1d, pin_conv_impulse_and_causality, pin_conv_identity_taps,
             pin_conv_finite_differences]
ALL_PINS = (FORWARD_PINS + BACKWARD_PINS + INITIAL_STATE_PINS + GATE_PINS + NORM_PINS + CONV_PINS
            + [pin_thread_invariance])
