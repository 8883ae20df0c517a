"""Pins of the fp64 backward oracle (oracle/backward.py) against things other than
itself: central finite differences of the forward oracle, exact rational
forward-mode derivatives (dual numbers over fractions.Fraction, alpha rational),
closed forms of the single-token case derived by hand, the chunk form against the
token form, and the beta = 0 invariant.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from oracle.backward import chunked_backward, token_backward_numpy
from oracle.token import token_recurrence_numpy


def _case(B, T, H, dk, dv, seed, h0=True, dhT=True, gate_lo=-0.6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = rng.uniform(gate_lo, 0.0, (B, T, H))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    do = rng.standard_normal((B, T, H, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, do=do)


def _loss(c, h0, dhT, cu=None, scale=None):
    o, hT = token_recurrence_numpy(c["q"], c["k"], c["v"], c["g"], c["beta"], h0, cu, scale)
    L = np.sum(o * c["do"])
    if dhT is not None:
        L += np.sum(hT * dhT)
    return L


@pytest.mark.parametrize("packed", [False, True])
def test_token_backward_matches_central_differences(packed):
    B, T, H, dk, dv = (1, 7, 2, 3, 2) if packed else (2, 5, 2, 3, 2)
    cu = np.array([0, 3, 7]) if packed else None
    N = 2
    c = _case(B, T, H, dk, dv, seed=11 + packed)
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal((N, H, dk, dv)) * 0.5
    dhT = rng.standard_normal((N, H, dk, dv))
    grads = token_backward_numpy(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], dhT, h0, cu)
    names = ["q", "k", "v", "g", "beta"]
    eps = 1e-6
    for name, gr in zip(names + ["h0"], grads):
        base = h0 if name == "h0" else c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            for sgn in (1, -1):
                pert = base.copy()
                pert[idx] += sgn * eps
                if name == "h0":
                    L = _loss(c, pert, dhT, cu)
                else:
                    cc = dict(c)
                    cc[name] = pert
                    L = _loss(cc, h0, dhT, cu)
                fd[idx] += sgn * L / (2 * eps)
        err = np.max(np.abs(fd - gr)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


class Dual:
    """a + b eps with eps^2 = 0, exact over Fractions (forward-mode derivative)."""

    def __init__(self, a, b=Fraction(0)):
        self.a, self.b = Fraction(a), Fraction(b)

    def __add__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a - o.a, self.b - o.b)

    def __rsub__(self, o):
        return Dual(o) - self

    def __mul__(self, o):
        o = o if isinstance(o, Dual) else Dual(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__


def _exact_loss(q, k, v, alpha, beta, h0, do, dhT, scale):
    """L = sum do.o + sum dhT.hT for one sequence and head, every entry a Dual; the
    recurrence written entrywise: S <- alpha S (I - beta k k^T) + beta v k^T."""
    T, dk = len(q), len(q[0])
    dv = len(v[0])
    S = [[h0[i][j] for i in range(dk)] for j in range(dv)]   # S = h0^T, dv x dk
    L = Dual(0)
    for t in range(T):
        Sk = [sum((S[j][i] * k[t][i] for i in range(dk)), Dual(0)) for j in range(dv)]
        S = [[alpha[t] * (S[j][i] - beta[t] * Sk[j] * k[t][i]) + beta[t] * v[t][j] * k[t][i]
              for i in range(dk)] for j in range(dv)]
        for j in range(dv):
            o = scale * sum((S[j][i] * q[t][i] for i in range(dk)), Dual(0))
            L = L + do[t][j] * o
    for j in range(dv):
        for i in range(dk):
            L = L + dhT[i][j] * S[j][i]
    return L


def test_token_backward_matches_exact_rational_derivatives():
    T, dk, dv = 3, 2, 2
    fr = lambda a, b: Fraction(a, b)  # noqa: E731
    q = [[fr(1, 2), fr(-1, 3)], [fr(2, 5), fr(1, 7)], [fr(-3, 4), fr(1, 2)]]
    k = [[fr(3, 5), fr(4, 5)], [fr(1, 1), fr(0, 1)], [fr(5, 13), fr(-12, 13)]]   # unit keys
    v = [[fr(1, 3), fr(-2, 1)], [fr(1, 4), fr(3, 5)], [fr(-1, 2), fr(1, 6)]]
    alpha = [fr(9, 10), fr(3, 4), fr(1, 2)]
    beta = [fr(1, 2), fr(1, 3), fr(3, 4)]
    h0 = [[fr(1, 5), fr(-1, 4)], [fr(1, 3), fr(1, 2)]]                         # dk x dv
    do = [[fr(1, 1), fr(-1, 2)], [fr(1, 3), fr(2, 3)], [fr(-1, 4), fr(1, 5)]]
    dhT = [[fr(1, 7), fr(0, 1)], [fr(-2, 3), fr(1, 9)]]
    scale = fr(1, 2)
    groups = {"q": q, "k": k, "v": v, "alpha": [[a] for a in alpha], "beta": [[b] for b in beta], "h0": h0}
    exact = {}
    for name, arr in groups.items():
        out = np.zeros((len(arr), len(arr[0])))
        for r in range(len(arr)):
            for c in range(len(arr[0])):
                D = {n: [[Dual(x) for x in row] for row in a] for n, a in groups.items()}
                D[name][r][c] = Dual(arr[r][c], 1)
                L = _exact_loss(D["q"], D["k"], D["v"], [x[0] for x in D["alpha"]], [x[0] for x in D["beta"]],
                                D["h0"], do, dhT, Dual(scale))
                out[r, c] = float(L.b)
        exact[name] = out
    f = lambda a: np.array([[float(x) for x in row] for row in a])  # noqa: E731
    qa, ka, va = f(q)[None, :, None, :], f(k)[None, :, None, :], f(v)[None, :, None, :]
    al = np.array([float(a) for a in alpha])
    g = np.log(al)[None, :, None]
    be = np.array([float(b) for b in beta])[None, :, None]
    doa = f(do)[None, :, None, :]
    dq, dk_, dv_, dg, db, dh0 = token_backward_numpy(qa, ka, va, g, be, doa, f(dhT)[None, None],
                                                     f(h0)[None, None], scale=float(scale))
    for name, got in [("q", dq[0, :, 0]), ("k", dk_[0, :, 0]), ("v", dv_[0, :, 0]),
                      ("beta", db[0, :, 0][:, None]), ("h0", dh0[0, 0])]:
        assert np.allclose(got, exact[name], rtol=1e-13, atol=1e-14), name
    # dL/dg = alpha dL/dalpha
    assert np.allclose(dg[0, :, 0], al * exact["alpha"][:, 0], rtol=1e-13, atol=1e-14)


def test_single_token_closed_forms():
    """T = 1, S1 = alpha S0 (I - beta k k^T) + beta v k^T, o = scale S1 q, L = <do, o>."""
    rng = np.random.default_rng(21)
    dk, dv, scale = 4, 3, 0.37
    q, k, v, do = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv), rng.standard_normal(dv)
    k /= np.linalg.norm(k)
    a, b = 0.8, 0.6
    h0 = rng.standard_normal((dk, dv))
    S0 = h0.T
    kq = k @ q
    S1 = a * S0 @ (np.eye(dk) - b * np.outer(k, k)) + b * np.outer(v, k)
    want = dict(
        q=scale * S1.T @ do,
        v=scale * b * kq * do,
        beta=scale * kq * do @ (v - a * S0 @ k),
        k=scale * b * ((v @ do - a * do @ S0 @ k) * q - a * kq * (S0.T @ do)),
        g=scale * a * do @ S0 @ (q - b * kq * k),
        h0=scale * a * np.outer(q - b * kq * k, do),
    )
    r = lambda x: x[None, None, None]  # noqa: E731
    dq, dk_, dv_, dg, db, dh0 = token_backward_numpy(r(q), r(k), r(v), np.log(a) * np.ones((1, 1, 1)),
                                                     b * np.ones((1, 1, 1)), r(do), None, h0[None, None],
                                                     scale=scale)
    got = dict(q=dq[0, 0, 0], k=dk_[0, 0, 0], v=dv_[0, 0, 0], beta=db[0, 0, 0], g=dg[0, 0, 0], h0=dh0[0, 0])
    for name in want:
        assert np.allclose(got[name], want[name], rtol=1e-12, atol=1e-13), name


@pytest.mark.parametrize("chunk,T,packed", [(4, 11, False), (4, 13, True), (64, 150, False), (64, 200, True)])
def test_chunked_backward_equals_token_backward(chunk, T, packed):
    H, dk, dv = 2, 8, 6
    if packed:
        cu = np.array([0, 1, T // 3, T // 3, T])        # a one-token and an empty sequence
        B, N = 1, 4
    else:
        cu, B, N = None, 2, 2
    c = _case(B, T, H, dk, dv, seed=31 + T)
    rng = np.random.default_rng(7)
    h0 = rng.standard_normal((N, H, dk, dv)) * 0.3
    dhT = rng.standard_normal((N, H, dk, dv))
    a = token_backward_numpy(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], dhT, h0, cu)
    b = chunked_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], dhT, h0, cu, chunk=chunk)
    for name, x, y in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], a, b):
        err = np.max(np.abs(x - y)) / max(1.0, np.max(np.abs(x)))
        assert err < 1e-11, (name, err)


def test_chunked_backward_strong_gates_and_no_initial_state():
    c = _case(1, 130, 1, 16, 16, seed=41, gate_lo=-3.0)
    a = token_backward_numpy(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"])
    b = chunked_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"])
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) / max(1.0, np.max(np.abs(x))) < 1e-11


def test_beta_zero_gives_no_value_or_key_gradient():
    c = _case(1, 70, 2, 8, 4, seed=51)
    c["beta"] = np.zeros_like(c["beta"])
    for fn in (token_backward_numpy, chunked_backward):
        dq, dk_, dv_, dg, db, dh0 = fn(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"],
                                       None, np.ones((1, 2, 8, 4)))
        assert np.all(dv_ == 0.0) and np.max(np.abs(dk_)) < 1e-14
        assert np.max(np.abs(dq)) > 0 and np.max(np.abs(db)) > 0
