"""Oracle A: the GDN recurrence, one token at a time, in fp64.  Test infrastructure only.

Follows the FlashQLA talk transcript (tokendh.com, "Qwen系列模型线性注意力高性能优化实践"):
the linear-attention section (a d x d state updated token by token with the
outer product of k and v), the GDN section (update gate beta, forget gate
alpha) and the sliding-window section (the factor I - beta k k^T, alpha and
beta in (0,1), L2-normalised keys).  The formula itself is not printed on the
pages (their displayed equations were lost in extraction); the form used is

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = scale * S_t q_t,

S_t in R^{dv x dk}, alpha_t = exp(g_t) with g stored as log alpha (the
Gamma-in-log-space passage of the algebraic-rewrites section).  The state is
exchanged K-major, h = S^T with shape [dk, dv].

Inputs are numpy arrays.  Dense layout: q, k [B, T, H, dk]; v [B, T, H, dv];
g, beta [B, T, H]; h0 [B, H, dk, dv] or None.  Packed (varlen) layout: B == 1
and ``cu_seqlens`` (length N+1) gives the sequence boundaries; then h0 is
[N, H, dk, dv].  Outputs: o with the shape of v, and the final state
[N, H, dk, dv].  Everything is computed in fp64 from the exact fp64 upcast of
the stored inputs.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        lib.gdn_oracle_token.argtypes = [d, d, d, d, d, d, ctypes.POINTER(ctypes.c_int64),
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_double, d, d, ctypes.c_int]
        lib.gdn_oracle_token.restype = ctypes.c_int
        lib.gdn_oracle_max_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def max_threads() -> int:
    return int(_lib().gdn_oracle_max_threads())


def _as_f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _offsets(B, T, cu_seqlens):
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("bad cu_seqlens")
    return cu


def token_recurrence(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, nthreads=0):
    """Oracle A in plain C (OpenMP over (sequence, head, value-row block)).

    Returns ``(o, hT)`` as fp64 arrays.
    """
    q, k, v, g, beta = map(_as_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros(v.shape, dtype=np.float64)
    hT = np.zeros((N, H, dk, dv), dtype=np.float64)
    h0a = None if h0 is None else _as_f64(h0)
    if h0a is not None and h0a.shape != (N, H, dk, dv):
        raise ValueError("h0 shape %r != %r" % (h0a.shape, (N, H, dk, dv)))
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))  # noqa: E731
    rc = _lib().gdn_oracle_token(
        P(q), P(k), P(v), P(g), P(beta), None if h0a is None else P(h0a),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), N, H, dk, dv, float(scale),
        P(o), P(hT), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return o, hT


def token_recurrence_numpy(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
    """The same recurrence in numpy, written with the explicit factor
    alpha (I - beta k k^T); slow, for tiny inputs (checks the C build)."""
    q, k, v, g, beta = map(_as_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    qf, kf, vf = q.reshape(-1, H, dk), k.reshape(-1, H, dk), v.reshape(-1, H, dv)
    gf, bf = g.reshape(-1, H), beta.reshape(-1, H)
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    eye = np.eye(dk)
    for n in range(N):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else _as_f64(h0)[n, h].T.copy()
            for t in range(cu[n], cu[n + 1]):
                kt, vt = kf[t, h], vf[t, h]
                a, b = np.exp(gf[t, h]), bf[t, h]
                S = a * S @ (eye - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
                o[t, h] = scale * S @ qf[t, h]
            hT[n, h] = S.T
    return o.reshape(v.shape), hT


def output_magnitude_numpy(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
    """Magnitude of every output's defining sum, m_t = scale * |S_t| |q_t| (absolute
    values taken elementwise, S_t the post-update state of the same recurrence).

    Each output o_t[j] = scale * sum_i S_t[j, i] q_t[i] is an inner product; a floating
    point evaluation of it errs by at most a small multiple of the unit roundoff times
    scale * sum_i |S_t[j, i] q_t[i]| = m_t[j], whatever |o_t[j]| is.  m_t is therefore the
    scale against which an output's error is judged when the sum cancels (an
    ill-conditioned inner product).  Same layouts as token_recurrence_numpy; slow, for
    small inputs.  Returns m with the shape of v.
    """
    q, k, v, g, beta = map(_as_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    qf, kf, vf = q.reshape(-1, H, dk), k.reshape(-1, H, dk), v.reshape(-1, H, dv)
    gf, bf = g.reshape(-1, H), beta.reshape(-1, H)
    m = np.zeros((B * T, H, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else _as_f64(h0)[n, h].T.copy()
            for t in range(cu[n], cu[n + 1]):
                kt, vt = kf[t, h], vf[t, h]
                S = np.exp(gf[t, h]) * S
                S = S + bf[t, h] * np.outer(vt - S @ kt, kt)
                m[t, h] = abs(scale) * np.abs(S) @ np.abs(qf[t, h])
    return m.reshape(v.shape)
