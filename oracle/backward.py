"""Backward of the Gated DeltaNet recurrence in fp64: gradients of a loss
L = <dO, O> + <dhT, hT> with respect to q, k, v, g, beta and the initial state.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: FlashQLA talk transcript (tokendh.com, "Qwen系列模型线性注意力高性能优化实践").
  * results and timeline sections: the operator repository has a backward with the
    forward's structure (about 2x faster than the Triton baseline), including the
    window-based intra-GPU sequence parallelism;
  * algebraic-rewrites section: in the backward, the gradient of K K^T flows back
    to K as A-side and transposed terms; the two are merged (DA + DA^T) before the
    single product with K, which also helps the later gate and beta reductions.
The pages print no backward formulas.  Both forms below are derived here from the
forward recurrence (the spec form, h = S^T):

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = scale S_t q_t,
    alpha_t = exp(g_t).

token_backward_numpy: reverse-mode adjoint of that recurrence, token by token.
Writing D_t = alpha_t S_{t-1} and u_t = v_t - D_t k_t, the step is
S_t = D_t + beta_t u_t k_t^T.  With G the gradient of L with respect to S_t
(carried backwards, G <- G + scale do_t q_t^T at each token):

    dq_t = scale S_t^T do_t        w = G k_t            dv_t = beta_t w
    dbeta_t = u_t . w              dk_t = beta_t (G^T u_t - D_t^T w)
    dD = G - beta_t w k_t^T        dg_t = <dD, D_t>     G <- alpha_t dD

and dh0 = G^T after the first token.

chunked_backward: the same gradients chunk by chunk, differentiating the WY form
(chunked-WY section; Gamma in log space as in the algebraic-rewrites section),
with the forward quantities of a chunk recomputed from its start state h:

    A = strict_lower(diag(beta) K K^T * Gamma),  T = (I + A)^{-1}
    V' = V - diag(gamma) K h,  U = T diag(beta) V'
    O = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)
    h' = gamma_n h + (diag(d) K)^T U,   d = exp(G_n - G)

taken backwards step by step (see the function), the K K^T gradient entering K
once as (dB + dB^T) K (the merged form).
"""
import numpy as np

from .token import _as_f64, _offsets


def token_backward_numpy(q, k, v, g, beta, do, dhT=None, h0=None, cu_seqlens=None, scale=None):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) of L = <do, o> + <dhT, hT>, where (o, hT)
    is the forward of token_recurrence_numpy on the same arguments.

    Layouts as the forward: q, k [B, T, H, dk]; v, do [B, T, H, dv]; g, beta [B, T, H];
    h0, dhT [N, H, dk, dv] (K-major, h = S^T) or None (zero).  dh0 is returned even
    when h0 is None (the gradient with respect to a zero initial state).
    """
    q, k, v, g, beta, do = map(_as_f64, (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    qf, kf, vf, dof = (x.reshape(-1, H, x.shape[-1]) for x in (q, k, v, do))
    gf, bf = g.reshape(-1, H), beta.reshape(-1, H)
    dq, dkk = np.zeros_like(qf), np.zeros_like(kf)
    dvv = np.zeros_like(vf)
    dg, db = np.zeros_like(gf), np.zeros_like(bf)
    dh0 = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else _as_f64(h0)[n, h].T.copy()
            states, Ds, us = [], [], []
            for t in range(cu[n], cu[n + 1]):      # forward, keeping what the adjoint needs
                kt, vt = kf[t, h], vf[t, h]
                D = np.exp(gf[t, h]) * S
                u = vt - D @ kt
                S = D + bf[t, h] * np.outer(u, kt)
                states.append(S)
                Ds.append(D)
                us.append(u)
            G = np.zeros((dv, dk)) if dhT is None else _as_f64(dhT)[n, h].T.copy()
            for i, t in reversed(list(enumerate(range(cu[n], cu[n + 1])))):
                kt, qt, b, a = kf[t, h], qf[t, h], bf[t, h], np.exp(gf[t, h])
                G = G + scale * np.outer(dof[t, h], qt)
                dq[t, h] = scale * states[i].T @ dof[t, h]
                w = G @ kt
                dvv[t, h] = b * w
                db[t, h] = us[i] @ w
                dkk[t, h] = b * (G.T @ us[i] - Ds[i].T @ w)
                dD = G - b * np.outer(w, kt)
                dg[t, h] = np.sum(dD * Ds[i])
                G = a * dD
            dh0[n, h] = G.T
    return (dq.reshape(q.shape), dkk.reshape(k.shape), dvv.reshape(v.shape), dg.reshape(g.shape),
            db.reshape(beta.shape), dh0)


def _chunk_forward(Qc, Kc, Vc, gc, bc, h, scale):
    """One chunk of the WY forward from start state h (dk x dv), every intermediate
    kept for the backward."""
    n = len(gc)
    G = np.cumsum(gc)
    lower = np.tril(np.ones((n, n), dtype=bool))
    Gam = np.where(lower, np.exp(np.where(lower, G[:, None] - G[None, :], 0.0)), 0.0)
    gam, d, gam_n = np.exp(G), np.exp(G[-1] - G), np.exp(G[-1])
    strict = np.tril(np.ones((n, n), dtype=bool), -1)
    KKt = Kc @ Kc.T
    A = np.where(strict, bc[:, None] * KKt * Gam, 0.0)
    Tm = np.linalg.inv(np.eye(n) + A)
    Kh = Kc @ h
    Vp = Vc - gam[:, None] * Kh
    U = Tm @ (bc[:, None] * Vp)
    Qh = Qc @ h
    QKt = Qc @ Kc.T
    P = QKt * Gam
    O = scale * (gam[:, None] * Qh + P @ U)
    h_next = gam_n * h + (d[:, None] * Kc).T @ U
    return dict(G=G, Gam=Gam, gam=gam, d=d, gam_n=gam_n, strict=strict, lower=lower, KKt=KKt,
                A=A, T=Tm, Kh=Kh, Vp=Vp, U=U, Qh=Qh, QKt=QKt, P=P, O=O, h_next=h_next)


def _chunk_backward(Qc, Kc, Vc, gc, bc, h, f, dO, dh_next, scale):
    """Gradients of one chunk (dQ, dK, dV, dg, dbeta, dh) given the gradients dO and
    dh_next of its outputs; f holds the chunk's recomputed forward."""
    Gam, gam, d, gam_n = f["Gam"], f["gam"], f["d"], f["gam_n"]
    U, Vp, Kh, Qh = f["U"], f["Vp"], f["Kh"], f["Qh"]
    # h' = gamma_n h + (diag(d) K)^T U
    dh = gam_n * dh_next
    dgam_n = np.sum(h * dh_next)
    dKd = U @ dh_next.T
    dU = (d[:, None] * Kc) @ dh_next
    dd = np.sum(Kc * dKd, axis=1)
    dK = d[:, None] * dKd
    # O = scale (diag(gamma) Q h + P U),  P = (Q K^T) * Gamma  (lower, diagonal included)
    dY = scale * dO
    dQ = gam[:, None] * (dY @ h.T)
    dh = dh + Qc.T @ (gam[:, None] * dY)
    dgam = np.sum(Qh * dY, axis=1)
    dP = np.where(f["lower"], dY @ U.T, 0.0)
    dU = dU + f["P"].T @ dY
    dQ = dQ + (dP * Gam) @ Kc
    dK = dK + (dP * Gam).T @ Qc
    dGam = dP * f["QKt"]
    # U = T diag(beta) V'   ((I + A) U = diag(beta) V')
    dRHS = f["T"].T @ dU
    db = np.sum(dRHS * Vp, axis=1)
    dVp = bc[:, None] * dRHS
    dA = np.where(f["strict"], -dRHS @ U.T, 0.0)
    # V' = V - diag(gamma) K h
    dV = dVp
    dK = dK - gam[:, None] * (dVp @ h.T)
    dh = dh - Kc.T @ (gam[:, None] * dVp)
    dgam = dgam - np.sum(dVp * Kh, axis=1)
    # A = strict_lower(diag(beta) (K K^T) * Gamma): the K K^T gradient dB enters K once,
    # merged with its transpose (K K^T is symmetric)
    db = db + np.sum(dA * f["KKt"] * Gam, axis=1)
    dB = bc[:, None] * dA * Gam
    dK = dK + (dB + dB.T) @ Kc
    dGam = dGam + dA * bc[:, None] * f["KKt"]
    # Gamma_ij = exp(G_i - G_j), gamma = exp(G), d = exp(G_n - G), gamma_n = exp(G_n)
    E = dGam * Gam
    dG = np.sum(E, axis=1) - np.sum(E, axis=0)
    dG = dG + dgam * gam - dd * d
    dG[-1] += np.sum(dd * d) + dgam_n * gam_n
    # G = cumsum(g) inside the chunk
    dg = np.cumsum(dG[::-1])[::-1]
    return dQ, dK, dV, dg, db, dh


def chunked_backward(q, k, v, g, beta, do, dhT=None, h0=None, cu_seqlens=None, scale=None, chunk=64):
    """The gradients of token_backward_numpy, computed chunk by chunk through the WY
    form (see the module docstring).  Same arguments and results."""
    q, k, v, g, beta, do = map(_as_f64, (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _offsets(B, T, cu_seqlens)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    qf, kf, vf, dof = (x.reshape(-1, H, x.shape[-1]) for x in (q, k, v, do))
    gf, bf = g.reshape(-1, H), beta.reshape(-1, H)
    dq, dkk, dvv = np.zeros_like(qf), np.zeros_like(kf), np.zeros_like(vf)
    dg, db = np.zeros_like(gf), np.zeros_like(bf)
    dh0 = np.zeros((N, H, dk, dv))
    for n in range(N):
        starts = list(range(cu[n], cu[n + 1], chunk))
        for h in range(H):
            hs = np.zeros((dk, dv)) if h0 is None else _as_f64(h0)[n, h].copy()
            fwd = []
            for s in starts:                       # forward: every chunk's start state
                e = min(s + chunk, cu[n + 1])
                f = _chunk_forward(qf[s:e, h], kf[s:e, h], vf[s:e, h], gf[s:e, h], bf[s:e, h], hs, scale)
                fwd.append((s, e, hs, f))
                hs = f["h_next"]
            dh = np.zeros((dk, dv)) if dhT is None else _as_f64(dhT)[n, h].copy()
            for s, e, hstart, f in reversed(fwd):
                dQ, dK, dV, dgc, dbc, dh = _chunk_backward(qf[s:e, h], kf[s:e, h], vf[s:e, h], gf[s:e, h],
                                                           bf[s:e, h], hstart, f, dof[s:e, h], dh, scale)
                dq[s:e, h], dkk[s:e, h], dvv[s:e, h], dg[s:e, h], db[s:e, h] = dQ, dK, dV, dgc, dbc
            dh0[n, h] = dh
    return (dq.reshape(q.shape), dkk.reshape(k.shape), dvv.reshape(v.shape), dg.reshape(g.shape),
            db.reshape(beta.shape), dh0)
