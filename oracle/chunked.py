"""Oracle B: the chunk-by-chunk (WY) form of the GDN forward, in fp64, written
separately from Oracle A.  Test infrastructure only.

Source: FlashQLA talk transcript (tokendh.com, "Qwen系列模型线性注意力高性能优化实践").
  * chunked-WY section: the step size of the recurrence grows from one token to a
    chunk of C = 64 through the WY representation; four steps per chunk:
    (1) K K^T inside the chunk and its C x C inverse, (2) the projections W and U
    built with that inverse, (3) the chunk-to-chunk state recurrence, (4) the output
    from the state.  gamma is the running product of the gate alpha inside a chunk.
  * algebraic-rewrites section: Gamma, the C x C matrix of gamma ratios, is formed
    in log space, Gamma_rs = exp(G_r - G_s); Gamma can be pulled out of the inverse
    (invert the Gamma-free matrix, then multiply Gamma back in); the forward merges
    the common terms of W and U by forming "V minus S" first and then applying gamma.
  * sequence-parallel section: a segment run from a wrong (zero) start gives S*;
    the start error propagates through a dk x dk matrix per chunk, these matrices
    compose by associativity into one correction M per segment; a short recurrence
    over segments then yields every segment's true start, and S and O are recomputed.
  * sliding-window section: with alpha < 1 the influence of an old state decays
    geometrically, so a segment may start from zero a window of chunks earlier.

The formulas are not printed on the pages (lost in extraction).  Writing the
recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T with h = S^T
and unrolling it over the rows r = 1..n of one chunk gives, with G = cumsum(g),
gamma = exp(G), Gamma_rs = exp(G_r - G_s) for r >= s and 0 above the diagonal:

    A  = strict_lower(diag(beta) K K^T * Gamma),   T = (I + A)^{-1}          step 1
    W  = T diag(beta*gamma) K,   Ut = T diag(beta) V                         step 2
    U  = Ut - W h,   h' = gamma_n h + (diag(exp(G_n - G)) K)^T U             step 3
    O  = scale (diag(gamma) Q h + ((Q K^T) * Gamma) U)                       step 4

Everything here is plain numpy on fp64; the triangular inverse uses scipy's
triangular solve as a library step.
"""
import numpy as np
from scipy.linalg import solve_triangular

C_DEFAULT = 64


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gate_matrices(g):
    """Chunk-local cumulative log-gate G, gamma = exp(G) and the Gamma matrix.

    The upper triangle is masked before exponentiation (exp(G_r - G_s) for r < s
    can overflow), the diagonal is 1.
    """
    g = _f64(g)
    G = np.cumsum(g)
    n = len(g)
    lower = np.tril(np.ones((n, n), dtype=bool))
    diff = np.where(lower, G[:, None] - G[None, :], 0.0)
    Gamma = np.where(lower, np.exp(diff), 0.0)
    return G, np.exp(G), Gamma


def _unit_lower_inverse(A):
    n = A.shape[0]
    eye = np.eye(n)
    return solve_triangular(eye + A, eye, lower=True, unit_diagonal=True)


def chunk_inverse(k, g, beta, gamma_extracted=False):
    """Step 1 for one chunk: T = (I + strict_lower(diag(beta) K K^T * Gamma))^{-1}.

    With ``gamma_extracted`` the Gamma-free matrix is inverted and Gamma is
    multiplied back in afterwards (T = Gamma * T'), as the algebraic-rewrites
    section describes; both give the same T up to rounding.
    Returns ``(T, A)`` where A is the strictly-lower matrix that was inverted
    (with Gamma in the default form, without it in the extracted form).
    """
    k, g, beta = _f64(k), _f64(g), _f64(beta)
    _, _, Gamma = gate_matrices(g)
    KK = k @ k.T
    if gamma_extracted:
        A0 = np.tril(beta[:, None] * KK, -1)
        return Gamma * _unit_lower_inverse(A0), A0
    A = np.tril(beta[:, None] * KK * Gamma, -1)
    return _unit_lower_inverse(A), A


def chunk_step(h, q, k, v, g, beta, scale, variant="wy", want_o=True):
    """One chunk of the WY form: returns ``(o, h_next)`` (o is None if not wanted).

    variant "wy"        -- steps 1-4 as listed in the module docstring;
            "vprime"    -- the merged form U = T diag(beta) (V - diag(gamma) K h);
            "gamma_ex"  -- T built from the Gamma-free inverse, then steps 2-4.
    """
    k, v, g, beta = _f64(k), _f64(v), _f64(g), _f64(beta)
    G, gamma, Gamma = gate_matrices(g)
    T, _ = chunk_inverse(k, g, beta, gamma_extracted=(variant == "gamma_ex"))
    if variant == "vprime":
        Vp = v - gamma[:, None] * (k @ h)
        U = T @ (beta[:, None] * Vp)
    else:
        W = T @ ((beta * gamma)[:, None] * k)
        Ut = T @ (beta[:, None] * v)
        U = Ut - W @ h
    o = None
    if want_o:
        q = _f64(q)
        o = scale * (gamma[:, None] * (q @ h) + ((q @ k.T) * Gamma) @ U)
    h_next = gamma[-1] * h + (np.exp(G[-1] - G)[:, None] * k).T @ U
    return o, h_next


def _seq_offsets(B, T, cu_seqlens):
    if cu_seqlens is None:
        return np.arange(B + 1, dtype=np.int64) * T
    assert B == 1
    return np.asarray(cu_seqlens, dtype=np.int64)


def _chunks(length, C):
    return [(s, min(s + C, length)) for s in range(0, length, C)]


def _run(h, q, k, v, g, beta, chunks, scale, variant, o_out=None):
    """Runs consecutive chunks of one (sequence, head) from state h.
    ``q/k/v/g/beta`` are that pair's token-major slices; writes o into o_out."""
    for (a, b) in chunks:
        o, h = chunk_step(h, None if o_out is None else q[a:b], k[a:b], v[a:b], g[a:b],
                          beta[a:b], scale, variant=variant, want_o=o_out is not None)
        if o_out is not None:
            o_out[a:b] = o
    return h


def _prep(q, k, v, g, beta, cu_seqlens, scale):
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = _seq_offsets(B, T, cu_seqlens)
    if scale is None:
        scale = dk ** -0.5
    flat = (q.reshape(-1, H, dk), k.reshape(-1, H, dk), v.reshape(-1, H, dv),
            g.reshape(-1, H), beta.reshape(-1, H))
    return flat, cu, scale, (B, T, H, dk, dv)


def chunked_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, C=C_DEFAULT,
                    variant="wy"):
    """The whole forward in the chunked form (no sequence splitting).

    Same layouts and return values as ``oracle.token.token_recurrence``.
    """
    (qf, kf, vf, gf, bf), cu, scale, (B, T, H, dk, dv) = _prep(q, k, v, g, beta, cu_seqlens, scale)
    N = len(cu) - 1
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        for h in range(H):
            st = np.zeros((dk, dv)) if h0 is None else _f64(h0)[n, h].copy()
            oo = np.zeros((e - s, dv))
            st = _run(st, qf[s:e, h], kf[s:e, h], vf[s:e, h], gf[s:e, h], bf[s:e, h],
                      _chunks(e - s, C), scale, variant, o_out=oo)
            o[s:e, h] = oo
            hT[n, h] = st
    return o.reshape(B, T, H, dv), hT


def segment_transition(k, g, beta):
    """The explicit product over the tokens of a segment of alpha_t (I - beta_t k_t k_t^T),
    later tokens on the left: the map h_start -> h_end with V = 0.  (Used to pin M.)"""
    k, g, beta = _f64(k), _f64(g), _f64(beta)
    dk = k.shape[1]
    M = np.eye(dk)
    for t in range(k.shape[0]):
        M = np.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ M
    return M


def _segments(nch, L):
    return [(j, min(j + L, nch)) for j in range(0, nch, L)]


def cp_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, seg_chunks=4,
               C=C_DEFAULT, variant="wy"):
    """Sequence-parallel forward with the wrong-start correction.

    Each sequence's chunks are cut into segments of ``seg_chunks`` chunks.  For
    segment j: S*_j = the segment run from a zero state; M_j = the segment run with
    V = 0 from the identity (the composed dk x dk correction).  Then
    h_start(0) = h0, h_start(j+1) = M_j h_start(j) + S*_j, and every segment is
    re-run from its true start to produce O.

    Returns ``(o, hT, info)``; info[(n, h)] = dict(S_star=[...], M=[...], h_start=[...]).
    """
    (qf, kf, vf, gf, bf), cu, scale, (B, T, H, dk, dv) = _prep(q, k, v, g, beta, cu_seqlens, scale)
    N = len(cu) - 1
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    info = {}
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        ch = _chunks(e - s, C)
        for h in range(H):
            args = (qf[s:e, h], kf[s:e, h], vf[s:e, h], gf[s:e, h], bf[s:e, h])
            zeros_v = np.zeros_like(args[2][:, :1]).repeat(dk, axis=1)
            segs = _segments(len(ch), seg_chunks)
            S_star, M = [], []
            for (a, b) in segs:
                S_star.append(_run(np.zeros((dk, dv)), *args, ch[a:b], scale, variant))
                M.append(_run(np.eye(dk), args[0], args[1], zeros_v, args[3], args[4], ch[a:b],
                              scale, variant))
            starts = [np.zeros((dk, dv)) if h0 is None else _f64(h0)[n, h].copy()]
            for j in range(len(segs) - 1):
                starts.append(M[j] @ starts[j] + S_star[j])
            oo = np.zeros((e - s, dv))
            st = starts[0]
            for j, (a, b) in enumerate(segs):
                st = _run(starts[j].copy(), *args, ch[a:b], scale, variant, o_out=oo)
            o[s:e, h] = oo
            hT[n, h] = st if segs else starts[0]
            info[(n, h)] = dict(S_star=S_star, M=M, h_start=starts)
    return o.reshape(B, T, H, dv), hT, info


def window_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, seg_chunks=4,
                   window=2, C=C_DEFAULT, variant="wy"):
    """Sequence-parallel forward with window-lookback starts.

    Segment j (chunks [j*L, ...)) starts from a zero state ``window`` chunks before
    its first chunk and runs those chunks without output; when the window reaches
    the start of the sequence it starts from h0 (or zero) at chunk 0, which is
    exact.  Segment 0 starts from h0.  Returns ``(o, hT, starts)`` with starts[(n,h)]
    the list of segment start states used.
    """
    (qf, kf, vf, gf, bf), cu, scale, (B, T, H, dk, dv) = _prep(q, k, v, g, beta, cu_seqlens, scale)
    N = len(cu) - 1
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    starts_all = {}
    for n in range(N):
        s, e = cu[n], cu[n + 1]
        ch = _chunks(e - s, C)
        for h in range(H):
            args = (qf[s:e, h], kf[s:e, h], vf[s:e, h], gf[s:e, h], bf[s:e, h])
            init = np.zeros((dk, dv)) if h0 is None else _f64(h0)[n, h].copy()
            oo = np.zeros((e - s, dv))
            starts = []
            st = init
            for (a, b) in _segments(len(ch), seg_chunks):
                if a == 0:
                    start = init.copy()
                elif a - window <= 0:
                    start = _run(init.copy(), *args, ch[0:a], scale, variant)
                else:
                    start = _run(np.zeros((dk, dv)), *args, ch[a - window:a], scale, variant)
                starts.append(start)
                st = _run(start.copy(), *args, ch[a:b], scale, variant, o_out=oo)
            o[s:e, h] = oo
            hT[n, h] = st
            starts_all[(n, h)] = starts
    return o.reshape(B, T, H, dv), hT, starts_all
