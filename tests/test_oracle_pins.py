"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- exact rational arithmetic, closed forms that follow from the
recurrence, invariants, and a second, separately written algorithm (the chunked
WY form against the token recurrence).

The recurrence (FlashQLA talk transcript, tokendh.com: linear-attention, GDN and
sliding-window sections) is S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = scale S_t q_t, alpha = exp(g), state exchanged K-major (h = S^T).
"""
import math
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
from oracle import chunked, gate, token


def rand_inputs(rng, B, T, H, dk, dv, gate_kind="sigmoid", normalize=True, h0=False, N=None):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if normalize:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    if gate_kind == "sigmoid":
        g = -np.log1p(np.exp(-(rng.standard_normal((B, T, H)) + 3.0)))
    elif gate_kind == "strong":
        g = np.log(rng.uniform(0.8, 0.95, size=(B, T, H)))
    else:
        g = np.zeros((B, T, H))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    hh = rng.standard_normal((N or B, H, dk, dv)) * 0.1 if h0 else None
    return q, k, v, g, beta, hh


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- build check


def test_c_oracle_matches_numpy_twin():
    """Build check of the C library (same recurrence, written with the explicit
    alpha (I - beta k k^T) factor in numpy).  Not a pin by itself."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, h0 = rand_inputs(rng, 2, 37, 3, 8, 5, h0=True)
    o1, h1 = token.token_recurrence(q, k, v, g, beta, h0, scale=0.3)
    o2, h2 = token.token_recurrence_numpy(q, k, v, g, beta, h0, scale=0.3)
    assert rel(o1, o2) < 1e-13 and rel(h1, h2) < 1e-13


# ---------------------------------------------------------------- exact arithmetic


def _frac_matmul(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def test_exact_rational_brute_force():
    """Tiny case in exact rational arithmetic, with the factor I - beta k k^T formed
    explicitly.  All inputs are dyadic (exact in fp64); alpha = exp(log alpha) is the
    only rounding on the oracle side."""
    rng = np.random.default_rng(5)
    dk, dv, T = 3, 2, 6
    K = [[Fr(int(x), 8) for x in rng.integers(-8, 9, dk)] for _ in range(T)]
    Q = [[Fr(int(x), 8) for x in rng.integers(-8, 9, dk)] for _ in range(T)]
    V = [[Fr(int(x), 4) for x in rng.integers(-8, 9, dv)] for _ in range(T)]
    Bt = [Fr(int(x), 8) for x in rng.integers(1, 8, T)]
    Al = [Fr(int(x), 8) for x in rng.integers(5, 9, T)]
    H0 = [[Fr(int(x), 16) for x in rng.integers(-4, 5, dv)] for _ in range(dk)]  # [dk][dv]
    scale = Fr(1, 2)
    S = [[H0[i][j] for i in range(dk)] for j in range(dv)]  # S = h0^T, dv x dk
    o_exact = []
    for t in range(T):
        fac = [[(Fr(1) if i == j else Fr(0)) - Bt[t] * K[t][i] * K[t][j] for j in range(dk)]
               for i in range(dk)]
        S = _frac_matmul(S, fac)
        S = [[Al[t] * S[r][c] + Bt[t] * V[t][r] * K[t][c] for c in range(dk)] for r in range(dv)]
        o_exact.append([scale * sum(S[r][c] * Q[t][c] for c in range(dk)) for r in range(dv)])
    f = lambda M: np.array([[float(x) for x in row] for row in M])  # noqa: E731
    q = f(Q)[None, :, None, :]
    k = f(K)[None, :, None, :]
    v = f(V)[None, :, None, :]
    beta = np.array([float(b) for b in Bt])[None, :, None]
    g = np.log(np.array([float(a) for a in Al]))[None, :, None]
    h0 = f(H0)[None, None]
    o, hT = token.token_recurrence(q, k, v, g, beta, h0, scale=0.5)
    assert rel(o[0, :, 0], f(o_exact)) < 1e-13
    assert rel(hT[0, 0], f(S).T) < 1e-13


# ---------------------------------------------------------------- closed forms


def test_state_orientation_single_token():
    """k = e_3, beta = 1, g = 0, zero start: S = v e_3^T, so the K-major state has
    row 3 equal to v and every other row zero."""
    dk, dv = 8, 6
    rng = np.random.default_rng(0)
    k = np.zeros((1, 1, 1, dk)); k[..., 3] = 1.0
    q = rng.standard_normal((1, 1, 1, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    o, hT = token.token_recurrence(q, k, v, np.zeros((1, 1, 1)), np.ones((1, 1, 1)), scale=1.0)
    expect = np.zeros((dk, dv)); expect[3] = v[0, 0, 0]
    np.testing.assert_array_equal(hT[0, 0], expect)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0] * q[0, 0, 0, 3], rtol=0, atol=1e-15)


def test_beta_one_writes_value_exactly():
    """With beta_t = 1 and a unit key, S_t k_t = alpha S k - alpha S k (k.k) + v = v
    whatever alpha and the prior state are."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, h0 = rand_inputs(rng, 2, 150, 2, 16, 12, h0=True)
    beta[:, -1, :] = 1.0
    _, hT = token.token_recurrence(q, k, v, g, beta, h0)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(hT[b, h].T @ k[b, -1, h], v[b, -1, h], rtol=0, atol=1e-13)


def test_orthonormal_keys_closed_form():
    """Zero start and orthonormal keys k_1..k_n: S_{t-1} k_t = 0, so
    S_t = sum_{j<=t} beta_j (prod_{j<l<=t} alpha_l) v_j k_j^T; both the state and every
    output follow in closed form."""
    rng = np.random.default_rng(2)
    dk, dv, n = 32, 8, 20
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T
    k = keys[None, :, None, :]
    q = rng.standard_normal((1, n, 1, dk))
    v = rng.standard_normal((1, n, 1, dv))
    g = np.log(rng.uniform(0.5, 1.0, size=(1, n, 1)))
    beta = rng.uniform(0.05, 1.0, size=(1, n, 1))
    o, hT = token.token_recurrence(q, k, v, g, beta, scale=0.7)
    a = np.exp(g[0, :, 0])
    b = beta[0, :, 0]
    for j in range(n):
        want = b[j] * np.prod(a[j + 1:]) * v[0, j, 0]
        np.testing.assert_allclose(hT[0, 0].T @ keys[j], want, rtol=1e-12, atol=1e-14)
    for t in range(n):
        S = sum(b[j] * np.prod(a[j + 1:t + 1]) * np.outer(v[0, j, 0], keys[j]) for j in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], 0.7 * S @ q[0, t, 0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("impl", ["token", "chunked"])
def test_basis_keys_with_repeats(impl):
    """k_t = q_t = e_{t mod m}, beta = 1, g = 0, zero start: each step overwrites
    column (t mod m) of S with v_t, so o_t = scale v_t.  Repeats inside a chunk
    exercise the chunk inverse."""
    dk, dv, m, T = 16, 8, 5, 150
    rng = np.random.default_rng(3)
    k = np.zeros((1, T, 1, dk))
    for t in range(T):
        k[0, t, 0, t % m] = 1.0
    v = rng.standard_normal((1, T, 1, dv))
    args = (k.copy(), k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)))
    if impl == "token":
        o, _ = token.token_recurrence(*args, scale=0.25)
    else:
        o, _ = chunked.chunked_forward(*args, scale=0.25)
    np.testing.assert_allclose(o, 0.25 * v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("gated", [False, True])
def test_beta_zero_keeps_state(gated):
    """beta = 0: nothing is written, S_t = exp(G_t) S_0 and o_t = scale exp(G_t) S_0 q_t.
    With g = 0 the state stays at its initial value exactly."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 90, 2, 8, 8, h0=True)
    beta[:] = 0.0
    if not gated:
        g[:] = 0.0
    o, hT = token.token_recurrence(q, k, v, g, beta, h0, scale=0.5)
    G = np.cumsum(g[0], axis=0)  # [T, H]
    for h in range(2):
        if not gated:
            np.testing.assert_array_equal(hT[0, h], h0[0, h])
        else:
            np.testing.assert_allclose(hT[0, h], np.exp(G[-1, h]) * h0[0, h], rtol=1e-13)
        want = 0.5 * np.exp(G[:, h])[:, None] * (q[0, :, h] @ h0[0, h])
        np.testing.assert_allclose(o[0, :, h], want, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- invariants


def test_causality_bitwise():
    rng = np.random.default_rng(6)
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 120, 2, 8, 8, h0=True)
    o1, _ = token.token_recurrence(q, k, v, g, beta, h0)
    t0 = 77
    q2, k2, v2, b2 = q.copy(), k.copy(), v.copy(), beta.copy()
    q2[:, t0:] = rng.standard_normal(q2[:, t0:].shape)
    k2[:, t0:] = rng.standard_normal(k2[:, t0:].shape)
    v2[:, t0:] += 3.0
    b2[:, t0:] = 0.9
    o2, _ = token.token_recurrence(q2, k2, v2, g, b2, h0)
    np.testing.assert_array_equal(o1[:, :t0], o2[:, :t0])
    assert not np.array_equal(o1[:, t0:], o2[:, t0:])


@pytest.mark.parametrize("t1", [64, 100])
def test_state_carry(t1):
    rng = np.random.default_rng(7)
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 200, 2, 8, 6, h0=True)
    o, hT = token.token_recurrence(q, k, v, g, beta, h0)
    sl = lambda a, s: a[:, s]  # noqa: E731
    oa, ha = token.token_recurrence(*(sl(a, slice(0, t1)) for a in (q, k, v, g, beta)), h0)
    ob, hb = token.token_recurrence(*(sl(a, slice(t1, None)) for a in (q, k, v, g, beta)), ha)
    assert rel(np.concatenate([oa, ob], axis=1), o) < 1e-13
    assert rel(hb, hT) < 1e-13


def test_linearity():
    """Zero start: o and the state are linear in V; o is linear in q."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, 70, 1, 8, 4)
    v2 = rng.standard_normal(v.shape)
    q2 = rng.standard_normal(q.shape)
    oa, ha = token.token_recurrence(q, k, v, g, beta)
    ob, hb = token.token_recurrence(q, k, v2, g, beta)
    oc, hc = token.token_recurrence(q, k, 2.0 * v - 0.5 * v2, g, beta)
    assert rel(oc, 2.0 * oa - 0.5 * ob) < 1e-12 and rel(hc, 2.0 * ha - 0.5 * hb) < 1e-12
    od, _ = token.token_recurrence(q2, k, v, g, beta)
    oe, _ = token.token_recurrence(q + 3.0 * q2, k, v, g, beta)
    assert rel(oe, oa + 3.0 * od) < 1e-12


# ---------------------------------------------------------------- Oracle B vs Oracle A


@pytest.mark.parametrize("variant", ["wy", "vprime", "gamma_ex"])
@pytest.mark.parametrize("dk,dv,T,gk", [(16, 8, 200, "sigmoid"), (8, 16, 129, "strong"),
                                        (16, 16, 64, "zero"), (8, 8, 1, "sigmoid")])
def test_chunked_matches_token(variant, dk, dv, T, gk):
    rng = np.random.default_rng(9)
    q, k, v, g, beta, h0 = rand_inputs(rng, 2, T, 2, dk, dv, gate_kind=gk, h0=True)
    o1, h1 = token.token_recurrence(q, k, v, g, beta, h0, scale=0.4)
    o2, h2 = chunked.chunked_forward(q, k, v, g, beta, h0, scale=0.4, variant=variant)
    assert rel(o2, o1) < 1e-12 and rel(h2, h1) < 1e-12


def test_chunked_matches_token_packed():
    rng = np.random.default_rng(10)
    cu = np.array([0, 1, 65, 129, 130, 330])
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 330, 3, 8, 8, h0=True, N=5)
    o1, h1 = token.token_recurrence(q, k, v, g, beta, h0, cu_seqlens=cu)
    o2, h2 = chunked.chunked_forward(q, k, v, g, beta, h0, cu_seqlens=cu)
    assert rel(o2, o1) < 1e-12 and rel(h2, h1) < 1e-12


def test_chunk_inverse_properties():
    """T is unit lower triangular and inverts I + A; the Gamma-extracted inverse
    equals Gamma * T' = T."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, _ = rand_inputs(rng, 1, 64, 1, 32, 8, gate_kind="strong")
    kk, gg, bb = k[0, :, 0], g[0, :, 0], beta[0, :, 0]
    T, A = chunked.chunk_inverse(kk, gg, bb)
    assert np.allclose(np.diag(T), 1.0) and np.allclose(np.triu(T, 1), 0.0)
    assert np.linalg.norm((np.eye(64) + A) @ T - np.eye(64)) < 1e-12
    T2, _ = chunked.chunk_inverse(kk, gg, bb, gamma_extracted=True)
    assert rel(T2, T) < 1e-13
    # Gamma: entry (r, s) is the product of alpha over tokens s+1..r
    _, gam, Gam = chunked.gate_matrices(gg)
    a = np.exp(gg)
    assert abs(Gam[10, 3] - np.prod(a[4:11])) < 1e-14 and Gam[3, 10] == 0.0
    assert abs(gam[5] - np.prod(a[:6])) < 1e-14


# ---------------------------------------------------------------- sequence parallel


def test_cp_identity_and_explicit_M():
    """h_end = M h_start + S* per segment, M equals the explicit product of
    alpha_t (I - beta_t k_t k_t^T), and the corrected forward equals Oracle A."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 64 * 7 + 13, 2, 16, 8, h0=True)
    o1, h1 = token.token_recurrence(q, k, v, g, beta, h0)
    o2, h2, info = chunked.cp_forward(q, k, v, g, beta, h0, seg_chunks=3)
    assert rel(o2, o1) < 1e-12 and rel(h2, h1) < 1e-12
    for h in range(2):
        it = info[(0, h)]
        for j in range(len(it["M"])):
            a, b = j * 3 * 64, min((j + 1) * 3 * 64, k.shape[1])
            M_explicit = chunked.segment_transition(k[0, a:b, h], g[0, a:b, h], beta[0, a:b, h])
            assert rel(it["M"][j], M_explicit) < 1e-12
            if j + 1 < len(it["h_start"]):
                nxt = it["M"][j] @ it["h_start"][j] + it["S_star"][j]
                assert rel(it["h_start"][j + 1], nxt) < 1e-14


@pytest.mark.parametrize("seg", [1, 2, 5])
def test_cp_any_segment_count(seg):
    rng = np.random.default_rng(14)
    q, k, v, g, beta, h0 = rand_inputs(rng, 2, 64 * 5 + 1, 1, 8, 8, gate_kind="zero", h0=True)
    o1, h1 = token.token_recurrence(q, k, v, g, beta, h0)
    o2, h2, _ = chunked.cp_forward(q, k, v, g, beta, h0, seg_chunks=seg)
    assert rel(o2, o1) < 1e-12 and rel(h2, h1) < 1e-12


def test_window_error_bound_and_exact_limit():
    """A segment started from zero W chunks early differs from the true start by at
    most ||S_old|| exp(sum of g over the window) (unit keys, beta in [0,1]); a window
    that reaches the sequence start is exact."""
    rng = np.random.default_rng(15)
    T, L = 64 * 8, 2
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, T, 1, 16, 8, gate_kind="strong", h0=True)
    _, _, info = chunked.cp_forward(q, k, v, g, beta, h0, seg_chunks=L)
    true_starts = info[(0, 0)]["h_start"]
    W = 2
    _, _, wstarts = chunked.window_forward(q, k, v, g, beta, h0, seg_chunks=L, window=W)
    ws = wstarts[(0, 0)]
    # per-token state before each window, from a plain token run
    for j in range(1, len(ws)):
        c0 = j * L
        if c0 - W <= 0:
            assert rel(ws[j], true_starts[j]) < 1e-13
            continue
        t_old = (c0 - W) * 64
        _, h_old = token.token_recurrence(*(a[:, :t_old] for a in (q, k, v, g, beta)), h0)
        bound = np.linalg.norm(h_old[0, 0], 2) * np.exp(g[0, t_old:c0 * 64, 0].sum())
        assert np.linalg.norm(ws[j] - true_starts[j], 2) <= bound * (1 + 1e-9)
    o1, _ = token.token_recurrence(q, k, v, g, beta, h0)
    o3, _, _ = chunked.window_forward(q, k, v, g, beta, h0, seg_chunks=L, window=100)
    assert rel(o3, o1) < 1e-12


# ---------------------------------------------------------------- gate scan


def test_window_decision_hand_cases():
    """Constant g = c per token: every chunk sums to 64c; the smallest W with
    64cW <= log(2^-24) = -16.64 is the answer.  g = 0 never qualifies."""
    le = math.log(2.0 ** -24)
    assert gate.window_chunks(np.full(64 * 20, -0.05), log_eps=le) == 6   # 5*-3.2 = -16 > -16.64
    assert gate.window_chunks(np.full(64 * 20, -0.3), log_eps=le) == 1
    assert gate.window_chunks(np.zeros(64 * 20), log_eps=le) == 0
    # one weak chunk in the middle forces a longer window
    g = np.full(64 * 20, -0.3)
    g[64 * 7:64 * 8] = 0.0
    assert gate.window_chunks(g, log_eps=le) == 2
    # w_max caps the answer
    assert gate.window_chunks(np.full(64 * 40, -0.01), log_eps=le, w_max=16) == 0


def test_window_decision_all_packed_hand_case():
    """window_chunks_all on packed and dense [B, T, H] gates: per-(sequence, head)
    answers worked by hand from constant per-head gates, so a sequence boundary off
    by one token, a transposed head index or a partial last chunk summed as full
    changes an answer.  log(2^-24) = -16.64; a full chunk of g = c sums to 64c."""
    le = math.log(2.0 ** -24)
    lens = [64 * 20, 64 * 3 + 10, 64, 0, 70]
    H = 2
    per_seq = [(-0.05, -0.3), (-0.3, 0.0), (-0.3, -0.05), (-0.3, -0.3), (-0.3, -0.2)]
    g = np.concatenate([np.tile(np.array(c, dtype=float), (n, 1)) for n, c in zip(lens, per_seq)])
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = gate.window_chunks_all(g[None], cu_seqlens=cu, log_eps=le)
    expect = np.array([
        [6, 1],   # 20 chunks: -3.2 per chunk needs 6 (5 give -16.0); -19.2 needs 1
        [2, 0],   # 3 full chunks and one of 10 tokens (-3.0): W = 1 fails on it, W = 2 holds
        [1, 0],   # one chunk: -19.2 qualifies; -3.2 cannot (no run longer than 1 chunk)
        [0, 0],   # empty sequence: no window
        [2, 0],   # 64 + 6 tokens: last chunk -1.8 (head 0) / -1.2 (head 1); head 1's two
    ])            # chunks sum to -14.0 > -16.64
    assert got.tolist() == expect.tolist(), got
    # dense [B, T, H]: two rows of 64 * 4 tokens with swapped per-head gates
    gd = np.stack([np.tile([-0.3, -0.05], (256, 1)), np.tile([-0.05, -0.3], (256, 1))])
    assert gate.window_chunks_all(gd, log_eps=le).tolist() == [[1, 0], [0, 1]]


def _chunks(sums, H=1):
    """Gates [1, 64 * len(sums), H] whose chunk c sums to sums[c] (every token of a
    chunk equal), the same on every head unless sums is a list of per-head lists."""
    cols = sums if H > 1 else [sums]
    g = np.stack([np.repeat(np.asarray(c, dtype=float) / 64.0, 64) for c in cols], axis=-1)
    return g[None]


def test_segment_windows_hand_cases():
    """Per-segment windows worked by hand (log(2^-24) = -16.64): a segment start st
    takes the smallest W whose W chunks before st sum to <= log eps, or W = st (the
    window reaches the sequence start); a head with a start that has none takes the
    correction (all its entries 0)."""
    le = math.log(2.0 ** -24)
    # -3.2 per chunk: 6 chunks needed (5 give -16.0); starts 8, 16, 24, 32
    assert gate.segment_windows(_chunks([-3.2] * 40), 8, log_eps=le)[:, 0].tolist() == [0, 6, 6, 6, 6]
    # L = 4: the start at chunk 4 reaches the sequence start with W = 4 (exact)
    assert gate.segment_windows(_chunks([-3.2] * 16), 4, log_eps=le)[:, 0].tolist() == [0, 4, 6, 6]
    # no decay: starts at 8 and 16 reach the sequence start (W = st <= 16) ...
    assert gate.segment_windows(_chunks([0.0] * 24), 8, log_eps=le)[:, 0].tolist() == [0, 8, 16]
    # ... but a start at 24 cannot: the whole head takes the correction
    assert gate.segment_windows(_chunks([0.0] * 40), 8, log_eps=le)[:, 0].tolist() == [0, 0, 0, 0, 0]
    # a weak stretch (chunks 10..13 without decay) inside the second segment only
    # lengthens the window of the start right after it; the whole-sequence rule
    # (window_chunks) needs 8 for every start
    sums = [-5.0] * 32
    sums[10:14] = [0.0] * 4
    got = gate.segment_windows(_chunks(sums), 8, log_eps=le)[:, 0].tolist()
    assert got == [0, 4, 8, 4], got
    assert gate.window_chunks(np.repeat(np.asarray(sums) / 64.0, 64), log_eps=le) == 8
    # w_max caps the search
    assert gate.segment_windows(_chunks([-3.2] * 40), 8, log_eps=le, w_max=5)[:, 0].tolist() == [0, 0, 0, 0, 0]


def test_segment_windows_packed_numbering_and_heads():
    """Packed sequences (segments numbered over the sequences in order, empty and
    one-segment sequences keep one row) and two heads with different gates."""
    le = math.log(2.0 ** -24)
    lens = [64 * 20, 64 * 3, 0, 64 * 9 + 5]
    per_head = (-0.05, -0.3)   # per token: -3.2 / -19.2 per full chunk
    g = np.concatenate([np.tile(np.array(per_head), (n, 1)) for n in lens])[None]
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = gate.segment_windows(g, 8, cu_seqlens=cu, log_eps=le)
    expect = [
        [0, 0], [6, 1], [6, 1],   # 20 chunks: starts 8 and 16
        [0, 0],                    # 3 chunks: one segment
        [0, 0],                    # empty: one segment
        [0, 0], [6, 1],            # 10 chunks (the last partial): start 8
    ]
    assert got.tolist() == expect, got.tolist()


# ---------------------------------------------------------------- output magnitude


def test_output_magnitude_closed_forms():
    """m_t = scale |S_t| |q_t|: (a) one token from a zero state, S_1 = beta v k^T, so
    m[j] = scale beta |v_j| sum_i |k_i q_i| (signed k and q); (b) with nonnegative
    k, q, v on that token every term of the inner product is >= 0, so m == o;
    (c) beta = 0, g = 0 from h0: m = scale |h0|^T |q| per token."""
    rng = np.random.default_rng(21)
    dk, dv = 8, 5
    k = rng.standard_normal((1, 1, 1, dk))
    k /= np.linalg.norm(k)
    q = rng.standard_normal((1, 1, 1, dk))
    v = rng.standard_normal((1, 1, 1, dv))
    b = np.full((1, 1, 1), 0.7)
    z = np.zeros((1, 1, 1))
    m = token.output_magnitude_numpy(q, k, v, z, b, scale=0.5)
    expect = 0.5 * 0.7 * np.abs(v[0, 0, 0]) * np.sum(np.abs(k * q))
    assert np.allclose(m[0, 0, 0], expect, rtol=1e-14, atol=0)
    ka, qa, va = np.abs(k), np.abs(q), np.abs(v)
    o, _ = token.token_recurrence(qa, ka, va, z, b, None, scale=0.5)
    m = token.output_magnitude_numpy(qa, ka, va, z, b, scale=0.5)
    assert np.allclose(m, o, rtol=1e-14, atol=0)
    T = 6
    h0 = rng.standard_normal((1, 1, dk, dv))
    qs = rng.standard_normal((1, T, 1, dk))
    m = token.output_magnitude_numpy(qs, rng.standard_normal((1, T, 1, dk)),
                                     rng.standard_normal((1, T, 1, dv)), np.zeros((1, T, 1)),
                                     np.zeros((1, T, 1)), h0, scale=0.25)
    assert np.allclose(m[0, :, 0], 0.25 * np.abs(qs[0, :, 0]) @ np.abs(h0[0, 0]), rtol=1e-14, atol=0)


def test_output_magnitude_bounds_output():
    """|o_t| <= m_t elementwise (triangle inequality) on a random gated packed case,
    with equality nowhere forced; and m is invariant under q -> -q."""
    rng = np.random.default_rng(22)
    q, k, v, g, beta, h0 = rand_inputs(rng, 1, 90, 2, 8, 6, h0=True, N=3)
    cu = [0, 30, 31, 90]
    o, _ = token.token_recurrence(q, k, v, g, beta, h0, cu_seqlens=cu, scale=0.4)
    m = token.output_magnitude_numpy(q, k, v, g, beta, h0, cu_seqlens=cu, scale=0.4)
    assert np.all(np.abs(o) <= m * (1 + 1e-12) + 1e-300)
    m2 = token.output_magnitude_numpy(-q, k, v, g, beta, h0, cu_seqlens=cu, scale=0.4)
    assert np.array_equal(m, m2)


# ---------------------------------------------------------------- FLA interface convention


def test_layout_orientation_and_gate_convention_match_fla_reference():
    """The pages say the API follows FLA's chunk_gated_delta_rule.  An FLA-convention
    reference ships with transformers (Qwen3-Next's torch_recurrent_gated_delta_rule:
    inputs [B, T, H, D], g = log alpha per token, beta per token, state [B, H, dk, dv],
    scale dk^-1/2, fp32).  Oracle A on the same fp32-rounded inputs must agree with it
    to fp32 rounding: this pins the token-major layout, the K-major state orientation
    and the log-gate convention against an implementation written by others."""
    os.environ.setdefault("HF_HUB_OFFLINE", "1")
    torch = pytest.importorskip("torch")
    mod = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")
    ref = mod.torch_recurrent_gated_delta_rule
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 2, 45, 3, 16, 8
    q, k, v, g, beta, h0 = rand_inputs(rng, B, T, H, dk, dv, h0=True)
    q, k, v, g, beta, h0 = (a.astype(np.float32).astype(np.float64) for a in (q, k, v, g, beta, h0))
    tt = lambda a: torch.from_numpy(a).float()  # noqa: E731
    o_ref, s_ref = ref(tt(q), tt(k), tt(v), tt(g), tt(beta), tt(h0), True)
    o, hT = token.token_recurrence(q, k, v, g, beta, h0, scale=dk ** -0.5)
    assert o_ref.shape == o.shape and s_ref.shape == hT.shape
    assert rel(o, o_ref.double().numpy()) < 1e-5
    assert rel(hT, s_ref.double().numpy()) < 1e-5
    # and a transposed state would not agree (dk != dv makes the shapes differ; with
    # dk == dv the transposed final state is far off)
    q2, k2, v2, g2, b2, h2 = rand_inputs(rng, 1, 20, 1, 8, 8, h0=True)
    q2, k2, v2, g2, b2, h2 = (a.astype(np.float32).astype(np.float64) for a in (q2, k2, v2, g2, b2, h2))
    _, s2 = ref(tt(q2), tt(k2), tt(v2), tt(g2), tt(b2), tt(h2), True)
    _, hT2 = token.token_recurrence(q2, k2, v2, g2, b2, h2, scale=8 ** -0.5)
    assert rel(hT2, s2.double().numpy()) < 1e-5
    assert rel(np.swapaxes(hT2, -1, -2), s2.double().numpy()) > 1e-2


def _load_worked_example():
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example_dk2.txt")
    toks, final = [], None
    for line in open(path):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "token":
            toks.append([float(x) for x in f[1:]])
        elif f[0] == "final":
            final = np.array([float(x) for x in f[1:]]).reshape(2, 2)
    return np.array(toks), final


def test_golden_worked_example():
    """Both oracles reproduce the hand-worked 3-token example in tests/golden."""
    toks, final = _load_worked_example()
    T = len(toks)
    k = toks[:, 1:3].reshape(1, T, 1, 2)
    v = toks[:, 3:5].reshape(1, T, 1, 2)
    q = toks[:, 5:7].reshape(1, T, 1, 2)
    beta = toks[:, 7].reshape(1, T, 1)
    g = np.log(toks[:, 8]).reshape(1, T, 1)
    o_ref = toks[:, 9:11]
    for fn in (token.token_recurrence, token.token_recurrence_numpy):
        o, hT = fn(q, k, v, g, beta, None, scale=1.0)
        assert np.allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-12), o
        assert np.allclose(hT[0, 0], final, rtol=0, atol=1e-12), hT
    o, hT = chunked.chunked_forward(q, k, v, g, beta, None, scale=1.0)
    assert np.allclose(o[0, :, 0], o_ref, rtol=0, atol=1e-12)
    assert np.allclose(hT[0, 0], final, rtol=0, atol=1e-12)
