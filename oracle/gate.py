"""Brute-force window-length decision for strongly decaying heads.  Test infrastructure only.

Source: FlashQLA talk transcript (tokendh.com), sliding-window section: because
alpha < 1 and ||I - beta k k^T|| <= 1 for L2-normalised k and beta in [0, 1], a
state's influence on later states shrinks by alpha at every token, so whenever a
head's alpha is not identically 1 a finite window exists beyond which old state
no longer matters; a light kernel scans each head's gates to decide which heads
get window-lookback starts.  The pages give no numbers for the window.

Reading taken (stated in the design notes): the error of starting a segment from
zero W chunks early is at most ||S_old|| * exp(sum of g over those W chunks).  A
(sequence, head) gets the smallest W in 1..w_max such that every run of W
consecutive chunks of that sequence has a gate sum <= log_eps; 0 means "not
eligible" (use the wrong-start correction instead).  Partial last chunks sum
their real tokens only.

Per-segment reading (segment_windows): the same bound only involves the W chunks
right before the start being approximated, so a segment starting at chunk st of
its sequence takes the smallest W in 1..min(w_max, st) whose W chunks before st sum
to <= log_eps, or W = st (the window reaches the sequence start, where the state is
known exactly); a (sequence, head) takes the correction if any of its segment
starts has no such W.
"""
import math

import numpy as np

LOG_EPS_DEFAULT = math.log(2.0 ** -24)
W_MAX_DEFAULT = 16


def chunk_sums(g, C=64):
    g = np.asarray(g, dtype=np.float64)
    return np.array([g[s:s + C].sum() for s in range(0, len(g), C)])


def max_window_sum(sums, W):
    """Largest sum over runs of W consecutive chunks (-inf... never: needs W <= len)."""
    return max(sums[c:c + W].sum() for c in range(0, len(sums) - W + 1))


def window_chunks(g, C=64, log_eps=LOG_EPS_DEFAULT, w_max=W_MAX_DEFAULT):
    """Smallest admissible window (in chunks) for one (sequence, head), or 0."""
    sums = chunk_sums(g, C)
    for W in range(1, min(w_max, len(sums)) + 1):
        if max_window_sum(sums, W) <= log_eps:
            return W
    return 0


def window_chunks_all(g, cu_seqlens=None, C=64, log_eps=LOG_EPS_DEFAULT, w_max=W_MAX_DEFAULT):
    """``g`` is [B, T, H]; returns int array [N, H]."""
    g = np.asarray(g, dtype=np.float64)
    B, T, H = g.shape
    if cu_seqlens is None:
        cu = np.arange(B + 1) * T
    else:
        cu = np.asarray(cu_seqlens)
    gf = g.reshape(-1, H)
    N = len(cu) - 1
    out = np.zeros((N, H), dtype=np.int64)
    for n in range(N):
        for h in range(H):
            out[n, h] = window_chunks(gf[cu[n]:cu[n + 1], h], C, log_eps, w_max)
    return out


def segment_windows(g, seg_chunks, cu_seqlens=None, C=64, log_eps=LOG_EPS_DEFAULT, w_max=W_MAX_DEFAULT):
    """``g`` is [B, T, H], the sequences cut into segments of ``seg_chunks`` chunks.
    Returns int array [total_segments, H] (segments numbered over the sequences in
    order): the lookback window of every segment start after a sequence's first, 0
    for first segments and for every segment of a (sequence, head) that has a
    segment start without a window (those take the correction)."""
    g = np.asarray(g, dtype=np.float64)
    B, T, H = g.shape
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens)
    gf = g.reshape(-1, H)
    rows = []
    for n in range(len(cu) - 1):
        nch = (cu[n + 1] - cu[n] + C - 1) // C
        segs = max(1, (nch + seg_chunks - 1) // seg_chunks)
        w = np.zeros((segs, H), dtype=np.int64)
        for h in range(H):
            sums = chunk_sums(gf[cu[n]:cu[n + 1], h], C)
            for j in range(1, segs):
                st = j * seg_chunks
                for W in range(1, min(w_max, st) + 1):
                    if W == st or sums[st - W:st].sum() <= log_eps:
                        w[j, h] = W
                        break
            if (w[1:, h] == 0).any():
                w[:, h] = 0
        rows.append(w)
    return np.concatenate(rows, axis=0)
