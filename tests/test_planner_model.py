"""The planner's per-kernel cost model (gdn_plan_predict_us, gdn_plan_segment_chunks),
on the host: the split decision's enable boundary over (B*H, T) has the shape the
model implies (splitting pays off for long sequences on few heads, never once one
unit per CU already fills the chip), the chosen length is the model's minimum, and
the modelled call is within 10% of the whole-call times measured on MI355X for the
five workloads (bench.py back-to-back calls, recorded with the plan's calibration)."""
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth

BHS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]
TS = [256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072]


def _meta(B, T, H, d=128, dtype=torch.bfloat16):
    q = torch.empty((B, T, H, d), dtype=dtype, device="meta")
    beta = torch.empty((B, T, H), dtype=dtype, device="meta")
    return q, beta


def _splits(bh, T, opts=None):
    H = min(bh, 16)
    q, beta = _meta(bh // H, T, H)
    return binding.plan_segment_chunks(q, q, beta, None, opts) < (T + 63) // 64


def test_enable_boundary_shape():
    grid = {(bh, T): _splits(bh, T) for bh in BHS for T in TS}
    for bh in BHS:          # once a sequence length splits, every longer one does
        row = [grid[(bh, T)] for T in TS]
        assert row == sorted(row), (bh, row)
    for T in TS:            # once a head count splits, every smaller one does
        col = [grid[(bh, T)] for bh in BHS]
        assert col == sorted(col, reverse=True), (T, col)
    assert not any(grid[(bh, T)] for bh in BHS for T in TS if bh >= 256)   # the chip is full
    assert not any(grid[(bh, T)] for bh in BHS for T in TS if T <= 512)    # too short to pay back
    assert grid[(1, 2048)] and grid[(64, 4096)] and grid[(128, 131072)]


def test_chosen_length_minimises_the_model():
    q, beta = _meta(4, 4096, 16)
    L = binding.plan_segment_chunks(q, q, beta)
    best = binding.plan_predict_us(q, q, beta)
    for cand in (8, 12, 16, 24, 32, 48, 64):
        o = binding.make_opts(force_segment_chunks=cand)
        assert binding.plan_predict_us(q, q, beta, None, o) >= best - 1e-9, cand
    assert L == 16


# Whole-call times measured on MI355X (bench.py, 10 back-to-back calls after a warm-up,
# default plan), and the share of (sequence, head) pairs without a lookback window
# (workload 4: head 3 has no decay).
MEASURED_US = {1: (44.7, 0.0), 2: (86.6, 0.0), 3: (323.5, 0.0), 4: (262.7, 0.25), 5: (287.7, 0.0)}


@pytest.mark.parametrize("w", sorted(MEASURED_US))
def test_model_predicts_the_measured_call_within_10_percent(w):
    sp = synth.WORKLOADS[w]
    dtype = torch.bfloat16 if sp.dtype == "bf16" else torch.float32
    q, beta = _meta(sp.B, sp.T, sp.H, sp.dk, dtype)
    cu = synth.generate(sp)["cu_seqlens"] if sp.packed else None
    meas, corr = MEASURED_US[w]
    pred = binding.plan_predict_us(q, q, beta, cu, None, corr)
    assert abs(pred / meas - 1.0) <= 0.10, (w, pred, meas)


def test_predict_rejects_bad_fraction():
    q, beta = _meta(1, 256, 1)
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(binding.GdnError):
            binding.plan_predict_us(q, q, beta, None, None, bad)


# Whole calls on a (B*H, T) grid (dense bf16, dk = dv = 128, H = min(B*H, 16), log gates
# log-sigmoid of N(3, 1) logits, so every head takes lookback windows: corrected
# fraction 0), measured on
# MI355X at the default plan (20 back-to-back calls, median of three runs).
GRID_MEASURED_US = {(1, 4, 2048): 46.1, (1, 4, 8192): 47.8, (1, 4, 32768): 54.7,
                    (1, 16, 2048): 48.1, (1, 16, 8192): 55.0, (1, 16, 32768): 155.5,
                    (4, 16, 2048): 56.4, (4, 16, 8192): 151.4, (4, 16, 32768): 504.7,
                    (16, 16, 2048): 134.8, (16, 16, 8192): 485.6, (16, 16, 32768): 1895.4}


@pytest.mark.parametrize("B,H,T", sorted(GRID_MEASURED_US))
def test_model_tracks_the_measured_grid(B, H, T):
    q, beta = _meta(B, T, H)
    pred = binding.plan_predict_us(q, q, beta)
    meas = GRID_MEASURED_US[(B, H, T)]
    assert abs(pred / meas - 1.0) <= 0.12, (B, H, T, pred, meas)
