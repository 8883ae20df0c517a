"""Seeded random sweep of the forward's configuration space against the fp64 oracle.

Each case draws, from its own seed: dense or packed input (packed lengths include
empty and sub-chunk sequences), dk and dv in {64, 128}, bf16 or fp32 storage (bf16 or
fp32 beta), a gate distribution per head (sigmoid gates, strong uniform gates or none
at all), an initial state or none, whether the final state is requested, and the
options (planner or a forced segment length, forced correction, the window cap,
64-column value blocks, no split).  Every (sequence, head) pair is compared with the
oracle: relative L2 per pair within 1e-2 (bf16 storage) or 1e-5 (fp32).  The inputs
come from the seeded generators in synth; nothing here is shared with the HIP path
but those inputs.

A second draw (draw_large_case) takes longer dense and packed inputs with the
planner's own split choices (no forced segment length), so the planner's decisions
are checked at realistic sizes.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from tests.gpu_util import TOL, assert_parity, compare_pairs, compare_pairs_magnitude, run_gpu

pytestmark = pytest.mark.gpu

CASES = 24


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    rng.random()
    dtype = "f32" if seed % 3 == 0 else "bf16"   # a third of the cases in fp32
    beta_dtype = dtype if rng.random() < 0.8 else ("f32" if dtype == "bf16" else "bf16")
    dk, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    H = int(rng.integers(1, 5))
    packed = rng.random() < 0.5
    if packed:
        n = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.choice([0, 1, 17, 63, 64, 65, 200, 640, 1100, 1600], size=n)]
        if sum(lens) == 0:
            lens[0] = 129
        B, T = 1, sum(lens)
    else:
        B, T = int(rng.integers(1, 4)), int(rng.choice([1, 65, 300, 777, 1300, 2100]))
        lens = None
    gate = str(rng.choice(["sigmoid", "uniform", "zero"], p=[0.5, 0.3, 0.2]))
    zero_heads = tuple(int(h) for h in range(H) if rng.random() < 0.3)
    h0_std = float(rng.choice([0.0, 0.05])) or None
    spec = synth.Spec("random%d" % seed, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, beta_dtype=beta_dtype,
                      gate=gate, zero_gate_heads=zero_heads, h0_std=None if packed else h0_std,
                      seed=2000 + seed)
    inp = synth.generate(spec)
    if packed:
        inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        inp["N"] = len(lens)
        if h0_std:
            g = torch.Generator().manual_seed(3000 + seed)
            inp["h0"] = (torch.randn(len(lens), H, dk, dv, generator=g) * h0_std).float()
    opts = dict(
        no_split=int(rng.random() < 0.1),
        force_segment_chunks=int(rng.choice([0, 1, 1, 2, 2, 3, 5])),
        force_correction=int(rng.random() < 0.3),
        window_max_chunks=int(rng.choice([0, 1, 4, 16])),
        value_block=int(rng.choice([0, 0, 64])),
        one_pass=int(rng.choice([0, 0, 1, -1])),
    )
    if seed % 4 == 3:   # one-chunk segments: long merge chains (the two-level tree)
        opts.update(no_split=0, force_segment_chunks=1)
    final = bool(rng.random() < 0.8)
    return inp, opts, final


@pytest.mark.parametrize("seed", range(CASES))
def test_random_configuration(seed):
    inp, kw, final = draw_case(seed)
    sp = inp["spec"]
    label = "case %d: B=%d T=%d H=%d dk=%d dv=%d %s beta %s gate %s zero %s packed %s h0 %s final %s opts %s" % (
        seed, sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.dtype, sp.beta_dtype, sp.gate, sp.zero_gate_heads,
        None if inp["cu_seqlens"] is None else inp["cu_seqlens"].tolist(), inp["h0"] is not None, final, kw)
    print(label, flush=True)
    o, hT = run_gpu(inp, opts=binding.make_opts(**kw), output_final_state=final)
    assert (hT is None) == (not final)
    errs = compare_pairs(inp, o, hT)
    assert_parity(errs, TOL[sp.dtype], label)


LARGE_CASES = 6


def draw_large_case(seed):
    rng = np.random.default_rng(90000 + seed)
    H = int(rng.integers(1, 9))
    dk, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
    packed = rng.random() < 0.5
    if packed:
        lens = [int(x) for x in rng.integers(0, 6000, size=int(rng.integers(1, 13)))]
        if sum(lens) == 0:
            lens[0] = 300
        B, T = 1, sum(lens)
    else:
        B, T = int(rng.integers(1, 3)), int(rng.integers(1000, 20000))
    gate = str(rng.choice(["sigmoid", "uniform", "zero"], p=[0.5, 0.3, 0.2]))
    zero_heads = tuple(int(h) for h in range(H) if rng.random() < 0.3)
    dtype = "bf16" if rng.random() < 0.8 else "f32"
    spec = synth.Spec("large%d" % seed, B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, gate=gate,
                      zero_gate_heads=zero_heads, h0_std=None if packed else 0.05, seed=95000 + seed)
    inp = synth.generate(spec)
    if packed:
        inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        inp["N"] = len(lens)
    opts = dict(force_correction=int(rng.random() < 0.2), window_max_chunks=int(rng.choice([0, 0, 4, 16])))
    return inp, opts


@pytest.mark.parametrize("seed", range(LARGE_CASES))
def test_random_large_configuration(seed):
    inp, kw = draw_large_case(seed)
    sp = inp["spec"]
    label = "large case %d: B=%d T=%d H=%d dk=%d dv=%d %s gate %s zero %s packed %s opts %s" % (
        seed, sp.B, sp.T, sp.H, sp.dk, sp.dv, sp.dtype, sp.gate, sp.zero_gate_heads,
        None if inp["cu_seqlens"] is None else inp["cu_seqlens"].tolist(), kw)
    print(label, flush=True)
    o, hT = run_gpu(inp, opts=binding.make_opts(**kw), output_final_state=True)
    assert_parity(compare_pairs(inp, o, hT), TOL[sp.dtype], label)


def test_fp32_ill_conditioned_single_token_case():
    """Seed 3609 of the sweep's draw: B = 3, T = 1, dk = 128, dv = 64, fp32.  Each
    output is one fp32 inner product o = scale beta (k . q) v whose terms cancel (for
    one pair sum |k_i q_i| / |k . q| is several hundred), so its relative L2 error says
    nothing about the kernel: no fp32 evaluation order of such a sum meets 1e-5
    relative.  The output is judged instead against the magnitude of its inner product
    (tests.gpu_util.compare_pairs_magnitude: ||o - o_ref|| / ||scale |S||q| || <= 1e-5);
    the final state, a plain product beta v k^T, keeps the 1e-5 relative bar."""
    inp, kw, _ = draw_case(3609)
    sp = inp["spec"]
    assert (sp.dtype, sp.B, sp.T, sp.dk, sp.dv) == ("f32", 3, 1, 128, 64)
    print("case 3609: B=%d T=%d H=%d dk=%d dv=%d %s opts %s" % (sp.B, sp.T, sp.H, sp.dk, sp.dv,
                                                                  sp.dtype, kw), flush=True)
    o, hT = run_gpu(inp, opts=binding.make_opts(**kw), output_final_state=True)
    errs = compare_pairs_magnitude(inp, o)
    # the case is the ill-conditioned one: some pair's |o| is far below its magnitude
    assert min(e[3] for e in errs) < 0.05, errs
    worst = max(e[2] for e in errs)
    print("  worst magnitude-relative error %.3e over %d pairs" % (worst, len(errs)), flush=True)
    assert worst <= TOL["f32"], errs
    assert max(e[3] for e in compare_pairs(inp, o, hT)) <= TOL["f32"]
