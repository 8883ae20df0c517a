"""GPU parity of the one-pass forward (one_pass = 1: the chunk inverse and P are
formed inside the fused kernel, fused_wy.hip) against the fp64 oracle, per (sequence,
head) relative L2 on o and on the final state.  Covers ragged last chunks, every
dk / dv combination, packed input with empty and sub-chunk sequences, initial and
final states, fp32 beta with bf16 q/k/v, gates from none to strong, split plans whose
segments start from a lookback window or from corrected starts, the closed forms the
method has (basis keys with repeats, beta = 0 without decay), causality, and the
Qwen-like workload at full size."""
import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from tests.gpu_util import TOL, assert_parity, compare_pairs, run_gpu, to_dev
from tests.test_gpu_parity import _basis_inputs

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="wy", B=1, T=256, H=1, dk=128, dv=128, dtype="bf16", seed=0)
    base.update(kw)
    return synth.Spec(**base)


def wy_opts(**kw):
    return binding.make_opts(one_pass=1, **kw)


CASES = [
    ("d128_ragged_h0", dict(B=2, T=1000, H=3, h0_std=0.05, seed=41)),
    ("d64", dict(B=2, T=257, H=2, dk=64, dv=64, seed=42)),
    ("dk64_dv128", dict(B=1, T=190, H=2, dk=64, dv=128, seed=43)),
    ("dk128_dv64", dict(B=1, T=190, H=2, dk=128, dv=64, seed=44)),
    ("one_token", dict(B=3, T=1, H=2, seed=45)),
    ("sub_chunk", dict(B=2, T=63, H=2, h0_std=0.05, seed=46)),
    ("one_chunk", dict(B=2, T=64, H=2, seed=47)),
    ("strong_gate", dict(B=1, T=700, H=2, gate="uniform", seed=48)),
    ("no_decay", dict(B=1, T=700, H=2, gate="zero", seed=49)),
    ("beta_fp32", dict(B=2, T=300, H=2, beta_dtype="f32", seed=50)),
    ("many_heads", dict(B=1, T=200, H=9, dk=64, dv=128, seed=51)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_wy_parity_small(name, kw):
    print("one-pass case %s: %s" % (name, kw), flush=True)
    inp = synth.generate(spec(name=name, **kw))
    o, hT = run_gpu(inp, opts=wy_opts())
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "one-pass " + name)


def test_wy_no_final_state():
    inp = synth.generate(spec(B=2, T=300, H=2, seed=52))
    o, hT = run_gpu(inp, opts=wy_opts(), output_final_state=False)
    assert hT is None
    assert_parity(compare_pairs(inp, o, None), TOL["bf16"], "one-pass no final state")


def packed(lengths, H, dk, dv, h0_std, seed):
    inp = synth.generate(spec(B=1, T=int(sum(lengths)), H=H, dk=dk, dv=dv, seed=seed))
    inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    inp["N"] = len(lengths)
    if h0_std:
        g = torch.Generator().manual_seed(seed + 1)
        inp["h0"] = (torch.randn(len(lengths), H, dk, dv, generator=g) * h0_std).float()
    return inp


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_wy_packed_with_empty_and_tiny(dk, dv):
    lengths = [0, 1, 17, 64, 65, 0, 200, 640]
    print("one-pass packed %s dk %d dv %d" % (lengths, dk, dv), flush=True)
    inp = packed(lengths, 2, dk, dv, 0.05, 53)
    o, hT = run_gpu(inp, opts=wy_opts())
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "one-pass packed")


@pytest.mark.parametrize("force_correction", [0, 1])
@pytest.mark.parametrize("seg", [1, 3, 5])
def test_wy_split_segments(seg, force_correction):
    """Forced segment lengths: segments after the first start from a lookback window
    (gated heads) or from the merge's corrected starts (the ungated head, or every head
    under force_correction); the split passes are the two-pass path's, pass 3 is the
    one-pass kernel."""
    print("one-pass split seg %d force_correction %d" % (seg, force_correction), flush=True)
    inp = synth.generate(spec(B=2, T=900, H=3, zero_gate_heads=(2,), h0_std=0.05, seed=54))
    o, hT = run_gpu(inp, opts=wy_opts(force_segment_chunks=seg, force_correction=force_correction))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "one-pass split %d/%d" % (seg, force_correction))


def test_wy_split_packed():
    lengths = [300, 0, 1000, 64, 129]
    inp = packed(lengths, 2, 128, 128, 0.05, 55)
    print("one-pass split packed %s" % lengths, flush=True)
    o, hT = run_gpu(inp, opts=wy_opts(force_segment_chunks=4))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "one-pass split packed")


@pytest.mark.parametrize("m,dk,dv", [(5, 128, 128), (17, 64, 128), (63, 128, 64)])
def test_wy_basis_keys_closed_form(m, dk, dv):
    """k_t = q_t = e_(t mod m) (repeats inside every chunk exercise the inverse), beta = 1,
    g = 0, zero start, v integers of at most 8 bits over 16: the delta rule replaces
    column t mod m of S by v_t, so o_t = scale v_t and row j < m of the final state is
    the last v with key e_j.  Every intermediate (T in {-1, 0, 1}, V' and U differences
    of two such values) is exact in bf16, so the kernel must match to the bit."""
    T, H = 300, 2
    inp = _basis_inputs(T, H, dk, dv, m, seed=60 + m, dtype=torch.bfloat16)
    o, hT = run_gpu(inp, opts=wy_opts())
    want_h = torch.zeros(1, H, dk, dv)
    for j in range(m):
        last = max(t for t in range(T) if t % m == j)
        want_h[0, :, j, :] = inp["v"][0, last].float()
    assert torch.equal(o.cpu(), inp["v"] * 0.125)
    assert torch.equal(hT.cpu(), want_h)


def test_wy_beta_zero_no_decay_keeps_state_bitwise():
    inp = synth.generate(spec(B=2, T=200, H=2, gate="zero", h0_std=0.1, seed=57))
    inp["beta"] = torch.zeros_like(inp["beta"])
    _, hT = run_gpu(inp, opts=wy_opts())
    assert torch.equal(hT.cpu(), inp["h0"])


def test_wy_causality_bitwise():
    inp = synth.generate(spec(B=1, T=400, H=2, seed=58))
    o1, _ = run_gpu(inp, opts=wy_opts())
    t0 = 150
    for key in ("q", "k", "v"):
        inp[key] = inp[key].clone()
        inp[key][:, t0:] = torch.randn_like(inp[key][:, t0:].float()).to(inp[key].dtype)
    o2, _ = run_gpu(inp, opts=wy_opts())
    assert torch.equal(o1[:, :t0].cpu(), o2[:, :t0].cpu())


def test_wy_qwen_like_full_size_every_pair():
    sp = synth.WORKLOADS[2]
    print("one-pass %s" % sp.name, flush=True)
    inp = synth.generate(sp)
    o, hT = run_gpu(inp, opts=wy_opts())
    errs = compare_pairs(inp, o, hT)
    assert len(errs) == 64
    assert_parity(errs, TOL["bf16"], "one-pass " + sp.name)
