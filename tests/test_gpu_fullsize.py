"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (default options: the planner's split, window and correction choices).

The fp64 oracle runs on every (sequence, head) pair of every workload (one oracle
call per sequence, parallel over its heads): 1 pair of the tiny workload, 64 of the
Qwen-like one, 256 of the packed one, 4 of the long one (including the ungated head
that takes the S*/M correction path) and 16 of the strongly gated one.  The whole
output is also checked to be finite.  Tolerance: relative L2 per (sequence, head),
1e-2 for bf16 storage, 1e-5 for fp32.
"""
import math
import time

import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from oracle import token
from tests.gpu_util import TOL, rel_l2, run_gpu, seq_bounds

pytestmark = pytest.mark.gpu

EXPECTED_PAIRS = {1: 1, 2: 64, 3: 256, 4: 4, 5: 16}


def oracle_heads(inp, n, heads):
    """fp64 oracle for sequence n and a list of heads (one call, parallel over heads)."""
    b, s, e = seq_bounds(inp)[n]
    idx = torch.tensor(heads)

    def sl(t):
        return synth.as_f64(t[b:b + 1, s:e].index_select(2, idx).contiguous())

    h0 = None
    if inp.get("h0") is not None:
        h0 = synth.as_f64(inp["h0"][n:n + 1].index_select(1, idx).contiguous())
    o, hT = token.token_recurrence(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                   sl(inp["beta"]), h0, scale=inp["scale"])
    return o[0], hT[0]


@pytest.mark.parametrize("w", [1, 2, 3, 4, 5])
def test_full_size_parity(w):
    t0 = time.time()
    spec = synth.WORKLOADS[w]
    print("workload %d %s: generating" % (w, spec.name), flush=True)
    inp = synth.generate(spec)
    seg = binding.plan_segment_chunks(inp["q"], inp["v"], inp["beta"], inp["cu_seqlens"])
    print("  planner segment chunks %d; running the HIP path" % seg, flush=True)
    o, hT = run_gpu(inp)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(hT).all())
    og = o.to("cpu").to(torch.float64).numpy()
    hg = hT.to("cpu").to(torch.float64).numpy()
    bounds = seq_bounds(inp)
    by_seq = {n: list(range(spec.H)) for n in range(len(bounds))}
    assert sum(len(v) for v in by_seq.values()) == EXPECTED_PAIRS[w]
    worst, checked = 0.0, 0
    for n, heads in by_seq.items():
        b, s, e = bounds[n]
        o_ref, h_ref = oracle_heads(inp, n, heads)
        for j, h in enumerate(heads):
            eo = rel_l2(og[b, s:e, h], o_ref[:, j])
            eh = rel_l2(hg[n, h], h_ref[j])
            if h < 2 or h == spec.H - 1:
                print("  seq %d head %2d (len %d): o %.3e state %.3e" % (n, h, e - s, eo, eh), flush=True)
            worst = max(worst, eo, eh)
            checked += 1
        del o_ref, h_ref
    tol = TOL[spec.dtype]
    print("  %d pairs checked, worst %.3e (tol %.0e), %.1f s" % (checked, worst, tol, time.time() - t0),
          flush=True)
    assert checked == EXPECTED_PAIRS[w]
    assert worst <= tol


def test_tensors_beyond_2pow31_elements():
    """Every input tensor holds more than 2^31 elements (T = 2^20 + 37 tokens, 16 heads,
    d = 128, bf16; a ragged last chunk), so any 32-bit element offset would wrap.  The
    inputs are drawn on the GPU from a seeded generator (q, k L2-normalised, v normal,
    g = log sigmoid(N(3, 1)) with the last head ungated, beta = sigmoid(N(0, 1))) and
    the oracle runs on the first and the last head; the last head sits at the largest
    offsets and takes the S*/M correction path."""
    T, H, D = (1 << 20) + 37, 16, 128
    assert T * H * D > 1 << 31
    t0 = time.time()
    gen = torch.Generator(device="cuda").manual_seed(31)

    def unit_rows():
        x = torch.randn((1, T, H, D), generator=gen, device="cuda")
        x /= x.norm(dim=-1, keepdim=True)
        return x.to(torch.bfloat16)

    q, k = unit_rows(), unit_rows()
    v = torch.randn((1, T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    x = torch.randn((1, T, H), generator=gen, device="cuda", dtype=torch.float64) + 3.0
    g = (-torch.log1p(torch.exp(-x))).to(torch.float32)
    g[:, :, H - 1] = 0.0
    beta = torch.sigmoid(torch.randn((1, T, H), generator=gen, device="cuda")).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(D)
    print("inputs ready (%.1f s); planner segment chunks %d" % (
        time.time() - t0, binding.plan_segment_chunks(q, v, beta)), flush=True)
    o, hT = binding.chunk_fwd(q, k, v, g, beta, None, scale=scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(hT).all())
    heads = torch.tensor([0, H - 1], device="cuda")
    pick = lambda t: synth.as_f64(t.index_select(2, heads).cpu())  # noqa: E731
    o_ref, h_ref = token.token_recurrence(pick(q), pick(k), pick(v), pick(g), pick(beta), None,
                                          scale=scale)
    og = o.index_select(2, heads).cpu().to(torch.float64).numpy()
    hg = hT.index_select(1, heads).cpu().to(torch.float64).numpy()
    worst = 0.0
    for j, h in enumerate([0, H - 1]):
        eo, eh = rel_l2(og[0, :, j], o_ref[0, :, j]), rel_l2(hg[0, j], h_ref[0, j])
        print("  head %2d: o %.3e state %.3e" % (h, eo, eh), flush=True)
        worst = max(worst, eo, eh)
    print("  worst %.3e, %.1f s" % (worst, time.time() - t0), flush=True)
    assert worst <= TOL["bf16"]
