"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (default options: the planner's split, window and correction choices).

The fp64 oracle runs on sampled (sequence, head) pairs — for the long workload every
head, including the ungated one that takes the S*/M correction path — and the
whole output is checked for properties that hold at any size (finite everywhere,
padded/untouched regions absent).  Tolerance: relative L2 per (sequence, head),
1e-2 for bf16 storage, 1e-5 for fp32.
"""
import time

import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from oracle import token
from tests.gpu_util import TOL, rel_l2, run_gpu, seq_bounds

pytestmark = pytest.mark.gpu

PAIRS = {
    1: [(0, 0)],
    2: [(0, 0), (1, 5), (2, 10), (3, 15)],
    3: [(n, (5 * n + 3) % 32) for n in range(8)],
    4: [(0, 0), (0, 1), (0, 2), (0, 3)],
    5: [(0, 0), (0, 7), (1, 3), (1, 6)],
}


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
    by_seq = {}
    for n, h in PAIRS[w]:
        by_seq.setdefault(n, []).append(h)
    worst = 0.0
    for n, heads in by_seq.items():
        b, s, e = bounds[n]
        o_ref, h_ref = oracle_heads(inp, n, heads)
        for j, h in enumerate(heads):
            eo = rel_l2(og[b, s:e, h], o_ref[:, j])
            eh = rel_l2(hg[n, h], h_ref[j])
            print("  seq %d head %2d (len %d): o %.3e state %.3e" % (n, h, e - s, eo, eh), flush=True)
            worst = max(worst, eo, eh)
    tol = TOL[spec.dtype]
    print("  worst %.3e (tol %.0e), %.1f s" % (worst, tol, time.time() - t0), flush=True)
    assert worst <= tol
