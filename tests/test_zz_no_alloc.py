"""gdn_chunk_fwd_noalloc (the allocation-free entry point) against gdn_chunk_fwd.

Both run the same plan and kernels; the only difference is where the scratch lives
(the library's built-in device array instead of a caller workspace), so the outputs
must be bitwise equal, and they must match the fp64 oracle within the bf16 bar.  Calls
in a row on the built-in array, each on a smaller input than the one before (the array
keeps the earlier calls' contents), each followed by the workspace call it is compared
with."""
import ctypes

import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from tests.gpu_util import TOL, assert_parity, compare_pairs, to_dev

pytestmark = pytest.mark.gpu


def run_both(inp, opts):
    d = to_dev(inp)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"])
    o_ref, h_ref = binding.chunk_fwd(*args, d["h0"], cu_seqlens=d["cu_seqlens"], scale=inp["scale"],
                                     opts=opts, cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    o = torch.full_like(o_ref, float("nan"))
    hT = torch.full_like(h_ref, float("nan"))
    binding.chunk_fwd_noalloc(*args, out=o, final_state_out=hT, initial_state=d["h0"],
                              cu_seqlens=d["cu_seqlens"], scale=inp["scale"], opts=opts,
                              cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    return o, hT, o_ref, h_ref


def test_noalloc_matches_workspace_call_in_a_row_each_smaller():
    big = synth.generate(synth.Spec("noalloc_big", B=2, T=1500, H=4, dk=128, dv=128, h0_std=0.05, seed=71))
    mid = synth.generate(synth.Spec("noalloc_mid", B=1, T=1200, H=3, dk=128, dv=128, zero_gate_heads=(1,),
                                    seed=73))
    small = synth.generate(synth.Spec("noalloc_small", B=1, T=300, H=2, dk=64, dv=128, seed=72))
    lens = [100, 0, 150, 50]
    small["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    small["N"] = len(lens)
    # first call: a split plan, every head corrected (segment maps, merge and starts
    # live in the scratch); second: smaller, split, one head without a window (the gate
    # scan's counters and pass 1's work list live there too); third: smaller, packed,
    # unsplit
    for inp, opts in ((big, binding.make_opts(force_segment_chunks=4, force_correction=1)),
                      (mid, binding.make_opts(force_segment_chunks=4)),
                      (small, binding.make_opts())):
        sp = inp["spec"]
        print("noalloc %s: B=%d T=%d H=%d dk=%d dv=%d" % (sp.name, sp.B, sp.T, sp.H, sp.dk, sp.dv), flush=True)
        o, hT, o_ref, h_ref = run_both(inp, opts)
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
        assert_parity(compare_pairs(inp, o, hT), TOL[sp.dtype], "noalloc " + sp.name)


def test_noalloc_rejects_problem_beyond_scratch():
    """A problem whose workspace exceeds the built-in array is rejected before anything
    is enqueued (no pointer is touched: all are null here)."""
    lib = binding.lib()
    s = binding.GdnShape(1, 1 << 22, 16, 128, 128, 1, binding.GDN_BF16, binding.GDN_BF16, None)
    need = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(s), None, ctypes.byref(need)) == 0
    assert need.value > binding.GDN_NOALLOC_SCRATCH_BYTES
    rc = lib.gdn_chunk_fwd_noalloc(None, None, None, None, None, None, None, ctypes.c_float(1.0), None,
                                   None, ctypes.byref(s), None, None)
    assert rc == binding.GDN_ERR_SCRATCH
