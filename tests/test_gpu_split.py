"""GPU parity of the sequence-split paths (gate scan, wrong-start correction with
merge, window-lookback starts) against the fp64 token-recurrence oracle, and
stage parity of the gate scan against its brute-force reference."""
import math

import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from oracle import gate
from tests.gpu_util import TOL, assert_parity, compare_pairs, rel_l2, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="split", B=1, T=64 * 14 + 23, H=3, dk=128, dv=128, dtype="bf16", seed=0,
                zero_gate_heads=(1,))
    base.update(kw)
    return synth.Spec(**base)


@pytest.mark.parametrize("seg", [1, 2, 3, 7])
@pytest.mark.parametrize("corr", [0, 1])
def test_split_parity_forced_segments(seg, corr):
    """Head 1 has g = 0 (correction path); heads 0 and 2 decay (window path unless
    the correction is forced).  Any segment count must give the unsplit result."""
    inp = synth.generate(spec(seed=60 + seg, h0_std=0.05))
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=seg, force_correction=corr))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "seg=%d corr=%d" % (seg, corr))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_parity_small_heads(dtype):
    inp = synth.generate(spec(B=2, T=64 * 9 + 5, H=2, dk=64, dv=64, dtype=dtype, seed=71,
                              zero_gate_heads=(0,), h0_std=0.1))
    for corr in (0, 1):
        o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=2, force_correction=corr))
        assert_parity(compare_pairs(inp, o, hT), TOL[dtype], "%s corr=%d" % (dtype, corr))


def _packed(lengths, H, seed, dk=128, dv=128, zero_heads=(1,)):
    T = int(sum(lengths))
    inp = synth.generate(spec(B=1, T=T, H=H, dk=dk, dv=dv, seed=seed, zero_gate_heads=zero_heads))
    inp["cu_seqlens"] = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    inp["N"] = len(lengths)
    g = torch.Generator().manual_seed(seed)
    inp["h0"] = (torch.randn(len(lengths), H, dk, dv, generator=g) * 0.03).float()
    return inp


@pytest.mark.parametrize("corr", [0, 1])
def test_split_parity_packed(corr):
    inp = _packed([64 * 9 + 7, 40, 0, 64 * 3, 64 * 6 + 1, 0], H=2, seed=72)
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=2, force_correction=corr))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "packed corr=%d" % corr)



@pytest.mark.parametrize("seg", [2, 3, 8])
@pytest.mark.parametrize("corr", [0, 1])
def test_packed_forced_segment_length_that_splits_nothing(seg, corr):
    """Packed sequences of at most 2 chunks over a packed T of 5 chunks, with a forced
    segment length >= 2: no sequence splits, and every sequence is one segment that
    starts from its own initial state (regression: the plan once kept the forced
    length, and the output kernel then read 3 segments of one sequence)."""
    inp = _packed([65, 63, 64, 1, 1, 64], H=2, seed=397)
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=seg, force_correction=corr))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "packed unsplit seg=%d corr=%d" % (seg, corr))

@pytest.mark.parametrize("seg", [1, 2])
def test_split_tree_merge(seg):
    """Merge chains longer than 72 steps run as a two-level tree (group maps
    composed in parallel, a chain over groups, then each group's own steps): 100
    steps for seg=1 (groups of 10); seg=2 gives a 50-step serial chain."""
    inp = synth.generate(spec(B=1, T=64 * 100 + 9, H=2, seed=75 + seg, zero_gate_heads=(0,),
                              h0_std=0.05))
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=seg, force_correction=1))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "tree merge seg=%d" % seg)


def test_split_tree_merge_packed():
    """Tree merge with sequences of different step counts (79, 16, 2, 0 steps, and
    an empty sequence): every sequence uses the same group length (9)."""
    inp = _packed([64 * 80, 64 * 17 - 5, 64 * 3, 0, 50], H=2, seed=78, zero_heads=(0, 1))
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=1))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "tree merge packed")


@pytest.mark.parametrize("N", [300, 1030])
def test_split_many_sequences(N):
    """Many short packed sequences (0 to 4 chunks, empty ones included), split into
    one-chunk segments: 300 sequences take the longest-first segment order table,
    1030 exceed its size limit and keep sequence order.  Both must give the unsplit
    result."""
    rng = np.random.default_rng(90 + N)
    lengths = rng.integers(0, 64 * 4 + 1, size=N)
    lengths[rng.integers(0, N, size=N // 10)] = 0
    inp = _packed(list(lengths), H=2, seed=91 + N, dk=64, dv=64, zero_heads=(0,))
    o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=1))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "N=%d" % N)


def test_split_value_block_64_and_dk64_dv128():
    inp = synth.generate(spec(B=1, T=64 * 8, H=2, dk=64, dv=128, seed=73, zero_gate_heads=(0,)))
    for vb in (64, 128):
        o, hT = run_gpu(inp, opts=binding.make_opts(force_segment_chunks=3, value_block=vb))
        assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "dk64 dv128 vb=%d" % vb)


def test_planner_default_split_parity():
    """A shape the planner splits by default (few heads, long sequence)."""
    inp = synth.generate(spec(B=1, T=64 * 48, H=2, seed=74, zero_gate_heads=(1,)))
    d = to_dev(inp)
    L = binding.plan_segment_chunks(d["q"], d["v"], d["beta"])
    assert L < 48, L
    o, hT = run_gpu(inp)
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "planner L=%d" % L)


@pytest.mark.parametrize("eps_bits", [24, 16])
@pytest.mark.parametrize("kind", ["sigmoid", "uniform", "mixed", "packed"])
def test_gate_scan_stage(kind, eps_bits):
    """GPU window decision vs the fp64 brute force: the GPU's W must be admissible in
    fp64 (every W-run sums to <= log eps) and minimal up to the 1e-3 margin band."""
    if kind == "packed":
        inp = _packed([64 * 30 + 5, 64 * 3, 17, 64 * 12], H=3, seed=81, zero_heads=(2,))
    else:
        gk = {"sigmoid": "sigmoid", "uniform": "uniform", "mixed": "sigmoid"}[kind]
        inp = synth.generate(spec(B=2, T=64 * 40 + 9, H=4, gate=gk, seed=82,
                                  zero_gate_heads=(3,) if kind == "mixed" else ()))
    d = to_dev(inp)
    le = math.log(2.0 ** -eps_bits)
    win = binding.gate_scan(d["g"], d["cu_seqlens"], inp.get("cu_seqlens"),
                            opts=binding.make_opts(window_log_eps=le)).cpu().numpy()
    if eps_bits == 16:   # the default for bf16 q/k/v
        win_default = binding.gate_scan(d["g"], d["cu_seqlens"], inp.get("cu_seqlens")).cpu().numpy()
        assert (win_default == win).all()
    g64 = synth.as_f64(inp["g"])
    B, T, H = g64.shape
    cu = (inp["cu_seqlens"].numpy() if inp.get("cu_seqlens") is not None
          else np.arange(B + 1) * T)
    gf = g64.reshape(-1, H)
    checked = 0
    for n in range(len(cu) - 1):
        for h in range(H):
            gs = gf[cu[n]:cu[n + 1], h]
            sums = gate.chunk_sums(gs)
            W = int(win[n, h])
            if W > 0:
                assert gate.max_window_sum(sums, W) <= le, (n, h, W)
                if W > 1:
                    assert gate.max_window_sum(sums, W - 1) > le - 2e-3, (n, h, W)
            else:
                for w in range(1, min(16, len(sums)) + 1):
                    assert gate.max_window_sum(sums, w) > le - 2e-3, (n, h, w)
            ref = gate.window_chunks(gs, log_eps=le - 1e-3)
            assert W == ref or abs(gate.max_window_sum(sums, max(W, ref)) - (le - 1e-3)) < 1e-3
            checked += 1
    print("gate scan windows:", win.tolist())
    assert checked > 0


def _stage_setup(inp, opts):
    d = to_dev(inp)
    spec = inp["spec"]
    N = inp.get("N", spec.B)
    nbytes = binding.workspace_bytes(d["q"], d["v"], d["beta"], d["cu_seqlens"], d["cu_host"], opts)
    new_ws = lambda: torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")  # noqa: E731
    outs = lambda: (torch.empty_like(d["v"]),  # noqa: E731
                    torch.empty((N, spec.H, spec.dk, spec.dv), dtype=torch.float32, device="cuda"))

    def run(stages, ws, o, hT):
        for st in stages:
            binding.chunk_fwd_stage(st, d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                    cu_seqlens=d["cu_seqlens"], scale=inp["scale"], opts=opts,
                                    cu_seqlens_host=d["cu_host"], out=o, final_state_out=hT,
                                    workspace=ws)
        torch.cuda.synchronize()

    def region(r):
        return binding.workspace_region(d["q"], d["v"], d["beta"], r, d["cu_seqlens"], d["cu_host"], opts)
    return d, new_ws, outs, run, region


SEGWIN_CASES = {
    "sigmoid_L8": (lambda: synth.generate(spec(B=2, T=64 * 40 + 9, H=4, seed=86, zero_gate_heads=())), 8),
    "uniform_L3": (lambda: synth.generate(spec(B=1, T=64 * 30, H=3, gate="uniform", seed=87, zero_gate_heads=())), 3),
    "mixed_L8": (lambda: synth.generate(spec(B=1, T=64 * 40, H=4, seed=88, zero_gate_heads=(2,))), 8),
    "zero_short_L8": (lambda: synth.generate(spec(B=1, T=64 * 24, H=2, seed=89, gate="zero", zero_gate_heads=())), 8),
    "packed_L4": (lambda: _packed([64 * 20 + 7, 64 * 3, 0, 64 * 9 + 5, 40], H=3, seed=90, zero_heads=(1,)), 4),
}


SUMS_CASES = dict(SEGWIN_CASES)
SUMS_CASES["odd_heads_L5"] = (lambda: synth.generate(spec(B=2, T=64 * 21 + 30, H=33, seed=91, zero_gate_heads=(4,))), 5)
SUMS_CASES["head_blocks_L4"] = (lambda: _packed([64 * 13 + 3, 64 * 2, 64 * 9], H=80, seed=92, zero_heads=(70,)), 4)


@pytest.mark.parametrize("case", sorted(SUMS_CASES))
def test_segment_windows_same_on_both_paths(case):
    """The one-pass path forms the chunk gate sums in a kernel of their own, the
    two-kernel path in the chunk inverse; both take the same wave scan over the same
    values, so the windows they decide are equal bit for bit (head counts that are
    odd and above one gate-sum block of 64 heads included)."""
    make, L = SUMS_CASES[case]
    inp = make()
    got = []
    for one_pass in (1, -1):
        opts = binding.make_opts(force_segment_chunks=L, one_pass=one_pass)
        d, new_ws, outs, run, region = _stage_setup(inp, opts)
        ws = new_ws()
        o, hT = outs()
        print("case %s one_pass=%d" % (case, one_pass), flush=True)
        run([binding.GDN_STAGE_INVERSE, binding.GDN_STAGE_GATE_SCAN], ws, o, hT)
        off, n = region(binding.GDN_REGION_SEGMENT_WINDOWS)
        got.append(ws[off:off + n].view(torch.int32).cpu())
    assert got[0].numel() > 0
    assert torch.equal(got[0], got[1])


@pytest.mark.parametrize("case", sorted(SEGWIN_CASES))
def test_segment_windows_stage(case):
    """The per-segment windows the gate scan writes (GDN_REGION_SEGMENT_WINDOWS)
    against the fp64 per-segment rule of oracle/gate.py: every GPU window is
    admissible in fp64 (its chunks sum to <= log eps, or it reaches the sequence
    start) and minimal up to the 1e-3 margin band; a pair the GPU sends to the
    correction has a start with no window below the band; decisions outside the
    band equal the oracle's."""
    make, L = SEGWIN_CASES[case]
    inp = make()
    opts = binding.make_opts(force_segment_chunks=L)
    d, new_ws, outs, run, region = _stage_setup(inp, opts)
    ws = new_ws()
    o, hT = outs()
    run([binding.GDN_STAGE_INVERSE, binding.GDN_STAGE_GATE_SCAN], ws, o, hT)
    off, n = region(binding.GDN_REGION_SEGMENT_WINDOWS)
    H = inp["spec"].H
    got = ws[off:off + n].view(torch.int32).reshape(-1, H).cpu().numpy()
    le = math.log(2.0 ** -16)          # bf16 default tolerance
    g64 = synth.as_f64(inp["g"])
    cu = None if inp.get("cu_seqlens") is None else inp["cu_seqlens"].numpy()
    ref = gate.segment_windows(g64, L, cu_seqlens=cu, log_eps=le - 1e-3)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    B, T, _ = g64.shape
    cuv = np.arange(B + 1) * T if cu is None else cu
    gf = g64.reshape(-1, H)
    row = 0
    for s_ in range(len(cuv) - 1):
        nch = (cuv[s_ + 1] - cuv[s_] + 63) // 64
        segs = max(1, (nch + L - 1) // L)
        for h in range(H):
            sums = gate.chunk_sums(gf[cuv[s_]:cuv[s_ + 1], h])
            col = got[row:row + segs, h]
            assert col[0] == 0, (s_, h)
            if segs > 1 and (col[1:] == 0).all():     # correction: some start has no window
                assert any(j * L > 16 and all(sums[j * L - w:j * L].sum() > le - 2e-3 for w in range(1, 17))
                           for j in range(1, segs)), (s_, h)
            else:
                for j in range(1, segs):
                    st, W = j * L, int(col[j])
                    assert 1 <= W <= min(16, st), (s_, h, j, W)
                    assert W == st or sums[st - W:st].sum() <= le, (s_, h, j, W)
                    for w in range(1, W):
                        assert sums[st - w:st].sum() > le - 2e-3, (s_, h, j, w)
            near = any(abs(sums[j * L - w:j * L].sum() - (le - 1e-3)) < 1e-3
                       for j in range(1, segs) for w in range(1, min(16, j * L) + 1))
            if not near:
                assert (col == ref[row:row + segs, h]).all(), (s_, h, col.tolist(), ref[row:row + segs, h].tolist())
        row += segs
    assert row == got.shape[0]
    print("segment windows", case, got.T.tolist())


STAGE_CASES = {
    "dense_split": (lambda: synth.generate(spec(seed=81, h0_std=0.05)),
                    dict(force_segment_chunks=3)),
    "dense_tree": (lambda: synth.generate(spec(T=64 * 80 + 9, seed=82)), dict(force_segment_chunks=1)),
    "packed_split": (lambda: _packed([64 * 9 + 7, 40, 0, 64 * 3, 64 * 6 + 1, 0], H=2, seed=83),
                     dict(force_segment_chunks=2)),
    "unsplit_f32": (lambda: synth.generate(spec(H=2, dk=64, dv=64, dtype="f32", seed=84)), dict(no_split=1)),
    "planner": (lambda: synth.generate(spec(T=64 * 64, seed=85)), dict()),
}


@pytest.mark.parametrize("case", sorted(STAGE_CASES))
def test_stages_one_by_one_equal_whole_call(case):
    """gdn_chunk_fwd_stage run for every stage in order reproduces gdn_chunk_fwd bit
    for bit (split with correction and window heads, tree merge, packed, unsplit)."""
    make, kw = STAGE_CASES[case]
    inp = make()
    opts = binding.make_opts(**kw)
    d, new_ws, outs, run, _ = _stage_setup(inp, opts)
    o_ref, h_ref = outs()
    binding.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], cu_seqlens=d["cu_seqlens"],
                      scale=inp["scale"], opts=opts, cu_seqlens_host=d["cu_host"], out=o_ref,
                      final_state_out=h_ref, workspace=new_ws())
    o, hT = outs()
    run(range(binding.GDN_NUM_STAGES), new_ws(), o, hT)
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), case
    assert_parity(compare_pairs(inp, o, hT), TOL[inp["spec"].dtype], "stages " + case)


@pytest.mark.parametrize("case", ["dense_split", "dense_tree", "packed_split"])
def test_segment_regions_carry_everything_the_next_stage_needs(case):
    """A second workspace that ran only the stages before the merge, given the S*/M
    region of the first (as a sequence split across GPUs would receive it), finishes
    with the first's result; so does one given only the segment-start region before
    the last stage."""
    make, kw = STAGE_CASES[case]
    inp = make()
    opts = binding.make_opts(**kw)
    d, new_ws, outs, run, region = _stage_setup(inp, opts)
    S = binding
    wa = new_ws()
    o_ref, h_ref = outs()
    run(range(S.GDN_NUM_STAGES), wa, o_ref, h_ref)
    for reg, before, after in [(S.GDN_REGION_SEGMENT_MAPS, [S.GDN_STAGE_INVERSE, S.GDN_STAGE_GATE_SCAN],
                                [S.GDN_STAGE_CP_MERGE, S.GDN_STAGE_FORWARD]),
                               (S.GDN_REGION_SEGMENT_STARTS, [S.GDN_STAGE_INVERSE, S.GDN_STAGE_GATE_SCAN],
                                [S.GDN_STAGE_FORWARD])]:
        off, n = region(reg)
        assert n > 0
        wb = new_ws()
        wb.fill_(0xA5)   # nothing of the first workspace leaks in
        o, hT = outs()
        run(before, wb, o, hT)
        wb[off:off + n].copy_(wa[off:off + n])
        run(after, wb, o, hT)
        assert torch.equal(o, o_ref) and torch.equal(hT, h_ref), (case, reg)


@pytest.mark.parametrize("case", ["dense_bf16", "dense_tree_f32", "packed_bf16"])
def test_segment_starts_stage_parity(case):
    """Stage parity of pass 1 and the merge: with every head on the correction path,
    the segment starts the merge writes (workspace region GDN_REGION_SEGMENT_STARTS,
    slot = global segment * H + head, K-major) equal the chunked oracle's
    h_start(j+1) = M_j h_start(j) + S*_j, segment by segment (relative L2 within the
    storage dtype's tolerance)."""
    from oracle import chunked
    L = 1 if case == "dense_tree_f32" else 2   # 80 merge steps: the tree
    if case == "dense_bf16":
        inp = synth.generate(spec(B=2, T=64 * 9 + 5, H=2, seed=91, h0_std=0.05))
    elif case == "dense_tree_f32":
        inp = synth.generate(spec(B=1, T=64 * 80 + 9, H=2, dk=64, dv=64, dtype="f32", seed=92))
    else:
        inp = _packed([64 * 7 + 3, 0, 64 * 5, 30], H=2, seed=93)
    sp = inp["spec"]
    opts = binding.make_opts(force_segment_chunks=L, force_correction=1)
    d, new_ws, outs, run, region = _stage_setup(inp, opts)
    ws = new_ws()
    o, hT = outs()
    run([binding.GDN_STAGE_INVERSE, binding.GDN_STAGE_GATE_SCAN, binding.GDN_STAGE_CP_PASS1,
         binding.GDN_STAGE_CP_MERGE], ws, o, hT)
    off, n = region(binding.GDN_REGION_SEGMENT_STARTS)
    H, dk, dv = sp.H, sp.dk, sp.dv
    starts = ws[off:off + n].view(torch.float32).reshape(-1, H, dk, dv).cpu().double().numpy()
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    _, _, info = chunked.cp_forward(*(synth.as_f64(inp[x]) for x in ("q", "k", "v", "g", "beta")),
                                    h0=synth.as_f64(inp["h0"]), cu_seqlens=cu, scale=inp["scale"],
                                    seg_chunks=L)
    lens = ([sp.T] * sp.B if cu is None else list(np.diff(cu)))
    base, worst, checked = 0, 0.0, 0
    for nseq, ln in enumerate(lens):
        nch = (int(ln) + 63) // 64
        segs = max(1, (nch + L - 1) // L)
        for h in range(H):
            ref = info[(nseq, h)]["h_start"]
            for j in range(1, len(ref)):   # segment 0 starts from h0, which the merge does not form
                e = rel_l2(starts[base + j, h], ref[j])
                worst = max(worst, e)
                checked += 1
        base += segs
    assert base == starts.shape[0]
    print("%s: %d segment starts, worst rel L2 %.3e" % (case, checked, worst), flush=True)
    assert checked > 0 and worst <= TOL[sp.dtype]


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (64, 64)])
@pytest.mark.parametrize("corr", [0, 1])
def test_one_pass_pass1_column_blocks(dk, dv, corr):
    """Pass 1 in the one-pass kernel: a unit's value block then its dk / dv
    transition-matrix blocks (three blocks at dk = 128, dv = 64), from the gate scan's
    work list (head 0 without decay) or every segment (forced correction)."""
    inp = synth.generate(spec(B=2, T=64 * 9 + 5, H=2, dk=dk, dv=dv, seed=140 + dk + dv + corr,
                              zero_gate_heads=(0,), h0_std=0.05))
    opts = binding.make_opts(force_segment_chunks=2, force_correction=corr, one_pass=1)
    assert binding.plan_one_pass(inp["q"], inp["v"], inp["beta"], None, opts)
    o, hT = run_gpu(inp, opts=opts)
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "one-pass pass 1 dk=%d dv=%d corr=%d" % (dk, dv, corr))
