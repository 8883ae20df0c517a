"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Element-by-element per (sequence, head) relative L2 on o and on the final state,
at sizes the oracle finishes in seconds (several chunks, ragged tails, packed
sequences, empty sequences), plus stage parity of the chunk inverse and the GPU
side of the invariants.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from oracle import chunked
from tests.gpu_util import TOL, assert_parity, compare_pairs, run_gpu, to_dev

pytestmark = pytest.mark.gpu


def spec(**kw):
    base = dict(name="t", B=1, T=256, H=1, dk=64, dv=64, dtype="bf16", seed=0)
    base.update(kw)
    return synth.Spec(**base)


CASES = [
    # name, spec kwargs, opts
    ("tiny_fp32_workload", dict(B=1, T=256, H=1, dk=64, dv=64, dtype="f32", seed=1)),
    ("fp32_ragged_h0", dict(B=2, T=200, H=2, dk=64, dv=64, dtype="f32", h0_std=0.1, seed=21)),
    ("fp32_dk128", dict(B=1, T=130, H=2, dk=128, dv=64, dtype="f32", seed=22)),
    ("bf16_d128_ragged_h0", dict(B=2, T=300, H=3, dk=128, dv=128, h0_std=0.05, seed=23)),
    ("bf16_d64", dict(B=2, T=257, H=2, dk=64, dv=64, seed=24)),
    ("bf16_dk64_dv128", dict(B=1, T=190, H=2, dk=64, dv=128, seed=25)),
    ("bf16_dk128_dv64", dict(B=1, T=190, H=2, dk=128, dv=64, seed=26)),
    ("bf16_strong_gate", dict(B=1, T=700, H=2, dk=128, dv=128, gate="uniform", seed=27)),
    ("bf16_no_decay", dict(B=1, T=700, H=2, dk=128, dv=128, gate="zero", seed=28)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_parity_small(name, kw):
    inp = synth.generate(spec(name=name, **kw))
    o, hT = run_gpu(inp)
    assert_parity(compare_pairs(inp, o, hT), TOL[inp["spec"].dtype], name)


@pytest.mark.parametrize("vb", [64, 128])
def test_parity_value_block(vb):
    inp = synth.generate(spec(B=2, T=333, H=2, dk=128, dv=128, h0_std=0.05, seed=29))
    o, hT = run_gpu(inp, opts=binding.make_opts(value_block=vb))
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "value_block %d" % vb)


def _packed(lengths, H, dk, dv, dtype, h0_std, seed):
    """Packed sequences with given lengths (built from one dense draw)."""
    T = int(sum(lengths))
    inp = synth.generate(spec(B=1, T=T, H=H, dk=dk, dv=dv, dtype=dtype, seed=seed))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    inp["cu_seqlens"] = torch.from_numpy(cu)
    inp["N"] = len(lengths)
    if h0_std:
        g = torch.Generator().manual_seed(seed)
        inp["h0"] = (torch.randn(len(lengths), H, dk, dv, generator=g) * h0_std).float()
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_parity_packed_with_empty_and_tiny(dtype):
    inp = _packed([1, 64, 0, 65, 200, 130, 3], H=2, dk=64, dv=64, dtype=dtype, h0_std=0.05, seed=31)
    o, hT = run_gpu(inp)
    assert_parity(compare_pairs(inp, o, hT), TOL[dtype], "packed_" + dtype)


def test_parity_packed_d128():
    inp = _packed([512, 77, 1000, 64], H=3, dk=128, dv=128, dtype="bf16", h0_std=0.02, seed=32)
    o, hT = run_gpu(inp)
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "packed_d128")


@pytest.mark.parametrize("dtype,dk", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_chunk_inverse_stage(dtype, dk):
    """T from the HIP step-1 kernel against the oracle's T (same stored K, g, beta),
    and the residual ||(I + A) T - I||_F / sqrt(C)."""
    inp = synth.generate(spec(B=1, T=64 * 3 + 17, H=2, dk=dk, dv=64, dtype=dtype, seed=41,
                              gate="uniform"))
    d = to_dev(inp)
    T = binding.chunk_inverse(d["k"], d["g"], d["beta"])
    torch.cuda.synchronize()
    Tg = T.to("cpu").to(torch.float64).numpy()
    k64, g64, b64 = (synth.as_f64(inp[x]) for x in ("k", "g", "beta"))
    tol = 1e-2 if dtype == "bf16" else 1e-5
    worst = 0.0
    for c in range(Tg.shape[0]):
        s, e = 64 * c, min(64 * c + 64, inp["spec"].T)
        for h in range(2):
            Tref, A = chunked.chunk_inverse(k64[0, s:e, h], g64[0, s:e, h], b64[0, s:e, h])
            n = e - s
            Tgc = Tg[c, h]
            # padded rows/cols are the identity
            assert np.allclose(Tgc[n:, n:], np.eye(64 - n)) and np.all(Tgc[:n, n:] == 0)
            assert np.all(np.triu(Tgc, 1) == 0) and np.all(np.diag(Tgc) == 1)
            err = np.linalg.norm(Tgc[:n, :n] - Tref) / np.linalg.norm(Tref)
            resid = np.linalg.norm((np.eye(n) + A) @ Tgc[:n, :n] - np.eye(n)) / np.sqrt(64)
            worst = max(worst, err, resid)
    print("chunk inverse worst rel err / residual %.3e (tol %.0e)" % (worst, tol))
    assert worst <= tol


def test_beta_zero_no_decay_keeps_state_bitwise():
    inp = synth.generate(spec(B=1, T=300, H=2, dk=128, dv=128, gate="zero", h0_std=0.1, seed=51))
    inp["beta"] = torch.zeros_like(inp["beta"])
    o, hT = run_gpu(inp)
    assert torch.equal(hT.cpu(), inp["h0"])
    assert_parity(compare_pairs(inp, o, hT), TOL["bf16"], "beta0")


def test_causality_bitwise():
    inp = synth.generate(spec(B=1, T=400, H=2, dk=128, dv=128, seed=52))
    o1, _ = run_gpu(inp)
    t0 = 150
    inp2 = dict(inp)
    for key in ("q", "k", "v"):
        x = inp[key].clone()
        x[:, t0:] = torch.flip(x[:, t0:], dims=[1])
        inp2[key] = x
    b = inp["beta"].clone()
    b[:, t0:] = 0.5
    inp2["beta"] = b
    o2, _ = run_gpu(inp2)
    assert torch.equal(o1[:, :t0].cpu(), o2[:, :t0].cpu())
    assert not torch.equal(o1[:, t0:].cpu(), o2[:, t0:].cpu())


@pytest.mark.parametrize("t1", [128, 100])
def test_state_carry(t1):
    inp = synth.generate(spec(B=1, T=320, H=2, dk=128, dv=128, h0_std=0.05, seed=53))
    o, hT = run_gpu(inp)
    a = dict(inp); b = dict(inp)
    for key in ("q", "k", "v", "g", "beta"):
        a[key] = inp[key][:, :t1].contiguous()
        b[key] = inp[key][:, t1:].contiguous()
    a["spec"] = spec(B=1, T=t1, H=2, dk=128, dv=128)
    oa, ha = run_gpu(a)
    b["h0"] = ha.cpu()
    b["spec"] = spec(B=1, T=320 - t1, H=2, dk=128, dv=128)
    ob, hb = run_gpu(b)
    oc = torch.cat([oa, ob], dim=1).float()
    rel_o = (oc - o.float()).norm() / o.float().norm()
    rel_h = (hb - hT).norm() / hT.norm()
    assert rel_o < 1e-2 and rel_h < 1e-2, (rel_o, rel_h)


def test_deterministic_repeat():
    inp = synth.generate(spec(B=2, T=500, H=2, dk=128, dv=128, seed=54))
    o1, h1 = run_gpu(inp)
    o2, h2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_packed_equals_separate_runs_bitwise():
    lengths = [200, 64, 129]
    inp = _packed(lengths, H=2, dk=128, dv=128, dtype="bf16", h0_std=0.02, seed=55)
    o, hT = run_gpu(inp)
    cu = inp["cu_seqlens"].numpy()
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        one = dict(inp)
        for key in ("q", "k", "v", "g", "beta"):
            one[key] = inp[key][:, s:e].contiguous()
        one["h0"] = inp["h0"][n:n + 1].contiguous()
        one["cu_seqlens"] = None
        one["spec"] = spec(B=1, T=e - s, H=2, dk=128, dv=128)
        o1, h1 = run_gpu(one)
        assert torch.equal(o1[0].cpu(), o[0, s:e].cpu())
        assert torch.equal(h1[0].cpu(), hT[n].cpu())


def _basis_inputs(T, H, dk, dv, m, seed, dtype):
    """k_t = q_t = e_{t mod m} (m < 64: keys repeat inside a chunk), beta = 1, g = 0,
    zero initial state, scale 1/8 (a power of two); v = integers in [-64, 64] / 16, so
    every sum or difference of two values is an integer of at most 8 bits over 16,
    exact in bf16."""
    g = torch.Generator().manual_seed(seed)
    idx = torch.arange(T) % m
    kq = torch.zeros(1, T, H, dk)
    kq[0, torch.arange(T), :, idx] = 1.0
    v = (torch.randint(-64, 65, (1, T, H, dv), generator=g).float() / 16).to(dtype)
    return dict(q=kq.to(dtype), k=kq.to(dtype).clone(), v=v, g=torch.zeros(1, T, H),
                beta=torch.ones(1, T, H).to(dtype), h0=None, cu_seqlens=None, scale=0.125)


@pytest.mark.parametrize("m,dk,dv", [(5, 128, 128), (17, 64, 128), (63, 128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_basis_keys_with_repeats(m, dk, dv, dtype):
    """Closed form: with k_t = q_t = e_{t mod m}, beta = 1, g = 0 and S_0 = 0, the
    delta rule replaces column t mod m of S by v_t, so o_t = scale v_t, and row j < m
    of the final state is v of the last token with key e_j.  Every intermediate of the
    chunked form is then exact in both precisions (T has entries in {-1, 0, 1}, the
    gates are exp(0) = 1, V' = v - h and U are differences of two values, all integers
    of at most 8 bits over 16, and the bf16 MFMA operands hold them exactly), so the
    GPU must match to the bit."""
    T, H = 300, 2
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    inp = _basis_inputs(T, H, dk, dv, m, seed=60 + m, dtype=tdt)
    o, hT = run_gpu(inp)
    want_h = torch.zeros(1, H, dk, dv)
    for j in range(m):
        last = max(t for t in range(T) if t % m == j)
        want_h[0, :, j, :] = inp["v"][0, last].float()
    want_o = inp["v"] * 0.125
    bad = (o.cpu().float() != want_o.float()).sum().item()
    print("basis keys m=%d %s: %d of %d outputs differ, max |diff| %.3e" % (
        m, dtype, bad, o.numel(), (o.cpu().float() - want_o.float()).abs().max().item()))
    assert torch.equal(o.cpu(), want_o)
    assert torch.equal(hT.cpu(), want_h)


def test_beta_one_last_token_closed_form():
    """Closed form: a delta-rule update with beta = 1 and a unit key makes the new state
    map that key to its value exactly, whatever alpha and the prior state: with beta = 1
    on the last token, sum_i hT[i, j] k_T[i] = v_T[j] (up to the bf16/fp32 rounding of
    the chunked products)."""
    inp = synth.generate(spec(B=2, T=333, H=3, dk=128, dv=128, h0_std=0.05, seed=61))
    beta = inp["beta"].clone()
    beta[:, -1] = 1.0
    inp["beta"] = beta
    o, hT = run_gpu(inp)
    k_last = inp["k"][:, -1].float()              # [B, H, dk]
    v_last = inp["v"][:, -1].float()              # [B, H, dv]
    got = torch.einsum("bhij,bhi->bhj", hT.cpu().float(), k_last)
    rel = (got - v_last).norm() / v_last.norm()
    assert rel < 1e-2, rel


@pytest.mark.parametrize("packed", [False, True])
def test_no_tokens_passes_state_through(packed):
    """Degenerate input: no tokens at all (dense T = 0, or packed sequences that are
    all empty).  The output is empty and the final state equals the initial state,
    bit for bit (no recurrence step touches it)."""
    H, dk, dv = 2, 128, 128
    if packed:
        inp = _packed([0, 0, 0], H=H, dk=dk, dv=dv, dtype="bf16", h0_std=0.1, seed=71)
    else:
        inp = synth.generate(spec(B=2, T=0, H=H, dk=dk, dv=dv, h0_std=0.1, seed=71))
    o, hT = run_gpu(inp)
    assert o.numel() == 0
    assert torch.equal(hT.cpu(), inp["h0"])
