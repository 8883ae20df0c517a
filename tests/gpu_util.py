"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and
compare per (sequence, head) with the fp64 oracle on the same stored inputs."""
import numpy as np
import torch

from gated_deltanet_chunked_fwd_amd import binding, synth
from oracle import token

# Tolerances: max over (sequence, head) of relative L2 error on o and on the final
# state; bf16 storage with fp32 accumulation vs fp32 storage.
TOL = {"bf16": 1e-2, "f32": 1e-5}


def to_dev(inp, device="cuda"):
    out = dict(inp)
    for key in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens"):
        if inp.get(key) is not None:
            out[key] = inp[key].to(device).contiguous()
    out["cu_host"] = inp.get("cu_seqlens")
    return out


def run_gpu(inp, opts=None, output_final_state=True):
    d = to_dev(inp)
    o, hT = binding.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                              cu_seqlens=d["cu_seqlens"], scale=inp["scale"],
                              output_final_state=output_final_state, opts=opts,
                              cu_seqlens_host=d["cu_host"])
    torch.cuda.synchronize()
    return o, hT


def seq_bounds(inp):
    spec = inp["spec"]
    if inp.get("cu_seqlens") is not None:
        cu = inp["cu_seqlens"].numpy().astype(np.int64)
        return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    return [(b, 0, spec.T) for b in range(spec.B)]


def oracle_pair(inp, n, h):
    """fp64 oracle for one (sequence, head): returns (o [len, dv], hT [dk, dv])."""
    b, s, e = seq_bounds(inp)[n]
    sl = lambda t: synth.as_f64(t[b:b + 1, s:e, h:h + 1])  # noqa: E731
    h0 = None if inp.get("h0") is None else synth.as_f64(inp["h0"][n:n + 1, h:h + 1])
    o, hT = token.token_recurrence(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                   sl(inp["beta"]), h0, scale=inp["scale"])
    return o[0, :, 0], hT[0, 0]


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    if nb < 1e-30:
        return float(np.linalg.norm(a - b))
    return float(np.linalg.norm(a - b) / nb)


def compare_pairs(inp, o_gpu, hT_gpu, pairs=None):
    """Per-(sequence, head) relative L2 errors of o and of the final state."""
    spec = inp["spec"]
    bounds = seq_bounds(inp)
    if pairs is None:
        pairs = [(n, h) for n in range(len(bounds)) for h in range(spec.H)]
    og = o_gpu.detach().to("cpu").to(torch.float64).numpy()
    hg = None if hT_gpu is None else hT_gpu.detach().to("cpu").to(torch.float64).numpy()
    errs = []
    for (n, h) in pairs:
        b, s, e = bounds[n]
        o_ref, h_ref = oracle_pair(inp, n, h)
        eo = rel_l2(og[b, s:e, h], o_ref) if e > s else 0.0
        eh = rel_l2(hg[n, h], h_ref) if hg is not None else 0.0
        errs.append((n, h, eo, eh))
    return errs


def assert_parity(errs, tol, label=""):
    worst_o = max(e[2] for e in errs)
    worst_h = max(e[3] for e in errs)
    msg = "%s worst rel L2: o %.3e, state %.3e (tol %.0e); %s" % (
        label, worst_o, worst_h, tol, [(n, h, "%.2e" % a, "%.2e" % b) for n, h, a, b in errs[:8]])
    print(msg, flush=True)
    assert worst_o <= tol and worst_h <= tol, msg


def compare_pairs_magnitude(inp, o_gpu, pairs=None):
    """Per-(sequence, head) output error judged against the magnitude of each output's
    inner product: ||o - o_ref||_2 / ||m||_2 with m_t = scale |S_t| |q_t| from the
    oracle (token.output_magnitude_numpy).  A floating point inner product errs by a
    multiple of the unit roundoff times m, whatever |o| is, so this criterion stays
    meaningful where o_t's inner product cancels.  Small inputs only (numpy oracle)."""
    spec = inp["spec"]
    bounds = seq_bounds(inp)
    if pairs is None:
        pairs = [(n, h) for n in range(len(bounds)) for h in range(spec.H)]
    og = o_gpu.detach().to("cpu").to(torch.float64).numpy()
    errs = []
    for (n, h) in pairs:
        b, s, e = bounds[n]
        if e == s:
            errs.append((n, h, 0.0, 0.0))
            continue
        o_ref, _ = oracle_pair(inp, n, h)
        sl = lambda t: synth.as_f64(t[b:b + 1, s:e, h:h + 1])  # noqa: E731
        h0 = None if inp.get("h0") is None else synth.as_f64(inp["h0"][n:n + 1, h:h + 1])
        m = token.output_magnitude_numpy(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["g"]),
                                         sl(inp["beta"]), h0, scale=inp["scale"])[0, :, 0]
        errs.append((n, h, float(np.linalg.norm(og[b, s:e, h] - o_ref) / max(np.linalg.norm(m), 1e-300)),
                     float(np.linalg.norm(o_ref) / max(np.linalg.norm(m), 1e-300))))
    return errs
