"""Benchmark of the GDN chunked-prefill forward on one MI355X.

One step = one gdn_chunk_fwd call (every stage of the forward) over one batch of
seeded synthetic input, all inputs resident in HBM.  Default workload: the
Qwen-like prefill (B=4, T=4096, H=16, dk=dv=128, bf16 q/k/v/o, fp32 g, bf16 beta,
zero initial state, fp32 final state).

Timing: W untimed warm-up steps, then a short stage pass (3 calls, each after a
cache eviction, every stage timed) that finds the dominant kernel.  The timed region
is exactly K back-to-back calls, after one cache eviction (512 MiB written, then
another 512 MiB read: this evicts the 256 MB MALL and the L2s and drains the dirty
lines), bracketed by device synchronisations and one pair of HIP events:
ms_per_step = region time / K.  Inside the region the dominant kernel is timed live
in every call, on the launch stream, by stop-only events that the library records
from kernel dispatches: from the end of the kernel launched before it to its own end
(a stop event adds nothing to the stream, while a start marker, like any separately
recorded event, idles the GPU for a few microseconds).  All events are created with
hipEventDisableSystemFence (no cache writeback when they complete).  For context,
path.ms_per_step_evicted_caches_median is the median of up to 10 calls that each
start after a cache eviction (each includes one start marker, a few microseconds).

Roofline (dominant kernel = the stage with the largest mean time; for the forward
stage that is fused_wy, the one-pass kernel, or fused_forward, the two-kernel
path's forward, whichever the plan runs):
  achieved = algorithmic bytes of that kernel per launch (stage_bytes(): for the
  pass that writes o, bytes per token-head = 2*(dk+dv)*e_qkv + e_g + e_beta plus
  the fp32 states) / its live mean duration; peak = 8000 GB/s.
traffic = HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (from
profiles/traffic_<kernel>.json) if those counters were taken on the current kernel
source, workload and segment length, else null.
roofline.whole_call: the same algorithmic bytes over the whole call (every launch,
ms_per_step), the figure the one-GPU target is stated on.

path.copy_gbs_context: read + write GB/s of a plain 512 MiB device copy on the same
stream, as context for what the HBM roofline allows in practice.

cpu_baseline: the fp64 oracle (plain C, OpenMP) on the host cores, rank 0 only.

Prints ONE JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
F32_PEAK_TFLOPS = 157.3
METRIC = "GDN fwd prefill ms & tokens/s at H=16,d=128,T=4k×4; % of MFMA/HBM roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="workload number (1-5)")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-split", type=int, default=0)
    ap.add_argument("--value-block", type=int, default=0)
    ap.add_argument("--one-pass", type=int, default=0, help="1: one-pass forward, -1: two-kernel path, 0: planner")
    ap.add_argument("--segment-chunks", type=int, default=0, help="force the split length (0: planner)")
    ap.add_argument("--batch", type=int, default=0,
                    help="override the workload's batch size B (dense workloads; occupancy sweeps)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (gdn_chunk_bwd) on the workload instead of the forward")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (the known-size kernel that "
                         "scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings) and exit")
    return ap.parse_args()


def copy_reference(mib):
    """Three torch copies of a known size: each moves mib MiB in and mib MiB out."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_each_way": n * 4, "copies": 3}), flush=True)


class Hip:
    """HIP events through the runtime torch already loaded (same soname).  Timing
    events are created with hipEventDisableSystemFence: a default event performs a
    system-scope release (cache writeback and invalidation) when it completes, which
    idles the GPU for several microseconds after every event and slows the work that
    follows; these events only time work (every read of them follows a device
    synchronisation)."""

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            rc = self.lib.hipEventCreateWithFlags(ctypes.addressof(arr) + i * ctypes.sizeof(ctypes.c_void_p),
                                                  self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
        return arr

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float(0.0)
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            return float("nan")
        return float(ms.value)


def algorithmic_bytes(spec, n_seqs, has_h0, has_hT):
    """Compulsory HBM bytes of the whole path: q, k, v, g, beta in; o out; fp32
    states in/out.  This is also the per-launch figure of the pass that writes o
    (fused_forward), which reads and writes exactly these tensors."""
    e = 2 if spec.dtype == "bf16" else 4
    eb = 2 if (spec.beta_dtype or spec.dtype) == "bf16" else 4
    th = spec.B * spec.T * spec.H
    per_th = 2 * (spec.dk + spec.dv) * e + 4 + eb
    state = n_seqs * spec.H * spec.dk * spec.dv * 4
    return th * per_th + state * (int(has_h0) + int(has_hT))


def stage_bytes(stage, spec, lengths, seg_chunks, windows, has_h0, has_hT):
    """Algorithmic bytes one launch of `stage` must move, from the tensors it reads
    and writes by definition (intermediates are counted where a stage's job is to
    produce or consume them: T for the chunk inverse, S*/M/h_start for the split).
      chunk_inverse: k, g, beta per token-head in; T (64 x 64) per chunk-head out.
      cp_pass1 / cp_merge: only (sequence, head) pairs without a lookback window
        (windows[n][h] == 0) and only their non-last segments.  Pass 1 reads k, v,
        g, beta of those segments and writes S* (fp32) and M (2 x bf16) per segment;
        the merge reads M and S* and writes h_start per segment boundary.
      gate_scan: the chunk gate sums (fp32 per chunk-head).
      fused_forward: the compulsory bytes of the path."""
    C = 64
    e = 2 if spec.dtype == "bf16" else 4
    eb = 2 if (spec.beta_dtype or spec.dtype) == "bf16" else 4
    H, dk, dv = spec.H, spec.dk, spec.dv
    chunks = [(n + C - 1) // C for n in lengths]
    if stage == "chunk_inverse":
        return sum(lengths) * H * (dk * e + 4 + eb) + sum(chunks) * H * C * C * e
    if stage == "gate_scan":
        return sum(chunks) * H * 4
    if stage in ("cp_pass1", "cp_merge"):
        total = 0
        for n, (ln, nch) in enumerate(zip(lengths, chunks)):
            segs = max(1, -(-nch // seg_chunks))
            for h in range(H):
                if windows is None or windows[n][h] != 0 or segs < 2:
                    continue
                toks = min(ln, (segs - 1) * seg_chunks * C)
                if stage == "cp_pass1":
                    total += toks * ((dk + dv) * e + 4 + eb) + (segs - 1) * (dk * dv * 4 + 2 * dk * dk * 2)
                else:
                    total += (segs - 1) * (2 * dk * dk * 2 + 2 * dk * dv * 4)
        return total
    return algorithmic_bytes(spec, len(lengths), has_h0, has_hT)


def algorithmic_flops(spec, triangular=False):
    """Per token-head: 6 dk dv (K h, Q h, K~^T U) + 4 C (dk + dv) (K K^T, Q K^T, T V', P U)
    + C^2/3 (triangular inverse), C = 64, full C x C tiles; triangular=True counts only
    the lower triangles of the four C x C products (2 C (dk + dv))."""
    C = 64
    th = spec.B * spec.T * spec.H
    tiles = (2 if triangular else 4) * C * (spec.dk + spec.dv)
    return th * (6 * spec.dk * spec.dv + tiles + C * C / 3.0)


def copy_bandwidth(hip, stream, torch, mib=512, reps=5):
    """Context for the HBM roofline: GB/s (read + write) of a plain device copy of
    mib MiB, timed with HIP events on the bench stream."""
    src = torch.ones(mib << 18, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = hip.events(2)
    hip.record(ev[0], stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.record(ev[1], stream)
    ms = hip.elapsed(ev[0], ev[1]) / reps
    return 2 * (mib << 20) / (ms * 1e-3) / 1e9


def source_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def traffic_for(kernel, kernel_src, workload, seg_chunks):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counters
    (profiles/traffic_<kernel>.json), if they were taken on this exact kernel source,
    workload and segment length; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % kernel)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_sha(kernel_src):
        return None
    if rec.get("workload_name") != workload or rec.get("segment_chunks") != seg_chunks:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, spec, min_seconds=10.0):
    """The fp64 oracle on the host cores: the whole workload, repeated until at least
    min_seconds of wall time have passed (about 0.3 s per pass for the Qwen-like
    workload on 16 cores), reported as the mean rate over the passes."""
    from gated_deltanet_chunked_fwd_amd import synth
    from oracle import token

    cores = len(os.sched_getaffinity(0))
    args = [synth.as_f64(inp[k]) for k in ("q", "k", "v", "g", "beta")]
    h0 = synth.as_f64(inp["h0"])
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    passes, t0 = 0, time.perf_counter()
    while True:
        token.token_recurrence(*args, h0, cu_seqlens=cu, scale=inp["scale"], nthreads=cores)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    tokens = spec.B * spec.T
    return {"value": passes * tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "whole workload (%d tokens x %d heads), fp64 token recurrence, %d passes "
                      "in %.1f s" % (tokens, spec.H, passes, dt)}


def backward_bytes(spec, n_seqs, has_h0):
    """Compulsory HBM bytes of the backward: q, k, v, dO, g, beta in; dq, dk, dv, dg,
    dbeta out; the fp32 final-state gradient in and the initial-state gradient out
    (plus the initial state in, when there is one)."""
    e = 2 if spec.dtype == "bf16" else 4
    eb = 2 if (spec.beta_dtype or spec.dtype) == "bf16" else 4
    th = spec.B * spec.T * spec.H
    per = (2 * spec.dk + 2 * spec.dv) * e + 4 + eb + (2 * spec.dk + spec.dv) * e + 4 + eb
    states = n_seqs * spec.H * spec.dk * spec.dv * 4 * (3 if has_h0 else 2)
    return th * per + states


def bench_backward(args):
    """One JSON line for gdn_chunk_bwd on the workload: K back-to-back calls after one
    cache eviction, bracketed by device synchronisations and one event pair; the
    roofline is the backward's algorithmic bytes over that mean time."""
    import torch

    from gated_deltanet_chunked_fwd_amd import binding, synth

    spec = synth.WORKLOADS[args.workload]
    inp = synth.generate(spec)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev).contiguous())
         for k in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    N = inp["N"]
    gen = torch.Generator().manual_seed(1234)
    do = torch.randn(inp["v"].shape, generator=gen).to(inp["v"].dtype).to(dev)
    dhT = torch.randn((N, spec.H, spec.dk, spec.dv), generator=gen).float().to(dev)
    nbytes = ctypes.c_size_t(0)
    sh = binding._Shape(d["q"], d["v"], d["beta"], d["cu_seqlens"], inp["cu_seqlens"])
    opts = binding.make_opts(no_split=args.no_split, force_segment_chunks=args.segment_chunks)
    if binding.lib().gdn_chunk_bwd_workspace_bytes(sh.ref(), ctypes.byref(opts), ctypes.byref(nbytes)) != 0:
        raise RuntimeError("gdn_chunk_bwd_workspace_bytes failed")
    ws = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=dev)

    def step():
        return binding.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, d["h0"], dhT,
                                 cu_seqlens=d["cu_seqlens"], scale=inp["scale"],
                                 cu_seqlens_host=inp["cu_seqlens"], workspace=ws, opts=opts)

    for _ in range(args.warmup):
        step()
    hip = Hip()
    ev = hip.events(2)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if not args.no_flush:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush.fill_(1)
        del flush
    torch.cuda.synchronize()
    hip.record(ev[0], stream)
    for _ in range(args.steps):
        step()
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed(ev[0], ev[1]) / args.steps
    alg = backward_bytes(spec, N, d["h0"] is not None)
    achieved = alg / (ms * 1e-3) / 1e9
    rec = {
        "metric": "GDN bwd chunked: ms & tokens/s; % of HBM roofline",
        "value": spec.B * spec.T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic (seeded)",
        "config": {"workload": spec.name, "B": spec.B, "T": spec.T, "H": spec.H, "dk": spec.dk,
                   "dv": spec.dv, "pass": "backward", "split_allowed": not args.no_split,
                   "segment_chunks": args.segment_chunks or None, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "the whole backward call",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes": alg},
    }
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.backward:
        bench_backward(args)
        return

    import torch

    from gated_deltanet_chunked_fwd_amd import binding, synth

    spec = synth.WORKLOADS[args.workload]
    if args.batch:
        if spec.packed:
            print("--batch applies to dense workloads only", file=sys.stderr)
            sys.exit(2)
        spec = synth.workload(args.workload, B=args.batch,
                              name="%s_batch%d" % (spec.name, args.batch))
    inp = synth.generate(spec)
    dev = torch.device("cuda:0")
    d = {k: (None if inp[k] is None else inp[k].to(dev).contiguous())
         for k in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens")}
    N = inp["N"]
    o = torch.empty_like(d["v"])
    hT = torch.empty((N, spec.H, spec.dk, spec.dv), dtype=torch.float32, device=dev)
    hip = Hip()
    stage_ev = hip.events(2 * binding.GDN_NUM_STAGES)
    opts_all = binding.make_opts(no_split=args.no_split, value_block=args.value_block, one_pass=args.one_pass,
                                 force_segment_chunks=args.segment_chunks,
                                 stage_events=ctypes.cast(stage_ev, ctypes.c_void_p))
    opts = binding.make_opts(no_split=args.no_split, value_block=args.value_block, one_pass=args.one_pass,
                             force_segment_chunks=args.segment_chunks)
    ws = torch.empty(max(binding.workspace_bytes(d["q"], d["v"], d["beta"], d["cu_seqlens"],
                                                 inp["cu_seqlens"], opts), 1),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush_rd = torch.ones(128 << 20, dtype=torch.int32, device=dev)   # 512 MiB

    def evict(i):
        # write 512 MiB, then read another 512 MiB: the read pushes the written (dirty)
        # lines out of the L2s and the MALL here, so their write-back is not billed to
        # the next step (a write-only flush halves the next kernel's HBM read rate)
        flush.fill_(i & 0xFF)
        flush_rd.sum()
    seg_chunks = binding.plan_segment_chunks(d["q"], d["v"], d["beta"], inp["cu_seqlens"], opts)
    one_pass = binding.plan_one_pass(d["q"], d["v"], d["beta"], inp["cu_seqlens"], opts)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def step(o_=None):
        binding.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                          cu_seqlens=d["cu_seqlens"], scale=inp["scale"], opts=o_ or opts,
                          cu_seqlens_host=inp["cu_seqlens"], out=o, final_state_out=hT,
                          workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def stage_pass(steps):
        """Per-stage mean ms over `steps` flushed steps, every stage timed."""
        out = {i: [] for i in range(binding.GDN_NUM_STAGES)}
        for i in range(steps):
            if not args.no_flush:
                evict(i)
            # stages that a step does not run keep stale events: mark them first
            for st in range(binding.GDN_NUM_STAGES):
                hip.record(stage_ev[2 * st], stream)
                hip.record(stage_ev[2 * st + 1], stream)
            step(opts_all)
            for st in range(binding.GDN_NUM_STAGES):
                out[st].append(hip.elapsed(stage_ev[2 * st], stage_ev[2 * st + 1]))
        return {binding.STAGE_NAMES[st]: sum(v) / len(v) for st, v in out.items()
                if sum(v) / len(v) > 1e-4}

    st_mean = stage_pass(3)
    dom = max(st_mean, key=st_mean.get)
    dom_idx = binding.STAGE_NAMES.index(dom)
    NS = binding.GDN_NUM_STAGES
    # the stage whose last kernel runs right before the dominant one
    lengths_h = ([spec.T] * spec.B if inp["cu_seqlens"] is None
                 else [int(inp["cu_seqlens"][i + 1] - inp["cu_seqlens"][i]) for i in range(N)])
    split = seg_chunks < max((n + 63) // 64 for n in lengths_h)
    launched = [0] + ([1, 2, 3] if split else []) + [4]
    prev_idx = launched[launched.index(dom_idx) - 1] if launched.index(dom_idx) > 0 else None

    def timing_opts(ev_prev_stop, ev_dom_stop, ev_dom_start=None):
        arr = (ctypes.c_void_p * (2 * NS))()
        arr[2 * dom_idx + 1] = ev_dom_stop
        if prev_idx is not None:
            arr[2 * prev_idx + 1] = ev_prev_stop
        else:
            arr[2 * dom_idx] = ev_dom_start
        o_ = binding.make_opts(no_split=args.no_split, value_block=args.value_block, one_pass=args.one_pass,
                               force_segment_chunks=args.segment_chunks,
                               stage_events=ctypes.cast(arr, ctypes.c_void_p))
        o_._keep = arr
        return o_

    # ---- the timed region: exactly K back-to-back calls (after one cache eviction),
    #      bracketed by device synchronisations and one event pair.  Inside it, the
    #      dominant kernel is timed live in every call by stop-only events recorded
    #      from kernel dispatches: the end of the kernel launched before it to its own
    #      end (a stop event adds nothing to the stream; a start event would idle the
    #      GPU for a few microseconds before the kernel).
    K = args.steps
    kev = hip.events(2 * K)
    call_opts = [timing_opts(kev[2 * i], kev[2 * i + 1], kev[2 * i]) for i in range(K)]
    region_ev = hip.events(2)
    if not args.no_flush:
        evict(0)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    hip.record(region_ev[0], stream)
    for i in range(K):
        step(call_opts[i])
    t_enqueued = time.perf_counter()
    hip.record(region_ev[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    host_ms = (t_enqueued - t_wall0) / K * 1e3   # host time to enqueue one call
    ms = hip.elapsed(region_ev[0], region_ev[1]) / K
    dom_ms_list = [hip.elapsed(kev[2 * i], kev[2 * i + 1]) for i in range(K)]

    # context, outside the timed region: calls that each start from evicted caches
    # (one start marker per call, which adds a few microseconds of idle GPU)
    cold_ms = []
    if not args.no_flush:
        cev = hip.events(2)
        cold_opts = timing_opts(None, cev[1], None)   # the call's end: the dominant kernel's stop
        for i in range(min(K, 10)):
            evict(i + 1)
            hip.record(cev[0], stream)
            step(cold_opts)
            cold_ms.append(hip.elapsed(cev[0], cev[1]))

    tokens = spec.B * spec.T
    dom_ms = sum(dom_ms_list) / len(dom_ms_list)
    has_h0 = d["h0"] is not None
    alg_bytes = algorithmic_bytes(spec, N, has_h0, True)
    cu_host = inp["cu_seqlens"]
    lengths = ([spec.T] * spec.B if cu_host is None
               else [int(cu_host[i + 1] - cu_host[i]) for i in range(N)])
    windows = None
    corrected = 0.0
    if seg_chunks < max((n + 63) // 64 for n in lengths):
        windows = binding.gate_scan(d["g"], d["cu_seqlens"], cu_host).cpu().tolist()
        flat = [w for row in windows for w in row]
        corrected = sum(1 for w in flat if w == 0) / max(1, len(flat))
    model_us = binding.plan_predict_us(d["q"], d["v"], d["beta"], cu_host, opts, corrected)
    dom_bytes = stage_bytes(dom, spec, lengths, seg_chunks, windows, has_h0, True)
    flops = algorithmic_flops(spec)
    copy_gbs = copy_bandwidth(hip, stream, torch)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    kernel = ("fused_wy" if one_pass else "fused_forward") if dom == "fused_forward" else dom
    ksrc = os.path.join(ROOT, "gated_deltanet_chunked_fwd_amd", "csrc", kernel + ".hip")
    traffic = traffic_for(kernel, ksrc, spec.name, seg_chunks) if dom == "fused_forward" else None
    call_achieved = alg_bytes / (ms * 1e-3) / 1e9
    mfma_peak = BF16_PEAK_TFLOPS if spec.dtype == "bf16" else F32_PEAK_TFLOPS
    rec = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded; q,k L2-normalised, g=log sigmoid(N(3,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": spec.name, "B": spec.B, "T": spec.T, "H": spec.H, "dk": spec.dk,
                   "dv": spec.dv, "chunk": 64, "initial_state": has_h0,
                   "final_state": True, "split_allowed": not args.no_split,
                   "segment_chunks": seg_chunks, "one_pass": one_pass, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": dom_bytes, "kernel_ms": dom_ms,
                     "whole_call": {"achieved": call_achieved, "frac": call_achieved / HBM_PEAK_GBS,
                                    "ms": ms, "algorithmic_bytes": alg_bytes}},
        "path": {"hbm_frac": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "mfma_frac": flops / (ms * 1e-3) / 1e12 / mfma_peak,
                 "algorithmic_flops": flops,
                 "algorithmic_flops_triangular": algorithmic_flops(spec, triangular=True),
                 "copy_gbs_context": copy_gbs, "stage_ms": st_mean,
                 "ms_per_step_evicted_caches_median":
                     sorted(cold_ms)[len(cold_ms) // 2] if cold_ms else None,
                 "dominant_ms_min": min(dom_ms_list),
                 "model_ms": model_us * 1e-3, "model_corrected_fraction": corrected,
                 "wall_s_timed_region": wall,
                 "host_ms_per_call": host_ms},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, spec)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
