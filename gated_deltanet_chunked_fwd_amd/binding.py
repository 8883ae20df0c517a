"""Thin ctypes binding over libgdn.so (the C ABI declared in include/gdn.h).

Argument marshalling only: every step of the forward runs in the library's HIP
kernels.  torch provides device memory (outputs, workspace) and the stream.  The
library must have been built (``gated_deltanet_chunked_fwd_amd.build``); if it is
missing, the first call raises -- there is no fallback.
"""
import ctypes
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

from .abi import (EXPORTS, GDN_BF16, GDN_ERR_ARG, GDN_ERR_HIP, GDN_ERR_SCRATCH,  # noqa: F401
                  GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_NOALLOC_SCRATCH_BYTES, GDN_F32, GDN_NUM_REGIONS, GDN_NUM_STAGES, GDN_OK,
                  GDN_REGION_CHUNK_INVERSE, GDN_REGION_SEGMENT_MAPS, GDN_REGION_SEGMENT_STARTS,
                  GDN_REGION_SEGMENT_WINDOWS, GDN_STAGE_CP_MERGE, GDN_STAGE_CP_PASS1, GDN_STAGE_FORWARD,
                  GDN_STAGE_GATE_SCAN, GDN_STAGE_INVERSE, STAGE_NAMES, GdnOpts, GdnShape, declare,
                  make_opts)


class GdnError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, status_str(status), status))
        self.status = status


_LIB = None


def lib():
    """Loads libgdn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        declare(L)
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().gdn_status_str(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond, what):
    if not cond:
        raise ValueError(what)


def _check_tensor(t, name, dtypes, shape, device, require_cuda):
    _need(isinstance(t, torch.Tensor), "%s must be a torch.Tensor" % name)
    if require_cuda:
        _need(t.is_cuda, "%s must be a device tensor" % name)
    if device is not None:
        _need(t.device == device, "%s is on %s, expected %s" % (name, t.device, device))
    _need(t.dtype in dtypes, "%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    _need(tuple(t.shape) == tuple(shape), "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    _need(t.is_contiguous(), "%s must be contiguous" % name)


def check_forward_args(q, k, v, g, beta, initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                       out=None, final_state_out=None, workspace=None, require_cuda=True):
    """Checks every tensor argument of chunk_fwd against the layouts of include/gdn.h
    (the library reinterprets raw pointers, so a wrong dtype or shape would be read
    past its end) and raises ValueError on the first mismatch.  Returns cu_seqlens as
    the int32 device tensor the library reads (an int64 cu_seqlens, FLA's convention,
    is converted)."""
    fp = (torch.bfloat16, torch.float32)
    _need(isinstance(q, torch.Tensor) and q.dim() == 4, "q must be a 4-D tensor [B, T, H, dk]")
    B, T, H, dk = q.shape
    dev = q.device
    _check_tensor(q, "q", fp, (B, T, H, dk), None, require_cuda)
    _check_tensor(k, "k", (q.dtype,), (B, T, H, dk), dev, require_cuda)
    _need(isinstance(v, torch.Tensor) and v.dim() == 4, "v must be a 4-D tensor [B, T, H, dv]")
    _check_tensor(v, "v", (q.dtype,), (B, T, H, v.shape[-1]), dev, require_cuda)
    dv = v.shape[-1]
    _check_tensor(g, "g", (torch.float32,), (B, T, H), dev, require_cuda)
    _check_tensor(beta, "beta", fp, (B, T, H), dev, require_cuda)
    N = B
    if cu_seqlens is not None:
        _need(B == 1, "packed sequences (cu_seqlens) need B == 1")
        _need(isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2,
              "cu_seqlens must be a 1-D tensor of N + 1 offsets")
        N = cu_seqlens.numel() - 1
        _check_tensor(cu_seqlens, "cu_seqlens", (torch.int32, torch.int64), (N + 1,), dev, require_cuda)
        if cu_seqlens_host is not None:
            _need(isinstance(cu_seqlens_host, torch.Tensor) and not cu_seqlens_host.is_cuda and
                  tuple(cu_seqlens_host.shape) == (N + 1,) and
                  cu_seqlens_host.dtype in (torch.int32, torch.int64),
                  "cu_seqlens_host must be a host int32/int64 tensor of N + 1 offsets")
            _need(int(cu_seqlens_host[-1]) == T and int(cu_seqlens_host[0]) == 0,
                  "cu_seqlens_host must start at 0 and end at T")
        if cu_seqlens.dtype == torch.int64:
            cu_seqlens = cu_seqlens.to(torch.int32)
    else:
        _need(cu_seqlens_host is None, "cu_seqlens_host given without cu_seqlens")
    if initial_state is not None:
        _check_tensor(initial_state, "initial_state", (torch.float32,), (N, H, dk, dv), dev, require_cuda)
    if out is not None:
        _check_tensor(out, "out", (q.dtype,), (B, T, H, dv), dev, require_cuda)
    if final_state_out is not None:
        _check_tensor(final_state_out, "final_state_out", (torch.float32,), (N, H, dk, dv), dev,
                      require_cuda)
    if workspace is not None:
        _need(isinstance(workspace, torch.Tensor) and workspace.dtype == torch.uint8 and
              workspace.dim() == 1 and workspace.is_contiguous() and workspace.device == dev,
              "workspace must be a contiguous 1-D uint8 tensor on the inputs' device")
    return cu_seqlens


def check_gate_args(g, cu_seqlens=None, require_cuda=True):
    """Checks the gate scan's arguments (g fp32 [B, T, H]); returns int32 cu_seqlens."""
    _need(isinstance(g, torch.Tensor) and g.dim() == 3, "g must be a 3-D tensor [B, T, H]")
    B, T, H = g.shape
    _check_tensor(g, "g", (torch.float32,), (B, T, H), None, require_cuda)
    if cu_seqlens is not None:
        _need(B == 1, "packed sequences (cu_seqlens) need B == 1")
        _need(isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2,
              "cu_seqlens must be a 1-D tensor of N + 1 offsets")
        _check_tensor(cu_seqlens, "cu_seqlens", (torch.int32, torch.int64), (cu_seqlens.numel(),), g.device,
                      require_cuda)
        if cu_seqlens.dtype == torch.int64:
            cu_seqlens = cu_seqlens.to(torch.int32)
    return cu_seqlens


def check_inverse_args(k, g, beta, cu_seqlens=None, require_cuda=True):
    """Checks gdn_chunk_inverse's arguments (k [B, T, H, dk] bf16/fp32, g fp32 and beta
    bf16/fp32 [B, T, H]); returns int32 cu_seqlens."""
    _need(isinstance(k, torch.Tensor) and k.dim() == 4, "k must be a 4-D tensor [B, T, H, dk]")
    B, T, H, dk = k.shape
    _check_tensor(k, "k", (torch.bfloat16, torch.float32), (B, T, H, dk), None, require_cuda)
    _check_tensor(g, "g", (torch.float32,), (B, T, H), k.device, require_cuda)
    _check_tensor(beta, "beta", (torch.bfloat16, torch.float32), (B, T, H), k.device, require_cuda)
    return check_gate_args(g, cu_seqlens, require_cuda)


class _Shape:
    """Builds a GdnShape and keeps the host cu_seqlens buffer alive."""

    def __init__(self, q, v, beta, cu_seqlens, cu_seqlens_host):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        self.cu_host = None
        N = B
        if cu_seqlens is not None:
            host = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.to("cpu")
            self.cu_host = host.to(torch.int32).contiguous()
            N = self.cu_host.numel() - 1
        self.s = GdnShape(B, T, H, dk, dv, N, _dtype_code(q), _dtype_code(beta),
                          None if self.cu_host is None else
                          ctypes.cast(self.cu_host.data_ptr(), ctypes.POINTER(ctypes.c_int32)))
        self.N = N

    def ref(self):
        return ctypes.byref(self.s)


def workspace_bytes(q, v, beta, cu_seqlens=None, cu_seqlens_host=None, opts=None) -> int:
    sh = _Shape(q, v, beta, cu_seqlens, cu_seqlens_host)
    n = ctypes.c_size_t(0)
    rc = lib().gdn_chunk_fwd_workspace_bytes(sh.ref(), None if opts is None else ctypes.byref(opts),
                                             ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_workspace_bytes")
    return int(n.value)


def chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None,
              output_final_state=True, opts: Optional[GdnOpts] = None, cu_seqlens_host=None,
              out=None, final_state_out=None, workspace=None, stage=None):
    """GDN chunked forward.  Returns ``(o, final_state)`` (final_state None if not requested).

    Layouts follow include/gdn.h: q, k [B,T,H,dk]; v [B,T,H,dv]; g, beta [B,T,H];
    initial_state / final_state [N,H,dk,dv] fp32; cu_seqlens int32 [N+1] on the device
    (B == 1).  ``cu_seqlens_host`` avoids a device-to-host copy of cu_seqlens.
    """
    cu_seqlens = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                    out, final_state_out, workspace)
    sh = _Shape(q, v, beta, cu_seqlens, cu_seqlens_host)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    o = out if out is not None else torch.empty_like(v)
    fs = None
    if output_final_state:
        fs = final_state_out if final_state_out is not None else torch.empty(
            (sh.N, H, dk, dv), dtype=torch.float32, device=q.device)
    opts_ref = None if opts is None else ctypes.byref(opts)
    n = ctypes.c_size_t(0)
    rc = lib().gdn_chunk_fwd_workspace_bytes(sh.ref(), opts_ref, ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_workspace_bytes")
    if workspace is None or workspace.numel() < n.value:
        if stage is not None:
            raise ValueError("a stage call needs the caller's workspace (workspace_bytes())")
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            ctypes.c_float(scale), _ptr(o), _ptr(fs), sh.ref(), opts_ref, _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(q.device))
    if stage is None:
        rc = lib().gdn_chunk_fwd(*args)
    else:
        rc = lib().gdn_chunk_fwd_stage(ctypes.c_int(stage), *args)
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd" if stage is None else "gdn_chunk_fwd_stage")
    return o, fs


def chunk_fwd_noalloc(q, k, v, g, beta, out, final_state_out=None, initial_state=None,
                      cu_seqlens=None, scale=None, opts: Optional[GdnOpts] = None,
                      cu_seqlens_host=None):
    """chunk_fwd through gdn_chunk_fwd_noalloc: the library takes its scratch from its
    built-in device array (GDN_NOALLOC_SCRATCH_BYTES per GPU) and allocates nothing;
    the caller passes the outputs (``out``, and ``final_state_out`` or None).  Calls that
    may overlap on one GPU share that array and must be serialised (one stream is
    enough).  Returns ``(out, final_state_out)``."""
    cu_seqlens = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                    out, final_state_out)
    _need(out is not None, "chunk_fwd_noalloc needs out=")
    sh = _Shape(q, v, beta, cu_seqlens, cu_seqlens_host)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    rc = lib().gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                     _ptr(cu_seqlens), ctypes.c_float(scale), _ptr(out),
                                     _ptr(final_state_out), sh.ref(),
                                     None if opts is None else ctypes.byref(opts), _stream(q.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_noalloc")
    return out, final_state_out


def chunk_fwd_stage(stage, q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None,
                    opts: Optional[GdnOpts] = None, cu_seqlens_host=None, out=None,
                    final_state_out=None, workspace=None):
    """One stage (GDN_STAGE_*) of chunk_fwd on the caller's workspace and outputs; the
    stages run in order give chunk_fwd's result (include/gdn.h, gdn_chunk_fwd_stage)."""
    if out is None or workspace is None:
        raise ValueError("chunk_fwd_stage needs out= and workspace= (shared by all stages)")
    return chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens, scale,
                     output_final_state=final_state_out is not None, opts=opts,
                     cu_seqlens_host=cu_seqlens_host, out=out, final_state_out=final_state_out,
                     workspace=workspace, stage=stage)


def workspace_region(q, v, beta, region, cu_seqlens=None, cu_seqlens_host=None, opts=None):
    """(offset, bytes) of a GDN_REGION_* inside chunk_fwd's workspace."""
    sh = _Shape(q, v, beta, cu_seqlens, cu_seqlens_host)
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = lib().gdn_chunk_fwd_workspace_region(sh.ref(), None if opts is None else ctypes.byref(opts),
                                              ctypes.c_int(region), ctypes.byref(off), ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_fwd_workspace_region")
    return int(off.value), int(n.value)


def chunk_inverse(k, g, beta, cu_seqlens=None, cu_seqlens_host=None):
    """Step 1 alone: returns T [total_chunks, H, 64, 64] in k's dtype."""
    cu_seqlens = check_inverse_args(k, g, beta, cu_seqlens)
    sh = _Shape(k, k, beta, cu_seqlens, cu_seqlens_host)
    nch = lib().gdn_total_chunks(sh.ref())
    if nch < 0:
        raise GdnError(int(nch), "gdn_total_chunks")
    H = k.shape[2]
    t = torch.empty((nch, H, 64, 64), dtype=k.dtype, device=k.device)
    ws = None
    nbytes = 0
    if cu_seqlens is not None:
        n = ctypes.c_size_t(0)
        lib().gdn_chunk_fwd_workspace_bytes(sh.ref(), None, ctypes.byref(n))
        ws = torch.empty(int(n.value), dtype=torch.uint8, device=k.device)
        nbytes = ws.numel()
    rc = lib().gdn_chunk_inverse(_ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), sh.ref(), _ptr(t),
                                 _ptr(ws), ctypes.c_size_t(nbytes), _stream(k.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_inverse")
    return t


def gate_scan(g, cu_seqlens=None, cu_seqlens_host=None, opts: Optional[GdnOpts] = None):
    """The gate scan alone: int32 [N, H] lookback windows (0 = none)."""
    cu_seqlens = check_gate_args(g, cu_seqlens)
    B, T, H = g.shape
    fake_q = torch.empty((B, T, H, 64), dtype=torch.bfloat16, device="meta")
    sh = _Shape(fake_q, fake_q, g, cu_seqlens, cu_seqlens_host)
    sh.s.dk = 64
    sh.s.dv = 64
    sh.s.qkv_dtype = GDN_BF16
    sh.s.beta_dtype = GDN_F32
    n = ctypes.c_size_t(0)
    rc = lib().gdn_gate_scan_workspace_bytes(sh.ref(), ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_gate_scan_workspace_bytes")
    ws = torch.empty(int(n.value), dtype=torch.uint8, device=g.device)
    out = torch.empty((sh.N, H), dtype=torch.int32, device=g.device)
    rc = lib().gdn_gate_scan(_ptr(g), _ptr(cu_seqlens), sh.ref(),
                             None if opts is None else ctypes.byref(opts), _ptr(out), _ptr(ws),
                             ctypes.c_size_t(ws.numel()), _stream(g.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_gate_scan")
    return out


def plan_segment_chunks(q, v, beta, cu_seqlens_host=None, opts: Optional[GdnOpts] = None) -> int:
    """Segment length (chunks) the planner picks; >= the longest sequence's chunks = no split."""
    cu = None if cu_seqlens_host is None else cu_seqlens_host
    sh = _Shape(q, v, beta, cu, cu_seqlens_host)
    r = lib().gdn_plan_segment_chunks(sh.ref(), None if opts is None else ctypes.byref(opts))
    if r < 0:
        raise GdnError(int(r), "gdn_plan_segment_chunks")
    return int(r)


def plan_one_pass(q, v, beta, cu_seqlens_host=None, opts: Optional[GdnOpts] = None) -> bool:
    """Whether gdn_chunk_fwd runs the one-pass forward (chunk inverses formed inside the
    forward kernel) for these inputs and options."""
    sh = _Shape(q, v, beta, cu_seqlens_host, cu_seqlens_host)
    r = lib().gdn_plan_one_pass(sh.ref(), None if opts is None else ctypes.byref(opts))
    if r < 0:
        raise GdnError(int(r), "gdn_plan_one_pass")
    return bool(r)


def chunk_bwd(q, k, v, g, beta, do, initial_state=None, d_final_state=None, cu_seqlens=None, scale=None,
              cu_seqlens_host=None, want_d_initial_state=True, workspace=None, opts: Optional[GdnOpts] = None):
    """Backward of chunk_fwd: the gradients of <do, o> + <d_final_state, final_state>.
    Returns ``(dq, dk, dv, dg, dbeta, d_initial_state)`` (the last None unless wanted);
    dq, dk, dv in q's dtype, dg fp32, dbeta in beta's dtype, d_initial_state fp32
    [N, H, dk, dv].  d_final_state None means zero.  opts: the split of the reverse
    sweep (force_segment_chunks, no_split)."""
    cu_seqlens = check_forward_args(q, k, v, g, beta, initial_state, cu_seqlens, cu_seqlens_host,
                                    None, d_final_state, None)
    _check_tensor(do, "do", (q.dtype,), tuple(v.shape), q.device, True)
    sh = _Shape(q, v, beta, cu_seqlens, cu_seqlens_host)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, db = torch.empty_like(g), torch.empty_like(beta)
    dh0 = torch.empty((sh.N, H, dk, dv), dtype=torch.float32, device=q.device) if want_d_initial_state else None
    n = ctypes.c_size_t(0)
    oref = None if opts is None else ctypes.byref(opts)
    rc = lib().gdn_chunk_bwd_workspace_bytes(sh.ref(), oref, ctypes.byref(n))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_bwd_workspace_bytes")
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(max(int(n.value), 1), dtype=torch.uint8, device=q.device)
    rc = lib().gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                             _ptr(cu_seqlens), ctypes.c_float(scale), _ptr(do), _ptr(d_final_state),
                             _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dh0), sh.ref(), oref,
                             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(q.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_chunk_bwd")
    return dq, dkk, dvv, dg, db, dh0


def plan_predict_us(q, v, beta, cu_seqlens_host=None, opts: Optional[GdnOpts] = None,
                    corrected_fraction=0.0) -> float:
    """The planner's modelled time (microseconds) of one chunk_fwd call for these inputs,
    with the given share of (sequence, head) pairs that take no lookback window."""
    sh = _Shape(q, v, beta, cu_seqlens_host, cu_seqlens_host)
    us = ctypes.c_double(0.0)
    rc = lib().gdn_plan_predict_us(sh.ref(), None if opts is None else ctypes.byref(opts),
                                   ctypes.c_double(corrected_fraction), ctypes.byref(us))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_plan_predict_us")
    return float(us.value)
