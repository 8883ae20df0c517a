"""ctypes declarations of the C ABI in include/gdn.h: constants, the gdn_shape and
gdn_opts structs and the entry points' argument types.  No torch: the binding and
host-only tools (the sanitizer driver of the tests) share it."""
import ctypes

GDN_OK, GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 0, -1, -2, -3, -4
GDN_ERR_SCRATCH = -5
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/gdn.h
GDN_BF16, GDN_F32 = 1, 2

# Symbols declared in include/gdn.h (checked by the CPU test of the boundary).
EXPORTS = ("gdn_chunk_fwd", "gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd_stage",
           "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes",
           "gdn_chunk_fwd_noalloc",
           "gdn_chunk_fwd_workspace_region", "gdn_chunk_inverse",
           "gdn_gate_scan", "gdn_gate_scan_workspace_bytes", "gdn_plan_segment_chunks", "gdn_plan_one_pass", "gdn_plan_predict_us",
           "gdn_total_chunks", "gdn_status_str")


class GdnShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("N", ctypes.c_int64),
                ("qkv_dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32),
                ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32))]


class GdnOpts(ctypes.Structure):
    _fields_ = [("no_split", ctypes.c_int32), ("force_segment_chunks", ctypes.c_int32),
                ("force_correction", ctypes.c_int32), ("window_log_eps", ctypes.c_float),
                ("window_max_chunks", ctypes.c_int32), ("lambda1_us", ctypes.c_float),
                ("lambda2_us", ctypes.c_float), ("value_block", ctypes.c_int32),
                ("one_pass", ctypes.c_int32), ("stage_events", ctypes.c_void_p)]


GDN_STAGE_INVERSE, GDN_STAGE_GATE_SCAN, GDN_STAGE_CP_PASS1, GDN_STAGE_CP_MERGE = 0, 1, 2, 3
GDN_STAGE_FORWARD, GDN_NUM_STAGES = 4, 5
GDN_REGION_CHUNK_INVERSE, GDN_REGION_SEGMENT_WINDOWS, GDN_REGION_SEGMENT_MAPS = 0, 1, 2
GDN_REGION_SEGMENT_STARTS, GDN_NUM_REGIONS = 3, 4
STAGE_NAMES = ("chunk_inverse", "gate_scan", "cp_pass1", "cp_merge", "fused_forward")


def declare(lib):
    """Sets the argument and result types of every entry point on a loaded library."""
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    shp, opt = ctypes.POINTER(GdnShape), ctypes.POINTER(GdnOpts)
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [shp, opt, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_int
    lib.gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, shp, opt,
                                  vp, sz, vp]
    lib.gdn_chunk_fwd.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, shp,
                                          opt, vp]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_stage.argtypes = [ctypes.c_int] + lib.gdn_chunk_fwd.argtypes
    lib.gdn_chunk_fwd_stage.restype = ctypes.c_int
    lib.gdn_chunk_fwd_workspace_region.argtypes = [shp, opt, ctypes.c_int, ctypes.POINTER(sz),
                                                   ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_workspace_region.restype = ctypes.c_int
    lib.gdn_chunk_inverse.argtypes = [vp, vp, vp, vp, shp, vp, vp, sz, vp]
    lib.gdn_chunk_inverse.restype = ctypes.c_int
    lib.gdn_gate_scan.argtypes = [vp, vp, shp, opt, vp, vp, sz, vp]
    lib.gdn_gate_scan.restype = ctypes.c_int
    lib.gdn_gate_scan_workspace_bytes.argtypes = [shp, ctypes.POINTER(sz)]
    lib.gdn_gate_scan_workspace_bytes.restype = ctypes.c_int
    lib.gdn_plan_segment_chunks.argtypes = [shp, opt]
    lib.gdn_plan_segment_chunks.restype = ctypes.c_int64
    lib.gdn_chunk_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp,
                                  vp, vp, shp, opt, vp, sz, vp]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [shp, opt, ctypes.POINTER(sz)]
    lib.gdn_chunk_bwd_workspace_bytes.restype = ctypes.c_int
    lib.gdn_plan_predict_us.argtypes = [shp, opt, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
    lib.gdn_plan_predict_us.restype = ctypes.c_int
    lib.gdn_plan_one_pass.argtypes = [shp, opt]
    lib.gdn_plan_one_pass.restype = ctypes.c_int
    lib.gdn_total_chunks.argtypes = [shp]
    lib.gdn_total_chunks.restype = ctypes.c_int64
    lib.gdn_status_str.argtypes = [ctypes.c_int]
    lib.gdn_status_str.restype = ctypes.c_char_p
    return lib


def make_opts(no_split=0, force_segment_chunks=0, force_correction=0, window_log_eps=0.0,
              window_max_chunks=0, lambda1_us=0.0, lambda2_us=0.0, value_block=0,
              one_pass=0, stage_events=None) -> GdnOpts:
    return GdnOpts(no_split, force_segment_chunks, force_correction, window_log_eps,
                   window_max_chunks, lambda1_us, lambda2_us, value_block, one_pass,
                   stage_events)
