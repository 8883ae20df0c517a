"""CPU-side checks of the C boundary: the library loads, exports every symbol
include/gdn.h declares, and rejects bad arguments before any HIP call (no GPU is
touched: every case here fails validation)."""
import ctypes
import os
import re

import pytest

from gated_deltanet_chunked_fwd_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(gdn_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_symbols()
    assert "gdn_chunk_fwd" in names and "gdn_chunk_fwd_workspace_bytes" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == set(names)


def shape(**kw):
    d = dict(B=1, T=128, H=2, dk=128, dv=128, N=1, qkv_dtype=B.GDN_BF16, beta_dtype=B.GDN_BF16,
             cu_seqlens_host=None)
    d.update(kw)
    return B.GdnShape(**d)


def ws_bytes(s, opts=None):
    n = ctypes.c_size_t(0)
    rc = B.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(s), None if opts is None else ctypes.byref(opts),
                                               ctypes.byref(n))
    return rc, n.value


def test_workspace_query():
    two_kernel = B.make_opts(one_pass=-1)
    rc, n = ws_bytes(shape(), two_kernel)
    assert rc == B.GDN_OK
    assert n >= 2 * 2 * 64 * 64 * 2  # two chunks x two heads of bf16 T
    rc32, n32 = ws_bytes(shape(qkv_dtype=B.GDN_F32))
    assert rc32 == B.GDN_OK and n32 > n
    # the one-pass forward (the bf16 default) keeps no T, so an unsplit plan needs less
    rc1, n1 = ws_bytes(shape())
    assert rc1 == B.GDN_OK and n1 < 2 * 2 * 64 * 64 * 2


def test_plan_one_pass_query():
    lib = B.lib()
    assert lib.gdn_plan_one_pass(ctypes.byref(shape()), None) == 1
    assert lib.gdn_plan_one_pass(ctypes.byref(shape(qkv_dtype=B.GDN_F32, beta_dtype=B.GDN_F32)), None) == 0
    for kw, want in [(dict(one_pass=-1), 0), (dict(one_pass=1), 1), (dict(value_block=64), 0),
                     (dict(value_block=128), 0), (dict(one_pass=1, value_block=64), 1)]:
        o = B.make_opts(**kw)
        assert lib.gdn_plan_one_pass(ctypes.byref(shape()), ctypes.byref(o)) == want, kw
    # fp32 has no one-pass kernel: forcing it still plans two kernels
    o = B.make_opts(one_pass=1)
    assert lib.gdn_plan_one_pass(ctypes.byref(shape(qkv_dtype=B.GDN_F32, beta_dtype=B.GDN_F32)),
                                 ctypes.byref(o)) == 0
    for bad in [dict(one_pass=2), dict(one_pass=-2), dict(value_block=32)]:
        o = B.make_opts(**bad)
        assert lib.gdn_plan_one_pass(ctypes.byref(shape()), ctypes.byref(o)) == B.GDN_ERR_ARG, bad


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), B.GDN_ERR_UNSUPPORTED),
    (dict(dv=32), B.GDN_ERR_UNSUPPORTED),
    (dict(qkv_dtype=7), B.GDN_ERR_UNSUPPORTED),
    (dict(H=0), B.GDN_ERR_ARG),
    (dict(T=-1), B.GDN_ERR_ARG),
    (dict(N=2), B.GDN_ERR_ARG),          # dense layout needs N == B
])
def test_bad_shapes_rejected(kw, code):
    rc, _ = ws_bytes(shape(**kw))
    assert rc == code


def test_bad_cu_seqlens_rejected():
    for vals, N, T in [([0, 10, 5], 2, 5), ([1, 10], 1, 10), ([0, 10], 1, 11)]:
        arr = (ctypes.c_int32 * len(vals))(*vals)
        s = shape(T=T, N=N, cu_seqlens_host=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        assert ws_bytes(s)[0] == B.GDN_ERR_ARG
    arr = (ctypes.c_int32 * 3)(0, 10, 30)
    s = shape(B=2, T=30, N=2, cu_seqlens_host=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    assert ws_bytes(s)[0] == B.GDN_ERR_ARG   # packed needs B == 1


def test_forward_rejects_before_launch():
    lib = B.lib()
    s = shape()
    fake = ctypes.c_void_p(4096)        # never dereferenced: validation fails first
    mis = ctypes.c_void_p(4096 + 2)
    args = [fake] * 5 + [None, None, ctypes.c_float(0.1), fake, None, ctypes.byref(s), None]
    # null q
    a = list(args); a[0] = None
    assert lib.gdn_chunk_fwd(*a, fake, ctypes.c_size_t(1 << 30), None) == B.GDN_ERR_ARG
    # misaligned v
    a = list(args); a[2] = mis
    assert lib.gdn_chunk_fwd(*a, fake, ctypes.c_size_t(1 << 30), None) == B.GDN_ERR_ARG
    # workspace too small
    assert lib.gdn_chunk_fwd(*args, fake, ctypes.c_size_t(16), None) == B.GDN_ERR_WORKSPACE
    # non-finite scale
    a = list(args); a[7] = ctypes.c_float(float("nan"))
    assert lib.gdn_chunk_fwd(*a, fake, ctypes.c_size_t(1 << 30), None) == B.GDN_ERR_ARG
    # device cu_seqlens without the host copy
    a = list(args); a[6] = fake
    assert lib.gdn_chunk_fwd(*a, fake, ctypes.c_size_t(1 << 30), None) == B.GDN_ERR_ARG


def test_status_strings():
    assert B.status_str(0) == "ok"
    assert "workspace" in B.status_str(B.GDN_ERR_WORKSPACE)
    assert B.status_str(12345) == "unknown status"


def plan_L(s, opts=None):
    return B.lib().gdn_plan_segment_chunks(ctypes.byref(s), None if opts is None else ctypes.byref(opts))


def test_plan_cache_follows_packed_lengths_and_options():
    """Plans are memoised per thread; a changed packed length (same buffer, same N and
    T), a different option or a sixth shape must never return a stale plan."""
    T = 8192 * 64
    a = (ctypes.c_int32 * 3)(0, T // 2, T)            # two equal sequences
    b_vals = (0, 64 * 16, T)                           # one short, one long
    b = (ctypes.c_int32 * 3)(*b_vals)
    sa = shape(T=T, N=2, H=4, cu_seqlens_host=ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)))
    sb = shape(T=T, N=2, H=4, cu_seqlens_host=ctypes.cast(b, ctypes.POINTER(ctypes.c_int32)))
    la, lb = plan_L(sa), plan_L(sb)
    assert la > 0 and lb > 0 and la != lb
    n_a = ws_bytes(sa)[1]
    for i, v in enumerate(b_vals):   # same pointer, new contents
        a[i] = v
    assert plan_L(sa) == lb and ws_bytes(sa)[1] == ws_bytes(sb)[1]
    a[1] = T // 2
    assert plan_L(sa) == la and ws_bytes(sa)[1] == n_a
    forced = B.make_opts(force_segment_chunks=7)
    assert plan_L(sa, forced) == 7 and plan_L(sa) == la
    assert plan_L(sa, B.make_opts(no_split=1)) > 8192 and plan_L(sa) == la
    # more distinct shapes than cache entries, twice round: answers stay the same
    shapes = [shape(T=64 * n, H=h) for n, h in [(300, 1), (700, 2), (1500, 1), (4000, 1), (9000, 1),
                                                 (20000, 1)]]
    first = [plan_L(s) for s in shapes]
    assert [plan_L(s) for s in shapes] == first
    assert [plan_L(s) for s in reversed(shapes)] == list(reversed(first))



@pytest.mark.parametrize("L", [2, 3, 5, 100])
def test_forced_segment_length_without_a_split_plans_one_segment(L):
    """Packed lengths whose longest sequence has 2 chunks while the packed T spans 5:
    a forced segment length >= 2 splits nothing, and the plan must then carry the
    same one-segment value as no_split (the kernels' decode without segment tables
    divides by it; a value of 2 there made them read 3 segments of one sequence)."""
    cu = (ctypes.c_int32 * 7)(0, 65, 128, 192, 193, 194, 258)
    s = shape(T=258, N=6, H=1, cu_seqlens_host=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)))
    unsplit = plan_L(s, B.make_opts(no_split=1))
    assert unsplit >= 5
    assert plan_L(s, B.make_opts(force_segment_chunks=L)) == unsplit
    assert plan_L(s, B.make_opts(force_segment_chunks=L, force_correction=1)) == unsplit
    assert plan_L(s, B.make_opts(force_segment_chunks=1)) == 1
    dense = shape(T=64 * 5, H=1)
    assert plan_L(dense, B.make_opts(force_segment_chunks=5)) == plan_L(dense, B.make_opts(no_split=1))


@pytest.mark.parametrize("seed", range(6))
def test_unsplit_plans_report_the_one_segment_value(seed):
    """Random packed and dense shapes with random forced lengths: a plan that splits
    nothing (value at or above the longest sequence's chunk count) reports exactly
    the one-segment value, and a forced length below it is kept as given."""
    import numpy as np
    rng = np.random.default_rng(500 + seed)
    one = 1073741823
    for _ in range(60):
        if rng.random() < 0.6:
            lens = [int(x) for x in rng.choice([0, 1, 40, 64, 65, 130, 700, 2000], size=int(rng.integers(1, 9)))]
            if sum(lens) == 0:
                lens[0] = 65
            cu = (ctypes.c_int32 * (len(lens) + 1))(0, *np.cumsum(lens).tolist())
            s = shape(T=sum(lens), N=len(lens), H=int(rng.integers(1, 5)),
                      cu_seqlens_host=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)))
            longest = max((n + 63) // 64 for n in lens)
        else:
            T = int(rng.integers(1, 64 * 40))
            Bn = int(rng.integers(1, 4))
            s = shape(T=T, B=Bn, N=Bn, H=int(rng.integers(1, 5)))
            longest = (T + 63) // 64
        L = int(rng.integers(1, 50))
        got = plan_L(s, B.make_opts(force_segment_chunks=L, force_correction=int(rng.random() < 0.5)))
        assert got == (L if L < longest else one), (L, longest, got)
        assert plan_L(s, B.make_opts(no_split=1)) == one
        assert plan_L(s) == one or 1 <= plan_L(s) < longest

def region(s, r, opts=None):
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    rc = B.lib().gdn_chunk_fwd_workspace_region(ctypes.byref(s), None if opts is None else ctypes.byref(opts),
                                                r, ctypes.byref(off), ctypes.byref(n))
    return rc, off.value, n.value


def test_workspace_regions():
    """The stage-connecting regions lie inside the workspace, 256-byte aligned and
    disjoint, with the sizes their layouts imply; the segment regions are empty when
    nothing is split, the chunk-inverse region on one-pass plans (the one-pass kernel
    forms T itself, in pass 1 too); unknown regions and stages are rejected before any
    launch."""
    T, H, d = 64 * 14 + 23, 3, 128
    s = shape(T=T, H=H, dk=d, dv=d)
    split = B.make_opts(force_segment_chunks=3)
    total = ctypes.c_size_t(0)
    assert B.lib().gdn_chunk_fwd_workspace_bytes(ctypes.byref(s), ctypes.byref(split), ctypes.byref(total)) == 0
    chunks, segs = 15, 5
    want = {B.GDN_REGION_CHUNK_INVERSE: 0, B.GDN_REGION_SEGMENT_WINDOWS: segs * H * 4,
            B.GDN_REGION_SEGMENT_STARTS: segs * H * d * d * 4}
    spans = []
    for r in range(B.GDN_NUM_REGIONS):
        rc, off, n = region(s, r, split)
        assert rc == B.GDN_OK and off % 256 == 0 and off + n <= total.value
        assert (n == 0) == (r == B.GDN_REGION_CHUNK_INVERSE), r
        if r in want:
            assert n == want[r], r
        if n:
            spans.append((off, off + n))
    two_kernel = B.make_opts(force_segment_chunks=3, one_pass=-1)
    assert region(s, B.GDN_REGION_CHUNK_INVERSE, two_kernel)[2] == chunks * H * 64 * 64 * 2
    rc, off, n = region(s, B.GDN_REGION_SEGMENT_MAPS, split)
    # S* (fp32) then M (2 x bf16) per slot, M at the next 256-byte boundary
    smap = segs * H * d * d * 4
    assert n == -(-smap // 256) * 256 + segs * H * 2 * d * d * 2
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    unsplit = B.make_opts(no_split=1)
    for r in (B.GDN_REGION_SEGMENT_WINDOWS, B.GDN_REGION_SEGMENT_MAPS, B.GDN_REGION_SEGMENT_STARTS):
        assert region(s, r, unsplit) == (B.GDN_OK, 0, 0)
    assert region(s, B.GDN_NUM_REGIONS)[0] == B.GDN_ERR_ARG
    assert region(s, -1)[0] == B.GDN_ERR_ARG
    fake = ctypes.c_void_p(4096)
    args = [fake] * 5 + [None, None, ctypes.c_float(0.1), fake, None, ctypes.byref(s), None,
            fake, ctypes.c_size_t(1 << 40), None]
    for bad in (-1, B.GDN_NUM_STAGES):
        assert B.lib().gdn_chunk_fwd_stage(bad, *args) == B.GDN_ERR_ARG


def test_oversized_launch_grids_rejected_before_any_launch():
    """2^20 one-token packed sequences x 128 heads: the unsplit forward would need
    2^27 units x 512 threads, beyond a dispatch's 2^32 - 1 work-items; the call must
    fail with GDN_ERR_UNSUPPORTED before anything is enqueued (fake pointers: any
    launch would fault, validation must stop it first)."""
    N, H = 1 << 20, 128
    cu = (ctypes.c_int32 * (N + 1))(*range(N + 1))
    s = shape(T=N, N=N, H=H, cu_seqlens_host=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)))
    fake = ctypes.c_void_p(4096)
    opts = B.make_opts(no_split=1)
    args = [fake] * 5 + [None, fake, ctypes.c_float(0.1), fake, None, ctypes.byref(s), ctypes.byref(opts),
            fake, ctypes.c_size_t(1 << 62), None]
    assert B.lib().gdn_chunk_fwd(*args) == B.GDN_ERR_UNSUPPORTED
    small = shape(T=N, N=N, H=2, cu_seqlens_host=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)))
    assert ws_bytes(small)[0] == B.GDN_OK   # the same sequences with few heads are fine


def test_noalloc_rejects_problem_beyond_scratch_before_any_launch():
    """gdn_chunk_fwd_noalloc refuses a problem whose workspace exceeds the built-in
    scratch (GDN_ERR_SCRATCH) before it touches a pointer or the device."""
    lib = B.lib()
    s = shape(B=1, T=1 << 22, H=16, N=1)
    need = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(s), None, ctypes.byref(need)) == B.GDN_OK
    assert need.value > B.GDN_NOALLOC_SCRATCH_BYTES
    rc = lib.gdn_chunk_fwd_noalloc(None, None, None, None, None, None, None, ctypes.c_float(1.0), None, None,
                                   ctypes.byref(s), None, None)
    assert rc == B.GDN_ERR_SCRATCH
    assert "scratch" in lib.gdn_status_str(rc).decode()
