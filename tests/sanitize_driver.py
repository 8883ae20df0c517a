"""Host-code driver for the sanitizer test (run in a subprocess with the AddressSanitizer
runtime preloaded; imports no torch).

  python tests/sanitize_driver.py abi <libgdn built with host ASan/UBSan>
      plans, workspace sizes and regions over many dense and packed shapes and
      options, the plan cache under in-place changes, and every validation path of
      the entry points with fake device pointers (each call fails before any launch).
  python tests/sanitize_driver.py oracle <liboracle built with ASan/UBSan>
      the C token recurrence on small dense and packed inputs, with 1 and 3 threads.
"""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def abi(path):
    from gated_deltanet_chunked_fwd_amd import abi as A
    lib = A.declare(ctypes.CDLL(path))
    rng = np.random.default_rng(7)
    keep = []

    def shape(B=1, T=1000, H=4, dk=128, dv=128, N=None, dt=A.GDN_BF16, bdt=A.GDN_BF16, lens=None):
        cu = None
        if lens is not None:
            arr = (ctypes.c_int32 * (len(lens) + 1))(*np.concatenate([[0], np.cumsum(lens)]).tolist())
            keep.append(arr)
            cu = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
            N, T = len(lens), int(sum(lens))
        return A.GdnShape(B, T, H, dk, dv, B if N is None else N, dt, bdt, cu)

    n_ok = 0
    for i in range(400):
        packed = rng.random() < 0.5
        kw = dict(H=int(rng.integers(1, 65)), dk=int(rng.choice([64, 128])), dv=int(rng.choice([64, 128])),
                  dt=int(rng.choice([A.GDN_BF16, A.GDN_F32])), bdt=int(rng.choice([A.GDN_BF16, A.GDN_F32])))
        if packed:
            n = int(rng.choice([1, 3, 17, 300, 1100, 2000]))
            kw["lens"] = rng.integers(0, 3000, size=n).tolist()
        else:
            kw.update(B=int(rng.integers(1, 9)), T=int(rng.choice([0, 1, 63, 64, 65, 4096, 131072])))
        s = shape(**kw)
        o = A.make_opts(no_split=int(rng.random() < 0.1), force_segment_chunks=int(rng.choice([0, 0, 1, 3, 16])),
                        force_correction=int(rng.random() < 0.2), window_max_chunks=int(rng.choice([0, 1, 16])),
                        value_block=int(rng.choice([0, 64, 128])), one_pass=int(rng.choice([-1, 0, 1])), lambda1_us=float(rng.choice([0.0, 1.0])),
                        lambda2_us=float(rng.choice([0.0, 5.0])))
        for opts in (None, ctypes.byref(o)):
            nb = ctypes.c_size_t(0)
            assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(s), opts, ctypes.byref(nb)) == A.GDN_OK
            L = lib.gdn_plan_segment_chunks(ctypes.byref(s), opts)
            assert L > 0
            assert lib.gdn_total_chunks(ctypes.byref(s)) >= 0
            for r in range(A.GDN_NUM_REGIONS):
                off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
                assert lib.gdn_chunk_fwd_workspace_region(ctypes.byref(s), opts, r, ctypes.byref(off),
                                                          ctypes.byref(n)) == A.GDN_OK
                assert off.value + n.value <= nb.value
            gb = ctypes.c_size_t(0)
            assert lib.gdn_gate_scan_workspace_bytes(ctypes.byref(s), ctypes.byref(gb)) == A.GDN_OK
            n_ok += 1
        if packed and len(kw["lens"]) > 1:   # the plan cache follows in-place changes
            arr = keep[-1]
            before = lib.gdn_plan_segment_chunks(ctypes.byref(s), None)
            arr[1] = 0
            lib.gdn_plan_segment_chunks(ctypes.byref(s), None)
            arr[1] = int(kw["lens"][0])
            assert lib.gdn_plan_segment_chunks(ctypes.byref(s), None) == before
    # validation paths: fake device pointers, every call must fail before a launch
    fake, mis = ctypes.c_void_p(4096), ctypes.c_void_p(4098)
    s = shape(B=2, T=300, H=3)
    big = ctypes.c_size_t(1 << 40)
    base = [fake] * 5 + [None, None, ctypes.c_float(0.1), fake, None, ctypes.byref(s), None, fake, big, None]
    bad = []
    for idx, val in [(0, None), (1, mis), (2, mis), (3, mis), (8, mis), (7, ctypes.c_float(float("inf"))),
                     (6, fake), (12, None), (13, ctypes.c_size_t(64)), (12, mis)]:
        a = list(base)
        a[idx] = val
        bad.append(a)
    for a in bad:
        assert lib.gdn_chunk_fwd(*a) < 0
        for st in (-1, 0, 4, 5):
            assert lib.gdn_chunk_fwd_stage(st, *a) < 0
    for kw in [dict(dk=96), dict(dv=32), dict(H=0), dict(T=-1), dict(dt=9), dict(N=5)]:
        s2 = shape(**kw)
        nb = ctypes.c_size_t(0)
        assert lib.gdn_chunk_fwd_workspace_bytes(ctypes.byref(s2), None, ctypes.byref(nb)) < 0
        assert lib.gdn_plan_segment_chunks(ctypes.byref(s2), None) < 0
    for opts in [A.make_opts(value_block=96), A.make_opts(value_block=32), A.make_opts(one_pass=2), A.make_opts(force_segment_chunks=-2),
                 A.make_opts(window_max_chunks=17), A.make_opts(window_log_eps=1.0),
                 A.make_opts(lambda1_us=-1.0)]:
        assert lib.gdn_plan_segment_chunks(ctypes.byref(s), ctypes.byref(opts)) < 0
    for vals in ([0, 10, 5], [1, 10], [0, 10]):
        arr = (ctypes.c_int32 * len(vals))(*vals)
        s3 = A.GdnShape(1, 11 if vals == [0, 10] else vals[-1], 2, 128, 128, len(vals) - 1, A.GDN_BF16,
                        A.GDN_BF16, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
        assert lib.gdn_plan_segment_chunks(ctypes.byref(s3), None) < 0
    assert lib.gdn_chunk_inverse(fake, fake, fake, None, ctypes.byref(s), None, None, ctypes.c_size_t(0), None) < 0
    assert lib.gdn_gate_scan(fake, None, ctypes.byref(s), None, None, None, ctypes.c_size_t(0), None) < 0
    for code in (0, -1, -2, -3, -4, 77):
        assert lib.gdn_status_str(code)
    print("abi ok: %d shape/option combinations" % n_ok, flush=True)


def oracle(path):
    lib = ctypes.CDLL(path)
    d = ctypes.POINTER(ctypes.c_double)
    lib.gdn_oracle_token.argtypes = [d, d, d, d, d, d, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, d, d,
                                     ctypes.c_int]
    lib.gdn_oracle_token.restype = ctypes.c_int
    rng = np.random.default_rng(3)
    P = lambda x: x.ctypes.data_as(d)  # noqa: E731
    for lens, H, dk, dv in [([37], 2, 64, 64), ([5, 0, 130, 64], 3, 128, 64), ([200], 1, 64, 128)]:
        T = sum(lens)
        q, k = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((T, H, dv))
        g = -rng.random((T, H)) * 0.1
        b = rng.random((T, H))
        h0 = rng.standard_normal((len(lens), H, dk, dv)) * 0.1
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        outs = []
        for nt in (1, 3):
            o = np.zeros((T, H, dv))
            hT = np.zeros((len(lens), H, dk, dv))
            rc = lib.gdn_oracle_token(P(q), P(k), P(v), P(g), P(b), P(h0),
                                      cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(lens), H, dk, dv,
                                      dk ** -0.5, P(o), P(hT), nt)
            assert rc == 0
            outs.append((o, hT))
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
        assert np.isfinite(outs[0][0]).all()
    print("oracle ok", flush=True)


if __name__ == "__main__":
    {"abi": abi, "oracle": oracle}[sys.argv[1]](sys.argv[2])
