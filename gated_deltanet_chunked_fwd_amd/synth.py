"""Seeded synthetic inputs for the GDN chunked forward.

This module holds no part of the method's arithmetic: it only draws random
tensors, normalises keys/queries, forms the stored log-gates and rounds to the
storage dtype.  Both the HIP path and the CPU oracle consume what it returns.

Recipe (the same for every workload; numbers are the workload table below):
  * generator ``numpy.random.Generator(PCG64(seed))``; draw order:
    (packed lengths) -> q -> k -> v -> gate variable -> beta variable -> h0;
  * normals are float32, drawn in C order of [B, T, H, D] / [B, T, H] / [N, H, dk, dv];
  * q and k are L2-normalised per (token, head) in float32, then cast;
  * sigmoid gates: x ~ N(mu, 1), g = log(sigmoid(x)) = -log1p(exp(-x)) in fp64, stored fp32;
    uniform gates: alpha ~ U[lo, hi] (fp64), g = log(alpha), stored fp32;
  * beta = sigmoid(y), y ~ N(0, 1);
  * bf16 casts are round-to-nearest-even (torch on the CPU);
  * packed lengths: draw n-1 ints uniform in [lo, hi], set the last to total - sum,
    accept if it is in [lo, hi], else redraw.

The pages (FlashQLA) benchmark Qwen3.5/3.6-series layer shapes with 8-128 GDN heads
and trained gates; no dataset is involved.  These workloads stand in for them.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass
class Spec:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str = "bf16"            # storage dtype of q, k, v, o ("bf16" or "f32")
    beta_dtype: Optional[str] = None  # defaults to dtype
    gate: str = "sigmoid"          # "sigmoid" | "uniform" | "zero"
    gate_mu: float = 3.0
    gate_lo: float = 0.80
    gate_hi: float = 0.95
    zero_gate_heads: tuple = ()    # heads whose g is overwritten with exact 0
    packed: Optional[tuple] = None  # (n_seqs, lo, hi): lengths summing to T
    h0_std: Optional[float] = None  # None -> zero initial state (h0 = None)
    seed: int = 0
    normalize_qk: bool = True
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads.  Seeds are the workload numbers.
WORKLOADS = {
    1: Spec("tiny_fp32_T256_H1_d64", B=1, T=256, H=1, dk=64, dv=64, dtype="f32", seed=1),
    2: Spec("qwen_like_B4_T4096_H16_d128", B=4, T=4096, H=16, dk=128, dv=128, seed=2),
    3: Spec("varlen_8seq_T32768_H32_d128", B=1, T=32768, H=32, dk=128, dv=128,
            packed=(8, 512, 8192), h0_std=0.02, seed=3),
    4: Spec("long_B1_T131072_H4_d128", B=1, T=131072, H=4, dk=128, dv=128,
            zero_gate_heads=(3,), seed=4),
    5: Spec("strong_gate_B2_T65536_H8_d128", B=2, T=65536, H=8, dk=128, dv=128,
            gate="uniform", seed=5),
}


def packed_lengths(rng, n, lo, hi, total):
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)


def _cast(x32: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def _l2n(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def generate(spec: Spec, seed: Optional[int] = None) -> dict:
    """Returns CPU torch tensors: q, k, v, g, beta, h0 (or None), cu_seqlens (int32
    or None), plus ``scale``, ``N`` and the spec."""
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    B, T, H, dk, dv = spec.B, spec.T, spec.H, spec.dk, spec.dv
    cu = None
    N = B
    if spec.packed is not None:
        n, lo, hi = spec.packed
        assert B == 1
        lens = packed_lengths(rng, n, lo, hi, T)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        N = n
    q = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    k = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    if spec.normalize_qk:
        q, k = _l2n(q), _l2n(k)
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    if spec.gate == "sigmoid":
        x = rng.standard_normal((B, T, H), dtype=np.float32).astype(np.float64) + spec.gate_mu
        g = (-np.log1p(np.exp(-x))).astype(np.float32)
    elif spec.gate == "uniform":
        a = rng.uniform(spec.gate_lo, spec.gate_hi, size=(B, T, H))
        g = np.log(a).astype(np.float32)
    elif spec.gate == "zero":
        g = np.zeros((B, T, H), dtype=np.float32)
    else:
        raise ValueError(spec.gate)
    for hh in spec.zero_gate_heads:
        g[:, :, hh] = 0.0
    y = rng.standard_normal((B, T, H), dtype=np.float32).astype(np.float64)
    beta = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)
    h0 = None
    if spec.h0_std is not None:
        h0 = (rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(spec.h0_std))
    bdt = spec.beta_dtype or spec.dtype
    return dict(
        q=_cast(q, spec.dtype), k=_cast(k, spec.dtype), v=_cast(v, spec.dtype),
        g=torch.from_numpy(g), beta=_cast(beta, bdt),
        h0=None if h0 is None else torch.from_numpy(h0),
        cu_seqlens=None if cu is None else torch.from_numpy(cu),
        scale=dk ** -0.5, N=N, spec=spec,
    )


def workload(i: int, **overrides) -> Spec:
    """A copy of workload ``i``'s spec with fields overridden (e.g. a shorter T)."""
    import dataclasses
    return dataclasses.replace(WORKLOADS[i], **overrides)


def as_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact fp64 upcast of a stored tensor, as a numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
