"""Plain, slow, obviously-correct CPU oracle for the Gated DeltaNet chunked forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  It
shares no code with the HIP library (``gated_deltanet_chunked_fwd_amd``) and never
imports it; the two meet only through the seeded input generators, which hold
none of the method's arithmetic.

Contents
  token      -- Oracle A: fp64 token-by-token recurrence (plain C via ctypes, plus a
                numpy twin used to check the C build on tiny inputs), and the
                magnitude scale*|S_t||q_t| of every output's inner product (the
                scale an output's rounding error is judged against when that inner
                product cancels).
  chunked    -- Oracle B: fp64 chunk-by-chunk WY form written from the pages' four
                steps, its algebraic variants, the sequence-parallel correction
                (wrong-start state S*, correction matrix M, merge) and the
                window-lookback start.
  gate       -- brute-force window-length decision for strongly decaying heads.
  backward   -- fp64 gradients of <dO, O> + <dhT, hT> with respect to q, k, v, g, beta
                and the initial state: the token-by-token adjoint of the recurrence,
                and separately the chunk-by-chunk backward of the WY form (with the
                DA + DA^T merge of the pages' algebraic-rewrites section).
  build      -- compiles the C part with gcc.

Every function cites the passage of the pages it follows.  The pages are three
web articles on FlashQLA; the primary one is the AICon talk transcript
"Qwen系列模型线性注意力高性能优化实践" (tokendh.com).
"""
from .token import output_magnitude_numpy, token_recurrence, token_recurrence_numpy  # noqa: F401
from .chunked import (  # noqa: F401
    chunk_inverse,
    chunked_forward,
    cp_forward,
    window_forward,
    segment_transition,
)
from .gate import segment_windows, window_chunks, window_chunks_all  # noqa: F401
from .backward import chunked_backward, token_backward_numpy  # noqa: F401
