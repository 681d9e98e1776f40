"""CPU oracle for exact softmax attention: TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct fp64 reference that the HIP path
is checked against. It is not part of the product: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with ``exact_tiled_attention_13_amd`` and never
imports it; the two meet only in the seeded input generators, which hold none
of the method's arithmetic.

Sources (web pages on FlashAttention-2; cited by title and section):

* "FlashAttention-2: atención eficiente en GPU para contextos largos"
  (iplexlaw, Spanish), sections "El coste de mover datos en secuencias largas"
  (attention materialises score and probability matrices) and "Bloques
  pequeños, normalización global" (online softmax keeps the global
  normalisation; blockwise-normalise-then-sum is a different computation;
  outputs and gradients are compared within a tolerance).
* "读懂FlashAttention-2：让长上下文注意力更高效地运行在GPU上" (the same article
  in Chinese), section "分块处理仍需保持全局归一化", which calls the method exact
  attention rather than a sparse approximation.

Modules:

* :mod:`oracle.attn_ref` -- the plain definition (forward, LSE and the
  analytic backward) in fp64 numpy, row-chunked.
* :mod:`oracle.online` -- the tile-by-tile online-softmax rewrite the pages
  describe, plus the per-block-normalised negative control.
* :mod:`oracle.brute` -- scalar-loop brute force for tiny inputs, written by a
  different algebraic route, used only to pin :mod:`oracle.attn_ref`.
* :mod:`oracle.gqa` -- grouped-query / multi-query attention (K and V shared
  by groups of query heads; page "FlashAttention-T: Optimización GPU para
  LLMs Escalables", section "Innovaciones técnicas frente a FlashAttention
  original"), defined head by head through :mod:`oracle.attn_ref`.

* :mod:`oracle.decode` -- decoding: a few new query rows against a key/value
  cache (bottom-right causal alignment), the attention restricted to a key
  chunk, and the exact merge of per-chunk (O, LSE) results (split-KV); page
  "FlashAttention-2: atención eficiente en GPU para contextos largos",
  section "Cómo documentar una diferencia técnica", which separates prefill
  from decoding.

* :mod:`oracle.fp8` -- the FP8 (E4M3) forward: the E4M3 rounding and the
  tiled online softmax with 8-bit probabilities (page "FlashAttention-T:
  Optimización GPU para LLMs Escalables", which names FP8 support only).

Every function is pinned by ``tests/test_oracle*.py`` (brute force, torch CPU
fp64 library routines, closed forms, invariants, finite differences and the
hand-derived fixtures in ``tests/golden/``). No function here is "parity
unpinned".
"""

from .attn_ref import (  # noqa: F401
    attn_fwd,
    attn_fwd_head,
    attn_fwd_rows,
    attn_bwd,
    attn_bwd_head,
)
from .gqa import attn_bwd_gqa, attn_fwd_gqa  # noqa: F401
from .decode import attn_decode, attn_decode_split, attn_partial, bytes_decode, merge_partials  # noqa: F401
from .fp8 import attn_fwd_fp8, quantize_e4m3, round_e4m3  # noqa: F401
