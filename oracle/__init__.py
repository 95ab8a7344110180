"""CPU oracle for the routed Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct statement of what the layer computes.  Only the test-suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls, links or imports
anything from here, and nothing here imports the GPU library: the two
share no code, no constants and no helpers.

Everything is NumPy in float64 unless a step fixes another precision
(the fp32 router logits, the fp32 routing keys, the bf16 / e4m3 storage
grids).

Sources (web pages; cited by title and section):

* [PB] "Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood TPU"
  (dev.infolabhq.com, English and Spanish versions), sections
  "The Architectural Constraints That Break Naive Sharding",
  "Fusing Three Collectives Into Two", "Three High-Leverage
  Optimizations" (table), "Roofline Validation".
* [IM] "Como o Google otimizou o Qwen 3.5 de 397B no TPU7x (Ironwood)"
  (imasters.com.br), sections "Por que esse modelo é difícil de servir",
  "O problema do sharding e a solução".
* [VN] "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood"
  (aihot.vn), section "3. Sparse Mixture-of-Experts (MoE)".

Where the pages leave a step open (the routing formula, the expert form,
the tie-break, the fp8 scaling granularity) the reading taken is stated
in the docstring of the function that implements it.

Pinned by ``tests/test_oracle.py`` (brute-force dense mixture, closed
forms, invariants, library casts, a hand-derived worked example).
"""

from .numerics import bf16_round, f32_round, e4m3_round, e4m3_encode, e4m3_decode
from .moe import (
    router_logits,
    route,
    pack_routing,
    unpack_routing,
    permute,
    silu,
    swiglu_expert,
    combine,
    layer_forward,
    layer_from_routing,
    token_output,
    quantize_rows_e4m3,
    layer_from_routing_fp8,
)

__all__ = [
    "bf16_round", "f32_round", "e4m3_round", "e4m3_encode", "e4m3_decode",
    "router_logits", "route", "pack_routing", "unpack_routing", "permute",
    "silu", "swiglu_expert", "combine", "layer_forward", "layer_from_routing",
    "token_output", "quantize_rows_e4m3", "layer_from_routing_fp8",
]
