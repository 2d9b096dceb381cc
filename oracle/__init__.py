"""fp64 CPU oracle for block-sparse masked attention (forwards, log-sum-exp, backwards).

TEST INFRASTRUCTURE ONLY. This package is the independent, slow, plainly
written reference that the GPU path is checked against. Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library itself never does, and this package imports nothing
from the library.

Every function states the passage of the source pages it follows:
  * "Attention Kernels — Splash, Flash, SDPA on TPU" (skills-for-agents
    attention.md), page 1;
  * "hstu_ops.py" (RecML ``recml/core/ops/hstu_ops.py``), page 2;
  * "JAX 到 VLIW，以及 Pallas / Splash Attention 复习笔记" (study notes on
    "From JAX to VLIW" and "When XLA Isn't Enough"), page 3.
"""

from .splash_oracle import (  # noqa: F401
    element_mask,
    padded_element_mask,
    next_nonempty,
    mask_info,
    mask_info_row,
    mask_info_dkv,
    softmax_attention,
    softmax_attention_rows,
    online_softmax_rows,
    pointwise_attention,
    pointwise_attention_rows,
    block_flops,
    element_flops,
    kv_head_of,
    partial_blocks,
    pointwise_attention_bwd,
    pointwise_attention_bwd_rows,
    softmax_lse,
    softmax_lse_rows,
    softmax_attention_bwd,
    softmax_attention_bwd_rows,
)
