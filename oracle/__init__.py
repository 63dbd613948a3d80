"""CPU oracle for sink attention, the MoE routing softmax and the bias / FP8 block-scaled GEMM
(float64, NumPy).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The HIP library's product path never imports it,
and it imports nothing from the HIP package.
"""
from .sink_attention import (  # noqa: F401
    NEG_INF,
    attend,
    causal_allowed,
    chunk_size,
    chunk_state,
    decode,
    decode_multi,
    decode_multi_split,
    decode_split,
    merge,
    online_row,
    prefill,
    prefill_at,
    prefill_split,
    sink_softmax,
    split_size,
)
from .moe_routing import moe_topk_softmax, topk_experts  # noqa: F401
from .gemm import e4m3_to_float, gemm_bias, gemm_fp8_block_scaled  # noqa: F401
