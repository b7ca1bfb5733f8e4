"""MI355X (gfx950) fine-grained Mixture-of-Experts layer forward.

The layer runs in hand-written HIP kernels behind the C ABI declared in
``include/moe.h`` (``libmoe_hip.so``); ``ops`` is its thin Python binding and
``workloads`` draws the seeded synthetic inputs.
"""
from . import ops  # noqa: F401
from .ops import (  # noqa: F401
    MoeLayer, gate_logits, route, permute, expert_ffn, combine,
    MODE_TOPK, MODE_HASH, OUT_BF16, OUT_F32,
)
