"""CPU oracle for the fine-grained MoE layer forward.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``sparse_moe_layer_04_amd``) never does and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64, built by
``oracle/build.py``); this module only marshals numpy arrays through ctypes.
Parity unpinned: the clamp form (symmetric vs gate-above-only), the shared
expert's form and the init-std reading are readings of what the pages leave
open; they are configurable, and every other step is pinned by the tests.
The microscaling weight encodings (OCP MXFP8: E4M3 values; OCP MXFP4: E2M1
values; one power-of-two scale per 32 values along K) follow the OCP
specification that the pages' "MxFP8" and "MxFP4" name; the clamp of the
shared exponent to [-110, 110] is a reading, not a rule of the pages.
"""
from .oracle import (  # noqa: F401
    MODE_TOPK,
    MODE_HASH,
    FLAG_BAD_INPUT_ID,
    FLAG_BAD_EXPERT_ID,
    library_path,
    load,
    f64_to_bf16,
    score,
    gate_logits,
    route,
    route_backward,
    permute,
    gather,
    expert_ffn,
    expert_ffn_rows,
    combine,
    combine_backward,
    swiglu_backward,
    grouped_gemm,
    grouped_wgrad,
    grouped_wgrad_entries,
    router_backward,
    round_bf16,
    add,
    layer_backward,
    tokens_forward,
    forward,
    forward_a8w4,
    tokens_forward_a8w4,
    quant_dequant_mxfp8,
    e4m3_decode,
    e4m3_encode,
    quant_mxfp8,
    dequant_mxfp8,
    e2m1_decode,
    e2m1_encode,
    quant_mxfp4,
    dequant_mxfp4,
)
