"""CPU oracle for the routed MoE expert FFN with block-scaled E4M3FN weights
(and MXFP4 weights: E2M1 codes with E8M0 scales per 32 elements).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
anything in this package: only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it.

Every function is plain numpy in float64, written step by step from the pages'
statement of the method; see ``moe_ref`` for the citation of each step.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against values that do not come from the oracle itself (torch's own E4M3FN
and E8M0 casts, E2M1 values worked by hand from the format, brute-force enumeration, closed forms computed by hand, library dense
MLPs, invariants).  Outputs at the full workload sizes have no printed values
on the pages; they are pinned only through those invariants.
"""
from .moe_ref import (  # noqa: F401
    E4M3FN_MAX,
    e4m3fn_table,
    e4m3fn_decode,
    dequantize_blocks,
    e2m1_table,
    e8m0_value,
    unpack_fp4,
    dequantize_mx,
    dequantize_weights,
    e4m3fn_encode_rne,
    quantize_rows_e4m3,
    quantize_rows_mxfp4,
    round_bf16,
    quantize_hidden_mxfp4,
    hidden_mxfp4_deviation,
    hidden_delta,
    mx_gemm_error_bound,
    dequantize_rows,
    route_softmax_topk,
    route_sigmoid_topk,
    router_logits,
    sort_by_expert,
    swiglu,
    relu2,
    expert_mlp,
    moe_ffn,
    moe_forward,
)
