"""CPU oracle for the fused GEMM-epilogue path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct float64 implementation of what the pages
define: a dense GEMM (float64 accumulation, numpy's float64 matmul serving as
the library step) followed by the *literal unfused* epilogue, one full-array
pass per op, then the output encoders (bf16 / OCP fp8-e4m3, both
round-to-nearest-even computed directly from the float64 value).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``gemm_epilogue_transformer_tiled_amd``) and never imports it; the only thing
both sides share is the seeded input generator in ``workloads``.

Sources (pages as titled):
  * "Lean4-TileLang Tensor Program Superoptimizer" write-up: section 7
    (SwiGLU graph, SiLU definition, the exp2 form of the sigmoid), section 8
    (plain tiled matmul), section 9 (RMSNorm scale and the row-scale rewrite),
    section 10 (RMSNorm-MLP graph).
  * "Optimising GPU kernels with TileLang: from GEMM to FlashAttention"
    tutorial: the fused bias + GELU epilogue paragraph.
  * "CODA: GEMM-epilogue for Transformer blocks" news item, section "How CODA
    works": the epilogue primitive set (scaling, reductions, pairwise
    transforms, accumulation).
  * "NVIDIA cuDNN Graph API" tutorial: the batched-matmul paragraph (host
    scalar alpha, bias, activation, AMAX on the result feeding fp8 scaling).

Every function is pinned by ``tests/test_oracle_*.py`` (brute force on tiny
inputs, closed forms, invariants, library special cases); no function here is
left unpinned.
"""
from .codecs import (  # noqa: F401
    BF16_MAX, E4M3_MAX, decode_bf16, decode_e4m3, encode_bf16, encode_e4m3,
)
from .ops import (  # noqa: F401
    act, act_grad, amax, bias_col, col_sum, gelu_tanh, gelu_tanh_grad, gemm, pairwise_act_mul,
    quant_fp8, relu, relu_grad, residual, row_rms_scale, row_scale, scale, silu, silu_exp2_form,
    silu_grad,
)
from .chain import OracleResult, run_chain, run_workload  # noqa: F401
