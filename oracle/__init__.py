"""CPU oracle for the weight-streaming skinny GEMM (NVFP4 / FP8 weights).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this package: only the tests, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` use it. It shares no code, tables, constants
or helpers with the HIP library; the two meet only through the seeded input
generators in ``workloads.py`` (which hold none of the method's arithmetic).

What it computes. The pages cited throughout are:

  [P3] https://reddlx.com/feed/productivity-ai-news, the post "Four Tesla
       V100s from 2017 matched my RTX 5090 on single-request Qwen 3.8 decode".
       Section names below are that post's headings.

The post's kernel keeps weights compressed (NVFP4 or FP8) in HBM and turns
each fragment into FP16 in registers, with no separate dequantize-to-FP16 pass
([P3] "What I actually built"); activations stay FP16 and FP4 / FP8 regions
keep their own formats ([P3] "v1.0 got us here. v1.1 removes its last
compromise."). Such a kernel reaches, up to summation order, the plain result

    y[m, n] = sum_k x[m, k] * wdq[n, k]

where wdq is the dequantized weight. The oracle writes that definition out in
float64 (``gemm.py``), together with the format tables and encoders
(``formats.py``), the quantizers that produce synthetic NVFP4 / FP8 weights
(``quantize.py``), the canonical byte layout of packed codes (``layout.py``)
the SwiGLU that a fused gate_up epilogue computes (``mlp.py``) and the offline
FP8 -> NVFP4 conversion (``requantize.py``).

The pages never define the bit formats; the oracle uses the public
definitions: E2M1 (OCP Microscaling spec v1.0, FP4 element type), E4M3 "FN"
(OCP 8-bit floating point spec: bias 7, max 448, no infinities, S.1111.111 is
NaN), NVFP4 = E2M1 codes with one E4M3 scale per 16 consecutive elements along
K and one fp32 per-tensor scale, FP8 = E4M3 codes with one fp32 scale per
output row. Every other reading (quantization recipe, nibble order, rounding,
saturation) is stated at the function that makes it.

Pins. Every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself: torch's float8_e4m3fn decoder and encoder, the
E2M1 value table of the OCP spec (``tests/golden/``), hand-computed cases,
closed-form invariants and an independent dequantize-then-matmul route.
"""

from .formats import (
    E2M1_MAX,
    E4M3_MAX,
    e2m1_table,
    e4m3_table,
    decode_e2m1,
    decode_e4m3,
    encode_e2m1,
    encode_e4m3,
)
from .quantize import quantize_nvfp4, quantize_fp8, nvfp4_tensor_scale
from .layout import pack_nibbles, unpack_nibbles
from .gemm import (
    dequantize_nvfp4,
    dequantize_fp8,
    skinny_gemm,
    gemm_nvfp4,
    gemm_fp8,
    tolerance,
    argmax_candidates,
)
from .mlp import down_tolerance, gated_mlp, silu, split_gate_up, swiglu, swiglu_tolerance
from .requantize import dequantize_fp8_f32, requantize_fp8_to_nvfp4

__all__ = [
    "E2M1_MAX", "E4M3_MAX", "e2m1_table", "e4m3_table", "decode_e2m1",
    "decode_e4m3", "encode_e2m1", "encode_e4m3", "quantize_nvfp4",
    "quantize_fp8", "nvfp4_tensor_scale", "pack_nibbles", "unpack_nibbles",
    "dequantize_nvfp4", "dequantize_fp8", "skinny_gemm", "gemm_nvfp4",
    "gemm_fp8", "tolerance", "argmax_candidates", "silu", "split_gate_up", "swiglu", "swiglu_tolerance", "down_tolerance", "gated_mlp",
    "dequantize_fp8_f32", "requantize_fp8_to_nvfp4",
]
